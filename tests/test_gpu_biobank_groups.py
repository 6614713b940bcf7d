"""Biobank-shaped genotype (200,000 individuals; 256 founders, mean segment
1,000 variants, 0.05% mutation) swept as independent column groups.

The full 200,000 x 2,000,000 matrix (about 1.2e11 nonzeros) cannot be
materialised on the host, so it is built and swept group by group: a column
group is a sub-grammar of its own (terminals carry their column, rules never
span two groups), all groups stay resident on the device, and y accumulates
across them (gcs_sweep_right, then gcs_sweep_right_acc).  This test runs the
first two 10,000-column groups at the full 200,000 rows and checks sampled
rows against the oracle, which sums the same rows over both groups' CSR.
"""
import sys
import time

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_biobank_two_column_groups(synth_mod, oracle_mod):
    import torch
    from grammar_compressed_sparse_amd import gcs
    spec = synth_mod.GENOTYPE_200000x2000000
    groups = [(0, 10_000), (10_000, 10_000)]
    x64 = synth_mod.normal(spec.n_cols, 401)
    x32 = x64.astype(np.float32)
    xd = torch.from_numpy(x32).cuda()
    rows = np.unique(np.concatenate([np.random.default_rng(7).choice(spec.n_rows, 512, replace=False),
                                     [0, spec.n_rows - 1]]))
    y32 = torch.empty(spec.n_rows, dtype=torch.float32, device="cuda")
    y64 = torch.empty(spec.n_rows, dtype=torch.float64, device="cuda")
    yo = np.zeros(rows.size)
    absum = np.zeros(rows.size)
    devs, grams = [], []
    for gi, (c0, nc) in enumerate(groups):
        t = time.time()
        rp, col, val = synth_mod.genotype(spec, col0=c0, ncols=nc)
        _say(f"group {gi}: columns [{c0}, {c0 + nc}) nnz={rp[-1]} generated in {time.time() - t:.0f}s")
        t = time.time()
        g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols, col_chunk=2000)
        st = g.stats()
        _say(f"group {gi}: grammar in {time.time() - t:.0f}s: |R|={st['n_rules']} pt={st['n_passthrough']} "
             f"L={st['depth']} |C|={st['c_len']}")
        d32, d64 = gcs.upload(g, gcs.PLUS_F32), gcs.upload(g, gcs.PLUS_F32_ACC_F64)
        devs += [d32, d64]
        _say(f"group {gi}: device bytes {d32.device_bytes} vs fp32 CSR {8 * int(rp[-1]) + 4 * (spec.n_rows + 1)}")
        if gi == 0:
            d32.sweep_right(xd, y32)
            d64.sweep_right(xd, y64)
        else:
            d32.sweep_right_acc(xd, y32)
            d64.sweep_right_acc(xd, y64)
        a, b = oracle_mod.spmv_f64_rows(rows, rp, col, val, x32.astype(np.float64))
        yo += a
        absum += b
        grams.append(g)
        del rp, col, val
    for d in devs:
        d.check()
    e32 = np.abs(y32.cpu().numpy()[rows].astype(np.float64) - yo)
    e64 = np.abs(y64.cpu().numpy()[rows] - yo)
    _say(f"max rel err fp32 {np.max(e32 / absum):.2e}, fp32 -> fp64 {np.max(e64 / absum):.2e}")
    assert np.all(e32 <= 1e-5 * absum)
    assert np.all(e64 <= 1e-12 * absum)
    # the two groups merged into one grammar (gcs_merge_grammars), one sweep
    del devs
    t = time.time()
    gm = gcs.merge_grammars(grams)
    _say(f"merged in {time.time() - t:.0f}s: {gm.stats()['nnz']} nonzeros, L={gm.stats()['depth']}")
    del grams
    dm = gcs.upload(gm, gcs.PLUS_F32)
    ym = dm.sweep_right(xd)
    dm.check()
    em = np.abs(ym.cpu().numpy()[rows].astype(np.float64) - yo)
    _say(f"merged: max rel err fp32 {np.max(em / absum):.2e}")
    assert np.all(em <= 1e-5 * absum)
