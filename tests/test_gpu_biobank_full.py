"""The 200,000 x 2,000,000 genotype at full size (about 1.2e11 nonzeros;
fp32 CSR about 982 GB, more than one GPU's 288 GB of HBM), as column groups
built by the device builder and all resident (page section 4.4: per column
chunk; section 7, item 1: biobank scale).

Every output is checked: y = M x in fp32 for all 200,000 rows against the
oracle (fp64 compensated, each group's CSR checked as it is generated, the
groups' partial sums added in fp64), within 1e-5 of the row's sum of |terms|;
x = ones for all rows bit for bit (integer row sums below 2^24 are exact in
fp32 in any order).  The fp32 -> fp64 accumulate policy is checked at 1e-12
on the first three groups (60,000 columns, all rows).
"""
import threading
import time

import numpy as np
import pytest

import helpers

pytestmark = pytest.mark.gpu

GROUP_COLS = 20_000


def _say(msg):
    helpers.progress(msg)


def test_biobank_full_f32_every_row(oracle_mod, synth_mod):
    import torch
    from grammar_compressed_sparse_amd import gcs, groups
    spec = synth_mod.GENOTYPE_200000x2000000
    x = synth_mod.normal(spec.n_cols, 401).astype(np.float32)
    xo = x.astype(np.float64)
    n = spec.n_rows
    yo, absum, ones = np.zeros(n), np.zeros(n), np.zeros(n, np.int64)
    lock = threading.Lock()
    one_i = np.ones(spec.n_cols, np.int64)

    def on_group(i, c0, nc, rp, col, val):
        a, b = oracle_mod.spmv_f64(rp, col, val, xo)
        r = oracle_mod.spmv_i64(rp, col, val, one_i)
        with lock:
            yo[:] += a
            absum[:] += b
            ones[:] += r

    t = time.time()
    cg = groups.build_column_groups(lambda c0, nc: synth_mod.genotype(spec, col0=c0, ncols=nc), n, spec.n_cols,
                                    GROUP_COLS, gcs.PLUS_F32, workers=3, on_group=on_group, log=_say)
    nnz = sum(s["nnz"] for s in cg.stats)
    _say(f"biobank: {len(cg.devices)} groups, nnz={nnz}, built in {time.time() - t:.0f}s, "
         f"device {cg.device_bytes / 1e9:.1f} GB")
    assert nnz > 1.2e11
    assert cg.device_bytes < 0.5 * torch.cuda.get_device_properties(0).total_memory
    y = cg.sweep_right(torch.from_numpy(x).cuda())
    cg.check()
    yh = y.cpu().numpy().astype(np.float64)
    err = np.abs(yh - yo)
    _say(f"fp32: all {n} rows, max rel err {np.max(err / np.maximum(absum, 1e-300)):.2e}")
    assert np.all(err <= 1e-5 * absum)
    y1 = cg.sweep_right(torch.ones(spec.n_cols, dtype=torch.float32, device="cuda"))
    cg.check()
    assert np.array_equal(y1.cpu().numpy().astype(np.int64), ones)
    cg.free()
    torch.cuda.empty_cache()


def test_biobank_acc_f64_three_groups_every_row(oracle_mod, synth_mod):
    import torch
    from grammar_compressed_sparse_amd import gcs, groups
    spec = synth_mod.GENOTYPE_200000x2000000
    ncols = 3 * GROUP_COLS
    x = synth_mod.normal(spec.n_cols, 401).astype(np.float32)
    xo = x.astype(np.float64)
    yo, absum = np.zeros(spec.n_rows), np.zeros(spec.n_rows)
    lock = threading.Lock()

    def on_group(i, c0, nc, rp, col, val):
        a, b = oracle_mod.spmv_f64(rp, col, val, xo)
        with lock:
            yo[:] += a
            absum[:] += b

    # the first three groups as a matrix of their own (columns beyond them empty)
    cg = groups.build_column_groups(lambda c0, nc: synth_mod.genotype(spec, col0=c0, ncols=nc), spec.n_rows,
                                    ncols, GROUP_COLS, gcs.PLUS_F32_ACC_F64, workers=3, on_group=on_group,
                                    log=_say)
    y = cg.sweep_right(torch.from_numpy(x[:ncols].copy()).cuda())
    cg.check()
    err = np.abs(y.cpu().numpy() - yo)
    _say(f"fp32 -> fp64: {spec.n_rows} rows, max rel err {np.max(err / np.maximum(absum, 1e-300)):.2e}")
    assert np.all(err <= 1e-12 * absum)
    cg.free()
    torch.cuda.empty_cache()
