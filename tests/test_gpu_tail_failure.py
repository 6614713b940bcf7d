"""A sweep whose persistent tail kernel gives up at a grid barrier must not
pass for a result.  The failure is forced from the host: GCS_TAIL_SPIN_LIMIT=0
at upload makes every barrier wait return at once for all workgroups but the
last arriver, so every kernel still exits normally.  Then y is poisoned (NaN;
0xFF for the Boolean policy), gcs_device_check reports GCS_ESTATE, gcs_bfs
returns GCS_ESTATE at the failing pass, and the mark is per sweep: a handle
uploaded without the knob, and the failing handle's own flag once checked,
are unaffected."""
import os

import numpy as np
import pytest

import helpers

pytestmark = pytest.mark.gpu


def _say(msg):
    helpers.progress(msg)


def _upload(gcs, g, policy, spin=None):
    old = os.environ.get("GCS_TAIL_SPIN_LIMIT")
    if spin is not None:
        os.environ["GCS_TAIL_SPIN_LIMIT"] = str(spin)
    try:
        return gcs.upload(g, policy)
    finally:
        if spin is not None:
            if old is None:
                del os.environ["GCS_TAIL_SPIN_LIMIT"]
            else:
                os.environ["GCS_TAIL_SPIN_LIMIT"] = old


def test_failed_tail_barrier_poisons_and_reports(oracle_mod, synth_mod):
    import torch
    from grammar_compressed_sparse_amd import gcs
    spec = synth_mod.GENOTYPE_512x4096
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols)
    x = synth_mod.normal(spec.n_cols, 101)
    xd = torch.from_numpy(x).cuda()
    _say("forced tail barrier failure: fp64 sweep on genotype 512x4096")
    bad = _upload(gcs, g, gcs.PLUS_F64, spin=0)
    y = bad.sweep_right(xd)
    with pytest.raises(gcs.GcsError, match="ESTATE"):
        bad.check()
    assert np.all(np.isnan(y.cpu().numpy()))
    bad.check()  # the flag was cleared by the report
    good = _upload(gcs, g, gcs.PLUS_F64)
    y2 = good.sweep_right(xd)
    good.check()
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    assert np.all(np.abs(y2.cpu().numpy() - yo) <= 1e-12 * absum)
    # int64: poisoned with INT64_MIN
    badi = _upload(gcs, g, gcs.PLUS_I64, spin=0)
    yi = badi.sweep_right(torch.ones(spec.n_cols, dtype=torch.int64, device="cuda"))
    with pytest.raises(gcs.GcsError, match="ESTATE"):
        badi.check()
    assert np.all(yi.cpu().numpy() == np.iinfo(np.int64).min)


def test_failed_tail_barrier_stops_bfs(synth_mod, oracle_mod):
    import torch
    from grammar_compressed_sparse_amd import gcs
    spec = synth_mod.GraphSpec(200_000, seed=8)
    rp, col = synth_mod.copy_graph(spec)
    g = gcs.build_grammar(rp, col, None, n_cols=spec.n)
    src = synth_mod.sources(spec.n, 16, 501)
    _say("forced tail barrier failure: Boolean pass and BFS on a 2e5-node copy graph")
    bad = _upload(gcs, g, gcs.BOOL_OR, spin=0)
    f = torch.zeros(spec.n, dtype=torch.uint8, device="cuda")
    f[torch.from_numpy(src).cuda()] = 1
    y = bad.sweep_right(f)
    with pytest.raises(gcs.GcsError, match="ESTATE"):
        bad.check()
    assert np.all(y.cpu().numpy() == 0xFF)
    with pytest.raises(gcs.GcsError, match="ESTATE"):
        bad.bfs(src)
    assert "BFS pass 1" in gcs.last_error()
    good = _upload(gcs, g, gcs.BOOL_OR)
    vis, counts = good.bfs(src)
    good.check()
    vo, co = oracle_mod.bfs(rp, col, src)
    assert np.array_equal(vis.cpu().numpy(), vo) and list(counts) == list(co)
