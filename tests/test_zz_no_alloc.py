"""gcs_sweep_right_batch_scratch (the batched sweep whose workspace is the
library's fixed 64 MiB device array, for callers that cannot allocate)
against gcs_sweep_right_batch with a caller-provided workspace: the same
results bit for bit, and the oracle's within the fp64 tolerance, on two calls
in a row, the second with a smaller input; a request larger than the array
is refused before any device work."""

import numpy as np
import pytest

import helpers

pytestmark = pytest.mark.gpu


def _say(msg):
    helpers.progress(msg)


def test_scratch_batch_matches_workspace_batch(oracle_mod, synth_mod):
    import torch
    from grammar_compressed_sparse_amd import gcs
    spec = synth_mod.GENOTYPE_512x4096
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols)
    dev = gcs.upload(g, gcs.PLUS_F64)
    small = synth_mod.GenotypeSpec(100, 700, 4, 50.0, 0.01, seed=31)
    rps, cols, vals = synth_mod.genotype(small)
    dsmall = gcs.upload(gcs.build_grammar(rps, cols, vals, n_cols=small.n_cols), gcs.PLUS_F64)
    rng = np.random.default_rng(11)
    # call 1: the 512 x 4096 grammar, 24 vectors; call 2: a smaller grammar
    # and fewer vectors (the array keeps call 1's contents)
    for d, (r, c, v), m, B in ((dev, (rp, col, val), spec.n_cols, 24), (dsmall, (rps, cols, vals), small.n_cols, 5)):
        _say(f"scratch batch: {d.sizes['y_len']} x {m}, B={B}, needs {d.batch_workspace_bytes(B)} bytes")
        assert d.batch_workspace_bytes(B) <= 64 << 20
        X = torch.from_numpy(rng.standard_normal((m, B))).cuda()
        Yw = d.sweep_right_batch(X)
        Ys = gcs.sweep_right_batch_scratch(d, X)
        d.check()
        assert torch.equal(Ys, Yw)
        Yh, Xh = Ys.cpu().numpy(), X.cpu().numpy()
        for b in range(B):
            yo, absum = oracle_mod.spmv_f64(r, c, v, Xh[:, b])
            assert np.all(np.abs(Yh[:, b] - yo) <= 1e-12 * absum)
        # accumulate mode and leaves in the sweep through the scratch too
        Ya = Ys.clone()
        gcs.sweep_right_batch_scratch(d, X, Ya, accumulate=True, leaves_in_sweep=True)
        Yb = Yw.clone()
        d.sweep_right_batch(X, Yb, accumulate=True, leaves_in_sweep=True)
        d.check()
        assert torch.equal(Ya, Yb)


def test_scratch_batch_boolean_and_refusal(synth_mod):
    import torch
    from grammar_compressed_sparse_amd import gcs
    gspec = synth_mod.GraphSpec(20_000, seed=8)
    rp, col = synth_mod.copy_graph(gspec)
    d = gcs.upload(gcs.build_grammar(rp, col, None, n_cols=gspec.n), gcs.BOOL_OR)
    X = torch.from_numpy((np.random.default_rng(12).random((gspec.n, 3)) < 0.01).astype(np.uint8)).cuda()
    Yw = d.sweep_right_batch(X)
    Ys = gcs.sweep_right_batch_scratch(d, X)
    d.check()
    assert torch.equal(Ys, Yw)
    # more than 64 MiB of batch workspace: refused on the host, no launch
    big = synth_mod.GenotypeSpec(2000, 12000, 32, 300.0, 0.002, seed=13)
    brp, bcol, bval = synth_mod.genotype(big)
    db = gcs.upload(gcs.build_grammar(brp, bcol, bval, n_cols=big.n_cols), gcs.PLUS_F64)
    assert db.batch_workspace_bytes(64) > 64 << 20
    Xb = torch.zeros((big.n_cols, 64), dtype=torch.float64, device="cuda")
    with pytest.raises(gcs.GcsError, match="ERANGE"):
        gcs.sweep_right_batch_scratch(db, Xb)
    assert "64 MiB" in gcs.last_error() or "67108864" in gcs.last_error()
