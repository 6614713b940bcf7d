"""Parity at full size: the 20,000 x 100,000 genotype matrix (about 6.2e8
nonzeros), built with the host builder's tiling (2,000-column tiles).

Every output is compared with the oracle (fp64 compensated over the whole
matrix, ~0.25 s per vector on 16 cores): fp32 and fp32 -> fp64 on all 20,000
rows, each of the 32 multiply-many vectors on all rows, and every column of
the batched B = 32 sweep on all rows; x = ones bit for bit against the
oracle's exact integer product.
"""
import time

import numpy as np
import pytest

import helpers

pytestmark = pytest.mark.gpu


def _say(msg):
    helpers.progress(msg)


@pytest.fixture(scope="module")
def big(synth_mod):
    import torch
    from grammar_compressed_sparse_amd import gcs
    assert torch.cuda.is_available()
    spec = synth_mod.GENOTYPE_20000x100000
    t = time.time()
    rp, col, val = synth_mod.genotype(spec)
    _say(f"generated genotype 20000x100000 nnz={rp[-1]} in {time.time() - t:.1f}s")
    t = time.time()
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols, col_chunk=2000)
    _say(f"built grammar in {time.time() - t:.1f}s: {g.stats()}")
    rows = None  # every row is checked
    return torch, gcs, spec, rp, col, val, g, rows


def _all_ok(y, oracle_mod, rp, col, val, x64, tol):
    """every row of y against the oracle; returns the largest relative error"""
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x64)
    err = np.abs(np.asarray(y, np.float64) - yo)
    assert np.all(y[absum == 0] == 0)
    assert np.all(err <= tol * absum), f"max rel err {np.max(err / np.maximum(absum, 1e-300))}"
    return float(np.max(err / np.maximum(absum, 1e-300)))


def test_fullsize_f32_every_row(big, oracle_mod, synth_mod):
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32)
    x = synth_mod.normal(spec.n_cols, 201).astype(np.float32)
    y = dev.sweep_right(torch.from_numpy(x).cuda())
    dev.check()
    e = _all_ok(y.cpu().numpy(), oracle_mod, rp, col, val, x.astype(np.float64), 1e-5)
    _say(f"fp32: all {spec.n_rows} rows, max rel err {e:.2e}")


def test_fullsize_ones_exact(big, oracle_mod):
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32)
    y = dev.sweep_right(torch.ones(spec.n_cols, dtype=torch.float32, device="cuda"))
    dev.check()
    sums = oracle_mod.spmv_i64(rp, col, val, np.ones(spec.n_cols, np.int64))
    assert np.array_equal(y.cpu().numpy().astype(np.int64), sums)


def test_fullsize_f32_acc_f64(big, oracle_mod, synth_mod):
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32_ACC_F64)
    x = synth_mod.normal(spec.n_cols, 202).astype(np.float32)
    y = dev.sweep_right(torch.from_numpy(x).cuda())
    dev.check()
    e = _all_ok(y.cpu().numpy(), oracle_mod, rp, col, val, x.astype(np.float64), 1e-12)
    _say(f"fp32 -> fp64: all rows, max rel err {e:.2e}")


def test_fullsize_multiply_many(big, oracle_mod, synth_mod):
    """32 successive independent fp32 vectors through one uploaded grammar,
    every row of every product."""
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32)
    worst = 0.0
    for seed in range(301, 333):
        x = synth_mod.normal(spec.n_cols, seed).astype(np.float32)
        y = dev.sweep_right(torch.from_numpy(x).cuda())
        worst = max(worst, _all_ok(y.cpu().numpy(), oracle_mod, rp, col, val, x.astype(np.float64), 1e-5))
    dev.check()
    _say(f"32 vectors: all rows each, max rel err {worst:.2e}")


def test_fullsize_batch32(big, oracle_mod, synth_mod):
    """Batched Y = M X with 32 fp32 vectors in one sweep: every row of every
    column against the oracle."""
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32)
    X = np.stack([synth_mod.normal(spec.n_cols, s) for s in range(301, 333)], axis=1).astype(np.float32)
    Y = dev.sweep_right_batch(torch.from_numpy(X).cuda())
    dev.check()
    Yh = Y.cpu().numpy()
    worst = 0.0
    for b in range(32):
        worst = max(worst, _all_ok(Yh[:, b], oracle_mod, rp, col, val, X[:, b].astype(np.float64), 1e-5))
    _say(f"batched B=32: all rows of every column, max rel err {worst:.2e}")
