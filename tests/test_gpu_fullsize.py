"""Parity at the benchmark's full size: the 20,000 x 100,000 genotype matrix
(about 6.2e8 nonzeros), built with the tiling bench.py uses (2,000-column
tiles) and swept in the same launch configuration.

The oracle evaluates sampled rows one by one (fp64, compensated); x = ones is
checked over every row (integer row sums below 2^24 are exact in fp32 in any
order).  The multiply-many workload (32 independent fp32 vectors through one
upload) is checked on sampled rows of every vector.
"""
import sys
import time

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


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
    rows = np.unique(np.concatenate([np.random.default_rng(2024).choice(spec.n_rows, 1024, replace=False),
                                     [0, spec.n_rows - 1]]))
    return torch, gcs, spec, rp, col, val, g, rows


def _rows_ok(y, rows, oracle_mod, rp, col, val, x64, tol):
    yo, absum = oracle_mod.spmv_f64_rows(rows, rp, col, val, x64)
    err = np.abs(y[rows].astype(np.float64) - yo)
    assert np.all(err <= tol * absum), f"max rel err {np.max(err / absum)}"
    return float(np.max(err / absum))


def test_fullsize_f32_sampled_rows(big, oracle_mod, synth_mod):
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32)
    x = synth_mod.normal(spec.n_cols, 201).astype(np.float32)
    y = dev.sweep_right(torch.from_numpy(x).cuda())
    dev.check()
    e = _rows_ok(y.cpu().numpy(), rows, oracle_mod, rp, col, val, x.astype(np.float64), 1e-5)
    _say(f"fp32: {rows.size} sampled rows, max rel err {e:.2e}")


def test_fullsize_ones_exact(big, oracle_mod):
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32)
    y = dev.sweep_right(torch.ones(spec.n_cols, dtype=torch.float32, device="cuda"))
    dev.check()
    sums = np.add.reduceat(val.astype(np.int64), rp[:-1]) * (np.diff(rp) > 0)
    assert np.array_equal(y.cpu().numpy().astype(np.int64), sums)


def test_fullsize_f32_acc_f64(big, oracle_mod, synth_mod):
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32_ACC_F64)
    x = synth_mod.normal(spec.n_cols, 202).astype(np.float32)
    y = dev.sweep_right(torch.from_numpy(x).cuda())
    dev.check()
    e = _rows_ok(y.cpu().numpy(), rows, oracle_mod, rp, col, val, x.astype(np.float64), 1e-12)
    _say(f"fp32 -> fp64: max rel err {e:.2e}")


def test_fullsize_multiply_many(big, oracle_mod, synth_mod):
    """32 successive independent fp32 vectors through one uploaded grammar."""
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32)
    sub = rows[::4]
    worst = 0.0
    for seed in range(301, 333):
        x = synth_mod.normal(spec.n_cols, seed).astype(np.float32)
        y = dev.sweep_right(torch.from_numpy(x).cuda())
        worst = max(worst, _rows_ok(y.cpu().numpy(), sub, oracle_mod, rp, col, val, x.astype(np.float64), 1e-5))
    dev.check()
    _say(f"32 vectors: {sub.size} sampled rows each, max rel err {worst:.2e}")


def test_fullsize_batch32(big, oracle_mod, synth_mod):
    """Batched Y = M X with 32 fp32 vectors in one sweep: sampled rows of
    every column against the oracle."""
    torch, gcs, spec, rp, col, val, g, rows = big
    dev = gcs.upload(g, gcs.PLUS_F32)
    X = np.stack([synth_mod.normal(spec.n_cols, s) for s in range(301, 333)], axis=1).astype(np.float32)
    Y = dev.sweep_right_batch(torch.from_numpy(X).cuda())
    dev.check()
    Yh = Y.cpu().numpy()
    sub = rows[::4]
    worst = 0.0
    for b in range(32):
        worst = max(worst, _rows_ok(Yh[:, b], sub, oracle_mod, rp, col, val, X[:, b].astype(np.float64), 1e-5))
    _say(f"batched B=32: {sub.size} sampled rows per column, max rel err {worst:.2e}")
