"""Tropical (min, +) policy on the GPU (through the C ABI) against the oracle:
bit-exact, since min never rounds and each sum is formed once, in the leaf
(section 5: combine = min, leaf = value + x[j], identity +inf)."""

import numpy as np
import pytest

import helpers

pytestmark = pytest.mark.gpu


def _say(msg):
    helpers.progress(msg)


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from grammar_compressed_sparse_amd import gcs
    return torch, gcs


@pytest.fixture(scope="module")
def c1(env, synth_mod):
    torch, gcs = env
    spec = synth_mod.GENOTYPE_512x4096
    rp, col, val = synth_mod.genotype(spec)
    return spec, rp, col, val, gcs.build_grammar(rp, col, val, n_cols=spec.n_cols)


@pytest.fixture(scope="module")
def graph(env, synth_mod):
    torch, gcs = env
    spec = synth_mod.GraphSpec(300_000, seed=55)
    rp, col = synth_mod.copy_graph(spec)
    return spec, rp, col, gcs.build_grammar(rp, col, None, n_cols=spec.n)


def _sweep(torch, dev, x):
    y = dev.sweep_right(torch.from_numpy(np.ascontiguousarray(x)).cuda())
    dev.check()
    return y.cpu().numpy()


@pytest.mark.parametrize("pol,dt", [("min_plus_f32", np.float32), ("min_plus_f64", np.float64)])
def test_min_plus_genotype(env, oracle_mod, c1, pol, dt):
    torch, gcs = env
    spec, rp, col, val, g = c1
    dev = gcs.upload(g, gcs.POLICY_NAMES[pol])
    x = np.random.default_rng(3).uniform(-10, 10, spec.n_cols).astype(dt)
    y = _sweep(torch, dev, x)
    assert y.dtype == dt
    assert np.array_equal(y, oracle_mod.spmv_min_plus(rp, col, val, x, dt))


def test_min_plus_graph_pass(env, oracle_mod, graph):
    torch, gcs = env
    spec, rp, col, g = graph
    dev = gcs.upload(g, gcs.MIN_PLUS_F32)
    x = np.random.default_rng(4).uniform(0, 100, spec.n).astype(np.float32)
    y = _sweep(torch, dev, x)
    assert np.array_equal(y, oracle_mod.spmv_min_plus(rp, col, None, x, np.float32))
    assert np.isinf(y[np.diff(rp) == 0]).all()


def test_bellman_ford_fixpoint(env, oracle_mod, synth_mod, graph):
    """d <- min(d, M d) from 16 sources with unit weights, to the fixpoint:
    the same distances as the oracle's passes, and the number of nodes at
    distance t equals the oracle BFS's new-node count of pass t."""
    torch, gcs = env
    spec, rp, col, g = graph
    dev = gcs.upload(g, gcs.MIN_PLUS_F32)
    src = synth_mod.sources(spec.n, 16, 501)
    d0 = np.full(spec.n, np.inf, np.float32)
    d0[src] = 0
    d = torch.from_numpy(d0).cuda()
    passes = 0
    while True:
        nd = torch.minimum(d, dev.sweep_right(d))
        passes += 1
        if torch.equal(nd, d):
            break
        d = nd
    dev.check()
    dg = d.cpu().numpy()
    do = d0.copy()
    for _ in range(passes):
        do = np.minimum(do, oracle_mod.spmv_min_plus(rp, col, None, do, np.float32))
    assert np.array_equal(dg, do)
    vis, counts = oracle_mod.bfs(rp, col, src)
    assert np.array_equal(np.isfinite(dg), vis.astype(bool))
    hist = np.bincount(dg[np.isfinite(dg)].astype(np.int64))
    assert hist[0] == len(np.unique(src))
    assert np.array_equal(hist[1:], counts[:len(hist) - 1])
    _say(f"Bellman-Ford fixpoint: {passes} passes, {int(np.isfinite(dg).sum())} nodes reach a source")


@pytest.mark.parametrize("tail", [("16", "1", "4096"), ("8", "1", "0"), ("64", "1000000", "100000000")])
def test_min_plus_tail_splits(env, oracle_mod, c1, monkeypatch, tail):
    torch, gcs = env
    spec, rp, col, val, g = c1
    monkeypatch.setenv("GCS_TAIL_WGS", tail[0])
    monkeypatch.setenv("GCS_TAIL_VB", tail[1])
    monkeypatch.setenv("GCS_TAIL_FLAT", tail[2])
    dev = gcs.upload(g, gcs.MIN_PLUS_F64)
    x = np.random.default_rng(5).standard_normal(spec.n_cols)
    assert np.array_equal(_sweep(torch, dev, x), oracle_mod.spmv_min_plus(rp, col, val, x, np.float64))


@pytest.mark.parametrize("pol,dt,B", [("min_plus_f32", np.float32, 8), ("min_plus_f64", np.float64, 3)])
def test_min_plus_batched(env, oracle_mod, c1, pol, dt, B):
    torch, gcs = env
    spec, rp, col, val, g = c1
    dev = gcs.upload(g, gcs.POLICY_NAMES[pol])
    X = np.random.default_rng(6).uniform(-3, 3, (spec.n_cols, B)).astype(dt)
    Y = dev.sweep_right_batch(torch.from_numpy(X).cuda())
    dev.check()
    Y = Y.cpu().numpy()
    for b in range(B):
        assert np.array_equal(Y[:, b], oracle_mod.spmv_min_plus(rp, col, val, np.ascontiguousarray(X[:, b]), dt))


def test_min_plus_empty_rows(env, oracle_mod):
    torch, gcs = env
    dense = np.zeros((9, 7))
    dense[1, [0, 3]] = [1.5, -2.0]
    dense[4, [0, 3]] = [1.5, -2.0]
    dense[7, [2, 5, 6]] = [4.0, 0.25, 1.0]
    rp = np.zeros(10, np.int64)
    rp[1:] = np.cumsum((dense != 0).sum(1))
    col = np.nonzero(dense)[1].astype(np.int32)
    val = dense[dense != 0]
    g = gcs.build_grammar(rp, col, val, n_cols=7)
    dev = gcs.upload(g, gcs.MIN_PLUS_F64)
    x = np.array([0.5, 1, 2, 3, 4, 5, 6], np.float64)
    y = _sweep(torch, dev, x)
    assert np.array_equal(y, oracle_mod.spmv_min_plus(rp, col, val, x, np.float64))
    assert np.isinf(y[[0, 2, 3, 5, 6, 8]]).all() and y[1] == 1.0 and y[7] == 5.25
