"""Parity of the batched right product Y = M X (gcs_sweep_right_batch, through
the C ABI) with the CPU oracle, column by column.

Tolerances are those of the single-vector sweep (per row r of column b,
s_rb = sum_j |M[r][j] X[j][b]|): 1e-12 s_rb for fp64 and fp32->fp64, 1e-5 s_rb
for fp32; int64, Boolean, X = ones and X = e_j columns bit-exact.
"""

import numpy as np
import pytest

import helpers as H

pytestmark = pytest.mark.gpu


def _say(msg):
    H.progress(msg)


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
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols)
    return spec, rp, col, val, g


def _batch(env, dev, X_np):
    torch, gcs = env
    X = torch.from_numpy(np.ascontiguousarray(X_np)).cuda()
    Y = dev.sweep_right_batch(X)
    dev.check()
    return Y.cpu().numpy()


def _cols_ok(Y, X, oracle_mod, rp, col, val, tol):
    worst = 0.0
    for b in range(X.shape[1]):
        yo, absum = oracle_mod.spmv_f64(rp, col, val, X[:, b].astype(np.float64))
        err = np.abs(Y[:, b].astype(np.float64) - yo)
        assert np.all(Y[absum == 0, b] == 0)
        assert np.all(err <= tol * absum), f"column {b}: max rel err {np.max(err / np.maximum(absum, 1e-300))}"
        worst = max(worst, float(np.max(err / np.maximum(absum, 1e-300))))
    return worst


@pytest.mark.parametrize("B", [1, 3, 8, 32, 64])
def test_batch_c1_f64(env, oracle_mod, synth_mod, c1, B):
    torch, gcs = env
    spec, rp, col, val, g = c1
    dev = gcs.upload(g, gcs.PLUS_F64)
    X = np.stack([synth_mod.normal(spec.n_cols, 1000 + b) for b in range(B)], axis=1)
    Y = _batch(env, dev, X)
    _say(f"C1 fp64 B={B}: max rel err {_cols_ok(Y, X, oracle_mod, rp, col, val, 1e-12):.2e}")
    # repeated batched sweeps are bit-identical
    Xt = torch.from_numpy(X).cuda()
    for _ in range(3):
        assert np.array_equal(dev.sweep_right_batch(Xt).cpu().numpy(), Y)


def test_batch_matches_single(env, synth_mod, c1):
    """Column b of a batched sweep against gcs_sweep_right on column b."""
    torch, gcs = env
    spec, rp, col, val, g = c1
    dev = gcs.upload(g, gcs.PLUS_F64)
    X = np.stack([synth_mod.normal(spec.n_cols, 2000 + b) for b in range(7)], axis=1)
    Y = _batch(env, dev, X)
    for b in range(7):
        y = dev.sweep_right(torch.from_numpy(np.ascontiguousarray(X[:, b])).cuda()).cpu().numpy()
        scale = np.abs(y) + 1.0
        assert np.all(np.abs(Y[:, b] - y) <= 1e-12 * scale * 200)


def test_batch_exact_policies(env, oracle_mod, synth_mod, c1):
    torch, gcs = env
    spec, rp, col, val, g = c1
    m = spec.n_cols
    # int64: exact
    dev = gcs.upload(g, gcs.PLUS_I64)
    Xi = np.stack([((np.arange(m, dtype=np.int64) * (7919 + 2 * b)) % 100_003) - 50_000 for b in range(5)], axis=1)
    Y = _batch(env, dev, Xi)
    for b in range(5):
        assert np.array_equal(Y[:, b], oracle_mod.spmv_i64(rp, col, val, np.ascontiguousarray(Xi[:, b])))
    # Boolean: exact
    dev = gcs.upload(g, gcs.BOOL_OR)
    Xb = np.stack([(synth_mod.normal(m, 50 + b) > 1.5).astype(np.uint8) for b in range(16)], axis=1)
    Y = _batch(env, dev, Xb)
    for b in range(16):
        assert np.array_equal(Y[:, b], oracle_mod.spmv_bool(rp, col, np.ascontiguousarray(Xb[:, b])))
    # fp32: X = ones and X = e_j columns give exact integers
    dev = gcs.upload(g, gcs.PLUS_F32)
    Xf = np.zeros((m, 4), np.float32)
    Xf[:, 0] = 1
    for b, j in ((1, 0), (2, 1234), (3, m - 1)):
        Xf[j, b] = 1
    Y = _batch(env, dev, Xf)
    for b in range(4):
        yo, _ = oracle_mod.spmv_f64(rp, col, val, Xf[:, b].astype(np.float64))
        assert np.array_equal(Y[:, b].astype(np.float64), yo)


def test_batch_accumulate(env, oracle_mod, synth_mod, c1):
    torch, gcs = env
    spec, rp, col, val, g = c1
    dev = gcs.upload(g, gcs.PLUS_F64)
    X = np.stack([synth_mod.normal(spec.n_cols, 3000 + b) for b in range(4)], axis=1)
    Y0 = np.stack([synth_mod.normal(spec.n_rows, 4000 + b) for b in range(4)], axis=1)
    Yt = torch.from_numpy(np.ascontiguousarray(Y0)).cuda()
    dev.sweep_right_batch(torch.from_numpy(X).cuda(), Yt, accumulate=True)
    dev.check()
    Y = Yt.cpu().numpy()
    for b in range(4):
        yo, absum = oracle_mod.spmv_f64(rp, col, val, np.ascontiguousarray(X[:, b]))
        assert np.all(np.abs(Y[:, b] - (Y0[:, b] + yo)) <= 1e-12 * (absum + np.abs(Y0[:, b])) * 2)


def test_batch_worked_example(env, worked_example):
    torch, gcs = env
    g = gcs.grammar_from_rules(**H.we_grammar_arrays(worked_example))
    dev = gcs.upload(g, gcs.PLUS_F64)
    x = np.array(worked_example["x"]["values"], np.float64)
    Y = _batch(env, dev, np.stack([x, 2 * x, -x], axis=1))
    rv = worked_example["root_values"]
    expect = np.array([rv["N%d" % r] for r in worked_example["C"]["row_roots"]])
    for b, f in enumerate((1.0, 2.0, -1.0)):
        assert np.all(np.abs(Y[:, b] - f * expect) <= 1e-12 * np.abs(expect) * 2)


def test_batch_identity_no_rules(env, oracle_mod):
    """Identity matrix: R is empty, L = 0, Y = X (level-0 emission only)."""
    torch, gcs = env
    n = 300
    rp = np.arange(n + 1, dtype=np.int64)
    col = np.arange(n, dtype=np.int32)
    val = np.full(n, 2.0)
    g = gcs.build_grammar(rp, col, val, n_cols=n)
    assert g.stats()["depth"] == 0
    dev = gcs.upload(g, gcs.PLUS_F64)
    X = np.random.default_rng(1).standard_normal((n, 5))
    Y = _batch(env, dev, X)
    assert np.array_equal(Y, 2.0 * X)


@pytest.mark.parametrize("B", [16])
def test_batch_genotype_mid_tiles(env, oracle_mod, synth_mod, B):
    torch, gcs = env
    spec = synth_mod.GenotypeSpec(2000, 12_000, 32, 300.0, 0.002, seed=12)
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols, col_chunk=997)
    X = np.stack([synth_mod.normal(spec.n_cols, 5000 + b) for b in range(B)], axis=1).astype(np.float32)
    dev = gcs.upload(g, gcs.PLUS_F32)
    e32 = _cols_ok(_batch(env, dev, X), X, oracle_mod, rp, col, val, 1e-5)
    dev = gcs.upload(g, gcs.PLUS_F32_ACC_F64)
    e64 = _cols_ok(_batch(env, dev, X), X, oracle_mod, rp, col, val, 1e-12)
    _say(f"genotype 2000x12000 B={B}: fp32 {e32:.2e}, fp32->fp64 {e64:.2e}")


def test_batch_copy_graph_multi_source(env, oracle_mod, synth_mod):
    """16 Boolean frontiers at once on the 3e5-node copy-model graph."""
    torch, gcs = env
    spec = synth_mod.GraphSpec(300_000, seed=55)
    rp, col = synth_mod.copy_graph(spec)
    g = gcs.build_grammar(rp, col, None, n_cols=spec.n)
    dev = gcs.upload(g, gcs.BOOL_OR)
    Xb = np.zeros((spec.n, 16), np.uint8)
    for b in range(16):
        Xb[synth_mod.sources(spec.n, 4, 600 + b), b] = 1
    Y = _batch(env, dev, Xb)
    for b in range(16):
        assert np.array_equal(Y[:, b], oracle_mod.spmv_bool(rp, col, np.ascontiguousarray(Xb[:, b])))


def test_batch_abi_errors(env, c1):
    torch, gcs = env
    spec, rp, col, val, g = c1
    dev = gcs.upload(g, gcs.PLUS_F64)
    for B in (0, 65):
        with pytest.raises(gcs.GcsError):
            dev.batch_workspace_bytes(B)
    X = torch.zeros((spec.n_cols, 4), dtype=torch.float64, device="cuda")
    Y = torch.zeros((spec.n_rows, 4), dtype=torch.float64, device="cuda")
    need = dev.batch_workspace_bytes(4)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    st = gcs._lib.gcs_sweep_right_batch(dev.handle, X.data_ptr(), Y.data_ptr(), 4, small.data_ptr(), small.numel(),
                                        0, torch.cuda.current_stream().cuda_stream)
    assert st == -1  # GCS_EINVAL: workspace too small, nothing launched
    with pytest.raises(gcs.GcsError):
        dev.sweep_right_batch(torch.zeros((spec.n_cols + 1, 4), dtype=torch.float64, device="cuda"))


@pytest.mark.parametrize("pol,dt,B", [("f64", np.float64, 1), ("f64", np.float64, 8), ("f32", np.float32, 32),
                                      ("i64", np.int64, 5), ("bool", np.uint8, 64), ("min_plus_f32", np.float32, 4),
                                      ("f32_acc_f64", np.float32, 6)])
def test_batch_leaves_in_sweep(env, synth_mod, c1, pol, dt, B):
    """GCS_BATCH_LEAVES_IN_SWEEP (no terminal array) gives the same bits as the
    sweep with the terminal array, in a workspace smaller by alpha rows."""
    torch, gcs = env
    spec, rp, col, val, g = c1
    dev = gcs.upload(g, gcs.POLICY_NAMES[pol])
    rng = np.random.default_rng(B)
    if dt == np.uint8:
        X = (rng.random((spec.n_cols, B)) < 0.05).astype(np.uint8)
    elif dt == np.int64:
        X = rng.integers(-1000, 1000, (spec.n_cols, B))
    else:
        X = rng.standard_normal((spec.n_cols, B)).astype(dt)
    Xt = torch.from_numpy(X).cuda()
    Ya = dev.sweep_right_batch(Xt)
    Yb = dev.sweep_right_batch(Xt, leaves_in_sweep=True)
    dev.check()
    assert torch.equal(Ya, Yb)
    alpha = g.stats()["n_terminals"]
    elem = {np.float64: 8, np.float32: 4, np.int64: 8, np.uint8: 1}[dt]
    if pol == "f32_acc_f64":
        elem = 8
    saved = dev.batch_workspace_bytes(B) - dev.batch_workspace_bytes(B, leaves_in_sweep=True)
    assert abs(saved - alpha * B * elem) < 512


def test_batch_leaves_in_sweep_graph(env, oracle_mod, synth_mod):
    torch, gcs = env
    spec = synth_mod.GraphSpec(300_000, seed=55)
    rp, col = synth_mod.copy_graph(spec)
    g = gcs.build_grammar(rp, col, None, n_cols=spec.n)
    dev = gcs.upload(g, gcs.BOOL_OR)
    Xb = np.zeros((spec.n, 32), np.uint8)
    for b in range(32):
        Xb[synth_mod.sources(spec.n, 4, 700 + b), b] = 1
    Y = dev.sweep_right_batch(torch.from_numpy(Xb).cuda(), leaves_in_sweep=True)
    dev.check()
    Y = Y.cpu().numpy()
    for b in range(32):
        assert np.array_equal(Y[:, b], oracle_mod.spmv_bool(rp, col, np.ascontiguousarray(Xb[:, b])))
    with pytest.raises(gcs.GcsError):  # unknown flag bit
        gcs._check(gcs._lib.gcs_batch_workspace_bytes(dev.handle, 4, 4, None))
