"""Degenerate shapes and accumulate mode for every kind of emission (slice
accumulators: fp64; direct into y: Boolean and tropical), single-vector and
batched, against the oracle (small integers and exact semirings: exact)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from grammar_compressed_sparse_amd import gcs
    return torch, gcs


def _matrix(case):
    if case == "identity":
        n = m = 700
        return n, m, np.arange(n + 1, dtype=np.int64), np.arange(n, dtype=np.int32)
    if case == "spine":
        n, m = 5, 300
        return n, m, np.arange(n + 1, dtype=np.int64) * m, np.tile(np.arange(m, dtype=np.int32), n)
    if case == "empty_rows":
        n, m = 100, 10
        rp = np.zeros(n + 1, np.int64)
        rp[51:] = 3
        return n, m, rp, np.array([1, 4, 9], np.int32)
    if case == "no_rows":
        return 0, 10, np.zeros(1, np.int64), np.zeros(0, np.int32)
    n, m = 10, 0  # no columns
    return n, m, np.zeros(n + 1, np.int64), np.zeros(0, np.int32)


def _x(pol, m, seed):
    rng = np.random.default_rng(seed)
    if pol == "bool":
        return (rng.random(m) < 0.3).astype(np.uint8)
    return (np.arange(m) % 13 - 6 + seed).astype(np.float64)


def _ref(oracle_mod, pol, rp, col, x):
    if pol == "bool":
        return oracle_mod.spmv_bool(rp, col, x)
    if pol == "min_plus_f64":
        return oracle_mod.spmv_min_plus(rp, col, None, x, np.float64)
    return oracle_mod.spmv_f64(rp, col, None, x)[0]


@pytest.mark.parametrize("case", ["identity", "spine", "empty_rows", "no_rows", "no_cols"])
@pytest.mark.parametrize("pol", ["f64", "bool", "min_plus_f64"])
def test_edges_single_and_batched(env, oracle_mod, case, pol):
    torch, gcs = env
    n, m, rp, col = _matrix(case)
    g = gcs.build_grammar(rp, col, None, n_cols=m)
    dev = gcs.upload(g, gcs.POLICY_NAMES[pol])
    x = _x(pol, m, 1)
    y = dev.sweep_right(torch.from_numpy(x).cuda())
    dev.check()
    assert y.shape == (n,) and np.array_equal(y.cpu().numpy(), _ref(oracle_mod, pol, rp, col, x))
    X = np.stack([_x(pol, m, s) for s in range(3)], axis=1)
    Y = dev.sweep_right_batch(torch.from_numpy(np.ascontiguousarray(X)).cuda())
    dev.check()
    assert Y.shape == (n, 3)
    for b in range(3):
        assert np.array_equal(Y[:, b].cpu().numpy(), _ref(oracle_mod, pol, rp, col, np.ascontiguousarray(X[:, b])))


@pytest.mark.parametrize("pol", ["bool", "min_plus_f64", "f64"])
def test_accumulate_every_emission_kind(env, oracle_mod, synth_mod, pol):
    """y (+)= M x: added for fp64, OR for Boolean, min for tropical, single
    and batched, on the 512 x 4096 genotype's column pattern."""
    torch, gcs = env
    spec = synth_mod.GENOTYPE_512x4096
    rp, col, _ = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, None, n_cols=spec.n_cols)
    dev = gcs.upload(g, gcs.POLICY_NAMES[pol])
    x = _x(pol, spec.n_cols, 3)
    y0 = _x(pol, spec.n_rows, 4)
    yt = torch.from_numpy(y0.copy()).cuda()
    dev.sweep_right_acc(torch.from_numpy(x).cuda(), yt)
    dev.check()
    ref = _ref(oracle_mod, pol, rp, col, x)
    if pol == "bool":
        expect = y0 | ref
    elif pol == "min_plus_f64":
        expect = np.minimum(y0, ref)
    else:
        expect = y0 + ref
    assert np.array_equal(yt.cpu().numpy(), expect)
    X = np.stack([_x(pol, spec.n_cols, 5 + b) for b in range(2)], axis=1)
    Y0 = np.stack([_x(pol, spec.n_rows, 7 + b) for b in range(2)], axis=1)
    Yt = torch.from_numpy(np.ascontiguousarray(Y0)).cuda()
    dev.sweep_right_batch(torch.from_numpy(np.ascontiguousarray(X)).cuda(), Yt, accumulate=True)
    dev.check()
    for b in range(2):
        ref = _ref(oracle_mod, pol, rp, col, np.ascontiguousarray(X[:, b]))
        y0b = Y0[:, b]
        expect = y0b | ref if pol == "bool" else (np.minimum(y0b, ref) if pol == "min_plus_f64" else y0b + ref)
        assert np.array_equal(Yt[:, b].cpu().numpy(), expect)


def _long_group_matrix():
    """4000 short random rows (3 columns) and 3 rows of 20000 random columns
    out of 100000: the long rows' bare terminals form (row, slice) groups of
    about 2400 roots, longer than one chunk round, while the level's mean
    stays below 8 roots per group (a two-lane team)."""
    rng = np.random.default_rng(2024)
    m = 100_000
    rows = [np.sort(rng.choice(m, 3, replace=False)) for _ in range(4000)]
    for i in (10, 2000, 3999):
        rows[i] = np.sort(rng.choice(m, 20_000, replace=False))
    rp = np.zeros(len(rows) + 1, np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    return len(rows), m, rp, np.concatenate(rows).astype(np.int32)


@pytest.mark.parametrize("pol", ["f64", "i64", "bool", "min_plus_f64"])
def test_stream_emission_long_groups(env, oracle_mod, monkeypatch, capfd, pol):
    """Chunked emission over groups longer than one round (1024 roots) keeps
    each group's partials across rounds: forced chunks equal forced teams bit
    for bit and the oracle (fp64 within 1e-12 of the row's absolute sum)."""
    torch, gcs = env
    n, m, rp, col = _long_group_matrix()
    g = gcs.build_grammar(rp, col, None, n_cols=m)
    rng = np.random.default_rng(5)
    x = {"bool": (rng.random(m) < 0.01).astype(np.uint8), "i64": rng.integers(-9, 10, m).astype(np.int64)}.get(
        pol, rng.standard_normal(m))
    ys, used = {}, {}
    monkeypatch.setenv("GCS_UPLOAD_TRACE", "1")
    monkeypatch.setenv("GCS_TAIL_WGS", "8")  # keep the level-1 launch out of the tail
    monkeypatch.setenv("GCS_LEVEL0_WINDOW", "0")  # Boolean level 0 through the level kernel
    for mode in ("0", "1"):
        monkeypatch.setenv("GCS_EMIT_STREAM", mode)
        capfd.readouterr()
        dev = gcs.upload(g, gcs.POLICY_NAMES[pol])
        err = capfd.readouterr().err
        used[mode] = [int(l.split("stream emission in ")[1].split()[0]) for l in err.splitlines()
                      if "stream emission in" in l]
        y = dev.sweep_right(torch.from_numpy(x).cuda())
        dev.check()
        ys[mode] = y.cpu().numpy()
        dev.free()
    assert used["0"] == [0] and used["1"][0] >= 1, used
    assert np.array_equal(ys["0"], ys["1"])
    if pol == "f64":
        yo, absum = oracle_mod.spmv_f64(rp, col, None, x)
        assert np.all(np.abs(ys["1"] - yo) <= 1e-12 * absum)
    else:
        assert np.array_equal(ys["1"], _ref(oracle_mod, pol, rp, col, x))


def _window_matrix():
    """2000 short random rows over 400000 columns and two rows of 200000
    random columns: a long row's bare terminals in one slice (about 25000)
    exceed a window chunk's 16384 roots."""
    rng = np.random.default_rng(404)
    m = 400_000
    rows = [np.sort(rng.choice(m, 1 + i % 7, replace=False)) for i in range(2000)]
    for i in (5, 1999):
        rows[i] = np.sort(rng.choice(m, 200_000, replace=False))
    rp = np.zeros(len(rows) + 1, np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    return len(rows), m, rp, np.concatenate(rows).astype(np.int32)


@pytest.mark.parametrize("split", [None, "1", "5"])
def test_boolean_window_emission(env, oracle_mod, monkeypatch, capfd, split):
    """Boolean level-0 emission from LDS windows of the bit-packed terminals
    (default, and with 1 and 5 sub-slices) equals the level-kernel emission
    without a cut and the oracle, overwrite and accumulate, including a row
    with more bare terminals than one window chunk holds."""
    torch, gcs = env
    n, m, rp, col = _window_matrix()
    g = gcs.build_grammar(rp, col, None, n_cols=m)
    rng = np.random.default_rng(6)
    x = (rng.random(m) < 0.002).astype(np.uint8)
    y0 = (rng.random(n) < 0.3).astype(np.uint8)
    ref = oracle_mod.spmv_bool(rp, col, x)
    monkeypatch.setenv("GCS_UPLOAD_TRACE", "1")
    ys = {}
    for mode in ("plain", "window"):
        if mode == "plain":
            monkeypatch.setenv("GCS_LEVEL0_SPLIT", "0")
        elif split is None:
            monkeypatch.delenv("GCS_LEVEL0_SPLIT", raising=False)
        else:
            monkeypatch.setenv("GCS_LEVEL0_SPLIT", split)
        capfd.readouterr()
        dev = gcs.upload(g, gcs.BOOL_OR)
        err = capfd.readouterr().err
        line = [l for l in err.splitlines() if "LDS windows" in l]
        assert len(line) == 1 and line[0].split("LDS windows ")[1].startswith("1" if mode == "window" else "0"), err
        y = dev.sweep_right(torch.from_numpy(x).cuda())
        ya = torch.from_numpy(y0.copy()).cuda()
        dev.sweep_right_acc(torch.from_numpy(x).cuda(), ya)
        dev.check()
        ys[mode] = (y.cpu().numpy(), ya.cpu().numpy())
        dev.free()
    assert np.array_equal(ys["window"][0], ref) and np.array_equal(ys["plain"][0], ref)
    assert np.array_equal(ys["window"][1], y0 | ref) and np.array_equal(ys["plain"][1], y0 | ref)


def _far_rows_matrix():
    """300,000 rows of which about one in 9,000 holds 1-40 random columns
    (row gaps above the 8,191 a word's increase holds, bridged by skip
    words), a run of 50 adjacent rows sharing 30 columns (rules) plus one
    column each, and the last row."""
    rng = np.random.default_rng(77)
    n, m = 300_000, 120_000
    rows = {}
    far = np.arange(0, n, 9_000) + rng.integers(0, 400, size=(n + 8_999) // 9_000)
    for r in far[far < n]:
        rows[int(r)] = rng.choice(m, int(rng.integers(1, 41)), replace=False)
    shared = rng.choice(m, 30, replace=False)
    for r in range(150_000, 150_050):
        rows[r] = np.unique(np.concatenate([shared, rng.choice(m, 1)]))
    rows[n - 1] = rng.choice(m, 7, replace=False)
    lens = np.zeros(n, np.int64)
    for r, c in rows.items():
        lens[r] = len(np.unique(c))
    rp = np.zeros(n + 1, np.int64)
    rp[1:] = np.cumsum(lens)
    col = np.concatenate([np.unique(rows[r]) for r in sorted(rows)])
    return n, m, rp, col.astype(np.int32)


@pytest.mark.parametrize("split", [None, "3"])
def test_boolean_window_far_rows(env, oracle_mod, monkeypatch, capfd, split):
    """Boolean level-0 words across row gaps longer than one word's increase
    (skip words): single vector overwrite and accumulate, and batched (B = 3,
    with and without the leaves in the sweep), equal the oracle, with and
    without windows."""
    torch, gcs = env
    n, m, rp, col = _far_rows_matrix()
    g = gcs.build_grammar(rp, col, None, n_cols=m)
    rng = np.random.default_rng(8)
    X = np.ascontiguousarray((rng.random((m, 3)) < np.array([0.3, 0.02, 1.0])).astype(np.uint8))
    refs = [oracle_mod.spmv_bool(rp, col, X[:, b].copy()) for b in range(3)]
    y0 = (rng.random(n) < 0.3).astype(np.uint8)
    monkeypatch.setenv("GCS_UPLOAD_TRACE", "1")
    if split is None:
        monkeypatch.delenv("GCS_LEVEL0_SPLIT", raising=False)
    else:
        monkeypatch.setenv("GCS_LEVEL0_SPLIT", split)
    for window in ("1", "0"):
        monkeypatch.setenv("GCS_LEVEL0_WINDOW", window)
        capfd.readouterr()
        dev = gcs.upload(g, gcs.BOOL_OR)
        err = capfd.readouterr().err
        line = [l for l in err.splitlines() if "LDS windows" in l]
        assert len(line) == 1 and line[0].split("LDS windows ")[1].startswith(window), err
        Xd = torch.from_numpy(X).cuda()
        for b in range(3):
            xb = torch.from_numpy(X[:, b].copy()).cuda()
            assert np.array_equal(dev.sweep_right(xb).cpu().numpy(), refs[b]), (window, b)
            ya = torch.from_numpy(y0.copy()).cuda()
            dev.sweep_right_acc(xb, ya)
            assert np.array_equal(ya.cpu().numpy(), y0 | refs[b]), (window, b)
        for leaves in (False, True):
            Y = dev.sweep_right_batch(Xd, leaves_in_sweep=leaves).cpu().numpy()
            for b in range(3):
                assert np.array_equal(Y[:, b], refs[b]), (window, leaves, b)
        dev.check()
        dev.free()


@pytest.mark.parametrize("pol,dt", [("min_plus_f32", np.float32), ("min_plus_f64", np.float64)])
def test_tropical_window_far_rows(env, oracle_mod, monkeypatch, capfd, pol, dt):
    """Tropical level-0 words (value windows in LDS, skip words across far
    rows, a lane's same-row words combined): single vector overwrite and
    accumulate, and batched (B = 3, with and without the leaves in the sweep)
    equal the oracle exactly, with and without windows."""
    torch, gcs = env
    n, m, rp, col = _far_rows_matrix()
    rng = np.random.default_rng(9)
    val = rng.integers(1, 5, size=col.size).astype(np.float64)
    g = gcs.build_grammar(rp, col, val, n_cols=m)
    X = (rng.random((m, 3)) * 10).astype(dt)
    X[rng.random((m, 3)) < np.array([0.5, 0.97, 0.0])] = np.inf
    X = np.ascontiguousarray(X)
    refs = [oracle_mod.spmv_min_plus(rp, col, val, X[:, b].copy(), dt) for b in range(3)]
    y0 = (rng.random(n) * 12).astype(dt)
    y0[rng.random(n) < 0.5] = np.inf
    monkeypatch.setenv("GCS_UPLOAD_TRACE", "1")
    monkeypatch.delenv("GCS_LEVEL0_SPLIT", raising=False)
    for window in ("1", "0"):
        monkeypatch.setenv("GCS_LEVEL0_WINDOW", window)
        capfd.readouterr()
        dev = gcs.upload(g, gcs.POLICY_NAMES[pol])
        err = capfd.readouterr().err
        line = [l for l in err.splitlines() if "LDS windows" in l]
        assert len(line) == 1 and line[0].split("LDS windows ")[1].startswith(window), err
        for b in range(3):
            xb = torch.from_numpy(X[:, b].copy()).cuda()
            assert np.array_equal(dev.sweep_right(xb).cpu().numpy(), refs[b]), (window, b)
            ya = torch.from_numpy(y0.copy()).cuda()
            dev.sweep_right_acc(xb, ya)
            assert np.array_equal(ya.cpu().numpy(), np.minimum(y0, refs[b])), (window, b)
        for leaves in (False, True):
            Y = dev.sweep_right_batch(torch.from_numpy(X).cuda(), leaves_in_sweep=leaves).cpu().numpy()
            for b in range(3):
                assert np.array_equal(Y[:, b], refs[b]), (window, leaves, b)
        dev.check()
        dev.free()
