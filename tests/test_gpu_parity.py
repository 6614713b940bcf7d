"""Parity of the HIP sweep (through the C ABI) with the CPU oracle.

Tolerances (per row r, s_r = sum_j |M[r][j] x[j]| from the oracle):
  fp64 and fp32->fp64 policies: |y_r - y_ref_r| <= 1e-12 s_r
  fp32 policy:                  |y_r - y_ref_r| <= 1e-5  s_r
  Boolean, int64, x = ones, x = e_j: bit-exact.
The fp32 bound holds with margin: the sweep sums each row as a tree of depth
at most L (levels) plus the C length of the row within one (row, level) group
plus L emissions, and the first-order rounding bound of such a sum is
depth * 2^-24 * s_r (Higham, Accuracy and Stability of Numerical Algorithms,
section 4.2); depths here stay below 170.
"""
import os

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


def _sweep(env, g, policy, x_np):
    torch, gcs = env
    dev = gcs.upload(g, policy)
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to("cuda")
    y = dev.sweep_right(x)
    dev.check()  # synchronises; raises if the persistent tail kernel flagged a failure
    return y.cpu().numpy(), dev


def _rel_ok(y, yo, absum, tol):
    err = np.abs(y.astype(np.float64) - yo)
    zero_rows = absum == 0
    assert np.all(y[zero_rows] == 0)
    assert np.all(err <= tol * absum), f"max rel err {np.max(err / np.maximum(absum, 1e-300))}"


def test_worked_example_eq23(env, worked_example):
    torch, gcs = env
    _say("worked example Eq. 2.3 grammar, fp64")
    g = gcs.grammar_from_rules(**H.we_grammar_arrays(worked_example))
    y, _ = _sweep(env, g, gcs.PLUS_F64, np.array(worked_example["x"]["values"], np.float64))
    rv = worked_example["root_values"]
    expect = np.array([rv["N%d" % r] for r in worked_example["C"]["row_roots"]])
    assert np.all(np.abs(y - expect) <= 1e-12 * np.abs(expect))


def test_worked_example_own_repair(env, oracle_mod, worked_example):
    torch, gcs = env
    rp, col, val = H.csr_from_dense(worked_example["M"]["rows"])
    g = gcs.build_grammar(rp, col, val, n_cols=7)
    x = np.array(worked_example["x"]["values"], np.float64)
    y, _ = _sweep(env, g, gcs.PLUS_F64, x)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    _rel_ok(y, yo, absum, 1e-12)


@pytest.fixture(scope="module")
def c1(env, synth_mod):
    torch, gcs = env
    spec = synth_mod.GENOTYPE_512x4096
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols)
    _say(f"genotype 512x4096 grammar: {g.stats()}")
    return spec, rp, col, val, g


def test_c1_f64(env, oracle_mod, synth_mod, c1):
    torch, gcs = env
    spec, rp, col, val, g = c1
    x = synth_mod.normal(spec.n_cols, 101)
    y, dev = _sweep(env, g, gcs.PLUS_F64, x)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    _rel_ok(y, yo, absum, 1e-12)
    # repeated sweeps are bit-identical (no atomics in the emission)
    xt = torch.from_numpy(x).cuda()
    for _ in range(10):
        assert np.array_equal(dev.sweep_right(xt).cpu().numpy(), y)


def test_c1_exact_cases(env, oracle_mod, synth_mod, c1):
    torch, gcs = env
    spec, rp, col, val, g = c1
    m = spec.n_cols
    for pol, dt in ((gcs.PLUS_F64, np.float64), (gcs.PLUS_F32, np.float32)):
        y, _ = _sweep(env, g, pol, np.ones(m, dt))
        yo, _ = oracle_mod.spmv_f64(rp, col, val, np.ones(m))
        assert np.array_equal(y.astype(np.float64), yo)  # integer row sums < 2^24
        for j in (0, 1234, m - 1):
            e = np.zeros(m, dt)
            e[j] = 1
            y, _ = _sweep(env, g, pol, e)
            yo, _ = oracle_mod.spmv_f64(rp, col, val, e)
            assert np.array_equal(y.astype(np.float64), yo)
    xi = (np.arange(m, dtype=np.int64) * 7919) % 100_003 - 50_000
    y, _ = _sweep(env, g, gcs.PLUS_I64, xi)
    assert np.array_equal(y, oracle_mod.spmv_i64(rp, col, val, xi))
    xb = (synth_mod.normal(m, 5) > 1.5).astype(np.uint8)
    y, _ = _sweep(env, g, gcs.BOOL_OR, xb)
    assert np.array_equal(y, oracle_mod.spmv_bool(rp, col, xb))


def test_c1_f32_policies(env, oracle_mod, synth_mod, c1):
    torch, gcs = env
    spec, rp, col, val, g = c1
    x32 = synth_mod.normal(spec.n_cols, 102).astype(np.float32)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x32.astype(np.float64))
    y, _ = _sweep(env, g, gcs.PLUS_F32, x32)
    _rel_ok(y, yo, absum, 1e-5)
    y, _ = _sweep(env, g, gcs.PLUS_F32_ACC_F64, x32)
    assert y.dtype == np.float64
    _rel_ok(y, yo, absum, 1e-12)


@pytest.mark.parametrize("col_chunk,row_chunk", [(0, 0), (997, 0), (1500, 333)])
def test_genotype_mid_tiles(env, oracle_mod, synth_mod, col_chunk, row_chunk):
    """Several tiles, ragged tails, many levels and thousands of blocks per launch."""
    torch, gcs = env
    spec = synth_mod.GenotypeSpec(2000, 12_000, 32, 300.0, 0.002, seed=12)
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols, col_chunk=col_chunk, row_chunk=row_chunk)
    st = g.stats()
    _say(f"genotype 2000x12000 tiles ({col_chunk},{row_chunk}): L={st['depth']} w*={st['max_width']}")
    x32 = synth_mod.normal(spec.n_cols, 7).astype(np.float32)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x32.astype(np.float64))
    y, _ = _sweep(env, g, gcs.PLUS_F32, x32)
    _rel_ok(y, yo, absum, 1e-5)
    y, _ = _sweep(env, g, gcs.PLUS_F64, x32.astype(np.float64))
    _rel_ok(y, yo, absum, 1e-12)


@pytest.mark.parametrize("tail", [("256", "2", "4096"), ("8", "1", "0"), ("64", "1000000", "0"),
                                  ("2048", "1", "4096"), ("64", "4", "100000000"), ("16", "1000000", "100000")])
def test_tail_split_bit_identical(env, oracle_mod, synth_mod, c1, monkeypatch, tail):
    """The persistent tail kernel (narrow levels behind grid barriers) gives the
    same bits as one launch per level, whatever the split and the tail grid."""
    torch, gcs = env
    spec, rp, col, val, g = c1
    x = synth_mod.normal(spec.n_cols, 303)
    monkeypatch.setenv("GCS_TAIL_WGS", "256")
    monkeypatch.setenv("GCS_TAIL_VB", "1")
    monkeypatch.setenv("GCS_TAIL_FLAT", "0")
    ref, dev = _sweep(env, g, gcs.PLUS_F64, x)
    n_ref = dev.sweep_launches()
    monkeypatch.setenv("GCS_TAIL_WGS", tail[0])
    monkeypatch.setenv("GCS_TAIL_VB", tail[1])
    monkeypatch.setenv("GCS_TAIL_FLAT", tail[2])
    y, dev = _sweep(env, g, gcs.PLUS_F64, x)
    _say(f"tail wgs={tail[0]} vb={tail[1]} flat={tail[2]}: {dev.sweep_launches()} launches (reference {n_ref})")
    assert np.array_equal(y, ref)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    _rel_ok(y, yo, absum, 1e-12)
    xt = torch.from_numpy(x).cuda()
    for _ in range(5):
        assert np.array_equal(dev.sweep_right(xt).cpu().numpy(), ref)
    dev.check()


def test_random_values_many_distinct(env, oracle_mod):
    torch, gcs = env
    rng = np.random.default_rng(3)
    n, m = 300, 500
    dense = (rng.random((n, m)) < 0.2) * rng.choice(np.linspace(-3, 3, 200), size=(n, m))
    dense[::7] = dense[0]  # repeated rows so that RePair finds pairs
    rp, col, val = H.csr_from_dense(dense.tolist())
    g = gcs.build_grammar(rp, col, val, n_cols=m)
    x = rng.standard_normal(m)
    y, _ = _sweep(env, g, gcs.PLUS_F64, x)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    _rel_ok(y, yo, absum, 1e-12)


@pytest.mark.parametrize("case", ["identity", "spine", "dense_row", "empty_rows", "no_rows", "no_cols"])
def test_edge_cases(env, oracle_mod, case):
    torch, gcs = env
    if case == "identity":
        n = m = 1000
        rp, col = np.arange(n + 1, dtype=np.int64), np.arange(n, dtype=np.int32)
    elif case == "spine":
        n, m = 5, 300
        rp, col = np.arange(n + 1, dtype=np.int64) * m, np.tile(np.arange(m, dtype=np.int32), n)
    elif case == "dense_row":
        n, m = 1, 70_000
        rp, col = np.array([0, m], np.int64), np.arange(m, dtype=np.int32)
    elif case == "empty_rows":
        n, m = 100, 10
        rp = np.zeros(n + 1, np.int64)
        rp[51:] = 3
        col = np.array([1, 4, 9], np.int32)
    elif case == "no_rows":
        n, m = 0, 10
        rp, col = np.zeros(1, np.int64), np.zeros(0, np.int32)
    else:
        n, m = 10, 0
        rp, col = np.zeros(n + 1, np.int64), np.zeros(0, np.int32)
    g = gcs.build_grammar(rp, col, None, n_cols=m)
    x = (np.arange(m) % 13 - 6).astype(np.float64)
    y, _ = _sweep(env, g, gcs.PLUS_F64, x)
    yo, _ = oracle_mod.spmv_f64(rp, col, None, x)
    assert y.shape == (n,) and np.array_equal(y, yo)  # small integers: exact


def test_bfs_copy_graph(env, oracle_mod, synth_mod):
    torch, gcs = env
    spec = synth_mod.GraphSpec(300_000, seed=55)
    rp, col = synth_mod.copy_graph(spec)
    g = gcs.build_grammar(rp, col, None, n_cols=spec.n)
    st = g.stats()
    _say(f"copy graph 300K: nnz={st['nnz']} R={st['n_rules']} L={st['depth']}")
    src = synth_mod.sources(spec.n, 16, 501)
    dev = gcs.upload(g, gcs.BOOL_OR)
    vis, counts = dev.bfs(src)
    vis_o, counts_o = oracle_mod.bfs(rp, col, src)
    assert np.array_equal(vis.cpu().numpy(), vis_o)
    assert np.array_equal(counts, counts_o)
    # one Boolean pass alone
    xb = np.zeros(spec.n, np.uint8)
    xb[src] = 1
    y, _ = _sweep(env, g, gcs.BOOL_OR, xb)
    assert np.array_equal(y, oracle_mod.spmv_bool(rp, col, xb))


def test_bfs_pass_cap_and_repeat(env, oracle_mod, synth_mod, graph300k):
    """The BFS fixpoint refuses to run past its pass cap (GCS_ERANGE after
    exactly cap passes), and the same handle then runs the whole fixpoint
    again, twice, with the oracle's counts (no state is left between
    fixpoints)."""
    torch, gcs = env
    spec, g = graph300k
    rp, col = synth_mod.copy_graph(spec)
    src = synth_mod.sources(spec.n, 16, 501)
    vis_o, counts_o = oracle_mod.bfs(rp, col, src)
    dev = gcs.upload(g, gcs.BOOL_OR)
    assert len(counts_o) > 3
    with pytest.raises(gcs.GcsError, match="ERANGE|more passes"):
        dev.bfs(src, max_passes=2)
    for _ in range(2):
        vis, counts = dev.bfs(src)
        assert np.array_equal(counts, counts_o) and np.array_equal(vis.cpu().numpy(), vis_o)
    vis, counts = dev.bfs(src, max_passes=len(counts_o))  # exactly enough passes
    assert np.array_equal(counts, counts_o)


def test_abi_errors_on_device(env):
    torch, gcs = env
    g = gcs.build_grammar(np.array([0, 2], np.int64), np.array([0, 1], np.int32), None, n_cols=2)
    dev = gcs.upload(g, gcs.PLUS_F32)
    with pytest.raises(gcs.GcsError):
        dev.sweep_right(torch.zeros(3, dtype=torch.float32, device="cuda"))  # wrong length
    with pytest.raises(gcs.GcsError):
        dev.sweep_right(torch.zeros(2, dtype=torch.float64, device="cuda"))  # wrong dtype
    with pytest.raises(gcs.GcsError, match="ESTATE"):
        dev.bfs([0])  # not Boolean (matrix is 1x2 and policy fp32)


def test_loaded_grammar_sweeps_identically(env, synth_mod, c1, tmp_path):
    """A grammar saved and loaded back (gcs_save_grammar / gcs_load_grammar)
    gives the same bits as the one it was saved from: single and batched."""
    torch, gcs = env
    spec, rp, col, val, g = c1
    g.save(tmp_path / "c1.gcs")
    h = gcs.load_grammar(tmp_path / "c1.gcs")
    x = synth_mod.normal(spec.n_cols, 404)
    ya, _ = _sweep(env, g, gcs.PLUS_F64, x)
    yb, _ = _sweep(env, h, gcs.PLUS_F64, x)
    assert np.array_equal(ya, yb)
    X = torch.from_numpy(np.stack([synth_mod.normal(spec.n_cols, 405 + b) for b in range(4)], axis=1)).cuda()
    da, db = gcs.upload(g, gcs.PLUS_F64), gcs.upload(h, gcs.PLUS_F64)
    assert torch.equal(da.sweep_right_batch(X), db.sweep_right_batch(X))
    da.check()
    db.check()


def test_loaded_graph_grammar_direct_policies(env, oracle_mod, synth_mod, graph300k, tmp_path, monkeypatch):
    """A graph grammar saved and loaded back sweeps like the original under
    the uploads that rebuild level 0's emission (Boolean LDS windows,
    tropical sub-slice cut, forced so that this small graph takes them) and
    equals the oracle."""
    torch, gcs = env
    spec, g = graph300k
    rp, col = synth_mod.copy_graph(spec)
    g.save(tmp_path / "graph.gcs")
    h = gcs.load_grammar(tmp_path / "graph.gcs")
    rng = np.random.default_rng(505)
    xb = (rng.random(spec.n) < 0.05).astype(np.uint8)
    xt = (rng.random(spec.n) * 9).astype(np.float32)
    xt[rng.random(spec.n) < 0.7] = np.inf
    monkeypatch.setenv("GCS_LEVEL0_SPLIT", "4")
    for policy, x, ref in ((gcs.BOOL_OR, xb, oracle_mod.spmv_bool(rp, col, xb)),
                           (gcs.MIN_PLUS_F32, xt, oracle_mod.spmv_min_plus(rp, col, None, xt, np.float32))):
        ya, _ = _sweep(env, g, policy, x)
        yb, _ = _sweep(env, h, policy, x)
        assert np.array_equal(ya, yb) and np.array_equal(yb, ref)


def test_handles_with_different_lds_images_interleave(env, oracle_mod, synth_mod, c1, monkeypatch):
    """Uploads whose narrow-level LDS images differ in size sweep in any
    interleaving (the kernel's dynamic-LDS limit is shared by all handles)."""
    torch, gcs = env
    spec, rp, col, val, g = c1
    x = synth_mod.normal(spec.n_cols, 406)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    devs = []
    for wgs, vb, flat in (("8", "1000000", "100000000"), ("16", "1", "4096"), ("8", "4", "2048")):
        monkeypatch.setenv("GCS_TAIL_WGS", wgs)
        monkeypatch.setenv("GCS_TAIL_VB", vb)
        monkeypatch.setenv("GCS_TAIL_FLAT", flat)
        devs.append(gcs.upload(g, gcs.PLUS_F64))
    xt = torch.from_numpy(x).cuda()
    ref = None
    for d in devs + devs[::-1] + devs:
        y = d.sweep_right(xt).cpu().numpy()
        d.check()
        _rel_ok(y, yo, absum, 1e-12)
        if ref is None:
            ref = y
        assert np.array_equal(y, ref)


@pytest.fixture(scope="module")
def graph300k(env, synth_mod):
    torch, gcs = env
    spec = synth_mod.GraphSpec(300_000, seed=55)
    rp, col = synth_mod.copy_graph(spec)
    return spec, gcs.build_grammar(rp, col, None, n_cols=spec.n)


def _stream_launches(gcs, g, policy, capfd):
    capfd.readouterr()
    dev = gcs.upload(g, policy)
    err = capfd.readouterr().err
    n = [int(l.split("stream emission in ")[1].split()[0]) for l in err.splitlines() if "stream emission in" in l]
    assert len(n) == 1, err
    return dev, n[0]


@pytest.mark.parametrize("pol", ["f64", "f32", "f32_acc_f64", "i64", "bool", "min_plus_f32"])
def test_stream_emission_bit_identical(env, graph300k, monkeypatch, capfd, pol):
    """Emission by chunks (stream_block) and by teams give the same bits:
    chunks forced wherever a level's team has at most two lanes, teams
    forced everywhere, and the default choice, on the 3e5-node copy graph
    (whose short groups take chunks by default) for every kind of policy."""
    torch, gcs = env
    spec, g = graph300k
    policy = gcs.POLICY_NAMES[pol]
    rng = np.random.default_rng(77)
    x = {"bool": (rng.random(spec.n) < 0.2).astype(np.uint8),
         "i64": rng.integers(-5, 6, spec.n).astype(np.int64),
         "f32": rng.standard_normal(spec.n).astype(np.float32),
         "f32_acc_f64": rng.standard_normal(spec.n).astype(np.float32)}.get(pol, rng.standard_normal(spec.n))
    if pol == "min_plus_f32":
        x = x.astype(np.float32)
    monkeypatch.setenv("GCS_UPLOAD_TRACE", "1")
    monkeypatch.setenv("GCS_LEVEL0_WINDOW", "0")  # Boolean level 0 through the level kernel
    ys, used = {}, {}
    for mode in ("default", "0", "1"):
        if mode == "default":
            monkeypatch.delenv("GCS_EMIT_STREAM", raising=False)
        else:
            monkeypatch.setenv("GCS_EMIT_STREAM", mode)
        dev, used[mode] = _stream_launches(gcs, g, policy, capfd)
        y = dev.sweep_right(torch.from_numpy(x).cuda())
        dev.check()
        ys[mode] = y.cpu().numpy()
        dev.free()
    _say(f"{pol}: stream launches default {used['default']}, forced {used['1']}")
    assert used["0"] == 0 and used["default"] > 0 and used["1"] >= used["default"]
    assert np.array_equal(ys["0"], ys["default"]) and np.array_equal(ys["1"], ys["default"])


@pytest.mark.parametrize("pol", ["bool", "min_plus_f32", "min_plus_f64"])
def test_level0_subslice_cut_identical(env, oracle_mod, synth_mod, graph300k, monkeypatch, capfd, pol):
    """Level-0 emission groups cut by column sub-slice (direct policies;
    Boolean: the word stream of LDS windows) give the same y as the grammar's
    own groups and as the oracle, single and batched (both columns, with and
    without the leaves in the sweep), for several cut counts."""
    torch, gcs = env
    spec, g = graph300k
    rp, col = synth_mod.copy_graph(spec)
    rng = np.random.default_rng(91)
    if pol == "bool":
        x = (rng.random(spec.n) < 0.1).astype(np.uint8)
        ref = oracle_mod.spmv_bool(rp, col, x)
        ref2 = oracle_mod.spmv_bool(rp, col, x[::-1].copy())
    else:
        dt = np.float32 if pol == "min_plus_f32" else np.float64
        x = (rng.random(spec.n) * 20).astype(dt)
        x[rng.random(spec.n) < 0.5] = np.inf
        ref = oracle_mod.spmv_min_plus(rp, col, None, x, dt)
        ref2 = oracle_mod.spmv_min_plus(rp, col, None, x[::-1].copy(), dt)
    X = np.ascontiguousarray(np.stack([x, x[::-1].copy()], axis=1))
    monkeypatch.setenv("GCS_UPLOAD_TRACE", "1")
    for cut in ("1", "3", "16"):
        monkeypatch.setenv("GCS_LEVEL0_SPLIT", cut)
        capfd.readouterr()
        dev = gcs.upload(g, gcs.POLICY_NAMES[pol])
        err = capfd.readouterr().err
        sub = [int(l.split("level-0 emission in ")[1].split()[0]) for l in err.splitlines() if "level-0 emission in" in l]
        assert sub == [int(cut)], err
        y = dev.sweep_right(torch.from_numpy(x).cuda())
        Y = dev.sweep_right_batch(torch.from_numpy(X).cuda())
        YL = dev.sweep_right_batch(torch.from_numpy(X).cuda(), leaves_in_sweep=True)
        dev.check()
        _say(f"{pol} cut {cut}: {err.strip().splitlines()[-1]}")
        assert np.array_equal(y.cpu().numpy(), ref)
        for Yv in (Y, YL):
            assert np.array_equal(Yv[:, 0].cpu().numpy(), ref)
            assert np.array_equal(Yv[:, 1].cpu().numpy(), ref2)
        dev.free()


def test_merged_column_groups(env, oracle_mod, synth_mod):
    """Three column groups of the 2000 x 12000 genotype built apart and merged
    (gcs_merge_grammars) sweep like the whole matrix: fp32 and fp64 within
    tolerance of the oracle, Boolean and tropical exactly."""
    torch, gcs = env
    spec = synth_mod.GenotypeSpec(2000, 12_000, 32, 300.0, 0.002, seed=12)
    rp, col, val = synth_mod.genotype(spec)
    parts = [gcs.build_grammar(*synth_mod.genotype(spec, col0=c0, ncols=nc), n_cols=spec.n_cols, col_chunk=2000)
             for c0, nc in ((0, 5000), (5000, 1), (5001, 6999))]
    g = gcs.merge_grammars(parts)
    assert g.stats()["nnz"] == int(rp[-1])
    x32 = synth_mod.normal(spec.n_cols, 8).astype(np.float32)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x32.astype(np.float64))
    y, _ = _sweep(env, g, gcs.PLUS_F32, x32)
    _rel_ok(y, yo, absum, 1e-5)
    y, _ = _sweep(env, g, gcs.PLUS_F64, x32.astype(np.float64))
    _rel_ok(y, yo, absum, 1e-12)
    xb = (x32 > 1.0).astype(np.uint8)
    y, _ = _sweep(env, g, gcs.BOOL_OR, xb)
    assert np.array_equal(y, oracle_mod.spmv_bool(rp, col, xb))
    xt = np.abs(x32)
    y, _ = _sweep(env, g, gcs.MIN_PLUS_F32, xt)
    assert np.array_equal(y, oracle_mod.spmv_min_plus(rp, col, val, xt, np.float32))


@pytest.mark.parametrize("pol", ["f64", "f32", "i64"])
def test_tail_launch_kinds_identical(env, synth_mod, c1, monkeypatch, pol):
    """The tail kernel as an ordinary launch (default) and as a cooperative
    launch (GCS_TAIL_COOP=1 at upload) runs the same schedule: bit-identical
    y over several sweeps, and no sweep flagged."""
    torch, gcs = env
    spec, rp, col, val, g = c1
    x = synth_mod.normal(spec.n_cols, 77)
    dt = {"f64": np.float64, "f32": np.float32, "i64": np.int64}[pol]
    xs = (np.round(x * 8) if pol == "i64" else x).astype(dt)
    ys = {}
    for coop in ("0", "1"):
        monkeypatch.setenv("GCS_TAIL_COOP", coop)
        dev = gcs.upload(g, gcs.POLICY_NAMES[pol])
        xd = torch.from_numpy(xs).cuda()
        runs = [dev.sweep_right(xd).cpu().numpy() for _ in range(3)]
        dev.check()
        ys[coop] = runs
        dev.free()
    for r in ys["0"] + ys["1"][1:]:
        assert np.array_equal(r, ys["1"][0])
