"""Host builder through the C ABI (no GPU): losslessness, RePair termination,
levels (Eq. 3.1), pass-through completion (section 4.2), width = live set,
and the uploaded layout executed by a host emulator against the oracle.

Page: "Right Multiplication on Grammar-Compressed Matrices" (arXiv
2607.24971v1).
"""
import collections
import random

import numpy as np
import pytest

import helpers as H


@pytest.fixture(scope="module")
def gcs():
    from grammar_compressed_sparse_amd import gcs as mod
    return mod


# ---------------------------------------------------------------- worked example


def test_worked_example_eq23_levels_and_completion(gcs, worked_example):
    """The pages' own grammar (Eq. 2.3/2.4): strata, depth, the lone pass-through."""
    arr = H.we_grammar_arrays(worked_example)
    g = gcs.grammar_from_rules(**arr)
    st = g.stats()
    ex = g.export()
    alpha = len(arr["term_col"])
    assert st["depth"] == worked_example["levels"]["L"] == 5
    strata = worked_example["levels"]["strata"]
    for k, names in enumerate(strata, start=1):
        assert sorted(int(i) + 1 for i in np.nonzero(ex["rule_level"] == k)[0]) == sorted(names)
    # section 4.2 / Figure 3.1: one pass-through P at level 3 carrying N4
    assert st["n_passthrough"] == worked_example["pass_through"]["count"] == 1
    lay = g.layout()
    lvl2, lvl3, lvl4 = lay["level_meta"][2], lay["level_meta"][3], lay["level_meta"][4]
    assert lvl3[1] == 1  # one pass-through node at level 3
    n4 = worked_example["pass_through"]["carried"]
    # its source is N4's slot among level 2's binary nodes
    src = lay["ptsrc"][lvl3[3]]
    assert lvl2[5] <= src < lvl2[5] + lvl2[0]
    # N4's only parent is N8, so no binary node of level 3 reads it directly
    assert src not in set(lay["child"][lvl3[2]:lvl3[2] + lvl3[0]].ravel().tolist())
    # N8 = N4 N7 (level 4) reads the pass-through slot of level 3, the only
    # level-4 read that lands in level 3's pass-through segment
    pt_slot = lvl3[5] + lvl3[0]
    reads = lay["child"][lvl4[2]:lvl4[2] + lvl4[0]]
    assert sum(int(a == pt_slot) + int(b == pt_slot) for a, b in reads) == 1
    w = g.level_widths()
    assert list(w) == [alpha, 3, 3, 4, 2, 1]
    assert st["max_width"] == 4 and st["n_rules"] + st["n_passthrough"] == 13
    lw, _, _ = H.live_widths(ex)
    assert list(lw[1:]) == list(w[1:])
    assert n4 == 4


def test_worked_example_emulated_values(gcs, worked_example):
    """Figure 4.2: roots N12, N8, N9 evaluate to 19.3, 20.7, 12.9 on x."""
    arr = H.we_grammar_arrays(worked_example)
    g = gcs.grammar_from_rules(**arr)
    ex, lay = g.export(), g.layout()
    x = worked_example["x"]["values"]
    y = H.emulate_layout(lay, ex, x)
    rv = worked_example["root_values"]
    expect = [rv["N%d" % r] for r in worked_example["C"]["row_roots"]]
    assert np.allclose(y, expect, rtol=0, atol=1e-12)
    assert np.allclose(H.w_array_sweep(ex, x), expect, rtol=0, atol=1e-12)


def test_worked_example_own_repair(gcs, oracle_mod, worked_example):
    rp, col, val = H.csr_from_dense(worked_example["M"]["rows"])
    g = gcs.build_grammar(rp, col, val, n_cols=7)
    ex = g.export()
    assert H.expand_rows(ex) == H.csrv_rows(rp, col, val, ex)
    assert list(ex["values"]) == worked_example["V"]["values"]
    st = g.stats()
    # three distinct rows, each compressed to one root (Eq. 2.4 has the same shape)
    assert st["c_len"] == 8 and st["n_terminals"] == 12
    x = worked_example["x"]["values"]
    y = H.emulate_layout(g.layout(), ex, x)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    assert np.all(np.abs(y - yo) <= 1e-12 * absum)


# ---------------------------------------------------------------- invariants


def _check_grammar(g, rp, col, val, single_tile=True):
    ex = g.export()
    st = g.stats()
    # lossless: expanding C through R gives the CSRV string exactly
    assert H.expand_rows(ex) == H.csrv_rows(rp, col, val, ex)
    a = st["n_terminals"]
    R = st["n_rules"]
    # topological numbering, levels by Eq. (3.1)
    assert np.all((ex["rule_a"] < a + np.arange(R)) & (ex["rule_b"] < a + np.arange(R)))
    assert np.array_equal(ex["rule_level"], H.levels_eq31(ex))
    assert st["depth"] == (int(ex["rule_level"].max()) if R else 0)
    # every rule is used at least twice in the parse of C (RePair only creates
    # a rule for a pair occurring twice)
    use = np.zeros(R, np.int64)
    for s in ex["c_sym"]:
        if s >= a:
            use[s - a] += 1
    for i in range(R - 1, -1, -1):
        for c in (ex["rule_a"][i], ex["rule_b"][i]):
            if c >= a:
                use[c - a] += use[i]
    assert R == 0 or use.min() >= 2
    # RePair ran to completion: no adjacent pair of C occurs twice
    if single_tile:
        pairs = collections.Counter()
        for r in range(len(ex["c_off"]) - 1):
            seq = ex["c_sym"][ex["c_off"][r]:ex["c_off"][r + 1]]
            pairs.update(zip(seq[:-1].tolist(), seq[1:].tolist()))
        assert not pairs or max(pairs.values()) < 2
    # completion: width of every level = live set of the uncompleted grammar
    lw, lv, P = H.live_widths(ex)
    w = g.level_widths()
    assert list(w[1:]) == list(lw[1:])
    pt = int(sum(max(0, P[v] - lv[v] - 1) for v in range(R)))
    assert st["n_passthrough"] == pt
    assert int(w[1:].sum()) == R + pt
    assert st["max_width"] == (int(w[1:].max()) if len(w) > 1 else 0)
    assert np.array_equal(ex["rule_plast"], P)
    return ex


def _random_csr(rng, n, m, density, nvals):
    rows = []
    for _ in range(n):
        cols = sorted(rng.sample(range(m), int(rng.random() * density * m)))
        rows.append(cols)
    rp = np.zeros(n + 1, np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    col = np.array([c for r in rows for c in r], np.int32)
    vals = [0.5 * (i + 1) for i in range(nvals)]
    val = np.array([rng.choice(vals) for _ in range(col.size)], np.float64)
    return rp, col, val


@pytest.mark.parametrize("repair", [0, 1], ids=["exact", "rounds"])
@pytest.mark.parametrize("seed,n,m,density,nvals", [(1, 30, 40, 0.5, 2), (2, 200, 60, 0.3, 1), (3, 5, 300, 0.9, 3),
                                                    (4, 100, 100, 0.05, 70), (5, 64, 8, 1.0, 2)])
def test_random_invariants_and_emulation(gcs, oracle_mod, seed, n, m, density, nvals, repair):
    rng = random.Random(seed)
    rp, col, val = _random_csr(rng, n, m, density, nvals)
    g = gcs.build_grammar(rp, col, val, n_cols=m, repair=repair)
    ex = _check_grammar(g, rp, col, val)
    x = np.array([rng.uniform(-1, 1) for _ in range(m)])
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    y = H.emulate_layout(g.layout(), ex, x)
    assert np.all(np.abs(y - yo) <= 1e-12 * absum + 1e-300)


@pytest.mark.parametrize("repair", [0, 1], ids=["exact", "rounds"])
def test_genotype_tiles_invariants(gcs, oracle_mod, synth_mod, repair):
    spec = synth_mod.GenotypeSpec(300, 3000, 8, 100.0, 0.005, seed=3)
    rp, col, val = synth_mod.genotype(spec)
    whole = gcs.build_grammar(rp, col, val, n_cols=3000, n_threads=1, repair=repair)
    _check_grammar(whole, rp, col, val)
    tiled = gcs.build_grammar(rp, col, val, n_cols=3000, n_threads=4, col_chunk=700, row_chunk=128, repair=repair)
    ex = _check_grammar(tiled, rp, col, val, single_tile=False)
    assert tiled.stats()["n_tiles"] == 5 * 3
    x = synth_mod.normal(3000, 77)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    for g in (whole, tiled):
        y = H.emulate_layout(g.layout(), g.export(), x)
        assert np.all(np.abs(y - yo) <= 1e-12 * absum)
    # Boolean and int64 emulation are exact
    xb = (synth_mod.normal(3000, 78) > 0.8).astype(np.uint8)
    yb = H.emulate_layout(tiled.layout(), ex, xb, op="bool", dtype=np.uint8)
    assert np.array_equal(yb, oracle_mod.spmv_bool(rp, col, xb))
    xi = np.arange(3000, dtype=np.int64) - 1500
    yi = H.emulate_layout(tiled.layout(), ex, xi, dtype=np.int64)
    assert np.array_equal(yi, oracle_mod.spmv_i64(rp, col, val, xi))
    # the grammar is much smaller than the matrix
    st = whole.stats()
    assert st["n_rules"] + st["n_passthrough"] < 0.5 * st["nnz"]


# ---------------------------------------------------------------- special cases


def test_identity_matrix(gcs):
    n = 50
    rp = np.arange(n + 1, dtype=np.int64)
    col = np.arange(n, dtype=np.int32)
    g = gcs.build_grammar(rp, col, None, n_cols=n)
    st = g.stats()
    assert st["n_rules"] == 0 and st["depth"] == 0 and st["c_len"] == n and st["max_width"] == 0
    ex = g.export()
    y = H.emulate_layout(g.layout(), ex, np.arange(n, dtype=np.float64))
    assert np.array_equal(y, np.arange(n, dtype=np.float64))


@pytest.mark.parametrize("repair", [0, 1], ids=["exact", "rounds"])
def test_identical_rows_spine(gcs, repair):
    n, k = 6, 33
    rp = np.arange(n + 1, dtype=np.int64) * k
    col = np.tile(np.arange(k, dtype=np.int32), n)
    g = gcs.build_grammar(rp, col, None, n_cols=k, repair=repair)
    st = g.stats()
    assert st["n_rules"] == k - 1 and st["c_len"] == n
    if repair == 1:
        # every pair has count n, so a round replaces the local maxima of the
        # pair hash along the row (about a third of the positions): the rows
        # become trees of logarithmic depth, not the exact form's spine
        assert st["depth"] <= 10
    _check_grammar(g, rp, col, None)
    y = H.emulate_layout(g.layout(), g.export(), np.ones(k))
    assert np.array_equal(y, np.full(n, float(k)))


@pytest.mark.parametrize("repair", [0, 1], ids=["exact", "rounds"])
def test_single_dense_row(gcs, repair):
    m = 1000
    rp = np.array([0, m], np.int64)
    col = np.arange(m, dtype=np.int32)
    g = gcs.build_grammar(rp, col, None, n_cols=m, repair=repair)
    assert g.stats()["n_rules"] == 0  # no pair occurs twice
    y = H.emulate_layout(g.layout(), g.export(), np.arange(m, dtype=np.float64))
    assert y[0] == m * (m - 1) / 2


@pytest.mark.parametrize("repair", [0, 1], ids=["exact", "rounds"])
@pytest.mark.parametrize("n,m", [(0, 0), (0, 5), (7, 0), (7, 9)])
def test_empty(gcs, n, m, repair):
    rp = np.zeros(n + 1, np.int64)
    g = gcs.build_grammar(rp, np.zeros(0, np.int32), None, n_cols=m, repair=repair)
    st = g.stats()
    assert st["nnz"] == 0 and st["n_rules"] == 0 and st["c_len"] == 0
    assert g.device_layout(gcs.PLUS_F32)["grammar_bytes"] > 0


# ---------------------------------------------------------------- error paths


def test_error_paths(gcs):
    rp = np.array([0, 2, 3], np.int64)
    with pytest.raises(gcs.GcsError, match="EINVAL"):
        gcs.build_grammar(rp, np.array([3, 1, 0], np.int32), None, n_cols=5)   # unsorted row
    with pytest.raises(gcs.GcsError, match="EINVAL"):
        gcs.build_grammar(rp, np.array([1, 1, 0], np.int32), None, n_cols=5)   # duplicate column
    with pytest.raises(gcs.GcsError, match="EINVAL"):
        gcs.build_grammar(rp, np.array([1, 7, 0], np.int32), None, n_cols=5)   # column >= n_cols
    with pytest.raises(gcs.GcsError, match="EINVAL"):
        gcs.build_grammar(np.array([0, 2, 1], np.int64), np.array([0, 1], np.int32), None, n_cols=5)
    with pytest.raises(gcs.GcsError, match="EINVAL"):
        gcs.build_grammar(rp, np.array([0, 1, 0], np.int32), np.array([1.0, np.nan, 2.0]), n_cols=5)
    with pytest.raises(gcs.GcsError, match="EINVAL"):  # non-topological rule
        gcs.grammar_from_rules(1, 2, [1.0], [0, 1], [0, 0], [2, 0], [1, 1], [0, 1], [2])
    with pytest.raises(gcs.GcsError, match="EINVAL"):  # C symbol out of range
        gcs.grammar_from_rules(1, 2, [1.0], [0, 1], [0, 0], [0], [1], [0, 1], [9])
    g = gcs.build_grammar(rp, np.array([0, 1, 0], np.int32), np.array([1.5, 2.0, 1.0]), n_cols=5)
    with pytest.raises(gcs.GcsError, match="EINVAL"):  # non-integral values under the int64 policy
        g.device_layout(gcs.PLUS_I64)
    with pytest.raises(gcs.GcsError, match="EINVAL"):
        g.device_layout(17)
    assert "policy" in gcs.last_error() or gcs.last_error()


def test_stored_zeros_dropped(gcs):
    rp = np.array([0, 3], np.int64)
    g = gcs.build_grammar(rp, np.array([0, 1, 2], np.int32), np.array([1.0, 0.0, 2.0]), n_cols=3)
    assert g.stats()["nnz"] == 2 and g.stats()["n_values"] == 2


def test_similar_row_tiles_copy_graph(gcs, oracle_mod, synth_mod):
    """Row tiles over a MinHash row order: still lossless, y in input row order."""
    spec = synth_mod.GraphSpec(20_000, seed=8)
    rp, col = synth_mod.copy_graph(spec)
    g = gcs.build_grammar(rp, col, None, n_cols=spec.n, row_chunk=3000, row_order=gcs.ROWS_SIMILAR, n_threads=4)
    assert g.stats()["n_tiles"] == 7
    ex = _check_grammar(g, rp, col, None, single_tile=False)
    xb = np.zeros(spec.n, np.uint8)
    xb[synth_mod.sources(spec.n, 200, 3)] = 1
    yb = H.emulate_layout(g.layout(), ex, xb, op="bool", dtype=np.uint8)
    assert np.array_equal(yb, oracle_mod.spmv_bool(rp, col, xb))
    nat = gcs.build_grammar(rp, col, None, n_cols=spec.n, row_chunk=3000)
    # grouping similar rows keeps more of the sharing than consecutive blocks
    assert g.stats()["c_len"] < nat.stats()["c_len"]


def test_merge_column_groups(gcs, oracle_mod, synth_mod):
    """Grammars of three column groups of one genotype matrix, built apart and
    merged (gcs_merge_grammars): lossless against the whole matrix, levels
    and completion as for any grammar, the product equal to the oracle's
    (host emulation of the merged layout), and the parts' counts adding up."""
    spec = synth_mod.GenotypeSpec(400, 6000, 8, 100.0, 0.005, seed=21)
    rp, col, val = synth_mod.genotype(spec)
    cuts = [(0, 2000), (2000, 1500), (3500, 2500)]
    parts = []
    for c0, nc in cuts:
        prp, pcol, pval = synth_mod.genotype(spec, col0=c0, ncols=nc)
        parts.append(gcs.build_grammar(prp, pcol, pval, n_cols=spec.n_cols))
    g = gcs.merge_grammars(parts)
    ex = _check_grammar(g, rp, col, val, single_tile=False)
    st, sts = g.stats(), [p.stats() for p in parts]
    assert st["nnz"] == int(rp[-1]) == sum(s["nnz"] for s in sts)
    for k in ("n_terminals", "n_rules", "c_len"):
        assert st[k] == sum(s[k] for s in sts)
    x = synth_mod.normal(spec.n_cols, 77)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    y = H.emulate_layout(g.layout(), ex, x)
    assert np.all(np.abs(y - yo) <= 1e-12 * absum + 1e-300)


def test_merge_refuses_bad_parts(gcs, synth_mod):
    spec = synth_mod.GenotypeSpec(50, 400, 4, 20.0, 0.01, seed=22)
    a = gcs.build_grammar(*synth_mod.genotype(spec, col0=0, ncols=200), n_cols=spec.n_cols)
    b = gcs.build_grammar(*synth_mod.genotype(spec, col0=200, ncols=200), n_cols=spec.n_cols)
    c = gcs.build_grammar(*synth_mod.genotype(spec, col0=100, ncols=200), n_cols=spec.n_cols)
    other = gcs.build_grammar(*synth_mod.genotype(synth_mod.GenotypeSpec(51, 400, 4, 20.0, 0.01, seed=22)),
                              n_cols=400)
    for bad in ([b, a], [a, c], [a, other]):  # unordered, overlapping, shape mismatch
        with pytest.raises(gcs.GcsError, match="EINVAL"):
            gcs.merge_grammars(bad)
    with pytest.raises(gcs.GcsError):
        gcs.merge_grammars([])
    assert gcs.merge_grammars([a]).stats()["nnz"] == a.stats()["nnz"]


def test_rounds_mode_shallower_copy_graph_and_options(gcs, synth_mod):
    """Round-based RePair against the one-pair-at-a-time form on a copy-model
    graph: lossless and complete (checked above for both), a grammar within a
    few per cent of the exact form's size, and never deeper; unknown modes are
    refused."""
    spec = synth_mod.GraphSpec(3_000, seed=9)
    rp, col = synth_mod.copy_graph(spec)
    ex_g = gcs.build_grammar(rp, col, None, n_cols=spec.n, repair=gcs.REPAIR_EXACT)
    ro_g = gcs.build_grammar(rp, col, None, n_cols=spec.n, repair=gcs.REPAIR_ROUNDS)
    _check_grammar(ro_g, rp, col, None)
    a, b = ex_g.stats(), ro_g.stats()
    assert b["n_rules"] + b["c_len"] <= 1.1 * (a["n_rules"] + a["c_len"])
    assert b["depth"] <= a["depth"]
    with pytest.raises(gcs.GcsError, match="EINVAL"):
        gcs.build_grammar(rp, col, None, n_cols=spec.n, repair=7)


@pytest.mark.parametrize("repair", [0, 1], ids=["exact", "rounds"])
def test_edge_spans(gcs, synth_mod, worked_example, repair):
    """gcs_edge_spans against the definition (section 4.1): the span of an
    edge is the level of the rule minus the level of its child (0 for a
    terminal); completion (section 4.2) carries a child for its longest
    nonterminal edge minus one level."""
    spec = synth_mod.GenotypeSpec(300, 3000, 8, 100.0, 0.005, seed=3)
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=3000, repair=repair)
    ex, st = g.export(), g.stats()
    a = st["n_terminals"]
    lv = ex["rule_level"]
    spans = []
    longest = np.zeros(st["n_rules"], np.int64)
    for i in range(st["n_rules"]):
        for c in (ex["rule_a"][i], ex["rule_b"][i]):
            d = int(lv[i] - (0 if c < a else lv[c - a]))
            spans.append(d)
            if c >= a:
                longest[c - a] = max(longest[c - a], d)
    h = g.edge_spans()
    assert h[0] == 0 and h.sum() == 2 * st["n_rules"]
    assert np.array_equal(h, np.bincount(spans, minlength=st["depth"] + 1))
    assert st["n_passthrough"] == int(np.maximum(longest - 1, 0).sum())
    # the pages' grammar (Eq. 2.3): one level-skipping nonterminal edge, N8 -> N4
    gw = gcs.grammar_from_rules(**H.we_grammar_arrays(worked_example))
    exw = gw.export()
    aw = len(exw["term_col"])
    skip = [(i + 1, int(c) - aw + 1) for i in range(len(exw["rule_a"])) for c in (exw["rule_a"][i], exw["rule_b"][i])
            if c >= aw and exw["rule_level"][i] - exw["rule_level"][c - aw] > 1]
    assert skip == [(8, 4)]
    assert gw.edge_spans().sum() == 2 * len(exw["rule_a"])
