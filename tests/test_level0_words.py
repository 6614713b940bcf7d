"""Level 0's word stream (gcs_level0_words), decoded on the host.

The direct policies (Boolean, tropical) upload level 0's roots, the bare
terminals of C, as one 32-bit word each: a terminal offset inside the chunk's
window and the row's increase over the previous word.  Decoding the stream
here must give back exactly the level-0 (row, terminal) pairs of the grammar's
own emission groups (gcs_export_layout), every chunk must keep its terminals
inside one window of at most 60 KB of the device terminal array and inside
one column slice, and rows must never decrease inside a chunk.  No device is
used.
"""
import numpy as np
import pytest

SKIP = (1 << 19) - 1
WIN_BYTES = 60 * 1024


def _level0_pairs(g):
    """(slice, row, terminal) of every level-0 root, from the exported layout
    (level 0's roots are terminals, whose arena offset is their index)."""
    lay = g.layout()
    g0, ng = int(lay["level_meta"][0, 6]), int(lay["level_meta"][0, 7])
    eoff = lay["eoff"][g0:g0 + ng + 1].astype(np.int64)
    grp = np.repeat(np.arange(ng), np.diff(eoff))
    sl = lay["slices"][0, 2]
    x = np.searchsorted(sl[:9], grp, side="right") - 1
    row = lay["erow"][g0:g0 + ng][grp].astype(np.int64)
    term = lay["epos"][eoff[0]:eoff[-1]].astype(np.int64)
    return x, row, term


def _decode(d):
    """rows, terminals and chunk index of every real word; checks the frame."""
    w, ch = d["words"].astype(np.int64), d["chunks"].astype(np.int64)
    assert ch.shape[0] > 0
    e0, e1 = ch[:, 0], ch[:, 1]
    assert e0[0] == 0 and e1[-1] == w.size and np.array_equal(e0[1:], e1[:-1])
    assert np.all(e1 > e0) and np.all(e0 % 8 == 0) and np.all(e1 % 8 == 0)
    assert np.all(ch[:, 6:] == 0)
    cid = np.repeat(np.arange(ch.shape[0]), e1 - e0)
    delta = w >> 19
    pos = w & SKIP
    cs = np.cumsum(delta)
    before = np.concatenate([[0], cs])[e0]  # increases before each chunk
    rows = ch[cid, 4] + cs - before[cid]
    # a chunk's first word is its first row's root
    assert np.all(delta[e0] == 0) and np.all(pos[e0] != SKIP)
    real = pos != SKIP
    return rows[real], ch[cid[real], 5] + pos[real], cid[real]


def _check_stream(g, policy, eb):
    """eb: bytes per terminal value, 0 for bits."""
    from grammar_compressed_sparse_amd import gcs
    d = g.level0_words(policy)
    ch = d["chunks"].astype(np.int64)
    b0, b1, t0 = ch[:, 2], ch[:, 3], ch[:, 5]
    assert np.all(b0 % 16 == 0) and np.all(b1 % 16 == 0) and np.all(b1 > b0) and np.all(b1 - b0 <= WIN_BYTES)
    assert np.array_equal(t0, b0 // eb if eb else b0 * 8)
    rows, terms, cid = _decode(d)
    st = g.stats()
    assert np.all(rows >= 0) and np.all(rows < st["n_rows"]) and np.all(terms < st["n_terminals"])
    # rows never decrease inside a chunk
    same = cid[1:] == cid[:-1]
    assert np.all(rows[1:][same] >= rows[:-1][same])
    # every terminal inside its chunk's window
    lo = terms * eb if eb else terms >> 3
    hi = lo + eb if eb else lo + 1
    assert np.all(lo >= b0[cid]) and np.all(hi <= b1[cid])
    # one column slice per chunk
    x, row, term = _level0_pairs(g)
    slice_of_term = np.full(st["n_terminals"], -1, np.int64)
    slice_of_term[term] = x
    xs = slice_of_term[terms]
    assert np.all(xs >= 0)
    first = np.ones(cid.size, bool)
    first[1:] = cid[1:] != cid[:-1]
    assert np.array_equal(xs, np.repeat(xs[first], np.diff(np.flatnonzero(np.append(first, True)))))
    # exactly the level-0 pairs of the grammar's groups
    got = np.lexsort((terms, rows))
    want = np.lexsort((term, row))
    assert np.array_equal(rows[got], row[want]) and np.array_equal(terms[got], term[want])
    return d


def _far_rows(seed=77):
    """300,000 rows, about one in 9,000 non-empty (gaps that need skip
    words), 50 adjacent rows sharing 30 columns (rules), and the last row."""
    rng = np.random.default_rng(seed)
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


@pytest.fixture(scope="module")
def graph_grammar(synth_mod):
    from grammar_compressed_sparse_amd import gcs
    spec = synth_mod.GraphSpec(60_000, seed=21)
    rp, col = synth_mod.copy_graph(spec)
    return gcs.build_grammar(rp, col, None, n_cols=spec.n)


@pytest.mark.parametrize("split", [None, "2", "16"])
def test_words_copy_graph(graph_grammar, monkeypatch, split):
    """Boolean, tropical fp32 and fp64 streams of a copy-model graph, with the
    default and forced sub-slice counts."""
    from grammar_compressed_sparse_amd import gcs
    if split is None:
        monkeypatch.delenv("GCS_LEVEL0_SPLIT", raising=False)
    else:
        monkeypatch.setenv("GCS_LEVEL0_SPLIT", split)
    monkeypatch.delenv("GCS_LEVEL0_WINDOW", raising=False)
    for pol, eb in ((gcs.BOOL_OR, 0), (gcs.MIN_PLUS_F32, 4), (gcs.MIN_PLUS_F64, 8)):
        d = graph_grammar.level0_words(pol)
        if d["words"].size == 0:
            # a forced cut too coarse for a 60 KB window of values: no stream
            assert split is not None and eb > 0 and d["n_sub"] == 0
            continue
        _check_stream(graph_grammar, pol, eb)
        if split is not None:
            assert d["n_sub"] == int(split)


def test_words_skip_rows(monkeypatch):
    """Row gaps wider than a word's 13-bit increase are bridged by skip words
    and decode to the same pairs."""
    from grammar_compressed_sparse_amd import gcs
    monkeypatch.delenv("GCS_LEVEL0_SPLIT", raising=False)
    monkeypatch.delenv("GCS_LEVEL0_WINDOW", raising=False)
    n, m, rp, col = _far_rows()
    g = gcs.build_grammar(rp, col, None, n_cols=m)
    d = _check_stream(g, gcs.BOOL_OR, 0)
    w = d["words"].astype(np.int64)
    assert np.any(((w & SKIP) == SKIP) & ((w >> 19) > 0))  # skip words exist
    _check_stream(g, gcs.MIN_PLUS_F64, 8)


def test_words_absent(synth_mod, monkeypatch):
    """No stream for a summing policy, nor with GCS_LEVEL0_WINDOW=0."""
    from grammar_compressed_sparse_amd import gcs
    spec = synth_mod.GENOTYPE_512x4096
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols)
    monkeypatch.delenv("GCS_LEVEL0_SPLIT", raising=False)
    monkeypatch.delenv("GCS_LEVEL0_WINDOW", raising=False)
    for pol in (gcs.PLUS_F32, gcs.PLUS_F64, gcs.PLUS_F32_ACC_F64):
        d = g.level0_words(pol)
        assert d["words"].size == 0 and d["chunks"].shape[0] == 0 and d["n_sub"] == 0
    _check_stream(g, gcs.MIN_PLUS_F64, 8)
    monkeypatch.setenv("GCS_LEVEL0_WINDOW", "0")
    assert g.level0_words(gcs.MIN_PLUS_F64)["words"].size == 0


def test_words_errors(graph_grammar, monkeypatch):
    """Capacities below the counts give GCS_ERANGE and an invalid policy or a
    missing count pointer GCS_EINVAL, nothing written past the capacity."""
    import ctypes
    from grammar_compressed_sparse_amd import gcs
    monkeypatch.delenv("GCS_LEVEL0_SPLIT", raising=False)
    monkeypatch.delenv("GCS_LEVEL0_WINDOW", raising=False)
    d = graph_grammar.level0_words(gcs.BOOL_OR)
    nw, nc = d["words"].size, d["chunks"].shape[0]
    assert nw > 8 and nc > 0
    lib, h = gcs._lib, graph_grammar._h
    cw, cc, cs = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int32(0)
    words = np.full(nw, 0xDEADBEEF, np.uint32)
    chunks = np.zeros((nc, 8), np.int32)
    st = lib.gcs_level0_words(h, gcs.BOOL_OR, words.ctypes.data, nw - 1, None, 0, ctypes.byref(cw), ctypes.byref(cc),
                              ctypes.byref(cs))
    assert st == -4 and cw.value == nw and np.all(words == 0xDEADBEEF)  # GCS_ERANGE, nothing copied
    st = lib.gcs_level0_words(h, gcs.BOOL_OR, None, 0, chunks.ctypes.data, 8 * nc - 1, ctypes.byref(cw),
                              ctypes.byref(cc), None)
    assert st == -4 and cc.value == nc
    assert lib.gcs_level0_words(h, 99, None, 0, None, 0, ctypes.byref(cw), ctypes.byref(cc), None) == -1
    assert lib.gcs_level0_words(h, gcs.BOOL_OR, None, 0, None, 0, None, ctypes.byref(cc), None) == -1
    assert lib.gcs_level0_words(None, gcs.BOOL_OR, None, 0, None, 0, ctypes.byref(cw), ctypes.byref(cc), None) == -1
