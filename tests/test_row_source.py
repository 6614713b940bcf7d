"""gcs_build_grammar_rows (the host builder pulling tiles from a row source,
section 2 'CSRV': the string is built row by row) and gcs_expand_row
(Lemma 2.2: a row's roots expand to its CSRV row), through the C ABI."""
import numpy as np
import pytest

import helpers as H


@pytest.fixture(scope="module")
def gcs():
    from grammar_compressed_sparse_amd import gcs as mod
    return mod


def _block(rp, col, val, row0, nrows, col0, ncols):
    """CSR of a block of a CSR matrix (row_ptr relative, absolute columns)."""
    out_rp = [0]
    cols, vals = [], []
    for r in range(row0, row0 + nrows):
        s, e = rp[r], rp[r + 1]
        c = col[s:e]
        m = (c >= col0) & (c < col0 + ncols)
        cols.append(c[m])
        vals.append(val[s:e][m] if val is not None else np.ones(int(m.sum())))
        out_rp.append(out_rp[-1] + int(m.sum()))
    return (np.array(out_rp, np.int64), np.concatenate(cols) if cols else np.zeros(0, np.int32),
            np.concatenate(vals) if vals else np.zeros(0))


@pytest.mark.parametrize("repair", [0, 1], ids=["exact", "rounds"])
@pytest.mark.parametrize("chunks", [(0, 0), (700, 128)])
def test_row_source_equals_csr_build(gcs, synth_mod, repair, chunks):
    spec = synth_mod.GenotypeSpec(300, 3000, 8, 100.0, 0.005, seed=3)
    rp, col, val = synth_mod.genotype(spec)
    cc, rc = chunks
    calls = []

    def source(row0, nrows, col0, ncols):
        calls.append((row0, nrows, col0, ncols))
        # regenerated from the seeded generator, block by block
        return synth_mod.genotype(spec, row0=row0, nrows=nrows, col0=col0, ncols=ncols)

    gs = gcs.build_grammar_rows(source, spec.n_rows, spec.n_cols, col_chunk=cc, row_chunk=rc, repair=repair,
                                n_threads=4)
    gc = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols, col_chunk=cc, row_chunk=rc, repair=repair,
                           n_threads=4)
    es, ec = gs.export(), gc.export()
    for k in ec:
        assert np.array_equal(es[k], ec[k]), k
    ls, lc = gs.layout(), gc.layout()
    for k in ("level_meta", "child", "ptsrc", "erow", "eoff", "epos"):
        assert np.array_equal(ls[k], lc[k]), k
    ntiles = gs.stats()["n_tiles"]
    assert len(set(calls)) == ntiles  # every tile pulled, none assembled whole (unless one tile)


def test_row_source_many_values_and_zeros(gcs):
    rng = np.random.default_rng(4)
    n, m = 60, 80
    dense = rng.integers(0, 3, (n, m)) * rng.choice(np.arange(1, 90) / 8.0, (n, m))  # > 64 values, zeros
    dense[rng.random((n, m)) < 0.3] = 0
    rp, col, val = H.csr_from_dense(dense.tolist())
    val = np.asarray(val, np.float64)
    val[::7] = 0.0  # stored zeros, dropped by CSRV

    def source(row0, nrows, col0, ncols):
        return _block(rp, col, val, row0, nrows, col0, ncols)

    gs = gcs.build_grammar_rows(source, n, m, col_chunk=30, row_chunk=25)
    gc = gcs.build_grammar(rp, col, val, n_cols=m, col_chunk=30, row_chunk=25)
    assert gc.stats()["n_values"] > 64
    es, ec = gs.export(), gc.export()
    for k in ec:
        assert np.array_equal(es[k], ec[k]), k


def test_row_source_errors(gcs):
    import ctypes
    # a source that reports failure (negative count): GCS_EINVAL, no grammar
    fail = gcs.ROW_SOURCE(lambda *a: -3)
    h = ctypes.c_void_p()
    st = gcs._lib.gcs_build_grammar_rows(fail, None, 5, 5, gcs.VAL_ONES, None, ctypes.byref(h))
    assert st == -1 and not h.value and "source" in gcs.last_error()
    # a source whose second answer differs from its first
    calls = []

    def fickle(ctx, r0, nr, c0, nc, rp, col, val, cap):
        calls.append(1)
        if rp:
            ctypes.memmove(rp, np.zeros(nr + 1, np.int64).ctypes.data, 8 * (nr + 1))
            return 0
        return 2
    st = gcs._lib.gcs_build_grammar_rows(gcs.ROW_SOURCE(fickle), None, 3, 3, gcs.VAL_ONES, None, ctypes.byref(h))
    assert st == -1 and len(calls) == 2
    with pytest.raises(gcs.GcsError, match="EINVAL"):  # a column outside the block
        gcs.build_grammar_rows(lambda r0, nr, c0, nc: (np.array([0] + [1] * nr, np.int64)[:nr + 1],
                                                       np.array([c0 + nc], np.int32), None),
                               3, 10, ones=True)


def test_row_source_error_propagates_exception(gcs):
    def bad(r0, nr, c0, nc):
        raise RuntimeError("source broke")
    with pytest.raises(RuntimeError, match="source broke"):
        gcs.build_grammar_rows(bad, 4, 4)


def test_expand_row_is_the_csrv_row(gcs, synth_mod, worked_example):
    """Every row expands to its CSRV string (terminal ids in column order)."""
    spec = synth_mod.GenotypeSpec(120, 900, 6, 60.0, 0.01, seed=5)
    rp, col, val = synth_mod.genotype(spec)
    for repair in (0, 1):
        g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols, repair=repair)
        ex = g.export()
        want = H.csrv_rows(rp, col, val, ex)
        for r in range(spec.n_rows):
            assert g.expand_row(r).tolist() == list(want[r])
    # the pages' worked example: row 1 (N9) and row 2 (N8), Eq. 2.1 / Eq. 2.4
    g = gcs.grammar_from_rules(**H.we_grammar_arrays(worked_example))
    ex = g.export()
    for r in range(8):
        terms = g.expand_row(r)
        cols = ex["term_col"][terms]
        assert np.all(np.diff(cols) > 0)
    with pytest.raises(gcs.GcsError, match="EINVAL"):
        g.expand_row(8)
