"""Pins for the CPU oracle, against facts the pages and the mathematics fix.

* the worked example: matrix of Eq. (2.1), x and root values of Figure 4.2,
  row roots of Eq. (2.4) (page "Right Multiplication on Grammar-Compressed
  Matrices", section 2 and Figure 4.2);
* exact rational dense products on small random matrices (non-square, so a
  transposed operand fails), with every entry and x exact;
* compensated summation on sums where plain fp64 summation loses the answer;
* closed forms: x = ones gives row sums, x = e_j gives column j;
* Boolean and int64 products against brute force; the BFS fixpoint against a
  Warshall closure (a different algorithm) and a path graph whose pass count
  is known in closed form.
"""
import random
from fractions import Fraction

import numpy as np
import pytest

U = 2.0 ** -53


def _we_dense(we):
    return we["M"]["rows"], we["x"]["values"]


def test_worked_example(oracle_mod, worked_example):
    rows, x = _we_dense(worked_example)
    rp, col, val = oracle_mod.dense_to_csr(rows)
    y, absum = oracle_mod.spmv_f64(rp, col, val, x)
    roots = worked_example["C"]["row_roots"]
    rv = worked_example["root_values"]
    expect = np.array([rv["N%d" % r] for r in roots])
    assert np.all(np.abs(y - expect) <= 1e-12 * absum)
    # the same rows agree with the exact rational product of Eq. (2.1) and x
    exact = oracle_mod.dense_product_exact(rows, x)
    for yi, ei in zip(y, exact):
        assert abs(Fraction(yi) - ei) <= Fraction(4 * U) * abs(ei)


def _random_dense(rng, n, m, density, kind):
    M = []
    for _ in range(n):
        row = []
        for _ in range(m):
            if rng.random() < density:
                if kind == "int":
                    row.append(rng.choice([1, 2, -3, 7]))
                else:
                    row.append(rng.uniform(-4, 4))
            else:
                row.append(0)
        M.append(row)
    return M


@pytest.mark.parametrize("n,m,density", [(1, 1, 1.0), (5, 17, 0.4), (17, 5, 0.6), (40, 64, 0.3), (64, 3, 0.9),
                                         (9, 30, 0.0)])
def test_dense_exact(oracle_mod, n, m, density):
    rng = random.Random(n * 1000 + m)
    M = _random_dense(rng, n, m, density, "float")
    x = [rng.uniform(-2, 2) for _ in range(m)]
    rp, col, val = oracle_mod.dense_to_csr(M)
    y, absum = oracle_mod.spmv_f64(rp, col, val, x)
    exact = oracle_mod.dense_product_exact(M, x)
    for r in range(n):
        a = sum(abs(Fraction(M[r][j]) * Fraction(x[j])) for j in range(m))
        assert abs(Fraction(y[r]) - exact[r]) <= Fraction(3 * U) * a + Fraction(2 * U) * abs(exact[r])
        assert abs(absum[r] - float(a)) <= 1e-12 * float(a)
    # the row-sampled entry point returns the same rows one by one
    rows = np.arange(n)[::-1].copy()
    ys, _ = oracle_mod.spmv_f64_rows(rows, rp, col, val, x)
    assert np.array_equal(ys, y[rows])


def test_compensated_sum(oracle_mod):
    # plain left-to-right fp64 summation returns 0.0 for both rows
    rows = [[1e16, 1.0, -1e16], [1.0, 1e100, 1.0, -1e100]]
    rp = np.array([0, 3, 7], np.int64)
    col = np.array([0, 1, 2, 0, 1, 2, 3], np.int32)
    val = np.array(rows[0] + rows[1], np.float64)
    y, _ = oracle_mod.spmv_f64(rp, col, val, np.ones(4))
    assert y[0] == 1.0 and y[1] == 2.0


def test_closed_forms_genotype(oracle_mod, synth_mod):
    rp, col, val = synth_mod.genotype(synth_mod.GENOTYPE_512x4096)
    n, m = 512, 4096
    # x = ones: y = row sums of the stored genotype values (exact integers)
    y, _ = oracle_mod.spmv_f64(rp, col, val, np.ones(m))
    sums = np.add.reduceat(val.astype(np.int64), rp[:-1]) * (np.diff(rp) > 0)
    assert np.array_equal(y, sums.astype(np.float64))
    # x = e_j: y = column j
    import scipy.sparse as sp
    A = sp.csr_matrix((val.astype(np.float64), col, rp), shape=(n, m)).toarray()
    for j in (0, 1, 777, m - 1):
        e = np.zeros(m)
        e[j] = 1.0
        y, _ = oracle_mod.spmv_f64(rp, col, val, e)
        assert np.array_equal(y, A[:, j])
    yi = oracle_mod.spmv_i64(rp, col, val, np.arange(m, dtype=np.int64) - 2000)
    assert np.array_equal(yi, A.astype(np.int64) @ (np.arange(m, dtype=np.int64) - 2000))


def test_bool_and_int_brute_force(oracle_mod):
    rng = random.Random(7)
    for n, m in [(1, 1), (13, 29), (50, 50), (7, 1)]:
        M = _random_dense(rng, n, m, 0.2, "int")
        rp, col, _ = oracle_mod.dense_to_csr(M)
        x = [rng.random() < 0.3 for _ in range(m)]
        yb = oracle_mod.spmv_bool(rp, col, np.array(x, np.uint8))
        for r in range(n):
            assert yb[r] == any(M[r][j] != 0 and x[j] for j in range(m))
        vi = np.array([M[r][j] for r in range(n) for j in range(m) if M[r][j] != 0], np.int8)
        xi = [rng.randrange(-1000, 1000) for _ in range(m)]
        yi = oracle_mod.spmv_i64(rp, col, vi, np.array(xi, np.int64))
        for r in range(n):
            assert yi[r] == sum(M[r][j] * xi[j] for j in range(m))


def test_bfs_path_closed_form(oracle_mod):
    # out-list of node i is {i+1}: every node reaches n-1, one new node per pass
    n = 40
    rp = np.arange(n + 1, dtype=np.int64).clip(max=n - 1)
    col = np.arange(1, n, dtype=np.int32)
    vis, counts = oracle_mod.bfs(rp, col, [n - 1])
    assert vis.all()
    assert list(counts) == [1] * (n - 1) + [0]


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_bfs_vs_warshall(oracle_mod, seed):
    rng = random.Random(seed)
    n = 45
    adj = [sorted(rng.sample(range(n), rng.choice([0, 1, 1, 2, 3]))) for _ in range(n)]
    rp = np.zeros(n + 1, np.int64)
    rp[1:] = np.cumsum([len(a) for a in adj])
    col = np.array([j for a in adj for j in a], np.int32)
    srcs = rng.sample(range(n), 3)
    vis, counts = oracle_mod.bfs(rp, col, srcs)
    assert sorted(np.nonzero(vis)[0].tolist()) == oracle_mod.reverse_reachable(adj, srcs)
    assert counts[-1] == 0 and counts.sum() + len(srcs) == vis.sum()


def _random_csr(rng, n, m, p_row_empty=0.2, max_deg=6):
    rows = []
    for _ in range(n):
        k = 0 if rng.random() < p_row_empty else rng.randint(1, max_deg)
        rows.append(sorted(rng.sample(range(m), min(k, m))))
    rp = np.zeros(n + 1, np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    col = np.array([j for r in rows for j in r], np.int32)
    return rows, rp, col


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_min_plus_brute_force(oracle_mod, seed):
    """Tropical pass written out term by term (section 5: combine = min,
    leaf = value + x[j], identity +inf), in fp64 (Python floats) and in fp32
    (numpy float32 scalars), against the oracle: bit-exact."""
    rng = random.Random(seed)
    n, m = 37, 23
    rows, rp, col = _random_csr(rng, n, m)
    val = np.array([rng.choice([-2.5, -1.0, 0.0, 0.125, 1.0, 3.75, 1e-3, 7.0]) for _ in range(col.size)])
    x = [rng.uniform(-5, 5) for _ in range(m)]
    y64 = oracle_mod.spmv_min_plus(rp, col, val, np.array(x), np.float64)
    y32 = oracle_mod.spmv_min_plus(rp, col, val, np.array(x, np.float32), np.float32)
    k = 0
    for r, cols in enumerate(rows):
        best64, best32 = float("inf"), np.float32(np.inf)
        for j in cols:
            t64 = float(val[k]) + x[j]
            t32 = np.float32(val[k]) + np.float32(x[j])
            best64 = t64 if t64 < best64 else best64
            best32 = t32 if t32 < best32 else best32
            k += 1
        assert y64[r] == best64
        assert y32[r] == best32 and y32.dtype == np.float32


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_min_plus_path_distances(oracle_mod, dtype):
    """Relaxing to the fixpoint on a path (out-list of i is {i+1}, unit
    weights) from node n-1 gives the closed-form distance n-1-i."""
    n = 30
    rp = np.arange(n + 1, dtype=np.int64).clip(max=n - 1)
    col = np.arange(1, n, dtype=np.int32)
    d = np.full(n, np.inf, dtype)
    d[n - 1] = 0.0
    for _ in range(n):
        d = np.minimum(d, oracle_mod.spmv_min_plus(rp, col, None, d, dtype))
    assert d.dtype == dtype
    assert np.array_equal(d, np.arange(n - 1, -1, -1, dtype=dtype))


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_min_plus_reduces_to_boolean(oracle_mod, dtype):
    """With zero weights and x in {0, +inf}, y[r] = 0 exactly where the
    Boolean pass of (x == 0) is 1, +inf elsewhere (empty rows included)."""
    rng = random.Random(9)
    n, m = 60, 40
    rows, rp, col = _random_csr(rng, n, m)
    xb = np.array([rng.random() < 0.3 for _ in range(m)], np.uint8)
    x = np.where(xb == 1, 0.0, np.inf).astype(dtype)
    y = oracle_mod.spmv_min_plus(rp, col, np.zeros(col.size), x, dtype)
    yb = oracle_mod.spmv_bool(rp, col, xb)
    assert np.array_equal(y == 0.0, yb == 1)
    assert np.all(np.isinf(y[yb == 0]))


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_min_plus_fixpoint_is_shortest_paths(oracle_mod, dtype):
    """Bellman-Ford from the tropical pass (d <- min(d, M d), section 5) on a
    random digraph with integer weights 1..9 equals scipy's Dijkstra
    distances to the source set (the row of i lists its out-edges, so d[i]
    is the distance from i to a source); integer sums below 2^24 are exact
    in fp32 too."""
    from scipy.sparse import csr_matrix
    from scipy.sparse.csgraph import shortest_path
    rng = random.Random(21)
    n = 120
    rows, rp, col = _random_csr(rng, n, n)
    w = np.array([rng.randint(1, 9) for _ in range(col.size)], np.float64)
    srcs = [3, 50, 97]
    d = np.full(n, np.inf, dtype)
    d[srcs] = 0
    for _ in range(n):
        nd = np.minimum(d, oracle_mod.spmv_min_plus(rp, col, w, d, dtype))
        if np.array_equal(nd, d):
            break
        d = nd
    A = csr_matrix((w, col, rp), shape=(n, n))
    ref = shortest_path(A.T.tocsr(), method="D", directed=True, indices=srcs).min(axis=0)
    assert np.array_equal(d.astype(np.float64), ref)
    assert np.isfinite(ref).sum() > n // 2  # the pin covers most nodes
