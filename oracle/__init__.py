"""CPU oracle for y = M x on the original (uncompressed) matrix.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; the product path never imports it.
It shares no code with the grammar builder or the HIP kernels and never reads
a grammar: it consumes the seeded CSR matrices of
``grammar_compressed_sparse_amd.synth`` (or small hand-written matrices).

Two layers:
  * ``oracle.c`` (built to ``liboracle.so`` with gcc/OpenMP): fp64
    Neumaier-compensated CSR SpMV, exact int64 SpMV, Boolean SpMV and the BFS
    fixpoint.  Page: "Right Multiplication on Grammar-Compressed Matrices"
    (arXiv 2607.24971v1), section 2 (Lemma 2.2 / Theorem 2.3: the sweep
    equals the plain product) and section 5 (Boolean semiring; one pass = one
    frontier expansion).
  * pure-Python references for tiny inputs (exact ``fractions.Fraction``
    dense products, Boolean closure) used to pin the C oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (OpenMP, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
               "-std=c11", "-Wall", "-o", tmp, os.path.join(_HERE, "oracle.c")]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_spmv_f64.argtypes = [I64, P, P, I32, P, P, P, P]
        lib.oracle_spmv_f64_rows.argtypes = [P, I64, P, P, I32, P, P, P, P]
        lib.oracle_spmv_i64.argtypes = [I64, P, P, I32, P, P, P]
        lib.oracle_spmv_bool.argtypes = [I64, P, P, P, P]
        lib.oracle_spmv_min_plus_f32.argtypes = [I64, P, P, I32, P, P, P]
        lib.oracle_spmv_min_plus_f64.argtypes = [I64, P, P, I32, P, P, P]
        lib.oracle_bfs.argtypes = [I64, P, P, P, I64, P, P, I64]
        lib.oracle_bfs.restype = I64
        lib.oracle_num_threads.restype = I32
        lib.oracle_set_threads.argtypes = [I32]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _vals(val):
    """(kind, pointer, keepalive) for the value array: None = all ones."""
    if val is None:
        return 0, None, None
    val = np.asarray(val)
    if val.dtype == np.int8:
        v = np.ascontiguousarray(val)
        return 1, _p(v), v
    v = np.ascontiguousarray(val, dtype=np.float64)
    return 2, _p(v), v


def _csr(row_ptr, col):
    return (np.ascontiguousarray(row_ptr, dtype=np.int64), np.ascontiguousarray(col, dtype=np.int32))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_threads(t: int) -> None:
    _load().oracle_set_threads(int(t))


def spmv_f64(row_ptr, col, val, x):
    """y = M x in fp64 (compensated), plus absum[r] = sum_j |M[r][j] x[j]|."""
    lib = _load()
    rp, cl = _csr(row_ptr, col)
    n = rp.shape[0] - 1
    kind, vp, keep = _vals(val)
    xx = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(n, np.float64)
    a = np.empty(n, np.float64)
    lib.oracle_spmv_f64(n, _p(rp), _p(cl), kind, vp, _p(xx), _p(y), _p(a))
    del keep
    return y, a


def spmv_f64_rows(rows, row_ptr, col, val, x):
    """The same as ``spmv_f64`` restricted to the listed rows (one by one)."""
    lib = _load()
    rp, cl = _csr(row_ptr, col)
    rr = np.ascontiguousarray(rows, dtype=np.int64)
    kind, vp, keep = _vals(val)
    xx = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(rr.shape[0], np.float64)
    a = np.empty(rr.shape[0], np.float64)
    lib.oracle_spmv_f64_rows(_p(rr), rr.shape[0], _p(rp), _p(cl), kind, vp, _p(xx), _p(y), _p(a))
    del keep
    return y, a


def spmv_i64(row_ptr, col, val, x):
    """Exact y = M x over int64 (values all-ones or int8)."""
    lib = _load()
    rp, cl = _csr(row_ptr, col)
    n = rp.shape[0] - 1
    kind, vp, keep = _vals(val)
    if kind == 2:
        raise ValueError("spmv_i64 takes integer matrix values")
    xx = np.ascontiguousarray(x, dtype=np.int64)
    y = np.empty(n, np.int64)
    lib.oracle_spmv_i64(n, _p(rp), _p(cl), kind, vp, _p(xx), _p(y))
    del keep
    return y


def spmv_bool(row_ptr, col, x):
    """y[r] = OR over the stored entries of row r of x[col] (bytes 0/1)."""
    lib = _load()
    rp, cl = _csr(row_ptr, col)
    n = rp.shape[0] - 1
    xx = np.ascontiguousarray(np.asarray(x) != 0, dtype=np.uint8)
    y = np.empty(n, np.uint8)
    lib.oracle_spmv_bool(n, _p(rp), _p(cl), _p(xx), _p(y))
    return y


def spmv_min_plus(row_ptr, col, val, x, dtype=np.float32):
    """Tropical y[r] = min over the stored entries of row r of (M[r][j] + x[j]),
    +inf for an empty row; every addition in ``dtype`` (float32 or float64)."""
    lib = _load()
    rp, cl = _csr(row_ptr, col)
    n = rp.shape[0] - 1
    kind, vp, keep = _vals(val)
    dt = np.dtype(dtype)
    xx = np.ascontiguousarray(x, dtype=dt)
    y = np.empty(n, dt)
    f = lib.oracle_spmv_min_plus_f32 if dt == np.float32 else lib.oracle_spmv_min_plus_f64
    f(n, _p(rp), _p(cl), kind, vp, _p(xx), _p(y))
    del keep
    return y


def bfs(row_ptr, col, sources, max_passes: int = 1 << 20):
    """BFS fixpoint from ``sources``: returns (visited bytes, new-node count per pass)."""
    lib = _load()
    rp, cl = _csr(row_ptr, col)
    n = rp.shape[0] - 1
    src = np.ascontiguousarray(sources, dtype=np.int64)
    vis = np.empty(n, np.uint8)
    counts = np.empty(min(max_passes, n + 2), np.int64)
    passes = lib.oracle_bfs(n, _p(rp), _p(cl), _p(src), src.shape[0], _p(vis), _p(counts),
                            min(max_passes, counts.shape[0]))
    if passes < 0:
        raise RuntimeError("oracle BFS did not reach its fixpoint")
    return vis, counts[:passes].copy()


# ---------------------------------------------------------------------------
# exact references for tiny inputs
# ---------------------------------------------------------------------------

def dense_product_exact(M, x):
    """Exact y = M x with rationals: M is a list of rows, entries exact (int or
    Fraction or float converted exactly); the plain definition of the product."""
    xs = [Fraction(v) for v in x]
    return [sum((Fraction(a) * xs[j] for j, a in enumerate(row) if a != 0), Fraction(0)) for row in M]


def dense_to_csr(M):
    """CSR (row_ptr, col, fp64 values) of a dense list-of-rows matrix."""
    rp, cl, vl = [0], [], []
    for row in M:
        for j, a in enumerate(row):
            if a != 0:
                cl.append(j)
                vl.append(float(a))
        rp.append(len(cl))
    return np.array(rp, np.int64), np.array(cl, np.int32), np.array(vl, np.float64)


def reverse_reachable(adj_rows, sources):
    """Set of nodes with a directed path to some source (Warshall closure of the
    out-list relation, a different algorithm from the frontier iteration)."""
    n = len(adj_rows)
    reach = [[False] * n for _ in range(n)]
    for i, outs in enumerate(adj_rows):
        reach[i][i] = True
        for j in outs:
            reach[i][j] = True
    for k in range(n):
        rk = reach[k]
        for i in range(n):
            if reach[i][k]:
                ri = reach[i]
                for j in range(n):
                    if rk[j]:
                        ri[j] = True
    src = set(int(s) for s in sources)
    return sorted(i for i in range(n) if any(reach[i][s] for s in src))
