"""Seeded synthetic inputs shared by the oracle and the grammar path.

Holds random number generation and CSR layout only (``synth.c``), none of the
grammar method's arithmetic.  Matrices come back as CSR: ``row_ptr`` int64
(n+1), ``col`` int32 (sorted, distinct per row), ``val`` int8 (genotypes) or
``None`` (Boolean graphs, every stored entry is 1).

Workload recipes (sizes and model parameters of the five benchmark inputs):

* genotype mosaic: each individual is the sum of two haplotypes; a haplotype
  is a mosaic of F founder haplotypes with geometric segment lengths of mean
  S, each segment's founder uniform over the F founders, plus independent
  per-site flips with probability mu.  Founder alleles at site j are
  Bernoulli(q_j) with q_j the folded (minor-allele) Beta(1/2, 1/2) frequency.
* copy-model digraph: node i draws a lognormal out-degree (mean 20, sigma 1),
  copies a window of a uniformly chosen earlier node's sorted out-list,
  replaces each copied entry with probability 0.05 by a uniform target, and
  sorts/de-duplicates.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libgcs_synth.so")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", "-std=gnu11",
               "-Wall", "-o", tmp, os.path.join(_HERE, "synth.c"), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


class _Geno(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("n_cols", ctypes.c_int64), ("founders", ctypes.c_int32),
                ("pad_", ctypes.c_int32), ("seg_mean", ctypes.c_double), ("mu", ctypes.c_double),
                ("seed", ctypes.c_uint64)]


class _Graph(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("mean_deg", ctypes.c_double), ("sigma", ctypes.c_double),
                ("p_replace", ctypes.c_double), ("seed", ctypes.c_uint64)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        lib.synth_genotype_block.argtypes = [ctypes.POINTER(_Geno), I64, I64, I64, I64, P, P, P, P]
        lib.synth_genotype_block.restype = ctypes.c_int
        lib.synth_site_maf.argtypes = [ctypes.POINTER(_Geno), I64]
        lib.synth_site_maf.restype = ctypes.c_double
        lib.synth_graph_degree.argtypes = [ctypes.POINTER(_Graph), I64]
        lib.synth_graph_degree.restype = I64
        lib.synth_graph_degree_sum.argtypes = [ctypes.POINTER(_Graph)]
        lib.synth_graph_degree_sum.restype = I64
        lib.synth_copy_graph.argtypes = [ctypes.POINTER(_Graph), P, P, I64]
        lib.synth_copy_graph.restype = I64
        lib.synth_normal_f64.argtypes = [I64, ctypes.c_uint64, P]
        lib.synth_sources.argtypes = [I64, I64, ctypes.c_uint64, P]
        lib.synth_sources.restype = I64
        lib.synth_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


@dataclass(frozen=True)
class GenotypeSpec:
    n_rows: int
    n_cols: int
    founders: int
    seg_mean: float
    mu: float
    seed: int

    def _c(self):
        return _Geno(self.n_rows, self.n_cols, self.founders, 0, float(self.seg_mean), float(self.mu),
                     self.seed & 0xFFFFFFFFFFFFFFFF)


@dataclass(frozen=True)
class GraphSpec:
    n: int
    mean_deg: float = 20.0
    sigma: float = 1.0
    p_replace: float = 0.05
    seed: int = 5

    def _c(self):
        return _Graph(self.n, float(self.mean_deg), float(self.sigma), float(self.p_replace),
                      self.seed & 0xFFFFFFFFFFFFFFFF)


def genotype(spec: GenotypeSpec, row0: int = 0, nrows: int | None = None, col0: int = 0,
             ncols: int | None = None):
    """CSR block of the genotype matrix: rows [row0, row0+nrows), columns
    [col0, col0+ncols) (absolute column indices).  Returns (row_ptr, col, val)."""
    lib = _load()
    nrows = spec.n_rows - row0 if nrows is None else nrows
    ncols = spec.n_cols - col0 if ncols is None else ncols
    if not (0 <= row0 and row0 + nrows <= spec.n_rows and 0 <= col0 and col0 + ncols <= spec.n_cols):
        raise ValueError("block outside the matrix")
    P = spec._c()
    cnt = np.zeros(max(nrows, 1), np.int64)
    if lib.synth_genotype_block(ctypes.byref(P), row0, nrows, col0, ncols, _p(cnt), None, None, None):
        raise MemoryError("genotype generator: allocation failed")
    row_ptr = np.zeros(nrows + 1, np.int64)
    np.cumsum(cnt[:nrows], out=row_ptr[1:])
    nnz = int(row_ptr[-1])
    col = np.empty(max(nnz, 1), np.int32)
    val = np.empty(max(nnz, 1), np.int8)
    if lib.synth_genotype_block(ctypes.byref(P), row0, nrows, col0, ncols, None, _p(row_ptr), _p(col), _p(val)):
        raise MemoryError("genotype generator: allocation failed")
    return row_ptr, col[:nnz], val[:nnz]


def site_maf(spec: GenotypeSpec, j: int) -> float:
    return float(_load().synth_site_maf(ctypes.byref(spec._c()), j))


def graph_degree(spec: GraphSpec, i: int) -> int:
    return int(_load().synth_graph_degree(ctypes.byref(spec._c()), i))


def copy_graph(spec: GraphSpec):
    """Copy-model digraph as CSR out-lists: (row_ptr, col); square n x n."""
    lib = _load()
    G = spec._c()
    cap = int(lib.synth_graph_degree_sum(ctypes.byref(G)))
    row_ptr = np.empty(spec.n + 1, np.int64)
    col = np.empty(max(cap, 1), np.int32)
    nnz = int(lib.synth_copy_graph(ctypes.byref(G), _p(row_ptr), _p(col), cap))
    if nnz < 0:
        raise RuntimeError("copy-model generator: capacity exceeded")
    if nnz < col.shape[0] // 2:
        col = col[:nnz].copy()
    return row_ptr, col[:nnz]


def normal(n: int, seed: int) -> np.ndarray:
    """n independent N(0,1) draws (fp64), Box-Muller on counter-based uniforms."""
    out = np.empty(max(n, 1), np.float64)
    _load().synth_normal_f64(n, seed & 0xFFFFFFFFFFFFFFFF, _p(out))
    return out[:n]


def sources(n: int, k: int, seed: int) -> np.ndarray:
    out = np.empty(max(k, 1), np.int64)
    if _load().synth_sources(n, k, seed & 0xFFFFFFFFFFFFFFFF, _p(out)) < 0:
        raise ValueError("more sources than nodes")
    return out[:k]


def num_threads() -> int:
    return int(_load().synth_num_threads())


# ---------------------------------------------------------------------------
# the benchmark workloads
# ---------------------------------------------------------------------------

GENOTYPE_512x4096 = GenotypeSpec(512, 4096, 16, 200.0, 0.005, seed=1)
GENOTYPE_20000x100000 = GenotypeSpec(20_000, 100_000, 64, 500.0, 0.001, seed=2)
GENOTYPE_200000x2000000 = GenotypeSpec(200_000, 2_000_000, 256, 1000.0, 0.0005, seed=4)
COPY_GRAPH_50M = GraphSpec(50_000_000, 20.0, 1.0, 0.05, seed=5)

# (matrix spec, weight-vector seeds) per workload
WORKLOADS = {
    "genotype_512x4096_f64": dict(matrix=GENOTYPE_512x4096, x_seeds=[101], dtype="f64"),
    "genotype_20000x100000_f32": dict(matrix=GENOTYPE_20000x100000, x_seeds=[201], dtype="f32"),
    "genotype_20000x100000_f32_x32": dict(matrix=GENOTYPE_20000x100000, x_seeds=list(range(301, 333)),
                                          dtype="f32"),
    "genotype_200000x2000000_f32": dict(matrix=GENOTYPE_200000x2000000, x_seeds=[401], dtype="f32"),
    "copy_graph_50M_bfs16": dict(matrix=COPY_GRAPH_50M, source_seed=501, n_sources=16, dtype="u8"),
}
