"""Python binding of the C ABI in ``include/gcs.h`` (argument marshalling only).

Every step of the product runs in ``libgcs.so``: the host builder (CSRV,
RePair, levels, pass-through completion, layout) and the HIP sweep.  PyTorch
provides device memory (``torch.empty(..., device='cuda')``) and streams.
There is no fallback: if the library is missing, importing this module fails.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import weakref

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_PKG, "libgcs.so")

if not os.path.exists(_SO):
    raise ImportError(f"{_SO} is not built; run __graft_entry__.build() (hipcc for gfx950)")
# torch first: it loads the HIP and HSA runtimes it was built with, and
# libgcs.so (which asks for the same sonames) then binds to those.  Loaded
# the other way round, the process would hold two HIP runtimes, and device
# memory of one is not usable from the other.
import torch as _torch_mod  # noqa: E402,F401

_lib = ctypes.CDLL(_SO)

# policies (gcs_policy)
PLUS_F64, PLUS_F32, PLUS_F32_ACC_F64, BOOL_OR, PLUS_I64, MIN_PLUS_F32, MIN_PLUS_F64 = range(7)
POLICY_NAMES = {"f64": PLUS_F64, "f32": PLUS_F32, "f32_acc_f64": PLUS_F32_ACC_F64, "bool": BOOL_OR, "i64": PLUS_I64,
                "min_plus_f32": MIN_PLUS_F32, "min_plus_f64": MIN_PLUS_F64}
VAL_ONES, VAL_I8, VAL_F64 = 0, 1, 2
PROFILE_LAUNCHES, PROFILE_LEVEL_SPAN = 0, 1  # gcs_profile_mode
BATCH_ACCUMULATE, BATCH_LEAVES_IN_SWEEP = 1, 2  # gcs_sweep_right_batch flags
_STATUS = {0: "GCS_OK", -1: "GCS_EINVAL", -2: "GCS_ENOMEM", -3: "GCS_EHIP", -4: "GCS_ERANGE", -5: "GCS_ESTATE"}


class GcsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class CsrView(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("n_cols", ctypes.c_int64), ("row_ptr", ctypes.c_void_p),
                ("col", ctypes.c_void_p), ("val_kind", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("val", ctypes.c_void_p)]


class BuildOpts(ctypes.Structure):
    _fields_ = [("n_threads", ctypes.c_int32), ("col_chunk", ctypes.c_int32), ("row_chunk", ctypes.c_int32),
                ("row_order", ctypes.c_int32), ("repair", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("n_rows", "n_cols", "nnz", "n_values", "n_terminals", "n_rules",
                                             "n_passthrough", "depth", "max_width", "c_len", "n_tiles",
                                             "n_emit_groups")] + \
               [(n, ctypes.c_double) for n in ("t_csrv_ms", "t_repair_ms", "t_layer_ms")]


class DevSizes(ctypes.Structure):
    _fields_ = [("grammar_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t), ("x_len", ctypes.c_int64),
                ("y_len", ctypes.c_int64), ("x_elem_bytes", ctypes.c_int32), ("y_elem_bytes", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_st = ctypes.c_int
_lib.gcs_last_error.restype = ctypes.c_char_p
_lib.gcs_build_grammar.argtypes = [ctypes.POINTER(CsrView), ctypes.POINTER(BuildOpts), ctypes.POINTER(_P)]
_lib.gcs_grammar_from_rules.argtypes = [_I64, _I64, _P, _I64, _P, _P, _I64, _P, _P, _I64, _P, _P, ctypes.POINTER(_P)]
_lib.gcs_grammar_stats.argtypes = [_P, ctypes.POINTER(Stats)]
_lib.gcs_merge_grammars.argtypes = [ctypes.POINTER(_P), ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_P)]
_lib.gcs_merge_grammars.restype = _st
_lib.gcs_level_widths.argtypes = [_P, _P, _I64]
_lib.gcs_edge_spans.argtypes = [_P, _P, _I64, ctypes.POINTER(_I64)]
_lib.gcs_edge_spans.restype = _st
_lib.gcs_export_grammar.argtypes = [_P] + [_P] * 9
_lib.gcs_layout_counts.argtypes = [_P, _P]
_lib.gcs_export_layout.argtypes = [_P] + [_P] * 6
_lib.gcs_export_slices.argtypes = [_P, _P, _P]
_lib.gcs_export_slices.restype = _st
_lib.gcs_level0_words.argtypes = [_P, ctypes.c_int, _P, _I64, _P, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                                  ctypes.POINTER(ctypes.c_int32)]
_lib.gcs_level0_words.restype = _st
_lib.gcs_save_grammar.argtypes = [_P, ctypes.c_char_p]
_lib.gcs_save_grammar.restype = _st
_lib.gcs_load_grammar.argtypes = [ctypes.c_char_p, ctypes.POINTER(_P)]
_lib.gcs_load_grammar.restype = _st
ROW_SOURCE = ctypes.CFUNCTYPE(ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                              ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64)
_lib.gcs_build_grammar_rows.argtypes = [ROW_SOURCE, _P, _I64, _I64, ctypes.c_int32, ctypes.POINTER(BuildOpts),
                                        ctypes.POINTER(_P)]
_lib.gcs_build_grammar_rows.restype = _st
_lib.gcs_expand_row.argtypes = [_P, _I64, _P, _I64, ctypes.POINTER(_I64)]
_lib.gcs_expand_row.restype = _st
_lib.gcs_build_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)]
_lib.gcs_build_workspace_bytes.restype = _st
_lib.gcs_build_grammar_gpu.argtypes = [ctypes.POINTER(CsrView), ctypes.POINTER(BuildOpts), _I64, _P, ctypes.c_size_t,
                                       _P, ctypes.POINTER(_P)]
_lib.gcs_build_grammar_gpu.restype = _st
_lib.gcs_free_grammar.argtypes = [_P]
_lib.gcs_free_grammar.restype = None
_lib.gcs_device_layout.argtypes = [_P, ctypes.c_int, ctypes.POINTER(DevSizes)]
_lib.gcs_upload.argtypes = [_P, ctypes.c_int, _P, ctypes.c_size_t, _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]
_lib.gcs_sweep_right.argtypes = [_P, _P, _P, _P]
_lib.gcs_sweep_right_acc.argtypes = [_P, _P, _P, _P]
_lib.gcs_bfs.argtypes = [_P, _P, _I64, _P, _P, _P, _P, _I64, ctypes.POINTER(_I64), _P]
_lib.gcs_batch_workspace_bytes.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
_lib.gcs_sweep_right_batch.argtypes = [_P, _P, _P, ctypes.c_int32, _P, ctypes.c_size_t, ctypes.c_int32, _P]
_lib.gcs_sweep_right_batch_scratch.argtypes = [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P]
_lib.gcs_sweep_right_batch_scratch.restype = _st
_lib.gcs_group_layout.argtypes = [ctypes.POINTER(_P), ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
_lib.gcs_group_layout.restype = _st
_lib.gcs_group_create.argtypes = [ctypes.POINTER(_P), ctypes.c_int32, _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]
_lib.gcs_group_create.restype = _st
_lib.gcs_group_sweep_right.argtypes = [_P, _P, _P, ctypes.c_int32, _P]
_lib.gcs_group_sweep_right.restype = _st
_lib.gcs_group_profile_begin.argtypes = [_P, _I64]
_lib.gcs_group_profile_begin.restype = _st
_lib.gcs_group_sweep_right_profiled.argtypes = [_P, _P, _P, ctypes.c_int32, _P]
_lib.gcs_group_sweep_right_profiled.restype = _st
_lib.gcs_group_profile_end.argtypes = [_P, _P, _I64, ctypes.POINTER(_I64)]
_lib.gcs_group_profile_end.restype = _st
_lib.gcs_group_launches.argtypes = [_P]
_lib.gcs_group_launches.restype = _I64
_lib.gcs_group_free.argtypes = [_P]
_lib.gcs_group_free.restype = None
_lib.gcs_sweep_launches.argtypes = [_P]
_lib.gcs_sweep_launches.restype = _I64
_lib.gcs_profile_begin.argtypes = [_P, _I64, ctypes.c_int32]
_lib.gcs_sweep_right_profiled.argtypes = [_P, _P, _P, _P]
_lib.gcs_sweep_right_acc_profiled.argtypes = [_P, _P, _P, _P]
_lib.gcs_sweep_right_acc_profiled.restype = _st
_lib.gcs_profile_end.argtypes = [_P, _P, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
_lib.gcs_device_check.argtypes = [_P, _P]
_lib.gcs_device_check.restype = _st
_lib.gcs_free_device.argtypes = [_P]
_lib.gcs_free_device.restype = None
for _f in ("gcs_build_grammar", "gcs_grammar_from_rules", "gcs_grammar_stats", "gcs_level_widths",
           "gcs_export_grammar", "gcs_layout_counts", "gcs_export_layout", "gcs_device_layout", "gcs_upload",
           "gcs_sweep_right", "gcs_sweep_right_acc", "gcs_bfs", "gcs_profile_begin", "gcs_sweep_right_profiled", "gcs_profile_end",
           "gcs_batch_workspace_bytes", "gcs_sweep_right_batch"):
    getattr(_lib, _f).restype = _st


def _check(status):
    if status != 0:
        raise GcsError(status, (_lib.gcs_last_error() or b"").decode())


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None and a.size else None


def last_error() -> str:
    return (_lib.gcs_last_error() or b"").decode()


def library_path() -> str:
    return _SO


class Grammar:
    """A host grammar owned by the library (``gcs_grammar``)."""

    def __init__(self, handle):
        self._h = handle

    @property
    def handle(self):
        return self._h

    def save(self, path):
        """gcs_save_grammar: write this grammar to ``path`` (load_grammar reads it back)."""
        _check(_lib.gcs_save_grammar(self._h, os.fsencode(path)))

    def stats(self) -> dict:
        s = Stats()
        _check(_lib.gcs_grammar_stats(self._h, ctypes.byref(s)))
        return {n: getattr(s, n) for n, _ in Stats._fields_}

    def level_widths(self) -> np.ndarray:
        L = self.stats()["depth"]
        w = np.zeros(L + 1, np.int64)
        _check(_lib.gcs_level_widths(self._h, _ptr(w), L + 1))
        return w

    def edge_spans(self) -> np.ndarray:
        """gcs_edge_spans: hist[d] = edges rule -> child spanning d levels."""
        L = self.stats()["depth"]
        h = np.zeros(L + 1, np.int64)
        mx = _I64(0)
        _check(_lib.gcs_edge_spans(self._h, _ptr(h), L + 1, ctypes.byref(mx)))
        return h

    def export(self) -> dict:
        s = self.stats()
        a, R, n, C = s["n_terminals"], s["n_rules"], s["n_rows"], s["c_len"]
        out = dict(values=np.zeros(s["n_values"], np.float64), term_col=np.zeros(a, np.int32),
                   term_val=np.zeros(a, np.int32), rule_a=np.zeros(R, np.int32), rule_b=np.zeros(R, np.int32),
                   rule_level=np.zeros(R, np.int32), rule_plast=np.zeros(R, np.int32),
                   c_off=np.zeros(n + 1, np.int64), c_sym=np.zeros(C, np.int32))
        _check(_lib.gcs_export_grammar(self._h, *[_ptr(out[k]) for k in (
            "values", "term_col", "term_val", "rule_a", "rule_b", "rule_level", "rule_plast", "c_off", "c_sym")]))
        return out

    def layout(self) -> dict:
        c = np.zeros(8, np.int64)
        _check(_lib.gcs_layout_counts(self._h, _ptr(c)))
        nl, ncp, nr, ng, ne, arena, ba, bb = (int(v) for v in c)
        out = dict(level_meta=np.zeros((nl, 8), np.int64), child=np.zeros((ncp, 2), np.int32),
                   ptsrc=np.zeros(nr, np.int32), erow=np.zeros(ng, np.int32), eoff=np.zeros(ng + 1, np.int32),
                   epos=np.zeros(ne, np.int32), arena=arena, buf_a=ba, buf_b=bb)
        _check(_lib.gcs_export_layout(self._h, *[_ptr(out[k]) for k in (
            "level_meta", "child", "ptsrc", "erow", "eoff", "epos")]))
        out["slices"] = np.zeros((nl, 3, 9), np.int64)
        out["col_cut"] = np.zeros(9, np.int32)
        _check(_lib.gcs_export_slices(self._h, _ptr(out["slices"]), _ptr(out["col_cut"])))
        return out

    def expand_row(self, r: int) -> np.ndarray:
        """gcs_expand_row: row r's C sequence expanded through R (terminal ids)."""
        n = _I64(0)
        st = _lib.gcs_expand_row(self._h, r, None, 0, ctypes.byref(n))
        if st not in (0, -4):
            _check(st)
        out = np.zeros(n.value, np.int32)
        _check(_lib.gcs_expand_row(self._h, r, _ptr(out), out.size, ctypes.byref(n)))
        return out

    def layout_meta(self) -> dict:
        """level_meta and eoff of the layout only (gcs_export_layout with the
        other arrays skipped): enough to count each level's nodes and roots."""
        c = np.zeros(8, np.int64)
        _check(_lib.gcs_layout_counts(self._h, _ptr(c)))
        nl, ng = int(c[0]), int(c[3])
        out = dict(level_meta=np.zeros((nl, 8), np.int64), eoff=np.zeros(ng + 1, np.int32))
        _check(_lib.gcs_export_layout(self._h, _ptr(out["level_meta"]), None, None, None, _ptr(out["eoff"]), None))
        return out

    def level0_words(self, policy: int) -> dict:
        """gcs_level0_words: level 0's word stream and chunk table as the
        upload for `policy` lays them out (empty arrays when it has none)."""
        nw, nc, ns = _I64(0), _I64(0), ctypes.c_int32(0)
        _check(_lib.gcs_level0_words(self._h, policy, None, 0, None, 0, ctypes.byref(nw), ctypes.byref(nc),
                                     ctypes.byref(ns)))
        words = np.zeros(nw.value, np.uint32)
        chunks = np.zeros((nc.value, 8), np.int32)
        _check(_lib.gcs_level0_words(self._h, policy, _ptr(words), words.size, _ptr(chunks), chunks.size,
                                     ctypes.byref(nw), ctypes.byref(nc), ctypes.byref(ns)))
        return {"words": words, "chunks": chunks, "n_sub": ns.value}

    def device_layout(self, policy: int) -> dict:
        d = DevSizes()
        _check(_lib.gcs_device_layout(self._h, policy, ctypes.byref(d)))
        return {n: getattr(d, n) for n, _ in DevSizes._fields_}

    def free(self):
        if self._h:
            _lib.gcs_free_grammar(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


ROWS_NATURAL, ROWS_SIMILAR = 0, 1
REPAIR_EXACT, REPAIR_ROUNDS = 0, 1  # gcs_repair_mode


def load_grammar(path) -> Grammar:
    """gcs_load_grammar: a grammar saved by Grammar.save."""
    h = _P()
    _check(_lib.gcs_load_grammar(os.fsencode(path), ctypes.byref(h)))
    return Grammar(h)


def _csr_view(row_ptr, col, val, n_cols):
    rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
    cl = np.ascontiguousarray(col, dtype=np.int32)
    n = rp.shape[0] - 1
    if n_cols is None:
        n_cols = int(cl.max()) + 1 if cl.size else 0
    if val is None:
        kind, vv = VAL_ONES, None
    elif np.asarray(val).dtype == np.int8:
        kind, vv = VAL_I8, np.ascontiguousarray(val)
    else:
        kind, vv = VAL_F64, np.ascontiguousarray(val, dtype=np.float64)
    view = CsrView(n, n_cols, rp.ctypes.data, cl.ctypes.data if cl.size else None, kind, 0,
                   vv.ctypes.data if vv is not None and vv.size else None)
    return view, (rp, cl, vv)  # the arrays must outlive the call


def build_grammar(row_ptr, col, val=None, n_cols=None, n_threads=0, col_chunk=0, row_chunk=0,
                  row_order=ROWS_NATURAL, repair=REPAIR_EXACT) -> Grammar:
    """gcs_build_grammar on a host CSR matrix (val: None = all ones, int8, or fp64)."""
    view, keep = _csr_view(row_ptr, col, val, n_cols)
    opts = BuildOpts(n_threads, col_chunk, row_chunk, row_order, repair, 0)
    h = _P()
    _check(_lib.gcs_build_grammar(ctypes.byref(view), ctypes.byref(opts), ctypes.byref(h)))
    return Grammar(h)


def build_grammar_rows(source, n_rows, n_cols, ones=False, n_threads=0, col_chunk=0, row_chunk=0,
                       repair=REPAIR_EXACT) -> Grammar:
    """gcs_build_grammar_rows: the host builder pulling tiles from
    source(row0, nrows, col0, ncols) -> (row_ptr, col, val), a block's CSR
    (row_ptr relative to the block, absolute columns; val ignored when
    ones).  The callback marshals the block into the library's buffers."""
    cache = {}
    err = []

    def cb(ctx, row0, nrows, col0, ncols, rp_p, col_p, val_p, cap):
        try:
            key = (row0, nrows, col0, ncols)
            if key not in cache:
                cache.clear()
                rp, col, val = source(row0, nrows, col0, ncols)
                rp = np.ascontiguousarray(rp, np.int64)
                col = np.ascontiguousarray(col, np.int32)
                val = None if ones or val is None else np.ascontiguousarray(val, np.float64)
                cache[key] = (rp, col, val)
            rp, col, val = cache[key]
            nnz = int(rp[-1]) if rp.size else 0
            if rp_p:
                if cap < nnz:
                    return -1
                ctypes.memmove(rp_p, rp.ctypes.data, rp.nbytes)
                if nnz:
                    ctypes.memmove(col_p, col.ctypes.data, 4 * nnz)
                    if val_p and val is not None:
                        ctypes.memmove(val_p, val.ctypes.data, 8 * nnz)
                cache.clear()
            return nnz
        except Exception as e:  # reported after the call
            err.append(e)
            return -1

    fn = ROW_SOURCE(cb)
    opts = BuildOpts(n_threads, col_chunk, row_chunk, ROWS_NATURAL, repair, 0)
    h = _P()
    st = _lib.gcs_build_grammar_rows(fn, None, n_rows, n_cols, VAL_ONES if ones else VAL_F64, ctypes.byref(opts),
                                     ctypes.byref(h))
    if err:
        raise err[0]
    _check(st)
    return Grammar(h)


def build_workspace_bytes(n_rows, n_cols, nnz, table_entries=0) -> int:
    """gcs_build_workspace_bytes: device bytes gcs_build_grammar_gpu needs."""
    b = ctypes.c_size_t(0)
    _check(_lib.gcs_build_workspace_bytes(n_rows, n_cols, nnz, table_entries, ctypes.byref(b)))
    return int(b.value)


def build_grammar_gpu(row_ptr, col, val=None, n_cols=None, n_threads=0, table_entries=0, workspace=None,
                      device="cuda", stream=None) -> Grammar:
    """gcs_build_grammar_gpu: CSRV and round-based RePair on the device, layout
    on the host.  The workspace is a caller-owned uint8 torch tensor (made
    here unless given, and only needed during the call)."""
    torch = _torch()
    view, keep = _csr_view(row_ptr, col, val, n_cols)
    nnz = int(keep[0][-1]) if keep[0].size else 0
    need = build_workspace_bytes(view.n_rows, view.n_cols, nnz, table_entries)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.numel() < need or not workspace.is_cuda:
        raise GcsError(-1, f"workspace must be a uint8 device tensor of at least {need} bytes")
    opts = BuildOpts(n_threads, 0, 0, ROWS_NATURAL, REPAIR_ROUNDS, 0)
    h = _P()
    with torch.cuda.device(workspace.device):
        _check(_lib.gcs_build_grammar_gpu(ctypes.byref(view), ctypes.byref(opts), table_entries,
                                          ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                          _stream_ptr(stream), ctypes.byref(h)))
    return Grammar(h)


def grammar_from_rules(n_rows, n_cols, values, term_col, term_val, rule_a, rule_b, c_off, c_sym) -> Grammar:
    """gcs_grammar_from_rules: an explicit (C, R, V) grammar."""
    v = np.ascontiguousarray(values, np.float64)
    tc = np.ascontiguousarray(term_col, np.int32)
    tv = np.ascontiguousarray(term_val, np.int32)
    a = np.ascontiguousarray(rule_a, np.int32)
    b = np.ascontiguousarray(rule_b, np.int32)
    co = np.ascontiguousarray(c_off, np.int64)
    cs = np.ascontiguousarray(c_sym, np.int32)
    h = _P()
    _check(_lib.gcs_grammar_from_rules(n_rows, n_cols, _ptr(v), v.size, _ptr(tc), _ptr(tv), tc.size, _ptr(a),
                                       _ptr(b), a.size, _ptr(co), _ptr(cs), ctypes.byref(h)))
    return Grammar(h)


def merge_grammars(parts, n_threads=0) -> Grammar:
    """gcs_merge_grammars: one grammar from grammars of disjoint, increasing
    column groups of the same matrix (the parts stay valid)."""
    hs = (_P * len(parts))(*[p._h for p in parts])
    h = _P()
    _check(_lib.gcs_merge_grammars(hs, len(parts), n_threads, ctypes.byref(h)))
    return Grammar(h)


# ---------------------------------------------------------------------------
# device side (torch supplies memory and streams)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


_X_DTYPES = {PLUS_F64: "float64", PLUS_F32: "float32", PLUS_F32_ACC_F64: "float32", BOOL_OR: "uint8",
             PLUS_I64: "int64", MIN_PLUS_F32: "float32", MIN_PLUS_F64: "float64"}
_Y_DTYPES = {PLUS_F64: "float64", PLUS_F32: "float32", PLUS_F32_ACC_F64: "float64", BOOL_OR: "uint8",
             PLUS_I64: "int64", MIN_PLUS_F32: "float32", MIN_PLUS_F64: "float64"}


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# Device handles still alive when the interpreter exits are freed by an
# atexit hook, registered at the first upload (after torch is imported, so it
# runs before torch's own exit handlers): no HIP call is left for object
# finalization, when the runtime may already be tearing down.
_LIVE = weakref.WeakSet()
_EXIT_HOOK = []


def _release_all():
    for d in list(_LIVE):
        try:
            d.free()
        except Exception:
            pass


class Device:
    """An uploaded grammar (``gcs_device``) plus the torch buffers it lives in."""

    def __init__(self, handle, policy, grammar_buf, workspace, sizes, device):
        if not _EXIT_HOOK:
            atexit.register(_release_all)
            _EXIT_HOOK.append(True)
        _LIVE.add(self)
        self._h = handle
        self.policy = policy
        self.grammar_buf = grammar_buf
        self.workspace = workspace
        self.sizes = sizes
        self.device = device
        torch = _torch()
        self.x_dtype = getattr(torch, _X_DTYPES[policy])
        self.y_dtype = getattr(torch, _Y_DTYPES[policy])

    @property
    def handle(self):
        return self._h

    @property
    def device_bytes(self) -> int:
        return self.grammar_buf.numel() + self.workspace.numel()

    def new_y(self):
        torch = _torch()
        return torch.empty(self.sizes["y_len"], dtype=self.y_dtype, device=self.device)

    def sweep_right(self, x, y=None, stream=None):
        return sweep_right(self, x, y, stream)

    def sweep_right_acc(self, x, y, stream=None):
        return sweep_right_acc(self, x, y, stream)

    def sweep_right_batch(self, X, Y=None, accumulate=False, leaves_in_sweep=False, stream=None):
        return sweep_right_batch(self, X, Y, accumulate, leaves_in_sweep, stream)

    def batch_workspace_bytes(self, nvec: int, leaves_in_sweep=False) -> int:
        n = ctypes.c_size_t(0)
        flags = BATCH_LEAVES_IN_SWEEP if leaves_in_sweep else 0
        _check(_lib.gcs_batch_workspace_bytes(self._h, nvec, flags, ctypes.byref(n)))
        return int(n.value)

    def bfs(self, sources, max_passes=1 << 16, stream=None):
        return bfs(self, sources, max_passes, stream)

    def check(self, stream=None):
        """gcs_device_check: synchronise and raise if a sweep failed on the device."""
        _check(_lib.gcs_device_check(self._h, _stream_ptr(stream)))

    def sweep_launches(self) -> int:
        return int(_lib.gcs_sweep_launches(self._h))

    def profile_begin(self, max_sweeps: int, mode: int = 0):
        """mode PROFILE_LAUNCHES: events around every launch; PROFILE_LEVEL_SPAN:
        one pair around the wide level launches of each sweep."""
        _check(_lib.gcs_profile_begin(self._h, max_sweeps, mode))

    def sweep_right_profiled(self, x, y, stream=None, accumulate=False):
        _check_xy(self, x, y)
        fn = _lib.gcs_sweep_right_acc_profiled if accumulate else _lib.gcs_sweep_right_profiled
        _check(fn(self._h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), _stream_ptr(stream)))
        return y

    def profile_end(self) -> np.ndarray:
        """Durations (ms), shape (sweeps, launches), or (sweeps, 1) for the span mode."""
        cap = 1 << 22
        buf = np.zeros(cap, np.float32)
        ns, nl = _I64(0), _I64(0)
        _check(_lib.gcs_profile_end(self._h, _ptr(buf), cap, ctypes.byref(ns), ctypes.byref(nl)))
        return buf[:ns.value * nl.value].reshape(ns.value, nl.value).copy()

    def free(self):
        if self._h:
            _lib.gcs_free_device(self._h)
            self._h = None
        _LIVE.discard(self)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class Group:
    """Uploads of a matrix's column groups swept as one (``gcs_group``)."""

    def __init__(self, devices, stream=None):
        torch = _torch()
        self.devices = list(devices)  # kept alive while the group lives
        hs = (_P * len(self.devices))(*[d.handle for d in self.devices])
        n = ctypes.c_size_t(0)
        _check(_lib.gcs_group_layout(hs, len(self.devices), ctypes.byref(n)))
        dev = self.devices[0].device
        self.table = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=dev)
        h = _P()
        with torch.cuda.device(dev):
            _check(_lib.gcs_group_create(hs, len(self.devices), ctypes.c_void_p(self.table.data_ptr()),
                                         self.table.numel(), _stream_ptr(stream), ctypes.byref(h)))
        self._h = h
        if not _EXIT_HOOK:
            atexit.register(_release_all)
            _EXIT_HOOK.append(True)
        _LIVE.add(self)

    def sweep_right(self, x, y=None, accumulate=False, stream=None, profiled=False):
        """gcs_group_sweep_right: y = M x (or y += M x) over every group."""
        d0 = self.devices[0]
        if y is None:
            y = d0.new_y()
        _check_xy(d0, x, y)
        torch = _torch()
        fn = _lib.gcs_group_sweep_right_profiled if profiled else _lib.gcs_group_sweep_right
        with torch.cuda.device(d0.device):
            _check(fn(self._h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), int(accumulate),
                      _stream_ptr(stream)))
        return y

    def profile_begin(self, max_sweeps: int):
        _check(_lib.gcs_group_profile_begin(self._h, max_sweeps))

    def profile_end(self) -> np.ndarray:
        """Span (ms) of the level launches of each profiled sweep."""
        buf = np.zeros(1 << 16, np.float32)
        n = _I64(0)
        _check(_lib.gcs_group_profile_end(self._h, _ptr(buf), buf.size, ctypes.byref(n)))
        return buf[:n.value].copy()

    def launches(self) -> int:
        return int(_lib.gcs_group_launches(self._h))

    def free(self):
        if getattr(self, "_h", None):
            _lib.gcs_group_free(self._h)
            self._h = None
        _LIVE.discard(self)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def upload(grammar: Grammar, policy, device="cuda", stream=None, workspace=None) -> Device:
    """gcs_device_layout + caller-owned torch allocations + gcs_upload.
    ``workspace``: a uint8 device tensor to use (and share with other
    uploads whose sweeps are all ordered on one stream) instead of a new one."""
    torch = _torch()
    policy = POLICY_NAMES.get(policy, policy)
    sz = grammar.device_layout(policy)
    dev = torch.device(device)
    if dev.type != "cuda":
        raise GcsError(-1, "upload needs a GPU device")
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    with torch.cuda.device(dev):
        gbuf = torch.empty(max(sz["grammar_bytes"], 256), dtype=torch.uint8, device=dev)
        if workspace is not None:
            if workspace.dtype != torch.uint8 or workspace.numel() < sz["workspace_bytes"] or \
                    workspace.device != dev:
                raise GcsError(-1, f"workspace must be a uint8 tensor of at least {sz['workspace_bytes']} bytes "
                                   f"on {dev}")
            wbuf = workspace
        else:
            wbuf = torch.empty(max(sz["workspace_bytes"], 256), dtype=torch.uint8, device=dev)
        h = _P()
        _check(_lib.gcs_upload(grammar.handle, policy, ctypes.c_void_p(gbuf.data_ptr()), gbuf.numel(),
                               ctypes.c_void_p(wbuf.data_ptr()), wbuf.numel(), _stream_ptr(stream),
                               ctypes.byref(h)))
    return Device(h, policy, gbuf, wbuf, sz, dev)


def _check_xy(dev, x, y):
    if not dev.handle:
        raise GcsError(-5, "device handle already freed")
    if x.dtype != dev.x_dtype or x.numel() != dev.sizes["x_len"] or not x.is_contiguous() or x.device != dev.device:
        raise GcsError(-1, f"x must be a contiguous {dev.x_dtype} tensor of {dev.sizes['x_len']} elements on "
                           f"{dev.device}")
    if y.dtype != dev.y_dtype or y.numel() != dev.sizes["y_len"] or not y.is_contiguous() or y.device != dev.device:
        raise GcsError(-1, f"y must be a contiguous {dev.y_dtype} tensor of {dev.sizes['y_len']} elements")


def sweep_right(dev: Device, x, y=None, stream=None):
    """gcs_sweep_right: y = M x on the device (async on the stream)."""
    if y is None:
        y = dev.new_y()
    _check_xy(dev, x, y)
    torch = _torch()
    with torch.cuda.device(dev.device):
        _check(_lib.gcs_sweep_right(dev.handle, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                    _stream_ptr(stream)))
    return y


def sweep_right_acc(dev: Device, x, y, stream=None):
    """gcs_sweep_right_acc: y (+)= M x on the device (async on the stream)."""
    _check_xy(dev, x, y)
    torch = _torch()
    with torch.cuda.device(dev.device):
        _check(_lib.gcs_sweep_right_acc(dev.handle, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                        _stream_ptr(stream)))
    return y


def sweep_right_batch(dev: Device, X, Y=None, accumulate=False, leaves_in_sweep=False, stream=None):
    """gcs_sweep_right_batch: Y = M X (or Y (+)= M X) for X of shape (x_len, B),
    B in 1..64, row-major; with leaves_in_sweep no terminal array is kept.  The
    batch workspace is a torch buffer kept on the device object (one per B and
    mode) and reused by later calls."""
    torch = _torch()
    if not dev.handle:
        raise GcsError(-5, "device handle already freed")
    if X.dim() != 2 or X.shape[0] != dev.sizes["x_len"] or X.dtype != dev.x_dtype or not X.is_contiguous() \
            or X.device != dev.device:
        raise GcsError(-1, f"X must be a contiguous {dev.x_dtype} tensor of shape ({dev.sizes['x_len']}, B) on "
                           f"{dev.device}")
    B = int(X.shape[1])
    if Y is None:
        Y = torch.empty((dev.sizes["y_len"], B), dtype=dev.y_dtype, device=dev.device)
    if tuple(Y.shape) != (dev.sizes["y_len"], B) or Y.dtype != dev.y_dtype or not Y.is_contiguous() \
            or Y.device != dev.device:
        raise GcsError(-1, f"Y must be a contiguous {dev.y_dtype} tensor of shape ({dev.sizes['y_len']}, {B})")
    flags = (BATCH_ACCUMULATE if accumulate else 0) | (BATCH_LEAVES_IN_SWEEP if leaves_in_sweep else 0)
    ws = dev.__dict__.setdefault("_batch_ws", {})
    key = (B, bool(leaves_in_sweep))
    if key not in ws:
        ws[key] = torch.empty(max(dev.batch_workspace_bytes(B, leaves_in_sweep), 1), dtype=torch.uint8,
                              device=dev.device)
    w = ws[key]
    with torch.cuda.device(dev.device):
        _check(_lib.gcs_sweep_right_batch(dev.handle, ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(Y.data_ptr()),
                                          B, ctypes.c_void_p(w.data_ptr()), w.numel(), flags, _stream_ptr(stream)))
    return Y


def sweep_right_batch_scratch(dev: Device, X, Y=None, accumulate=False, leaves_in_sweep=False, stream=None):
    """gcs_sweep_right_batch_scratch: Y = M X with the library's fixed 64 MiB
    scratch as the batch workspace (no allocation in the library; Y is made
    here only when not given)."""
    torch = _torch()
    if not dev.handle:
        raise GcsError(-5, "device handle already freed")
    if X.dim() != 2 or X.shape[0] != dev.sizes["x_len"] or X.dtype != dev.x_dtype or not X.is_contiguous() \
            or X.device != dev.device:
        raise GcsError(-1, f"X must be a contiguous {dev.x_dtype} tensor of shape ({dev.sizes['x_len']}, B) on "
                           f"{dev.device}")
    B = int(X.shape[1])
    if Y is None:
        Y = torch.empty((dev.sizes["y_len"], B), dtype=dev.y_dtype, device=dev.device)
    if tuple(Y.shape) != (dev.sizes["y_len"], B) or Y.dtype != dev.y_dtype or not Y.is_contiguous() \
            or Y.device != dev.device:
        raise GcsError(-1, f"Y must be a contiguous {dev.y_dtype} tensor of shape ({dev.sizes['y_len']}, {B})")
    flags = (BATCH_ACCUMULATE if accumulate else 0) | (BATCH_LEAVES_IN_SWEEP if leaves_in_sweep else 0)
    with torch.cuda.device(dev.device):
        _check(_lib.gcs_sweep_right_batch_scratch(dev.handle, ctypes.c_void_p(X.data_ptr()),
                                                  ctypes.c_void_p(Y.data_ptr()), B, flags, _stream_ptr(stream)))
    return Y


def bfs(dev: Device, sources, max_passes=1 << 16, stream=None):
    """gcs_bfs: BFS fixpoint from ``sources``; returns (visited uint8 tensor, counts)."""
    torch = _torch()
    n = dev.sizes["y_len"]
    srcs = np.asarray(sources, np.int64)
    if srcs.size and (srcs.min() < 0 or srcs.max() >= n):
        raise GcsError(-1, "BFS source outside [0, n)")
    with torch.cuda.device(dev.device):
        src = torch.as_tensor(srcs).to(dev.device)
        f = torch.empty(n, dtype=torch.uint8, device=dev.device)
        vis = torch.empty(n, dtype=torch.uint8, device=dev.device)
        y = torch.empty(n, dtype=torch.uint8, device=dev.device)
        counts = np.zeros(max_passes, np.int64)
        passes = ctypes.c_int64(0)
        _check(_lib.gcs_bfs(dev.handle, ctypes.c_void_p(src.data_ptr()) if src.numel() else None, src.numel(),
                            ctypes.c_void_p(f.data_ptr()), ctypes.c_void_p(vis.data_ptr()),
                            ctypes.c_void_p(y.data_ptr()), _ptr(counts), max_passes, ctypes.byref(passes),
                            _stream_ptr(stream)))
    return vis, counts[:passes.value].copy()
