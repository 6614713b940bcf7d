"""Matrices too large for one grammar build, as independent column groups.

Page "Right Multiplication on Grammar-Compressed Matrices" (arXiv
2607.24971v1), section 4.4: the engine is built per column chunk.  A terminal
carries its column, so no rule of one group references another group's
terminals: each group of consecutive columns is a grammar of its own, and the
product is the sum (OR, min) of the groups' products.

Each group is built by the device builder (gcs_build_grammar_gpu), uploaded,
and its host grammar dropped; all groups stay resident.  For the plus-times
policies the groups are then swept together (gcs_group_*): one launch per
level covers that level of every group, each group with its own workspace.
Otherwise a sweep runs gcs_sweep_right on the first group and
gcs_sweep_right_acc on every other one into the same y, all on one stream,
so the groups share one workspace (value arena and counters; see
gcs_upload).  Building overlaps across a few worker
threads, each with its own build workspace and stream: while one worker's
group is in the device rounds, others generate their CSR or lay out their
grammar on the host (the library calls release the GIL).

This module only schedules library calls; every step of building and sweeping
runs in libgcs.
"""
from __future__ import annotations

import threading
import time
from concurrent.futures import ThreadPoolExecutor

from . import gcs


class ColumnGroups:
    """Resident column groups of one matrix (see build_column_groups)."""

    def __init__(self, devices, bounds, stats, n_rows, n_cols, shared, build_s, fused=None):
        self.devices = devices
        self.bounds = bounds
        self.stats = stats
        self.n_rows, self.n_cols = n_rows, n_cols
        self.shared = shared
        self.build_s = build_s
        # gcs.Group per batch of groups: a batch's level k in one launch,
        # batches one after the other (accumulating into y)
        self.fused = fused

    @property
    def device_bytes(self) -> int:
        """Grammar images of every group plus each distinct workspace once."""
        seen, total = set(), 0
        for d in self.devices:
            total += d.grammar_buf.numel()
            if d.workspace.data_ptr() not in seen:
                seen.add(d.workspace.data_ptr())
                total += d.workspace.numel()
        return total

    def new_y(self):
        return self.devices[0].new_y()

    def sweep_right(self, x, y=None, stream=None):
        """y = M x over all groups (asynchronous on the stream)."""
        if y is None:
            y = self.new_y()
        if self.fused is not None:
            for b, grp in enumerate(self.fused):
                grp.sweep_right(x, y, accumulate=b > 0, stream=stream)
            return y
        self.devices[0].sweep_right(x, y, stream)
        for d in self.devices[1:]:
            d.sweep_right_acc(x, y, stream)
        return y

    def profile_begin(self, max_sweeps, mode):
        if self.fused is not None:
            for grp in self.fused:
                grp.profile_begin(max_sweeps)
            return
        for d in self.devices:
            d.profile_begin(max_sweeps, mode)

    def sweep_right_profiled(self, x, y, stream=None):
        if self.fused is not None:
            for b, grp in enumerate(self.fused):
                grp.sweep_right(x, y, accumulate=b > 0, stream=stream, profiled=True)
            return y
        self.devices[0].sweep_right_profiled(x, y, stream)
        for d in self.devices[1:]:
            d.sweep_right_profiled(x, y, stream, accumulate=True)
        return y

    def profile_end(self):
        """Level-launch spans (ms) of each profiled sweep: per batch of a
        fused sweep an array over sweeps; otherwise, per group, its device's
        profile_end array."""
        if self.fused is not None:
            return [grp.profile_end() for grp in self.fused]
        return [d.profile_end() for d in self.devices]

    def check(self, stream=None):
        for d in self.devices:
            d.check(stream)

    def launches_per_sweep(self) -> int:
        if self.fused is not None:
            return sum(grp.launches() for grp in self.fused)
        return sum(d.sweep_launches() for d in self.devices)

    def free(self):
        if self.fused is not None:
            for grp in self.fused:
                grp.free()
            self.fused = None
        for d in self.devices:
            d.free()
        self.devices = []


def build_column_groups(source, n_rows, n_cols, group_cols, policy, workers=3, table_entries=1 << 28,
                        n_threads=0, on_group=None, on_built=None, log=None, device="cuda",
                        fuse=True, fuse_batch=25) -> ColumnGroups:
    """Build, upload and keep resident every group of `group_cols` consecutive
    columns of an n_rows x n_cols matrix.

    source(col0, ncols) -> (row_ptr, col, val): the CSR of columns
    [col0, col0 + ncols) of all rows, absolute column indices (val: None,
    int8 or float64, at most 64 distinct values).  on_group(i, col0, ncols,
    row_ptr, col, val), if given, sees each group's CSR before it is dropped,
    and on_built(i, grammar, device) each host grammar before it is freed
    (both called from the worker threads).  With fuse (plus-times policies
    only) the groups are swept in batches of fuse_batch (gcs_group_*: one
    launch per level for a whole batch); the groups of a batch need their
    own workspaces, batches run one after the other, so group i shares its
    workspace with the groups i +- fuse_batch.  Without, all groups share one
    workspace and are swept one after the other.  A workspace is sized by the
    first group that uses it (with a margin) and replaced for later groups if
    one needs more."""
    fuse = fuse and policy in (gcs.PLUS_F64, gcs.PLUS_F32, gcs.PLUS_F32_ACC_F64, gcs.PLUS_I64)
    torch = gcs._torch()
    policy = gcs.POLICY_NAMES.get(policy, policy)
    bounds = [(c0, min(group_cols, n_cols - c0)) for c0 in range(0, n_cols, group_cols)]
    t_start = time.perf_counter()
    lock = threading.Lock()
    shared = {}  # workspace slot -> tensor
    local = threading.local()
    build_ws = {}  # per worker thread: its build workspace (replaced, never accumulated)

    def work(i):
        c0, nc = bounds[i]
        t0 = time.perf_counter()
        rp, col, val = source(c0, nc)
        t_gen = time.perf_counter() - t0
        if on_group is not None:
            on_group(i, c0, nc, rp, col, val)
        nnz = int(rp[-1])
        need = gcs.build_workspace_bytes(n_rows, n_cols, nnz, table_entries)
        ws = getattr(local, "ws", None)
        if ws is None or ws.numel() < need:
            # groups differ slightly in size: leave a margin so that a worker
            # allocates its workspace once, and drop the old one first
            local.ws = None
            with lock:
                build_ws.pop(threading.get_ident(), None)
            local.ws = torch.empty(max(int(need * 1.05), 256), dtype=torch.uint8, device=device)
            with lock:
                build_ws[threading.get_ident()] = local.ws
        if getattr(local, "stream", None) is None:
            local.stream = torch.cuda.Stream(device=device)
        t1 = time.perf_counter()
        g = gcs.build_grammar_gpu(rp, col, val, n_cols=n_cols, n_threads=n_threads, table_entries=table_entries,
                                  workspace=local.ws, device=device, stream=local.stream)
        t_build = time.perf_counter() - t1
        del rp, col, val
        slot = i % max(1, fuse_batch) if fuse else 0
        need_ws = g.device_layout(policy)["workspace_bytes"]
        with lock:
            if slot not in shared or shared[slot].numel() < need_ws:
                shared[slot] = torch.empty(max(int(need_ws * 1.25), 256), dtype=torch.uint8, device=device)
            wsh = shared[slot]
        dev = gcs.upload(g, policy, device=device, stream=local.stream, workspace=wsh)
        st = g.stats()
        st.update(col0=c0, ncols=nc, t_gen_s=t_gen, t_build_s=t_build)
        if on_built is not None:
            on_built(i, g, dev)
        g.free()
        if log is not None:
            log(f"group {i}: columns [{c0}, {c0 + nc}) nnz={st['nnz']} |R|={st['n_rules']} L={st['depth']} "
                f"generated {t_gen:.1f}s, built {t_build:.1f}s (RePair {st['t_repair_ms'] / 1e3:.2f}s, layout "
                f"{st['t_layer_ms'] / 1e3:.2f}s), {dev.grammar_buf.numel() / 1e6:.0f} MB; "
                f"{time.perf_counter() - t_start:.0f}s since start")
        return dev, st

    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        results = list(ex.map(work, range(len(bounds))))
    torch.cuda.synchronize(device)
    build_ws.clear()
    local = None
    torch.cuda.empty_cache()
    devs = [r[0] for r in results]
    fused = None
    if fuse:
        nb = max(1, fuse_batch)
        fused = [gcs.Group(devs[b:b + nb]) for b in range(0, len(devs), nb)]
    return ColumnGroups(devs, bounds, [r[1] for r in results], n_rows, n_cols, shared,
                        time.perf_counter() - t_start, fused)
