"""Benchmark: the right product y = M x swept over a layered RePair grammar.

One step = one sweep (terminal array, every level with its emission, final
emission) over the uploaded grammar with x already in HBM.  The grammar is
built and uploaded before the timed region (a one-time cost, reported
separately as on the pages' Table B.1).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

The default workload is the largest configuration, the 200,000 x 2,000,000
genotype (about 1.2e11 nonzeros), built as 100 column groups on the device
(about five minutes) and swept whole; genotype_20000x100000_f32 and the other
WORKLOADS names in grammar_compressed_sparse_amd/synth select the others.

Prints one JSON line (metric, value = nnz/s, roofline of the level kernel,
CPU baseline = the oracle on the host cores, footprint vs CSR).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def level_bytes(lay, elem, yelem):
    """Algorithmic bytes of each level launch k = 1..L: child indices (8 B per
    binary node, 4 B per pass-through node), one write per completed node, one
    read of every value of level k-1 (the terminal array for k = 1), and the
    emission of level k-1 (erow + eoff per group, 4 B epos per root, y read and
    written per group)."""
    meta = lay["level_meta"]
    L = meta.shape[0] - 1
    eoff = lay["eoff"]
    out = []
    for k in range(1, L + 1):
        nb, npt = int(meta[k][0]), int(meta[k][1])
        if k == 1:
            prev_w = int(lay["alpha"])
        else:
            prev_w = int(meta[k - 1][0] + meta[k - 1][1])
        g0, ng = int(meta[k - 1][6]), int(meta[k - 1][7])
        roots = int(eoff[g0 + ng] - eoff[g0]) if ng else 0
        b = 8 * nb + 4 * npt + elem * (nb + npt) + elem * prev_w + 8 * ng + 4 * roots + 2 * yelem * ng
        out.append(b)
    return np.array(out, np.float64)


class CpuLeg:
    """The CPU leg of the bench, and the only code in this file that runs the
    oracle (test infrastructure, never the measured path): it times the
    oracle on the host cores (cpu_baseline) and checks sampled outputs of the
    GPU sweep against it.  --no-cpu-baseline skips the leg, timing and checks
    alike."""

    def __init__(self):
        import oracle
        self.o = oracle

    def threads(self):
        return self.o.num_threads()

    def rows_f64(self, rows, rp, col, val, x64):
        """(y, sum of |terms|) of the given rows, fp64 compensated."""
        return self.o.spmv_f64_rows(rows, rp, col, val, x64)

    def check_rows(self, what, y_rows, rows, rp, col, val, x64, tol):
        """max relative error of y_rows against the oracle; exits if above tol."""
        yo, absum = self.rows_f64(rows, rp, col, val, x64)
        err = float(np.max(np.abs(np.asarray(y_rows, np.float64) - yo) / np.maximum(absum, 1e-300)))
        if err > tol:
            raise SystemExit(f"{what} disagrees with the oracle: max rel err {err:.2e} (tol {tol})")
        return err

    def spmv_bool(self, rp, col, x):
        return self.o.spmv_bool(rp, col, x)

    def spmv_min_plus(self, rp, col, x, dtype):
        return self.o.spmv_min_plus(rp, col, None, x, dtype)

    def bfs(self, rp, col, src):
        return self.o.bfs(rp, col, src)

    def baseline(self, rp, col, val, x64, nnz, budget_s=10.0):
        """The oracle (fp64 compensated CSR SpMV) on all host cores over the
        full matrix for about budget_s, then on one core over a row sample of
        about a fifth of that time (context: the single-thread rate)."""
        oracle = self.o
        passes, t0 = 0, time.perf_counter()
        while True:
            oracle.spmv_f64(rp, col, val, x64)
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget_s or passes >= 50:
                break
        cores = oracle.num_threads()
        out = {"value": nnz * passes / el, "unit": "nnz/s", "cores": cores, "kind": "oracle",
               "sample": f"the full matrix, {passes} fp64 compensated CSR passes ({el:.1f} s)"}
        # one core: every k-th row, sized to about budget_s / 5 at the single-thread rate
        n = rp.shape[0] - 1
        per_core = nnz * passes / el / max(cores, 1)
        k = max(1, int(np.ceil(nnz / (per_core * budget_s / 5))))
        rows = np.arange(0, n, k)
        oracle.set_threads(1)
        try:
            t0 = time.perf_counter()
            oracle.spmv_f64_rows(rows, rp, col, val, x64)
            el1 = time.perf_counter() - t0
        finally:
            oracle.set_threads(cores)
        nnz1 = int((rp[rows + 1] - rp[rows]).sum())
        out["one_core"] = {"value": nnz1 / el1, "unit": "nnz/s",
                           "sample": f"rows 0, {k}, {2 * k}, ... ({rows.size} rows, {nnz1} nonzeros, {el1:.1f} s)"}
        return out


def csr_comparator(torch, rp, col, val, x, steps):
    """rocSPARSE CSR SpMV through torch.sparse (context: time and footprint)."""
    try:
        n = rp.shape[0] - 1
        m = x.numel()
        crow = torch.from_numpy(rp.astype(np.int32)).cuda()
        ci = torch.from_numpy(col).cuda()
        vv = torch.from_numpy(val.astype(np.float32)).cuda()
        A = torch.sparse_csr_tensor(crow, ci, vv, size=(n, m))
        y = torch.mv(A, x)
        for _ in range(3):
            y = torch.mv(A, x)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            y = torch.mv(A, x)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        nbytes = crow.numel() * 4 + ci.numel() * 4 + vv.numel() * 4 + x.numel() * 4 + y.numel() * 4
        del A, crow, ci, vv
        torch.cuda.empty_cache()
        return {"ms_per_spmv": ms, "device_bytes": nbytes, "via": "torch.mv on a sparse CSR tensor (int32, fp32)"}
    except Exception as e:  # context only
        return {"error": str(e)[:200]}


def bench_batched(torch, gcs, leg, synth, dev, lay, rp, col, val, spec, elem, xdt, batches, steps):
    """Batched right product Y = M X (B vectors per sweep) on the same upload:
    sampled rows of two columns checked against the oracle (CPU leg), then K timed
    sweeps; algorithmic bytes = the per-level formula with B-wide values, plus
    the leaf (descriptors, x rows, terminal rows) and the slice reduction.
    rocSPARSE SpMM (torch.sparse.mm on a CSR tensor) at the same B is context."""
    nnz = int(rp[-1])
    n, m = spec.n_rows, spec.n_cols
    alpha = int(lay["alpha"])
    rows = np.unique(np.concatenate([np.arange(0, n, max(1, n // 256)), [n - 1]]))
    crow = torch.from_numpy(rp.astype(np.int32)).cuda()
    A = torch.sparse_csr_tensor(crow, torch.from_numpy(col).cuda(), torch.from_numpy(val.astype(xdt)).cuda(),
                                size=(n, m))
    out = []
    for B in batches:
        X = torch.from_numpy(np.stack([synth.normal(m, 7000 + b) for b in range(B)], axis=1).astype(xdt)).cuda()
        Y = dev.sweep_right_batch(X)
        dev.check()
        Yh = Y.cpu().numpy()
        worst = None
        if leg is not None:
            tol = 1e-5 if elem == 4 else 1e-12
            worst = max(leg.check_rows(f"batched sweep (B={B}), column {b}", Yh[rows, b], rows, rp, col, val,
                                       X[:, b].cpu().numpy().astype(np.float64), tol) for b in (0, B - 1))
        for _ in range(3):
            dev.sweep_right_batch(X, Y)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            dev.sweep_right_batch(X, Y)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        sv = B * elem
        meta, eoff = lay["level_meta"], lay["eoff"]
        L = meta.shape[0] - 1
        g0, ng = int(meta[L][6]), int(meta[L][7])
        last_emit = 8 * ng + 4 * int(eoff[g0 + ng] - eoff[g0]) + 2 * sv * ng if ng else 0
        # levels and emissions, then the leaf (descriptors, x rows, terminal
        # rows), the accumulator clear and the slice reduction into Y
        alg = float(level_bytes(lay, sv, sv).sum() + last_emit + alpha * (8 + sv) + m * sv + 8 * n * sv +
                    9 * n * sv)
        # the same sweep without a terminal array (leaves evaluated in place)
        Yl = dev.sweep_right_batch(X, leaves_in_sweep=True)
        dev.check()
        if not torch.equal(Yl, Y):
            raise SystemExit(f"batched sweep with leaves in the sweep (B={B}) differs")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            dev.sweep_right_batch(X, Yl, leaves_in_sweep=True)
        torch.cuda.synchronize()
        ms_leaves = (time.perf_counter() - t0) * 1e3 / steps
        del Yl
        Z = torch.sparse.mm(A, X)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            Z = torch.sparse.mm(A, X)
        torch.cuda.synchronize()
        ms_csr = (time.perf_counter() - t0) * 1e3 / 3
        del Z, X, Y
        out.append({"B": B, "ms_per_sweep": ms, "ms_per_vector": ms / B, "nnz_per_s": nnz * B / (ms * 1e-3),
                    "alg_bytes_per_sweep": alg, "achieved_GBs": alg / (ms * 1e-3) / 1e9,
                    "frac_hbm_peak": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "max_rel_err_sampled": worst,
                    "workspace_bytes": dev.batch_workspace_bytes(B), "rocsparse_spmm_ms": ms_csr,
                    "leaves_in_sweep": {"ms_per_sweep": ms_leaves,
                                        "workspace_bytes": dev.batch_workspace_bytes(B, leaves_in_sweep=True)}})
        log(f"batched B={B}: {ms:.3f} ms per sweep ({ms / B:.4f} ms per vector), rocSPARSE SpMM {ms_csr:.3f} ms")
    del A, crow
    torch.cuda.empty_cache()
    return out


KERNEL_SOURCE = os.path.join(ROOT, "grammar_compressed_sparse_amd", "csrc", "kernels.hpp")
# the layout (node order, slices, emission groups) decides the kernels' access
# pattern as much as their code does
LAYOUT_SOURCE = os.path.join(ROOT, "grammar_compressed_sparse_amd", "csrc", "builder.cpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "level_kernel_traffic.json")
GROUP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "level_group_kernel_traffic.json")
L2_FILE = os.path.join(ROOT, "profiles", "l2_requests.json")
# L2 request rate of the chip: 8 XCDs x 16 L2 channels, one request per
# channel per clock at 2.4 GHz (G requests/s).  A 4-byte gather costs a whole
# request, so a gather-bound kernel meets this bound long before the HBM one.
L2_REQ_PEAK_G = 8 * 16 * 2.4


def grammar_bytes(st) -> int:
    """Bytes of the grammar a sweep streams: 8 per binary rule (two child
    references), 4 per pass-through node, 8 per entry of C (reference and
    row position), 4 per terminal."""
    return 8 * st["n_rules"] + 4 * st["n_passthrough"] + 8 * st["c_len"] + 4 * st["n_terminals"]


def l2_bound(kernel, workload, launch_avg_us):
    """The second bound of the roofline: L2 requests per launch of `kernel`
    on `workload` from the committed counter record (while the kernel
    source's hash still matches), their rate over the bench's own launch
    time, against L2_REQ_PEAK_G."""
    if not os.path.exists(L2_FILE):
        return None
    with open(L2_FILE) as f:
        rec = json.load(f).get(f"{kernel}:{workload}")
    if not rec or rec.get("source_sha256") != kernel_source_hash():
        return None
    rate = rec["requests_per_launch"] / (launch_avg_us * 1e-6) / 1e9
    return {"bound": "l2_requests", "requests_per_launch": rec["requests_per_launch"], "achieved": rate,
            "peak": L2_REQ_PEAK_G, "unit": "G requests/s", "frac": rate / L2_REQ_PEAK_G,
            "hit_rate": rec["hit_rate"],
            "peak_basis": "8 XCDs x 16 L2 channels x 2.4 GHz, one request per channel per clock"}


def filter_counters(in_dir, out_dir, kernel, n_copies=20):
    """Reduce a counter run's CSV to what the summaries read: every row of the
    dispatches of gcs::kernel and of the first n_copies copy dispatches (the
    calibration copies are issued first).  A run that builds many grammars
    makes hundreds of thousands of other dispatches, far more than the
    summaries need."""
    import csv
    import glob
    fs = glob.glob(os.path.join(in_dir, "**", "*counter_collection.csv"), recursive=True)
    os.makedirs(out_dir, exist_ok=True)
    with open(fs[0]) as f:
        rd = csv.DictReader(f)
        rows = list(rd)
        fields = rd.fieldnames
    copies = sorted({int(r["Dispatch_Id"]) for r in rows if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")})
    keep_copy = set(copies[:n_copies])
    out = [r for r in rows if f"gcs::{kernel}<" in r["Kernel_Name"] or int(r["Dispatch_Id"]) in keep_copy]
    with open(os.path.join(out_dir, "filtered_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(out)
    print(f"{len(out)} of {len(rows)} rows kept")


def summarize_l2(hit_dir, out_md, kernel, workload, commands):
    """L2 requests (TCC_HIT_sum + TCC_MISS_sum) per dispatch of gcs::kernel
    from one --pmc TCC_HIT_sum TCC_MISS_sum run: the mean over the run's
    dispatches is recorded in L2_FILE under kernel:workload with the kernel
    source's hash, and summarised in out_md."""
    import csv
    import glob
    fs = glob.glob(os.path.join(hit_dir, "**", "*counter_collection.csv"), recursive=True)
    per = {}
    for r in csv.DictReader(open(fs[0])):
        if f"gcs::{kernel}<" not in r["Kernel_Name"]:
            continue
        name = r["Counter_Name"]
        if not name.startswith(("TCC_HIT", "TCC_MISS")):
            continue  # other counters of the same pass
        h = per.setdefault(int(r["Dispatch_Id"]), [0.0, 0.0])
        h[0 if name.startswith("TCC_HIT") else 1] += float(r["Counter_Value"])
    v = np.array(list(per.values()))
    req = v.sum(axis=1)
    rec = {"source_sha256": kernel_source_hash(), "kernel": kernel, "workload": workload,
           "launches": int(v.shape[0]), "requests_per_launch": float(req.mean()),
           "hit_rate": float(v[:, 0].sum() / req.sum())}
    allrec = {}
    if os.path.exists(L2_FILE):
        with open(L2_FILE) as f:
            allrec = json.load(f)
    allrec[f"{kernel}:{workload}"] = rec
    with open(L2_FILE, "w") as f:
        json.dump(allrec, f, indent=1)
    lines = [f"# L2 requests of {kernel} on {workload}", "",
             "Command (run from /tmp with TMPDIR=/tmp; R = repository root):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", f"- {rec['launches']} dispatches of gcs::{kernel}; L2 requests (hits + misses, all XCDs) per "
                  f"dispatch: mean {rec['requests_per_launch'] / 1e6:.2f} M, median {np.median(req) / 1e6:.2f} M, "
                  f"max {req.max() / 1e6:.2f} M; hit rate {rec['hit_rate']:.3f}",
              f"- request peak: {L2_REQ_PEAK_G:.1f} G requests/s (8 XCDs x 16 channels x 2.4 GHz)",
              f"- kernel and layout source sha256[:16] = {rec['source_sha256']}"]
    with open(out_md, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def kernel_source_hash() -> str:
    """Hash of the device source and of the layout code, without their
    comments and with whitespace runs collapsed: a comment edit keeps the
    recorded counter profile valid, any change to the code voids it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in (KERNEL_SOURCE, LAYOUT_SOURCE):
        with open(path) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def copy_achievable_gbs(torch, mib=2048, reps=10):
    """Achievable HBM bandwidth on this device: a device-to-device copy of
    `mib` MiB (read + written bytes / time, HIP events, after two warm-up
    copies), the practical ceiling beside the 8 TB/s specification."""
    src = torch.empty(mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)  # 4-byte elements, vectorized copy
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    gbs = 2 * src.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    log(f"achievable copy bandwidth: {gbs:.0f} GB/s ({mib} MiB device-to-device)")
    return gbs


def random_gather_rates(torch, windows=(1 << 20, 8 << 20, 1 << 30), n=1 << 26, reps=5):
    """Measured ceiling for gather-bound kernels: 4-byte random gathers per
    second (torch.take with int64 indices, n per launch) when every run of
    consecutive outputs reads at random inside one window of `w` bytes of
    the source, for a few window sizes; HIP events, after one warm-up."""
    out = {}
    src = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(12345)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for w in windows:
        per = w // 4
        base = (torch.arange(n, device="cuda", dtype=torch.int64) // per) * per % src.numel()
        idx = base + torch.randint(0, per, (n,), device="cuda", generator=g, dtype=torch.int64)
        dst = torch.take(src, idx)
        e0.record()
        for _ in range(reps):
            dst = torch.take(src, idx)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[str(w)] = n / (ms * 1e-3) / 1e9
        del idx, base, dst
    del src
    torch.cuda.empty_cache()
    log("random 4-byte gathers (torch.take): " + ", ".join(f"{int(w) >> 20} MiB windows {r:.0f} G/s"
                                                         for w, r in out.items()))
    return out


def sweep_breakdown(trace, pol):
    """Lines describing the launches of one sweep of policy `pol` (leaf_kernel
    up to the tail_kernel) in a rocprofv3 kernel trace, averaged over the
    sweeps of the run that have the usual number of launches."""
    trace = sorted(trace, key=lambda r: int(r["Start_Timestamp"]))
    sweeps, cur = [], None
    for r in trace:
        n = r["Kernel_Name"]
        if pol not in n:
            continue
        short = n.split("(")[0].split("<")[0].replace("void ", "").replace("gcs::", "")
        if short == "leaf_kernel":
            cur = []
            sweeps.append(cur)
        if cur is not None:
            cur.append((short, int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    sweeps = [sw for sw in sweeps if sw and sw[-1][0] == "tail_kernel"]
    if not sweeps:
        return []
    nl = int(np.median([len(sw) for sw in sweeps]))
    sweeps = [sw for sw in sweeps if len(sw) == nl]
    dur = np.array([[(e - b) / 1e3 for _, b, e in sw] for sw in sweeps])
    span = np.array([(sw[-1][2] - sw[0][1]) / 1e3 for sw in sweeps])
    mean = dur.mean(axis=0)
    return ["", f"## One sweep of {pol} ({len(sweeps)} sweeps of {nl} launches)", "",
            f"- per sweep (medians): kernel time {np.median(dur.sum(axis=1)):.1f} us, first launch start to last "
            f"launch end {np.median(span):.1f} us",
            "- mean duration per launch, us: leaf " + f"{mean[0]:.1f}; levels 1-8: " +
            " ".join(f"{v:.1f}" for v in mean[1:min(9, nl - 1)]) +
            f"; remaining {max(nl - 10, 0)} wide launches {mean[9:nl - 1].sum():.1f} in total; tail {mean[-1]:.1f}"]


def summarize_kernel_trace(kt_dir, out_md, title, commands, policies=("PolBoolOr", "PolMinPlusF32")):
    """Text summary of a rocprofv3 kernel trace (no counters): the kernel time
    table and, per policy, the launches of one sweep (leaf_kernel up to the
    tail_kernel) averaged over the sweeps of the run."""
    import csv
    import glob

    def rows(pat):
        fs = glob.glob(os.path.join(kt_dir, "**", pat), recursive=True)
        return list(csv.DictReader(open(fs[0]))) if fs else []

    stats = rows("*kernel_stats.csv")
    lines = [f"# rocprofv3 summary: {title}", "", "Command (run from /tmp with TMPDIR=/tmp; R = repository root):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "## Kernel time (--kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats[:14]:
        name = r["Name"].split("(")[0].replace("void ", "")
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    trace = rows("*kernel_trace.csv")
    for pol in policies:
        lines += sweep_breakdown(trace, pol)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_rocprof(kt_dir, fetch_dir, write_dir, out_md, copy_mib, commands):
    """Turn rocprofv3 CSV output (kernel trace stats; FETCH_SIZE and WRITE_SIZE
    counter collections that include a known-size copy) into the text summary
    under profiles/ and the traffic record bench.py reads."""
    import csv
    import glob

    def rows(d, pat):
        fs = glob.glob(os.path.join(d, "**", pat), recursive=True)
        return list(csv.DictReader(open(fs[0]))) if fs else []

    stats = rows(kt_dir, "*kernel_stats.csv")
    lines = ["# rocprofv3 summary: level_kernel on genotype_20000x100000_f32", "",
             "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "## Kernel time (--kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"].split("(")[0].replace("void ", "")
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    lines += sweep_breakdown(rows(kt_dir, "*kernel_trace.csv"), "PolPlusF32")
    rec = {"source_sha256": kernel_source_hash(), "copy_bytes": copy_mib << 20}
    for tag, d in (("fetch", fetch_dir), ("write", write_dir)):
        cname = "FETCH_SIZE" if tag == "fetch" else "WRITE_SIZE"
        cc = [r for r in rows(d, "*counter_collection.csv") if r.get("Counter_Name", cname) == cname]
        # the calibration copies: the first five large copy dispatches of the
        # run (issued before anything else; later large copies, such as the
        # achievable-bandwidth copy, are not of the calibrated size)
        cc_sorted = sorted(cc, key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in cc_sorted if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")]
        big = [v for v in copies if v > 0.25 * copy_mib * 1024][:5]
        lvl = [float(r["Counter_Value"]) * 1024 for r in cc if "level_kernel" in r["Kernel_Name"]]
        rec[tag + "_kib_copy"] = sum(big) / len(big)
        rec[tag + "_bytes_per_launch"] = sum(lvl) / max(len(lvl), 1)
        rec[tag + "_launches"] = len(lvl)
    scale_f = rec["copy_bytes"] / (rec["fetch_kib_copy"] * 1024)
    scale_w = rec["copy_bytes"] / (rec["write_kib_copy"] * 1024)
    rec["scale_fetch"], rec["scale_write"] = scale_f, scale_w
    rec["traffic_bytes_per_launch"] = rec["fetch_bytes_per_launch"] * scale_f + rec["write_bytes_per_launch"] * scale_w
    # the batched level kernel (context): mean scaled HBM bytes per dispatch
    # and the summed bytes and kernel time over all of its dispatches
    bt = {}
    for tag, d, sc in (("fetch", fetch_dir, scale_f), ("write", write_dir, scale_w)):
        cname = "FETCH_SIZE" if tag == "fetch" else "WRITE_SIZE"
        cc = [r for r in rows(d, "*counter_collection.csv") if r.get("Counter_Name", cname) == cname]
        v = [float(r["Counter_Value"]) * 1024 * sc for r in cc if "level_batch_kernel" in r["Kernel_Name"]]
        bt[tag] = (sum(v), len(v))
    kt_batch = [r for r in stats if "level_batch_kernel" in r["Name"]]
    if bt["fetch"][1] and kt_batch:
        total_ns = sum(float(r["TotalDurationNs"]) for r in kt_batch)
        calls = sum(int(r["Calls"]) for r in kt_batch)
        per = (bt["fetch"][0] / bt["fetch"][1] + bt["write"][0] / max(bt["write"][1], 1))
        rec["batch_traffic_bytes_per_dispatch"] = per
        rec["batch_kernel_avg_ns"] = total_ns / calls
        rec["batch_traffic_GBs"] = per / (total_ns / calls)
    lines += ["", "## HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              f"- calibration: one copy dispatch of {rec['copy_bytes'] / 2**20:.0f} MiB read "
              f"{rec['fetch_kib_copy']:.1f} KiB and wrote {rec['write_kib_copy']:.1f} KiB "
              f"(scale {scale_f:.5f} / {scale_w:.5f})",
              f"- level_kernel, mean over {rec['fetch_launches']} dispatches: FETCH "
              f"{rec['fetch_bytes_per_launch'] / 1e6:.2f} MB, WRITE {rec['write_bytes_per_launch'] / 1e6:.2f} MB, "
              f"traffic {rec['traffic_bytes_per_launch'] / 1e6:.2f} MB per launch (scaled)",
              f"- kernel and layout source sha256[:16] = {rec['source_sha256']}"]
    if "batch_traffic_GBs" in rec:
        lines += [f"- level_batch_kernel (batched sweeps of the same run): {rec['batch_traffic_bytes_per_dispatch'] / 1e6:.2f} "
                  f"MB of HBM traffic per dispatch on average, {rec['batch_kernel_avg_ns'] / 1e3:.1f} us average "
                  f"duration: {rec['batch_traffic_GBs']:.0f} GB/s measured"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print("\n".join(lines))


def summarize_group_trace(kt_dir, out_md, title, commands, bench_log=None):
    """Text summary of a rocprofv3 kernel trace of the column-group bench:
    the kernel time table, and per product (leaf_group_kernel ... the last
    reduce_group_kernel of its batches) the level_group_kernel launches'
    kernel time against the bench's own HIP-event span of the same launches."""
    import csv
    import glob

    def rows(pat):
        fs = glob.glob(os.path.join(kt_dir, "**", pat), recursive=True)
        return list(csv.DictReader(open(fs[0]))) if fs else []

    stats = rows("*kernel_stats.csv")
    lines = [f"# rocprofv3 summary: {title}", "", "Command (run from /tmp with TMPDIR=/tmp; R = repository root):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "## Kernel time (--kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | max us | total ms | share |", "|---|---|---|---|---|---|---|"]
    for r in stats[:16]:
        name = r["Name"].split("(")[0].replace("void ", "")
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                     f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / 1e6:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    trace = sorted(rows("*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    lv = [r for r in trace if "level_group_kernel" in r["Kernel_Name"]]
    if lv:
        d = np.array([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in lv])
        lines += ["", "## level_group_kernel (the dominant kernel)", "",
                  f"- {len(lv)} launches, average duration {d.mean():.1f} us (median {np.median(d):.1f} us), "
                  f"{d.sum() / 1e3:.1f} ms in all"]
        # batch sweeps: the group launches up to and including a reduce_group_kernel
        prods, cur = [], []
        for r in trace:
            n = r["Kernel_Name"]
            if "group_kernel" in n:
                cur.append(r)
            if "reduce_group_kernel" in n and cur:
                prods.append(cur)
                cur = []
        if prods:
            lvl_ms = [sum((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in p
                          if "level_group_kernel" in r["Kernel_Name"]) / 1e6 for p in prods]
            span_ms = [(int(p[-1]["End_Timestamp"]) - int(p[0]["Start_Timestamp"])) / 1e6 for p in prods]
            lines += [f"- per batch sweep (leaf to reduction, {len(prods)} batch sweeps): level kernel time "
                      f"{np.median(lvl_ms):.2f} ms, first start to last end {np.median(span_ms):.2f} ms (medians)"]
    if bench_log and os.path.exists(bench_log):
        with open(bench_log) as f:
            js = [ln for ln in f if ln.startswith("{")]
        if js:
            b = json.loads(js[-1])
            rf = b["roofline"]
            lines += ["", "## The same run's bench line", "",
                      f"- {b['ms_per_step']:.2f} ms per product, value {b['value']:.4g} nnz/s; roofline: "
                      f"{rf['launches']} level launches per product, span {rf['launch_avg_us']:.1f} us per launch "
                      f"(gaps included), achieved {rf['achieved']:.0f} GB/s = {rf['frac']:.3f} of peak"]
    with open(out_md, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_group_counters(fetch_dir, write_dir, out_md, copy_mib, commands, bench_logs):
    """HBM traffic of level_group_kernel from a --pmc FETCH_SIZE run and a
    --pmc WRITE_SIZE run of the default bench (each calibrated by device
    copies of a known size issued first): mean scaled bytes per dispatch,
    written to GROUP_TRAFFIC_FILE with the kernel source's hash (bench.py
    reports it as roofline.traffic only while that hash still matches) and
    summarised in out_md."""
    import csv
    import glob

    def rows(d, pat):
        fs = glob.glob(os.path.join(d, "**", pat), recursive=True)
        return list(csv.DictReader(open(fs[0]))) if fs else []

    rec = {"source_sha256": kernel_source_hash(), "copy_bytes": copy_mib << 20, "kernel": "level_group_kernel"}
    for tag, d in (("fetch", fetch_dir), ("write", write_dir)):
        cname = "FETCH_SIZE" if tag == "fetch" else "WRITE_SIZE"
        cc = sorted((r for r in rows(d, "*counter_collection.csv") if r.get("Counter_Name", cname) == cname),
                    key=lambda r: int(r["Dispatch_Id"]))
        copies = [float(r["Counter_Value"]) for r in cc if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")]
        big = [v for v in copies if v > 0.25 * copy_mib * 1024][:5]
        lvl = [float(r["Counter_Value"]) * 1024 for r in cc if "level_group_kernel" in r["Kernel_Name"]]
        rec[tag + "_kib_copy"] = sum(big) / len(big)
        rec[tag + "_scale"] = rec["copy_bytes"] / (rec[tag + "_kib_copy"] * 1024)
        rec[tag + "_bytes_per_launch"] = sum(lvl) / max(len(lvl), 1) * rec[tag + "_scale"]
        rec[tag + "_launches"] = len(lvl)
    rec["traffic_bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    alg = None
    for lg in bench_logs:
        if os.path.exists(lg):
            js = [ln for ln in open(lg) if ln.startswith("{")]
            if js:
                alg = json.loads(js[-1])["roofline"]["bytes_per_launch_avg"]
    lines = ["# HBM traffic of level_group_kernel on genotype_200000x2000000_f32 (the default bench)", "",
             "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", f"- calibration: a device copy of {copy_mib} MiB reads {rec['fetch_kib_copy']:.1f} KiB "
                  f"(FETCH_SIZE) and writes {rec['write_kib_copy']:.1f} KiB (WRITE_SIZE): scales "
                  f"{rec['fetch_scale']:.4f} / {rec['write_scale']:.4f}",
              f"- level_group_kernel, mean over {rec['fetch_launches']} / {rec['write_launches']} dispatches: "
              f"FETCH {rec['fetch_bytes_per_launch'] / 1e6:.1f} MB, WRITE {rec['write_bytes_per_launch'] / 1e6:.1f} MB, "
              f"traffic {rec['traffic_bytes_per_launch'] / 1e6:.1f} MB per launch (scaled)"]
    if alg:
        rec["algorithmic_bytes_per_launch"] = alg
        lines.append(f"- algorithmic bytes per launch (the bench's formula): {alg / 1e6:.1f} MB; traffic / "
                     f"algorithmic = {rec['traffic_bytes_per_launch'] / alg:.2f}")
    lines.append(f"- kernel and layout source sha256[:16] = {rec['source_sha256']}")
    with open(GROUP_TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    with open(out_md, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_per_level(kt_dir, fetch_dir, write_dir, levels_json, out_md, copy_mib, commands):
    """Per-level hardware-counter table of one sweep: every level_kernel
    dispatch of a single-vector sweep is matched to its level k by its order
    after the sweep's leaf_kernel; FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, scaled by the same counters on a known-size copy) are averaged
    per level over the run's sweeps, and divided by the mean kernel duration
    of that level from the kernel trace.  levels_json: the bench's JSON line
    run with GCS_BENCH_LEVELS=1 (algorithmic bytes per level)."""
    import csv
    import glob

    def rows(d, pat):
        fs = glob.glob(os.path.join(d, "**", pat), recursive=True)
        return list(csv.DictReader(open(fs[0]))) if fs else []

    def per_level(recs, key):
        """level k -> list of values, from dispatches in dispatch order"""
        recs = sorted(recs, key=lambda r: int(r["Dispatch_Id"]))
        out, k = {}, None
        for r in recs:
            n = r["Kernel_Name"]
            if "leaf_kernel" in n and "batch" not in n:
                k = 0
            elif "level_kernel" in n and k is not None:
                k += 1
                out.setdefault(k, []).append(key(r))
            elif "tail_kernel" in n:
                k = None
        return out

    with open(levels_json) as f:
        line = [ln for ln in f if ln.startswith("{")][-1]
    lv = {p["k"]: p for p in json.loads(line)["config"]["per_level"]}
    copy = copy_mib << 20
    scales = {}
    vals = {}
    for tag, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        cc = [r for r in rows(d, "*counter_collection.csv") if r.get("Counter_Name", tag) == tag]
        big = [float(r["Counter_Value"]) for r in sorted(cc, key=lambda r: int(r["Dispatch_Id"]))
               if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer") and float(r["Counter_Value"]) > 0.25 * copy_mib * 1024][:5]
        scales[tag] = copy / (sum(big) / len(big) * 1024)
        vals[tag] = per_level(cc, lambda r: float(r["Counter_Value"]) * 1024 * scales[tag])
    kt = rows(kt_dir, "*kernel_trace.csv")
    dur = per_level([dict(r, Dispatch_Id=r.get("Dispatch_Id", r.get("Correlation_Id", 0))) for r in kt],
                    lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Per-level HBM traffic: level_kernel on genotype_20000x100000_f32, one sweep", "",
             "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", f"FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the same counters on {copy_mib} MiB "
                  f"device copies (scale {scales['FETCH_SIZE']:.4f} / {scales['WRITE_SIZE']:.4f}); a level "
                  "launch k computes level k and emits level k-1. Durations: mean kernel time of that launch in "
                  "the kernel trace. Algorithmic bytes as in bench.py's level formula.", "",
              "| k | width | algorithmic MB | FETCH MB | WRITE MB | traffic / algorithmic | us | algorithmic GB/s | "
              "measured GB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(vals["FETCH_SIZE"]):
        if k not in lv or k not in vals["WRITE_SIZE"] or k not in dur:
            continue
        f = float(np.mean(vals["FETCH_SIZE"][k]))
        w = float(np.mean(vals["WRITE_SIZE"][k]))
        us = float(np.mean(dur[k]))
        a = float(lv[k]["bytes"])
        lines.append(f"| {k} | {lv[k]['width']} | {a / 1e6:.1f} | {f / 1e6:.1f} | {w / 1e6:.1f} | {(f + w) / a:.2f} | "
                     f"{us:.1f} | {a / (us * 1e-6) / 1e9:.0f} | {(f + w) / (us * 1e-6) / 1e9:.0f} |")
    with open(out_md, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def bench_tropical(args, torch, gcs, leg, g, rp, col, spec, src, vis_o, counts_o):
    """Tropical (min, +) policy with unit weights on the same graph: K timed
    single passes from d0 (0 at the sources, +inf elsewhere), one checked
    bit for bit against the oracle, then Bellman-Ford d <- min(d, M d) to the
    fixpoint, whose distances must be the oracle BFS's levels (both checks
    in the CPU leg; vis_o and counts_o are its BFS, None without it)."""
    nnz = int(rp[-1])
    t_up = time.perf_counter()
    dev = gcs.upload(g, gcs.MIN_PLUS_F32)
    torch.cuda.synchronize()
    t_up = time.perf_counter() - t_up
    d0 = torch.full((spec.n,), float("inf"), dtype=torch.float32, device="cuda")
    d0[torch.from_numpy(src).cuda()] = 0
    y = dev.new_y()
    for _ in range(max(args.warmup, 1)):
        dev.sweep_right(d0, y)
    dev.check()
    if leg is not None and not np.array_equal(y.cpu().numpy(),
                                              leg.spmv_min_plus(rp, col, d0.cpu().numpy(), np.float32)):
        raise SystemExit("tropical pass disagrees with the oracle")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dev.sweep_right(d0, y)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # the relaxation d <- min(d, M d) as one accumulate sweep into a copy of
    # d (y = y (+) M d with (+) = min); the same time as a plain sweep and a
    # separate minimum (0.16 s for the copy graph's fixpoint either way: the
    # dense passes are bound by reading y before each finite update)
    t0 = time.perf_counter()
    d, passes = d0, 0
    while True:
        nd = d.clone()
        dev.sweep_right_acc(d, nd)
        passes += 1
        if torch.equal(nd, d):
            break
        d = nd
    torch.cuda.synchronize()
    bf_s = time.perf_counter() - t0
    dev.check()
    dh = d.cpu().numpy()
    hist = np.bincount(dh[np.isfinite(dh)].astype(np.int64))
    if vis_o is not None and not (np.array_equal(np.isfinite(dh), vis_o.astype(bool)) and
                                  np.array_equal(hist[1:], counts_o[:len(hist) - 1])):
        raise SystemExit("Bellman-Ford distances disagree with the oracle BFS levels")
    out = {"ms_per_pass": ms, "nnz_per_s": nnz / (ms * 1e-3), "upload_s": t_up, "bellman_ford_passes": passes,
           "bellman_ford_s": bf_s, "max_distance": int(len(hist) - 1)}
    log(f"tropical: {ms:.2f} ms per pass; Bellman-Ford fixpoint in {passes} passes, {bf_s:.2f} s")
    dev.free()
    return out


def bench_biobank(args, wl, spec, leg):
    """The 200,000 x 2,000,000 genotype (about 1.2e11 nonzeros; fp32 CSR about
    982 GB, beyond one GPU's 288 GB) as independent column groups of
    args.group_cols columns, each built by the device builder and all kept
    resident (grammar_compressed_sparse_amd.groups); one step sweeps every
    group into one y.  The CPU leg checks 4,098 seeded rows against the oracle
    (on each group's CSR as it is generated) and times the oracle on one group."""
    import threading

    import torch
    from grammar_compressed_sparse_amd import gcs, groups, synth

    acc64 = args.policy == "f32_acc_f64"
    policy = gcs.PLUS_F32_ACC_F64 if acc64 else gcs.PLUS_F32
    tol = 1e-12 if acc64 else 1e-5
    yelem = 8 if acc64 else 4
    x64 = synth.normal(spec.n_cols, wl["x_seeds"][0])
    x32 = x64.astype(np.float32)
    xo = x32.astype(np.float64)  # the values the device sees
    xd = torch.from_numpy(x32).cuda()
    rows = np.unique(np.concatenate([np.random.default_rng(7).choice(spec.n_rows, 4096, replace=False),
                                     [0, spec.n_rows - 1]]))
    yo, absum = np.zeros(rows.size), np.zeros(rows.size)
    lock = threading.Lock()
    nnz_of, lbytes, espan = {}, {}, {}

    def on_group(i, c0, nc, rp, col, val):
        if leg is not None:
            a, b = leg.rows_f64(rows, rp, col, val, xo)
            with lock:
                yo[:] += a
                absum[:] += b

    def on_built(i, g, dev):
        st = g.stats()
        lay = g.layout_meta()
        lay["alpha"] = st["n_terminals"]
        nwide = dev.sweep_launches() - 2
        lb = level_bytes(lay, yelem, yelem)
        # the emission of the last level (its own launch in a fused sweep)
        meta, eoff = lay["level_meta"], lay["eoff"]
        L = meta.shape[0] - 1
        g0, ng = int(meta[L][6]), int(meta[L][7])
        last = 8 * ng + 4 * int(eoff[g0 + ng] - eoff[g0]) + 2 * yelem * ng if ng else 0
        sp = g.edge_spans()
        with lock:
            nnz_of[i] = st["nnz"]
            lbytes[i] = (float(lb[:max(nwide, 0)].sum()), float(lb.sum() + last), nwide, L + 1)
            for d, c in enumerate(sp.tolist()):
                if c:
                    espan[d] = espan.get(d, 0) + c

    log(f"building {spec.n_rows}x{spec.n_cols} as groups of {args.group_cols} columns "
        f"({args.build_workers} build workers)")
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated()
    cg = groups.build_column_groups(lambda c0, nc: synth.genotype(spec, col0=c0, ncols=nc), spec.n_rows,
                                    spec.n_cols, args.group_cols, policy, workers=args.build_workers,
                                    table_entries=1 << 28, on_group=on_group, on_built=on_built, log=log,
                                    fuse=not args.no_fuse, fuse_batch=args.fuse_batch)
    fused = cg.fused is not None
    nnz = sum(nnz_of.values())
    torch.cuda.synchronize()
    mem_resident = torch.cuda.memory_allocated() - mem0  # cross-check of the footprint (torch's own count)
    log(f"built {len(cg.devices)} groups in {cg.build_s:.0f}s: nnz={nnz}, device {cg.device_bytes / 1e9:.1f} GB")
    y = cg.sweep_right(xd)
    cg.check()
    err = None
    if leg is not None:
        err = float(np.max(np.abs(y.cpu().numpy()[rows].astype(np.float64) - yo) / np.maximum(absum, 1e-300)))
        log(f"sampled-row check: {rows.size} rows, max rel err {err:.2e} (tol {tol})")
        if err > tol:
            raise SystemExit(f"biobank sweep disagrees with the oracle: {err:.2e}")
    for _ in range(args.warmup):
        cg.sweep_right(xd, y)
    torch.cuda.synchronize()
    # timed region: K full sweeps with HIP events (on the sweep's stream)
    # around the level launches, the dominant kernel: fused, one pair around
    # all level launches of a sweep (level_group_kernel); otherwise one pair
    # per group around its wide level launches (level_kernel)
    cg.profile_begin(args.steps, gcs.PROFILE_LEVEL_SPAN)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        cg.sweep_right_profiled(xd, y)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    spans = cg.profile_end()
    cg.check()
    ms_per_step = elapsed * 1e3 / args.steps
    all_bytes = sum(v[1] for v in lbytes.values())
    # sustained: back-to-back products for at least 1.5 s (after the timed region)
    torch.cuda.synchronize()
    t_s, n_s = time.perf_counter(), 0
    while True:
        for _ in range(5):
            cg.sweep_right(xd, y)
        n_s += 5
        torch.cuda.synchronize()
        if time.perf_counter() - t_s >= 1.5:
            break
    sustained = {"seconds": time.perf_counter() - t_s, "products": n_s}
    sustained["nnz_per_s"] = nnz * n_s / sustained["seconds"]
    cg.check()
    if fused:
        span_ms = float(sum(float(sp.mean()) for sp in spans))  # per full sweep, over the batches
        wide_bytes = all_bytes
        nwide = cg.launches_per_sweep() - 2 * len(cg.fused)  # every level launch (leaves and reductions aside)
        kernel = (f"level_group_kernel (one launch per level, each covering that level of a batch of "
                  f"{args.fuse_batch} column groups; per batch timed from before its first to after its last "
                  f"level launch, gaps included)")
    else:
        span_ms = float(sum(float(sp[:, 0].mean()) for sp in spans))  # per full sweep
        wide_bytes = sum(v[0] for v in lbytes.values())
        nwide = sum(v[2] for v in lbytes.values())
        kernel = ("level_kernel (the wide levels of every group's sweep, one launch each; each group timed "
                  "from before its first to after its last wide launch)")
    achieved = wide_bytes / (span_ms * 1e-3) / 1e9
    log(f"{ms_per_step:.2f} ms per sweep ({nnz / (ms_per_step * 1e-3):.3e} nnz/s); wide levels {nwide} launches in "
        f"{span_ms:.2f} ms, {wide_bytes / 1e9:.1f} GB -> {achieved:.0f} GB/s")
    cpu = None
    if leg is not None:
        # the oracle on the host cores over group 0 (regenerated), about 10 s
        rp, col, val = synth.genotype(spec, col0=0, ncols=args.group_cols)
        g_nnz = int(rp[-1])
        passes, t0 = 0, time.perf_counter()
        while True:
            leg.o.spmv_f64(rp, col, val, xo)
            passes += 1
            el = time.perf_counter() - t0
            if el >= 10.0 or passes >= 50:
                break
        cores = leg.threads()
        cpu = {"value": g_nnz * passes / el, "unit": "nnz/s", "cores": cores, "kind": "oracle",
               "sample": f"column group 0 (columns [0, {args.group_cols}), all {spec.n_rows} rows, {g_nnz} "
                         f"nonzeros), {passes} fp64 compensated CSR passes ({el:.1f} s)"}
        # one core, over every 8th row of the same group (context: the single-thread rate)
        rows1 = np.arange(0, spec.n_rows, 8)
        leg.o.set_threads(1)
        try:
            t0 = time.perf_counter()
            leg.o.spmv_f64_rows(rows1, rp, col, val, xo)
            el1 = time.perf_counter() - t0
        finally:
            leg.o.set_threads(cores)
        nnz1 = int((rp[rows1 + 1] - rp[rows1]).sum())
        cpu["one_core"] = {"value": nnz1 / el1, "unit": "nnz/s",
                           "sample": f"rows 0, 8, 16, ... of column group 0 ({rows1.size} rows, {nnz1} nonzeros, "
                                     f"{el1:.1f} s)"}
        del rp, col, val
    copy_gbs = None if args.calibrate_copy_mib else copy_achievable_gbs(torch)
    gathers = None if args.calibrate_copy_mib else random_gather_rates(torch)
    traffic = None  # HBM bytes per level_group_kernel launch from the committed counters, if still current
    if fused and not acc64 and args.fuse_batch == 25 and os.path.exists(GROUP_TRAFFIC_FILE):
        with open(GROUP_TRAFFIC_FILE) as f:
            rec = json.load(f)
        if rec.get("source_sha256") == kernel_source_hash():
            traffic = rec["traffic_bytes_per_launch"]
    csr_bytes = 8 * nnz + 4 * (spec.n_rows + 1) + 4 * spec.n_cols + 4 * spec.n_rows
    eng_bytes = cg.device_bytes + 4 * spec.n_cols + yelem * spec.n_rows
    sts = cg.stats
    out = {
        "metric": "nnz/s for y=Mx sweep; achieved HBM GB/s (% peak); device bytes vs CSR",
        "value": nnz * args.steps / elapsed, "unit": "nnz/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32->f64" if acc64 else "f32",
        "data": "synthetic (seeded genotype mosaic)",
        "config": {"workload": args.workload, "n_rows": spec.n_rows, "n_cols": spec.n_cols, "nnz": nnz,
                   "founders": spec.founders, "seg_mean": spec.seg_mean, "mu": spec.mu, "seed": spec.seed,
                   "policy": args.policy, "groups": len(cg.devices), "group_cols": args.group_cols,
                   "fused_group_sweep": fused, "fuse_batch": args.fuse_batch if fused else None,
                   "builder": "device (round-based RePair on the GPU; levels and layout on the host)",
                   "build_s": cg.build_s,
                   "grammar": {"n_rules": sum(s["n_rules"] for s in sts),
                               "n_passthrough": sum(s["n_passthrough"] for s in sts),
                               "c_len": sum(s["c_len"] for s in sts),
                               "n_terminals": sum(s["n_terminals"] for s in sts),
                               "depth_max": max(s["depth"] for s in sts),
                               "max_width_max": max(s["max_width"] for s in sts),
                               "edge_spans": {str(d): espan[d] for d in sorted(espan)}},
                   "launches_per_sweep": cg.launches_per_sweep(),
                   "max_rel_err_sampled": err, "sampled_rows": int(rows.size),
                   "device_bytes": eng_bytes, "csr_bytes_analytic": csr_bytes,
                   "footprint_ratio_csr_over_engine": csr_bytes / eng_bytes,
                   "device_bytes_torch_allocated": int(mem_resident),
                   "hbm_bytes_total": int(torch.cuda.get_device_properties(0).total_memory),
                   "grammar_bytes_per_s": sum(grammar_bytes(s) for s in sts) / (ms_per_step * 1e-3),
                   "sustained": sustained,
                   "wide_levels": nwide, "level_span_ms": span_ms,
                   "bytes_per_sweep": all_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "achieved_from_traffic": (traffic / (span_ms * 1e-3 / max(nwide, 1)) / 1e9) if traffic else None,
                     "kernel": kernel,
                     "launches": nwide, "launch_avg_us": span_ms * 1e3 / max(nwide, 1),
                     "bytes_per_launch_avg": wide_bytes / max(nwide, 1),
                     "copy_achievable_GBs": copy_gbs, "frac_of_copy": achieved / copy_gbs if copy_gbs else None,
                     # the L2 record was taken with the default fp32 policy and batch size
                     "second_bound": l2_bound("level_group_kernel", args.workload, span_ms * 1e3 / max(nwide, 1))
                     if fused and not acc64 and args.fuse_batch == 25 else None,
                     "random_gather_G_per_s_by_window_bytes": gathers},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    cg.free()


def bench_graph(args, wl, spec, leg):
    """Boolean policy on the copy-model digraph: K single passes y = M f from
    the seeded sources (edges/s per pass), then the BFS fixpoint, with the
    oracle's BFS timed on the host cores beside it (CPU leg)."""
    import torch
    from grammar_compressed_sparse_amd import gcs, synth

    t = time.perf_counter()
    rp, col = synth.copy_graph(spec)
    nnz = int(rp[-1])
    log(f"generated copy graph n={spec.n} edges={nnz} in {time.perf_counter() - t:.1f}s")
    t = time.perf_counter()
    g = gcs.build_grammar(rp, col, None, n_cols=spec.n, row_chunk=(spec.n + 127) // 128,
                          row_order=gcs.ROWS_SIMILAR)
    build_s = time.perf_counter() - t
    st = g.stats()
    log(f"grammar built in {build_s:.1f}s: {st}")
    src = synth.sources(spec.n, wl["n_sources"], wl["source_seed"])
    t = time.perf_counter()
    dev = gcs.upload(g, gcs.BOOL_OR)
    torch.cuda.synchronize()
    upload_s = time.perf_counter() - t
    log(f"Boolean upload (host layout of level 0 included) in {upload_s:.1f}s")
    f = torch.zeros(spec.n, dtype=torch.uint8, device="cuda")
    f[torch.from_numpy(src).cuda()] = 1
    y = dev.new_y()
    for _ in range(args.warmup):
        dev.sweep_right(f, y)
    dev.check()
    if leg is not None and not np.array_equal(y.cpu().numpy(), leg.spmv_bool(rp, col, f.cpu().numpy())):
        raise SystemExit("Boolean pass disagrees with the oracle")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dev.sweep_right(f, y)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dev.check()
    roofline = graph_window_roofline(args, gcs, g, dev, f, y)
    t = time.perf_counter()
    vis, counts = dev.bfs(src)
    torch.cuda.synchronize()
    bfs_s = time.perf_counter() - t
    dev.check()
    vis_o = counts_o = cpu = None
    if leg is not None:
        t = time.perf_counter()
        vis_o, counts_o = leg.bfs(rp, col, src)
        bfs_cpu_s = time.perf_counter() - t
        if not (np.array_equal(counts, counts_o) and np.array_equal(vis.cpu().numpy(), vis_o)):
            raise SystemExit("BFS disagrees with the oracle")
        cpu = {"value": nnz * len(counts_o) / bfs_cpu_s, "unit": "nnz/s", "cores": leg.threads(),
               "kind": "oracle", "sample": f"the oracle's BFS fixpoint ({len(counts_o)} Boolean passes "
                                           f"over all edges, {bfs_cpu_s:.1f} s)"}
    tropical = bench_tropical(args, torch, gcs, leg, g, rp, col, spec, src, vis_o, counts_o)
    del g
    # context: rocSPARSE fp32 CSR SpMV (unit values) on the same graph and frontier
    csr = None
    if not args.no_csr:
        csr = csr_comparator(torch, rp, col, np.ones(nnz, np.float32), f.float(), min(args.steps, 20))
        log(f"rocSPARSE fp32 CSR SpMV on the graph: {csr}")
    dev_bytes = dev.device_bytes + 2 * spec.n
    csr_bytes = 4 * nnz + 4 * (spec.n + 1) + 2 * spec.n
    out = {
        "metric": "nnz/s for y=Mx sweep; achieved HBM GB/s (% peak); device bytes vs CSR",
        "value": nnz * args.steps / elapsed, "unit": "nnz/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic (seeded copy-model digraph)",
        "config": {"workload": args.workload, "n": spec.n, "nnz": nnz, "sources": len(src),
                   "grammar": {k: st[k] for k in ("n_rules", "n_passthrough", "depth", "max_width", "c_len",
                                                  "n_terminals", "n_tiles", "n_emit_groups")},
                   "build_s": build_s, "upload_s": upload_s, "bfs_passes": len(counts), "bfs_s": bfs_s,
                   "visited": int(vis.sum().item()),
                   "device_bytes": dev_bytes, "csr_bytes_analytic": csr_bytes,
                   "footprint_ratio_csr_over_engine": csr_bytes / dev_bytes, "tropical": tropical,
                   "csr_rocsparse_fp32": csr},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def graph_window_roofline(args, gcs, g, dev, f, y):
    """The largest single kernel of a Boolean pass: level 0's word-stream
    emission (window_emit_kernel), launched right after the terminal array
    and level 1's launch.  Algorithmic bytes per launch: 4 per word plus
    each chunk's window of terminal bits, loaded once (the words and chunk
    table as the upload lays them out, from gcs_level0_words on the host);
    duration: HIP events around every launch of args.steps passes (after
    the timed region)."""
    lw = g.level0_words(gcs.BOOL_OR)
    if lw["words"].size == 0:
        return None
    ch = lw["chunks"].astype(np.int64)
    alg = 4 * int(lw["words"].size) + int((ch[:, 3] - ch[:, 2]).sum())
    idx = 2 if int(g.level_widths()[1]) > 0 else 1  # leaf, level 1 (if any), then the words
    dev.profile_begin(args.steps, gcs.PROFILE_LAUNCHES)
    for _ in range(args.steps):
        dev.sweep_right_profiled(f, y)
    launch_ms = dev.profile_end()
    dev.check()
    us = float(launch_ms[:, idx].mean() * 1e3)
    achieved = alg / (us * 1e-6) / 1e9
    log(f"window_emit_kernel: {alg / 1e9:.2f} GB algorithmic per launch in {us:.0f} us: {achieved:.0f} GB/s")
    return {"bound": "hbm", "achieved": achieved, "peak": 8000.0, "unit": "GB/s", "frac": achieved / 8000.0,
            "traffic": None,
            "kernel": "window_emit_kernel (level 0's 32-bit words and each chunk's LDS window of terminal bits; "
                      "HIP events around each launch)",
            "launch_avg_us": us, "bytes_per_launch": alg, "words": int(lw["words"].size),
            "chunks": int(ch.shape[0])}


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-kernel-trace":
        # bench.py --summarize-kernel-trace KT_DIR OUT_MD TITLE "command" ...
        summarize_kernel_trace(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-group-counters":
        # bench.py --summarize-group-counters FETCH_DIR WRITE_DIR OUT_MD COPY_MIB BENCH_LOG "command" ...
        summarize_group_counters(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), sys.argv[7:],
                                 [sys.argv[6]])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-group-trace":
        # bench.py --summarize-group-trace KT_DIR OUT_MD TITLE BENCH_LOG "command" ...
        summarize_group_trace(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[6:], bench_log=sys.argv[5])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--filter-counters":
        # bench.py --filter-counters IN_DIR OUT_DIR KERNEL
        filter_counters(sys.argv[2], sys.argv[3], sys.argv[4])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-l2":
        # bench.py --summarize-l2 HIT_DIR OUT_MD KERNEL WORKLOAD "command" ...
        summarize_l2(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-per-level":
        # bench.py --summarize-per-level KT_DIR FETCH_DIR WRITE_DIR LEVELS_JSON OUT_MD COPY_MIB "command" ...
        summarize_per_level(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], int(sys.argv[7]),
                            sys.argv[8:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-rocprof":
        # bench.py --summarize-rocprof KT_DIR FETCH_DIR WRITE_DIR OUT_MD COPY_MIB "command" ...
        summarize_rocprof(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], int(sys.argv[6]), sys.argv[7:])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="genotype_200000x2000000_f32")
    ap.add_argument("--col-chunk", type=int, default=2000)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg: the oracle's timing and the sampled checks against it")
    ap.add_argument("--no-csr", action="store_true")
    ap.add_argument("--group-cols", type=int, default=20_000,
                    help="columns per group of the 200,000 x 2,000,000 workload (each group one device build)")
    ap.add_argument("--build-workers", type=int, default=4,
                    help="groups of the 200,000 x 2,000,000 workload built concurrently")
    ap.add_argument("--no-fuse", action="store_true",
                    help="200,000 x 2,000,000 workload: sweep the column groups one after the other (shared "
                         "workspace) instead of one launch per level for all groups")
    ap.add_argument("--fuse-batch", type=int, default=25,
                    help="200,000 x 2,000,000 workload: column groups per fused sweep (each needs its own "
                         "workspace; batches share them)")
    ap.add_argument("--policy", default="f32", choices=["f32", "f32_acc_f64"],
                    help="200,000 x 2,000,000 workload: fp32, or fp32 x with fp64 accumulation")
    ap.add_argument("--batches", default="32,64",
                    help="batched sweeps (Y = M X) to time after the headline, comma-separated B; empty: none")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run 5 device-to-device copies of this many MiB (a known-size reference kernel "
                         "for hardware traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the sweep is a single-GPU engine here (multi-GPU sharding is a "
              "design note, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from grammar_compressed_sparse_amd import gcs, synth

    leg = None if args.no_cpu_baseline else CpuLeg()
    if args.calibrate_copy_mib:
        nb = args.calibrate_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration: 5 copies of {args.calibrate_copy_mib} MiB ({nb} bytes read and written per copy)")
        del src, dst

    wl = synth.WORKLOADS[args.workload]
    spec = wl["matrix"]
    if isinstance(spec, synth.GraphSpec):
        return bench_graph(args, wl, spec, leg)
    if spec.n_rows * spec.n_cols > 1e11:
        return bench_biobank(args, wl, spec, leg)
    t = time.perf_counter()
    rp, col, val = synth.genotype(spec)
    nnz = int(rp[-1])
    log(f"generated {spec.n_rows}x{spec.n_cols} nnz={nnz} in {time.perf_counter() - t:.1f}s")
    t = time.perf_counter()
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols, col_chunk=args.col_chunk)
    build_s = time.perf_counter() - t
    st = g.stats()
    log(f"grammar built in {build_s:.1f}s: {st}")
    lay = g.layout()
    lay["alpha"] = st["n_terminals"]
    policy = gcs.PLUS_F32 if wl["dtype"] == "f32" else gcs.PLUS_F64
    xdt = np.float32 if wl["dtype"] == "f32" else np.float64
    elem = 4 if wl["dtype"] == "f32" else 8

    torch.cuda.init()
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    t = time.perf_counter()
    dev = gcs.upload(g, policy)
    torch.cuda.synchronize()
    upload_s = time.perf_counter() - t
    upload_peak = torch.cuda.max_memory_allocated() - mem0  # cross-check of the footprint
    xs = [torch.from_numpy(synth.normal(spec.n_cols, s).astype(xdt)).cuda() for s in wl["x_seeds"]]
    y = dev.new_y()
    log(f"uploaded {dev.device_bytes / 1e6:.1f} MB in {upload_s:.2f}s; {dev.sweep_launches()} launches per sweep")

    # correctness on sampled rows (outside the timed region; CPU leg)
    dev.sweep_right(xs[0], y)
    dev.check()
    if leg is not None:
        rows = np.unique(np.concatenate([np.arange(0, spec.n_rows, max(1, spec.n_rows // 512)), [spec.n_rows - 1]]))
        tol = 1e-5 if elem == 4 else 1e-12
        err = leg.check_rows("sweep", y.cpu().numpy()[rows], rows, rp, col, val,
                             xs[0].cpu().numpy().astype(np.float64), tol)
        log(f"sampled-row check: {rows.size} rows, max rel err {err:.2e} (tol {tol})")

    for i in range(args.warmup):
        dev.sweep_right(xs[i % len(xs)], y)
    torch.cuda.synchronize()
    # timed region: K sweeps, each with one pair of HIP events (on the sweep's
    # stream) around its wide level launches, the dominant kernel
    dev.profile_begin(args.steps, gcs.PROFILE_LEVEL_SPAN)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        dev.sweep_right_profiled(xs[i % len(xs)], y)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    spans = dev.profile_end()[:, 0]
    span_ms = float(spans.mean())
    dev.check()
    ms_per_step = elapsed * 1e3 / args.steps
    # sustained: back-to-back sweeps for at least 1.5 s (after the timed region)
    torch.cuda.synchronize()
    t0, sweeps = time.perf_counter(), 0
    while True:
        for i in range(50):
            dev.sweep_right(xs[i % len(xs)], y)
        sweeps += 50
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= 1.5:
            break
    sustained = {"seconds": time.perf_counter() - t0, "sweeps": sweeps}
    sustained["nnz_per_s"] = nnz * sweeps / sustained["seconds"]
    dev.check()
    # breakdown (after the timed region): events around every launch, which
    # add a gap between launches, so these sum to more than a clean sweep
    dev.profile_begin(args.steps, gcs.PROFILE_LAUNCHES)
    for i in range(args.steps):
        dev.sweep_right_profiled(xs[i % len(xs)], y)
    launch_ms = dev.profile_end()  # (steps, launches)
    dev.check()
    L = st["depth"]
    # launch 0 = terminal array, 1..k0-1 = wide levels (each with the emission
    # of the level below), last = the persistent tail (levels k0..L, the last
    # emission and the slice reduction)
    nwide = launch_ms.shape[1] - 2
    lvl_ms = launch_ms[:, 1:1 + nwide].mean(axis=0)
    tail_ms = float(launch_ms[:, -1].mean())
    lb_all = level_bytes(lay, elem, elem)
    lb = lb_all[:nwide]
    if nwide > 0:
        achieved = lb.sum() / (span_ms * 1e-3) / 1e9
        kernel = ("level_kernel (the wide levels of a sweep, one launch each; timed from before the first to "
                  "after the last, gaps between launches included)")
    else:
        # every level fits the persistent tail: that launch is the dominant
        # kernel (its time from the per-launch breakdown)
        achieved = lb_all.sum() / (tail_ms * 1e-3) / 1e9
        kernel = "tail_kernel (all levels in one persistent launch)"
    per_level = [{"k": k + 1, "width": int(lay["level_meta"][k + 1][0] + lay["level_meta"][k + 1][1]),
                  "bytes": int(lb[k]), "us": float(lvl_ms[k] * 1e3),
                  "GBs": float(lb[k] / (lvl_ms[k] * 1e-3) / 1e9)} for k in range(nwide)]
    widest = int(np.argmax([p["width"] for p in per_level])) if per_level else 0

    per_vector = None
    if len(xs) > 1:
        # multiply-many: one sweep per vector, latency of each measured with
        # events on the sweep's stream (after the timed region)
        lat = []
        for xv in xs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dev.sweep_right(xv, y)
            e1.record()
            e1.synchronize()
            lat.append(e0.elapsed_time(e1))
        lat = np.array(lat)
        per_vector = {"vectors": len(xs), "median_ms": float(np.median(lat)), "p90_ms": float(np.percentile(lat, 90)),
                      "aggregate_nnz_per_s": float(nnz * len(xs) / (lat.sum() * 1e-3))}
        log(f"per-vector latency over {len(xs)} vectors: median {per_vector['median_ms']:.3f} ms, "
            f"p90 {per_vector['p90_ms']:.3f} ms")

    csr_bytes = 8 * nnz + 4 * (spec.n_rows + 1) + 4 * spec.n_cols + 4 * spec.n_rows
    eng_bytes = dev.device_bytes + xs[0].numel() * elem + y.numel() * elem
    csr = None if args.no_csr else csr_comparator(torch, rp, col, val, xs[0], min(args.steps, 20))
    batched = None
    if args.batches:
        batched = bench_batched(torch, gcs, leg, synth, dev, lay, rp, col, val, spec, elem, xdt,
                                [int(b) for b in args.batches.split(",")], min(args.steps, 20))
    cpu = None
    if leg is not None:
        cpu = leg.baseline(rp, col, val, xs[0].cpu().numpy().astype(np.float64), nnz)

    # (not in counter runs: its copies would mix with the calibration's)
    copy_gbs = None if args.calibrate_copy_mib else copy_achievable_gbs(torch)
    gathers = None if args.calibrate_copy_mib else random_gather_rates(torch)
    traffic = None  # HBM bytes per level_kernel launch from the committed counter profile, if still current
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        if (rec.get("source_sha256") == kernel_source_hash() and args.workload == "genotype_20000x100000_f32"
                and nwide > 0):
            traffic = rec["traffic_bytes_per_launch"]
    value = nnz * args.steps / elapsed
    out = {
        "metric": "nnz/s for y=Mx sweep; achieved HBM GB/s (% peak); device bytes vs CSR",
        "value": value,
        "unit": "nnz/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if elem == 4 else "f64",
        "data": "synthetic (seeded genotype mosaic)",
        "config": {
            "workload": args.workload,
            "n_rows": spec.n_rows, "n_cols": spec.n_cols, "nnz": nnz,
            "founders": spec.founders, "seg_mean": spec.seg_mean, "mu": spec.mu, "seed": spec.seed,
            "vectors": len(xs),
            "multiply_many": per_vector,
            "grammar": dict({k: st[k] for k in ("n_rules", "n_passthrough", "depth", "max_width", "c_len",
                                                "n_terminals", "n_tiles", "n_emit_groups")},
                            edge_spans={str(d): int(c) for d, c in enumerate(g.edge_spans().tolist()) if c}),
            "build_s": build_s, "upload_s": upload_s,
            "launches_per_sweep": int(launch_ms.shape[1]),
            "grammar_bytes_per_s": grammar_bytes(st) / (ms_per_step * 1e-3),
            "device_bytes": eng_bytes, "csr_bytes_analytic": csr_bytes,
            "upload_bytes_torch_peak": int(upload_peak),
            "footprint_ratio_csr_over_engine": csr_bytes / eng_bytes,
            "csr_rocsparse": csr,
            "batched": batched,
            "per_level_widest": per_level[widest] if per_level else None,
            "wide_levels": nwide,
            "level_span_us": span_ms * 1e3,
            "level_span_us_median": float(np.median(spans) * 1e3),
            "sustained": sustained,
            "level_us_total_launch_events": float(lvl_ms.sum() * 1e3),
            "leaf_us": float(launch_ms[:, 0].mean() * 1e3),
            "tail_us": tail_ms * 1e3,
            "tail_levels": L - nwide,
            "tail_bytes": float(lb_all[nwide:].sum()),
        },
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel,
                     "launches": int(max(nwide, 1)),
                     "launch_avg_us": span_ms * 1e3 / nwide if nwide > 0 else tail_ms * 1e3,
                     "achieved_from_traffic": (traffic / (span_ms * 1e-3 / max(nwide, 1)) / 1e9) if traffic else None,
                     "copy_achievable_GBs": copy_gbs, "frac_of_copy": achieved / copy_gbs if copy_gbs else None,
                     "bytes_per_launch_avg": float(lb.sum() / nwide if nwide > 0 else lb_all.sum()),
                     "bytes_per_sweep": float(lb_all.sum()),
                     "second_bound": l2_bound("level_kernel", args.workload, span_ms * 1e3 / nwide)
                     if nwide > 0 else None,
                     "random_gather_G_per_s_by_window_bytes": gathers},
        "cpu_baseline": cpu,
    }
    if os.environ.get("GCS_BENCH_LEVELS"):
        out["config"]["per_level"] = per_level
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
