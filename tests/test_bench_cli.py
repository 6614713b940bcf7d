"""Host-side checks of bench.py's contract (no device): more than one GPU is
refused with a message and no result line, and the source hash that decides
whether recorded hardware-counter figures still apply (kernels and layout)
ignores comments and whitespace but not code."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert '"metric"' not in r.stdout


def test_kernel_source_hash(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    code = "template <class P>\n__global__ void k(int* p) {\n    p[0] = 1;  // store\n}\n"
    variants = {
        "base": code,
        "comment": code.replace("// store", "// a different comment") + "/* trailing\n block */\n",
        "spaces": code.replace("    p[0] = 1;", "\tp[0]   =   1;"),
        "code": code.replace("p[0] = 1;", "p[0] = 2;"),
    }
    hashes = {}
    for name, text in variants.items():
        f = tmp_path / f"{name}.hpp"
        f.write_text(text)
        monkeypatch.setattr(bench, "KERNEL_SOURCE", str(f))
        hashes[name] = bench.kernel_source_hash()
    # the layout source counts as well
    lay = tmp_path / "layout.cpp"
    lay.write_text("int order;\n")
    monkeypatch.setattr(bench, "LAYOUT_SOURCE", str(lay))
    before = bench.kernel_source_hash()
    lay.write_text("int order = 1;\n")
    assert bench.kernel_source_hash() != before
    lay.write_text("int order;  // comment\n")
    assert bench.kernel_source_hash() == before
    assert hashes["base"] == hashes["comment"] == hashes["spaces"]
    assert hashes["code"] != hashes["base"]


def _counter_csv(path, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_l2_record_and_bound(tmp_path, monkeypatch):
    """summarize_l2 averages TCC_HIT_sum + TCC_MISS_sum over the dispatches of
    the named kernel only (level_kernel is not level_group_kernel or
    level_batch_kernel), records them under kernel:workload with the source
    hash, and l2_bound turns them into a rate against the request peak; a
    changed kernel source voids the record."""
    sys.path.insert(0, ROOT)
    import bench
    d = tmp_path / "pmc"
    d.mkdir()
    rows = []
    for i in range(4):  # level_kernel: 900 + 100 i hits, 100 misses
        rows += [(i, "void gcs::level_kernel<gcs::PolPlusF32>(gcs::LevelArgs)", "TCC_HIT_sum", 900 + 100 * i),
                 (i, "void gcs::level_kernel<gcs::PolPlusF32>(gcs::LevelArgs)", "TCC_MISS_sum", 100)]
    rows += [(10, "void gcs::level_batch_kernel<gcs::PolPlusF32, 4, false>(x)", "TCC_HIT_sum", 1e9),
             (11, "void gcs::level_group_kernel<gcs::PolPlusF32>(x)", "TCC_MISS_sum", 1e9)]
    _counter_csv(d / "run_counter_collection.csv", rows)
    src = tmp_path / "k.hpp"
    src.write_text("int a;\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    monkeypatch.setattr(bench, "LAYOUT_SOURCE", str(src))
    monkeypatch.setattr(bench, "L2_FILE", str(tmp_path / "l2.json"))
    bench.summarize_l2(str(d), str(tmp_path / "out.md"), "level_kernel", "wl", ["cmd"])
    b = bench.l2_bound("level_kernel", "wl", launch_avg_us=1.0)
    assert b["requests_per_launch"] == 1150.0  # mean of 1000, 1100, 1200, 1300
    assert abs(b["hit_rate"] - 4200 / 4600) < 1e-12
    assert abs(b["achieved"] - 1150.0 / 1e-6 / 1e9) < 1e-9 and b["unit"] == "G requests/s"
    assert abs(b["frac"] - b["achieved"] / bench.L2_REQ_PEAK_G) < 1e-12
    assert bench.l2_bound("level_kernel", "other", 1.0) is None
    src.write_text("int b;\n")
    assert bench.l2_bound("level_kernel", "wl", 1.0) is None


def test_grammar_bytes_formula():
    """(8 N_bin + 4 N_pt + 8 |C| + 4 alpha): the bytes of the grammar a sweep
    streams."""
    sys.path.insert(0, ROOT)
    import bench
    st = {"n_rules": 10, "n_passthrough": 3, "c_len": 7, "n_terminals": 5}
    assert bench.grammar_bytes(st) == 8 * 10 + 4 * 3 + 8 * 7 + 4 * 5


def test_group_counters_record_and_filter(tmp_path, monkeypatch):
    """filter_counters keeps the named kernel's dispatches and the first
    copies only; summarize_group_counters scales FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) by what the same counter reads for the 1 GiB
    calibration copies, takes each counter's rows by name (a pass may carry
    others), and records the mean bytes per launch with the source hash."""
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "k.hpp"
    src.write_text("int a;\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(src))
    monkeypatch.setattr(bench, "LAYOUT_SOURCE", str(src))
    monkeypatch.setattr(bench, "GROUP_TRAFFIC_FILE", str(tmp_path / "gt.json"))
    kern = "void gcs::level_group_kernel<gcs::PolPlusF32>(x)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE reads half of the copied bytes (scale 2), WRITE_SIZE all of them
    fetch = [(1, copy, "FETCH_SIZE", 512 * 1024), (2, copy, "FETCH_SIZE", 512 * 1024)]
    fetch += [(10 + i, kern, "FETCH_SIZE", 1000 + 100 * i) for i in range(3)]
    fetch += [(100 + i, "void gcs::gb::k_count(x)", "FETCH_SIZE", 9e9) for i in range(50)]
    write = [(1, copy, "WRITE_SIZE", 1024 * 1024), (1, copy, "TCC_HIT_sum", 5)]
    write += [(10 + i, kern, "WRITE_SIZE", 400) for i in range(3)]
    write += [(10 + i, kern, "TCC_MISS_sum", 7e9) for i in range(3)]
    for name, rows in (("f", fetch), ("w", write)):
        raw = tmp_path / ("raw_" + name)
        raw.mkdir()
        _counter_csv(raw / "x_counter_collection.csv", rows)
        bench.filter_counters(str(raw), str(tmp_path / name), "level_group_kernel", n_copies=2)
    import csv
    kept = list(csv.DictReader(open(tmp_path / "f" / "filtered_counter_collection.csv")))
    assert {r["Dispatch_Id"] for r in kept} == {"1", "2", "10", "11", "12"}
    bench.summarize_group_counters(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "out.md"), 1024, ["cmd"],
                                   [])
    import json
    rec = json.load(open(tmp_path / "gt.json"))
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    assert abs(rec["fetch_bytes_per_launch"] - 1100 * 1024 * 2.0) < 1e-6
    assert abs(rec["write_bytes_per_launch"] - 400 * 1024) < 1e-6
    assert rec["traffic_bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["source_sha256"] == bench.kernel_source_hash()
