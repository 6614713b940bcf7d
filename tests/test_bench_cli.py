"""Host-side checks of bench.py's contract (no device): more than one GPU is
refused with a message and no result line, and the kernel-source hash that
decides whether recorded hardware-counter traffic still applies ignores
comments and whitespace but not code."""
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
    assert hashes["base"] == hashes["comment"] == hashes["spaces"]
    assert hashes["code"] != hashes["base"]
