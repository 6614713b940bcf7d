"""The C-ABI library loads and exports every function include/gcs.h declares
(no compute calls: this runs without a GPU)."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(gcs_[a-z0-9_]+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


def test_exports_every_declared_symbol():
    from grammar_compressed_sparse_amd import gcs
    lib = ctypes.CDLL(gcs.library_path())
    names = declared_functions()
    assert len(names) >= 18
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, missing


def test_header_compiles_as_c():
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        with open(src, "w") as f:
            f.write('#include "gcs.h"\nint main(void){ gcs_stats s; (void)s; return 0; }\n')
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-c", src, "-o",
                        os.path.join(d, "t.o")], check=True)
