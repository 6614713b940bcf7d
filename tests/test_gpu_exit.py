"""A process that leaves device handles alive at exit must still end cleanly.

Handles not freed by the program (a Device, a batch Group) are released by
the library binding's atexit hook, before torch's and the HIP runtime's own
teardown, so no HIP call is left for object finalization at interpreter
shutdown.  Each case runs in a child process (the parent's GPU state is not
touched) with both tail launch kinds, and must exit with status 0."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np
import torch
from grammar_compressed_sparse_amd import gcs, synth
spec = synth.GENOTYPE_512x4096
rp, col, val = synth.genotype(spec)
g = gcs.build_grammar_gpu(rp, col, val, n_cols=spec.n_cols)
d = gcs.upload(g, gcs.PLUS_F64)
x = torch.from_numpy(np.random.default_rng(1).standard_normal(spec.n_cols)).cuda()
y = d.sweep_right(x)
d.check()
ws = torch.empty(d.workspace.numel() * 2, dtype=torch.uint8, device="cuda")
d2 = gcs.upload(g, gcs.PLUS_F64, workspace=ws)
grp = gcs.Group([d2])
y2 = grp.sweep_right(x, d2.new_y())
torch.cuda.synchronize()
assert torch.equal(y, y2)
print("child done", flush=True)
# d, d2 and grp are left alive on purpose
"""


@pytest.mark.parametrize("coop", ["0", "1"])
def test_exit_with_live_handles_is_clean(coop):
    env = dict(os.environ, GCS_TAIL_COOP=coop, PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    print(f"child process with live handles at exit, GCS_TAIL_COOP={coop}", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert "child done" in r.stdout
    assert r.returncode == 0, r.stderr[-2000:]
