"""The device builder (gcs_build_grammar_gpu) through the C ABI.

Its grammar must be the host round-based RePair's bit for bit (the same
rules in the same order, the same C, hence the same layout), on inputs that
cover the value kinds (Boolean, int8, fp64 with stored zeros), empty and
single rows, identical rows, and a graph whose pair table has to grow during
a round.  The sweep of the device-built grammar is then checked against the
oracle (fp64, 1e-12 of the row's sum of |terms|).
"""
import random
import time

import numpy as np
import pytest

import helpers as H

pytestmark = pytest.mark.gpu


def _say(msg):
    H.progress(msg)


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from grammar_compressed_sparse_amd import gcs
    return torch, gcs


def _random_zeros(seed):
    rng = random.Random(seed)
    n, m = 300, 200
    rows = []
    for r in range(n):
        if r % 7 == 3:
            rows.append([])  # empty rows
            continue
        rows.append(sorted(rng.sample(range(m), rng.randint(1, 60))))
    rp = np.zeros(n + 1, np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    col = np.array([c for r in rows for c in r], np.int32)
    vals = [0.0, -1.5, 0.25, 3.0, 7.5]  # some stored zeros, dropped by CSRV
    val = np.array([rng.choice(vals) for _ in range(col.size)], np.float64)
    return rp, col, val, m


def _case(name, worked_example, synth_mod):
    if name == "worked_example":
        rp, col, val = H.csr_from_dense(worked_example["M"]["rows"])
        return rp, col, val, 7
    if name == "genotype_512x4096":
        spec = synth_mod.GENOTYPE_512x4096
        return (*synth_mod.genotype(spec), spec.n_cols)
    if name == "genotype_2000x12000":
        spec = synth_mod.GenotypeSpec(2000, 12000, 32, 300.0, 0.002, seed=13)
        return (*synth_mod.genotype(spec), spec.n_cols)
    if name == "copy_graph_20000":
        spec = synth_mod.GraphSpec(20_000, seed=8)
        rp, col = synth_mod.copy_graph(spec)
        return rp, col, None, spec.n
    if name == "random_f64_zeros_empty_rows":
        return _random_zeros(5)
    if name == "identical_rows":
        n, k = 40, 97
        return np.arange(n + 1, dtype=np.int64) * k, np.tile(np.arange(k, dtype=np.int32), n), None, k
    if name == "single_row":
        return np.array([0, 500], np.int64), np.arange(0, 1000, 2, dtype=np.int32), None, 1000
    if name == "empty":
        return np.zeros(8, np.int64), np.zeros(0, np.int32), None, 9
    raise KeyError(name)


CASES = ["worked_example", "genotype_512x4096", "genotype_2000x12000", "copy_graph_20000",
         "random_f64_zeros_empty_rows", "identical_rows", "single_row", "empty"]


@pytest.mark.parametrize("name", CASES)
def test_device_builder_equals_host_rounds(env, oracle_mod, synth_mod, worked_example, name):
    torch, gcs = env
    rp, col, val, m = _case(name, worked_example, synth_mod)
    _say(f"device builder vs host rounds: {name} rows={rp.size - 1} nnz={int(rp[-1])}")
    t = time.time()
    gd = gcs.build_grammar_gpu(rp, col, val, n_cols=m)
    td = time.time() - t
    t = time.time()
    gh = gcs.build_grammar(rp, col, val, n_cols=m, repair=gcs.REPAIR_ROUNDS)
    th = time.time() - t
    sd, sh = gd.stats(), gh.stats()
    _say(f"  device {td:.2f}s host {th:.2f}s |R|={sd['n_rules']} |C|={sd['c_len']} L={sd['depth']}")
    for k in ("nnz", "n_values", "n_terminals", "n_rules", "n_passthrough", "depth", "max_width", "c_len",
              "n_emit_groups"):
        assert sd[k] == sh[k], k
    ed, eh = gd.export(), gh.export()
    for k in eh:
        assert np.array_equal(ed[k], eh[k]), k
    ld, lh = gd.layout(), gh.layout()
    for k in ("level_meta", "child", "ptsrc", "erow", "eoff", "epos", "slices", "col_cut"):
        assert np.array_equal(ld[k], lh[k]), k
    if int(rp[-1]) == 0:
        return
    vv = np.ones(int(rp[-1])) if val is None else val
    x = np.random.default_rng(3).standard_normal(m)
    dev = gcs.upload(gd, gcs.PLUS_F64)
    y = dev.sweep_right(torch.from_numpy(x).cuda())
    dev.check()
    yo, absum = oracle_mod.spmv_f64(rp, col, vv, x)
    err = np.abs(y.cpu().numpy() - yo)
    assert np.all(err <= 1e-12 * absum)


def test_device_builder_table_and_workspace_errors(env, synth_mod):
    torch, gcs = env
    spec = synth_mod.GraphSpec(20_000, seed=8)
    rp, col = synth_mod.copy_graph(spec)
    _say("device builder: table of 1024 slots for ~4e5 distinct pairs -> GCS_ENOMEM")
    with pytest.raises(gcs.GcsError, match="ENOMEM"):
        gcs.build_grammar_gpu(rp, col, None, n_cols=spec.n, table_entries=1024)
    with pytest.raises(gcs.GcsError, match="EINVAL"):  # not a power of two
        gcs.build_workspace_bytes(10, 10, 100, 3000)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(gcs.GcsError, match="EINVAL"):
        gcs.build_grammar_gpu(rp, col, None, n_cols=spec.n, workspace=small)
    with pytest.raises(gcs.GcsError, match="EINVAL"):  # more than 64 distinct values
        rp1 = np.array([0, 100], np.int64)
        gcs.build_grammar_gpu(rp1, np.arange(100, dtype=np.int32), np.arange(1, 101, dtype=np.float64),
                              n_cols=100)
    # a smaller table than the default still gives the same grammar
    a = gcs.build_grammar_gpu(rp, col, None, n_cols=spec.n, table_entries=1 << 20).export()
    b = gcs.build_grammar_gpu(rp, col, None, n_cols=spec.n).export()
    for k in a:
        assert np.array_equal(a[k], b[k]), k
