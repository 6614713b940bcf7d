"""Column groups swept together (gcs_group_*): every group's level k in one
launch, then one reduction of every group's slice accumulators.  The result
must equal, bit for bit, gcs_sweep_right on group 0 followed by
gcs_sweep_right_acc on the others (the same additions in the same order),
and the oracle within the policy's tolerance."""

import numpy as np
import pytest

import helpers

pytestmark = pytest.mark.gpu


def _say(msg):
    helpers.progress(msg)


@pytest.fixture(scope="module")
def parts(synth_mod):
    from grammar_compressed_sparse_amd import gcs
    spec = synth_mod.GenotypeSpec(2000, 12000, 32, 300.0, 0.002, seed=13)
    rp, col, val = synth_mod.genotype(spec)
    # four groups of unequal width (one built on the device), and an empty one
    cuts = [(0, 2500), (2500, 4000), (6500, 3000), (9500, 2500)]
    gs = []
    for i, (c0, nc) in enumerate(cuts):
        prp, pcol, pval = synth_mod.genotype(spec, col0=c0, ncols=nc)
        if i == 1:
            gs.append(gcs.build_grammar_gpu(prp, pcol, pval, n_cols=spec.n_cols))
        else:
            gs.append(gcs.build_grammar(prp, pcol, pval, n_cols=spec.n_cols))
    gs.append(gcs.build_grammar(np.zeros(spec.n_rows + 1, np.int64), np.zeros(0, np.int32), None,
                                n_cols=spec.n_cols))
    return spec, rp, col, val, gs


@pytest.mark.parametrize("policy", ["f32", "f64", "f32_acc_f64", "i64"])
def test_group_sweep_equals_chain_and_oracle(parts, oracle_mod, synth_mod, policy):
    import torch
    from grammar_compressed_sparse_amd import gcs
    spec, rp, col, val, gs = parts
    pol = gcs.POLICY_NAMES[policy]
    _say(f"group sweep: {len(gs)} groups, policy {policy}")
    devs = [gcs.upload(g, pol) for g in gs]
    grp = gcs.Group(devs)
    assert grp.launches() == max(g.stats()["depth"] for g in gs) + 1 + 2
    if policy == "i64":
        xh = np.arange(spec.n_cols, dtype=np.int64) % 7 - 3
    else:
        xh = synth_mod.normal(spec.n_cols, 77).astype(np.float64 if policy == "f64" else np.float32)
    x = torch.from_numpy(xh).cuda()
    y = grp.sweep_right(x)
    yc = devs[0].sweep_right(x)
    for d in devs[1:]:
        d.sweep_right_acc(x, yc)
    for d in devs:
        d.check()
    assert torch.equal(y, yc)
    yh = y.cpu().numpy()
    if policy == "i64":
        assert np.array_equal(yh, oracle_mod.spmv_i64(rp, col, val, xh))
    else:
        yo, absum = oracle_mod.spmv_f64(rp, col, val, xh.astype(np.float64))
        tol = 1e-5 if policy == "f32" else 1e-12
        assert np.all(np.abs(yh.astype(np.float64) - yo) <= tol * absum)
    # accumulate: y + M x, again bit for bit against the chain
    y2 = y.clone()
    grp.sweep_right(x, y2, accumulate=True)
    yc2 = yc.clone()
    for d in devs:
        d.sweep_right_acc(x, yc2)
    assert torch.equal(y2, yc2)
    # profiled sweeps give one span per sweep
    grp.profile_begin(3)
    for _ in range(3):
        grp.sweep_right(x, y, profiled=True)
    spans = grp.profile_end()
    assert spans.shape == (3,) and np.all(spans > 0)
    grp.free()


def test_group_refusals(parts):
    import torch
    from grammar_compressed_sparse_amd import gcs
    spec, rp, col, val, gs = parts
    ws = torch.empty(max(gs[0].device_layout(gcs.PLUS_F32)["workspace_bytes"],
                         gs[2].device_layout(gcs.PLUS_F32)["workspace_bytes"]), dtype=torch.uint8, device="cuda")
    shared = [gcs.upload(gs[0], gcs.PLUS_F32, workspace=ws), gcs.upload(gs[2], gcs.PLUS_F32, workspace=ws)]
    with pytest.raises(gcs.GcsError, match="EINVAL"):  # overlapping workspaces
        gcs.Group(shared)
    mixed = [gcs.upload(gs[0], gcs.PLUS_F32), gcs.upload(gs[2], gcs.PLUS_F64)]
    with pytest.raises(gcs.GcsError, match="EINVAL"):  # two policies
        gcs.Group(mixed)
    with pytest.raises(gcs.GcsError, match="EINVAL"):  # not a plus-times policy
        gcs.Group([gcs.upload(gs[0], gcs.BOOL_OR)])
