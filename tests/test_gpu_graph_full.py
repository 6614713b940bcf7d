"""Full-size graph workload: the 50M-node copy-model digraph (about 1e9 edges),
Boolean policy, BFS fixpoint from 16 seeded sources; bit-exact against the
oracle (visited set and the new-node count of every pass).

The grammar is built over 128 row tiles in MinHash row order (rows that share
many out-neighbours share a tile), RePair running on the tiles in parallel.
This is the heaviest test (about 1 GB of edges generated sequentially, a
multi-minute host build); it prints each step.
"""
import time

import numpy as np
import pytest

import helpers

pytestmark = pytest.mark.gpu


def _say(msg):
    helpers.progress(msg)


def test_copy_graph_50M_bfs(synth_mod, oracle_mod):
    import torch
    from grammar_compressed_sparse_amd import gcs
    wl = synth_mod.WORKLOADS["copy_graph_50M_bfs16"]
    spec = wl["matrix"]
    t = time.time()
    rp, col = synth_mod.copy_graph(spec)
    _say(f"generated copy graph n={spec.n} edges={rp[-1]} in {time.time() - t:.0f}s")
    t = time.time()
    g = gcs.build_grammar(rp, col, None, n_cols=spec.n, row_chunk=(spec.n + 127) // 128,
                          row_order=gcs.ROWS_SIMILAR)
    st = g.stats()
    _say(f"grammar in {time.time() - t:.0f}s: {st}")
    src = synth_mod.sources(spec.n, wl["n_sources"], wl["source_seed"])
    dev = gcs.upload(g, gcs.BOOL_OR)
    lay = g.device_layout(gcs.BOOL_OR)
    del g
    torch.cuda.synchronize()
    t = time.time()
    vis, counts = dev.bfs(src)
    torch.cuda.synchronize()
    dev.check()
    _say(f"GPU BFS: {len(counts)} passes in {time.time() - t:.2f}s, visited {int(vis.sum().item())}, "
         f"device bytes {lay['grammar_bytes'] + lay['workspace_bytes']}")
    t = time.time()
    vis_o, counts_o = oracle_mod.bfs(rp, col, src)
    _say(f"oracle BFS: {len(counts_o)} passes in {time.time() - t:.1f}s on {oracle_mod.num_threads()} threads")
    assert np.array_equal(counts, counts_o)
    assert np.array_equal(vis.cpu().numpy(), vis_o)
    # one Boolean pass alone from the sources
    xb = torch.zeros(spec.n, dtype=torch.uint8, device="cuda")
    xb[torch.from_numpy(src).cuda()] = 1
    y = dev.sweep_right(xb)
    dev.check()
    xh = np.zeros(spec.n, np.uint8)
    xh[src] = 1
    assert np.array_equal(y.cpu().numpy(), oracle_mod.spmv_bool(rp, col, xh))
