"""Seeded generators: determinism, block consistency and the statistics the
workload recipes promise (about 30% nonzero genotypes; mean out-degree 20)."""
import math

import numpy as np


def test_genotype_deterministic_and_sorted(synth_mod):
    s = synth_mod.GENOTYPE_512x4096
    a = synth_mod.genotype(s)
    b = synth_mod.genotype(s)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    rp, col, val = a
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0)
    for r in range(0, 512, 37):
        c = col[rp[r]:rp[r + 1]]
        assert np.all(np.diff(c) > 0) and c.min() >= 0 and c.max() < 4096
    assert set(np.unique(val).tolist()) <= {1, 2}


def test_genotype_blocks_match_whole(synth_mod):
    s = synth_mod.GenotypeSpec(300, 2000, 8, 50.0, 0.01, seed=9)
    rp, col, val = synth_mod.genotype(s)
    A = np.zeros((300, 2000), np.int8)
    for r in range(300):
        A[r, col[rp[r]:rp[r + 1]]] = val[rp[r]:rp[r + 1]]
    for (r0, nr, c0, nc) in [(0, 300, 0, 2000), (17, 100, 333, 901), (299, 1, 1999, 1), (5, 0, 0, 10)]:
        brp, bcol, bval = synth_mod.genotype(s, r0, nr, c0, nc)
        B = np.zeros((nr, 2000), np.int8)
        for r in range(nr):
            B[r, bcol[brp[r]:brp[r + 1]]] = bval[brp[r]:brp[r + 1]]
        assert np.array_equal(B[:, c0:c0 + nc], A[r0:r0 + nr, c0:c0 + nc])
        assert not B[:, :c0].any() and not B[:, c0 + nc:].any()


def test_genotype_density(synth_mod):
    # folded Beta(1/2,1/2) allele frequency q: P(genotype != 0) = 2E[q] - E[q^2]
    # = 2(1/2 - 1/pi) - (3/8 - 1/pi) ~= 0.3067 before mutation/founder sampling
    rp, col, val = synth_mod.genotype(synth_mod.GENOTYPE_512x4096)
    frac = rp[-1] / (512 * 4096)
    assert 0.28 < frac < 0.33
    s2 = synth_mod.GenotypeSpec(400, 100_000, 64, 500.0, 0.001, seed=2)
    rp, _, _ = synth_mod.genotype(s2, 0, 400)
    assert 0.29 < rp[-1] / (400 * 100_000) < 0.32
    expect = 2 * (0.5 - 1 / math.pi) - (3 / 8 - 1 / math.pi)
    mafs = np.array([synth_mod.site_maf(s2, j) for j in range(20000)])
    assert abs(np.mean(2 * mafs - mafs ** 2) - expect) < 0.01
    assert mafs.max() <= 0.5


def test_copy_graph(synth_mod):
    g = synth_mod.GraphSpec(50_000, seed=5)
    rp, col = synth_mod.copy_graph(g)
    rp2, col2 = synth_mod.copy_graph(g)
    assert np.array_equal(rp, rp2) and np.array_equal(col, col2)
    deg = np.diff(rp)
    assert deg.min() >= 1 and 18.5 < deg.mean() < 21.0
    for r in range(0, 50_000, 997):
        c = col[rp[r]:rp[r + 1]]
        assert np.all(np.diff(c) > 0) and c.min() >= 0 and c.max() < 50_000


def test_normal_and_sources(synth_mod):
    z = synth_mod.normal(200_000, 101)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert np.array_equal(z[:10], synth_mod.normal(10, 101))
    s = synth_mod.sources(1000, 16, 501)
    assert len(set(s.tolist())) == 16 and s.min() >= 0 and s.max() < 1000
