"""Serialized grammar (gcs_save_grammar / gcs_load_grammar): a loaded grammar
is the grammar that was saved (every exported array and the whole device
layout equal), it still evaluates M x through the layout, and damaged files
are refused."""
import os

import numpy as np
import pytest

import helpers as H


@pytest.fixture(scope="module")
def gcs():
    from grammar_compressed_sparse_amd import gcs as m
    return m


def _same(a, b):
    ea, eb = a.export(), b.export()
    assert ea.keys() == eb.keys()
    for k in ea:
        assert np.array_equal(np.asarray(ea[k]), np.asarray(eb[k])), k
    la, lb = a.layout(), b.layout()
    assert la.keys() == lb.keys()
    for k in la:
        assert np.array_equal(np.asarray(la[k]), np.asarray(lb[k])), k
    sa, sb = a.stats(), b.stats()
    for k in sa:
        if not k.startswith("t_"):
            assert sa[k] == sb[k], k
    assert np.array_equal(a.level_widths(), b.level_widths())
    for p in (0, 1, 3):
        assert a.device_layout(p) == b.device_layout(p)


def test_round_trip_genotype(gcs, oracle_mod, synth_mod, tmp_path):
    spec = synth_mod.GenotypeSpec(300, 3000, 8, 100.0, 0.005, seed=3)
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols, col_chunk=700, row_chunk=128)
    path = tmp_path / "g.gcs"
    g.save(path)
    h = gcs.load_grammar(path)
    _same(g, h)
    x = synth_mod.normal(spec.n_cols, 9)
    yo, absum = oracle_mod.spmv_f64(rp, col, val, x)
    y = H.emulate_layout(h.layout(), h.export(), x)
    assert np.all(np.abs(y - yo) <= 1e-12 * absum + 1e-300)


def test_round_trip_graph_and_empty(gcs, synth_mod, tmp_path):
    spec = synth_mod.GraphSpec(20_000, seed=8)
    rp, col = synth_mod.copy_graph(spec)
    g = gcs.build_grammar(rp, col, None, n_cols=spec.n, row_chunk=2500, row_order=gcs.ROWS_SIMILAR)
    g.save(tmp_path / "graph.gcs")
    _same(g, gcs.load_grammar(tmp_path / "graph.gcs"))
    e = gcs.build_grammar(np.zeros(1, np.int64), np.zeros(0, np.int32), None, n_cols=5)
    e.save(tmp_path / "empty.gcs")
    _same(e, gcs.load_grammar(tmp_path / "empty.gcs"))


def test_damaged_files_refused(gcs, synth_mod, tmp_path):
    spec = synth_mod.GenotypeSpec(100, 800, 4, 50.0, 0.01, seed=4)
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols)
    path = tmp_path / "g.gcs"
    g.save(path)
    blob = path.read_bytes()

    def refused(data, what):
        p = tmp_path / "bad.gcs"
        p.write_bytes(data)
        with pytest.raises(gcs.GcsError, match=what):
            gcs.load_grammar(p)

    flipped = bytearray(blob)
    flipped[len(blob) // 2] ^= 0x40
    refused(bytes(flipped), "checksum|corrupt|inconsistent")
    refused(blob[:len(blob) - 9], "truncated|checksum|corrupt")
    refused(blob[:40], "truncated|corrupt")
    refused(b"NOTAGRAM" + blob[8:], "not a serialized grammar")
    refused(blob + b"\0", "checksum")
    version = bytearray(blob)
    version[8] ^= 0x01
    refused(bytes(version), "version")
    with pytest.raises(gcs.GcsError):
        gcs.load_grammar(tmp_path / "does_not_exist.gcs")
    with pytest.raises(gcs.GcsError):
        g.save(tmp_path / "no_such_dir" / "g.gcs")


def _checksum(data: bytes) -> int:
    """The file's trailing checksum (multiply-xorshift over 8-byte words,
    a partial last word zero-padded), restated to forge consistent files."""
    M = (1 << 64) - 1
    h = 0x9E3779B97F4A7C15

    def mix(h, w):
        h ^= (w + 0x9E3779B97F4A7C15 + ((h << 6) & M) + (h >> 2)) & M
        h = (h * 0xBF58476D1CE4E5B9) & M
        return h ^ (h >> 31)

    n = len(data) // 8 * 8
    for w in np.frombuffer(data[:n], dtype="<u8").tolist():
        h = mix(h, w)
    if len(data) > n:
        h = mix(h, int.from_bytes(data[n:] + b"\0" * (8 - len(data) + n), "little"))
    return h


def test_upload_refuses_a_forged_layout(gcs, synth_mod, tmp_path):
    """A file with a valid checksum but a child index outside the arena loads,
    and the upload's bounds check refuses it before touching a device."""
    import ctypes
    spec = synth_mod.GenotypeSpec(60, 500, 4, 50.0, 0.01, seed=4)
    rp, col, val = synth_mod.genotype(spec)
    g = gcs.build_grammar(rp, col, val, n_cols=spec.n_cols)
    assert g.stats()["n_rules"] > 0
    path = tmp_path / "g.gcs"
    g.save(path)
    blob = bytearray(path.read_bytes())
    assert _checksum(bytes(blob[:-8])) == int.from_bytes(blob[-8:], "little")
    # walk to the child array: header 8 + 16, scalars 80, col_cut 36, times 24
    off = 8 + 16 + 80 + 36 + 24
    sizes = [8, 4, 4, 4, 4, 8, 4, 4, 4, 8]  # V tcol tval ra rb c_off c_sym lvl plast levels
    for sz in sizes:
        n = int.from_bytes(blob[off:off + 8], "little")
        off += 8 + n * sz
    n_child = int.from_bytes(blob[off:off + 8], "little")
    assert n_child == 2 * g.stats()["n_rules"]
    blob[off + 8:off + 12] = (1 << 30).to_bytes(4, "little")
    body = bytes(blob[:-8])
    blob[-8:] = _checksum(body).to_bytes(8, "little")
    bad = tmp_path / "forged.gcs"
    bad.write_bytes(bytes(blob))
    h = gcs.load_grammar(bad)
    out = ctypes.c_void_p()
    st = gcs._lib.gcs_upload(h.handle, gcs.PLUS_F64, ctypes.c_void_p(1 << 20), 1 << 40, ctypes.c_void_p(1 << 21),
                             1 << 40, None, ctypes.byref(out))
    assert st == -5 and b"layout check" in gcs._lib.gcs_last_error()
