"""CPU checks of the tuned per-shape table (tuning/table.json, written on the GPU
by tuning/sweep.py) and of the include build.py generates from it."""
import json
import os

import pytest

from mamba_ssd_chunked_03_amd import build

TABLE = build.TABLE_JSON


def test_include_matches_table(tmp_path, monkeypatch):
    monkeypatch.setattr(build, "BUILD_DIR", str(tmp_path))
    path = build.write_table_include()
    text = open(path).read()
    if not os.path.exists(TABLE):
        assert "kTunedScanCount = 0;" in text
        return
    t = json.load(open(TABLE))
    rows = t["state_passing"]
    assert "kTunedScanCount = %d;" % len(rows) in text
    for e in rows:
        assert "{%d, %d, %d}," % (e["chunks_per_seq"], e["lanes"], e["variant"]) in text


def test_table_rows_are_the_measured_best():
    if not os.path.exists(TABLE):
        pytest.skip("no tuned table")
    t = json.load(open(TABLE))
    assert t["generated_by"].endswith("tuning/sweep.py")
    seen = set()
    for e in t["state_passing"]:
        us = {int(k): v for k, v in e["us"].items()}
        assert set(us) == set(range(1, 8))
        assert e["variant"] == min(us, key=us.get)          # the fastest variant was kept
        assert 1 <= e["variant"] <= 7
        assert e["lanes"] == e["seqs"] * e["heads"] * 64 * 128 // 4
        key = (e["chunks_per_seq"], e["lanes"])
        assert key not in seen
        seen.add(key)


def _nearest(rows, chain, lanes):
    import math
    best, bv = None, None
    for e in rows:
        d = (math.log2(chain) - math.log2(e["chunks_per_seq"])) ** 2 + \
            (math.log2(lanes) - math.log2(e["lanes"])) ** 2
        if best is None or d < best:
            best, bv = d, e["variant"]
    return bv


def test_library_looks_up_the_nearest_measured_shape():
    from mamba_ssd_chunked_03_amd import ssd
    if not os.path.exists(ssd.LIB_PATH):
        pytest.skip("libssd.so not built")
    import ctypes
    L = ssd.lib()
    rows = json.load(open(TABLE))["state_passing"] if os.path.exists(TABLE) else []
    # (batch or nseq, seqlen, heads, packed): the layer, long-context and packed workloads, and others
    for batch, seqlen, H, packed in ((2, 8192, 64, 0), (1, 131072, 32, 0), (5, 65536, 64, 1),
                                     (1, 1024, 4, 0), (8, 65536, 64, 0), (3, 700, 16, 0)):
        p = ssd.Problem(1 if packed else batch, seqlen, H, 64, 128, 1, batch if packed else 0,
                        ssd.BF16, 1, 0)
        v = L.ssd_scan_variant(ctypes.byref(p), 256, packed)
        nck = L.ssd_num_chunks(ctypes.byref(p), 256, packed)
        chain = -(-nck // batch) if packed else nck // batch
        lanes = batch * H * 64 * 128 // 4
        if rows:
            assert v == _nearest(rows, chain, lanes), (batch, seqlen, H, v)
        else:
            assert 1 <= v <= 4
        for forced in range(1, 8):
            p.flags = ssd.FLAG_SCAN_VARIANT(forced)
            assert L.ssd_scan_variant(ctypes.byref(p), 256, packed) == forced
        p.flags = ssd.FLAG_SEQUENTIAL_SCAN
        assert L.ssd_scan_variant(ctypes.byref(p), 256, packed) == 5
