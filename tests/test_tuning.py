"""CPU checks of the tuned per-shape table (tuning/table.json, written on the GPU
by tuning/sweep.py) and of the include build.py generates from it."""
import json
import os

import pytest

from mamba_ssd_chunked_03_amd import build

TABLE = build.TABLE_JSON


def test_include_matches_table(tmp_path, monkeypatch):
    monkeypatch.setattr(build, "BUILD_DIR", str(tmp_path))
    scan_path, cs_path = build.write_table_include()
    text, cs_text = open(scan_path).read(), open(cs_path).read()
    t = json.load(open(TABLE)) if os.path.exists(TABLE) else {}
    rows = t.get("state_passing", [])
    assert "kTunedScanCount = %d;" % len(rows) in text
    for e in rows:
        assert "{%d, %d, %d}," % (e["chunks_per_seq"], e["lanes"], e["variant"]) in text
    cs = t.get("chunk_state", [])
    assert "kTunedCsCount = %d;" % len(cs) in cs_text
    for e in cs:
        assert "{%d, %d, %d, %d, %d}," % (e["headdim"], e["dstate"], e["heads_per_group"], e["chunk"],
                                          e["variant"]) in cs_text


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


def test_chunk_state_rows_are_the_measured_best():
    if not os.path.exists(TABLE):
        pytest.skip("no tuned table")
    rows = json.load(open(TABLE)).get("chunk_state", [])
    seen = set()
    for e in rows:
        us = {int(k): v for k, v in e["us"].items()}
        assert set(us) <= {1, 2, 3} and 1 in us
        assert e["variant"] == min(us, key=us.get)
        key = (e["headdim"], e["dstate"], e["heads_per_group"], e["chunk"])
        assert key not in seen
        seen.add(key)


def _valid_cs(P, N, hpg, Q):
    """Which chunk-state forms a bf16 problem can run (the rule the library states)."""
    lds2 = 2 * (2 * 64 * (P + 16) * 2 + 256 * 4 + 5 * 4) + 64 * (N + 16) * 2
    two = hpg % 2 == 0 and (64 * (N // 8)) % 512 == 0 and lds2 <= 80 * 1024
    return {1} | ({2} if two else set()) | ({3} if two and Q == 256 and hpg == 8 else set())


def test_library_looks_up_the_chunk_state_table():
    from mamba_ssd_chunked_03_amd import ssd
    if not os.path.exists(ssd.LIB_PATH):
        pytest.skip("libssd.so not built")
    import ctypes
    L = ssd.lib()
    rows = json.load(open(TABLE)).get("chunk_state", []) if os.path.exists(TABLE) else []
    table = {(e["headdim"], e["dstate"], e["heads_per_group"], e["chunk"]): e["variant"] for e in rows}
    for P in (32, 64, 128):
        for N in (32, 64, 128):
            for hpg in (1, 2, 3, 4, 8, 16):
                for Q in (64, 128, 256):
                    p = ssd.Problem(2, 1000, 16 * hpg, P, N, 16, 0, ssd.BF16, 1, 0)
                    valid = _valid_cs(P, N, hpg, Q)
                    v = L.ssd_cs_variant(ctypes.byref(p), Q, 0)
                    want = table.get((P, N, hpg, Q))
                    assert v == (want if want in valid else max(valid)), (P, N, hpg, Q, v)
                    for forced in (1, 2, 3):
                        p.flags = ssd.FLAG_CS_VARIANT(forced)
                        got = L.ssd_cs_variant(ctypes.byref(p), Q, 0)
                        assert got == (forced if forced in valid else 0), (P, N, hpg, Q, forced)
                    p.flags = 0
                    # C.B^T inside the chunk-state kernel is variant 3 (forward kernel mask 0xB)
                    assert (L.ssd_fwd_kernel_mask(ctypes.byref(p), Q, 0) == 0xB) == (v == 3)
    p = ssd.Problem(1, 100, 8, 16, 16, 1, 0, ssd.F32, 1, 0)   # fp32: one form
    assert L.ssd_cs_variant(ctypes.byref(p), 64, 0) == 1
    p.flags = ssd.FLAG_CS_VARIANT(2)
    assert L.ssd_cs_variant(ctypes.byref(p), 64, 0) == 0
