"""CPU tests of the rocprofv3 summary helpers (synthetic CSV input)."""
import csv
import json

from mamba_ssd_chunked_03_amd import profiling

TRACE_COLS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
PMC_COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write(path, cols, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerows(rows)
    return str(path)


def test_kernel_keys():
    k = profiling.kernel_key
    assert k("void ssd::chunk_state_bf16_kernel<64, 128, 0>(ssd::ChunkMap)") == "chunk_state"
    assert k("void ssd::chunk_state_bf16_kernel<64, 128, 1>(ssd::ChunkMap)") == "dstates"
    assert k("void ssd::chunk_state_bf16_kernel<64, 128, 1, 2>(ssd::ChunkMap)") == "dstates"
    assert k("void ssd::chunk_state_bf16_kernel<64, 128, 2, 1>(ssd::ChunkMap)") == "chunk_state"
    assert k("void ssd::chunk_state_bf16_kernel<64, 128, 0, 2>(ssd::ChunkMap)") == "chunk_state"
    assert k("void ssd::state_passing_kernel<16, 4, unsigned short, 1>(x)") == "reverse_state_passing"
    assert k("void ssd::state_passing_kernel<16, 4, unsigned short, 0>(x)") == "state_passing"
    assert k("void ssd::state_passing_seq_kernel<unsigned short, 0, 1>(x)") == "state_passing"
    assert k("void ssd::state_passing_seq_kernel<unsigned short, 1, 4>(x)") == "reverse_state_passing"
    assert k("void ssd::state_passing_seq_kernel<float, 0, 8>(x)") == "state_passing"
    assert k("void ssd::fwd_chained_kernel<64, 128>(ssd::ChunkMap)") == "fwd_chained"
    assert k("ssd::chain_clear_kernel(int*, long)") == "fwd_chained"
    assert k("void ssd::bwd_dc_bf16_kernel<64, 128>(x)") == "bwd_dc"
    assert k("void ssd::bwd_dcb_bf16_kernel<64>(x)") == "bwd_dcb"
    assert k("void ssd::bwd_dbc_bf16_kernel<64, 128>(x)") == "bwd_dbc"
    assert k("void ssd::bwd_reduce_kernel(int)") == "bwd_finalize"
    assert k("void ssd::bmm_chunk_bf16_kernel<128, true>(x)") == "bmm_chunk"
    assert k("void ssd::bmm_chunk_bf16_kernel<128, false>(x)") == "bmm_chunk_cb_only"
    assert k("void ssd::gated_rmsnorm_bwd_kernel<true>(x)") == "gated_rmsnorm_bwd"
    assert k("void ssd::norm_dw_reduce_kernel(int)") == "gated_rmsnorm_bwd"
    assert k("void ssd::gated_rmsnorm_fwd_kernel<false>(x)") == "gated_rmsnorm_fwd"
    assert k("void ssd::chunk_state_f32_kernel<64, 128>(ssd::ChunkMap)") == "chunk_state_f32"
    assert k("void ssd::scan_rows_f32_kernel<64, true>(x)") == "scan_rows_f32"
    assert k("void ssd::bwd_dcb_f32_kernel(ssd::ChunkMap)") == "bwd_dcb_f32"
    assert k("void ssd::bwd_dc_f32_kernel<128>(x)") == "bwd_dc_f32"
    assert all(key in profiling.KERNEL_FILES for key in ("chunk_state_f32", "scan_rows_f32", "bwd_dcb_f32"))
    assert k("void at::native::elementwise_kernel<4>(x)") is None


def test_stats_table(tmp_path):
    rows = [["void ssd::bwd_dx_bf16_kernel<64, 128>(a)", 100, 1100],      # alone
            ["void ssd::bwd_dx_bf16_kernel<64, 128>(a)", 2000, 5000],     # meets the bwd_dc below
            ["void ssd::bwd_dc_bf16_kernel<64, 128>(a)", 4000, 4500],
            ["void ssd::bwd_finalize_kernel(a)", 6000, 6500],
            ["void ssd::bwd_reduce_kernel(a)", 6600, 6700],
            ["void at::native::other(a)", 9000, 9999]]
    p = write(tmp_path / "t.csv", TRACE_COLS, rows)
    text, total = profiling.stats_table(p, "cmd")
    assert abs(total["bwd_dx"] - 1.0) < 1e-9            # the launch alone: 1000 ns
    assert abs(total["bwd_finalize"] - 0.6) < 1e-9      # 500 + 100 ns per launch
    assert total["bwd_dc"] != total["bwd_dc"]           # never alone: no figure (nan)
    line = [l for l in text.splitlines() if l.startswith("| bwd_dx |")][0]
    assert "| 2 | 1 | 1.0 | 1 | 3.0 | 1.0 | 3.0 |" in line
    assert "at::native" not in text


def test_traffic_calibration(tmp_path):
    copy = "void ssd::copy_kernel(a)"
    dx = "void ssd::bwd_dx_bf16_kernel<64, 128>(a)"
    cf = write(tmp_path / "cf.csv", PMC_COLS, [[1, copy, "FETCH_SIZE", 131072.0]])   # 256 MiB read
    cw = write(tmp_path / "cw.csv", PMC_COLS, [[1, copy, "WRITE_SIZE", 262144.0]])
    f = write(tmp_path / "f.csv", PMC_COLS, [[5, dx, "FETCH_SIZE", 1000.0], [6, dx, "FETCH_SIZE", 3000.0]])
    w = write(tmp_path / "w.csv", PMC_COLS, [[5, dx, "WRITE_SIZE", 512.0]])
    res = profiling.traffic(f, w, cf, cw, 268435456)
    assert res["bwd_dx"]["fetch_bytes"] == 2000 * 2048  # each counter unit is 2 KiB here
    assert res["bwd_dx"]["write_bytes"] == 512 * 1024
    assert res["bwd_dx"]["source_sha"] == profiling.source_hash("bwd_dx")
    out = tmp_path / "t.json"
    profiling.main(["traffic", "--fetch", f, "--write", w, "--copy-fetch", cf, "--copy-write", cw,
                    "--copy-bytes", "268435456", "--out", str(out)])
    assert json.load(open(out))["bwd_dx"]["bytes_per_launch"] == 2000 * 2048 + 512 * 1024


def test_mlp_littles_law(tmp_path):
    dx = "void ssd::bwd_dx_bf16_kernel<64, 128>(a)"
    cols = PMC_COLS + ["Start_Timestamp", "End_Timestamp"]
    # 2 CUs in 2 XCDs; 1000 ns at 2 cycles/ns = 2000 cycles per CU (GRBM sums both XCDs: 4000)
    vals = {"TCP_TCC_READ_REQ_sum": 400.0, "TCP_TCC_READ_REQ_LATENCY_sum": 400.0 * 500,
            "TA_TA_BUSY_sum": 2000.0, "TA_ADDR_STALLED_BY_TC_CYCLES_sum": 1000.0,
            "SQ_WAVE_CYCLES": 100.0, "SQ_WAIT_ANY": 25.0, "SQ_BUSY_CYCLES": 1.0, "GRBM_GUI_ACTIVE": 4000.0}
    rows = [[d, dx, c, v, 10_000 * d, 10_000 * d + 1000] for d in (1, 2) for c, v in vals.items()]
    p = write(tmp_path / "m.csv", cols, rows)
    res = profiling.mlp(p, cus=2, xcds=2)["bwd_dx"]
    assert res["launches"] == 2 and abs(res["us"] - 1.0) < 1e-12
    assert abs(res["clock_ghz"] - 2.0) < 1e-12
    assert res["latency_cycles"] == 500.0
    assert res["in_flight_per_cu"] == 400.0 * 500 / (2 * 2000)   # 50 requests per CU
    assert res["ta_busy"] == 0.5 and res["ta_stalled_by_l1"] == 0.25 and res["wave_wait_frac"] == 0.25
    assert res["requested_mb"] == 400 * 128 / 1e6
    assert res["mfma_gflop"] is None and res["mfma_busy"] is None   # not in this pass
    agent = write(tmp_path / "a.csv", ["Name", "Cu_Count", "Num_Xcc", "Simd_Per_Cu"], [["gfx950", 2, 2, 4]])
    assert profiling.agent_counts(agent) == (2, 2, 4)
    md = profiling.mlp_md({"bwd_dx": res}, "t", ["cmd"], "sum", 2, 2)
    assert "| bwd_dx | 1.0 | 0.00 | 0 | 500 | 50.0 | 12.8 | 0.50 | 0.25 | 0.25 | - | - |" in md
    # with the MFMA counters: 2 CUs x 4 SIMDs x 2000 cycles; 4000 busy cycles -> 0.25
    vals.update({"SQ_INSTS_VALU_MFMA_MOPS_BF16": 2e6, "SQ_VALU_MFMA_BUSY_CYCLES": 4000.0, "SQ_INSTS_MFMA": 10.0})
    rows = [[d, dx, c, v, 10_000 * d, 10_000 * d + 1000] for d in (1, 2) for c, v in vals.items()]
    res = profiling.mlp(write(tmp_path / "m2.csv", cols, rows), cus=2, xcds=2, simds_per_cu=4)["bwd_dx"]
    assert res["mfma_gflop"] == 2e6 * 512 / 1e9 and res["mfma_busy"] == 0.25 and res["mfma_insts"] == 10.0


def test_issue_mix(tmp_path):
    """VALU issue time: 4 cycles per wave instruction, 16 per transcendental one, over
    CUs x SIMDs at the given clock, as a fraction of the first run's duration."""
    dx = "void ssd::bwd_dx_bf16_kernel<64, 128>(a)"
    cols = PMC_COLS + ["Start_Timestamp", "End_Timestamp"]
    run_a = {"SQ_WAVE_CYCLES": 100.0, "SQ_INSTS_VALU": 1000.0, "SQ_INSTS_VALU_TRANS_F32": 100.0,
             "SQ_INSTS_SALU": 7.0, "SQ_INSTS_LDS": 60.0}
    run_b = {"SQ_WAIT_ANY": 25.0, "SQ_LDS_BANK_CONFLICT": 30.0, "SQ_INSTS_MFMA": 5.0}
    pa = write(tmp_path / "a.csv", cols, [[d, dx, c, v, 10_000 * d, 10_000 * d + 1000]
                                          for d in (1, 2) for c, v in run_a.items()])
    pb = write(tmp_path / "b.csv", cols, [[d, dx, c, v, 10_000 * d, 10_000 * d + 3000]
                                          for d in (1, 2) for c, v in run_b.items()])
    e = profiling.issue_mix([pa, pb], cus=2, simds_per_cu=4, ghz=2.0)["bwd_dx"]
    # (1000 x 4 + 100 x 12) cycles over 8 SIMDs = 650 cycles = 325 ns of a 1000 ns launch
    assert abs(e["us"] - 1.0) < 1e-12 and abs(e["valu_issue_us"] - 0.325) < 1e-12
    assert abs(e["valu_issue_frac"] - 0.325) < 1e-12
    assert e["wave_wait_frac"] == 0.25 and e["lds_conflict_per_inst"] == 0.5
    assert (e["valu"], e["trans"], e["salu"], e["lds"], e["mfma"]) == (1000.0, 100.0, 7.0, 60.0, 5.0)
    md = profiling.issue_md({"bwd_dx": e}, "t", ["cmd"], "sum", 2, 4, 2.0)
    assert "| bwd_dx | 1.0 | 0.00 | 0.00 | 0.00 | 0.00 | 0.00 | 0.3 | 0.33 | 0.25 | 0.50 |" in md
    # a kernel missing a counter the summary uses is left out
    assert profiling.issue_mix([pa], cus=2, simds_per_cu=4, ghz=2.0) == {}


def test_kernels_table_keeps_forms_apart(tmp_path):
    rows = [["void ssd::state_passing_kernel<8, 4, unsigned short, 0>(a)", 0, 4000],
            ["void ssd::state_passing_seq_kernel<unsigned short, 0, 1>(a)", 10000, 13000],
            ["void ssd::state_passing_seq_kernel<unsigned short, 0, 1>(a)", 20000, 23200],
            ["void ssd::bwd_dx_bf16_kernel<64, 128>(a)", 30000, 31000]]
    p = write(tmp_path / "t.csv", TRACE_COLS, rows)
    text = profiling.kernels_table(p, "cmd", keys=["state_passing"])
    lines = [l for l in text.splitlines() if l.startswith("| state_passing |")]
    assert len(lines) == 2 and not any("bwd_dx" in l for l in text.splitlines())
    assert "| 1 | 1 | 4.0 |" in [l for l in lines if "state_passing_kernel<" in l][0]
    assert "| 2 | 2 | 3.1 |" in [l for l in lines if "seq_kernel" in l][0]


def test_request_sizes(tmp_path):
    # two passes for the path, two for the copy; the finalize's two kernels make one launch
    fin, red = "void ssd::bwd_finalize_kernel(x)", "void ssd::bwd_reduce_kernel(int)"
    dx = "void ssd::bwd_dx_bf16_kernel<64, 128>(x)"
    a = write(tmp_path / "a.csv", PMC_COLS, [
        [1, dx, "TCC_EA0_RDREQ_sum", 1000], [1, dx, "TCC_EA0_RDREQ_32B_sum", 0],
        [1, dx, "TCC_BUBBLE_sum", 0], [1, dx, "TCC_EA0_WRREQ_sum", 400],
        [2, dx, "TCC_EA0_RDREQ_sum", 1200], [2, dx, "TCC_EA0_WRREQ_sum", 400],
        [3, fin, "TCC_EA0_RDREQ_sum", 300], [4, red, "TCC_EA0_RDREQ_sum", 10]])
    b = write(tmp_path / "b.csv", PMC_COLS, [[1, dx, "TCC_EA0_WRREQ_64B_sum", 400]])
    ca = write(tmp_path / "ca.csv", PMC_COLS, [[1, "void ssd::copy_kernel(x)", "TCC_EA0_RDREQ_sum", 2048],
                                               [1, "void ssd::copy_kernel(x)", "TCC_EA0_WRREQ_sum", 4096]])
    res, cp = profiling.request_sizes([a, b], [ca])
    assert res["bwd_dx"]["TCC_EA0_RDREQ_sum"] == 1100 and res["bwd_dx"]["TCC_EA0_WRREQ_64B_sum"] == 400
    assert res["bwd_finalize"]["TCC_EA0_RDREQ_sum"] == 310
    md = profiling.request_md(res, cp, 262144, "t", ["cmd"], "summary")
    assert "2048 read requests (128.0 bytes each) and 4096 write requests (64.0 bytes each)" in md
    assert "| bwd_dx | 1100 | 0 | 0 | 0.1 | 400 | 400 | 0.0 |" in md
