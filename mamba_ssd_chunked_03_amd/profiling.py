"""Summaries of rocprofv3 output for the kernels of the SSD path.

Two inputs, both written by rocprofv3 with ``-f csv``:

* a kernel trace (``--kernel-trace``): per-kernel launch counts and average
  durations -> a markdown table;
* counter runs (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``) of the same
  program and of a plain copy of known size: HBM bytes per launch of every
  kernel, each counter scaled by what it reads for the copy (so the result is
  in bytes whatever unit and instance sum the counter uses) -> a JSON table
  keyed by kernel, with a hash of the kernel's source so that a reader can tell
  whether the numbers still describe the code.

Kernels are named as bench.py names them; one "launch" of bwd_finalize is its
two kernels (the per-chunk pass and the per-head reduction), and one of
gated_rmsnorm_bwd its two (the rows and the dweight reduction).

    python -m mamba_ssd_chunked_03_amd.profiling stats TRACE.csv OUT.md --command "..."
    python -m mamba_ssd_chunked_03_amd.profiling traffic --fetch F.csv --write W.csv \\
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes 268435456 --out profiles/traffic.json

A third summary, ``mlp``, reads one counter run with the MLP_COUNTERS below
(one pass: 4 SQ, 2 TCP, 2 TA and 1 GRBM counters) and reports, per kernel, how
the vector memory path was used: L1-to-L2 read requests per launch, their mean
latency, the mean number in flight per compute unit (Little's law: total
latency cycles over elapsed cycles), and how often the texture address unit
was busy or held up by the L1.  Per compute unit a kernel can read at most
(requests in flight x 128 bytes / latency), which is what bounds the staged
kernels below the HBM peak.

    python -m mamba_ssd_chunked_03_amd.profiling mlp --pmc DIR --md OUT.md --command "..."

A fourth, ``issue``, reads two counter runs holding ISSUE_COUNTERS (8 SQ
counters each) and reports the instruction mix per kernel: VALU, transcendental,
scalar, LDS and MFMA instructions per launch, and the time the VALU instructions
alone occupy the SIMDs (a wave64 instruction takes 4 cycles on a 16-lane SIMD, a
transcendental one 16) as a fraction of the kernel's duration.

    python -m mamba_ssd_chunked_03_amd.profiling issue --pmc DIR_A DIR_B --md OUT.md --command "..."
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import shlex
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# kernel (as bench.py names it) -> source file holding it
KERNEL_FILES = {
    "chunk_cumsum": "k_cumsum.hip", "chunk_state": "k_chunk_state.hip",
    "state_passing": "k_state_passing.hip", "bmm_chunk": "k_bmm.hip",
    "chunk_scan": "k_chunk_scan.hip", "dstates": "k_chunk_state.hip",
    "reverse_state_passing": "k_state_passing.hip", "bwd_dx": "k_bwd.hip", "bwd_dcb": "k_bwd.hip",
    "bwd_dc": "k_bwd.hip", "bwd_db": "k_bwd.hip", "bwd_finalize": "k_bwd.hip",
    "bwd_dbc": "k_bwd_dbc.hip",  # dB and dC with their dCB and decay-gradient sums, one kernel
    "bmm_chunk_cb_only": "k_bmm.hip",  # C.B^T without its transpose (a forward that keeps nothing)
    "gated_rmsnorm_fwd": "k_norm.hip", "gated_rmsnorm_bwd": "k_norm.hip",  # the layer's norm
    "fwd_chained": "k_fwd_chained.hip",  # the fused chained forward (its clear and empty-final kernels too)
    # the fp32 path's kernels, under their own names
    "chunk_state_f32": "k_f32.hip", "bmm_chunk_f32": "k_f32.hip", "scan_rows_f32": "k_f32.hip",
    "bwd_dx_f32": "k_f32.hip", "bwd_dcb_f32": "k_f32.hip", "bwd_dc_f32": "k_f32.hip",
    "bwd_db_f32": "k_f32.hip",
}
# headers whose code is compiled into every kernel
SHARED_HEADERS = ("common.hpp", "internal.hpp", "layout.hpp", "scan_rows.hpp")


def source_hash(kernel):
    """Hash of the kernel's source file and the headers every kernel includes."""
    h = hashlib.sha256()
    for name in (KERNEL_FILES[kernel],) + SHARED_HEADERS:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_key(name):
    """bench.py's name for a launched kernel (None for kernels outside the path)."""
    base = re.search(r"ssd::(\w+)", name)
    if not base:
        return None
    base = base.group(1)
    targs = re.search(r"<([^>]*)>", name)
    targ = [t.strip() for t in targs.group(1).split(",")] if targs else []
    last = targ[-1] if targ else ""
    if base.endswith("_f32_kernel"):  # the fp32 path: chunk_state_f32, scan_rows_f32, bwd_dx_f32, ...
        return base[:-len("_kernel")]
    if base.startswith("chunk_state"):
        # chunk_state_bf16_kernel<P, N, MODE, heads per workgroup>: MODE 1 is the backward's dstates
        return "dstates" if len(targ) >= 3 and targ[2] == "1" else "chunk_state"
    if base == "state_passing_kernel":
        return "reverse_state_passing" if last == "1" else "state_passing"
    if base == "state_passing_seq_kernel":
        # state_passing_seq_kernel<output type, REV, loads in flight>
        return "reverse_state_passing" if len(targ) >= 2 and targ[1] == "1" else "state_passing"
    if base in ("fwd_chained_kernel", "chain_clear_kernel", "chain_empty_final_kernel"):
        return "fwd_chained"
    if base.startswith("bmm_chunk_bf16"):
        return "bmm_chunk_cb_only" if last == "false" else "bmm_chunk"
    for prefix, key in (("chunk_cumsum", "chunk_cumsum"), ("bmm_chunk", "bmm_chunk"),
                        ("chunk_scan", "chunk_scan"), ("bwd_dx_", "bwd_dx"), ("bwd_dcb_", "bwd_dcb"), ("bwd_dbc_", "bwd_dbc"),
                        ("bwd_dc_", "bwd_dc"), ("bwd_db_", "bwd_db"), ("bwd_finalize", "bwd_finalize"),
                        ("bwd_reduce", "bwd_finalize"), ("gated_rmsnorm_fwd", "gated_rmsnorm_fwd"),
                        ("gated_rmsnorm_bwd", "gated_rmsnorm_bwd"), ("norm_dw_reduce", "gated_rmsnorm_bwd"),
                        ("copy_kernel", "copy")):
        if base.startswith(prefix):
            return key
    return None


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError("none of %s in %s" % (names, list(row)))


def _one(pattern):
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_times(trace_csv):
    """{key: {name: [(duration ns, overlapped)]}} from a kernel-trace CSV.

    A launch is "overlapped" when its [start, end) interval meets that of any
    other kernel in the trace (the path runs some kernels on a second stream),
    so that its duration is not the kernel's alone."""
    spans = []
    for row in _rows(trace_csv):
        name = _col(row, "Kernel_Name", "Name")
        spans.append((int(_col(row, "Start_Timestamp")), int(_col(row, "End_Timestamp")), name))
    spans.sort()
    over = [False] * len(spans)
    for i, (s0, e0, _) in enumerate(spans):
        j = i + 1
        while j < len(spans) and spans[j][0] < e0:
            over[i] = over[j] = True
            j += 1
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for (s0, e0, name), ov in zip(spans, over):
        key = kernel_key(name)
        if key is None:
            continue
        short = re.search(r"ssd::(\w+(?:<[^>]*>)?)", name).group(1)
        out[key][short].append((e0 - s0, ov))
    return out


def _mean(v):
    return sum(v) / len(v) if v else float("nan")


def stats_table(trace_csv, command, summary_cmd=""):
    times = kernel_times(trace_csv)
    lines = ["Profiled with (from the repository root, one MI355X):", "", "    " + command, ""]
    if summary_cmd:
        lines += ["Summarised with:", "", "    " + summary_cmd, ""]
    lines += ["Per kernel of the path (bench.py's names): launches and durations from the kernel "
              "trace; a bwd_finalize launch is its two kernels.  Inside ssd_fwd / ssd_bwd some "
              "kernels run side by side on two streams, and the program also times each kernel "
              "on its own; a launch counts as overlapped when its interval meets another "
              "kernel's, and the two kinds are averaged apart.", "",
              "| Kernel | Launched kernels | Launches | Alone | Alone avg (us) | Overlapped "
              "| Overlapped avg (us) | Min (us) | Max (us) |",
              "|---|---|---|---|---|---|---|---|---|"]
    total = {}
    for key in KERNEL_FILES:
        if key not in times:
            continue
        ks = times[key]
        n = min(len(v) for v in ks.values())
        # a multi-kernel launch (bwd_finalize) counts as alone only when all its kernels are
        alone = sum(_mean([t for t, ov in v if not ov]) for v in ks.values()) / 1e3
        lapped = sum(_mean([t for t, ov in v if ov]) for v in ks.values()) / 1e3
        n_alone = min(sum(1 for _, ov in v if not ov) for v in ks.values())
        n_over = max(sum(1 for _, ov in v if ov) for v in ks.values())
        mn = sum(min(t for t, _ in v) for v in ks.values()) / 1e3
        mx = sum(max(t for t, _ in v) for v in ks.values()) / 1e3
        total[key] = alone
        fmt = lambda x: "-" if x != x else "%.1f" % x
        lines.append("| %s | %s | %d | %d | %s | %d | %s | %.1f | %.1f |" % (
            key, ", ".join("`%s`" % s for s in sorted(ks)), n, n_alone, fmt(alone), n_over,
            fmt(lapped), mn, mx))
    lines += ["", "Sum of the averages alone (one of each kernel): %.1f us"
              % sum(v for v in total.values() if v == v)]
    return "\n".join(lines) + "\n", total


def kernels_table(trace_csv, command, summary_cmd="", keys=None):
    """One row per launched kernel (template instance) rather than per path kernel:
    for traces of programs that launch several forms of one kernel (a comparison of
    variants), whose launches must not be summed or averaged together."""
    times = kernel_times(trace_csv)
    lines = ["Profiled with (from the repository root, one MI355X):", "", "    " + command, ""]
    if summary_cmd:
        lines += ["Summarised with:", "", "    " + summary_cmd, ""]
    lines += ["One row per launched kernel (its template arguments name the form).  A launch "
              "counts as overlapped when its interval meets another kernel's; the two kinds are "
              "averaged apart.", "",
              "| Kernel | Launched kernel | Launches | Alone | Alone avg (us) | Overlapped "
              "| Overlapped avg (us) | Min (us) | Max (us) |",
              "|---|---|---|---|---|---|---|---|---|"]
    fmt = lambda x: "-" if x != x else "%.1f" % x
    for key in KERNEL_FILES:
        if key not in times or (keys and key not in keys):
            continue
        for short in sorted(times[key]):
            v = times[key][short]
            alone = _mean([t for t, ov in v if not ov]) / 1e3
            lapped = _mean([t for t, ov in v if ov]) / 1e3
            lines.append("| %s | `%s` | %d | %d | %s | %d | %s | %.1f | %.1f |" % (
                key, short, len(v), sum(1 for _, ov in v if not ov), fmt(alone),
                sum(1 for _, ov in v if ov), fmt(lapped), min(t for t, _ in v) / 1e3,
                max(t for t, _ in v) / 1e3))
    return "\n".join(lines) + "\n"


def counter_means(counter_csv, counter):
    """{key: (mean value per launch, launches)} for one counter; a launch of a
    multi-kernel key sums its kernels' means."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for row in _rows(counter_csv):
        if _col(row, "Counter_Name") != counter:
            continue
        name = _col(row, "Kernel_Name")
        key = kernel_key(name)
        if key is None:
            continue
        per[key][name].append(float(_col(row, "Counter_Value")))
    return {k: (sum(sum(v) / len(v) for v in d.values()), min(len(v) for v in d.values()))
            for k, d in per.items()}


MLP_COUNTERS = ("TCP_TCC_READ_REQ_sum", "TCP_TCC_READ_REQ_LATENCY_sum", "TA_TA_BUSY_sum",
                "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_BUSY_CYCLES",
                "GRBM_GUI_ACTIVE")
# optional in the same pass: executed MFMA work, for the cross-check of the
# algorithmic flops (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of 512 flops)
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA")
MOPS_FLOPS = 512
LINE_BYTES = 128  # one L1-to-L2 read request


def agent_counts(agent_csv):
    """(compute units, XCDs, SIMDs per CU) of the GPU agent in a rocprofv3 agent-info CSV."""
    for row in _rows(agent_csv):
        if "gfx" in row.get("Name", ""):
            return (int(row["Cu_Count"]), int(row.get("Num_Xcc") or 1),
                    int(row.get("Simd_Per_Cu") or 4))
    raise ValueError("no GPU agent in %s" % agent_csv)


def mlp(counter_csv, cus, xcds, simds_per_cu=4):
    """{key: figures} from one counter run holding MLP_COUNTERS.

    Per kernel name: the mean of each counter and of the dispatch duration over
    its launches; a key with several kernels sums them.  Elapsed cycles per
    compute unit = GRBM_GUI_ACTIVE / XCDs (the counter sums the XCDs' clocks)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(dict)
    for row in _rows(counter_csv):
        name = _col(row, "Kernel_Name")
        key = kernel_key(name)
        if key is None or key == "copy":
            continue
        vals[(key, name)][_col(row, "Counter_Name")].append(float(_col(row, "Counter_Value")))
        durs[(key, name)][_col(row, "Dispatch_Id")] = (int(_col(row, "End_Timestamp"))
                                                       - int(_col(row, "Start_Timestamp")))
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    for (key, name), d in vals.items():
        for c, v in d.items():
            tot[key][c] += _mean(v)
        tot[key]["_ns"] += _mean(list(durs[(key, name)].values()))
        tot[key]["_launches"] = len(durs[(key, name)])
    out = {}
    for key, t in tot.items():
        if any(c not in t for c in MLP_COUNTERS):
            continue
        cyc = t["GRBM_GUI_ACTIVE"] / xcds
        req = t["TCP_TCC_READ_REQ_sum"]
        out[key] = {
            "launches": int(t["_launches"]), "us": t["_ns"] / 1e3, "clock_ghz": cyc / t["_ns"],
            "read_requests": req, "requested_mb": req * LINE_BYTES / 1e6,
            "latency_cycles": t["TCP_TCC_READ_REQ_LATENCY_sum"] / req if req else float("nan"),
            "in_flight_per_cu": t["TCP_TCC_READ_REQ_LATENCY_sum"] / (cus * cyc),
            "ta_busy": t["TA_TA_BUSY_sum"] / (cus * cyc),
            "ta_stalled_by_l1": t["TA_ADDR_STALLED_BY_TC_CYCLES_sum"] / (cus * cyc),
            "wave_wait_frac": t["SQ_WAIT_ANY"] / t["SQ_WAVE_CYCLES"],
            "mfma_gflop": (t["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * MOPS_FLOPS / 1e9
                           if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in t else None),
            "mfma_insts": t.get("SQ_INSTS_MFMA"),
            "mfma_busy": (t["SQ_VALU_MFMA_BUSY_CYCLES"] / (cus * simds_per_cu * cyc)
                          if "SQ_VALU_MFMA_BUSY_CYCLES" in t else None),
            "source_sha": source_hash(key) if key in KERNEL_FILES else ""}
    return out


ISSUE_COUNTERS = (("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
                   "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS"),
                  ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_ANY",
                   "SQ_INSTS_MFMA", "SQ_INST_CYCLES_VALU", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_MISC"))
# the ones the summary uses (gfx950 returns no SQ_INST_CYCLES_VALU)
ISSUE_USED = ("SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VALU_TRANS_F32",
              "SQ_WAIT_ANY", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_MFMA")
VALU_CYCLES, TRANS_CYCLES = 4, 16  # per wave64 instruction on a 16-lane SIMD (transcendentals: quarter rate)


def issue_mix(counter_csvs, cus, simds_per_cu, ghz):
    """{key: figures} from counter runs holding ISSUE_COUNTERS.  Per kernel name the
    mean of each counter over its launches (a key with several kernels sums them);
    the duration is the mean dispatch time of the first run."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(dict)
    for n, path in enumerate(counter_csvs):
        for row in _rows(path):
            name = _col(row, "Kernel_Name")
            key = kernel_key(name)
            if key is None or key == "copy":
                continue
            vals[(key, name)][_col(row, "Counter_Name")].append(float(_col(row, "Counter_Value")))
            if n == 0:
                durs[(key, name)][_col(row, "Dispatch_Id")] = (int(_col(row, "End_Timestamp"))
                                                               - int(_col(row, "Start_Timestamp")))
    tot = collections.defaultdict(lambda: collections.defaultdict(float))
    for (key, name), d in vals.items():
        for c, v in d.items():
            tot[key][c] += _mean(v)
        if durs[(key, name)]:
            tot[key]["_ns"] += _mean(list(durs[(key, name)].values()))
    out = {}
    for key, t in tot.items():
        if any(c not in t for c in ISSUE_USED) or not t["_ns"]:
            continue
        valu, trans = t["SQ_INSTS_VALU"], t["SQ_INSTS_VALU_TRANS_F32"]
        issue_us = (valu * VALU_CYCLES + trans * (TRANS_CYCLES - VALU_CYCLES)) / (cus * simds_per_cu) / ghz / 1e3
        out[key] = {
            "us": t["_ns"] / 1e3, "valu": valu, "trans": trans, "salu": t["SQ_INSTS_SALU"],
            "lds": t["SQ_INSTS_LDS"], "mfma": t["SQ_INSTS_MFMA"], "valu_issue_us": issue_us,
            "valu_issue_frac": issue_us / (t["_ns"] / 1e3),
            "wave_wait_frac": t["SQ_WAIT_ANY"] / t["SQ_WAVE_CYCLES"],
            "lds_conflict_per_inst": t["SQ_LDS_BANK_CONFLICT"] / t["SQ_INSTS_LDS"] if t["SQ_INSTS_LDS"] else 0.0,
            "source_sha": source_hash(key) if key in KERNEL_FILES else ""}
    return out


def issue_md(res, title, commands, summary_cmd, cus, simds_per_cu, ghz):
    lines = (["# " + title, ""] if title else []) + [
        "Counter runs (from the repository root, one MI355X, one rocprofv3 pass each):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "Summarised with:", "", "    " + summary_cmd, "",
              "Instructions are wave instructions per launch (SQ_INSTS_VALU, SQ_INSTS_VALU_TRANS_F32, "
              "SQ_INSTS_SALU, SQ_INSTS_LDS, SQ_INSTS_MFMA). VALU issue = the SIMD time of the VALU "
              "instructions alone, %d cycles each (a wave64 instruction on a 16-lane SIMD) and %d for a "
              "transcendental one, over %d compute units x %d SIMDs at %.1f GHz, as a fraction of the "
              "kernel's duration in the first run; MFMA instructions run on their own unit and are not "
              "in it. Waves waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES. LDS conflict = SQ_LDS_BANK_CONFLICT "
              "cycles per LDS instruction."
              % (VALU_CYCLES, TRANS_CYCLES, cus, simds_per_cu, ghz), "",
              "| Kernel | us | VALU (M) | of them transcendental (M) | SALU (M) | LDS (M) | MFMA (M) "
              "| VALU issue (us) | VALU issue / duration | Waves waiting | LDS conflict | Source hash |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for key in KERNEL_FILES:
        if key in res:
            e = res[key]
            lines.append("| %s | %.1f | %.2f | %.2f | %.2f | %.2f | %.2f | %.1f | %.2f | %.2f | %.2f | %s |" % (
                key, e["us"], e["valu"] / 1e6, e["trans"] / 1e6, e["salu"] / 1e6, e["lds"] / 1e6,
                e["mfma"] / 1e6, e["valu_issue_us"], e["valu_issue_frac"], e["wave_wait_frac"],
                e["lds_conflict_per_inst"], e["source_sha"]))
    return "\n".join(lines) + "\n"


def mlp_md(res, title, commands, summary_cmd, cus, xcds):
    def opt(v, f):
        return "-" if v is None or not v else f % v

    lines = (["# " + title, ""] if title else []) + [
        "Counter run (from the repository root, one MI355X, one rocprofv3 pass):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "Summarised with:", "", "    " + summary_cmd, "",
              "%d compute units in %d XCDs. Requests are L1-to-L2 reads of %d-byte lines "
              "(TCP_TCC_READ_REQ); latency is TCP_TCC_READ_REQ_LATENCY per request, in cycles; "
              "in flight = total latency cycles / (compute units x elapsed cycles); TA busy and TA "
              "held by L1 are fractions of elapsed cycles per compute unit (TA_TA_BUSY, "
              "TA_ADDR_STALLED_BY_TC_CYCLES); waves waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES. "
              "MFMA GFLOP executed = SQ_INSTS_VALU_MFMA_MOPS_BF16 x %d; MFMA busy = "
              "SQ_VALU_MFMA_BUSY_CYCLES per SIMD over elapsed cycles. Durations are those of the "
              "counter run."
              % (cus, xcds, LINE_BYTES, MOPS_FLOPS), "",
              "| Kernel | us | Read requests (M) | Requested (MB) | Latency (cycles) | In flight per CU "
              "| Per-CU read rate (B/cycle) | TA busy | TA held by L1 | Waves waiting "
              "| MFMA GFLOP executed | MFMA busy | Source hash |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for key in KERNEL_FILES:
        if key in res:
            e = res[key]
            lines.append("| %s | %.1f | %.2f | %.0f | %.0f | %.1f | %.1f | %.2f | %.2f | %.2f | %s | %s | %s |" % (
                key, e["us"], e["read_requests"] / 1e6, e["requested_mb"], e["latency_cycles"],
                e["in_flight_per_cu"], e["in_flight_per_cu"] * LINE_BYTES / e["latency_cycles"],
                e["ta_busy"], e["ta_stalled_by_l1"], e["wave_wait_frac"],
                opt(e.get("mfma_gflop"), "%.1f"), opt(e.get("mfma_busy"), "%.3f"), e["source_sha"]))
    return "\n".join(lines) + "\n"


def traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes):
    cf = counter_means(copy_fetch_csv, "FETCH_SIZE")["copy"][0]
    cw = counter_means(copy_write_csv, "WRITE_SIZE")["copy"][0]
    fs, ws = copy_bytes / cf, copy_bytes / cw
    fetch = counter_means(fetch_csv, "FETCH_SIZE")
    write = counter_means(write_csv, "WRITE_SIZE")
    out = {"_calibration": {"copy_bytes": copy_bytes, "fetch_bytes_per_unit": fs,
                            "write_bytes_per_unit": ws}}
    for key in KERNEL_FILES:
        if key not in fetch or key not in write:
            continue
        fb, wb = fetch[key][0] * fs, write[key][0] * ws
        out[key] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                    "bytes_per_launch": round(fb + wb), "launches": fetch[key][1],
                    "source_sha": source_hash(key)}
    return out


REQ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_WRREQ_sum",
                "TCC_EA0_WRREQ_64B_sum")


def request_sizes(csv_paths, copy_paths):
    """Mean per launch of the L2-to-memory request counters, per kernel of the path
    and for the copy kernel, from one or more counter CSVs (one rocprofv3 pass
    each: the counters do not all fit one pass); a launch of a multi-kernel key
    sums its kernels' means."""
    def load(paths):
        per = {}
        for path in paths:
            for c in REQ_COUNTERS:
                for key, (mean, _) in counter_means(path, c).items():
                    per.setdefault(key, {})[c] = mean
        return per
    return load(csv_paths), load(copy_paths).get("copy", {})


def request_md(res, cp, copy_bytes, title, commands, summary_cmd):
    lines = (["# " + title, ""] if title else []) + [
        "Counter runs (from the repository root, one MI355X, one rocprofv3 pass each):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "Summarised with:", "", "    " + summary_cmd, ""]
    rd, wr = cp.get("TCC_EA0_RDREQ_sum", 0.0), cp.get("TCC_EA0_WRREQ_sum", 0.0)
    if rd and wr:
        lines += ["The copy kernel moves %d bytes each way: %.0f read requests (%.1f bytes each) and %.0f "
                  "write requests (%.1f bytes each)." % (copy_bytes, rd, copy_bytes / rd, wr, copy_bytes / wr), ""]
    lines += ["Mean per launch.  The 32-byte read requests and the 128-byte ones the derived FETCH_SIZE "
              "counts as bubbles (`TCC_BUBBLE`) are listed beside all read requests; the reads at 128 "
              "bytes each are the kernel's HBM read bytes.", "",
              "| Kernel | read requests | of them 32-byte | TCC_BUBBLE | reads at 128 B (MB) | write requests | "
              "of them 64-byte | writes at 64 B (MB) |", "|---|---|---|---|---|---|---|---|"]
    for key in KERNEL_FILES:
        v = res.get(key)
        if not v:
            continue
        r, r32, bub = v.get("TCC_EA0_RDREQ_sum", 0), v.get("TCC_EA0_RDREQ_32B_sum", 0), v.get("TCC_BUBBLE_sum", 0)
        w, w64 = v.get("TCC_EA0_WRREQ_sum", 0), v.get("TCC_EA0_WRREQ_64B_sum", 0)
        lines.append("| %s | %.0f | %.0f | %.0f | %.1f | %.0f | %.0f | %.1f |" % (
            key, r, r32, bub, r * 128 / 1e6, w, w64, w * 64 / 1e6))
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace", help="kernel trace CSV, or a directory searched for one")
    s.add_argument("out")
    s.add_argument("--title", default="")
    s.add_argument("--command", required=True)
    s.add_argument("--per-kernel", action="store_true",
                   help="one row per launched kernel form (comparisons of variants)")
    s.add_argument("--keys", nargs="*", help="only these path kernels (with --per-kernel)")
    t = sub.add_parser("traffic")
    for n in ("fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument("--" + n, required=True, help="counter CSV, or a directory searched for one")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--md", help="also write a markdown summary here")
    t.add_argument("--title", default="")
    t.add_argument("--command", action="append", default=[],
                   help="a profiling command to record in the markdown (repeatable)")
    q = sub.add_parser("reqsize")
    q.add_argument("--pmc", nargs="+", required=True, help="counter run directories of the path")
    q.add_argument("--copy", nargs="+", required=True, help="counter run directories of the copy kernel")
    q.add_argument("--copy-bytes", type=int, required=True)
    q.add_argument("--md", required=True)
    q.add_argument("--title", default="")
    q.add_argument("--command", action="append", default=[])
    m = sub.add_parser("mlp")
    m.add_argument("--pmc", required=True, help="counter run directory (counter and agent CSVs)")
    m.add_argument("--md", required=True)
    m.add_argument("--json", help="also write the figures here")
    m.add_argument("--title", default="")
    m.add_argument("--command", action="append", default=[])
    i = sub.add_parser("issue")
    i.add_argument("--pmc", nargs=2, required=True, help="the two counter run directories (ISSUE_COUNTERS)")
    i.add_argument("--md", required=True)
    i.add_argument("--ghz", type=float, default=2.4, help="shader clock for the VALU issue time")
    i.add_argument("--title", default="")
    i.add_argument("--command", action="append", default=[])
    a = ap.parse_args(argv)
    here = "python -m mamba_ssd_chunked_03_amd.profiling " + shlex.join(argv if argv else sys.argv[1:])

    def csv_in(p, kind):
        return p if os.path.isfile(p) else _one(os.path.join(p, "**", "*%s.csv" % kind))

    if a.cmd == "reqsize":
        res, cp = request_sizes([csv_in(p, "counter_collection") for p in a.pmc],
                                [csv_in(p, "counter_collection") for p in a.copy])
        with open(a.md, "w") as f:
            f.write(request_md(res, cp, a.copy_bytes, a.title, a.command, here))
    elif a.cmd == "issue":
        cus, _, spc = agent_counts(csv_in(a.pmc[0], "agent_info"))
        res = issue_mix([csv_in(p, "counter_collection") for p in a.pmc], cus, spc, a.ghz)
        with open(a.md, "w") as f:
            f.write(issue_md(res, a.title, a.command, here, cus, spc, a.ghz))
    elif a.cmd == "mlp":
        cus, xcds, spc = agent_counts(csv_in(a.pmc, "agent_info"))
        res = mlp(csv_in(a.pmc, "counter_collection"), cus, xcds, spc)
        with open(a.md, "w") as f:
            f.write(mlp_md(res, a.title, a.command, here, cus, xcds))
        if a.json:
            with open(a.json, "w") as f:
                json.dump(res, f, indent=1, sort_keys=True)
                f.write("\n")
    elif a.cmd == "stats":
        if a.per_kernel:
            text = kernels_table(csv_in(a.trace, "kernel_trace"), a.command, here, a.keys)
        else:
            text, _ = stats_table(csv_in(a.trace, "kernel_trace"), a.command, here)
        with open(a.out, "w") as f:
            f.write(("# " + a.title + "\n\n" if a.title else "") + text)
    else:
        res = traffic(csv_in(a.fetch, "counter_collection"), csv_in(a.write, "counter_collection"),
                      csv_in(a.copy_fetch, "counter_collection"),
                      csv_in(a.copy_write, "counter_collection"), a.copy_bytes)
        with open(a.out, "w") as f:
            json.dump(res, f, indent=1, sort_keys=True)
            f.write("\n")
        if a.md:
            with open(a.md, "w") as f:
                f.write(traffic_md(res, a.title, a.command, here))


def traffic_md(res, title, commands, summary_cmd):
    cal = res["_calibration"]
    lines = (["# " + title, ""] if title else []) + [
        "Counter runs (from the repository root, one MI355X, one rocprofv3 pass each):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", "Summarised with:", "", "    " + summary_cmd, "",
              "Calibration: a copy of %d bytes reads as %.1f bytes per FETCH_SIZE unit and %.1f "
              "bytes per WRITE_SIZE unit; every kernel's counters are scaled by those factors."
              % (cal["copy_bytes"], cal["fetch_bytes_per_unit"], cal["write_bytes_per_unit"]), "",
              "| Kernel | HBM read (MB) | HBM written (MB) | Total per launch (MB) | Source hash |",
              "|---|---|---|---|---|"]
    for key in KERNEL_FILES:
        if key in res:
            e = res[key]
            lines.append("| %s | %.1f | %.1f | %.1f | %s |" % (
                key, e["fetch_bytes"] / 1e6, e["write_bytes"] / 1e6, e["bytes_per_launch"] / 1e6,
                e["source_sha"]))
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    main()
