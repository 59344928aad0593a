#!/usr/bin/env python3
"""Offline sweep for the per-shape table of the cross-chunk state passing.

For a grid of shapes (chunks per sequence x independent lanes, at headdim 64 and
dstate 128), every state-passing variant (SSD_FLAG_SCAN_VARIANT 1..7: the
associative scan at four segment shapes, the sequential carry with 1, 4 and 8
chunks of loads in flight) is timed on the GPU through ssd_stage_state_passing,
and the fastest is written to tuning/table.json beside all the timings.  build.py
compiles that file into the library, where variant 0 (the default) looks up the
measured shape nearest to a problem's.  This is the analogue of the pages'
offline configuration generator (aitrends.kr/articles/109906, "putting autotune
results into the training pipeline"): tuned once per GPU, saved to a file,
loaded with no search at run time.

Run on the GPU:  python mamba_ssd_chunked_03_amd/tuning/sweep.py [--out PATH]
Then rebuild (python __graft_entry__.py) so that the library uses the table.
"""
import argparse
import ctypes
import datetime
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

VARIANTS = {1: "associative 4x2", 2: "associative 8x4", 3: "associative 16x4", 4: "associative 16x8",
            5: "sequential, 1 chunk in flight", 6: "sequential, 4 chunks in flight",
            7: "sequential, 8 chunks in flight"}
CHUNKS = (4, 8, 16, 32, 64, 128, 256, 512)
# sequences x heads at headdim 64, dstate 128 (lanes = seqs * heads * 2048)
LANE_SHAPES = ((1, 16), (1, 64), (4, 64), (8, 64))
P, N, Q = 64, 128, 256
MAX_STATE_BYTES = 2 << 30  # skip shapes whose chunk states pass 2 GiB


def time_variant(lib, ssd, torch, prob, T, decay, Hp, final, ws, v, reps):
    prob.flags = ssd.FLAG_SCAN_VARIANT(v)
    st = torch.cuda.current_stream()
    args = (ctypes.byref(prob), ctypes.c_void_p(T.data_ptr()), ctypes.c_void_p(decay.data_ptr()), None,
            None, Q, ctypes.c_void_p(Hp.data_ptr()), ctypes.c_void_p(final.data_ptr()),
            ctypes.c_void_p(ws.data_ptr()), ws.numel(), ctypes.c_void_p(st.cuda_stream))
    fn = lib.ssd_stage_state_passing
    for _ in range(3):
        if fn(*args) != 0:
            raise RuntimeError("variant %d failed" % v)
    torch.cuda.synchronize()
    res = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn(*args)
        e1.record(st)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e3 / reps)
    res.sort()
    return res[len(res) // 2]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(HERE, "table.json"))
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    import torch
    from mamba_ssd_chunked_03_amd import ssd
    if not torch.cuda.is_available():
        sys.exit("sweep.py needs a GPU")
    lib = ssd.lib()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(1)
    rows = []
    for chunks in CHUNKS:
        for seqs, heads in LANE_SHAPES:
            lanes = seqs * heads * P * N // 4
            nck = seqs * chunks
            if nck * heads * P * N * 4 > MAX_STATE_BYTES:
                continue
            prob = ssd.Problem(seqs, chunks * Q, heads, P, N, 1, 0, ssd.BF16, 1, 0)
            T = torch.randn(nck, heads, P, N, generator=gen, device=dev)
            decay = -torch.rand(nck, heads, generator=gen, device=dev) * 8.0   # log2 units
            Hp = torch.empty(nck, heads, P, N, device=dev)
            final = torch.empty(seqs, heads, P, N, device=dev)
            ws = torch.empty(max(1, lib.ssd_stage_workspace_bytes(ctypes.byref(prob), Q, 0)),
                             dtype=torch.uint8, device=dev)
            us = {v: time_variant(lib, ssd, torch, prob, T, decay, Hp, final, ws, v, args.reps)
                  for v in VARIANTS}
            best = min(us, key=us.get)
            nbytes = nck * heads * P * N * 8 + nck * heads * 4 + 2 * seqs * heads * P * N * 4
            rows.append({"chunks_per_seq": chunks, "lanes": lanes, "seqs": seqs, "heads": heads,
                         "variant": best, "us": {str(v): round(t, 2) for v, t in us.items()},
                         "best_frac_hbm": round(nbytes / (us[best] * 1e-6) / 8e12, 3)})
            print("chunks %4d lanes %8d: best %d (%s) %.1f us; %s" % (
                chunks, lanes, best, VARIANTS[best], us[best],
                " ".join("%d:%.1f" % (v, t) for v, t in us.items())), flush=True)
            del T, decay, Hp, final, ws
            torch.cuda.empty_cache()
    out = {"generated_by": "mamba_ssd_chunked_03_amd/tuning/sweep.py",
           "date": datetime.date.today().isoformat(),
           "gpu": torch.cuda.get_device_name(dev),
           "shape": "headdim %d, dstate %d, chunk %d, fp32 chunk states in, fp32 passed states out" % (P, N, Q),
           "variants": {str(k): v for k, v in VARIANTS.items()},
           "state_passing": rows}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", args.out)


if __name__ == "__main__":
    main()
