#!/usr/bin/env python3
"""Offline sweep for the per-shape table of the library's shape choices.

State passing: for a grid of shapes (chunks per sequence x independent lanes, at
headdim 64 and dstate 128), every state-passing variant (SSD_FLAG_SCAN_VARIANT
1..7: the associative scan at four segment shapes, the sequential carry with 1, 4
and 8 chunks of loads in flight) is timed on the GPU through
ssd_stage_state_passing.

Chunk-state kernels: for a grid of (headdim, dstate, heads per group, chunk size)
at 2 x 8192 tokens and 64 heads, every form the shape allows (SSD_FLAG_CS_VARIANT
1..3: one head per workgroup; two heads of a group per workgroup; two heads with
C.B^T formed inside) is timed as a training step (ssd_fwd keeping its
intermediates, then ssd_bwd from them), the forward alone beside it.

The fastest of each is written to tuning/table.json beside all the timings.
build.py compiles that file into the library, where variant 0 (the default)
looks up the measured shape nearest to a problem's (state passing) or equal to
it (chunk-state kernels).  This is the analogue of the pages'
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


CS_VARIANTS = {1: "one head per workgroup, C.B^T by its own kernel",
               2: "two heads per workgroup, C.B^T by its own kernel",
               3: "two heads per workgroup, C.B^T inside the chunk-state kernel"}
CS_HEADDIMS, CS_DSTATES, CS_HPG, CS_CHUNKS = (32, 64, 128), (64, 128), (2, 4, 8, 16), (128, 256)
CS_BATCH, CS_SEQLEN, CS_HEADS = 2, 8192, 64


def median_ms(torch, fn, reps):
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    res = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / reps)
    res.sort()
    return res[len(res) // 2]


def sweep_chunk_state(torch, ssd, dev, reps):
    """Training-step and forward ms of every chunk-state form each shape allows."""
    lib = ssd.lib()
    gen = torch.Generator(device=dev).manual_seed(2)
    rows = []
    B, L, H = CS_BATCH, CS_SEQLEN, CS_HEADS
    for P in CS_HEADDIMS:
        for N in CS_DSTATES:
            for hpg in CS_HPG:
                G = H // hpg
                x = torch.randn(B, L, H, P, generator=gen, device=dev).to(torch.bfloat16)
                Bm = (torch.randn(B, L, G, N, generator=gen, device=dev) / N ** 0.5).to(torch.bfloat16)
                C = (torch.randn(B, L, G, N, generator=gen, device=dev) / N ** 0.5).to(torch.bfloat16)
                dy = torch.randn(B, L, H, P, generator=gen, device=dev).to(torch.bfloat16)
                dt = torch.randn(B, L, H, generator=gen, device=dev)
                bias = torch.rand(H, generator=gen, device=dev) * 2 - 4
                A = -torch.exp(torch.rand(H, generator=gen, device=dev) * math.log(16))
                D = torch.randn(H, generator=gen, device=dev)
                for Q in CS_CHUNKS:
                    valid = []
                    for v in CS_VARIANTS:
                        prob = ssd.problem(x, Bm, flags=ssd.FLAG_CS_VARIANT(v))
                        if lib.ssd_cs_variant(ctypes.byref(prob), Q, 0) == v:
                            valid.append(v)
                    if len(valid) < 2:
                        continue  # one form: nothing to choose
                    need = lib.ssd_bwd_workspace_bytes(ctypes.byref(ssd.problem(x, Bm)), Q, 0)
                    ws = torch.empty(need, dtype=torch.uint8, device=dev)
                    step, fwd = {}, {}
                    for v in valid:
                        kw = dict(D=D, dt_bias=bias, chunk_size=Q, cs_variant=v)
                        f, y, fin = ssd.fwd(x, dt, A, Bm, C, workspace=ws, save_for_backward=True, prepare=True, **kw)
                        f()
                        b, _ = ssd.bwd(x, dt, A, Bm, C, dy, workspace=ws, from_saved=True, prepare=True, **kw)
                        fp, _, _ = ssd.fwd(x, dt, A, Bm, C, out=y, final=fin, prepare=True, **kw)
                        step[v] = median_ms(torch, lambda: (f(), b()), reps)
                        fwd[v] = median_ms(torch, fp, reps)
                    best = min(step, key=step.get)
                    rows.append({"headdim": P, "dstate": N, "heads_per_group": hpg, "chunk": Q,
                                 "variant": best, "us": {str(v): round(t * 1e3, 1) for v, t in step.items()},
                                 "fwd_us": {str(v): round(t * 1e3, 1) for v, t in fwd.items()}})
                    print("P %3d N %3d heads/group %2d chunk %3d: best %d; step %s; fwd %s" % (
                        P, N, hpg, Q, best, " ".join("%d:%.1f" % (v, t * 1e3) for v, t in step.items()),
                        " ".join("%d:%.1f" % (v, t * 1e3) for v, t in fwd.items())), flush=True)
                    del ws
                del x, Bm, C, dy, dt
                torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=os.path.join(HERE, "table.json"))
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--only", choices=("state_passing", "chunk_state"), default=None,
                    help="sweep one section; the other is kept from the existing table")
    args = ap.parse_args()
    import torch
    from mamba_ssd_chunked_03_amd import ssd
    if not torch.cuda.is_available():
        sys.exit("sweep.py needs a GPU")
    lib = ssd.lib()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(1)
    old = {}
    if args.only and os.path.exists(args.out):
        with open(args.out) as f:
            old = json.load(f)
    rows = []
    for chunks in (CHUNKS if args.only != "chunk_state" else ()):
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
    if args.only == "chunk_state":
        rows = old.get("state_passing", [])
    cs_rows = sweep_chunk_state(torch, ssd, dev, args.reps) if args.only != "state_passing" \
        else old.get("chunk_state", [])
    out = {"generated_by": "mamba_ssd_chunked_03_amd/tuning/sweep.py",
           "date": datetime.date.today().isoformat(),
           "gpu": torch.cuda.get_device_name(dev),
           "shape": "headdim %d, dstate %d, chunk %d, fp32 chunk states in, fp32 passed states out" % (P, N, Q),
           "variants": {str(k): v for k, v in VARIANTS.items()},
           "state_passing": rows,
           "chunk_state_shape": "%d x %d tokens, %d heads, bf16; us = training step (forward keeping its "
                                "intermediates, then the backward), fwd_us = forward alone" % (
                                    CS_BATCH, CS_SEQLEN, CS_HEADS),
           "chunk_state_variants": {str(k): v for k, v in CS_VARIANTS.items()},
           "chunk_state": cs_rows}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", args.out)


if __name__ == "__main__":
    main()
