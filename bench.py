#!/usr/bin/env python3
"""Benchmark of the SSD chunked scan on one MI355X.

Workload: the Mamba-2 layer shape the pages measure on (batch 2, sequence
length 8192, bf16), with seeded synthetic inputs: 64 heads of headdim 64,
dstate 128, 8 groups, chunk 256 (dt raw N(0,1), bias U[-4,-2], softplus in the
kernel, zero initial state, dout N(0,1)).  One step is one pass of the whole
path: ssd_fwd keeping its intermediates, then ssd_bwd reusing them (a training
step); the variant whose backward recomputes them is timed and reported too.  Inputs and outputs
are resident in HBM before timing starts; the K timed steps are bracketed by
torch.cuda.synchronize() and HIP events recorded on the stream the library
launches on (torch's current stream).

Printed (last line, JSON): tokens/s of the step, ms per step, every kernel's
time and algorithmic HBM rate (each kernel timed on its own: the step's own
launch re-issued through the single-kernel flags of ssd_fwd / ssd_bwd, with
HIP events on the library's stream), the roofline of the dominant kernel, and
the CPU oracle timed on a bounded sample.
"""
import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD layer tokens/s + ms/call (fwd, fwd+bwd) & % HBM peak, B=2 L=8192"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense
MFMA_F32_PEAK_TFLOPS = 157.3    # dense fp32 matrix
FLUSH_BYTES = 512 << 20         # > the 256 MB last-level cache, read before each cold call
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # 50 untimed steps (~40 ms) bring the GPU to its working clock first: after 5,
    # a 20-step window read ~6 % slower than the same steps later in the run
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernels", action="store_true", help="skip the per-kernel timings")
    ap.add_argument("--fwd-only", action="store_true", help="time ssd_fwd alone as the step")
    ap.add_argument("--no-ab", action="store_true",
                    help="skip the state-passing and chained-forward comparisons")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the long-context and packed workloads reported beside the headline")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run the library's plain copy kernel (counter calibration)")
    return ap.parse_args()


def kernel_bytes(B, L, H, P, N, G, Q, nck, nseq, esz, init=True, d_final=False):
    """Algorithmic HBM bytes of each kernel of the step: every array the kernel
    must read is read once and every array it produces is written once (no
    cache re-reads, no padding tiles; C.B^T and its adjoint count as their causal
    triangle, R and K as one value per token and head).  Passed states and their
    adjoints are bf16 on this path; chunk states and their adjoints fp32."""
    tok = B * L
    f32_tok = nck * H * Q * 4           # one fp32 value per (chunk slot, head, token)
    dt = tok * H * 4
    decay = nck * H * 4
    st32 = nck * H * P * N * 4          # chunk states T, adjoint chunk states U
    st16 = nck * H * P * N * esz        # passed states H, their adjoints dE
    x = tok * H * P * esz
    bc = tok * G * N * esz
    tri = nck * G * (Q * (Q + 1) // 2) * esz
    s0 = nseq * H * P * N * 4
    return {
        "chunk_cumsum": dt + 2 * f32_tok + decay,        # (stage entry point; inside chunk_state)
        "chunk_state": dt + x + bc + 2 * f32_tok + decay + st32,  # with the cumsum formed inline
        "state_passing": st32 + decay + st16 + (s0 if init else 0) + s0,
        "bmm_chunk": 2 * bc + 2 * tri,                   # CB and its transpose (saved for bwd)
        "chunk_scan": 2 * x + bc + tri + 2 * f32_tok + st16,
        "dstates": x + bc + f32_tok + st32,
        "reverse_state_passing": st32 + decay + st16 + (s0 if d_final else 0) + s0,
        "bwd_dx": 3 * x + bc + tri + 2 * f32_tok + decay + 2 * st16 + 2 * f32_tok,
        "bwd_dcb": 2 * x + tri + 2 * f32_tok + tri + 2 * f32_tok,
        "bwd_dc": 2 * bc + x + tri + f32_tok + st16 + bc + f32_tok,
        "bwd_db": x + bc + tri + 2 * f32_tok + st16 + bc,
        # the one kernel for dB and dC: x, dy, B, C, C.B^T, acs, delta, H, dE read;
        # dB, dC, r, R, K written
        "bwd_dbc": 2 * x + 2 * bc + tri + 2 * f32_tok + 2 * st16 + 2 * bc + 3 * f32_tok,
        "bwd_finalize": dt + 6 * f32_tok + dt,
    }


def kernel_flops(B, L, H, P, N, G, Q, nck):
    """Algorithmic matrix-product flops of each kernel (causal triangles only;
    the bf16 hi/lo split of chunk_state is not counted).  Kernels without
    products are absent."""
    tok = B * L
    state = 2 * tok * H * P * N                 # a per-token P x N contraction
    tri = Q * (Q + 1)                           # 2 x causal entries of one chunk
    return {
        "chunk_state": state,
        "bmm_chunk": nck * G * N * tri,
        "chunk_scan": nck * H * P * tri + state,
        "dstates": state,
        "bwd_dx": nck * H * P * tri + state,
        "bwd_dcb": nck * H * P * tri,
        "bwd_dc": nck * G * N * tri + state,
        "bwd_db": nck * G * N * tri + state,
        "bwd_dbc": nck * H * P * tri + 2 * (nck * G * N * tri + state),
    }


def load_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current source of this kernel (else None)."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(kernel)
    from mamba_ssd_chunked_03_amd.profiling import source_hash
    if not e or e.get("source_sha") != source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(with_bwd, budget_s=10.0):
    """The oracle as it stands, on a bounded sample of the same workload: batch
    row 0 with all 64 heads, in windows of 512 tokens (fresh seeded inputs per
    window) until about ``budget_s`` seconds of CPU work; the oracle's cost is
    linear in tokens at a fixed head count, so tokens/s carries over."""
    import threadpoolctl
    from mamba_ssd_chunked_03_amd import inputs
    from oracle import recurrence
    threadpoolctl.threadpool_limits(1)  # the reported core count is the one used
    T = 512
    done, sec = 0, 0.0
    while sec < budget_s and done < 8192:
        inp = inputs.make_inputs(1, T, 64, 64, 128, 8, io="bf16", bwd=True, seed=100 + done)
        a = inputs.to_f64(inp)
        t0 = time.perf_counter()
        recurrence.fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], D=a["D"], dt_bias=a["dt_bias"],
                       init=a["init"], dt_softplus=True)
        if with_bwd:
            recurrence.bwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["dout"], D=a["D"],
                           dt_bias=a["dt_bias"], init=a["init"], dt_softplus=True)
        sec += time.perf_counter() - t0
        done += T
    return {"value": round(done / sec, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "batch row 0, 64 heads, %d tokens in 512-token windows, %s, fp64 numpy "
                      "token loop, %.1f s" % (done, "fwd+bwd" if with_bwd else "fwd", sec),
            "cpu": platform.processor() or platform.machine()}


def _worker_init():
    sys.path.insert(0, ROOT)
    import threadpoolctl
    threadpoolctl.threadpool_limits(1)  # one thread per worker: cores = workers
    from mamba_ssd_chunked_03_amd import inputs  # noqa: F401  (imports before timing)
    from oracle import recurrence  # noqa: F401


def _oracle_window(args):
    """One 512-token window of the oracle on a subset of heads (a worker task)."""
    seed, heads, with_bwd = args
    if seed < 0:
        return 0.0  # start-up task
    from mamba_ssd_chunked_03_amd import inputs
    from oracle import recurrence
    inp = inputs.make_inputs(1, 512, 64, 64, 128, 8, io="bf16", bwd=True, seed=seed)
    a = inputs.to_f64(inp)
    t0 = time.perf_counter()
    recurrence.fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], D=a["D"], dt_bias=a["dt_bias"],
                   init=a["init"], dt_softplus=True, heads=heads)
    if with_bwd:
        recurrence.bwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["dout"], D=a["D"],
                       dt_bias=a["dt_bias"], init=a["init"], dt_softplus=True, heads=heads)
    return time.perf_counter() - t0


def cpu_baseline_parallel(with_bwd):
    """The same oracle with independent 512-token windows (all 64 heads each)
    spread over a process pool, one window per worker (spawned workers: they
    import only numpy and the oracle)."""
    import multiprocessing as mp
    nproc = max(1, min(16, os.cpu_count() or 1))
    windows = nproc
    tasks = [(100 + 512 * wi, None, with_bwd) for wi in range(windows)]
    with mp.get_context("spawn").Pool(nproc, initializer=_worker_init) as pool:
        pool.map(_oracle_window, [(-1, None, False)] * nproc, chunksize=1)  # workers started
        t0 = time.perf_counter()
        pool.map(_oracle_window, tasks, chunksize=1)
        sec = time.perf_counter() - t0
    done = 512 * windows
    return {"value": round(done / sec, 2), "unit": "tokens/s", "cores": nproc, "kind": "oracle",
            "sample": "batch row 0, 64 heads, %d tokens in 512-token windows, one per "
                      "single-threaded process of %d (input generation included), %s, %.1f s"
                      % (done, nproc, "fwd+bwd" if with_bwd else "fwd", sec)}


class Workload:
    """One named workload on the GPU: seeded inputs resident in HBM, workspaces,
    and the library calls marshalled once (the timed loops only issue them)."""

    def __init__(self, cfg_id, dev, with_bwd=True, inp=None, chunk=None):
        import ctypes
        import torch
        from mamba_ssd_chunked_03_amd import inputs, ssd
        self.cfg_id = cfg_id
        if inp is None:  # a named workload, else the given inputs at the given chunk size
            self.Q = Q = inputs.CONFIGS[cfg_id]["chunk"]
            inp = inputs.config_inputs(cfg_id)
        else:
            self.Q = Q = chunk
        self.sha256 = input_sha256(inp)
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        self.d = d
        x, Bm = d["x"], d["B"]
        self.cu = d["cu_seqlens"]
        self.packed = int(self.cu is not None)
        self.lengths = None if self.cu is None else [int(b - a) for a, b in zip(inp["cu_seqlens"][:-1],
                                                                              inp["cu_seqlens"][1:])]
        self.Bsz, self.L, self.H, self.P = x.shape
        self.G, self.N = Bm.shape[2], Bm.shape[3]
        self.nseq = len(self.lengths) if self.packed else self.Bsz
        self.prob = prob = ssd.problem(x, Bm, self.cu)
        lib = ssd.lib()
        ws_f = torch.empty(lib.ssd_fwd_workspace_bytes(ctypes.byref(prob), Q, self.packed),
                           dtype=torch.uint8, device=dev)
        self.y = torch.empty_like(x)
        self.final = torch.empty(self.nseq, self.H, self.P, self.N, dtype=torch.float32, device=dev)
        self.common = dict(D=d["D"], dt_bias=d["dt_bias"], init=d["init"], cu_seqlens=self.cu, chunk_size=Q)
        self.args = (x, d["dt"], d["A"], Bm, d["C"])
        self.fwd, _, _ = ssd.fwd(*self.args, workspace=ws_f, out=self.y, final=self.final, prepare=True,
                                 **self.common)
        self.with_bwd = with_bwd and d["dout"] is not None
        self.fwd_mask = lib.ssd_fwd_kernel_mask(ctypes.byref(prob), Q, self.packed)
        self.bwd_mask = lib.ssd_bwd_kernel_mask(ctypes.byref(prob), Q, self.packed)
        self.ws_b = torch.empty(lib.ssd_bwd_workspace_bytes(ctypes.byref(prob), Q, self.packed),
                                dtype=torch.uint8, device=dev)
        # the training forward keeps its intermediates for the backward
        self.fwd_save, _, _ = ssd.fwd(*self.args, workspace=self.ws_b, out=self.y, final=self.final,
                                      save_for_backward=True, prepare=True, **self.common)
        self.grads = None
        if self.with_bwd:
            self.bwd_saved, self.grads = ssd.bwd(*self.args, d["dout"], workspace=self.ws_b,
                                                 from_saved=True, prepare=True, **self.common)
            self.bwd_recompute, _ = ssd.bwd(*self.args, d["dout"], workspace=self.ws_b, grads=self.grads,
                                            prepare=True, **self.common)

    @property
    def tokens(self):
        return self.Bsz * self.L

    def chunks(self):
        """chunk slots that hold tokens (packed sequences: each cut from its own start)"""
        if self.packed:
            return sum((n + self.Q - 1) // self.Q for n in self.lengths)
        return self.Bsz * ((self.L + self.Q - 1) // self.Q)

    def step(self):
        if self.with_bwd:
            self.fwd_save()
            self.bwd_saved()
        else:
            self.fwd()

    def kernel_launches(self):
        """name -> a launch of that kernel alone, on the buffers of a complete call"""
        from mamba_ssd_chunked_03_amd import ssd
        self.fwd_save()
        if self.with_bwd:
            self.bwd_saved()
        fns = {}
        for k, name in enumerate(ssd.FWD_KERNELS, 1):
            if not self.fwd_mask & (1 << (k - 1)):
                continue
            fns[name] = ssd.fwd(*self.args, workspace=self.ws_b, out=self.y, final=self.final,
                                save_for_backward=True, only_kernel=k, prepare=True, **self.common)[0]
        if self.with_bwd:
            for k, name in enumerate(ssd.BWD_KERNELS, 1):
                if not self.bwd_mask & (1 << (k - 1)):
                    continue
                if k == 4 and not self.bwd_mask & 16:
                    name = ssd.BWD_FUSED_KERNEL
                fns[name] = ssd.bwd(*self.args, self.d["dout"], workspace=self.ws_b, from_saved=True,
                                    grads=self.grads, only_kernel=k, prepare=True, **self.common)[0]
        return fns

    def fused_bwd_ab(self, tm, per):
        """The backward from a saved forward with dB and dC formed by three kernels
        (the default) against one kernel over one pass of x and dy
        (SSD_FLAG_BWD_FUSED), and the training step with each; warm and cold ms."""
        from mamba_ssd_chunked_03_amd import ssd
        if not self.with_bwd:
            return None
        fused, _ = ssd.bwd(*self.args, self.d["dout"], workspace=self.ws_b, from_saved=True, grads=self.grads,
                           fused=True, prepare=True, **self.common)
        res = {}
        for key, fn in (("three_kernels", self.bwd_saved), ("one_kernel", fused)):
            med, lo, hi = tm.trials(fn, per)
            step = lambda fn=fn: (self.fwd_save(), fn())
            smed = tm.trials(step, per)[0]
            res[key] = {"bwd_ms": round(med, 4), "bwd_ms_min": round(lo, 4), "bwd_ms_max": round(hi, 4),
                        "bwd_ms_cold": round(tm.cold(fn, wait=True), 4), "step_ms": round(smed, 4)}
            print("bench: backward %-10s %.4f ms (step %.4f ms)" % (key, med, smed), file=sys.stderr, flush=True)
        self.bwd_saved()  # the gradients of the default path again
        return res

    def chained_ab(self, tm, per):
        """The fused single-pass forward (SSD_FLAG_CHAINED_FWD: C.B^T kernel, then one
        kernel with the chunk carry handed from workgroup to workgroup) against the
        staged forward, both plain and keeping the intermediates for the backward;
        warm and cold ms."""
        from mamba_ssd_chunked_03_amd import ssd
        import ctypes
        import torch
        res = {}
        for save in (False, True):
            ws = self.ws_b if save else torch.empty_like(self.ws_b[:max(1, ssd.lib().ssd_fwd_workspace_bytes(
                ctypes.byref(self.prob), self.Q, self.packed))])
            for key, ch in (("staged", False), ("chained", True)):
                fn = ssd.fwd(*self.args, workspace=ws, out=self.y, final=self.final, save_for_backward=save,
                             chained=ch, prepare=True, **self.common)[0]
                med, lo, hi = tm.trials(fn, per)
                e = res.setdefault("save" if save else "plain", {})
                e[key] = {"ms": round(med, 4), "ms_min": round(lo, 4), "ms_max": round(hi, 4),
                          "ms_cold": round(tm.cold(fn, wait=True), 4)}
                print("bench: forward %s %-8s %.4f ms" % ("save " if save else "plain", key, med),
                      file=sys.stderr, flush=True)
        self.fwd_save()  # the workspace holds the default path's intermediates again
        if self.with_bwd:
            self.bwd_saved()
        return res

    def assoc_variant(self):
        """The associative-scan segment shape sized to this workload's chains
        (the library's rule when it has no tuned table)."""
        chain = self.chunks() // self.nseq
        return 1 if chain <= 8 else 2 if chain <= 32 else 3 if chain <= 64 else 4

    def scan_ab(self, tm, per):
        """The state-passing kernels timed alone as the log-depth associative scan
        (segments sized to the chains), as the plain sequential-carry loop it
        replaces (SSD_FLAG_SEQUENTIAL_SCAN), and as the tuned table's choice (the
        default), on the same buffers: warm and cold ms and fraction of 8 TB/s."""
        from mamba_ssd_chunked_03_amd import ssd
        nbytes, _ = self.alg()
        res = {}
        for key, v in (("associative", self.assoc_variant()), ("sequential", 5), ("table", 0)):
            self.fwd_save()
            if self.with_bwd:
                self.bwd_saved()
            runs = {"state_passing": ssd.fwd(*self.args, workspace=self.ws_b, out=self.y, final=self.final,
                                             save_for_backward=True, only_kernel=2, scan_variant=v,
                                             prepare=True, **self.common)[0]}
            if self.with_bwd:
                runs["reverse_state_passing"] = ssd.bwd(*self.args, self.d["dout"], workspace=self.ws_b,
                                                        from_saved=True, grads=self.grads, only_kernel=2,
                                                        scan_variant=v, prepare=True, **self.common)[0]
            for name, fn in runs.items():
                ms = tm.trials(fn, per)[0]
                ms_cold = tm.cold(fn)
                e = res.setdefault(name, {"alg_bytes": nbytes[name]})
                e[key] = {"variant": v, "ms": round(ms, 4), "ms_cold": round(ms_cold, 4),
                          "frac_hbm": round(nbytes[name] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "frac_hbm_cold": round(nbytes[name] / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                print("bench: %s %-12s %.4f ms (cold %.4f)" % (name, key, ms, ms_cold), file=sys.stderr,
                      flush=True)
        self.fwd_save()  # the workspace holds the default path's intermediates again
        if self.with_bwd:
            self.bwd_saved()
        return res

    def alg(self):
        """algorithmic bytes and flops per kernel of this workload's step"""
        nck = self.chunks()
        nbytes = kernel_bytes(self.Bsz, self.L, self.H, self.P, self.N, self.G, self.Q, nck, self.nseq, 2,
                              init=self.d["init"] is not None, d_final=False)
        nflops = kernel_flops(self.Bsz, self.L, self.H, self.P, self.N, self.G, self.Q, nck)
        # where the chunk-state kernel forms C.B^T (and its transpose) itself, its
        # bytes and flops are that kernel's and no C.B^T kernel is launched
        if not self.fwd_mask & 4:
            nbytes["chunk_state"] += nbytes["bmm_chunk"] - self.tokens * self.G * self.N * 2  # (B read once)
            nflops["chunk_state"] += nflops["bmm_chunk"]
        return nbytes, nflops


def input_sha256(inp):
    """SHA-256 of every input tensor's bytes as drawn on the host (the bits the
    GPU and the oracle both consume)."""
    import hashlib
    out = {}
    for k, v in sorted(inp.items()):
        if hasattr(v, "numpy"):
            t = v.detach().cpu().contiguous()
            if t.dtype.is_floating_point and t.element_size() == 2:
                t = t.view(dtype=__import__("torch").int16)
            out[k] = hashlib.sha256(t.numpy().tobytes()).hexdigest()
    return out


class Timer:
    """Timing helpers: HIP events on torch's current stream, which is the stream
    every library call of the step is issued on (a call's side-stream kernels are
    joined back to it before the call's last kernel)."""

    def __init__(self, dev):
        import torch
        self.torch = torch
        self.flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def timed(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(st)
        for _ in range(steps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        return e0.elapsed_time(e1) / steps, wall

    def trials(self, fn, per, n=7, warmup=2):
        """median / min / max ms per call over n back-to-back windows of `per` calls"""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        res = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(per):
                fn()
            e1.record(st)
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) / per)
        res.sort()
        return res[n // 2], res[0], res[-1]

    def cold(self, fn, n=7, wait=False):
        """median ms of single calls, each after a 512 MiB read (outside the event pair)
        that replaces the last-level cache's contents with clean lines.  A single
        kernel is issued right behind the read, long before the read ends.  wait: the
        host waits for the read first, for calls of many kernels (a training step's
        launches take the host about as long, ~0.1 ms, as the read takes the GPU, so
        issued right behind it, later launches could arrive after the GPU had run dry
        and that idle time would be timed; after the wait only the first launch's
        issue is)."""
        torch = self.torch
        st = torch.cuda.current_stream()
        res = []
        for _ in range(n):
            self.flush.sum()
            if wait:
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fn()
            e1.record(st)
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1))
        res.sort()
        return res[n // 2]


def kernel_table(w, tm, per, label=""):
    """Every kernel of a workload's step on its own (the step's own launch re-issued
    through the single-kernel flags), warm and cold, against its algorithmic bytes."""
    from mamba_ssd_chunked_03_amd import ssd
    nbytes, nflops = w.alg()
    kernels = {}
    for name, fn in w.kernel_launches().items():
        ms, ms_min, ms_max = tm.trials(fn, per)
        ms_cold = tm.cold(fn)
        gbs = nbytes[name] / (ms * 1e-3) / 1e9
        e = {"ms": round(ms, 4), "ms_min": round(ms_min, 4), "ms_max": round(ms_max, 4),
             "ms_cold": round(ms_cold, 4), "alg_bytes": nbytes[name], "GB/s": round(gbs, 1),
             "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
             "frac_hbm_cold": round(nbytes[name] / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if name in nflops:
            tf = nflops[name] / (ms * 1e-3) / 1e12
            e["alg_tflops"] = round(tf, 1)
            e["frac_mfma"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
        kernels[name] = e
        print("bench: %skernel %-22s %.4f ms (cold %.4f)  %.0f GB/s" % (label, name, ms, ms_cold, gbs),
              file=sys.stderr, flush=True)

    def aggregate(names):
        b = sum(kernels[n]["alg_bytes"] for n in names)
        t = sum(kernels[n]["ms"] for n in names)
        tc = sum(kernels[n]["ms_cold"] for n in names)
        return {"ms": round(t, 4), "alg_bytes": b, "GB/s": round(b / (t * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "frac_hbm_cold": round(b / (tc * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    names = list(kernels)
    kernels["_forward_aggregate"] = aggregate([n for n in ssd.FWD_KERNELS if n in kernels])
    if w.with_bwd:
        kernels["_backward_aggregate"] = aggregate(
            [n for n in list(ssd.BWD_KERNELS) + [ssd.BWD_FUSED_KERNEL] if n in kernels])
    kernels["_all"] = aggregate(names)
    return kernels


def other_workload(cfg_id, dev, tm, steps, label, ab=True):
    """Forward (and, where the workload has one, training step) timings of another
    named workload, with its kernel table; reported beside the headline."""
    from mamba_ssd_chunked_03_amd import inputs
    c = inputs.CONFIGS[cfg_id]
    w = Workload(cfg_id, dev)
    per = max(1, steps // 4)
    fwd_med, fwd_min, fwd_max = tm.trials(w.fwd, per)
    res = {"workload": "%s: batch %d, %d tokens%s, %d heads, headdim %d, dstate %d, %d groups, chunk %d, "
                       "bf16" % (label, w.Bsz, w.L, "" if not w.packed else
                                 " packed in %d sequences %s" % (w.nseq, w.lengths),
                                 w.H, w.P, w.N, w.G, w.Q),
           "input_sha256": w.sha256,
           "fwd": {"ms": round(fwd_med, 4), "ms_min": round(fwd_min, 4), "ms_max": round(fwd_max, 4),
                   "ms_cold": round(tm.cold(w.fwd, wait=True), 4),
                   "tokens/s": round(w.tokens / (fwd_med * 1e-3), 1)}}
    print("bench: %s fwd %.3f ms" % (label, fwd_med), file=sys.stderr, flush=True)
    if w.with_bwd:
        st_med, st_min, st_max = tm.trials(w.step, per)
        res["fwd_bwd"] = {"ms": round(st_med, 4), "ms_min": round(st_min, 4), "ms_max": round(st_max, 4),
                          "ms_cold": round(tm.cold(w.step, wait=True), 4),
                          "tokens/s": round(w.tokens / (st_med * 1e-3), 1),
                          "bwd_ms": round(tm.trials(w.bwd_saved, per)[0], 4)}
        print("bench: %s fwd+bwd %.3f ms" % (label, st_med), file=sys.stderr, flush=True)
    res["kernels"] = kernel_table(w, tm, per, label + " ")
    if ab:
        res["state_passing_ab"] = w.scan_ab(tm, per)
        res["fused_chained_forward"] = w.chained_ab(tm, per)
        res["bwd_dbdc_ab"] = w.fused_bwd_ab(tm, per)
    del w
    return res


def fp32_layer(dev, tm, steps):
    """The layer workload's shape with fp32 io, which runs the fp32 path (true fp32
    products on the fp32 matrix cores): forward, and the training step (forward
    keeping its intermediates, then backward), against the dense fp32 matrix peak.
    Reported beside the headline, not as it."""
    from mamba_ssd_chunked_03_amd import inputs
    B, L, H, P, N, G, Q = 2, 8192, 64, 64, 128, 8, 256
    w = Workload(None, dev, inp=inputs.make_inputs(B, L, H, P, N, G, io="f32", init="zeros", bwd=True, seed=5),
                 chunk=Q)
    per = max(1, steps // 4)
    fl = kernel_flops(B, L, H, P, N, G, Q, w.chunks())
    fwd_fl = fl["chunk_state"] + fl["bmm_chunk"] + fl["chunk_scan"]
    bwd_fl = fl["dstates"] + fl["bwd_dx"] + fl["bwd_dcb"] + fl["bwd_dc"] + fl["bwd_db"]
    res = {"workload": "fp32 io: batch %d, seqlen %d, %d heads, headdim %d, dstate %d, %d groups, chunk %d"
                       % (B, L, H, P, N, G, Q), "input_sha256": w.sha256}
    for name, fn, flops in (("fwd", w.fwd, fwd_fl), ("bwd", w.bwd_saved, bwd_fl), ("fwd_bwd", w.step, None)):
        ms, ms_min, ms_max = tm.trials(fn, per)
        r = {"ms": round(ms, 4), "ms_min": round(ms_min, 4), "ms_max": round(ms_max, 4),
             "tokens/s": round(B * L / (ms * 1e-3), 1)}
        if flops:
            tf = flops / (ms * 1e-3) / 1e12
            r.update({"alg_tflops": round(tf, 1), "frac_mfma_f32": round(tf / MFMA_F32_PEAK_TFLOPS, 4)})
        res[name] = r
        print("bench: fp32 layer %s %.3f ms" % (name, ms), file=sys.stderr, flush=True)
    del w
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: libssd times one GPU (the SSD scan over one GPU's share of the batch); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    from mamba_ssd_chunked_03_amd import ssd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            ssd.util_copy(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": args.steps}))
        return
    have_bwd = not args.fwd_only
    w = Workload(2, dev, with_bwd=have_bwd)
    tm = Timer(dev)
    Bsz, L, H, P, N, G = w.Bsz, w.L, w.H, w.P, w.N, w.G
    x, y = w.d["x"], w.y

    def step_recompute():
        w.fwd()
        w.bwd_recompute()

    print("bench: warmup %d, steps %d, bwd %s" % (args.warmup, args.steps, have_bwd), file=sys.stderr, flush=True)
    ms_step, wall_step = tm.timed(w.step, args.steps, args.warmup)
    ms_fwd, _ = tm.timed(w.fwd, args.steps, 2)
    ms_bwd = ms_step_rc = None
    if have_bwd:
        ms_fwd_save, _ = tm.timed(w.fwd_save, args.steps, 2)
        ms_bwd, _ = tm.timed(w.bwd_saved, args.steps, 2)
        ms_step_rc, _ = tm.timed(step_recompute, args.steps, 2)
    tokens = w.tokens
    print("bench: step %.3f ms (wall %.3f), fwd %.3f ms" % (ms_step, wall_step, ms_fwd), file=sys.stderr, flush=True)
    step_med, step_min, step_max = tm.trials(w.step, max(1, args.steps // 2))
    step_cold = tm.cold(w.step, wait=True)
    print("bench: step over 7 trials: median %.3f ms (min %.3f, max %.3f); cold %.3f ms"
          % (step_med, step_min, step_max, step_cold), file=sys.stderr, flush=True)

    # every kernel of the step on its own: the same launch (arguments, grid,
    # buffers) as inside the step, re-issued through the single-kernel flags
    kernels = {}
    roof = scan_ab = chain_ab = split_ab = None
    if not args.no_kernels:
        kernels = kernel_table(w, tm, max(1, args.steps // 2))
        names = [n for n in kernels if not n.startswith("_")]
        dom = max(names, key=lambda k: kernels[k]["ms"])
        s = kernels[dom]
        roof = {"kernel": dom, "bound": "hbm", "achieved": s["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": s["frac_hbm"], "traffic": load_traffic(dom),
                "alg_bytes_per_launch": s["alg_bytes"], "avg_launch_ms": s["ms"]}
        if not args.no_ab:
            scan_ab = w.scan_ab(tm, max(1, args.steps // 2))
            chain_ab = w.chained_ab(tm, max(1, args.steps // 2))
            split_ab = w.fused_bwd_ab(tm, max(1, args.steps // 2))

    # the layer's gated RMSNorm on the SSD output (rows = batch x seqlen, dim =
    # heads x headdim, 8 groups of dim / 8 columns), gate and upstream gradient seeded
    norm = None
    if not args.no_kernels:
        rows, dim = Bsz * L, H * P
        group = dim // G
        gen = torch.Generator(device=dev).manual_seed(7)
        yn = y.view(rows, dim)
        zn = torch.randn(rows, dim, generator=gen, device=dev).to(torch.bfloat16)
        wn = torch.rand(dim, generator=gen, device=dev) + 0.5
        dn = torch.randn(rows, dim, generator=gen, device=dev).to(torch.bfloat16)
        rstd = torch.empty(rows, dim // group, device=dev)
        nfwd, _ = ssd.gated_rmsnorm_fwd(yn, zn, wn, group, 1e-5, rstd=rstd, prepare=True)
        nbwd, _ = ssd.gated_rmsnorm_bwd(dn, yn, zn, wn, group, 1e-5, prepare=True)
        mat = rows * dim * 2
        nb = {"fwd": 3 * mat + dim * 4 + rows * (dim // group) * 4,   # y, z, w -> out, rstd
              "bwd": 5 * mat + 2 * dim * 4}                            # dout, y, z, w -> dy, dz, dw
        norm = {"workload": "gated RMSNorm of the SSD output: %d rows x %d columns, groups of %d, "
                            "bf16" % (rows, dim, group)}
        for name, fn in (("fwd", nfwd), ("bwd", nbwd)):
            ms, ms_min, ms_max = tm.trials(fn, max(1, args.steps // 2))
            ms_cold = tm.cold(fn)
            gbs = nb[name] / (ms * 1e-3) / 1e9
            norm[name] = {"ms": round(ms, 4), "ms_min": round(ms_min, 4), "ms_max": round(ms_max, 4),
                          "ms_cold": round(ms_cold, 4), "alg_bytes": nb[name], "GB/s": round(gbs, 1),
                          "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                          "frac_hbm_cold": round(nb[name] / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            print("bench: gated_rmsnorm %s %.4f ms (cold %.4f)  %.0f GB/s" % (name, ms, ms_cold, gbs),
                  file=sys.stderr, flush=True)
        norm["page_context"] = ("the pages' _layer_norm_bwd: 0.09 ms on one B200, bf16, batch 2, "
                                "seqlen 8192 (layer dimensions not printed); another machine's number")

    # the other full-size workloads, reported beside the headline (not the headline)
    others = None
    if not args.no_others:
        sha = w.sha256
        del w
        torch.cuda.empty_cache()
        others = {"long_context": other_workload(3, dev, tm, args.steps, "long context", not args.no_ab),
                  "packed": other_workload(4, dev, tm, args.steps, "packed sequences", not args.no_ab),
                  "fp32_layer": fp32_layer(dev, tm, args.steps)}
    else:
        sha = w.sha256

    cpu = cpu_par = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(have_bwd)
        try:
            cpu_par = cpu_baseline_parallel(have_bwd)
        except Exception as e:  # a host that cannot start worker processes
            cpu_par = {"error": repr(e)}

    out = {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the pages' layer workload)",
        "config": {"workload": "SSD layer %s, batch 2, seqlen 8192, 64 heads, headdim 64, "
                               "dstate 128, 8 groups, chunk 256" % ("fwd+bwd" if have_bwd else "fwd"),
                   "global_batch": Bsz, "seq_len": L, "parallelism": "single GPU"},
        "input_sha256": sha,
        "fwd": {"ms": round(ms_fwd, 4), "tokens/s": round(tokens / (ms_fwd * 1e-3), 1)},
        "fwd_bwd": None if not have_bwd else {
            "ms": round(ms_step, 4), "fwd_save_ms": round(ms_fwd_save, 4), "bwd_ms": round(ms_bwd, 4),
            "tokens/s": round(tokens / (ms_step * 1e-3), 1),
            "note": "forward keeps its intermediates for the backward (SSD_FLAG_SAVE_FOR_BWD)",
            "recompute_variant_ms": round(ms_step_rc, 4)},
        "step_trials": {"median_ms": round(step_med, 4), "min_ms": round(step_min, 4),
                        "max_ms": round(step_max, 4), "cold_ms": round(step_cold, 4),
                        "note": "7 windows of steps/2 back-to-back steps; cold = single steps "
                                "after a 512 MiB read that evicts the last-level cache (the host "
                                "waits for the read, then issues the step)"},
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_baseline_parallel": cpu_par,
        "gated_rmsnorm": norm,
        "state_passing_ab": scan_ab,
        "fused_chained_forward": chain_ab,
        "bwd_dbdc_ab": split_ab,
        "other_workloads": others,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
