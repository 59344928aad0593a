"""ctypes binding over libssd.so (argument marshalling only).

Every step of the scan runs in the library's HIP kernels; this module checks
tensor placement and layout, allocates outputs and the workspace with torch
(device memory only), passes raw device pointers and torch's current HIP
stream, and turns a non-zero status into an exception.  There is no fallback:
if the library is missing, or a tensor is not on a GPU, it raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd.so")

F32, BF16 = 0, 1
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "nseq",
                 "io_dtype", "dt_softplus", "flags")]

class NormProblem(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("dim", ctypes.c_int32), ("group", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("eps", ctypes.c_float)]


FLAG_SAVE_FOR_BWD, FLAG_FROM_SAVED, FLAG_ONE_STREAM, FLAG_SEQUENTIAL_SCAN, FLAG_CHAINED_FWD = \
    1, 2, 4, 8, 16
FLAG_BWD_FUSED = 32
BWD_KERNELS = ("dstates", "reverse_state_passing", "bwd_dx", "bwd_dcb", "bwd_dc", "bwd_db",
               "bwd_finalize")
# kernel 4 where ssd_bwd_kernel_mask leaves bits 4 and 5 clear (one kernel for dB and dC)
BWD_FUSED_KERNEL = "bwd_dbc"


# "chunk_state" forms delta and the within-chunk cumsum too (one kernel on the bf16 path)
FWD_KERNELS = ("chunk_state", "state_passing", "bmm_chunk", "chunk_scan")


def FLAG_BWD_KERNEL(k):
    """ssd_bwd launches only its k-th kernel (1-based, order of BWD_KERNELS)."""
    return int(k) << 8


def FLAG_SCAN_VARIANT(v):
    """State-passing kernel: 0 the tuned table's choice, 1..4 associative scan
    (4x2, 8x4, 16x4, 16x8 waves x chunks), 5..7 sequential carry with 1, 4, 8
    chunks of loads in flight."""
    return int(v) << 16


def FLAG_CS_VARIANT(v):
    """Chunk-state kernels: 0 the tuned table's choice, 1 one head per workgroup,
    2 two heads per workgroup, 3 two heads with C.B^T formed inside."""
    return int(v) << 20


def FLAG_FWD_KERNEL(k):
    """ssd_fwd launches only its k-th kernel (1-based, order of FWD_KERNELS)."""
    return int(k) << 12


_SIGS = {
    "ssd_abi_version": ([], _I32),
    "ssd_fwd_kernel_mask": ([_P, _I32, _I32], _I32),
    "ssd_bwd_kernel_mask": ([_P, _I32, _I32], _I32),
    "ssd_scan_variant": ([_P, _I32, _I32], _I32),
    "ssd_cs_variant": ([_P, _I32, _I32], _I32),
    "ssd_fwd_chained_error_offset": ([_P, _I32, _I32], _I64),
    "ssd_status_string": ([_I32], ctypes.c_char_p),
    "ssd_num_chunks": ([_P, _I32, _I32], _I64),
    "ssd_fwd_workspace_bytes": ([_P, _I32, _I32], _SZ),
    "ssd_bwd_workspace_bytes": ([_P, _I32, _I32], _SZ),
    "ssd_stage_workspace_bytes": ([_P, _I32, _I32], _SZ),
    "ssd_fwd": ([_P] + [_P] * 9 + [_I32, _P, _P, _P, _SZ, _P], _I32),
    "ssd_bwd": ([_P] + [_P] * 9 + [_I32] + [_P] * 11 + [_SZ, _P], _I32),
    "ssd_fwd_noalloc": ([_P] + [_P] * 9 + [_I32, _P, _P, _P], _I32),
    "ssd_stage_chunk_cumsum": ([_P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _SZ, _P], _I32),
    "ssd_stage_chunk_state": ([_P, _P, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P], _I32),
    "ssd_stage_state_passing": ([_P, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P], _I32),
    "ssd_stage_bmm_chunk": ([_P, _P, _P, _P, _I32, _P, _P, _SZ, _P], _I32),
    "ssd_stage_chunk_scan": ([_P] + [_P] * 8 + [_I32, _P, _P, _SZ, _P], _I32),
    "ssd_util_copy": ([_P, _P, _SZ, _P], _I32),
    "ssd_gated_rmsnorm_bwd_workspace_bytes": ([_P], _SZ),
    "ssd_gated_rmsnorm_fwd": ([_P] + [_P] * 5 + [_P], _I32),
    "ssd_gated_rmsnorm_bwd": ([_P] + [_P] * 8 + [_SZ, _P], _I32),
}
EXPORTS = tuple(_SIGS)
# The argument lists above follow this version of include/ssd.h (SSD_ABI_VERSION).
ABI_VERSION = 11

_lib = None


def lib():
    """Load libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssd.so is not built; run __graft_entry__.build() "
                               "(or python mamba_ssd_chunked_03_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        if L.ssd_abi_version() != ABI_VERSION:
            raise RuntimeError("libssd.so has ABI version %d, this binding expects %d; rebuild it"
                               % (L.ssd_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


class SSDError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__("libssd: %s (status %d)" % (lib().ssd_status_string(status).decode(), status))


def _check(status, keep=None):
    # keep: objects the marshalled arguments point into (held by the caller's closure)
    if status != 0:
        raise SSDError(status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libssd needs GPU tensors (got one on %s)" % t.device)
        if not t.is_contiguous():
            raise ValueError("libssd needs contiguous tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _expect(t, name, shape, dtype, required=True):
    """Raise ValueError unless t (None allowed when not required) has exactly this
    shape and dtype.  The library sees only pointers, so a tensor of the wrong size
    or element type would make its kernels read or write past the tensor."""
    if t is None:
        if required:
            raise ValueError("%s is required" % name)
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(int(v) for v in shape),
                                                             tuple(t.shape)))


def _dims(x, B, cu_seqlens):
    """(batch, seqlen, nheads, headdim, ngroups, dstate, nstates, io dtype) of a problem,
    from x and B, after checking their rank and dtype."""
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("x must be a 4-D tensor (batch, seqlen, nheads, headdim)")
    if not isinstance(B, torch.Tensor) or B.dim() != 4:
        raise ValueError("B must be a 4-D tensor (batch, seqlen, ngroups, dstate)")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    _expect(B, "B", (batch, seqlen, ngroups, dstate), x.dtype)
    if cu_seqlens is not None:
        if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D tensor of nseq + 1 offsets")
        if cu_seqlens.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
        if batch != 1:
            raise ValueError("packed sequences (cu_seqlens) must come in one batch row")
        nst = cu_seqlens.numel() - 1
    else:
        nst = batch
    return batch, seqlen, nheads, headdim, ngroups, dstate, nst, x.dtype


def _check_inputs(x, dt, A, B, C, D, dt_bias, init, cu_seqlens):
    """Shapes and dtypes of ssd_fwd's / ssd_bwd's inputs; returns _dims()."""
    dims = _dims(x, B, cu_seqlens)
    batch, seqlen, H, P, G, N, nst, io = dims
    _expect(C, "C", (batch, seqlen, G, N), io)
    _expect(dt, "dt", (batch, seqlen, H), torch.float32)
    _expect(A, "A", (H,), torch.float32)
    _expect(D, "D", (H,), torch.float32, required=False)
    _expect(dt_bias, "dt_bias", (H,), torch.float32, required=False)
    _expect(init, "init", (nst, H, P, N), torch.float32, required=False)
    return dims


def problem(x, B, cu_seqlens=None, dt_softplus=True, flags=0):
    batch, seqlen, nheads, headdim, ngroups, dstate, nst, dtype = _dims(x, B, cu_seqlens)
    io = {torch.float32: F32, torch.bfloat16: BF16}[dtype]
    nseq = 0 if cu_seqlens is None else nst
    return Problem(batch, seqlen, nheads, headdim, dstate, ngroups, nseq, io, int(bool(dt_softplus)),
                   int(flags))


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ws(nbytes, dev):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


def num_chunks(prob, chunk_size, packed):
    return lib().ssd_num_chunks(ctypes.byref(prob), chunk_size, int(packed))


def fwd(x, dt, A, B, C, D=None, dt_bias=None, init=None, cu_seqlens=None, chunk_size=256,
        dt_softplus=True, workspace=None, out=None, final=None, save_for_backward=False,
        only_kernel=0, prepare=False, one_stream=False, sequential_scan=False, scan_variant=0,
        chained=False, cs_variant=0):
    """y, final_states = SSD(x, ...) on the GPU.  Shapes as in include/ssd.h.

    save_for_backward: keep the intermediates in ``workspace`` (which must hold
    bwd_workspace_bytes) so that bwd(..., workspace=that, from_saved=True) skips
    the recompute.
    only_kernel: k >= 1 launches only the k-th forward kernel (profiling; needs the
    workspace, out and final of a complete call on the same inputs).
    prepare: launch nothing; return (launch, out, final) where launch() issues the
    call with the arguments marshalled here (timing loops).
    one_stream: queue every kernel on the current stream (the library then uses no
    stream of its own).
    sequential_scan: the state passing walks the chunks with a sequential carry
    instead of the associative scan (a comparison point).
    scan_variant: force a state-passing kernel (FLAG_SCAN_VARIANT); 0 = tuned table.
    chained: the fused single-pass forward (chained scan across chunks).
    cs_variant: force a chunk-state form (FLAG_CS_VARIANT); 0 = tuned table."""
    if only_kernel and (workspace is None or out is None):
        raise ValueError("only_kernel needs the workspace and outputs of a complete call")
    batch, seqlen, H, P, G, N, nst, io = _check_inputs(x, dt, A, B, C, D, dt_bias, init, cu_seqlens)
    _expect(out, "out", x.shape, io, required=False)
    _expect(final, "final", (nst, H, P, N), torch.float32, required=False)
    _expect(workspace, "workspace", (workspace.numel(),) if workspace is not None else (0,),
            torch.uint8, required=False)
    dev = _dev(x, dt, A, B, C, D, dt_bias, init, cu_seqlens, workspace, out, final)
    prob = problem(x, B, cu_seqlens, dt_softplus,
                   (FLAG_SAVE_FOR_BWD if save_for_backward else 0) | FLAG_FWD_KERNEL(only_kernel) |
                   (FLAG_ONE_STREAM if one_stream else 0) |
                   (FLAG_SEQUENTIAL_SCAN if sequential_scan else 0) | FLAG_SCAN_VARIANT(scan_variant) |
                   (FLAG_CHAINED_FWD if chained else 0) | FLAG_CS_VARIANT(cs_variant))
    L = lib()
    packed = int(cu_seqlens is not None)
    if save_for_backward:
        need = L.ssd_bwd_workspace_bytes(ctypes.byref(prob), chunk_size, packed)
    else:
        need = L.ssd_fwd_workspace_bytes(ctypes.byref(prob), chunk_size, packed)
    if workspace is None:
        workspace = _ws(need, dev)
    if out is None:
        out = torch.empty_like(x)
    if final is None:
        nst = prob.nseq if packed else prob.batch
        final = torch.empty(nst, prob.nheads, prob.headdim, prob.dstate, dtype=torch.float32, device=dev)
    args = (ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(init), _ptr(cu_seqlens), chunk_size, _ptr(out), _ptr(final),
            _ptr(workspace), workspace.numel(), _stream(dev))
    keep = (prob, workspace)

    def launch():
        _check(L.ssd_fwd(*args), keep)

    if prepare:
        return launch, out, final
    launch()
    return out, final


# SSD_NOALLOC_SCRATCH_BYTES of include/ssd.h: the largest forward workspace fwd_noalloc takes
NOALLOC_SCRATCH_BYTES = 64 << 20


def fwd_noalloc(x, dt, A, B, C, D=None, dt_bias=None, init=None, cu_seqlens=None, chunk_size=256,
                dt_softplus=True, out=None, final=None):
    """fwd() through ssd_fwd_noalloc: no workspace, the library's fixed device array
    instead (problems whose forward workspace exceeds NOALLOC_SCRATCH_BYTES raise).
    Pass out and final to allocate nothing here either."""
    batch, seqlen, H, P, G, N, nst, io = _check_inputs(x, dt, A, B, C, D, dt_bias, init, cu_seqlens)
    _expect(out, "out", x.shape, io, required=False)
    _expect(final, "final", (nst, H, P, N), torch.float32, required=False)
    dev = _dev(x, dt, A, B, C, D, dt_bias, init, cu_seqlens, out, final)
    prob = problem(x, B, cu_seqlens, dt_softplus)
    if out is None:
        out = torch.empty_like(x)
    if final is None:
        final = torch.empty(nst, H, P, N, dtype=torch.float32, device=dev)
    _check(lib().ssd_fwd_noalloc(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B),
                                 _ptr(C), _ptr(D), _ptr(init), _ptr(cu_seqlens), chunk_size, _ptr(out),
                                 _ptr(final), _stream(dev)))
    return out, final


def bwd(x, dt, A, B, C, dout, D=None, dt_bias=None, init=None, d_final=None, cu_seqlens=None,
        chunk_size=256, dt_softplus=True, workspace=None, from_saved=False, grads=None,
        only_kernel=0, prepare=False, one_stream=False, sequential_scan=False, scan_variant=0,
        fused=False, cs_variant=0):
    """Gradients of <dout, y> + <d_final, final> (dict of GPU tensors).

    fused: dB and dC from one kernel, one pass over x and dy (SSD_FLAG_BWD_FUSED),
    instead of the three-kernel form.
    cs_variant: force a chunk-state form (FLAG_CS_VARIANT) for the recompute and
    the adjoint chunk states; 0 = tuned table.
    from_saved: ``workspace`` holds the intermediates of a save_for_backward
    fwd call on the same inputs; the recompute is skipped.
    grads: a dict returned by an earlier call, written again instead of new tensors.
    only_kernel: k >= 1 launches only the k-th backward kernel (profiling; needs
    from_saved and the workspace and grads of a complete call on the same inputs).
    prepare: launch nothing; return (launch, grads) (see fwd)."""
    batch, seqlen, H, P, G, N, nst, io = _check_inputs(x, dt, A, B, C, D, dt_bias, init, cu_seqlens)
    _expect(dout, "dout", x.shape, io)
    _expect(d_final, "d_final", (nst, H, P, N), torch.float32, required=False)
    _expect(workspace, "workspace", (workspace.numel(),) if workspace is not None else (0,),
            torch.uint8, required=False)
    if grads is not None:
        want = {"dx": (x.shape, io), "ddt": (dt.shape, torch.float32), "dA": ((H,), torch.float32),
                "dB": (B.shape, io), "dC": (C.shape, io), "dD": ((H,), torch.float32),
                "d_dt_bias": ((H,), torch.float32), "d_init": ((nst, H, P, N), torch.float32)}
        for k, (shape, dtype) in want.items():
            _expect(grads.get(k), "grads['%s']" % k, shape, dtype,
                    required=k not in ("dD", "d_dt_bias", "d_init"))
        if (D is None) != (grads.get("dD") is None):
            raise ValueError("grads['dD'] must be given exactly when D is")
    dev = _dev(x, dt, A, B, C, dout, D, dt_bias, init, d_final, cu_seqlens, workspace,
               *([] if grads is None else [v for v in grads.values() if v is not None]))
    if from_saved and workspace is None:
        raise ValueError("from_saved needs the forward's workspace")
    if only_kernel and (not from_saved or grads is None):
        raise ValueError("only_kernel needs from_saved and the grads of a complete call")
    flags = (FLAG_FROM_SAVED if from_saved else 0) | FLAG_BWD_KERNEL(only_kernel) | \
        (FLAG_ONE_STREAM if one_stream else 0) | (FLAG_SEQUENTIAL_SCAN if sequential_scan else 0) | \
        FLAG_SCAN_VARIANT(scan_variant) | (FLAG_BWD_FUSED if fused else 0) | FLAG_CS_VARIANT(cs_variant)
    prob = problem(x, B, cu_seqlens, dt_softplus, flags)
    L = lib()
    packed = int(cu_seqlens is not None)
    need = L.ssd_bwd_workspace_bytes(ctypes.byref(prob), chunk_size, packed)
    if workspace is None:
        workspace = _ws(need, dev)
    nst = prob.nseq if packed else prob.batch
    g = grads if grads is not None else {
        "dx": torch.empty_like(x), "ddt": torch.empty_like(dt), "dA": torch.empty_like(A),
        "dB": torch.empty_like(B), "dC": torch.empty_like(C),
        "dD": None if D is None else torch.empty_like(D),
        "d_dt_bias": torch.empty(prob.nheads, dtype=torch.float32, device=dev),
        "d_init": torch.empty(nst, prob.nheads, prob.headdim, prob.dstate, dtype=torch.float32, device=dev),
    }
    args = (ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(init), _ptr(cu_seqlens), chunk_size, _ptr(dout), _ptr(d_final),
            _ptr(g["dx"]), _ptr(g["ddt"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
            _ptr(g["dD"]), _ptr(g["d_dt_bias"]), _ptr(g["d_init"]),
            _ptr(workspace), workspace.numel(), _stream(dev))
    keep = (prob, workspace)

    def launch():
        _check(L.ssd_bwd(*args), keep)

    if prepare:
        return launch, g
    launch()
    return g


# ------------------------------------------------------------ single stages ----
class Stages:
    """Run one forward stage at a time on explicit buffers (tests, timing)."""

    def __init__(self, x, B, cu_seqlens=None, chunk_size=256, dt_softplus=True):
        self.dims = _dims(x, B, cu_seqlens)
        self.dev = _dev(x, B, cu_seqlens)
        self.prob = problem(x, B, cu_seqlens, dt_softplus)
        self.Q = chunk_size
        self.cu = cu_seqlens
        self.packed = int(cu_seqlens is not None)
        self.nck = num_chunks(self.prob, chunk_size, self.packed)
        if self.nck < 0:
            raise SSDError(3)
        self.ws = _ws(lib().ssd_stage_workspace_bytes(ctypes.byref(self.prob), chunk_size, self.packed), self.dev)
        self.io_dtype = x.dtype

    def _f(self, *shape):
        return torch.empty(*shape, dtype=torch.float32, device=self.dev)

    def _call(self, name, *args):
        _check(getattr(lib(), name)(ctypes.byref(self.prob), *args))

    def _need(self, *checks):
        """Check (tensor, name, shape, dtype, required) tuples, then placement."""
        for t, name, shape, dtype, req in checks:
            _expect(t, name, shape, dtype, required=req)
        ts = [c[0] for c in checks if c[0] is not None]
        if _dev(*ts) not in (None, self.dev):
            raise ValueError("all tensors must be on one device")

    def _shapes(self):
        batch, seqlen, H, P, G, N, nst, io = self.dims
        f = torch.float32
        return dict(x=((batch, seqlen, H, P), io), B=((batch, seqlen, G, N), io),
                    dt=((batch, seqlen, H), f), head=((H,), f), tok=((self.nck, H, self.Q), f),
                    decay=((self.nck, H), f), state=((self.nck, H, P, N), f),
                    init=((nst, H, P, N), f), CB=((self.nck, G, self.Q, self.Q), io))

    def chunk_cumsum(self, dt, A, dt_bias=None, out=None):
        p = self.prob
        s = self._shapes()
        delta, acs, decay = out or (self._f(self.nck, p.nheads, self.Q), self._f(self.nck, p.nheads, self.Q),
                                    self._f(self.nck, p.nheads))
        self._need((dt, "dt", *s["dt"], True), (A, "A", *s["head"], True),
                   (dt_bias, "dt_bias", *s["head"], False), (delta, "delta", *s["tok"], True),
                   (acs, "acs", *s["tok"], True), (decay, "chunk_decay", *s["decay"], True))
        self._call("ssd_stage_chunk_cumsum", _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(self.cu), self.Q,
                   _ptr(delta), _ptr(acs), _ptr(decay), _ptr(self.ws), self.ws.numel(), _stream(self.dev))
        return delta, acs, decay

    def chunk_state(self, x, B, delta, acs, out=None):
        p = self.prob
        T = out if out is not None else self._f(self.nck, p.nheads, p.headdim, p.dstate)
        s = self._shapes()
        self._need((x, "x", *s["x"], True), (B, "B", *s["B"], True), (delta, "delta", *s["tok"], True),
                   (acs, "acs", *s["tok"], True), (T, "states", *s["state"], True))
        self._call("ssd_stage_chunk_state", _ptr(x), _ptr(B), _ptr(delta), _ptr(acs), _ptr(self.cu),
                   self.Q, _ptr(T), _ptr(self.ws), self.ws.numel(), _stream(self.dev))
        return T

    def state_passing(self, T, decay, init=None, out=None, sequential=False, variant=0):
        """sequential: the sequential-carry kernel instead of the associative scan;
        variant: force a state-passing kernel (FLAG_SCAN_VARIANT), 0 = tuned table"""
        p = self.prob
        nst = p.nseq if self.packed else p.batch
        Hp, final = out or (self._f(self.nck, p.nheads, p.headdim, p.dstate),
                            self._f(nst, p.nheads, p.headdim, p.dstate))
        s = self._shapes()
        self._need((T, "states", *s["state"], True), (decay, "chunk_decay", *s["decay"], True),
                   (init, "init", *s["init"], False), (Hp, "passed", *s["state"], True),
                   (final, "final", *s["init"], False))
        prob = self.prob
        if sequential or variant:
            prob = Problem(*[getattr(p, n) for n, _ in Problem._fields_])
            prob.flags = p.flags | (FLAG_SEQUENTIAL_SCAN if sequential else 0) | FLAG_SCAN_VARIANT(variant)
        _check(lib().ssd_stage_state_passing(ctypes.byref(prob), _ptr(T), _ptr(decay), _ptr(init),
                                             _ptr(self.cu), self.Q, _ptr(Hp), _ptr(final), _ptr(self.ws),
                                             self.ws.numel(), _stream(self.dev)))
        return Hp, final

    def bmm_chunk(self, B, C, out=None):
        p = self.prob
        CB = out if out is not None else torch.empty(self.nck, p.ngroups, self.Q, self.Q,
                                                     dtype=self.io_dtype, device=self.dev)
        s = self._shapes()
        self._need((B, "B", *s["B"], True), (C, "C", *s["B"], True), (CB, "CB", *s["CB"], True))
        self._call("ssd_stage_bmm_chunk", _ptr(B), _ptr(C), _ptr(self.cu), self.Q, _ptr(CB),
                   _ptr(self.ws), self.ws.numel(), _stream(self.dev))
        return CB

    def chunk_scan(self, x, C, CB, delta, acs, Hp, D=None, out=None):
        y = out if out is not None else torch.empty_like(x)
        s = self._shapes()
        self._need((x, "x", *s["x"], True), (C, "C", *s["B"], True), (CB, "CB", *s["CB"], True),
                   (delta, "delta", *s["tok"], True), (acs, "acs", *s["tok"], True),
                   (Hp, "passed", *s["state"], True), (D, "D", *s["head"], False),
                   (y, "out", *s["x"], True))
        self._call("ssd_stage_chunk_scan", _ptr(x), _ptr(C), _ptr(CB), _ptr(delta), _ptr(acs), _ptr(Hp),
                   _ptr(D), _ptr(self.cu), self.Q, _ptr(y), _ptr(self.ws), self.ws.numel(),
                   _stream(self.dev))
        return y


def util_copy(dst, src):
    dev = _dev(dst, src)
    _check(lib().ssd_util_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(), _stream(dev)))


def norm_problem(y, group, eps):
    """y: (..., dim) bf16; rows = the product of the leading sizes."""
    if not isinstance(y, torch.Tensor) or y.dim() < 1:
        raise ValueError("y must be a tensor of rank >= 1")
    if y.dtype != torch.bfloat16:
        raise ValueError("the gated RMSNorm takes bfloat16 y, z")
    dim = y.shape[-1]
    return NormProblem(y.numel() // dim if dim else 0, dim, int(group), BF16, float(eps))


def gated_rmsnorm_fwd(y, z, weight, group, eps=1e-5, out=None, rstd=None, prepare=False):
    """out = RMSNorm(y * silu(z)) * weight over groups of `group` columns of the
    last dimension (z may be None: no gate).  rstd: optional (rows, dim // group)
    float32 output.  Returns out (or (launch, out) when prepare is set)."""
    p = norm_problem(y, group, eps)
    _expect(z, "z", y.shape, y.dtype, required=False)
    _expect(weight, "weight", (p.dim,), torch.float32)
    _expect(out, "out", y.shape, y.dtype, required=False)
    if rstd is not None:
        if p.group <= 0 or p.dim % p.group:
            raise ValueError("group must divide the last dimension")
        _expect(rstd, "rstd", (p.rows, p.dim // p.group), torch.float32)
    dev = _dev(y, z, weight, out, rstd)
    out = torch.empty_like(y) if out is None else out
    args = (ctypes.byref(p), _ptr(y), _ptr(z), _ptr(weight), _ptr(out), _ptr(rstd), _stream(dev))
    L = lib()

    def launch():
        _check(L.ssd_gated_rmsnorm_fwd(*args), keep=p)

    if prepare:
        return launch, out
    launch()
    return out


def gated_rmsnorm_bwd(dout, y, z, weight, group, eps=1e-5, workspace=None, grads=None, prepare=False):
    """Gradients (dy, dz, dweight) of <dout, gated_rmsnorm_fwd(y, z, weight)>;
    dz is None without a gate.  Returns them (or (launch, grads) with prepare)."""
    p = norm_problem(y, group, eps)
    _expect(dout, "dout", y.shape, y.dtype)
    _expect(z, "z", y.shape, y.dtype, required=False)
    _expect(weight, "weight", (p.dim,), torch.float32)
    if grads is not None:
        _expect(grads[0], "dy", y.shape, y.dtype)
        _expect(grads[1], "dz", y.shape, y.dtype, required=z is not None)
        if z is None and grads[1] is not None:
            raise ValueError("dz must be None without a gate")
        _expect(grads[2], "dweight", (p.dim,), torch.float32)
    _expect(workspace, "workspace", (workspace.numel(),) if workspace is not None else (0,),
            torch.uint8, required=False)
    dev = _dev(dout, y, z, weight, workspace, *([] if grads is None else [g for g in grads if g is not None]))
    if grads is None:
        grads = (torch.empty_like(y), None if z is None else torch.empty_like(z),
                 torch.empty_like(weight))
    dy, dz, dw = grads
    need = lib().ssd_gated_rmsnorm_bwd_workspace_bytes(ctypes.byref(p))
    ws = workspace if workspace is not None else _ws(need, dev)
    args = (ctypes.byref(p), _ptr(dout), _ptr(y), _ptr(z), _ptr(weight), _ptr(dy), _ptr(dz), _ptr(dw),
            _ptr(ws), ws.numel(), _stream(dev))

    L = lib()

    def launch():
        _check(L.ssd_gated_rmsnorm_bwd(*args), keep=(p, ws))

    if prepare:
        return launch, grads
    launch()
    return grads
