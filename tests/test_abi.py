"""CPU tests of the C ABI: exports match include/ssd.h, host validation returns
the documented status before anything is queued, workspace arithmetic.
No call here reaches a kernel: every argument set is rejected by validation.
"""
import ctypes
import os
import re

import pytest

from mamba_ssd_chunked_03_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, VARLEN, HIP = range(8)
FAKE = 0x10000  # 16-byte-aligned stand-in address; validation never dereferences it


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ssd.LIB_PATH):
        pytest.skip("libssd.so not built")
    return ssd.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree(L):
    names = declared_functions()
    assert "ssd_fwd" in names and "ssd_bwd" in names
    assert set(names) == set(ssd.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_strings(L):
    assert L.ssd_abi_version() == ssd.ABI_VERSION
    hdr = open(os.path.join(ROOT, "include", "ssd.h")).read()
    assert "#define SSD_ABI_VERSION %d" % ssd.ABI_VERSION in hdr
    for s in range(8):
        assert len(L.ssd_status_string(s)) > 0
    assert L.ssd_status_string(99) == b"unknown status"


def prob(**kw):
    d = dict(batch=2, seqlen=1000, nheads=8, headdim=64, dstate=128, ngroups=2, nseq=0,
             io_dtype=1, dt_softplus=1, flags=0)
    d.update(kw)
    return ssd.Problem(*[d[n] for n, _ in ssd.Problem._fields_])


def fwd_status(L, p, Q=256, x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, out=FAKE, ws=FAKE,
               ws_bytes=None, cu=None, init=None):
    pp = None if p is None else ctypes.byref(p)
    if ws_bytes is None:
        ws_bytes = L.ssd_fwd_workspace_bytes(pp, Q, int(cu is not None)) if p is not None else 0
    return L.ssd_fwd(pp, x, dt, None, A, B, C, None, init, cu, Q, out, None, ws, ws_bytes, None)


def test_null_problem(L):
    assert fwd_status(L, None) == NULL


def test_bwd_validation(L):
    # ssd_bwd through the binding's argtypes (counts must match the header)
    p = prob()
    pp = ctypes.byref(p)
    need = L.ssd_bwd_workspace_bytes(pp, 256, 0)
    args = [FAKE] * 9
    args[2] = None                      # dt_bias
    args[6] = None                      # D
    args[7] = None                      # init
    args[8] = None                      # cu_seqlens
    grads = [FAKE] * 10                 # dout, d_final, dx, ddt, dA, dB, dC, dD, d_dt_bias, d_init
    grads[1] = None
    grads[7] = None
    assert L.ssd_bwd(None, *args, 256, *grads, FAKE, need, None) == NULL
    assert L.ssd_bwd(pp, *args, 96, *grads, FAKE, need, None) == UNSUP
    g2 = list(grads); g2[0] = None      # dout missing
    assert L.ssd_bwd(pp, *args, 256, *g2, FAKE, need, None) == NULL
    g3 = list(grads); g3[4] = FAKE + 4  # dA misaligned
    assert L.ssd_bwd(pp, *args, 256, *g3, FAKE, need, None) == ALIGN
    assert L.ssd_bwd(pp, *args, 256, *grads, FAKE, need - 1, None) == WS


@pytest.mark.parametrize("kw,code", [
    (dict(ngroups=3), SHAPE), (dict(nheads=0), SHAPE), (dict(batch=-1), SHAPE),
    (dict(seqlen=-5), SHAPE), (dict(dt_softplus=2), SHAPE),
    (dict(headdim=48), UNSUP), (dict(dstate=256), UNSUP), (dict(io_dtype=5), UNSUP),
    # bf16 with headdim or dstate 16 runs on the fp32 matrix-core kernels
    (dict(headdim=16), OK), (dict(dstate=16), OK), (dict(headdim=16, dstate=16), OK),
    (dict(headdim=16, dstate=16, io_dtype=0), OK),
    # one chunk's token rows must span less than 2^31 bytes (32-bit offsets)
    (dict(nheads=16384, ngroups=8, headdim=128), UNSUP),
    (dict(nheads=8192, ngroups=8, headdim=128), OK),
    (dict(nheads=16384, ngroups=16384, headdim=32, dstate=128), UNSUP),
])
def test_shape_validation(L, kw, code):
    p = prob(**kw)
    st = fwd_status(L, p)
    if code == OK:
        # valid problem: prove validation passed by making only the workspace wrong
        assert fwd_status(L, p, ws_bytes=1) == WS
    else:
        assert st == code


@pytest.mark.parametrize("Q", [32, 96, 512, 0])
def test_chunk_size_unsupported(L, Q):
    assert fwd_status(L, prob(), Q=Q) == UNSUP


def test_null_pointers(L):
    p = prob()
    for field in ("x", "dt", "A", "B", "C", "out"):
        assert fwd_status(L, p, **{field: None}) == NULL, field
    # no tokens: data pointers may be NULL; then the workspace is what is checked
    p0 = prob(seqlen=0)
    assert L.ssd_fwd_workspace_bytes(ctypes.byref(p0), 256, 0) == 0


def test_alignment(L):
    p = prob()
    assert fwd_status(L, p, x=FAKE + 4) == ALIGN
    assert fwd_status(L, p, out=FAKE + 8) == ALIGN
    assert fwd_status(L, p, init=FAKE + 2) == ALIGN


def test_workspace(L):
    p = prob()
    need = L.ssd_fwd_workspace_bytes(ctypes.byref(p), 256, 0)
    assert fwd_status(L, p, ws_bytes=need - 1) == WS
    assert fwd_status(L, p, ws=None) == WS
    assert L.ssd_bwd_workspace_bytes(ctypes.byref(p), 256, 0) > need


def test_flags(L):
    assert fwd_status(L, prob(flags=64)) == UNSUP  # an unknown bit
    assert fwd_status(L, prob(flags=ssd.FLAG_BWD_FUSED), ws_bytes=1) == WS  # accepted
    assert fwd_status(L, prob(flags=ssd.FLAG_CHAINED_FWD), ws_bytes=1) == WS  # accepted
    assert fwd_status(L, prob(flags=ssd.FLAG_CHAINED_FWD | ssd.FLAG_FWD_KERNEL(1))) == UNSUP
    assert fwd_status(L, prob(flags=ssd.FLAG_CHAINED_FWD, io_dtype=0)) == UNSUP      # fp32 io
    assert fwd_status(L, prob(flags=ssd.FLAG_CHAINED_FWD, dstate=32)) == UNSUP       # dstate 32
    assert fwd_status(L, prob(flags=ssd.FLAG_SEQUENTIAL_SCAN), ws_bytes=1) == WS  # accepted
    assert fwd_status(L, prob(flags=ssd.FLAG_SCAN_VARIANT(7)), ws_bytes=1) == WS  # accepted
    assert fwd_status(L, prob(flags=ssd.FLAG_SCAN_VARIANT(8))) == UNSUP
    assert fwd_status(L, prob(flags=ssd.FLAG_SCAN_VARIANT(15))) == UNSUP
    assert fwd_status(L, prob(flags=ssd.FLAG_SEQUENTIAL_SCAN | ssd.FLAG_SCAN_VARIANT(2))) == UNSUP
    assert fwd_status(L, prob(flags=ssd.FLAG_ONE_STREAM), ws_bytes=1) == WS  # accepted
    assert fwd_status(L, prob(flags=ssd.FLAG_BWD_KERNEL(3))) == UNSUP  # needs FROM_SAVED
    assert fwd_status(L, prob(flags=ssd.FLAG_BWD_KERNEL(8))) == UNSUP
    p = prob(flags=ssd.FLAG_FROM_SAVED | ssd.FLAG_BWD_KERNEL(7))
    assert fwd_status(L, p, ws_bytes=1) == WS  # accepted: only the workspace is wrong
    assert fwd_status(L, prob(flags=ssd.FLAG_FWD_KERNEL(5))) == UNSUP
    assert fwd_status(L, prob(flags=ssd.FLAG_FWD_KERNEL(4)), ws_bytes=1) == WS
    p = prob(flags=1)  # keeping the forward's intermediates needs the backward-sized workspace
    fwd_need = L.ssd_fwd_workspace_bytes(ctypes.byref(p), 256, 0)
    assert fwd_status(L, p, ws_bytes=fwd_need) == WS


def test_packed_requires_batch_one(L):
    p = prob(batch=2, nseq=3)
    assert fwd_status(L, p, cu=FAKE) == SHAPE


def test_num_chunks(L):
    p = prob(batch=2, seqlen=1000)
    assert L.ssd_num_chunks(ctypes.byref(p), 256, 0) == 2 * 4
    q = prob(batch=1, seqlen=65536, nseq=8)
    assert L.ssd_num_chunks(ctypes.byref(q), 256, 1) == (65536 + 8 * 255) // 256
    assert L.ssd_num_chunks(ctypes.byref(prob(nheads=7)), 256, 0) == -1


def test_workspace_bytes_layout(L):
    # forward workspace = delta, acs (nck,H,Q) + decay (nck,H) + chunk states
    # (nck,H,P,N) fp32 + passed states (nck,H,P,N) in the io dtype + CB (nck,G,Q,Q)
    # io dtype + the chained forward's 16 + nck*H int32 words, each rounded up to
    # 256 bytes
    up = lambda n: (n + 255) // 256 * 256
    nck = 64
    for io, es in ((1, 2), (0, 4)):
        p = prob(batch=2, seqlen=8192, nheads=64, headdim=64, dstate=128, ngroups=8, io_dtype=io)
        exp = (2 * up(nck * 64 * 256 * 4) + up(nck * 64 * 4) + up(nck * 64 * 64 * 128 * 4)
               + up(nck * 64 * 64 * 128 * es) + up(nck * 8 * 256 * 256 * es) + up((16 + nck * 64) * 4))
        assert L.ssd_fwd_workspace_bytes(ctypes.byref(p), 256, 0) == exp, io


def test_stage_validation(L):
    p = prob()
    pp = ctypes.byref(p)
    assert L.ssd_stage_chunk_cumsum(pp, None, None, FAKE, None, 256, FAKE, FAKE, FAKE, None, 0, None) == NULL
    assert L.ssd_stage_state_passing(pp, FAKE, FAKE, None, None, 100, FAKE, None, None, 0, None) == UNSUP
    assert L.ssd_stage_bmm_chunk(pp, FAKE + 4, FAKE, None, 256, FAKE, None, 0, None) == ALIGN
    assert L.ssd_util_copy(FAKE, FAKE, 17, None) == ALIGN
    assert L.ssd_util_copy(None, FAKE, 16, None) == NULL


def nprob(**kw):
    d = dict(rows=100, dim=4096, group=512, io_dtype=1, eps=1e-5)
    d.update(kw)
    return ssd.NormProblem(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(), OK), (dict(group=4096), OK), (dict(group=256, dim=512), OK), (dict(dim=8192, group=2048), OK),
    (dict(rows=-1), SHAPE), (dict(dim=0), SHAPE), (dict(group=0), SHAPE),
    (dict(io_dtype=0), UNSUP), (dict(dim=4000), UNSUP), (dict(dim=8704), UNSUP),
    (dict(group=128), UNSUP), (dict(group=768), UNSUP), (dict(dim=1536, group=1024), UNSUP),
    (dict(eps=-1.0), UNSUP), (dict(eps=float("inf")), UNSUP), (dict(eps=float("nan")), UNSUP),
])
def test_norm_validation(L, kw, code):
    p = nprob(**kw)
    # a misaligned output is only reported once the problem has passed validation,
    # and nothing is launched either way
    st = L.ssd_gated_rmsnorm_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE + 8, None, None)
    need = L.ssd_gated_rmsnorm_bwd_workspace_bytes(ctypes.byref(p))
    if code == OK:
        assert st == ALIGN
        # and the backward's: make only its workspace wrong
        assert need == min(p.rows, 1024) * p.dim * 4
        assert L.ssd_gated_rmsnorm_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, need - 1, None) == WS
    else:
        assert st == code and need == 0


def test_norm_pointers(L):
    p = nprob()
    assert L.ssd_gated_rmsnorm_fwd(ctypes.byref(p), None, None, FAKE, FAKE, None, None) == NULL
    assert L.ssd_gated_rmsnorm_fwd(ctypes.byref(p), FAKE, None, FAKE, FAKE + 8, None, None) == ALIGN
    need = L.ssd_gated_rmsnorm_bwd_workspace_bytes(ctypes.byref(p))
    # dz must be given exactly when z is
    assert L.ssd_gated_rmsnorm_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                   FAKE, need, None) == NULL
    assert L.ssd_gated_rmsnorm_bwd(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, need, None) == NULL
    assert L.ssd_gated_rmsnorm_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                   FAKE, need, None) == NULL
    # no rows: nothing to do, no data pointers needed
    p0 = nprob(rows=0)
    assert L.ssd_gated_rmsnorm_fwd(ctypes.byref(p0), None, None, FAKE, None, None, None) == OK


def test_fwd_kernel_mask(L):
    # the chunk-state kernel forms C.B^T where each head pair of a group owns one
    # 64-row block of the chunk: bf16, chunk 256, eight heads per group
    layer = dict(batch=2, seqlen=8192, nheads=64, headdim=64, dstate=128, ngroups=8, io_dtype=1)
    mask = lambda Q=256, packed=0, **kw: L.ssd_fwd_kernel_mask(ctypes.byref(prob(**{**layer, **kw})), Q, packed)
    assert mask() == 0xB
    assert mask(nheads=32, ngroups=4, seqlen=131072, batch=1) == 0xB   # long-context shape
    assert mask(batch=1, seqlen=65536, nseq=8, packed=1) == 0xB         # packed sequences
    assert mask(dstate=64) == 0xB
    assert mask(Q=128) == 0xF and mask(Q=64) == 0xF                    # fewer row blocks than pairs
    assert mask(ngroups=16) == 0xF and mask(ngroups=4) == 0xF          # 4 or 16 heads per group
    assert mask(io_dtype=0) == 0xF                                      # fp32 path
    assert mask(headdim=128) == 0xF                                     # one head per workgroup
    assert mask(nheads=-1) == 0                                         # invalid problem


def test_noalloc_host_validation(L):
    """ssd_fwd_noalloc rejects, before any HIP call, what the host can detect: flags
    other than SSD_FLAG_ONE_STREAM, NULL or misaligned pointers, and a forward
    workspace larger than its fixed device array."""
    def st(p, Q=256, x=FAKE, out=FAKE):
        return L.ssd_fwd_noalloc(ctypes.byref(p), x, FAKE, None, FAKE, FAKE, FAKE, None, None, None, Q,
                                 out, None, None)
    big = prob(batch=2, seqlen=8192, nheads=64)
    assert L.ssd_fwd_workspace_bytes(ctypes.byref(big), 256, 0) > ssd.NOALLOC_SCRATCH_BYTES
    assert st(big) == WS
    assert st(prob(flags=ssd.FLAG_SAVE_FOR_BWD)) == UNSUP
    assert st(prob(flags=ssd.FLAG_FWD_KERNEL(2))) == UNSUP
    assert st(prob(), x=None) == NULL
    assert st(prob(), out=FAKE + 8) == ALIGN
    assert st(prob(), Q=100) == UNSUP
    hdr = open(HEADER).read()
    assert "#define SSD_NOALLOC_SCRATCH_BYTES (%du << 20)" % (ssd.NOALLOC_SCRATCH_BYTES >> 20) in hdr


def test_bwd_kernel_mask(L):
    # with SSD_FLAG_BWD_FUSED one kernel forms dB and dC on the bf16 path
    # (kernels 5 and 6 launch nothing)
    layer = dict(batch=2, seqlen=8192, nheads=64, headdim=64, dstate=128, ngroups=8, io_dtype=1)
    mask = lambda Q=256, packed=0, **kw: L.ssd_bwd_kernel_mask(ctypes.byref(prob(**{**layer, **kw})), Q, packed)
    F = ssd.FLAG_BWD_FUSED
    assert mask() == 0x7F                                               # the three-kernel default
    assert mask(flags=F) == 0x4F
    assert mask(flags=F, Q=64) == 0x4F and mask(flags=F, headdim=128, dstate=32) == 0x4F
    assert mask(flags=F, batch=1, seqlen=65536, nseq=8, packed=1) == 0x4F
    assert mask(flags=F, io_dtype=0, headdim=16, dstate=16) == 0x7F     # fp32 path
    assert mask(nheads=-1) == 0                                         # invalid problem
