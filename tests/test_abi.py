"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, its host-only functions are bit-exact, and every argument check rejects
bad input before touching the device (fake device addresses are never read)."""
import ctypes
import os
import re

import pytest

import oracle
from long_context_exact_ra_amd import ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(ra.lib_path()),
                                reason="libra.so not built (python -m long_context_exact_ra_amd.build)")


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "ra.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ra.load()
    declared = _declared_symbols()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(ra.exported_symbols()) == declared


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 7, 8, 64, 127, 128])
def test_ring_schedule_bit_exact(N):
    for rank in range(N):
        assert ra.ring_schedule(rank, N) == oracle.ring_schedule(rank, N)
        for t in range(N):
            assert ra.ring_block(rank, N, t) == oracle.ring_schedule(rank, N)[t]


def test_ring_block_rejects_bad_arguments():
    for args in [(0, 0, 0), (-1, 4, 0), (4, 4, 0), (0, 4, -1), (0, 4, 4)]:
        assert ra.ring_block(*args) == -ra.RA_EINVAL
    lib = ra.load()
    out = (ctypes.c_int32 * 4)()
    assert lib.ra_ring_schedule(0, 0, out) == ra.RA_EINVAL
    assert lib.ra_ring_schedule(4, 4, out) == ra.RA_EINVAL
    assert lib.ra_ring_schedule(0, 4, None) == ra.RA_EINVAL


def test_kv_head_map():
    assert [ra.kv_head(h, 28, 4) for h in range(28)] == [oracle.kv_head(h, 28, 4) for h in range(28)]
    assert ra.kv_head(0, 6, 4) == -ra.RA_EINVAL
    assert ra.kv_head(6, 6, 3) == -ra.RA_EINVAL


def test_strerror():
    for code in (0, 1, 2, 3):
        assert ra.load().ra_strerror(code)
    assert ra.load().ra_last_hip_error() == 0


# Fake but 16-byte aligned "device" addresses: validation must reject before use.
P = ctypes.c_void_p(0x10000)
P2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)


def _share(**kw):
    args = dict(rank=3, N=8, L=8 * 64, H=4, H_kv=2, d=128, B=1, dtype=ra.RA_BF16, Q=P, K=P,
                V=P, scale=0.088, O=P2, m=None, l=None, cast=None, trace=None, stream=None)
    args.update(kw)
    return ra.load().ra_share_forward(
        args["rank"], args["N"], args["L"], args["H"], args["H_kv"], args["d"], args["B"],
        args["dtype"], args["Q"], args["K"], args["V"], args["scale"], args["O"], args["m"],
        args["l"], args["cast"], args["trace"], args["stream"])


@pytest.mark.parametrize("kw", [
    dict(N=0), dict(rank=-1), dict(rank=8), dict(L=8 * 64 + 1), dict(L=-8),
    dict(H=5), dict(H_kv=0), dict(d=96), dict(d=256), dict(B=0), dict(dtype=7),
    dict(scale=0.0), dict(scale=-1.0), dict(scale=float("nan")), dict(scale=float("inf")),
    dict(Q=None), dict(K=None), dict(V=None), dict(O=None), dict(Q=MIS), dict(O=MIS),
    dict(m=MIS), dict(cast=MIS), dict(trace=ctypes.c_void_p(0x10002)),
])
def test_share_forward_rejects(kw):
    assert _share(**kw) == ra.RA_EINVAL


def test_share_forward_empty_sequence_is_noop():
    assert _share(L=0, Q=None, K=None, V=None, O=None) == ra.RA_OK


def _shape(**kw):
    s = ra.RaShape(B=1, H=4, H_kv=2, d=128, l_q=100, l_kv=64, kv_head_stride=0,
                   kv_batch_stride=0, dtype=ra.RA_BF16)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _step(s, scale=0.1, ptrs=None):
    p = ptrs or [P] * 6
    return ra.load().ra_step(*p, scale, ctypes.byref(s), None)


@pytest.mark.parametrize("kw", [
    dict(B=0), dict(H=3), dict(H_kv=0), dict(d=32), dict(dtype=2), dict(l_q=-1),
    dict(l_kv=-1), dict(kv_head_stride=64 * 128 - 8), dict(kv_head_stride=64 * 128 + 4),
    dict(kv_batch_stride=12), dict(kv_head_stride=-8),
])
def test_step_rejects_bad_shape(kw):
    assert _step(_shape(**kw)) == ra.RA_EINVAL


def test_step_rejects_bad_pointers_and_scale():
    s = _shape()
    assert _step(s, scale=0.0) == ra.RA_EINVAL
    assert _step(s, scale=float("nan")) == ra.RA_EINVAL
    for i in range(6):
        ptrs = [P] * 6
        ptrs[i] = None
        assert _step(s, ptrs=ptrs) == ra.RA_EINVAL
        ptrs[i] = MIS
        assert _step(s, ptrs=ptrs) == ra.RA_EINVAL
    assert ra.load().ra_step(P, P, P, P, P, P, 0.1, None, None) == ra.RA_EINVAL


def test_step_empty_is_noop():
    assert _step(_shape(l_q=0), ptrs=[None] * 6) == ra.RA_OK
    assert _step(_shape(l_kv=0), ptrs=[None] * 6) == ra.RA_OK


def test_finalize_and_init_validation():
    lib = ra.load()
    s = _shape()
    assert lib.ra_finalize(None, P, ctypes.byref(s), None, None) == ra.RA_EINVAL
    assert lib.ra_finalize(P, MIS, ctypes.byref(s), None, None) == ra.RA_EINVAL
    assert lib.ra_finalize(P, P, ctypes.byref(s), MIS, None) == ra.RA_EINVAL
    assert lib.ra_finalize(P, P, None, None, None) == ra.RA_EINVAL
    assert lib.ra_state_init(P, None, P, ctypes.byref(s), None) == ra.RA_EINVAL
    assert lib.ra_state_init(P, P, P, None, None) == ra.RA_EINVAL
    empty = _shape(l_q=0)
    assert lib.ra_finalize(None, None, ctypes.byref(empty), None, None) == ra.RA_OK
    assert lib.ra_state_init(None, None, None, ctypes.byref(empty), None) == ra.RA_OK


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros((1, 2, 4, 64))
    k = torch.zeros((1, 2, 16, 64))
    o = torch.zeros((1, 2, 4, 64))
    with pytest.raises(ValueError):
        ra.share_forward(0, 4, 16, 2, 2, 64, 1, q, k, k, 0.125, o)


def test_binding_refuses_broadcast_kv_blocks():
    """A stride of 0 means 'contiguous default' to the library, so an expanded K/V
    block (one head or batch entry broadcast) must be refused by the binding rather
    than read as separate heads past the tensor's end."""
    import torch
    q = torch.zeros((2, 4, 8, 64), dtype=torch.bfloat16)
    k = torch.zeros((2, 2, 16, 64), dtype=torch.bfloat16)
    heads = k[:, :1].expand(2, 2, 16, 64)
    batch = k[:1].expand(2, 2, 16, 64)
    for blk in (heads, batch):
        with pytest.raises(ValueError):
            ra.make_shape(q, blk)
        with pytest.raises(ValueError):
            ra.step(q, blk, blk, None, None, None, 0.125)
    # a single head (or batch entry) broadcast over nothing is still a valid block
    one = torch.zeros((1, 1, 16, 64), dtype=torch.bfloat16)
    s = ra.make_shape(torch.zeros((1, 4, 8, 64), dtype=torch.bfloat16),
                      one.expand(1, 1, 16, 64))
    assert s.H_kv == 1 and s.l_kv == 16


def test_bf16_heads_beyond_the_32_bit_buffer_range_are_unsupported():
    # One bf16 K/V head of 2^23 rows x 128 dims is 2^31 bytes: past the kernel's
    # 32-bit buffer range, refused before any device call.
    assert _share(N=8, L=1 << 23, d=128) == ra.RA_ENOTSUP
    assert _share(N=8, L=1 << 24, d=64) == ra.RA_ENOTSUP
    assert _step(_shape(l_kv=1 << 23, kv_head_stride=0)) == ra.RA_ENOTSUP


# ------------------------------------------------------------------ causal share

@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
@pytest.mark.parametrize("N,L", [(1, 64), (4, 64), (8, 8 * 256), (64, 64 * 128)])
def test_causal_pairs_match_the_oracle_count(layout, N, L):
    import oracle
    for r in sorted({0, 1 % N, N // 2, N - 1}):
        assert ra.causal_pairs(r, N, L, layout) == oracle.causal_pairs(r, N, L, layout)


def test_causal_pairs_rejects_bad_arguments():
    lib = ra.load()
    for args in [(0, 0, 64, 0), (4, 4, 64, 0), (-1, 4, 64, 0), (0, 4, 65, 0), (0, 4, -4, 0),
                 (0, 4, 64, 3), (0, 4, 64, -1), (0, 2, 6, ra.RA_LAYOUT_ZIGZAG)]:
        assert lib.ra_causal_pairs(*args) == -ra.RA_EINVAL


def _causal(**kw):
    args = dict(rank=3, N=8, L=8 * 128, H=4, H_kv=2, d=128, B=1, dtype=ra.RA_BF16, layout=0,
                Q=P, K=P, V=P, scale=0.088, O=P2, m=None, l=None, cast=None, stream=None)
    args.update(kw)
    return ra.load().ra_causal_share_forward(
        args["rank"], args["N"], args["L"], args["H"], args["H_kv"], args["d"], args["B"],
        args["dtype"], args["layout"], args["Q"], args["K"], args["V"], args["scale"],
        args["O"], args["m"], args["l"], args["cast"], args["stream"])


@pytest.mark.parametrize("kw", [
    dict(layout=3), dict(layout=-1), dict(layout=2, L=8 * 64), dict(layout=2, L=8 * 192),
    dict(N=0), dict(rank=8), dict(L=8 * 128 + 1), dict(H=5), dict(d=96), dict(dtype=9),
    dict(scale=0.0), dict(Q=None), dict(O=MIS), dict(m=MIS), dict(cast=MIS),
])
def test_causal_share_rejects(kw):
    assert _causal(**kw) == ra.RA_EINVAL


def test_causal_share_limits_and_noop():
    assert _causal(L=0, Q=None, K=None, V=None, O=None) == ra.RA_OK
    assert _causal(N=8, L=1 << 23, d=128) == ra.RA_ENOTSUP


# ------------------------------------------------------------------ backward

def _backward(causal=False, **kw):
    args = dict(rank=3, N=8, L=8 * 128, H=4, H_kv=2, d=128, B=1, dtype=ra.RA_BF16, layout=0,
                Q=P, K=P, V=P, O=P2, dO=P, m=P2, l=P2, scale=0.088, dQ=P2, dK=P2, dV=P2,
                ws=P2, stream=None)
    args.update(kw)
    tail = (args["Q"], args["K"], args["V"], args["O"], args["dO"], args["m"], args["l"],
            args["scale"], args["dQ"], args["dK"], args["dV"], args["ws"], args["stream"])
    head = (args["rank"], args["N"], args["L"], args["H"], args["H_kv"], args["d"], args["B"],
            args["dtype"])
    lib = ra.load()
    if causal:
        return lib.ra_causal_share_backward(*head, args["layout"], *tail)
    return lib.ra_share_backward(*head, *tail)


BACKWARD_REJECTS = [
    dict(N=0), dict(rank=-1), dict(rank=8), dict(L=8 * 128 + 1), dict(L=-8), dict(H=5),
    dict(H_kv=0), dict(d=96), dict(B=0), dict(dtype=7), dict(scale=0.0),
    dict(scale=float("nan")), dict(Q=None), dict(K=None), dict(V=None), dict(O=None),
    dict(dO=None), dict(m=None), dict(l=None), dict(dQ=None), dict(dK=None), dict(dV=None),
    dict(ws=None), dict(O=MIS), dict(dQ=MIS), dict(ws=MIS),
]


@pytest.mark.parametrize("kw", BACKWARD_REJECTS)
def test_share_backward_rejects(kw):
    assert _backward(**kw) == ra.RA_EINVAL


@pytest.mark.parametrize("kw", BACKWARD_REJECTS + [
    dict(layout=3), dict(layout=-1), dict(layout=2, L=8 * 64), dict(layout=2, L=8 * 192)])
def test_causal_share_backward_rejects(kw):
    assert _backward(causal=True, **kw) == ra.RA_EINVAL


def test_backward_limits_and_noop():
    for causal in (False, True):
        assert _backward(causal, L=0, Q=None, K=None, V=None, dQ=None) == ra.RA_OK
        # fp32 inputs: the backward kernels take bf16 only
        assert _backward(causal, dtype=ra.RA_F32) == ra.RA_ENOTSUP
        assert _backward(causal, N=8, L=1 << 23, d=128) == ra.RA_ENOTSUP
    lib = ra.load()
    assert lib.ra_share_backward_workspace(2, 3, 100) == 8 * 2 * 3 * 100
    assert lib.ra_share_backward_workspace(-1, 3, 100) == -ra.RA_EINVAL


# ------------------------------------------------------------------ FP8

def test_fp8_tiles():
    lib = ra.load()
    assert [lib.ra_fp8_tiles(s) for s in (0, 1, 63, 64, 65, 16384)] == [0, 1, 1, 1, 2, 256]
    assert lib.ra_fp8_tiles(-1) == -ra.RA_EINVAL


def _quant(**kw):
    args = dict(kind=ra.RA_FP8_ROWS, B=1, Hx=2, n_seg=4, seg=100, d=128, x=P, codes=P2,
                descale=P, stream=None)
    args.update(kw)
    return ra.load().ra_quantize_fp8(args["kind"], args["B"], args["Hx"], args["n_seg"],
                                     args["seg"], args["d"], args["x"], args["codes"],
                                     args["descale"], args["stream"])


@pytest.mark.parametrize("kw", [
    dict(kind=2), dict(kind=-1), dict(B=0), dict(Hx=0), dict(n_seg=0), dict(seg=-1),
    dict(d=96), dict(x=None), dict(codes=None), dict(descale=None), dict(x=MIS),
    dict(codes=MIS), dict(descale=MIS)])
def test_quantize_fp8_rejects(kw):
    assert _quant(**kw) == ra.RA_EINVAL


def test_quantize_fp8_empty_is_noop():
    assert _quant(seg=0, x=None, codes=None, descale=None) == ra.RA_OK
    assert _quant(kind=ra.RA_FP8_VT, seg=0) == ra.RA_OK


def _fp8(**kw):
    args = dict(rank=3, N=8, L=8 * 128, H=4, H_kv=2, d=128, B=1, Q=P, qs=P2, K=P, ks=P2, V=P,
                vs=P2, scale=0.088, O=P2, m=None, l=None, cast=None, stream=None)
    args.update(kw)
    return ra.load().ra_share_forward_fp8(
        args["rank"], args["N"], args["L"], args["H"], args["H_kv"], args["d"], args["B"],
        args["Q"], args["qs"], args["K"], args["ks"], args["V"], args["vs"], args["scale"],
        args["O"], args["m"], args["l"], args["cast"], args["stream"])


@pytest.mark.parametrize("kw", [
    dict(N=0), dict(rank=8), dict(rank=-1), dict(L=8 * 128 + 1), dict(L=-8), dict(H=5),
    dict(H_kv=0), dict(d=96), dict(B=0), dict(scale=0.0), dict(scale=float("inf")),
    dict(Q=None), dict(qs=None), dict(K=None), dict(ks=None), dict(V=None), dict(vs=None),
    dict(O=None), dict(O=MIS), dict(vs=MIS), dict(m=MIS), dict(cast=MIS)])
def test_share_forward_fp8_rejects(kw):
    assert _fp8(**kw) == ra.RA_EINVAL


def test_share_forward_fp8_limits_and_noop():
    assert _fp8(L=0, Q=None, K=None, V=None, O=None) == ra.RA_OK
    # one K head of L*d bytes must stay below 2^31 (32-bit buffer range)
    assert _fp8(N=8, L=1 << 24, d=128) == ra.RA_ENOTSUP


def _cfp8(**kw):
    args = dict(rank=3, N=8, L=8 * 128, H=4, H_kv=2, d=128, B=1, layout=0, Q=P, qs=P2, K=P,
                ks=P2, V=P, vs=P2, scale=0.088, O=P2, m=None, l=None, cast=None, stream=None)
    args.update(kw)
    return ra.load().ra_causal_share_forward_fp8(
        args["rank"], args["N"], args["L"], args["H"], args["H_kv"], args["d"], args["B"],
        args["layout"], args["Q"], args["qs"], args["K"], args["ks"], args["V"], args["vs"],
        args["scale"], args["O"], args["m"], args["l"], args["cast"], args["stream"])


@pytest.mark.parametrize("kw", [
    dict(layout=3), dict(layout=-1), dict(layout=2, L=8 * 64), dict(layout=2, L=8 * 192),
    dict(N=0), dict(rank=8), dict(H=5), dict(d=96), dict(scale=0.0), dict(Q=None),
    dict(vs=MIS), dict(O=MIS)])
def test_causal_share_forward_fp8_rejects(kw):
    assert _cfp8(**kw) == ra.RA_EINVAL


def test_causal_share_forward_fp8_noop():
    assert _cfp8(L=0, Q=None, K=None, V=None, O=None) == ra.RA_OK


# ------------------------------------------------------------------ allocation-free backward

def test_backward_noalloc_rejects_before_device_work():
    lib = ra.load()

    def call(**kw):
        a = dict(rank=0, N=4, L=1024, H=2, H_kv=2, d=128, B=1, dtype=ra.RA_BF16, scale=0.088)
        a.update(kw)
        return lib.ra_share_backward_noalloc(a["rank"], a["N"], a["L"], a["H"], a["H_kv"],
                                             a["d"], a["B"], a["dtype"], P, P, P, P, P, P, P,
                                             a["scale"], P, P, P, None)
    assert call(N=0) == ra.RA_EINVAL
    assert call(rank=4) == ra.RA_EINVAL
    assert call(L=1000, N=3) == ra.RA_EINVAL
    assert call(H=3, H_kv=2) == ra.RA_EINVAL
    assert call(scale=float("nan")) == ra.RA_EINVAL
    assert call(dtype=ra.RA_F32) == ra.RA_ENOTSUP
    assert call(L=0) == ra.RA_OK
    # 8 bytes per query row: 2^20 rows fit, one more query row per head does not
    rows = ra.NOALLOC_SCRATCH_BYTES // 8
    assert lib.ra_share_backward_workspace(1, 16, rows // 16) == ra.NOALLOC_SCRATCH_BYTES
    assert call(H=16, H_kv=16, N=1, L=rows // 16 + 1) == ra.RA_ESCRATCH
    assert call(B=2, H=64, H_kv=8, N=8, L=8 * 16384) == ra.RA_ESCRATCH
    assert b"scratch" in lib.ra_strerror(ra.RA_ESCRATCH)


def test_quantize_fp8_hadamard_rejects():
    lib = ra.load()
    f = ctypes.c_void_p(0x30000)
    assert lib.ra_quantize_fp8_hadamard(1, 2, 1, 64, 96, P, f, 0, P, f, None) == ra.RA_EINVAL
    assert lib.ra_quantize_fp8_hadamard(1, 2, 0, 64, 128, P, f, 0, P, f, None) == ra.RA_EINVAL
    assert lib.ra_quantize_fp8_hadamard(0, 2, 1, 64, 128, P, f, 0, P, f, None) == ra.RA_EINVAL
    assert lib.ra_quantize_fp8_hadamard(1, 2, 1, 64, 128, P, None, 1, P, f, None) == ra.RA_EINVAL
    assert lib.ra_quantize_fp8_hadamard(1, 2, 1, 64, 128, P, f, 1, None, f, None) == ra.RA_EINVAL
    assert lib.ra_quantize_fp8_hadamard(1, 2, 1, 0, 128, None, None, 1, None, None,
                                        None) == ra.RA_OK


# ------------------------------------------------------------------ sizes beyond 64 bits

BIG = 2**31 - 1
TOP = 2**63 - 1


def test_sizes_beyond_64_bits_are_unsupported():
    """Products of the size arguments that overflow int64 are rejected as unsupported,
    not wrapped round into small (and so accepted) values."""
    for dtype in (ra.RA_F32, ra.RA_BF16):
        assert _share(rank=0, N=1, L=1024, B=BIG, H=BIG, H_kv=BIG, dtype=dtype) == ra.RA_ENOTSUP
    assert _share(rank=7, N=8, L=TOP - TOP % 8, H=1, H_kv=1, dtype=ra.RA_F32) == ra.RA_ENOTSUP
    for causal in (False, True):
        assert _backward(causal, rank=0, N=1, L=1024, B=BIG, H=BIG, H_kv=BIG) == ra.RA_ENOTSUP
    assert _fp8(rank=0, N=1, L=1024, B=BIG, H=BIG, H_kv=BIG) == ra.RA_ENOTSUP
    assert _fp8(rank=7, N=8, L=TOP - TOP % 8, H=1, H_kv=1) == ra.RA_ENOTSUP
    assert _quant(B=BIG, Hx=BIG, n_seg=BIG, seg=256) == ra.RA_ENOTSUP
    assert _quant(B=1, Hx=1, n_seg=BIG, seg=TOP) == ra.RA_ENOTSUP
    lib = ra.load()
    assert lib.ra_share_backward_workspace(BIG, BIG, TOP) == -ra.RA_ENOTSUP
    assert lib.ra_fp8_tiles(TOP) == TOP // 64 + 1
    for layout in range(3):
        assert lib.ra_causal_pairs(0, 2, TOP - TOP % 4, layout) == -ra.RA_ENOTSUP
    # counts just below 2^63 stay exact: each query's key count rises by a fixed step
    # along the share (contiguous 1, striped N), so the total is an arithmetic series,
    # l * (first + last) / 2, taken here in Python's exact integers
    N, L = 2, 2**32
    l = L // N
    for layout, first, step in ((0, l + 1, 1), (1, 2, N)):
        last = first + (l - 1) * step
        want = l * (first + last) // 2
        assert 2**62 < want < 2**63
        assert lib.ra_causal_pairs(1, N, L, layout) == want
