"""ctypes binding of libra.so, the ring-attention share library (include/ra.h).

Argument marshalling only: every entry point takes torch tensors that already live
in GPU memory, checks that they are device tensors of the expected shape (a host
pointer handed to a kernel would fault the GPU), and passes their data pointers and
torch's current HIP stream to the C function of the same name.  Every computation
runs in the library's HIP kernels; there is no fallback path, and a missing library
raises an error.
"""
from __future__ import annotations

import ctypes
import os

import torch

RA_OK, RA_EINVAL, RA_ENOTSUP, RA_EHIP, RA_ESCRATCH = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 8 << 20
RA_F32, RA_BF16 = 0, 1
RA_LAYOUT_CONTIGUOUS, RA_LAYOUT_STRIPED, RA_LAYOUT_ZIGZAG = 0, 1, 2
RA_FP8_ROWS, RA_FP8_VT = 0, 1
LAYOUTS = {"contiguous": RA_LAYOUT_CONTIGUOUS, "striped": RA_LAYOUT_STRIPED,
           "zigzag": RA_LAYOUT_ZIGZAG}

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libra.so")
_lib = None


class RaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = ""
        if status == RA_EHIP and _lib is not None:
            detail = f" (hipError {_lib.ra_last_hip_error()})"
        msg = _lib.ra_strerror(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg}{detail}")


class RaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("l_q", ctypes.c_int64), ("l_kv", ctypes.c_int64),
                ("kv_head_stride", ctypes.c_int64), ("kv_batch_stride", ctypes.c_int64),
                ("dtype", ctypes.c_int32)]


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libra.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m long_context_exact_ra_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    shp = ctypes.POINTER(RaShape)
    sigs = {
        "ra_ring_block": (i32, [i32, i32, i32]),
        "ra_ring_schedule": (ctypes.c_int, [i32, i32, ctypes.POINTER(i32)]),
        "ra_kv_head": (i32, [i32, i32, i32]),
        "ra_state_init": (ctypes.c_int, [vp, vp, vp, shp, vp]),
        "ra_step": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, f32, shp, vp]),
        "ra_finalize": (ctypes.c_int, [vp, vp, shp, vp, vp]),
        "ra_share_forward": (ctypes.c_int, [i32, i32, i64, i32, i32, i32, i32, i32, vp, vp,
                                            vp, f32, vp, vp, vp, vp, vp, vp]),
        "ra_causal_share_forward": (ctypes.c_int, [i32, i32, i64, i32, i32, i32, i32, i32,
                                                   i32, vp, vp, vp, f32, vp, vp, vp, vp,
                                                   vp]),
        "ra_causal_pairs": (i64, [i32, i32, i64, i32]),
        "ra_share_backward": (ctypes.c_int, [i32, i32, i64, i32, i32, i32, i32, i32, vp, vp,
                                             vp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp]),
        "ra_causal_share_backward": (ctypes.c_int, [i32, i32, i64, i32, i32, i32, i32, i32,
                                                    i32, vp, vp, vp, vp, vp, vp, vp, f32, vp,
                                                    vp, vp, vp, vp]),
        "ra_share_backward_workspace": (i64, [i32, i32, i64]),
        "ra_share_backward_noalloc": (ctypes.c_int, [i32, i32, i64, i32, i32, i32, i32, i32,
                                                     vp, vp, vp, vp, vp, vp, vp, f32, vp, vp,
                                                     vp, vp]),
        "ra_fp8_tiles": (i64, [i64]),
        "ra_quantize_fp8": (ctypes.c_int, [i32, i32, i32, i32, i64, i32, vp, vp, vp, vp]),
        "ra_quantize_fp8_hadamard": (ctypes.c_int, [i32, i32, i32, i64, i32, vp, vp, i32, vp,
                                                    vp, vp]),
        "ra_share_forward_fp8": (ctypes.c_int, [i32, i32, i64, i32, i32, i32, i32, vp, vp, vp,
                                                vp, vp, vp, f32, vp, vp, vp, vp, vp]),
        "ra_causal_share_forward_fp8": (ctypes.c_int, [i32, i32, i64, i32, i32, i32, i32, i32,
                                                       vp, vp, vp, vp, vp, vp, f32, vp, vp, vp,
                                                       vp, vp]),
        "ra_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "ra_last_hip_error": (ctypes.c_int, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols() -> list[str]:
    return ["ra_ring_block", "ra_ring_schedule", "ra_kv_head", "ra_state_init", "ra_step",
            "ra_finalize", "ra_share_forward", "ra_causal_share_forward", "ra_causal_pairs",
            "ra_share_backward", "ra_causal_share_backward", "ra_share_backward_workspace",
            "ra_share_backward_noalloc",
            "ra_fp8_tiles", "ra_quantize_fp8", "ra_quantize_fp8_hadamard",
            "ra_share_forward_fp8",
            "ra_causal_share_forward_fp8", "ra_strerror",
            "ra_last_hip_error"]


# ------------------------------------------------------------------ helpers

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (fp32 or bf16)")


def _dev(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor in GPU memory")
    # The library launches on the current device: memory of another GPU is refused here
    # rather than handed to a kernel that cannot address it.
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"{name} is on {t.device}, but calls run on the current device "
                         f"cuda:{cur} (select it with torch.cuda.device)")
    return ctypes.c_void_p(t.data_ptr())


def _need_shape(t: torch.Tensor, shape, name: str, dtype=None, contiguous=True):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    elif stream.device.index != torch.cuda.current_device():
        raise ValueError(f"the stream belongs to {stream.device}, but calls run on the "
                         f"current device cuda:{torch.cuda.current_device()}")
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != RA_OK:
        raise RaError(status, what)


# ------------------------------------------------------------------ host-only calls

def ring_block(rank: int, N: int, t: int) -> int:
    return int(load().ra_ring_block(rank, N, t))


def ring_schedule(rank: int, N: int) -> list[int]:
    out = (ctypes.c_int32 * max(N, 1))()
    _check(load().ra_ring_schedule(rank, N, out), "ra_ring_schedule")
    return [int(x) for x in out[:N]]


def kv_head(h: int, H: int, H_kv: int) -> int:
    return int(load().ra_kv_head(h, H, H_kv))


# ------------------------------------------------------------------ device calls

def make_shape(Q_i: torch.Tensor, K_blk: torch.Tensor | None = None) -> RaShape:
    B, H, l_q, d = Q_i.shape
    s = RaShape(B=B, H=H, H_kv=H, d=d, l_q=l_q, l_kv=0, kv_head_stride=0,
                kv_batch_stride=0, dtype=_dtype_code(Q_i))
    if K_blk is not None:
        Bk, H_kv, l_kv, dk = K_blk.shape
        if Bk != B or dk != d:
            raise ValueError("K block does not match Q_i")
        if K_blk.stride(3) != 1 or K_blk.stride(2) != d:
            raise ValueError("K/V block rows must be contiguous [.., l_kv, d]")
        # The library reads a stride of 0 as "contiguous default", so a broadcast
        # (expanded) head or batch axis would be taken for separate heads past the
        # tensor's end: refuse it; the caller materialises such a block.
        if (H_kv > 1 and K_blk.stride(1) == 0) or (B > 1 and K_blk.stride(0) == 0):
            raise ValueError("K/V block must not be broadcast along heads or batch "
                             "(stride 0); pass a materialised block")
        s.H_kv, s.l_kv = H_kv, l_kv
        s.kv_head_stride, s.kv_batch_stride = K_blk.stride(1), K_blk.stride(0)
    return s


def state_init(O_acc: torch.Tensor, m: torch.Tensor, l: torch.Tensor, stream=None):
    B, H, l_q, d = O_acc.shape
    _need_shape(O_acc, (B, H, l_q, d), "O_acc", torch.float32)
    _need_shape(m, (B, H, l_q), "m", torch.float32)
    _need_shape(l, (B, H, l_q), "l", torch.float32)
    s = RaShape(B=B, H=H, H_kv=H, d=d, l_q=l_q, dtype=RA_F32)
    _check(load().ra_state_init(_dev(O_acc, "O_acc"), _dev(m, "m"), _dev(l, "l"),
                                ctypes.byref(s), _stream(stream)), "ra_state_init")


def step(Q_i, K_blk, V_blk, O_acc, m, l, scale: float, stream=None):
    """Merge one K/V block into the running state (O_acc, m, l) in place."""
    s = make_shape(Q_i, K_blk)
    _need_shape(Q_i, Q_i.shape, "Q_i")
    if V_blk.shape != K_blk.shape or V_blk.stride() != K_blk.stride() or V_blk.dtype != Q_i.dtype \
            or K_blk.dtype != Q_i.dtype:
        raise ValueError("K_blk and V_blk must match in shape, strides and dtype with Q_i")
    B, H, l_q, d = Q_i.shape
    _need_shape(O_acc, (B, H, l_q, d), "O_acc", torch.float32)
    _need_shape(m, (B, H, l_q), "m", torch.float32)
    _need_shape(l, (B, H, l_q), "l", torch.float32)
    _check(load().ra_step(_dev(Q_i, "Q_i"), _dev(K_blk, "K_blk"), _dev(V_blk, "V_blk"),
                          _dev(O_acc, "O_acc"), _dev(m, "m"), _dev(l, "l"), float(scale),
                          ctypes.byref(s), _stream(stream)), "ra_step")


def finalize(O_acc, l, O_out=None, dtype=None, stream=None):
    """O_acc /= l in place; O_out (optional) receives the result in `dtype`."""
    B, H, l_q, d = O_acc.shape
    _need_shape(O_acc, (B, H, l_q, d), "O_acc", torch.float32)
    _need_shape(l, (B, H, l_q), "l", torch.float32)
    code = RA_F32
    if O_out is not None:
        code = _dtype_code(O_out)
        _need_shape(O_out, (B, H, l_q, d), "O_out")
    elif dtype is not None:
        code = RA_BF16 if dtype == torch.bfloat16 else RA_F32
    s = RaShape(B=B, H=H, H_kv=H, d=d, l_q=l_q, dtype=code)
    _check(load().ra_finalize(_dev(O_acc, "O_acc"), _dev(l, "l"), ctypes.byref(s),
                              _dev(O_out, "O_out"), _stream(stream)), "ra_finalize")


def share_forward(rank: int, N: int, L: int, H: int, H_kv: int, d: int, B: int,
                  Q_i, K, V, scale: float, O, m_out=None, l_out=None, O_cast=None,
                  sched_trace=None, stream=None):
    """Rank `rank`'s whole share in one launch (see ra_share_forward in ra.h)."""
    if N < 1 or L % N != 0:
        raise ValueError("L must be a multiple of N >= 1")
    l = L // N
    dt = Q_i.dtype
    _need_shape(Q_i, (B, H, l, d), "Q_i")
    _need_shape(K, (B, H_kv, L, d), "K", dt)
    _need_shape(V, (B, H_kv, L, d), "V", dt)
    _need_shape(O, (B, H, l, d), "O", torch.float32)
    if m_out is not None:
        _need_shape(m_out, (B, H, l), "m_out", torch.float32)
    if l_out is not None:
        _need_shape(l_out, (B, H, l), "l_out", torch.float32)
    if O_cast is not None:
        _need_shape(O_cast, (B, H, l, d), "O_cast", dt)
    if sched_trace is not None:
        _need_shape(sched_trace, (N,), "sched_trace", torch.int32)
    _check(load().ra_share_forward(
        rank, N, L, H, H_kv, d, B, _dtype_code(Q_i), _dev(Q_i, "Q_i"), _dev(K, "K"),
        _dev(V, "V"), float(scale), _dev(O, "O"), _dev(m_out, "m_out"), _dev(l_out, "l_out"),
        _dev(O_cast, "O_cast"), _dev(sched_trace, "sched_trace"), _stream(stream)),
        "ra_share_forward")


def _layout_code(layout) -> int:
    if isinstance(layout, str):
        if layout not in LAYOUTS:
            raise ValueError(f"unknown layout {layout!r}")
        return LAYOUTS[layout]
    return int(layout)


def causal_share_forward(rank: int, N: int, L: int, H: int, H_kv: int, d: int, B: int,
                         layout, Q_i, K, V, scale: float, O, m_out=None, l_out=None,
                         O_cast=None, stream=None):
    """Rank `rank`'s causal share in one launch (see ra_causal_share_forward in ra.h).
    `layout` is "contiguous", "striped", "zigzag" or an ra_layout code; K and V hold the
    sequence in member-major order."""
    if N < 1 or L % N != 0:
        raise ValueError("L must be a multiple of N >= 1")
    l = L // N
    dt = Q_i.dtype
    _need_shape(Q_i, (B, H, l, d), "Q_i")
    _need_shape(K, (B, H_kv, L, d), "K", dt)
    _need_shape(V, (B, H_kv, L, d), "V", dt)
    _need_shape(O, (B, H, l, d), "O", torch.float32)
    if m_out is not None:
        _need_shape(m_out, (B, H, l), "m_out", torch.float32)
    if l_out is not None:
        _need_shape(l_out, (B, H, l), "l_out", torch.float32)
    if O_cast is not None:
        _need_shape(O_cast, (B, H, l, d), "O_cast", dt)
    _check(load().ra_causal_share_forward(
        rank, N, L, H, H_kv, d, B, _dtype_code(Q_i), _layout_code(layout), _dev(Q_i, "Q_i"),
        _dev(K, "K"), _dev(V, "V"), float(scale), _dev(O, "O"), _dev(m_out, "m_out"),
        _dev(l_out, "l_out"), _dev(O_cast, "O_cast"), _stream(stream)),
        "ra_causal_share_forward")


def causal_pairs(rank: int, N: int, L: int, layout) -> int:
    """(query, key) pairs of member `rank`'s causal share per (batch, head) (host only)."""
    n = int(load().ra_causal_pairs(rank, N, L, _layout_code(layout)))
    if n < 0:
        raise RaError(-n, "ra_causal_pairs")
    return n


def _backward(rank, N, L, H, H_kv, d, B, layout, Q_i, K, V, O, dO, m, l, scale, dQ, dK, dV,
              workspace, stream):
    if N < 1 or L % N != 0:
        raise ValueError("L must be a multiple of N >= 1")
    lq = L // N
    dt = Q_i.dtype
    _need_shape(Q_i, (B, H, lq, d), "Q_i")
    _need_shape(K, (B, H_kv, L, d), "K", dt)
    _need_shape(V, (B, H_kv, L, d), "V", dt)
    _need_shape(O, (B, H, lq, d), "O", torch.float32)
    _need_shape(dO, (B, H, lq, d), "dO", dt)
    _need_shape(m, (B, H, lq), "m", torch.float32)
    _need_shape(l, (B, H, lq), "l", torch.float32)
    _need_shape(dQ, (B, H, lq, d), "dQ", torch.float32)
    _need_shape(dK, (B, H_kv, L, d), "dK", torch.float32)
    _need_shape(dV, (B, H_kv, L, d), "dV", torch.float32)
    nbytes = int(load().ra_share_backward_workspace(B, H, lq))
    if nbytes < 0:
        raise RaError(-nbytes, "ra_share_backward_workspace")
    if workspace is None:
        workspace = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=Q_i.device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    args = (_dev(Q_i, "Q_i"), _dev(K, "K"), _dev(V, "V"), _dev(O, "O"), _dev(dO, "dO"),
            _dev(m, "m"), _dev(l, "l"), float(scale), _dev(dQ, "dQ"), _dev(dK, "dK"),
            _dev(dV, "dV"), _dev(workspace, "workspace"), _stream(stream))
    if layout is None:
        _check(load().ra_share_backward(rank, N, L, H, H_kv, d, B, _dtype_code(Q_i), *args),
               "ra_share_backward")
    else:
        _check(load().ra_causal_share_backward(rank, N, L, H, H_kv, d, B, _dtype_code(Q_i),
                                               _layout_code(layout), *args),
               "ra_causal_share_backward")


def share_backward(rank: int, N: int, L: int, H: int, H_kv: int, d: int, B: int, Q_i, K, V, O,
                   dO, m, l, scale: float, dQ, dK, dV, workspace=None, stream=None):
    """Gradients of rank `rank`'s share (see ra_share_backward in ra.h): dQ is written,
    dK and dV are added to.  `workspace` (a uint8 device tensor of
    ra_share_backward_workspace bytes) is allocated here when not given."""
    _backward(rank, N, L, H, H_kv, d, B, None, Q_i, K, V, O, dO, m, l, scale, dQ, dK, dV,
              workspace, stream)


def share_backward_noalloc(rank: int, N: int, L: int, H: int, H_kv: int, d: int, B: int, Q_i,
                           K, V, O, dO, m, l, scale: float, dQ, dK, dV, stream=None):
    """share_backward without a workspace argument: the library's static scratch serves
    (see ra_share_backward_noalloc in ra.h; raises RaError(RA_ESCRATCH) for problems
    larger than NOALLOC_SCRATCH_BYTES of workspace)."""
    if N < 1 or L % N != 0:
        raise ValueError("L must be a multiple of N >= 1")
    lq = L // N
    dt = Q_i.dtype
    _need_shape(Q_i, (B, H, lq, d), "Q_i")
    _need_shape(K, (B, H_kv, L, d), "K", dt)
    _need_shape(V, (B, H_kv, L, d), "V", dt)
    _need_shape(O, (B, H, lq, d), "O", torch.float32)
    _need_shape(dO, (B, H, lq, d), "dO", dt)
    _need_shape(m, (B, H, lq), "m", torch.float32)
    _need_shape(l, (B, H, lq), "l", torch.float32)
    _need_shape(dQ, (B, H, lq, d), "dQ", torch.float32)
    _need_shape(dK, (B, H_kv, L, d), "dK", torch.float32)
    _need_shape(dV, (B, H_kv, L, d), "dV", torch.float32)
    _check(load().ra_share_backward_noalloc(
        rank, N, L, H, H_kv, d, B, _dtype_code(Q_i), _dev(Q_i, "Q_i"), _dev(K, "K"),
        _dev(V, "V"), _dev(O, "O"), _dev(dO, "dO"), _dev(m, "m"), _dev(l, "l"), float(scale),
        _dev(dQ, "dQ"), _dev(dK, "dK"), _dev(dV, "dV"), _stream(stream)),
        "ra_share_backward_noalloc")


def causal_share_backward(rank: int, N: int, L: int, H: int, H_kv: int, d: int, B: int,
                          layout, Q_i, K, V, O, dO, m, l, scale: float, dQ, dK, dV,
                          workspace=None, stream=None):
    """Gradients of rank `rank`'s causal share under `layout` (see ra_causal_share_backward
    in ra.h); arguments as in share_backward."""
    _backward(rank, N, L, H, H_kv, d, B, layout, Q_i, K, V, O, dO, m, l, scale, dQ, dK, dV,
              workspace, stream)


# ------------------------------------------------------------------ FP8

def fp8_tiles(seg: int) -> int:
    """ceil(seg / 64): scale blocks per segment / stored V tiles per member block."""
    n = int(load().ra_fp8_tiles(seg))
    if n < 0:
        raise RaError(-n, "ra_fp8_tiles")
    return n


def quantize_fp8(kind, x, n_seg: int, codes, descale, stream=None):
    """Block quantization of bf16 x [B, Hx, n_seg*seg, d] to E4M3 (see ra_quantize_fp8 in
    ra.h).  kind "rows" (Q, K): codes uint8 like x, descale [B, Hx, n_seg, T]; kind "vt"
    (V): codes uint8 [B, Hx, n_seg, T, d, 64], descale [B, Hx, d]."""
    k = {"rows": RA_FP8_ROWS, "vt": RA_FP8_VT}.get(kind, kind)
    B, Hx, R, d = x.shape
    if n_seg < 1 or R % n_seg != 0:
        raise ValueError("rows must split evenly into n_seg segments")
    seg = R // n_seg
    T = fp8_tiles(seg)
    _need_shape(x, (B, Hx, R, d), "x", torch.bfloat16)
    if k == RA_FP8_ROWS:
        _need_shape(codes, (B, Hx, R, d), "codes", torch.uint8)
        _need_shape(descale, (B, Hx, n_seg, T), "descale", torch.float32)
    else:
        _need_shape(codes, (B, Hx, n_seg, T, d, 64), "codes", torch.uint8)
        _need_shape(descale, (B, Hx, d), "descale", torch.float32)
    _check(load().ra_quantize_fp8(int(k), B, Hx, n_seg, seg, d, _dev(x, "x"),
                                  _dev(codes, "codes"), _dev(descale, "descale"),
                                  _stream(stream)), "ra_quantize_fp8")


def quantize_fp8_hadamard(x, signs, n_seg: int, codes, descale, query_side: bool,
                          stream=None):
    """Incoherent processing then rows-mode block quantization of bf16 x [B, Hx,
    n_seg*seg, d] (see ra_quantize_fp8_hadamard in ra.h): signs is a float32 device
    tensor [d]; query_side folds 1/d into the descales (quantize Q with True, K with
    False, the same signs)."""
    B, Hx, R, d = x.shape
    if n_seg < 1 or R % n_seg != 0:
        raise ValueError("rows must split evenly into n_seg segments")
    seg = R // n_seg
    T = fp8_tiles(seg)
    _need_shape(x, (B, Hx, R, d), "x", torch.bfloat16)
    _need_shape(signs, (d,), "signs", torch.float32)
    _need_shape(codes, (B, Hx, R, d), "codes", torch.uint8)
    _need_shape(descale, (B, Hx, n_seg, T), "descale", torch.float32)
    _check(load().ra_quantize_fp8_hadamard(B, Hx, n_seg, seg, d, _dev(x, "x"),
                                           _dev(signs, "signs"), int(bool(query_side)),
                                           _dev(codes, "codes"), _dev(descale, "descale"),
                                           _stream(stream)), "ra_quantize_fp8_hadamard")


def share_forward_fp8(rank: int, N: int, L: int, H: int, H_kv: int, d: int, B: int, Q8, qs, K8,
                      ks, V8t, vs, scale: float, O, m_out=None, l_out=None, O_cast=None,
                      stream=None, layout=None):
    """Rank `rank`'s share from E4M3 inputs (see ra_share_forward_fp8 in ra.h); with
    `layout`, the causal share of ra_causal_share_forward_fp8."""
    if N < 1 or L % N != 0:
        raise ValueError("L must be a multiple of N >= 1")
    l = L // N
    T = fp8_tiles(l)
    _need_shape(Q8, (B, H, l, d), "Q8", torch.uint8)
    _need_shape(qs, (B, H, 1, T), "q_descale", torch.float32)
    _need_shape(K8, (B, H_kv, L, d), "K8", torch.uint8)
    _need_shape(ks, (B, H_kv, N, T), "k_descale", torch.float32)
    _need_shape(V8t, (B, H_kv, N, T, d, 64), "V8t", torch.uint8)
    _need_shape(vs, (B, H_kv, d), "v_descale", torch.float32)
    _need_shape(O, (B, H, l, d), "O", torch.float32)
    if m_out is not None:
        _need_shape(m_out, (B, H, l), "m_out", torch.float32)
    if l_out is not None:
        _need_shape(l_out, (B, H, l), "l_out", torch.float32)
    if O_cast is not None:
        _need_shape(O_cast, (B, H, l, d), "O_cast", torch.bfloat16)
    args = (_dev(Q8, "Q8"), _dev(qs, "q_descale"), _dev(K8, "K8"), _dev(ks, "k_descale"),
            _dev(V8t, "V8t"), _dev(vs, "v_descale"), float(scale), _dev(O, "O"),
            _dev(m_out, "m_out"), _dev(l_out, "l_out"), _dev(O_cast, "O_cast"), _stream(stream))
    if layout is None:
        _check(load().ra_share_forward_fp8(rank, N, L, H, H_kv, d, B, *args),
               "ra_share_forward_fp8")
    else:
        _check(load().ra_causal_share_forward_fp8(rank, N, L, H, H_kv, d, B,
                                                  _layout_code(layout), *args),
               "ra_causal_share_forward_fp8")
