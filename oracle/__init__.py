"""Plain fp64 CPU oracle for one ring member's attention share.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The product path (the HIP library and
its Python binding) never imports, loads or calls anything here, and this package
imports nothing from the product path.

Contents
--------
ring_schedule(rank, N)
    The ring visiting order: at step t, rank i works on K/V block (i - t) mod N
    (slowleelab "Ring Attention" page, L3 definition and the 4.2 algorithm).
kv_head(h, H, H_kv)
    Grouped-query head sharing, contiguous groups (lnwmold page, section 2.2).
attention_rows(...)
    The plain definition softmax(Q K^T * scale) V over a set of key ranges, fp64,
    every score materialised (C code in ra_oracle.c).  Returns the normalised
    output together with the row maximum M and the sum Z of exp(s - M).
causal_share(...), token_positions(...), causal_pairs(...)
    The causal share: a query attends only to keys at or before its own position in
    the sequence (slowleelab page, 4.5 limitation 2 and 4.8), for three ways of
    assigning tokens to ring members: contiguous blocks (the plain split of L2), the
    striped (interleaved) assignment of Striped Attention (4.8), and the zigzag
    assignment of two mirrored chunks per member (named in 4.5; the exact chunk
    pairing is this package's reading, see token_positions).
share_backward(...), share_backward_rows(...)
    Gradients of a share's output with respect to the resident queries and to every
    K/V row it read, from the plain definition (aliyun page, FlashAttention section:
    the backward pass recomputes the scores from the stored output and softmax
    statistics instead of storing the attention matrix; the gradient itself is that of
    softmax(scale Q K^T) V).  fp64 numpy, every matrix materialised.
fp8 (submodule)
    OCP E4M3 encoding, block quantization of Q/K (64-row blocks) and V (per channel,
    stored tile-transposed), and the share over such inputs as the plain definition on
    the dequantized values (aliyun page, FlashAttention-3: FP8 products with block
    quantization).
online_step(...)
    One merge of a K/V block into the running state (O_acc, m, l), in the order of
    the per-step pseudocode on the slowleelab page (section 4.3), fp64 numpy, with
    the readings listed in the design notes (row-wise max, exp(S - m_new) in both
    the sum and the output, division deferred to the final rescale, initial state
    O = 0, m = -inf, l = 0).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ra_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libra_oracle.so")
_lib = None

F32 = 0
BF16 = 1
F64 = 2


def build(force: bool = True) -> str:
    """Compile ra_oracle.c with gcc (fp64, OpenMP) into oracle/libra_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.ra_oracle_rows.restype = ctypes.c_int
        lib.ra_oracle_rows.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_double, i64p, ctypes.c_int64, i64p, i64p,
            ctypes.c_int, f64p, f64p, f64p, ctypes.c_int]
        lib.ra_oracle_rows_masked.restype = ctypes.c_int
        lib.ra_oracle_rows_masked.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_double, i64p, ctypes.c_int64, i64p, i64p,
            ctypes.c_int, i64p, i64p, f64p, f64p, f64p, ctypes.c_int]
        lib.ra_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ra_oracle_max_threads())


def ring_schedule(rank: int, N: int) -> list[int]:
    """K/V block used by `rank` at steps t = 0..N-1: (rank - t) mod N.

    slowleelab page, L3: at step t GPU i receives K/V block (i-t)%N from GPU i-1 and
    passes it on to GPU i+1; the N=4 table in 4.2 shows step 0 using the local block.
    Python's % already yields the non-negative remainder.
    """
    if N < 1 or not 0 <= rank < N:
        raise ValueError("need N >= 1 and 0 <= rank < N")
    return [(rank - t) % N for t in range(N)]


def kv_head(h: int, H: int, H_kv: int) -> int:
    """K/V head shared by query head h: contiguous groups of H/H_kv query heads."""
    if H % H_kv != 0 or not 0 <= h < H:
        raise ValueError("need H % H_kv == 0 and 0 <= h < H")
    return h // (H // H_kv)


def _raw(a: np.ndarray):
    """(dtype code, contiguous buffer) of an fp32 array, a bf16-bits uint16 array or an
    fp64 array."""
    if a.dtype == np.float32:
        return F32, np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return BF16, np.ascontiguousarray(a)
    if a.dtype == np.float64:
        return F64, np.ascontiguousarray(a)
    raise TypeError("inputs must be float32, float64, or uint16 arrays holding bf16 bits")


def attention_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                   rows=None, key_ranges=None, nthreads: int | None = None,
                   qpos=None, kpos=None):
    """The plain definition over the listed key ranges, for the listed query rows.

    Q: [B, H, l_q, d]; K, V: [B, H_kv, L, d]; all float32, all float64, or all uint16
    bf16 bits.
    rows: flat indices (b*H + h)*l_q + r (default: every row).
    key_ranges: list of (lo, hi) half-open key ranges (default: all L keys).
    scale: the fp32 scale the GPU uses, widened to fp64 here.
    qpos, kpos: optional causal mask; key k is used for selected row i only if
    kpos[k] <= qpos[i] (qpos has one entry per selected row, kpos one per key row).
    Returns (O [n, d] float64 normalised, M [n] float64, Z [n] float64).
    """
    dq, Qb = _raw(Q)
    dk, Kb = _raw(K)
    dv, Vb = _raw(V)
    if not dq == dk == dv:
        raise TypeError("Q, K and V must share a dtype")
    B, H, l_q, d = Qb.shape
    Bk, H_kv, L, dk_ = Kb.shape
    if Vb.shape != Kb.shape or Bk != B or dk_ != d:
        raise ValueError("shape mismatch")
    if rows is None:
        rows = np.arange(B * H * l_q, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if key_ranges is None:
        key_ranges = [(0, L)]
    lo = np.ascontiguousarray(np.array([r[0] for r in key_ranges], dtype=np.int64))
    hi = np.ascontiguousarray(np.array([r[1] for r in key_ranges], dtype=np.int64))
    n = rows.shape[0]
    O = np.empty((n, d), dtype=np.float64)
    M = np.empty((n,), dtype=np.float64)
    Z = np.empty((n,), dtype=np.float64)
    if nthreads is None:
        nthreads = max_threads()
    i64p = ctypes.POINTER(ctypes.c_int64)
    f64p = ctypes.POINTER(ctypes.c_double)
    if (qpos is None) != (kpos is None):
        raise ValueError("qpos and kpos go together")
    if qpos is not None:
        qpos = np.ascontiguousarray(np.asarray(qpos, dtype=np.int64))
        kpos = np.ascontiguousarray(np.asarray(kpos, dtype=np.int64))
        if qpos.shape != (n,) or kpos.shape != (L,):
            raise ValueError("qpos needs one entry per selected row, kpos one per key row")
        qp, kp = qpos.ctypes.data_as(i64p), kpos.ctypes.data_as(i64p)
    else:
        qp = kp = None
    rc = _load().ra_oracle_rows_masked(
        dq, Qb.ctypes.data, l_q, Kb.ctypes.data, Vb.ctypes.data, L, B, H, H_kv, d,
        float(scale), rows.ctypes.data_as(i64p), n, lo.ctypes.data_as(i64p),
        hi.ctypes.data_as(i64p), len(key_ranges), qp, kp, O.ctypes.data_as(f64p),
        M.ctypes.data_as(f64p), Z.ctypes.data_as(f64p), int(nthreads))
    if rc != 0:
        raise ValueError(f"ra_oracle_rows_masked failed with code {rc}")
    return O, M, Z


def share(Q, K, V, scale, rank: int, N: int, rows=None, steps: int | None = None,
          nthreads=None):
    """Rank `rank`'s share after `steps` ring steps (default all N): the definition
    restricted to the keys of blocks ring_schedule(rank, N)[:steps]."""
    L = K.shape[2]
    if L % N != 0:
        raise ValueError("L must split evenly into N blocks")
    l = L // N
    order = ring_schedule(rank, N)[: (N if steps is None else steps)]
    ranges = [(j * l, (j + 1) * l) for j in order]
    return attention_rows(Q, K, V, scale, rows=rows, key_ranges=ranges, nthreads=nthreads)


LAYOUTS = ("contiguous", "striped", "zigzag")


def token_positions(layout: str, rank: int, N: int, l: int) -> np.ndarray:
    """Global sequence positions of ring member `rank`'s l local tokens, in local order.

    contiguous: the plain Ring Attention split, member i holds tokens i*l .. (i+1)*l-1
                (slowleelab page, L2 problem statement: the sequence is split evenly
                into N blocks, block i on GPU i).
    striped:    Striped Attention's interleaved assignment (slowleelab page, 4.8):
                member i holds tokens i, i+N, i+2N, ...; local token x is x*N + i.
    zigzag:     the sequence is cut into 2N equal chunks of l/2 tokens and member i
                holds chunk i followed by chunk 2N-1-i (reading of the "Zigzag Ring"
                named in 4.5: each member pairs an early chunk with its mirror image,
                which evens out causal work); l must be even.
    """
    if N < 1 or not 0 <= rank < N or l < 0:
        raise ValueError("need N >= 1, 0 <= rank < N, l >= 0")
    x = np.arange(l, dtype=np.int64)
    if layout == "contiguous":
        return rank * l + x
    if layout == "striped":
        return x * N + rank
    if layout == "zigzag":
        if l % 2:
            raise ValueError("zigzag needs an even block length")
        h = l // 2
        return np.where(x < h, rank * h + x, (2 * N - 1 - rank) * h + (x - h))
    raise ValueError(f"unknown layout {layout!r}")


def layout_positions(layout: str, N: int, L: int) -> np.ndarray:
    """Position of every row of a member-major [.., L, ..] tensor: row j*l + x holds
    member j's local token x.  Gathering a sequence-ordered tensor with this index
    gives the member-major layout a ring would hold."""
    if L % N:
        raise ValueError("L must split evenly into N blocks")
    l = L // N
    return np.concatenate([token_positions(layout, j, N, l) for j in range(N)])


def causal_share(Q, K, V, scale, rank: int, N: int, layout: str, rows=None, nthreads=None):
    """Rank `rank`'s causal share: every key of the whole sequence whose position is
    at or before the query's own (slowleelab page, 4.5 limitation 2).

    Q is the member's [B, H, l, d] block in local order; K and V are [B, H_kv, L, d] in
    member-major layout (block j = member j's tokens, local order).  The visiting
    order of the ring does not change the result, so all keys are listed at once.
    """
    B, H, l, d = Q.shape
    L = K.shape[2]
    if L != N * l:
        raise ValueError("K/V must hold N blocks of the query block's length")
    if rows is None:
        rows = np.arange(B * H * l, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    qpos = token_positions(layout, rank, N, l)[rows % l]
    kpos = layout_positions(layout, N, L)
    return attention_rows(Q, K, V, scale, rows=rows, key_ranges=[(0, L)],
                          nthreads=nthreads, qpos=qpos, kpos=kpos)


def causal_pairs(rank: int, N: int, L: int, layout: str) -> int:
    """Number of (query, key) pairs that member `rank`'s causal share evaluates for one
    (batch, head): for each local query, the keys of the sequence at or before it."""
    l = L // N
    q = token_positions(layout, rank, N, l)
    # positions 0..L-1 are each held once, so the keys at or before p number p + 1
    return int(np.sum(q + 1))


def _f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of float32 arrays or bf16 bit patterns (uint16) to float64."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    raise TypeError("inputs must be float32 arrays or uint16 arrays holding bf16 bits")


def _head_backward(q, k, v, do, scale, mask=None):
    """One (query head, kv head) pair: q, do [n, d]; k, v [m, d] fp64; mask [n, m] bool
    (True = admissible) or None.  The softmax of each query row is over its admissible
    keys; the gradient of O = P V is taken through P = softmax(S), S = scale q k^T:
        dV = P^T dO,  dP = dO V^T,
        dS = P * (dP - sum_k P dP)      (the softmax Jacobian, row by row)
        dQ = scale dS K,  dK = scale dS^T Q."""
    S = scale * (q @ k.T)
    if mask is not None:
        S = np.where(mask, S, -np.inf)
    M = S.max(axis=1, keepdims=True)
    P = np.exp(S - M)
    P /= P.sum(axis=1, keepdims=True)
    dV = P.T @ do
    dP = do @ v.T
    dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
    return scale * (dS @ k), scale * (dS.T @ q), dV


def share_backward(Q, K, V, dO, scale, rank: int = 0, N: int = 1, layout: str | None = None):
    """Gradients of member `rank`'s share output O_i = softmax(scale Q_i K^T) V over all L
    keys (or, with `layout`, over its admissible keys as in causal_share), given the
    upstream gradient dO_i.  Returns (dQ_i [B, H, l, d], dK [B, H_kv, L, d],
    dV [B, H_kv, L, d]) in fp64: dK and dV hold this member's contribution to every key
    row; with grouped K/V heads the contributions of a group's query heads add up.
    The ring order does not enter: the share is a softmax over a set of keys."""
    q, k, v, do = (_f64(x) for x in (Q, K, V, dO))
    B, H, l, d = q.shape
    H_kv, L = k.shape[1], k.shape[2]
    g = H // H_kv
    mask = None
    if layout is not None:
        mask = (layout_positions(layout, N, L)[None, :]
                <= token_positions(layout, rank, N, l)[:, None])
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            a, bk, c = _head_backward(q[b, h], k[b, h // g], v[b, h // g], do[b, h], scale, mask)
            dQ[b, h] = a
            dK[b, h // g] += bk
            dV[b, h // g] += c
    return dQ, dK, dV


def share_backward_rows(Q, K, V, dO, scale, heads, q_rows, k_rows, chunk: int = 512,
                        rank: int = 0, N: int = 1, layout: str | None = None):
    """Sampled gradients for large shares, without materialising l x L per head at once.
    heads: list of (b, h) query heads; q_rows / k_rows: local query rows and key rows to
    report for each of them.  Returns, per head, (dQ[q_rows] [nq, d], dK_part[k_rows],
    dV_part[k_rows]) where the K/V parts are this query head's contribution only.
    Same formulas as share_backward, evaluated in query chunks (with `layout`, each
    chunk's scores are restricted to the admissible keys as in causal_share), with
    plain PyTorch CPU operations in float64 so that the elementwise work of a 128K share
    runs on every host core."""
    import torch

    q_all, k_all, v_all, do_all = Q, K, V, dO
    H = q_all.shape[1]
    H_kv = k_all.shape[1]
    g = H // H_kv
    qpos = kpos = None
    if layout is not None:
        qpos = torch.from_numpy(token_positions(layout, rank, N, q_all.shape[2]))
        kpos = torch.from_numpy(layout_positions(layout, N, k_all.shape[2]))
    kr = torch.as_tensor(np.asarray(k_rows, dtype=np.int64))
    qr = np.asarray(q_rows, dtype=np.int64)
    out = []
    for (b, h) in heads:
        q = torch.from_numpy(_f64(q_all[b, h]))
        k = torch.from_numpy(_f64(k_all[b, h // g]))
        v = torch.from_numpy(_f64(v_all[b, h // g]))
        do = torch.from_numpy(_f64(do_all[b, h]))
        l = q.shape[0]
        dK = torch.zeros((kr.numel(), q.shape[1]), dtype=torch.float64)
        dV = torch.zeros_like(dK)
        dQ = torch.zeros((len(qr), q.shape[1]), dtype=torch.float64)
        for c0 in range(0, l, chunk):
            c1 = min(l, c0 + chunk)
            sel = np.nonzero((qr >= c0) & (qr < c1))[0]
            if kr.numel() == 0 and sel.size == 0:
                continue  # this chunk adds nothing that was asked for
            S = scale * (q[c0:c1] @ k.T)
            if qpos is not None:
                S = torch.where(kpos[None, :] <= qpos[c0:c1, None], S,
                                torch.tensor(-math.inf, dtype=torch.float64))
            P = torch.exp(S - S.max(dim=1, keepdim=True).values)
            P /= P.sum(dim=1, keepdim=True)
            dP = do[c0:c1] @ v.T
            dS = P * (dP - torch.sum(P * dP, dim=1, keepdim=True))
            dV += P[:, kr].T @ do[c0:c1]
            dK += scale * (dS[:, kr].T @ q[c0:c1])
            if sel.size:
                dQ[torch.from_numpy(sel)] = scale * (dS[torch.from_numpy(qr[sel] - c0)] @ k)
        out.append((dQ.numpy(), dK.numpy(), dV.numpy()))
    return out


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def init_state(rows: int, d: int):
    """Initial running state: O = 0, m = -inf, l = 0 (the pages leave it unstated)."""
    return (np.zeros((rows, d)), np.full((rows,), -np.inf), np.zeros((rows,)))


def online_step(state, q: np.ndarray, k_blk: np.ndarray, v_blk: np.ndarray, scale: float):
    """Merge one K/V block into (O_acc, m, l), fp64, rows independent.

    q: [R, d]; k_blk, v_blk: [n, d] (fp64).  Follows the slowleelab page's per-step
    pseudocode (section 4.3): block scores, new running maximum, rescale of the old sum
    and old output by exp(m - m_new), accumulation of the block's exponentials.  The
    maximum is taken per row, the exponentials are taken relative to m_new, and no
    division happens here (it is the final rescale, see finalize()).
    """
    O, m, l = state
    S = (q @ k_blk.T) * scale                      # [R, n]
    m_new = np.maximum(m, S.max(axis=1))
    alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
    P = np.exp(S - m_new[:, None])
    l_new = alpha * l + P.sum(axis=1)
    O_new = alpha[:, None] * O + P @ v_blk
    return O_new, m_new, l_new


def finalize(state):
    """The final rescale O / l, applied once after the last step."""
    O, m, l = state
    return O / l[:, None]
