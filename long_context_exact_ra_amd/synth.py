"""Seeded synthetic inputs for the ring-attention share.

This module holds no arithmetic of the method: it only draws the Q, K, V tensors
that the GPU library and the CPU oracle both consume, from a seeded torch CPU
generator, in the order Q, K, V, as fp32 normal samples, cast to bf16 with
round-to-nearest-even where the workload is bf16.

The workloads stand in for the shapes the pages discuss: a 128K sequence split
into 8 blocks of 16K with 32 heads of dimension 128 (agentalpha interview page,
the Ring Attention answer and its communication-cost follow-up), a 28-query /
4-kv-head GQA model at 131072 tokens (lnwmold page, section 3.1), and the
million-token context (slowleelab page, L2 and 4.6).
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    H_kv: int
    d: int
    L: int
    N: int
    dtype: str          # "f32" or "bf16"
    seed: int
    qk_std: float = 1.0  # std of Q and K samples (V is always std 1)
    rank: int = 0        # the ring member whose share is measured
    full_q: bool = False  # True: Q covers all L rows (every rank's share is checked)

    @property
    def l(self) -> int:
        return self.L // self.N

    @property
    def q_rows(self) -> int:
        return self.L if self.full_q else self.l

    def flops(self) -> float:
        """Both contractions of one rank's share, non-causal: 4 * B * H * l * L * d."""
        return 4.0 * self.B * self.H * self.l * self.L * self.d


WORKLOADS = {
    "tiny_f32_L256_N4": Workload("tiny_f32_L256_N4", 1, 2, 2, 64, 256, 4, "f32", 1001,
                                 full_q=True),
    "share_L32K_N8": Workload("share_L32K_N8", 1, 32, 32, 128, 32768, 8, "bf16", 1002,
                              rank=3),
    "share_L128K_N8": Workload("share_L128K_N8", 1, 32, 32, 128, 131072, 8, "bf16", 1003,
                               rank=3),
    "gqa_L128K_N8_28q4kv": Workload("gqa_L128K_N8_28q4kv", 1, 28, 4, 128, 131072, 8,
                                    "bf16", 1004, rank=3),
    "share_L1M_N64_std3": Workload("share_L1M_N64_std3", 1, 4, 4, 128, 1048576, 64,
                                   "bf16", 1005, qk_std=3.0, rank=37),
}

HEADLINE = "share_L128K_N8"


def draw(B: int, H: int, H_kv: int, d: int, q_rows: int, L: int, dtype: str, seed: int,
         qk_std: float = 1.0, v_std: float = 1.0):
    """Q [B,H,q_rows,d], K and V [B,H_kv,L,d] on the CPU, drawn in the order Q, K, V."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((B, H, q_rows, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H_kv, L, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H_kv, L, d), generator=g, dtype=torch.float32)
    if qk_std != 1.0:
        q.mul_(qk_std)
        k.mul_(qk_std)
    if v_std != 1.0:
        v.mul_(v_std)
    if dtype == "bf16":
        q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    elif dtype != "f32":
        raise ValueError(dtype)
    return q, k, v


def draw_workload(w: Workload):
    return draw(w.B, w.H, w.H_kv, w.d, w.q_rows, w.L, w.dtype, w.seed, qk_std=w.qk_std)


def to_oracle_array(t: torch.Tensor):
    """Host numpy view of a tensor's stored bits: float32 as is, bf16 as uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def sample_rows(B: int, H: int, q_rows: int, per_head: int, seed: int, tile: int = 256):
    """Flat row indices (b*H + h)*q_rows + r for a seeded sample that covers every
    (batch, head), the first and last row, and both sides of every `tile` boundary
    in turn (the boundaries are spread across heads so the count stays bounded)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed) + 7)
    out = []
    n_bound = max(1, q_rows // tile)
    i = 0
    for b in range(B):
        for h in range(H):
            picks = {0, q_rows - 1}
            t = (i % n_bound) * tile
            for r in (t - 1, t, t + tile - 1, t + tile):
                if 0 <= r < q_rows:
                    picks.add(r)
            while len(picks) < min(per_head, q_rows):
                picks.add(int(torch.randint(0, q_rows, (1,), generator=g)))
            out.extend((b * H + h) * q_rows + r for r in sorted(picks))
            i += 1
    return out


def boundary_rows(B: int, H: int, q_rows: int, min_total: int, seed: int, tile: int = 256):
    """Flat row indices (b*H + h)*q_rows + r, sorted, covering in every (batch, head) the
    first and last row and both sides of every `tile` boundary, topped up with seeded
    random rows (spread evenly over the heads) until there are at least `min_total`."""
    g = torch.Generator(device="cpu").manual_seed(int(seed) + 11)
    n_heads = B * H
    per_head = -(-max(min_total, 1) // n_heads)
    out = []
    for bh in range(n_heads):
        picks = {0, q_rows - 1}
        for t in range(tile, q_rows, tile):
            picks.update((t - 1, t))
        target = min(q_rows, max(per_head, len(picks)))
        while len(picks) < target:
            picks.add(int(torch.randint(0, q_rows, (1,), generator=g)))
        out.extend(bh * q_rows + r for r in sorted(picks))
    return out
