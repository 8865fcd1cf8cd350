"""The allocation-free backward (ra_share_backward_noalloc) against ra_share_backward.

Both run the same kernels on the same inputs; the only difference is where the per-row
workspace lives (the library's static device array instead of a caller buffer), so the
gradients must be equal bit for bit.  Two calls in a row, the second smaller, so the
second call runs on an array that still holds the first call's contents."""
import math

import pytest
import torch

from long_context_exact_ra_amd import ra, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    ra.load()
    return torch.device("cuda:0")


def _both(dev, B, H, H_kv, d, N, l, rank, seed):
    L = N * l
    q, k, v = synth.draw(B, H, H_kv, d, l, L, "bf16", seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn((B, H, l, d), generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(d)
    O = torch.empty((B, H, l, d), dtype=torch.float32, device=dev)
    m = torch.empty((B, H, l), dtype=torch.float32, device=dev)
    lo = torch.empty_like(m)
    ra.share_forward(rank, N, L, H, H_kv, d, B, qd, kd, vd, scale, O, m, lo)
    out = []
    for fn in ("share_backward", "share_backward_noalloc"):
        dQ = torch.full((B, H, l, d), float("nan"), dtype=torch.float32, device=dev)
        dK = torch.zeros((B, H_kv, L, d), dtype=torch.float32, device=dev)
        dV = torch.zeros_like(dK)
        getattr(ra, fn)(rank, N, L, H, H_kv, d, B, qd, kd, vd, O, dod, m, lo, scale, dQ, dK,
                        dV)
        torch.cuda.synchronize()
        out.append((dQ, dK, dV))
    return out


def test_noalloc_backward_equals_workspace_backward_twice(dev):
    # first call: GQA, d = 128, ragged blocks; second: smaller, d = 64
    for case in ((1, 4, 2, 128, 4, 300, 1, 901), (1, 2, 2, 64, 2, 130, 0, 902)):
        (a, b) = _both(dev, *case)
        for name, x, y in zip(("dQ", "dK", "dV"), a, b):
            assert torch.isfinite(x).all(), f"{case} {name}"
            assert torch.equal(x, y), f"{case} {name}: max diff {(x - y).abs().max().item()}"
        print(f"noalloc {case}: bitwise equal", flush=True)


def test_noalloc_backward_refuses_oversized_problems(dev):
    B, H, d, N = 1, 16, 64, 1
    l = ra.NOALLOC_SCRATCH_BYTES // (8 * H) + 1
    q = torch.zeros((B, H, l, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((B, H, l, d), dtype=torch.bfloat16, device=dev)
    f = torch.zeros((B, H, l, d), dtype=torch.float32, device=dev)
    s = torch.zeros((B, H, l), dtype=torch.float32, device=dev)
    with pytest.raises(ra.RaError) as e:
        ra.share_backward_noalloc(0, N, l, H, H, d, B, q, k, k, f, q, s, s, 0.125, f, f, f)
    assert e.value.status == ra.RA_ESCRATCH
