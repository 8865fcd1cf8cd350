"""Pins of the causal share oracle (CPU only).

The causal share keeps, for each query, only the keys at or before its own sequence
position (slowleelab "Ring Attention" page, 4.5 limitation 2), under three ways of
assigning tokens to ring members (contiguous blocks, Striped Attention's interleaving,
zigzag mirrored chunks).  The pins below tie the oracle to things outside itself:
torch's causal scaled-dot-product attention on the whole sequence (a library routine),
the count of causal pairs of a sequence, and the permutation property of the layouts.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _sdpa_causal(Q, K, V, scale):
    """torch's causal attention in fp64 on the CPU; K/V heads repeated for GQA."""
    q = torch.from_numpy(Q.astype(np.float64))
    k = torch.from_numpy(K.astype(np.float64))
    v = torch.from_numpy(V.astype(np.float64))
    g = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(g, dim=1)
    v = v.repeat_interleave(g, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=True, scale=scale).numpy()


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
@pytest.mark.parametrize("N", [2, 3, 5])
def test_layout_positions_are_a_permutation(layout, N):
    L = N * 8
    pos = oracle.layout_positions(layout, N, L)
    assert sorted(pos.tolist()) == list(range(L))


def test_single_member_equals_torch_causal_attention():
    rng = np.random.default_rng(11)
    Q = rng.standard_normal((1, 2, 37, 16)).astype(np.float32)
    K = rng.standard_normal((1, 2, 37, 16)).astype(np.float32)
    V = rng.standard_normal((1, 2, 37, 16)).astype(np.float32)
    for layout in ("contiguous", "striped"):
        O, M, Z = oracle.causal_share(Q, K, V, 0.25, 0, 1, layout)
        ref = _sdpa_causal(Q, K, V, 0.25).reshape(-1, 16)
        np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    # the first query sees only itself: weight 1 on its own value row, Z = 1
    assert np.allclose(O[0], V[0, 0, 0]) and Z[0] == 1.0


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
@pytest.mark.parametrize("N,l", [(2, 6), (3, 4), (5, 8)])
def test_members_reassemble_causal_attention_of_the_sequence(layout, N, l):
    """Every member's causal share, put back in sequence order, is causal attention over
    the whole sequence: the ring split changes where work happens, not the result."""
    rng = np.random.default_rng(100 + 10 * N + l)
    B, H, H_kv, d = 2, 4, 2, 8
    L = N * l
    Qs = rng.standard_normal((B, H, L, d)).astype(np.float32)
    Ks = rng.standard_normal((B, H_kv, L, d)).astype(np.float32)
    Vs = rng.standard_normal((B, H_kv, L, d)).astype(np.float32)
    ref = _sdpa_causal(Qs, Ks, Vs, 0.3)
    perm = oracle.layout_positions(layout, N, L)
    Kmm, Vmm = Ks[:, :, perm], Vs[:, :, perm]
    for r in range(N):
        tok = oracle.token_positions(layout, r, N, l)
        O, _, _ = oracle.causal_share(Qs[:, :, tok], Kmm, Vmm, 0.3, r, N, layout)
        np.testing.assert_allclose(O.reshape(B, H, l, d), ref[:, :, tok], rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout", oracle.LAYOUTS)
def test_causal_pairs_cover_the_sequence_once(layout):
    N, L = 4, 64
    assert sum(oracle.causal_pairs(r, N, L, layout) for r in range(N)) == L * (L + 1) // 2


def test_causal_work_per_member():
    N, L = 4, 64
    l = L // N
    contiguous = [oracle.causal_pairs(r, N, L, "contiguous") for r in range(N)]
    # member r sees r full blocks plus a triangle of its own block
    assert contiguous == [r * l * l + l * (l + 1) // 2 for r in range(N)]
    # zigzag: every member does exactly the same work
    assert len({oracle.causal_pairs(r, N, L, "zigzag") for r in range(N)}) == 1
    # striped: member r + 1 sees one more key per query than member r
    striped = [oracle.causal_pairs(r, N, L, "striped") for r in range(N)]
    assert all(b - a == l for a, b in zip(striped, striped[1:]))


def test_row_with_no_admissible_key_is_an_error():
    Q = np.zeros((1, 1, 2, 4), np.float32)
    K = np.zeros((1, 1, 2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.attention_rows(Q, K, K, 1.0, qpos=[0, 1], kpos=[5, 6])


def test_zigzag_needs_even_blocks():
    with pytest.raises(ValueError):
        oracle.token_positions("zigzag", 0, 2, 5)
