"""CPU check that the sampled-row gradient magnitudes used by the full-size backward
tests equal the dense ones (test_gpu_backward.magnitudes and the causal
masked_magnitudes) on a small share: every head of a GQA group, every layout."""
import numpy as np
import pytest

import test_gpu_backward as tb
import test_gpu_causal_backward as tcb

HEADS = [(0, 0), (0, 1), (0, 2), (0, 3)]
QR, KR = [0, 5, 95], [0, 100, 383]


def test_sampled_equal_dense_magnitudes():
    q, k, v, do = tb._draw(1, 4, 2, 64, 96, 384, 5)
    mq, mk, mv = tb.magnitudes(q, k, v, do, 0.125)
    ms = tb.sampled_magnitudes(q, k, v, do, 0.125, HEADS, QR, KR, chunk=32)
    for i, (b, h) in enumerate(HEADS):
        np.testing.assert_allclose(ms[i][0], mq[b, h, QR], rtol=1e-10)
    np.testing.assert_allclose(ms[0][1] + ms[1][1], mk[0, 0, KR], rtol=1e-10)
    np.testing.assert_allclose(ms[2][2] + ms[3][2], mv[0, 1, KR], rtol=1e-10)


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_sampled_equal_dense_masked_magnitudes(layout):
    q, k, v, do = tb._draw(1, 4, 2, 64, 96, 384, 6)
    mq, mk, mv, _ = tcb.masked_magnitudes(q, k, v, do, 0.125, 1, 4, layout)
    ms = tb.sampled_magnitudes(q, k, v, do, 0.125, HEADS, QR, KR, chunk=32, rank=1, N=4,
                               layout=layout)
    for i, (b, h) in enumerate(HEADS):
        np.testing.assert_allclose(ms[i][0], mq[b, h, QR], rtol=1e-10)
    np.testing.assert_allclose(ms[0][1] + ms[1][1], mk[0, 0, KR], rtol=1e-10, atol=1e-300)
    np.testing.assert_allclose(ms[2][2] + ms[3][2], mv[0, 1, KR], rtol=1e-10, atol=1e-300)
