"""Pins of the oracle's LM head (logits = h @ W), the reference of the
LM-head GEMM and of the statistics path's exact-product logits.

"Introspective Diffusion Language Models | Summary", section 3.3: one extend
forward scores the clean positions and the mask positions together; its LM
head maps each hidden state (a row of h, [M, H]) to a row of vocabulary
logits through the head W [H, V].  These pins fix the operand order and the
layout: row m of the result is sum_k h[m, k] * W[k, :].
"""

import numpy as np
import pytest

from isd_inputs import bf16_bits_to_f32, gen_exact_head
from oracle import isd_oracle as O


def test_hand_worked_product():
    # worked by hand: row m of h picks a combination of the rows of w
    h = np.array([[1, 2, 0, -1],
                  [0, 1, 3, 0],
                  [2, 0, 1, 1]], dtype=np.float64)
    w = np.array([[1, 0, 2, 0, 1],
                  [0, 1, 0, 3, 1],
                  [1, 1, 0, 0, 2],
                  [0, 2, 1, 1, 0]], dtype=np.float64)
    expected = np.array([[1, 0, 1, 5, 3],     # w0 + 2 w1 - w3
                         [3, 4, 0, 3, 7],     # w1 + 3 w2
                         [3, 3, 5, 1, 4]],    # 2 w0 + w2 + w3
                        dtype=np.float64)
    got = O.lm_head(h, w)
    assert got.shape == (3, 5)
    np.testing.assert_array_equal(got, expected)


def test_one_hot_rows_select_rows_of_the_head():
    # a square head that is not symmetric: a transposed operand fails
    rng = np.random.default_rng(5)
    K = 6
    w = rng.integers(-9, 10, size=(K, K)).astype(np.float64)
    assert not np.array_equal(w, w.T)
    order = np.array([3, 0, 5, 1, 4, 2])
    h = np.eye(K)[order]
    np.testing.assert_array_equal(O.lm_head(h, w), w[order])


def test_rectangular_shapes_follow_h_rows_and_w_columns():
    h = np.zeros((2, 3))
    w = np.zeros((3, 7))
    assert O.lm_head(h, w).shape == (2, 7)
    with pytest.raises(ValueError):
        O.lm_head(h, np.zeros((7, 3)))   # W given as [V, H] is rejected by the shapes


def test_exact_head_inputs_against_explicit_loops():
    M, K, N = 6, 128, 300
    d = gen_exact_head(M, K, N, seed=4)
    h = bf16_bits_to_f32(d["h"]).astype(np.float64)
    w = bf16_bits_to_f32(d["wt"]).astype(np.float64).T      # wt is [N, K]
    got = O.lm_head(h, w)
    rng = np.random.default_rng(9)
    for m, n in zip(rng.integers(0, M, 40), rng.integers(0, N, 40)):
        acc = 0.0
        for k in range(K):
            acc += float(h[m, k]) * float(w[k, n])
        assert got[m, n] == acc
    # every product of these inputs is a multiple of 2^-7: exact in fp64 and fp32
    assert np.array_equal(got * 128, np.round(got * 128))
