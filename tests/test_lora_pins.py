"""Pins of the segment-gated LoRA oracle (``isd_oracle.lora_gemm``).

h_j = W x_j + [j is a mask position] B A x_j ("Introspective Diffusion
Language Models | Summary", appendix G and section 3.2).

* Brute force: explicit loops over every output element on tiny inputs.
* Gating: clean rows equal the base projection exactly, and mask rows differ
  from it by exactly B A x_j.
* Closed forms: one-hot adapters move a chosen input coordinate to a chosen
  output; a rank-1 adapter adds (a . x) b.
* Linearity in x, and the extend layout of the mask.
"""

import numpy as np
import pytest

from isd_inputs import extend_mask
from oracle import isd_oracle as O


def _rand(rng, M=6, K=5, N=4, r=3):
    return (rng.standard_normal((M, K)), rng.standard_normal((N, K)),
            rng.standard_normal((r, K)), rng.standard_normal((N, r)))


def test_bruteforce_loops():
    rng = np.random.default_rng(1)
    x, w, a, b = _rand(rng)
    mask = np.array([0, 1, 1, 0, 1, 0])
    h = O.lora_gemm(x, w, a, b, mask)
    M, K = x.shape
    N, r = b.shape
    for j in range(M):
        for n in range(N):
            base = sum(w[n, k] * x[j, k] for k in range(K))
            lora = sum(b[n, s] * sum(a[s, k] * x[j, k] for k in range(K)) for s in range(r))
            assert h[j, n] == pytest.approx(base + (lora if mask[j] else 0.0), rel=1e-12, abs=1e-12)


def test_gating_separates_clean_and_mask_rows():
    rng = np.random.default_rng(2)
    x, w, a, b = _rand(rng, M=8)
    mask = extend_mask(2, 2)                      # [0, 0, 1, 1, 0, 0, 1, 1]
    assert mask.tolist() == [0, 0, 1, 1, 0, 0, 1, 1]
    h = O.lora_gemm(x, w, a, b, mask)
    h0 = O.lora_gemm(x, w, a, b, np.zeros(8, int))
    clean = mask == 0
    np.testing.assert_array_equal(h[clean], h0[clean])
    delta = h[~clean] - h0[~clean]
    np.testing.assert_allclose(delta, (b @ (a @ x[~clean].T)).T, rtol=1e-12, atol=1e-12)
    # with a zero adapter every row is the base projection
    np.testing.assert_array_equal(O.lora_gemm(x, w, 0 * a, b, mask), h0)


def test_one_hot_adapter_moves_one_coordinate():
    rng = np.random.default_rng(3)
    M, K, N, r = 4, 7, 5, 2
    x = rng.standard_normal((M, K))
    w = np.zeros((N, K))
    a = np.zeros((r, K))
    b = np.zeros((N, r))
    a[1, 4] = 1.0          # adapter channel 1 reads input coordinate 4
    b[3, 1] = 2.0          # and writes twice it to output 3
    h = O.lora_gemm(x, w, a, b, np.ones(M, int))
    expect = np.zeros((M, N))
    expect[:, 3] = 2.0 * x[:, 4]
    np.testing.assert_array_equal(h, expect)


def test_rank_one_closed_form():
    rng = np.random.default_rng(4)
    M, K, N = 5, 9, 6
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K))
    av = rng.standard_normal(K)
    bv = rng.standard_normal(N)
    h = O.lora_gemm(x, w, av[None, :], bv[:, None], np.ones(M, int))
    for j in range(M):
        np.testing.assert_allclose(h[j], w @ x[j] + (av @ x[j]) * bv, rtol=1e-12, atol=1e-12)


def test_linear_in_x():
    rng = np.random.default_rng(5)
    x1, w, a, b = _rand(rng)
    x2 = rng.standard_normal(x1.shape)
    mask = np.array([1, 0, 1, 1, 0, 1])
    lhs = O.lora_gemm(x1 + 3.0 * x2, w, a, b, mask)
    rhs = O.lora_gemm(x1, w, a, b, mask) + 3.0 * O.lora_gemm(x2, w, a, b, mask)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
