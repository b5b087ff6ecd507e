"""Pins of the verification variants of the oracle ("Introspective Diffusion
Language Models | Summary", section 3.3 for argmax proposals and the
relaxed-acceptance ablation of section 4).

* Argmax proposals with a sampled anchor (q_onehot): identical to verifying
  against explicit one-hot proposal rows, ratio P(x), output law P.
* Relaxed acceptance min(1, (1 + tau) r): tau = 0 is the exact rule; for
  tau > 0 the exact emitted law (bisected from the oracle's decisions) equals
  the closed form Q(i) a_i + (1 - sum_x Q(x) a_x) R_i / Z with
  a_i = min(1, (1 + tau) P(i)/Q(i)), which is no longer P.
"""

import numpy as np
import pytest

from oracle import isd_oracle as O
from tests.test_oracle_pins import _emitted_law, _logits_from_probs, _rand_probs


@pytest.fixture
def rng():
    return np.random.default_rng(20261203)


def test_onehot_flag_equals_explicit_onehot_rows(rng):
    B, L, V = 4, 5, 12
    p = rng.normal(0, 2, (B, L, V))
    x = rng.integers(0, V, (B, L))
    q = np.full((B, L, V), -np.inf)
    np.put_along_axis(q, x[..., None], 0.0, axis=-1)
    ua, ur = rng.random((B, L)), rng.random((B, L))
    a = O.verify_sample(p, q, x, ua, ur)
    b = O.verify_sample(p, None, x, ua, ur, q_onehot=True)
    for key in ("accept_len", "out_tokens", "n_emitted", "p_x", "q_x", "ratio", "alpha"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    np.testing.assert_allclose(b["ratio"], b["p_x"], rtol=1e-15)


def test_onehot_flag_keeps_law_P_bruteforce(rng):
    V = 6
    P = _rand_probs(rng, V)
    for xv in range(V):
        Q = np.zeros(V)
        Q[xv] = 1.0
        law = _emitted_law(P[None], Q[None], Q[None], 0, q_onehot=True)
        np.testing.assert_allclose(law, P, rtol=0, atol=1e-12)


def test_relax_zero_is_exact_rule(rng):
    B, L, V = 6, 4, 20
    p, q = rng.normal(0, 2, (B, L, V)), rng.normal(0, 2, (B, L, V))
    x = rng.integers(0, V, (B, L))
    ua, ur = rng.random((B, L)), rng.random((B, L))
    a = O.verify_sample(p, q, x, ua, ur)
    b = O.verify_sample(p, q, x, ua, ur, relax=0.0)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


@pytest.mark.parametrize("tau", [0.1, 0.5, 1.0])
@pytest.mark.parametrize("V", [3, 5])
def test_relaxed_law_closed_form_bruteforce(rng, tau, V):
    P = _rand_probs(rng, V)
    Q = _rand_probs(rng, V)
    law = _emitted_law(P[None], Q[None], Q[None], 0, relax=tau)
    acc = np.minimum(1.0, (1.0 + tau) * P / Q)
    R = np.maximum(0.0, P - Q)
    expect = Q * acc + (1.0 - (Q * acc).sum()) * R / R.sum()
    np.testing.assert_allclose(law, expect, rtol=0, atol=1e-12)
    assert np.abs(law - P).max() > 1e-3      # relaxation gives up the anchor law


def test_relax_accepts_at_least_as_often(rng):
    B, L, V = 64, 6, 30
    p, q = rng.normal(0, 2, (B, L, V)), rng.normal(0, 2, (B, L, V))
    x = rng.integers(0, V, (B, L))
    ua, ur = rng.random((B, L)), rng.random((B, L))
    j0 = O.verify_sample(p, q, x, ua, ur)["accept_len"]
    j1 = O.verify_sample(p, q, x, ua, ur, relax=0.3)["accept_len"]
    assert np.all(j1 >= j0) and np.any(j1 > j0)


def test_relax_rejects_negative():
    with pytest.raises(ValueError):
        O.verify_sample(np.zeros((1, 1, 2)), np.zeros((1, 1, 2)), np.zeros((1, 1), int),
                        np.zeros((1, 1)), np.zeros((1, 1)), relax=-0.1)
