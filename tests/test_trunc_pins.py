"""Pins of the oracle's top-k / top-p truncated sampling laws.

* With nothing truncated the law is the plain softmax, and top-k = 1 is the
  one-hot argmax (lowest index on ties).
* Hand-worked rows fix the ranking (ties to the lower index), the top-k cut
  and the top-p rule "keep a ranked entry while the mass before it is below p".
* On rows of distinct values the law equals the top-k then top-p logits
  warpers of the transformers library, an independent implementation of the
  same truncation ("Introspective Diffusion Language Models | Summary",
  section 4.1 samples with top-k 50 and top-p 0.95).
* The ISD rule on truncated P and Q, with proposals drawn from truncated Q,
  emits the truncated anchor law exactly (section 3.3: verification must use
  the law of the proposal mechanism actually used), and using the untruncated
  Q in the ratio instead does not.
"""

import numpy as np
import pytest

from oracle import isd_oracle as O
from tests.test_oracle_pins import _emitted_law


def _law(z, **kw):
    return O.truncated_probs(np.asarray(z, dtype=np.float64), **kw)[0]


def test_no_truncation_is_softmax():
    rng = np.random.default_rng(1)
    z = rng.standard_normal((4, 37)) * 3
    for T in (0.5, 1.0, 2.0):
        got, margin = O.truncated_probs(z, T, top_k=37, top_p=1.0)
        np.testing.assert_allclose(got, O.softmax(z, T), rtol=1e-13, atol=0)
        assert np.all(np.isinf(margin))
        got0, _ = O.truncated_probs(z, T, top_k=0, top_p=1.0)
        np.testing.assert_allclose(got0, O.softmax(z, T), rtol=1e-13, atol=0)


def test_top1_is_argmax_first():
    rng = np.random.default_rng(2)
    z = np.round(rng.standard_normal((50, 20)) * 2) / 2     # many ties
    got = _law(z, top_k=1)
    expect = np.zeros_like(z)
    expect[np.arange(50), O.argmax_first(z)] = 1.0
    np.testing.assert_array_equal(got, expect)


def test_hand_worked_rows():
    # ranking of [1, 3, 3, 2, 0]: idx 1, idx 2 (tie, lower index first), idx 3, idx 0, idx 4
    z = [1.0, 3.0, 3.0, 2.0, 0.0]
    e = np.exp
    np.testing.assert_allclose(_law(z, top_k=1), [0, 1, 0, 0, 0])
    np.testing.assert_allclose(_law(z, top_k=2), [0, 0.5, 0.5, 0, 0])
    d3 = 2 * e(3) + e(2)
    np.testing.assert_allclose(_law(z, top_k=3), [0, e(3) / d3, e(3) / d3, e(2) / d3, 0])
    # uniform row: ties only; top-k keeps the lowest indices
    np.testing.assert_allclose(_law([2.0] * 4, top_k=2), [0.5, 0.5, 0, 0])
    # top-p on probabilities 0.5, 0.3, 0.15, 0.05: masses before each rank 0, 0.5, 0.8, 0.95
    z = np.log([0.15, 0.5, 0.05, 0.3])
    np.testing.assert_allclose(_law(z, top_p=0.45), [0, 1, 0, 0], atol=1e-15)
    np.testing.assert_allclose(_law(z, top_p=0.55), [0, 0.5 / 0.8, 0, 0.3 / 0.8], atol=1e-15)
    np.testing.assert_allclose(_law(z, top_p=0.9), [0.15 / 0.95, 0.5 / 0.95, 0, 0.3 / 0.95],
                               atol=1e-15)
    np.testing.assert_allclose(_law(z, top_p=0.99), [0.15, 0.5, 0.05, 0.3], atol=1e-15)
    # top-p works inside the top-k renormalised law: with k = 2 the masses are 0.625, 0.375
    np.testing.assert_allclose(_law(z, top_k=2, top_p=0.6), [0, 1, 0, 0], atol=1e-15)
    np.testing.assert_allclose(_law(z, top_k=2, top_p=0.7), [0, 0.625, 0, 0.375], atol=1e-15)
    # uniform row with top-p: masses before ranks 0, 0.25, 0.5, 0.75
    np.testing.assert_allclose(_law([0.0] * 4, top_p=0.3), [0.5, 0.5, 0, 0], atol=1e-15)
    # a rank whose mass before it equals p exactly is cut (strict '<')
    np.testing.assert_allclose(_law([0.0] * 4, top_p=0.5), [0.5, 0.5, 0, 0], atol=1e-15)
    np.testing.assert_allclose(_law([0.0] * 4, top_p=0.25), [1, 0, 0, 0], atol=1e-15)
    # -0 and +0 tie, so the lower index ranks first
    np.testing.assert_allclose(_law([-0.0, 0.0, -1.0], top_k=1), [1, 0, 0])
    np.testing.assert_allclose(_law([0.0, -0.0, -1.0], top_k=1), [1, 0, 0])


def test_margin_reports_the_top_p_boundary():
    z = np.log([0.5, 0.3, 0.2])
    _, m = O.truncated_probs(z, top_p=0.8 + 1e-12)
    assert m < O.TRUNC_WINDOW
    _, m = O.truncated_probs(z, top_p=0.65)
    assert m == pytest.approx(0.15)


def test_top_p_keeps_smallest_prefix_property():
    rng = np.random.default_rng(3)
    for _ in range(40):
        V = int(rng.integers(2, 60))
        z = rng.standard_normal(V) * rng.uniform(0.5, 4)
        top_p = float(rng.uniform(0.05, 0.99))
        law = _law(z, top_p=top_p)
        P = O.softmax(z)
        kept = law > 0
        order = np.argsort(-z, kind="stable")
        n = int(kept.sum())
        # the kept set is a prefix of the ranking ...
        assert set(np.nonzero(kept)[0]) == set(order[:n])
        # ... whose mass reaches p, and dropping its last entry falls below p
        assert P[order[:n]].sum() >= top_p - 1e-12
        assert P[order[:n - 1]].sum() < top_p + 1e-12
        np.testing.assert_allclose(law[kept], P[kept] / P[kept].sum(), rtol=1e-12)


@pytest.mark.parametrize("top_k,top_p", [(5, 1.0), (50, 0.95), (7, 0.6), (0, 0.9), (1, 0.5)])
def test_matches_library_warpers(top_k, top_p):
    torch = pytest.importorskip("torch")
    lp = pytest.importorskip("transformers.generation.logits_process")
    rng = np.random.default_rng(4)
    V = 300
    z = rng.permutation(V) * 0.013 + rng.standard_normal(V) * 2.0    # distinct values
    assert len(np.unique(z)) == V
    for T in (1.0, 0.7):
        t = torch.tensor(z[None] / T, dtype=torch.float64)
        if top_k:
            t = lp.TopKLogitsWarper(top_k)(None, t)
        if top_p < 1.0:
            t = lp.TopPLogitsWarper(top_p)(None, t)
        expect = torch.softmax(t, dim=-1)[0].numpy()
        got, margin = O.truncated_probs(z, T, top_k=top_k, top_p=top_p)
        assert margin > 1e-6        # no row here sits on the top-p boundary
        np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-300)


def _trunc_rows(rng, L, V, **kw):
    z = rng.standard_normal((L, V)) * 1.5
    return z, O.truncated_probs(z, **kw)[0]


@pytest.mark.parametrize("top_k,top_p", [(3, 1.0), (0, 0.7), (4, 0.8)])
def test_truncated_verification_emits_truncated_anchor_law(top_k, top_p):
    rng = np.random.default_rng(5)
    V = 6
    zp, Pt = _trunc_rows(rng, 1, V, top_k=top_k, top_p=top_p)
    zq, Qt = _trunc_rows(rng, 1, V, top_k=top_k, top_p=top_p)
    # the helper takes probability rows (it passes their logarithms to the
    # oracle); give it the untruncated softmax rows and let the oracle truncate
    law = _emitted_law(np.exp(zp - zp.max()) / np.exp(zp - zp.max()).sum(),
                       np.exp(zq - zq.max()) / np.exp(zq - zq.max()).sum(), Qt, 0,
                       top_k=top_k, top_p=top_p)
    np.testing.assert_allclose(law, Pt[0], rtol=0, atol=1e-12)


def test_untruncated_ratio_breaks_the_law():
    """Proposals drawn from truncated Q but verified against the full Q: the
    emitted law is no longer the truncated P (the pin above would catch an
    oracle that truncated only one side)."""
    rng = np.random.default_rng(6)
    V = 6
    zp = rng.standard_normal((1, V)) * 1.5
    zq = rng.standard_normal((1, V)) * 1.5
    Pt = O.truncated_probs(zp, top_k=3)[0]
    Qt = O.truncated_probs(zq, top_k=3)[0]
    P = O.softmax(zp)
    Q = O.softmax(zq)
    law = _emitted_law(Pt, Q, Qt, 0)
    assert np.abs(law - Pt[0]).max() > 1e-3
    assert np.abs(law - P[0]).max() > 1e-6


def test_truncation_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.truncated_probs(np.zeros(4), top_k=-1)
    with pytest.raises(ValueError):
        O.truncated_probs(np.zeros(4), top_p=0.0)
    with pytest.raises(ValueError):
        O.truncated_probs(np.full(4, -np.inf), top_k=2)
