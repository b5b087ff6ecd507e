"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than its own formulas:
library routines (scipy softmax/logsumexp, numpy searchsorted/argmax),
closed forms (E_{x~q} min(1, p/q) = 1 - TV(p, q); the accept-length law),
special cases (p == q; one-hot rows reduce sample mode to greedy mode;
argmax proposals), brute force on tiny vocabularies (the exact law of the
emitted token, obtained by bisecting the oracle's own decisions as a black
box) and an empirical test over 10^6 draws.

The law tests are the ones that pin the method's central claim: acceptance
together with the residual correction leaves the anchor distribution intact
("Introspective Diffusion Language Models | Summary", section 3.2).
"""

import numpy as np
import pytest
from scipy import special, stats

from oracle import isd_oracle as O


def _logits_from_probs(P):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(P, dtype=np.float64))


def _rand_probs(rng, V, zeros=0):
    w = rng.gamma(0.7, size=V)
    if zeros:
        w[rng.choice(V, size=zeros, replace=False)] = 0.0
    return w / w.sum()


# ---------------------------------------------------------------------------
# Softmax and gathered probabilities against library routines
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1.0, 0.7, 2.5])
def test_softmax_matches_scipy(rng, T):
    a = rng.normal(0, 4, size=(3, 5, 257))
    ours = O.softmax(a, T)
    ref = special.softmax(a / T, axis=-1)
    np.testing.assert_allclose(ours, ref, rtol=1e-13, atol=0)
    lse = special.logsumexp(a / T, axis=-1, keepdims=True)
    np.testing.assert_allclose(np.log(ours), a / T - lse, rtol=0, atol=1e-12)


def test_gathered_probabilities_match_scipy(rng):
    B, L, V = 4, 3, 50
    p = rng.normal(0, 2, (B, L, V))
    q = p + rng.normal(0, 0.5, (B, L, V))
    x = rng.integers(0, V, (B, L))
    out = O.verify_sample(p, q, x, rng.random((B, L)), rng.random((B, L)))
    Pref = special.softmax(p, axis=-1)
    Qref = special.softmax(q, axis=-1)
    for b in range(B):
        for k in range(L):
            assert out["p_x"][b, k] == pytest.approx(Pref[b, k, x[b, k]], rel=1e-13)
            assert out["q_x"][b, k] == pytest.approx(Qref[b, k, x[b, k]], rel=1e-13)


def test_temperature_is_logit_scaling(rng):
    B, L, V = 3, 4, 40
    p = rng.normal(0, 3, (B, L, V))
    q = p + rng.normal(0, 1, (B, L, V))
    x = rng.integers(0, V, (B, L))
    ua, ur = rng.random((B, L)), rng.random((B, L))
    a = O.verify_sample(p, q, x, ua, ur, temperature=2.0)
    b = O.verify_sample(p / 2.0, q / 2.0, x, ua, ur, temperature=1.0)
    for key in ("accept_len", "out_tokens", "n_emitted"):
        np.testing.assert_array_equal(a[key], b[key])
    np.testing.assert_allclose(a["alpha"], b["alpha"], rtol=1e-14)


# ---------------------------------------------------------------------------
# alpha: special cases and closed forms
# ---------------------------------------------------------------------------

def test_identical_rows_accept_everything(rng):
    """p == q (the same values): every ratio is 1, alpha is 1, all L accepted."""
    B, L, V = 16, 8, 300
    p = rng.normal(0, 3, (B, L, V))
    x = rng.integers(0, V, (B, L))
    ua = rng.random((B, L))
    ua[0, :] = np.nextafter(1.0, 0.0)
    out = O.verify_sample(p, p.copy(), x, ua, rng.random((B, L)))
    assert np.all(out["ratio"] == 1.0)
    assert np.all(out["alpha"] == 1.0)
    assert np.all(out["accept_len"] == L)
    assert np.all(out["n_emitted"] == L)
    np.testing.assert_array_equal(out["out_tokens"], x)


@pytest.mark.parametrize("V", [3, 6, 11])
def test_expected_ratio_is_one_minus_tv(rng, V):
    """E_{x~Q} min(1, P(x)/Q(x)) = sum_i min(P_i, Q_i) = 1 - TV(P, Q)."""
    for trial in range(5):
        P = _rand_probs(rng, V, zeros=trial % 2)
        Q = _rand_probs(rng, V)
        p = np.broadcast_to(_logits_from_probs(P), (V, 1, V))
        q = np.broadcast_to(_logits_from_probs(Q), (V, 1, V))
        x = np.arange(V)[:, None]
        r = O.verify_sample(p, q, x, np.zeros((V, 1)), np.zeros((V, 1)))["ratio"][:, 0]
        expected = np.dot(Q, r)
        assert expected == pytest.approx(1.0 - 0.5 * np.abs(P - Q).sum(), abs=1e-13)
        alpha = O.alpha_sample(p, q, x)
        assert np.dot(Q, alpha) == pytest.approx(1.0 - 0.5 * np.abs(P - Q).sum(), abs=1e-13)


def test_alpha_averages_all_positions():
    """alpha is the mean over all L positions, including those after j."""
    P0, Q0 = [0.1, 0.9], [0.5, 0.5]
    p = np.stack([_logits_from_probs(P0), [0.3, -0.2], [1.0, 2.0]])[None]
    q = np.stack([_logits_from_probs(Q0), [0.3, -0.2], [1.0, 2.0]])[None]
    x = np.array([[0, 1, 0]])
    out = O.verify_sample(p, q, x, np.array([[0.5, 0.0, 0.0]]), np.array([[0.3, 0.3, 0.3]]))
    assert out["accept_len"][0] == 0
    assert out["ratio"][0, 0] == pytest.approx(0.2, rel=1e-12)
    assert out["alpha"][0] == pytest.approx((0.2 + 1.0 + 1.0) / 3.0, rel=1e-12)
    # residual max(0, P0 - Q0) = [0, 0.4]: the correction is token 1 for any draw
    assert out["out_tokens"][0].tolist() == [1, -1, -1]
    assert out["n_emitted"][0] == 1


# ---------------------------------------------------------------------------
# Brute-force law of the emitted token on tiny vocabularies
# ---------------------------------------------------------------------------

def _bisect_threshold(f, lo, hi, iters=64):
    """Smallest u in (lo, hi] where the monotone step function f changes from f(lo)."""
    a = f(lo)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if f(mid) == a:
            lo = mid
        else:
            hi = mid
    return hi


def _step_measures(f, V):
    """Lebesgue measure of {u in [0,1): f(u) = i} for a monotone step function f."""
    meas = np.zeros(V)
    top = np.nextafter(1.0, 0.0)
    u = 0.0
    cur = f(u)
    while True:
        if f(top) == cur:
            meas[cur] += 1.0 - u
            return meas
        b = _bisect_threshold(f, u, top)
        meas[cur] += b - u
        u, cur = b, f(b)


def _emitted_law(P_rows, Q_rows, xs_weight, pos, **variant):
    """Exact law of the token emitted at position ``pos`` given every earlier
    position accepted, by bisecting the oracle's decisions as a black box.

    P_rows/Q_rows: [L, V] probabilities; xs_weight: Q_rows (proposals are drawn
    from them independently)."""
    L, V = P_rows.shape
    p = _logits_from_probs(P_rows)[None]
    q = _logits_from_probs(Q_rows)[None]
    law = np.zeros(V)
    for xv in range(V):
        wx = xs_weight[pos, xv]
        if wx == 0:
            continue
        x = np.zeros((1, L), dtype=np.int64)
        x[0, pos] = xv
        ua = np.zeros((1, L))            # earlier positions: u = 0 < r (forced accept)
        ur = np.zeros((1, L))

        def accepted(u):
            ua[0, pos] = u
            o = O.verify_sample(p, q, x, ua, ur, **variant)
            return int(o["accept_len"][0] > pos)

        # earlier positions must accept at u = 0, i.e. their ratio must be > 0
        acc_measure = _step_measures(accepted, 2)[1]

        ua[0, pos] = np.nextafter(1.0, 0.0)  # force a rejection here if possible

        def corrected(u):
            ur[0, pos] = u
            o = O.verify_sample(p, q, x, ua, ur, **variant)
            return int(o["out_tokens"][0, pos])

        if acc_measure < 1.0:
            res = _step_measures(corrected, V)
        else:
            res = np.zeros(V)
        law[xv] += wx * acc_measure
        law += wx * (1.0 - acc_measure) * res
    return law


@pytest.mark.parametrize("V", [2, 3, 5, 8])
def test_emitted_token_law_equals_anchor_bruteforce(rng, V):
    for trial in range(3):
        P = _rand_probs(rng, V, zeros=1 if (V > 2 and trial == 1) else 0)
        Q = _rand_probs(rng, V)
        law = _emitted_law(P[None], Q[None], Q[None], 0)
        np.testing.assert_allclose(law, P, rtol=0, atol=1e-12)


def test_emitted_token_law_later_position_bruteforce(rng):
    """With L = 3, the token emitted at position 2 (after two accepts) has law P_2."""
    V, L = 5, 3
    P = np.stack([_rand_probs(rng, V) for _ in range(L)])
    Q = np.stack([_rand_probs(rng, V) for _ in range(L)])
    law = _emitted_law(P, Q, Q, 2)
    np.testing.assert_allclose(law, P[2], rtol=0, atol=1e-12)


def test_argmax_proposal_law_bruteforce(rng):
    """Argmax proposals verified with their own one-hot law: r = P(x), the
    residual is P with x removed and renormalised, and the output law is P."""
    V = 6
    P = _rand_probs(rng, V)
    for xv in range(V):
        Q = np.zeros(V)
        Q[xv] = 1.0
        law = _emitted_law(P[None], Q[None], Q[None], 0)
        np.testing.assert_allclose(law, P, rtol=0, atol=1e-12)
        p = _logits_from_probs(P)[None, None]
        q = _logits_from_probs(Q)[None, None]
        r = O.verify_sample(p, q, np.array([[xv]]), np.zeros((1, 1)), np.zeros((1, 1)))["ratio"]
        assert r[0, 0] == pytest.approx(P[xv], rel=1e-13)


def test_emitted_token_law_empirical_chi2():
    """10^6 independent draws (x ~ Q by an independent sampler, ua, ur uniform):
    the emitted-token histogram passes a chi-square test against P."""
    rng = np.random.default_rng(7)
    V, N = 5, 1_000_000
    P = np.array([0.05, 0.4, 0.15, 0.3, 0.1])
    Q = np.array([0.3, 0.1, 0.25, 0.05, 0.3])
    p = np.broadcast_to(_logits_from_probs(P), (N, 1, V))
    q = np.broadcast_to(_logits_from_probs(Q), (N, 1, V))
    x = rng.choice(V, size=(N, 1), p=Q)
    out = O.verify_sample(p, q, x, rng.random((N, 1)), rng.random((N, 1)))
    counts = np.bincount(out["out_tokens"][:, 0], minlength=V)
    _, pval = stats.chisquare(counts, N * P)
    assert pval > 1e-4
    # the same draws would fail against the proposal law
    _, pval_q = stats.chisquare(counts, N * Q)
    assert pval_q < 1e-12


def test_accept_length_law_chi2():
    """Pr[j = m] = (prod_{k<m} beta_k)(1 - beta_m), Pr[j = L] = prod beta_k,
    with beta_k = sum_i min(P_k, Q_k)."""
    rng = np.random.default_rng(11)
    V, L, N = 5, 4, 200_000
    P = np.stack([_rand_probs(rng, V) for _ in range(L)])
    Q = np.stack([_rand_probs(rng, V) for _ in range(L)])
    beta = np.minimum(P, Q).sum(axis=-1)
    x = np.stack([rng.choice(V, size=N, p=Q[k]) for k in range(L)], axis=1)
    p = np.broadcast_to(_logits_from_probs(P), (N, L, V))
    q = np.broadcast_to(_logits_from_probs(Q), (N, L, V))
    out = O.verify_sample(p, q, x, rng.random((N, L)), rng.random((N, L)))
    hist = np.bincount(out["accept_len"], minlength=L + 1)
    law = np.array([np.prod(beta[:m]) * (1 - beta[m]) for m in range(L)] + [np.prod(beta)])
    assert law.sum() == pytest.approx(1.0, abs=1e-12)
    _, pval = stats.chisquare(hist, N * law)
    assert pval > 1e-4


# ---------------------------------------------------------------------------
# The inverse-CDF draw
# ---------------------------------------------------------------------------

def test_inverse_cdf_matches_searchsorted(rng):
    for V in (1, 2, 7, 64, 1000):
        for _ in range(50):
            w = rng.random(V) * (rng.random(V) > 0.3)
            if w.sum() == 0:
                w[rng.integers(V)] = 1.0
            u = rng.random()
            cum = np.cumsum(w)
            ref = int(np.searchsorted(cum, u * cum[-1], side="right"))
            idx, _, _ = O.inverse_cdf(w, np.float64(u))
            assert int(idx) == ref


def test_inverse_cdf_special_cases():
    w = np.array([0.0, 0.0, 0.25, 0.0, 0.75, 0.0])
    # u = 0 selects the first index with positive weight (never a zero-weight one)
    assert int(O.inverse_cdf(w, np.float64(0.0))[0]) == 2
    # just below 1 selects the last positive weight
    assert int(O.inverse_cdf(w, np.float64(np.nextafter(1.0, 0.0)))[0]) == 4
    # boundary: cum = [0,0,.25,.25,1,1]; u*Z = 0.25 exactly -> strictly greater rule picks 4
    assert int(O.inverse_cdf(w, np.float64(0.25))[0]) == 4
    # a single positive weight is chosen for every u
    one = np.zeros(9)
    one[5] = 3.0
    for u in (0.0, 0.1, 0.5, 0.999999):
        assert int(O.inverse_cdf(one, np.float64(u))[0]) == 5
    # margins: distance from u to the chosen token's two cumulative boundaries
    idx, margin, _ = O.inverse_cdf(np.array([1.0, 1.0, 2.0]), np.float64(0.3))
    assert int(idx) == 1 and margin == pytest.approx(0.05, abs=1e-15)


def test_inverse_cdf_overshoot_clamps_to_last_positive():
    w = np.array([0.5, 0.5, 0.0])
    idx, _, _ = O.inverse_cdf(w, np.float64(1.0))
    assert int(idx) == 1


# ---------------------------------------------------------------------------
# Greedy (strict) mode
# ---------------------------------------------------------------------------

def test_greedy_emits_anchor_argmax(rng):
    B, L, V = 64, 8, 97
    p = rng.normal(0, 1, (B, L, V))
    g = np.argmax(p, axis=-1)
    x = np.where(rng.random((B, L)) < 0.7, g, rng.integers(0, V, (B, L)))
    out = O.verify_greedy(p, x)
    for b in range(B):
        n = out["n_emitted"][b]
        np.testing.assert_array_equal(out["out_tokens"][b, :n], g[b, :n])
        assert np.all(out["out_tokens"][b, n:] == -1)
        mism = np.nonzero(x[b] != g[b])[0]
        assert out["accept_len"][b] == (mism[0] if mism.size else L)
    np.testing.assert_allclose(out["alpha"], (x == g).mean(axis=-1))


def test_greedy_equals_sample_mode_on_one_hot_rows(rng):
    """Sample mode on one-hot P = onehot(argmax p), Q = onehot(x) reproduces
    greedy decisions, corrections and alpha exactly."""
    B, L, V = 200, 6, 31
    p = rng.normal(0, 1, (B, L, V))
    g = O.argmax_first(p)
    x = np.where(rng.random((B, L)) < 0.6, g, rng.integers(0, V, (B, L)))
    grid = np.arange(V)
    P1 = np.where(grid[None, None, :] == g[..., None], 0.0, -np.inf)
    Q1 = np.where(grid[None, None, :] == x[..., None], 0.0, -np.inf)
    s = O.verify_sample(P1, Q1, x, rng.random((B, L)), rng.random((B, L)))
    gr = O.verify_greedy(p, x)
    for key in ("accept_len", "out_tokens", "n_emitted"):
        np.testing.assert_array_equal(s[key], gr[key])
    np.testing.assert_allclose(s["alpha"], gr["alpha"], rtol=0, atol=0)


def test_greedy_ties_pick_lowest_index():
    row = np.array([1.0, 3.0, -2.0, 3.0, 3.0, 0.0])
    assert int(O.argmax_first(row)) == 1
    zeros = np.array([-1.0, -0.0, 0.0, -5.0])
    assert int(O.argmax_first(zeros)) == 1
    assert int(O.argmax_first(np.full(7, -np.inf))) == 0
    p = np.stack([row, row])[None]
    out = O.verify_greedy(p, np.array([[3, 1]]))
    assert out["accept_len"][0] == 0 and out["out_tokens"][0].tolist() == [1, -1]


# ---------------------------------------------------------------------------
# Non-finite inputs, determinism
# ---------------------------------------------------------------------------

def test_neg_inf_logits_have_zero_probability(rng):
    V = 20
    p = rng.normal(0, 1, (1, 1, V))
    p[0, 0, ::2] = -np.inf
    q = p.copy()
    q[0, 0, 1] += 2.0
    P = O.softmax(p)
    assert np.all(P[0, 0, ::2] == 0.0)
    for u in np.linspace(0, 0.999, 200):
        tok, _, _, _ = O.propose_sample(p[0, 0], np.float64(u))
        assert int(tok) % 2 == 1
        out = O.verify_sample(p, q, np.array([[1]]), np.array([[0.9999]]), np.array([[u]]))
        assert out["out_tokens"][0, 0] % 2 == 1


def test_zero_anchor_probability_is_never_accepted(rng):
    """A proposal the anchor gives probability 0 has ratio 0 and must be
    rejected even for the smallest draw u = 0 (else the emitted law would put
    mass on a token with P = 0)."""
    V = 9
    p = rng.normal(0, 1, (1, 2, V))
    q = rng.normal(0, 1, (1, 2, V))
    p[0, 0, 4] = -np.inf
    out = O.verify_sample(p, q, np.array([[4, 0]]), np.zeros((1, 2)), np.zeros((1, 2)))
    assert out["ratio"][0, 0] == 0.0
    assert out["accept_len"][0] == 0
    assert out["out_tokens"][0, 0] != 4


def test_non_finite_rows_raise():
    with pytest.raises(ValueError):
        O.softmax(np.full((2, 5), -np.inf))
    with pytest.raises(ValueError):
        O.softmax(np.array([0.0, np.nan, 1.0]))
    with pytest.raises(ValueError):
        O.softmax(np.array([0.0, np.inf, 1.0]))


def test_deterministic(rng):
    B, L, V = 8, 4, 500
    p = rng.normal(0, 3, (B, L, V))
    q = p + rng.normal(0, 0.7, (B, L, V))
    x = rng.integers(0, V, (B, L))
    ua, ur = rng.random((B, L)), rng.random((B, L))
    a = O.verify_sample(p, q, x, ua, ur)
    b = O.verify_sample(p.copy(), q.copy(), x.copy(), ua.copy(), ur.copy())
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_propose_draw_law_matches_softmax_bruteforce(rng):
    """The proposal draw is an exact draw from softmax(qn/T): the measure of u
    giving token i equals its probability (scipy softmax)."""
    V = 7
    qn = rng.normal(0, 2, V)
    for T in (1.0, 0.5):
        meas = _step_measures(lambda u: int(O.propose_sample(qn, np.float64(u), T)[0]), V)
        np.testing.assert_allclose(meas, special.softmax(qn / T), rtol=0, atol=1e-12)


def test_bf16_decoding_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0xFF80, 0x7F80, 0x0000, 0x8000, 0x3FC0, 0x0001],
                    dtype=np.uint16)
    vals = O.decode_logits(bits, "bf16")
    assert vals[0] == 1.0 and vals[1] == -2.0
    assert np.isneginf(vals[2]) and np.isposinf(vals[3])
    assert vals[4] == 0.0 and vals[5] == 0.0 and np.signbit(vals[5])
    assert vals[6] == 1.5
    assert vals[7] == 2.0 ** -133


def test_cdf_interval_hand_case_and_inverse_cdf():
    # weights 1, 2, 3, 4 (total 10): token i owns [cum_{i-1}, cum_i) / 10
    w = np.array([1.0, 2.0, 3.0, 4.0])
    for i, (lo, hi) in enumerate([(0.0, 0.1), (0.1, 0.3), (0.3, 0.6), (0.6, 1.0)]):
        a, b = O.cdf_interval(w, i)
        assert abs(a - lo) < 1e-15 and abs(b - hi) < 1e-15
    # every uniform of a token's interval draws that token
    rng = np.random.default_rng(3)
    w = rng.random(50) * (rng.random(50) < 0.7)
    for u in rng.random(400):
        t = int(O.inverse_cdf(w, np.array(u))[0])
        lo, hi = O.cdf_interval(w, t)
        assert lo <= u < hi and w[t] > 0


def test_residual_weights_hand_case_and_fallback():
    P = np.array([[0.5, 0.3, 0.2, 0.0], [0.25, 0.25, 0.25, 0.25]])
    Q = np.array([[0.2, 0.4, 0.1, 0.3], [0.25, 0.25, 0.25, 0.25]])
    W, fb = O.residual_weights(P, Q)
    np.testing.assert_allclose(W[0], [0.3, 0.0, 0.1, 0.0], atol=1e-15)
    assert not fb[0] and fb[1]
    np.testing.assert_array_equal(W[1], P[1])       # equal laws: the draw falls back to P
