"""Pins of the multi-step decoding-loop oracle (oracle/isd_decode.py).

* The printed tokens-per-forward formula equals the long-run reward of the
  two-state chain that the loop's reading defines (an independent derivation),
  and its limits are N at full acceptance and 1 at none ("Introspective
  Diffusion Language Models | Summary", section 3.2 and appendix B).
* The ledger follows the loop's rules on hand cases.
* The input construction gives every verify position the overlap a.
* A Monte-Carlo run of the oracle's own loop, on those inputs, measures the
  tokens per forward that the formula predicts.
"""

import numpy as np
import pytest

from isd_inputs.decode import DECODE_CONFIGS, decode_step_inputs, pair
from oracle import isd_decode as D
from oracle import isd_oracle as O


@pytest.mark.parametrize("N", range(2, 10))
def test_tpf_limits(N):
    assert D.tpf_closed_form(1.0, N) == pytest.approx(N, abs=1e-12)
    assert D.tpf_closed_form(0.0, N) == pytest.approx(1.0, abs=1e-12)


@pytest.mark.parametrize("N", range(2, 10))
@pytest.mark.parametrize("a", [0.0, 0.1, 0.35, 0.5, 0.7, 0.83, 0.9, 0.99, 1.0])
def test_tpf_formula_equals_stationary_chain(a, N):
    assert D.tpf_closed_form(a, N) == pytest.approx(D.tpf_stationary(a, N), rel=1e-12, abs=1e-12)


def test_tpf_matches_pages_table_regime():
    # TPF rises with the stride at fixed acceptance and never exceeds N
    for a in (0.6, 0.9):
        vals = [D.tpf_closed_form(a, N) for N in range(2, 9)]
        assert all(b > c for b, c in zip(vals[1:], vals[:-1]))
        assert all(v <= N for v, N in zip(vals, range(2, 9)))


def test_ledger_hand_cases():
    L = 4
    state = np.array([D.VERIFY, D.VERIFY, D.VERIFY, D.RECOVER, D.RECOVER])
    j = np.array([4, 0, 2, -1, 4])
    emitted, nxt, bonus, anchor = D.ledger_step(state, j, L)
    assert emitted.tolist() == [5, 1, 3, 1, 1]
    assert nxt.tolist() == [D.VERIFY, D.RECOVER, D.RECOVER, D.VERIFY, D.VERIFY]
    assert bonus.tolist() == [True, False, False, False, False]
    assert anchor.tolist() == [False, False, False, True, True]


@pytest.mark.parametrize("a", [0.0, 0.3, 0.75, 1.0])
def test_overlap_construction(a):
    cfg = dict(DECODE_CONFIGS["cpu_mc"], a=a, C=3, L=2, V=200)
    P, Q = pair(5, cfg)
    Pp = O.softmax(P.astype(np.float64))
    Qq = O.softmax(Q.astype(np.float64))
    beta = np.minimum(Pp, Qq).sum(axis=-1)
    np.testing.assert_allclose(beta, a, atol=1e-6)


def _run_loop(cfg, steps):
    C, L = cfg["C"], cfg["L"]
    state = np.full(C, D.RECOVER, dtype=np.int32)
    x = np.zeros((C, L), dtype=np.int64)
    tokens = np.zeros(C, dtype=np.int64)
    forwards = np.zeros(C, dtype=np.int64)
    for t in range(steps):
        d = decode_step_inputs(t, cfg)
        out = D.decode_step(state, d["p"].astype(np.float64), d["q"].astype(np.float64), x,
                            d["ua"], d["ur"], d["qn"].astype(np.float64), d["up"], d["ub"],
                            d["uz"], cfg["T"])
        tokens += out["emitted"]
        forwards += 1
        state = out["next_state"]
        x = out["next_tokens"]
    return tokens, forwards


def test_loop_tokens_per_forward_monte_carlo():
    cfg = DECODE_CONFIGS["cpu_mc"]
    tokens, forwards = _run_loop(cfg, cfg["steps"])
    per_seq = tokens / forwards
    tpf = tokens.sum() / forwards.sum()
    sem = per_seq.std(ddof=1) / np.sqrt(len(per_seq))
    expect = D.tpf_closed_form(cfg["a"], cfg["L"] + 1)
    assert abs(tpf - expect) < 4 * sem + 0.01, (tpf, expect, sem)


def test_loop_limits_full_and_no_acceptance():
    for a, N_expect in ((1.0, None), (0.0, 1.0)):
        cfg = dict(DECODE_CONFIGS["cpu_mc"], a=a, C=4, V=32)
        tokens, forwards = _run_loop(cfg, 30)
        L = cfg["L"]
        if a == 1.0:
            # one recovery step (1 token), then 29 all-accept steps (L + 1 each)
            assert tokens.tolist() == [1 + 29 * (L + 1)] * 4
        else:
            # every verify step rejects at j = 0 and emits the correction only
            assert tokens.tolist() == [30] * 4
