"""The parity tests' comparison rule, on the CPU: with the oracle's own
outputs standing in for the GPU's, compare() passes; at a flagged near tie it
accepts either side of the boundary, and it rejects choices the oracle's
numbers do not allow (a token far from the uniform's cumulative position, a
correction with no residual weight, a kept proposal whose ratio is below its
uniform)."""

import numpy as np
import pytest

from oracle import isd_oracle as O
from tests.isd_testlib import compare, oracle_step

OUT_KEYS = ("accept_len", "out_tokens", "n_emitted", "p_x", "q_x", "alpha", "next_tokens",
            "qnext_x")


def _inputs():
    rng = np.random.default_rng(0)
    C, L, V = 6, 4, 50
    p = rng.normal(0, 2, (C, L, V)).astype(np.float32)
    q = (p + rng.normal(0, 0.5, (C, L, V))).astype(np.float32)
    qn = rng.normal(0, 2, (C, L, V)).astype(np.float32)
    Q = O.softmax(q.astype(np.float64))
    x = np.array([[rng.choice(V, p=Q[c, k]) for k in range(L)] for c in range(C)], np.int32)
    ua, ur, up = (rng.random((C, L)).astype(np.float32) for _ in range(3))
    d = dict(p=p, q=q, qn=qn, x=x, ua=ua, ur=ur, up=up)
    # a decision near tie at sequence 0, position 0: ua just below the ratio
    P = O.softmax(p.astype(np.float64))
    r00 = O.accept_ratio(P[0, 0, x[0, 0]], Q[0, 0, x[0, 0]])
    d["ua"][0, 0] = np.float32(min(r00, 0.999999)) - np.float32(2e-7)
    # a proposal near tie at (1, 0): up on the boundary after token t
    Qn = O.softmax(qn[1, 0].astype(np.float64))
    t = int(np.argmax(Qn))
    d["up"][1, 0] = np.float32(np.cumsum(Qn)[t])
    return d, t


def _fake_gpu(ref):
    return {k: np.array(ref[k], copy=True) for k in OUT_KEYS}


def test_oracle_outputs_pass_and_flags_are_validated():
    d, _ = _inputs()
    ref = oracle_step(d, "f32", "sample", 1.0)
    assert ref["flagged"][0] and ref["next_flagged"][1, 0]
    st = compare(_fake_gpu(ref), ref, label="self")
    assert st["validated"] >= 2


def test_either_side_of_a_flagged_proposal_boundary_is_valid():
    d, t = _inputs()
    ref = oracle_step(d, "f32", "sample", 1.0)
    g = _fake_gpu(ref)
    other = t + 1 if ref["next_tokens"][1, 0] == t else t
    g["next_tokens"][1, 0] = other
    compare(g, ref, label="across the boundary")
    g["next_tokens"][1, 0] = (t + 25) % 50
    with pytest.raises(AssertionError, match="proposal"):
        compare(g, ref, label="far token")


def test_flagged_decision_may_go_either_way_but_the_correction_must_be_valid():
    d, _ = _inputs()
    ref = oracle_step(d, "f32", "sample", 1.0)
    assert ref["accept_len"][0] > 0          # the oracle kept x_0 (ua just below r)
    g = _fake_gpu(ref)
    # the GPU rejects x_0 instead and draws the correction from row 0's residual
    P = O.softmax(d["p"][0, 0].astype(np.float64))
    Q = O.softmax(d["q"][0, 0].astype(np.float64))
    W, _ = O.residual_weights(P, Q)
    corr = int(O.inverse_cdf(W, np.array(float(d["ur"][0, 0])))[0])
    g["accept_len"][0], g["n_emitted"][0] = 0, 1
    g["out_tokens"][0] = [corr, -1, -1, -1]
    compare(g, ref, label="rejected at the tie")
    g["out_tokens"][0, 0] = int(np.argmin(W))      # a token with no residual weight
    assert W[g["out_tokens"][0, 0]] == 0
    with pytest.raises(AssertionError, match="correction"):
        compare(g, ref, label="bad correction")


def test_keeping_a_proposal_below_its_uniform_is_rejected():
    d, _ = _inputs()
    ref = oracle_step(d, "f32", "sample", 1.0)
    c = int(np.nonzero(~ref["flagged"] & (ref["accept_len"] < 4))[0][0])
    g = _fake_gpu(ref)
    g["accept_len"][c] += 1
    with pytest.raises(AssertionError):
        compare(g, ref, label="unflagged accept_len")
