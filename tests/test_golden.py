"""The oracle against the hand-worked cases in tests/golden/hand_cases.json,
and against its own committed outputs on the tiny workload (a regression pin:
tests/golden/config1_oracle.json is written by tests/golden/make_golden.py,
which calls only the oracle and the input generators)."""

import json
import os

import numpy as np
import pytest

from isd_inputs import CONFIGS, gen_step
from oracle import isd_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ln(P):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(P, dtype=np.float64))


@pytest.mark.parametrize("case", _load("hand_cases.json")["verify"], ids=lambda c: c["name"])
def test_hand_verify_cases(case):
    p = _ln(case["P"])[None]
    q = _ln(case["Q"])[None]
    out = O.verify_sample(p, q, np.array([case["x"]]), np.array([case["ua"]]),
                          np.array([case["ur"]]))
    np.testing.assert_allclose(out["ratio"][0], case["ratio"], rtol=1e-12)
    assert out["alpha"][0] == pytest.approx(case["alpha"], rel=1e-12)
    assert int(out["accept_len"][0]) == case["accept_len"]
    assert out["out_tokens"][0].tolist() == case["out_tokens"]
    assert int(out["n_emitted"][0]) == case["n_emitted"]


@pytest.mark.parametrize("case", _load("hand_cases.json")["propose"], ids=lambda c: c["name"])
def test_hand_propose_cases(case):
    tok, prob, _, _ = O.propose_sample(_ln(case["Qn"]), np.float64(case["up"]))
    assert int(tok) == case["token"]
    assert prob == pytest.approx(case["Qn"][case["token"]], rel=1e-12)


@pytest.mark.parametrize("case", _load("hand_cases.json")["greedy"], ids=lambda c: c["name"])
def test_hand_greedy_cases(case):
    out = O.verify_greedy(np.array(case["p"], dtype=np.float64)[None], np.array([case["x"]]))
    assert int(out["accept_len"][0]) == case["accept_len"]
    assert out["out_tokens"][0].tolist() == case["out_tokens"]
    assert int(out["n_emitted"][0]) == case["n_emitted"]
    assert out["alpha"][0] == pytest.approx(case["alpha"], rel=1e-12)


def test_tiny_workload_regression():
    gold = _load("config1_oracle.json")["steps"]
    cfg = CONFIGS[1]
    assert len(gold) == cfg["steps"]
    for g in gold[::7]:
        d = gen_step(1, g["step"])
        v = O.verify_sample(O.decode_logits(d["p"], "f32"), O.decode_logits(d["q"], "f32"),
                            d["x"], d["ua"], d["ur"], cfg["T"])
        tok, prob, _, _ = O.propose_sample(O.decode_logits(d["qn"], "f32"), d["up"], cfg["T"])
        assert v["accept_len"].tolist() == g["accept_len"]
        assert v["out_tokens"].tolist() == g["out_tokens"]
        assert tok.tolist() == g["next_tokens"]
        np.testing.assert_allclose(v["alpha"], g["alpha"], rtol=1e-14)
        np.testing.assert_allclose(v["p_x"], g["p_x"], rtol=1e-14)
        np.testing.assert_allclose(prob, g["next_prob"], rtol=1e-14)
