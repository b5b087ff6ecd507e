"""GPU parity of the verification variants against the oracle: relaxed
acceptance min(1, (1 + tau) P(x)/Q(x)) and argmax proposals with a sampled
anchor (Q = onehot(x), q not read) ("Introspective Diffusion Language Models |
Summary", section 3.3 and the relaxed-acceptance ablation of section 4)."""

import numpy as np
import pytest

from isd_inputs import CONFIGS, gen_step
from tests.isd_testlib import compare, log, oracle_step, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def isd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import speculative_verification_amd as isd_mod
    isd_mod.lib()
    return isd_mod


def _argmax_proposals(d, dtype):
    """x = argmax of the proposal rows (the picks an argmax proposer makes)."""
    from oracle import isd_oracle as O
    return O.argmax_first(O.decode_logits(d["q"], dtype)).astype(np.int32)


def _run(isd, dd, cfg, **variant):
    import torch
    q = None if variant.get("q_onehot") else dd["q"]
    o = isd.step(dd["p"], q, dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"],
                 temperature=cfg["T"], **variant)
    torch.cuda.synchronize()
    return to_host(o)


@pytest.mark.parametrize("tau", [0.25, 1.0])
def test_relaxed_acceptance_midsize(isd, tau):
    cfg = dict(CONFIGS[2], C=8, L=8, V=10000)
    totals = dict(j_gain=0)
    for step in range(6):
        d = gen_step(2, 500 + step, cfg=cfg)
        dd = to_device(d, cfg["dtype"])
        g = _run(isd, dd, cfg, relax=tau)
        ref = oracle_step(d, cfg["dtype"], "sample", cfg["T"], relax=tau)
        compare(g, ref, label=f"relax {tau} step {step}")
        exact = oracle_step(d, cfg["dtype"], "sample", cfg["T"])
        totals["j_gain"] += int((ref["accept_len"] - exact["accept_len"]).sum())
        assert np.all(ref["accept_len"] >= exact["accept_len"])
    log(f"relax {tau}: accepted positions gained over the exact rule {totals['j_gain']}")


def test_onehot_proposals_midsize(isd):
    cfg = dict(CONFIGS[2], C=8, L=8, V=10000)
    for step in range(6):
        d = gen_step(2, 600 + step, cfg=cfg)
        d["x"] = _argmax_proposals(d, cfg["dtype"])
        dd = to_device(d, cfg["dtype"])
        g = _run(isd, dd, cfg, q_onehot=True)
        ref = oracle_step(d, cfg["dtype"], "sample", cfg["T"], q_onehot=True)
        compare(g, ref, label=f"onehot step {step}")
        assert np.all(g["q_x"] == 1.0)


def test_onehot_and_relax_full_size(isd):
    """Both variants together at the serving shape, C=64, L=8, V=151936."""
    cfg = CONFIGS[2]
    seqs = np.arange(cfg["C"])
    d = gen_step(2, 7, seqs=seqs, workers=8)
    d["x"] = _argmax_proposals(d, cfg["dtype"])
    dd = to_device(d, cfg["dtype"])
    g = _run(isd, dd, cfg, q_onehot=True, relax=0.5)
    ref = oracle_step(d, cfg["dtype"], "sample", cfg["T"], relax=0.5, q_onehot=True)
    st = compare(g, ref, label="full onehot+relax")
    log(f"full-size one-hot + relax 0.5: {st}")
    for key, ws in list(isd.isd._ws_cache.items()):
        isd.check_device_error(ws)
