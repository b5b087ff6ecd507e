"""GPU parity of the verification variants against the oracle: relaxed
acceptance min(1, (1 + tau) P(x)/Q(x)), argmax proposals with a sampled anchor
(Q = onehot(x), q not read) and the Gumbel-max correction on Philox4x32-10
("Introspective Diffusion Language Models | Summary", section 3.3 and the
relaxed-acceptance ablation of section 4)."""

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


def _gumbel_case(isd, cfg, seed, label, **variant):
    d = gen_step(2, seed, cfg=cfg)
    if variant.get("q_onehot"):
        d["x"] = _argmax_proposals(d, cfg["dtype"])
    dd = to_device(d, cfg["dtype"])
    g = _run(isd, dd, cfg, sampler="gumbel", **variant)
    ref = oracle_step(d, cfg["dtype"], "sample", cfg["T"], sampler="gumbel", **variant)
    st = compare(g, ref, label=label)
    cdf = oracle_step(d, cfg["dtype"], "sample", cfg["T"], **variant)
    # the decision does not depend on the sampler; the corrections do
    np.testing.assert_array_equal(ref["accept_len"], cdf["accept_len"])
    drawn = int((ref["accept_len"] < cfg["L"]).sum())
    same = int(sum(ref["out_tokens"][c, j] == cdf["out_tokens"][c, j]
                   for c, j in enumerate(ref["accept_len"]) if j < cfg["L"]))
    return st, drawn, same


@pytest.mark.parametrize("V,dtype", [(10000, "bf16"), (5003, "bf16"), (4099, "f32")])
def test_gumbel_correction_midsize(isd, V, dtype):
    """Several tiles and a ragged tail; V = 5003 in bf16 and f32 rows take the
    unaligned (scalar-load) path."""
    cfg = dict(CONFIGS[2], C=8, L=8, V=V, dtype=dtype)
    drawn = same = flags = 0
    for step in range(6):
        st, n, k = _gumbel_case(isd, cfg, 700 + step, f"gumbel V={V} {dtype} step {step}")
        drawn, same, flags = drawn + n, same + k, flags + st["resid_flags"]
    log(f"gumbel V={V} {dtype}: {drawn} corrections compared, {flags} excluded near ties, "
        f"{same} equal to the inverse-CDF draw")
    assert drawn > 0


def test_gumbel_with_onehot_and_relax(isd):
    cfg = dict(CONFIGS[2], C=8, L=8, V=10000)
    for step in range(4):
        _gumbel_case(isd, cfg, 800 + step, f"gumbel onehot+relax step {step}", q_onehot=True,
                     relax=0.5)


def test_gumbel_full_size_and_workspace(isd):
    """The serving shape C=64, L=8, V=151936; the workspace is zero again after
    Gumbel-max launches of both sizes."""
    import torch
    cfg = CONFIGS[2]
    seqs = np.arange(cfg["C"])
    d = gen_step(2, 9, seqs=seqs, workers=8)
    dd = to_device(d, cfg["dtype"])
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    o = isd.step(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"],
                 temperature=cfg["T"], sampler="gumbel", ws=ws)
    torch.cuda.synchronize()
    g = to_host(o)
    assert not torch.nonzero(ws).numel(), "workspace not zero after a Gumbel-max step"
    ref = oracle_step(d, cfg["dtype"], "sample", cfg["T"], sampler="gumbel")
    st = compare(g, ref, label="full gumbel")
    log(f"full-size Gumbel-max: {st}")
    # the same workspace serves a smaller Gumbel-max call next
    small = dict(CONFIGS[2], C=3, L=4, V=7001)
    d2 = gen_step(2, 10, cfg=small)
    dd2 = to_device(d2, small["dtype"])
    o2 = isd.verify_step(dd2["p"], dd2["q"], dd2["x"], dd2["ua"], dd2["ur"], sampler="gumbel",
                         ws=ws)
    torch.cuda.synchronize()
    assert not torch.nonzero(ws).numel()
    ref2 = oracle_step(d2, small["dtype"], "sample", small["T"], sampler="gumbel")
    compare(to_host(o2), ref2, propose=False, label="small gumbel verify")
    isd.check_device_error(ws)
