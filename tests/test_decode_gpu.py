"""GPU parity of the multi-step decoding loop (masked step, bonus and anchor
draws, device ledger) against the loop oracle, and its tokens per forward
against the closed form ("Introspective Diffusion Language Models | Summary",
section 3.2 and appendix B)."""

import numpy as np
import pytest

from isd_inputs import CONFIGS, gen_step
from isd_inputs.decode import DECODE_CONFIGS, decode_step_inputs
from oracle import isd_decode as D
from tests.isd_testlib import log, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def isd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import speculative_verification_amd as isd_mod
    isd_mod.lib()
    return isd_mod


def _dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


@pytest.mark.parametrize("mode", ["sample", "greedy"])
def test_masked_step(isd, mode):
    """Active sequences get exactly the unmasked results; masked-out ones get
    the idle outputs and leave the workspace clean."""
    import torch
    cfg_id = 2 if mode == "sample" else 3
    cfg = dict(CONFIGS[cfg_id], C=8, L=8, V=10000)
    d = gen_step(cfg_id, 77, cfg=cfg)
    dd = to_device(d, cfg["dtype"])
    args = (dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"])
    full = to_host(isd.step(*args, mode=mode, temperature=cfg["T"]))
    vmask = np.array([1, 0, 1, 1, 0, 0, 1, 0], dtype=np.int32)
    pmask = np.array([0, 1, 1, 0, 1, 0, 1, 1], dtype=np.int32)
    for rep in range(3):
        o = isd.step_masked(*args, _dev(vmask), _dev(pmask), mode=mode, temperature=cfg["T"])
        torch.cuda.synchronize()
        h = to_host(o)
        on, off = vmask == 1, vmask == 0
        for key in ("accept_len", "n_emitted", "out_tokens", "p_x", "q_x", "alpha"):
            np.testing.assert_array_equal(h[key][on], full[key][on], err_msg=key)
        assert np.all(h["accept_len"][off] == -1) and np.all(h["n_emitted"][off] == 0)
        assert np.all(h["out_tokens"][off] == -1)
        assert np.all(h["p_x"][off] == 0) and np.all(h["alpha"][off] == 0)
        pon, poff = pmask == 1, pmask == 0
        np.testing.assert_array_equal(h["next_tokens"][pon], full["next_tokens"][pon])
        assert np.all(h["next_tokens"][poff] == -1) and np.all(h["qnext_x"][poff] == 0)
    # the unmasked step still agrees after masked launches on the same workspace
    again = to_host(isd.step(*args, mode=mode, temperature=cfg["T"]))
    for key in full:
        np.testing.assert_array_equal(again[key], full[key], err_msg=key)
    for key, ws in list(isd.isd._ws_cache.items()):
        isd.check_device_error(ws)


def _loop_buffers(cfg):
    """Device buffers of one layout [C, L+1, V] for p, q and qn."""
    import torch
    C, L, V = cfg["C"], cfg["L"], cfg["V"]
    z = lambda: torch.zeros((C, L + 1, V), dtype=torch.float32, device="cuda")  # noqa: E731
    return z(), z(), z()


def _run_gpu_loop(isd, cfg, steps, *, check_oracle, history=0):
    import torch
    C, L, V, T = cfg["C"], cfg["L"], cfg["V"], cfg["T"]
    dec = isd.Decoder(C, L, "cuda", history=history, temperature=T)
    p_b, q_b, qn_b = _loop_buffers(cfg)
    oracle_hist = [[] for _ in range(C)]
    stats = dict(flags=0)
    for t in range(steps):
        d = decode_step_inputs(t, cfg)
        p_b.copy_(torch.from_numpy(d["p"]))
        q_b[:, :L].copy_(torch.from_numpy(d["q"]))
        qn_b[:, :L].copy_(torch.from_numpy(d["qn"]))
        x_before = dec.x.cpu().numpy().astype(np.int64)
        state_before = dec.state.cpu().numpy()
        o = dec.step(p_b, q_b, qn_b, _dev(d["ua"]), _dev(d["ur"]), _dev(d["up"]), _dev(d["ub"]),
                     _dev(d["uz"]))
        if not check_oracle:
            continue
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in o.items()}
        r = D.decode_step(state_before, d["p"].astype(np.float64), d["q"].astype(np.float64),
                          x_before, d["ua"], d["ur"], d["qn"].astype(np.float64), d["up"],
                          d["ub"], d["uz"], T)
        ok = ~r["flagged"]
        stats["flags"] += int((~ok).sum())
        np.testing.assert_array_equal(g["accept_len"][ok], r["accept_len"][ok], err_msg=f"step {t}")
        for c in np.nonzero(ok & ~r["resid_flagged"])[0]:
            np.testing.assert_array_equal(g["out_tokens"][c], r["out_tokens"][c],
                                          err_msg=f"step {t} seq {c}")
        okb = ok & ~r["bonus_flagged"]
        np.testing.assert_array_equal(g["bonus"][okb], r["bonus"][okb], err_msg=f"step {t} bonus")
        oka = ~r["anchor_flagged"]
        np.testing.assert_array_equal(g["anchor"][oka], r["anchor"][oka], err_msg=f"step {t} anchor")
        okn = ~r["next_flagged"]
        np.testing.assert_array_equal(g["next_tokens"][okn], r["next_tokens"][okn],
                                      err_msg=f"step {t} next")
        np.testing.assert_array_equal(dec.state.cpu().numpy()[ok], r["next_state"][ok],
                                      err_msg=f"step {t} state")
        # what each sequence emitted this step: the oracle's tokens, or the
        # GPU's where the oracle flagged a near tie (those were left out of
        # the comparisons above), so the ledger is checked end to end always
        for c in range(C):
            flagged = (not ok[c]) or r["resid_flagged"][c] or r["bonus_flagged"][c] or \
                r["anchor_flagged"][c]
            src = g if flagged else r
            if state_before[c] == D.VERIFY:
                j = int(src["accept_len"][c])
                emitted = list(src["out_tokens"][c, : min(j + 1, L)]) + \
                    ([int(src["bonus"][c])] if j == L else [])
            else:
                emitted = [int(src["anchor"][c])]
            if not flagged:
                assert len(emitted) == r["emitted"][c]
            oracle_hist[c] += [int(v) for v in emitted]
    torch.cuda.synchronize()
    return dec, oracle_hist, stats


def test_decoder_chain_matches_oracle(isd):
    cfg = DECODE_CONFIGS["gpu_chain"]
    steps = cfg["steps"]
    cap = steps * (cfg["L"] + 1)
    dec, oracle_hist, stats = _run_gpu_loop(isd, cfg, steps, check_oracle=True, history=cap)
    tokens = dec.tokens.cpu().numpy()
    hist = dec.history.cpu().numpy()
    assert np.all(dec.forwards.cpu().numpy() == steps)
    for c in range(cfg["C"]):
        assert tokens[c] == len(oracle_hist[c])
        np.testing.assert_array_equal(hist[c, : tokens[c]], oracle_hist[c])
    log(f"decode chain: {steps} steps x {cfg['C']} sequences, tokens per sequence "
        f"{tokens.tolist()}, flags {stats['flags']}")
    for key, ws in list(isd.isd._ws_cache.items()):
        isd.check_device_error(ws)


def test_decoder_tokens_per_forward(isd):
    """Uniform acceptance a at stride N = L + 1: the measured tokens per
    forward agree with (2 + a + ... + a^(N-2)) / (2 - a^(N-1))."""
    cfg = DECODE_CONFIGS["gpu_tpf"]
    dec, _, _ = _run_gpu_loop(isd, cfg, cfg["steps"], check_oracle=False)
    tokens = dec.tokens.cpu().numpy().astype(np.float64)
    forwards = dec.forwards.cpu().numpy().astype(np.float64)
    per_seq = tokens / forwards
    tpf = tokens.sum() / forwards.sum()
    sem = per_seq.std(ddof=1) / np.sqrt(len(per_seq))
    expect = D.tpf_closed_form(cfg["a"], cfg["L"] + 1)
    log(f"tokens per forward: measured {tpf:.4f} +- {sem:.4f}, closed form {expect:.4f} "
        f"(a={cfg['a']}, N={cfg['L'] + 1}, {int(forwards.sum())} forwards)")
    # the loop starts in recovery: allow the one-step transient on top of 4 sigma
    assert abs(tpf - expect) < 4 * sem + expect / cfg["steps"]
    for key, ws in list(isd.isd._ws_cache.items()):
        isd.check_device_error(ws)
