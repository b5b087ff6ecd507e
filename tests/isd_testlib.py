"""Shared helpers of the GPU parity tests: upload seeded inputs, run the CPU
oracle on the same bytes, and compare under the tolerance rule.

Tolerance rule (probabilities and decisions):
* p_x, q_x, alpha, qnext_x: relative error <= 1e-5 against the fp64 oracle;
* accept_len, out_tokens, n_emitted, next_tokens: identical, except that a
  sequence whose accept decision (some k <= j) has |ua - r| < 1e-6 is left
  out of the token comparison, and so is a drawn token whose uniform lies
  within 1e-6 of one of its two cumulative boundaries (oracle values).
  Every such exclusion is counted and reported.
* greedy mode: everything identical, no exclusions.
"""

from __future__ import annotations

import sys

import numpy as np

from oracle import isd_oracle as O

RTOL = 1e-5
ATOL_PROB = 1e-30


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(d: dict, dtype: str):
    """Upload generator output (numpy) as torch device tensors."""
    import torch
    dev = torch.device("cuda", 0)
    out = {}
    for key in ("p", "q", "qn"):
        a = d[key]
        if dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        out[key] = t
    for key in ("x",):
        out[key] = torch.from_numpy(np.ascontiguousarray(d[key])).to(dev)
    for key in ("ua", "ur", "up"):
        out[key] = torch.from_numpy(np.ascontiguousarray(d[key])).to(dev)
    return out


def to_host(o: dict) -> dict:
    return {k: v.detach().cpu().numpy() for k, v in o.items()}


def oracle_step(d: dict, dtype: str, mode: str, T: float, chunk: int = 8, relax: float = 0.0,
                q_onehot: bool = False, sampler: str = "cdf") -> dict:
    """Oracle outputs for every sequence in d (chunked to bound memory);
    relax, q_onehot and sampler select the verification variants (sample
    mode).  The Gumbel-max key takes each sequence's index in the whole call."""
    n = d["x"].shape[0]
    parts = []
    for s0 in range(0, n, chunk):
        sl = slice(s0, min(n, s0 + chunk))
        p = O.decode_logits(d["p"][sl], dtype)
        qn = O.decode_logits(d["qn"][sl], dtype)
        if mode == "greedy":
            v = O.verify_greedy(p, d["x"][sl])
            g = v["argmax"]
            match = d["x"][sl] == g
            v["p_x"] = match.astype(np.float64)
            v["q_x"] = np.ones_like(v["p_x"])
            v["flagged"] = np.zeros(match.shape[0], bool)
            v["resid_flagged"] = np.zeros(match.shape[0], bool)
            tok = O.propose_greedy(qn)
            prob = np.ones(tok.shape)
            pflag = np.zeros(tok.shape, bool)
        else:
            q = None if q_onehot else O.decode_logits(d["q"][sl], dtype)
            v = O.verify_sample(p, q, d["x"][sl], d["ua"][sl], d["ur"][sl], T, relax=relax,
                                q_onehot=q_onehot, sampler=sampler,
                                seq_ids=np.arange(sl.start, sl.stop))
            tok, prob, _, pflag = O.propose_sample(qn, d["up"][sl], T)
        parts.append(dict(accept_len=v["accept_len"], out_tokens=v["out_tokens"],
                          n_emitted=v["n_emitted"], p_x=v["p_x"], q_x=v["q_x"],
                          alpha=v["alpha"], flagged=v["flagged"],
                          resid_flagged=v["resid_flagged"], next_tokens=tok,
                          qnext_x=prob, next_flagged=pflag))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def compare(gpu: dict, ref: dict, *, verify=True, propose=True, label="") -> dict:
    """Asserts the tolerance rule; returns counts of comparisons and exclusions."""
    stats = dict(sequences=0, decision_flags=0, resid_flags=0, propose_flags=0, positions=0)
    if verify:
        C, L = ref["out_tokens"].shape
        stats["sequences"] = C
        stats["positions"] = C * L
        np.testing.assert_allclose(gpu["p_x"], ref["p_x"], rtol=RTOL, atol=ATOL_PROB,
                                   err_msg=f"{label} p_x")
        np.testing.assert_allclose(gpu["q_x"], ref["q_x"], rtol=RTOL, atol=ATOL_PROB,
                                   err_msg=f"{label} q_x")
        np.testing.assert_allclose(gpu["alpha"], ref["alpha"], rtol=RTOL, atol=0,
                                   err_msg=f"{label} alpha")
        ok = ~ref["flagged"]
        stats["decision_flags"] = int((~ok).sum())
        for key in ("accept_len", "n_emitted"):
            bad = np.nonzero(ok & (gpu[key] != ref[key]))[0]
            assert bad.size == 0, f"{label} {key} differs at sequences {bad[:10]}: " \
                                  f"gpu {gpu[key][bad[:10]]} oracle {ref[key][bad[:10]]}"
        j = ref["accept_len"]
        for c in np.nonzero(ok)[0]:
            g, r = gpu["out_tokens"][c], ref["out_tokens"][c]
            if j[c] < L and ref["resid_flagged"][c]:
                stats["resid_flags"] += 1
                keep = np.arange(L) != j[c]
                assert np.array_equal(g[keep], r[keep]), f"{label} out_tokens seq {c}: {g} vs {r}"
            else:
                assert np.array_equal(g, r), f"{label} out_tokens seq {c}: gpu {g} oracle {r}"
    if propose:
        okp = ~ref["next_flagged"]
        stats["propose_flags"] = int((~okp).sum())
        bad = np.argwhere(okp & (gpu["next_tokens"] != ref["next_tokens"]))
        assert bad.size == 0, f"{label} next_tokens differ at {bad[:10].tolist()}: gpu " \
                              f"{gpu['next_tokens'][tuple(bad[:10].T)]} oracle " \
                              f"{ref['next_tokens'][tuple(bad[:10].T)]}"
        np.testing.assert_allclose(gpu["qnext_x"][okp], ref["qnext_x"][okp], rtol=RTOL,
                                   atol=ATOL_PROB, err_msg=f"{label} qnext_x")
    return stats
