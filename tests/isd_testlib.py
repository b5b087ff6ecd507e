"""Shared helpers of the GPU parity tests: upload seeded inputs, run the CPU
oracle on the same bytes, and compare under the tolerance rule.

Tolerance rule (probabilities and decisions):
* p_x, q_x, alpha, qnext_x: relative error <= 1e-5 against the fp64 oracle;
* accept_len, out_tokens, n_emitted, next_tokens: identical, except for the
  decisions the oracle flags as near ties: a sequence whose accept decision
  (some k <= j) has |ua - r| < 1e-6, and a drawn token whose uniform lies
  within 1e-6 of one of its two cumulative boundaries (oracle values).
* a flagged case is not skipped: the GPU's choice must be one the oracle's
  own numbers allow within a small tolerance (``DECISION_TOL`` for an accept
  test, ``DRAW_TOL`` on the cumulative weight for an inverse-CDF draw,
  ``GUMBEL_TOL`` on the score for a Gumbel-max draw), and a drawn token must
  carry positive weight.  Every flagged case is counted and reported.
* greedy mode: everything identical, no exclusions.
"""

from __future__ import annotations

import os
import sys

import numpy as np

from oracle import isd_oracle as O

RTOL = 1e-5
ATOL_PROB = 1e-30
# Validity windows of flagged cases.  The kernels' ratios carry ~1e-7
# relative error and their cumulative weights ~1e-7 * P_max / Z, so a
# flagged choice that is still correct lies far inside these.
DECISION_TOL = 1e-6
DRAW_TOL = 1e-5
GUMBEL_TOL = 2 * O.GUMBEL_WINDOW


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


def _oracle_chunk(job):
    d, sl, dtype, mode, T, relax, q_onehot, sampler, top_k, top_p, ids = job
    os.environ["OMP_NUM_THREADS"] = "1"
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
                            q_onehot=q_onehot, sampler=sampler, seq_ids=ids[sl],
                            top_k=top_k, top_p=top_p)
        tok, prob, _, pflag = O.propose_sample(qn, d["up"][sl], T, top_k=top_k, top_p=top_p)
    return dict(accept_len=v["accept_len"], out_tokens=v["out_tokens"],
                n_emitted=v["n_emitted"], p_x=v["p_x"], q_x=v["q_x"], alpha=v["alpha"],
                flagged=v["flagged"], resid_flagged=v["resid_flagged"], next_tokens=tok,
                qnext_x=prob, next_flagged=pflag)


_POOL_INPUT = {}


def _oracle_chunk_shared(args):
    sl, rest = args
    return _oracle_chunk((_POOL_INPUT["d"], sl) + rest)


def oracle_step(d: dict, dtype: str, mode: str, T: float, chunk: int = 8, relax: float = 0.0,
                q_onehot: bool = False, sampler: str = "cdf", top_k: int = 0,
                top_p: float = 1.0, seq_ids=None, workers: int = 1) -> dict:
    """Oracle outputs for every sequence in d (chunked to bound memory, over
    `workers` forked processes when > 1); relax, q_onehot, sampler and
    top_k / top_p select the verification variants (sample mode).  The
    Gumbel-max key takes each sequence's index in the whole call (seq_ids,
    default 0..C-1).  The result carries the inputs and options under
    "_ctx", which compare() uses to validate flagged cases."""
    n = d["x"].shape[0]
    ids = np.arange(n) if seq_ids is None else np.asarray(seq_ids)
    rest = (dtype, mode, T, relax, q_onehot, sampler, top_k, top_p, ids)
    slices = [slice(s0, min(n, s0 + chunk)) for s0 in range(0, n, chunk)]
    if workers > 1 and len(slices) > 1:
        import multiprocessing as mp
        _POOL_INPUT["d"] = d
        pool = mp.get_context("fork").Pool(min(workers, len(slices)))
        try:
            parts = pool.map(_oracle_chunk_shared, [(sl, rest) for sl in slices], chunksize=1)
        finally:
            pool.close()
            pool.join()
            _POOL_INPUT.clear()
    else:
        parts = [_oracle_chunk((d, sl) + rest) for sl in slices]
    ref = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    ref["_ctx"] = dict(d=d, dtype=dtype, mode=mode, T=T, relax=relax, q_onehot=q_onehot,
                       sampler=sampler, top_k=top_k, top_p=top_p, seq_ids=ids)
    return ref


# ---------------------------------------------------------------------------
# Validity of flagged cases
# ---------------------------------------------------------------------------

def _draw_valid(w, u, tok) -> bool:
    """An inverse-CDF draw of `tok` with uniform u is valid if tok carries
    weight and u lies within DRAW_TOL of its cumulative interval."""
    if not 0 <= tok < w.size or not w[tok] > 0:
        return False
    lo, hi = O.cdf_interval(w, int(tok))
    return lo - DRAW_TOL <= u <= hi + DRAW_TOL


def _gumbel_valid(w, key0, key1, j, tok) -> bool:
    if not 0 <= tok < w.size or not w[tok] > 0:
        return False
    g = O.gumbel_noise(key0, key1, j, w.size)
    with np.errstate(divide="ignore"):
        score = np.where(w > 0, np.log(w), -np.inf) + g
    return score[tok] >= score.max() - GUMBEL_TOL


def _laws(ctx, c):
    """P [L, V], Q [L, V] (None rows for one-hot q) and the top-p margin of
    sequence c, from the oracle's own functions."""
    d, dt, T = ctx["d"], ctx["dtype"], ctx["T"]
    p = O.decode_logits(d["p"][c], dt)
    P, mp = O.sampling_law(p, T, ctx["top_k"], ctx["top_p"])
    margin = float(np.min(mp))
    if ctx["q_onehot"]:
        Q = np.zeros_like(P)
        Q[np.arange(P.shape[0]), d["x"][c]] = 1.0
    else:
        Q, mq = O.sampling_law(O.decode_logits(d["q"][c], dt), T, ctx["top_k"], ctx["top_p"])
        margin = min(margin, float(np.min(mq)))
    return P, Q, margin


def _validate_sequence(g, ctx, c, label):
    """The GPU's decisions and correction for sequence c against the oracle's
    own ratios and residual weights (a flagged sequence); returns False when
    the sequence's truncated laws are themselves at a cut boundary."""
    d = ctx["d"]
    L = d["x"].shape[1]
    P, Q, margin = _laws(ctx, c)
    if margin < O.TRUNC_WINDOW:
        return False
    x = d["x"][c].astype(np.int64)
    px, qx = P[np.arange(L), x], Q[np.arange(L), x]
    r = O.accept_ratio((1.0 + ctx["relax"]) * px, qx)
    j = int(g["accept_len"][c])
    ua = d["ua"][c].astype(np.float64)
    assert 0 <= j <= L, f"{label} seq {c}: accept_len {j}"
    for k in range(j):
        assert ua[k] < r[k] + DECISION_TOL, f"{label} seq {c}: kept x_{k} with u={ua[k]} r={r[k]}"
    if j < L:
        assert ua[j] >= r[j] - DECISION_TOL, f"{label} seq {c}: rejected x_{j} with u={ua[j]} r={r[j]}"
    assert g["n_emitted"][c] == j + (j < L), f"{label} seq {c}: n_emitted"
    np.testing.assert_array_equal(g["out_tokens"][c][:j], x[:j], err_msg=f"{label} seq {c} prefix")
    assert np.all(g["out_tokens"][c][j + 1:] == -1), f"{label} seq {c}: padding"
    if j < L:
        _validate_correction(g, ctx, c, j, P[j], Q[j], label)
    return True


def _validate_correction(g, ctx, c, j, Pj, Qj, label):
    W, _ = O.residual_weights(Pj, Qj)
    tok = int(g["out_tokens"][c][j])
    u = float(ctx["d"]["ur"][c, j])
    if ctx["sampler"] == "gumbel":
        bits = np.asarray(ctx["d"]["ur"][c, j], dtype=np.float32).view(np.uint32)
        ok = _gumbel_valid(W, int(bits), int(ctx["seq_ids"][c]), j, tok)
    else:
        ok = _draw_valid(W, u, tok)
    assert ok, f"{label} seq {c}: correction {tok} at j={j} is not a valid draw for u={u}"


def _validate_proposal(g, ctx, c, k, label):
    d = ctx["d"]
    qn = O.decode_logits(d["qn"][c, k], ctx["dtype"])
    Qn, _ = O.sampling_law(qn, ctx["T"], ctx["top_k"], ctx["top_p"])
    tok = int(g["next_tokens"][c, k])
    u = float(d["up"][c, k])
    assert _draw_valid(Qn, u, tok), f"{label} proposal ({c}, {k}): {tok} invalid for u={u}"


def compare(gpu: dict, ref: dict, *, verify=True, propose=True, label="") -> dict:
    """Asserts the tolerance rule; returns counts of comparisons and of the
    flagged cases (each validated when the oracle's inputs are attached)."""
    ctx = ref.get("_ctx")
    stats = dict(sequences=0, decision_flags=0, resid_flags=0, propose_flags=0, positions=0,
                 validated=0)
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
                if ctx is not None:
                    P, Q, _ = _laws(ctx, c)
                    _validate_correction(gpu, ctx, c, int(j[c]), P[j[c]], Q[j[c]], label)
                    stats["validated"] += 1
            else:
                assert np.array_equal(g, r), f"{label} out_tokens seq {c}: gpu {g} oracle {r}"
        if ctx is not None:
            for c in np.nonzero(~ok)[0]:
                stats["validated"] += int(_validate_sequence(gpu, ctx, c, label))
    if propose:
        okp = ~ref["next_flagged"]
        stats["propose_flags"] = int((~okp).sum())
        bad = np.argwhere(okp & (gpu["next_tokens"] != ref["next_tokens"]))
        assert bad.size == 0, f"{label} next_tokens differ at {bad[:10].tolist()}: gpu " \
                              f"{gpu['next_tokens'][tuple(bad[:10].T)]} oracle " \
                              f"{ref['next_tokens'][tuple(bad[:10].T)]}"
        np.testing.assert_allclose(gpu["qnext_x"][okp], ref["qnext_x"][okp], rtol=RTOL,
                                   atol=ATOL_PROB, err_msg=f"{label} qnext_x")
        if ctx is not None and ctx["mode"] != "greedy":
            for c, k in np.argwhere(~okp):
                _validate_proposal(gpu, ctx, int(c), int(k), label)
                stats["validated"] += 1
    return stats
