"""Seeded inputs for the multi-step decoding loop with a set acceptance rate.

Each verify position's pair of rows is built so that the anchor P and the
proposal law Q overlap by exactly ``a``: P lives on a random half A of the
vocabulary, a second law D on the other half B, and Q = a * P + (1 - a) * D.
Then sum_i min(P_i, Q_i) = a, which is the probability that a proposal drawn
from Q passes the accept test, so every position accepts with probability a
independently of the others.  Logits are float32 (log of the normalised
laws; -inf off the support).

Steps chain like a model's forward passes: the mask rows ``qn`` of step t are
the proposal rows ``q`` of step t + 1, so ``pair(t + 1)`` is drawn at step t.
Each (step, role, sequence) has its own generator,
``SeedSequence([0x15D, 6, step, role, sequence])``.
"""

from __future__ import annotations

import numpy as np

SEED_BASE = 0x15D
WORKLOAD = 6

# roles of the per-step generators
_PAIR, _ANCHOR, _UNIFORMS = 0, 1, 2

DECODE_CONFIGS = {
    # CPU Monte Carlo of the loop (oracle only)
    "cpu_mc": dict(C=16, L=3, V=64, a=0.7, sigma=1.5, T=1.0, steps=400),
    # GPU parity of the chained loop
    "gpu_chain": dict(C=16, L=4, V=5000, a=0.75, sigma=2.0, T=1.0, steps=24),
    # GPU Monte Carlo of tokens per forward, stride N = L + 1 = 8
    "gpu_tpf": dict(C=64, L=7, V=4096, a=0.8, sigma=2.0, T=1.0, steps=100),
}


def _rng(step: int, role: int, seq: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [SEED_BASE, WORKLOAD, int(step), int(role), int(seq)])))


def _log_normalised(logits64: np.ndarray, support: np.ndarray) -> np.ndarray:
    """log of softmax over `support` (float64), -inf elsewhere."""
    out = np.full(logits64.shape, -np.inf)
    z = logits64[support]
    z = z - z.max()
    out[support] = z - np.log(np.exp(z).sum())
    return out


_pair_cache: dict = {}


def pair(step: int, cfg: dict):
    """(P logits, Q logits) of the verify positions of `step`: float32 [C, L, V].
    The last few pairs are kept, since consecutive steps share one."""
    key = (int(step),) + tuple(sorted((k, cfg[k]) for k in ("C", "L", "V", "a", "sigma")))
    hit = _pair_cache.get(key)
    if hit is None:
        hit = _make_pair(step, cfg)
        if len(_pair_cache) >= 4:
            _pair_cache.pop(next(iter(_pair_cache)))
        _pair_cache[key] = hit
    return hit[0].copy(), hit[1].copy()


def _make_pair(step: int, cfg: dict):
    C, L, V, a, s = cfg["C"], cfg["L"], cfg["V"], cfg["a"], cfg["sigma"]
    P = np.empty((C, L, V), dtype=np.float32)
    Q = np.empty((C, L, V), dtype=np.float32)
    for c in range(C):
        rng = _rng(step, _PAIR, c)
        for k in range(L):
            A = np.zeros(V, dtype=bool)
            A[rng.permutation(V)[: V // 2]] = True
            lp = _log_normalised(s * rng.standard_normal(V), A)
            ld = _log_normalised(s * rng.standard_normal(V), ~A)
            with np.errstate(divide="ignore"):
                lq = np.log(a * np.exp(lp) + (1.0 - a) * np.exp(ld))
            P[c, k] = lp.astype(np.float32)
            Q[c, k] = lq.astype(np.float32)
    return P, Q


def decode_step_inputs(step: int, cfg: dict) -> dict:
    """Inputs of one step of the loop, except the pending proposals x (which
    the previous step draws):

    p [C, L+1, V]: rows 0..L-1 are this step's anchors P; row L is a fresh
        anchor row for the bonus draw (row 0 also serves recovering sequences);
    q [C, L, V]: this step's proposal rows Q (the previous step's qn);
    qn [C, L, V]: the next step's proposal rows;
    ua, ur, up [C, L] and ub, uz [C]: float32 uniforms in [0, 1).
    """
    C, L, V, s = cfg["C"], cfg["L"], cfg["V"], cfg["sigma"]
    P, Q = pair(step, cfg)
    _, Qn = pair(step + 1, cfg)
    p = np.empty((C, L + 1, V), dtype=np.float32)
    p[:, :L] = P
    u = np.empty((C, 3 * L + 2), dtype=np.float32)
    for c in range(C):
        p[c, L] = (s * _rng(step, _ANCHOR, c).standard_normal(V)).astype(np.float32)
        u[c] = _rng(step, _UNIFORMS, c).random(3 * L + 2, dtype=np.float32)
    return dict(p=p, q=Q, qn=Qn, ua=u[:, :L].copy(), ur=u[:, L:2 * L].copy(),
                up=u[:, 2 * L:3 * L].copy(), ub=u[:, 3 * L].copy(), uz=u[:, 3 * L + 1].copy())
