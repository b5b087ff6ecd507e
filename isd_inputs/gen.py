"""Seeded input generators for the five ISD workloads.

Every sequence of every step has its own generator, seeded with
``SeedSequence([0x15D, config, step, sequence])`` (PCG64), so any single
sequence can be regenerated on its own.  Logits are drawn in float32 and, for
bf16 workloads, rounded to bf16 with round-to-nearest-even; proposals are then
drawn from the *rounded* proposal logits, so the proposal distribution is
exactly the one the verifier sees.

The proposal tokens x ~ softmax(q/T) are drawn with the Gumbel-max trick
(argmax of q/T plus Gumbel noise), a sampler unrelated to the inverse-CDF draw
the step itself uses.

Workloads (C sequences, L strided positions, vocabulary V):

1. tiny:     C=1,   L=4,  V=1000,   fp32, p=N(0,2^2), q=p+N(0,0.5^2), T=1
2. serving:  C=64,  L=8,  V=151936, bf16, p=N(0,3^2), q=p+N(0,0.7^2), T=1
3. greedy:   C=64,  L=8,  V=151936, bf16, p=-1.1*ln(rank) under a random
             per-row permutation + N(0,0.3^2), q=p+N(0,1), x=argmax q
4. lm_head:  h [C*2L, 4096] ~ N(0,1), W [4096, V] ~ N(0,0.02^2), both bf16
5. high_concurrency: C=256, L=16, V=151936, bf16, p=N(0,5^2), q=p+N(0,0.3^2)

In every sampled workload the mask-position (next-proposal) logits qn use the
proposal construction on a fresh anchor draw, and the accept, residual and
proposal uniforms are float32 in [0, 1), one per position each.
"""

from __future__ import annotations

import numpy as np

SEED_BASE = 0x15D

CONFIGS = {
    1: dict(name="tiny", mode="sample", C=1, L=4, V=1000, dtype="f32", T=1.0,
            steps=100, sigma_p=2.0, sigma_q=0.5),
    2: dict(name="serving", mode="sample", C=64, L=8, V=151936, dtype="bf16", T=1.0,
            steps=1000, sigma_p=3.0, sigma_q=0.7),
    3: dict(name="greedy", mode="greedy", C=64, L=8, V=151936, dtype="bf16", T=1.0,
            steps=1000, zipf=1.1, sigma_p=0.3, sigma_q=1.0),
    4: dict(name="lm_head", mode="sample", C=64, L=8, V=151936, H=4096, dtype="bf16",
            T=1.0, steps=20, sigma_h=1.0, sigma_w=0.02),
    5: dict(name="high_concurrency", mode="sample", C=256, L=16, V=151936, dtype="bf16",
            T=1.0, steps=500, sigma_p=5.0, sigma_q=0.3),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """float32 values of bf16 bit patterns (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg_id: int, step: int, seq: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [SEED_BASE, int(cfg_id), int(step), int(seq)])))


def _encode(a32: np.ndarray, dtype: str):
    """(raw buffer, float64 view of the encoded values)."""
    if dtype == "bf16":
        raw = f32_to_bf16_bits(a32)
        return raw, bf16_bits_to_f32(raw).astype(np.float64)
    raw = np.ascontiguousarray(a32, dtype=np.float32)
    return raw, raw.astype(np.float64)


def _gumbel_argmax(logits64: np.ndarray, temperature: float, rng) -> np.ndarray:
    """One draw per row from softmax(logits/T) by the Gumbel-max trick."""
    u = rng.random(logits64.shape)
    u = np.clip(u, np.finfo(np.float64).tiny, 1.0 - np.finfo(np.float64).epsneg)
    g = -np.log(-np.log(u))
    return np.argmax(logits64 / temperature + g, axis=-1).astype(np.int32)


def _zipf_rows(rng, L: int, V: int, s: float) -> np.ndarray:
    """-s * ln(rank) under an independent random rank permutation per row."""
    out = np.empty((L, V), dtype=np.float32)
    base = np.arange(1, V + 1, dtype=np.float64)
    for k in range(L):
        out[k] = (-s * np.log(rng.permutation(base))).astype(np.float32)
    return out


def gen_sequence(cfg_id: int, step: int, seq: int, cfg: dict | None = None) -> dict:
    """Inputs of one sequence: p, q, qn [L, V] raw; x [L] int32; ua, ur, up [L]."""
    cfg = CONFIGS[cfg_id] if cfg is None else cfg
    L, V, dtype, T = cfg["L"], cfg["V"], cfg["dtype"], cfg["T"]
    rng = _rng(cfg_id, step, seq)
    if cfg["mode"] == "greedy":
        p32 = _zipf_rows(rng, L, V, cfg["zipf"])
        p32 += np.float32(cfg["sigma_p"]) * rng.standard_normal((L, V), dtype=np.float32)
        q32 = p32 + np.float32(cfg["sigma_q"]) * rng.standard_normal((L, V), dtype=np.float32)
        pn32 = _zipf_rows(rng, L, V, cfg["zipf"])
        pn32 += np.float32(cfg["sigma_p"]) * rng.standard_normal((L, V), dtype=np.float32)
        qn32 = pn32 + np.float32(cfg["sigma_q"]) * rng.standard_normal((L, V), dtype=np.float32)
        p, _ = _encode(p32, dtype)
        q, q64 = _encode(q32, dtype)
        qn, _ = _encode(qn32, dtype)
        x = np.argmax(q64, axis=-1).astype(np.int32)
    else:
        sp, sq = np.float32(cfg["sigma_p"]), np.float32(cfg["sigma_q"])
        p32 = sp * rng.standard_normal((L, V), dtype=np.float32)
        q32 = p32 + sq * rng.standard_normal((L, V), dtype=np.float32)
        pn32 = sp * rng.standard_normal((L, V), dtype=np.float32)
        qn32 = pn32 + sq * rng.standard_normal((L, V), dtype=np.float32)
        p, _ = _encode(p32, dtype)
        q, q64 = _encode(q32, dtype)
        qn, _ = _encode(qn32, dtype)
        x = _gumbel_argmax(q64, T, rng)
    u = rng.random((3, L), dtype=np.float32)
    return dict(p=p, q=q, qn=qn, x=x, ua=u[0].copy(), ur=u[1].copy(), up=u[2].copy())


def _gen_one(args):
    cfg_id, step, seq, cfg = args
    return gen_sequence(cfg_id, step, seq, cfg)


def gen_step(cfg_id: int, step: int, seqs=None, cfg: dict | None = None,
             workers: int = 1) -> dict:
    """Batched inputs of the sequences ``seqs`` (default all C) of one step.

    Returns p, q, qn [n, L, V] (uint16 bf16 bits or float32), x [n, L] int32
    and ua, ur, up [n, L] float32, plus ``seqs``.
    """
    cfg = CONFIGS[cfg_id] if cfg is None else cfg
    seqs = list(range(cfg["C"])) if seqs is None else list(seqs)
    n, L, V = len(seqs), cfg["L"], cfg["V"]
    ldt = np.uint16 if cfg["dtype"] == "bf16" else np.float32
    out = dict(p=np.empty((n, L, V), ldt), q=np.empty((n, L, V), ldt),
               qn=np.empty((n, L, V), ldt), x=np.empty((n, L), np.int32),
               ua=np.empty((n, L), np.float32), ur=np.empty((n, L), np.float32),
               up=np.empty((n, L), np.float32))
    jobs = [(cfg_id, step, s, cfg) for s in seqs]
    if workers > 1 and n > 1:
        import multiprocessing as mp
        # workers exit on their own (close/join): a terminate() would signal
        # them, which profilers that hook signals in forked children mishandle
        pool = mp.get_context("fork").Pool(workers)
        try:
            results = pool.imap(_gen_one, jobs, chunksize=max(1, n // (4 * workers)))
            for i, r in enumerate(results):
                for key in ("p", "q", "qn", "x", "ua", "ur", "up"):
                    out[key][i] = r[key]
        finally:
            pool.close()
            pool.join()
    else:
        for i, job in enumerate(jobs):
            r = _gen_one(job)
            for key in ("p", "q", "qn", "x", "ua", "ur", "up"):
                out[key][i] = r[key]
    out["seqs"] = np.asarray(seqs, dtype=np.int64)
    return out


def gen_head_weights(cfg_id: int = 4, cfg: dict | None = None) -> np.ndarray:
    """Shared LM-head weights W [H, V] as bf16 bits, from one fixed seed."""
    cfg = CONFIGS[cfg_id] if cfg is None else cfg
    rng = _rng(cfg_id, 0xFFFF, 0)
    H, V = cfg["H"], cfg["V"]
    w = np.empty((H, V), dtype=np.uint16)
    rows = 256
    for r0 in range(0, H, rows):
        r1 = min(H, r0 + rows)
        w[r0:r1] = f32_to_bf16_bits(np.float32(cfg["sigma_w"]) *
                                    rng.standard_normal((r1 - r0, V), dtype=np.float32))
    return w


def gen_hidden(cfg_id: int, step: int, cfg: dict | None = None) -> np.ndarray:
    """Hidden states h [C*2L, H] as bf16 bits: per sequence L verify rows then L mask rows."""
    cfg = CONFIGS[cfg_id] if cfg is None else cfg
    rng = _rng(cfg_id, step, 0xFFFE)
    M, H = cfg["C"] * 2 * cfg["L"], cfg["H"]
    return f32_to_bf16_bits(np.float32(cfg["sigma_h"]) *
                            rng.standard_normal((M, H), dtype=np.float32))


def gen_uniforms(cfg_id: int, steps: int, first_step: int = 0, cfg: dict | None = None) -> np.ndarray:
    """Fresh accept/residual/proposal uniforms for a run of steps that reuse a
    few resident logits sets: float32 [steps, 3, C, L] in [0, 1), seeded per
    step with SeedSequence([0x15D, config, step, 0xA11])."""
    cfg = CONFIGS[cfg_id] if cfg is None else cfg
    out = np.empty((steps, 3, cfg["C"], cfg["L"]), dtype=np.float32)
    for i in range(steps):
        rng = _rng(cfg_id, first_step + i, 0xA11)
        out[i] = rng.random((3, cfg["C"], cfg["L"]), dtype=np.float32)
    return out


def host_bytes_per_step(cfg_id: int, cfg: dict | None = None) -> int:
    """Bytes of the three logits tensors of one step."""
    cfg = CONFIGS[cfg_id] if cfg is None else cfg
    es = 2 if cfg["dtype"] == "bf16" else 4
    return 3 * cfg["C"] * cfg["L"] * cfg["V"] * es
