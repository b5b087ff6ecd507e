"""Seeded inputs of the segment-gated LoRA projection.

The residual variant of ISD applies a low-rank adapter only at the mask
positions of an extend forward ("Introspective Diffusion Language Models |
Summary", section 3.2 and appendix G).  The workload is one projection of such
a forward: x [M, K] holds, per sequence, L clean/anchor rows then L mask rows
(M = C * 2L); W [N, K] is the base weight, A [r, K] and B [N, r] the adapter,
all in the torch Linear layout (output features first).  Values are drawn in
float32 and rounded to bf16 (round to nearest even):

    x ~ N(0, 1),  W ~ N(0, 0.02^2),  A ~ N(0, 1/K),  B ~ N(0, 0.02^2)

B is drawn non-zero (a trained adapter, not one at initialisation), so the
adapter term is of the same order as a base term's spread.  The mask is 1 on
the mask rows.  Each tensor has its own generator,
``SeedSequence([0x15D, 7, seed, role])``.
"""

from __future__ import annotations

import numpy as np

from .gen import f32_to_bf16_bits

SEED_BASE = 0x15D
WORKLOAD = 7

# roles of the per-tensor generators
_X, _W, _A, _B = 0, 1, 2, 3

LORA_CONFIGS = {
    # an 8B model's fused MLP gate/up projection at the serving batch, rank-128 adapter
    "mlp_up": dict(C=64, L=8, K=4096, N=24576, r=128),
    # midsize parity case: several tiles in every dimension, ragged M and N
    "mid": dict(C=5, L=10, K=512, N=1000, r=64),
}


def _rng(seed: int, role: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [SEED_BASE, WORKLOAD, int(seed), int(role)])))


def _bf16(rng, shape, sigma) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    rows = max(1, (1 << 22) // max(1, shape[1]))
    for r0 in range(0, shape[0], rows):
        r1 = min(shape[0], r0 + rows)
        out[r0:r1] = f32_to_bf16_bits(np.float32(sigma) *
                                      rng.standard_normal((r1 - r0, shape[1]), dtype=np.float32))
    return out


def extend_mask(C: int, L: int) -> np.ndarray:
    """int32 [C * 2L]: 0 on the L clean rows, 1 on the L mask rows of each sequence."""
    return np.tile(np.r_[np.zeros(L, np.int32), np.ones(L, np.int32)], C)


def gen_lora(cfg: dict, seed: int = 0, weights: bool = True) -> dict:
    """x, (W, A, B) as bf16 bits and the mask; ``weights=False`` skips the weights."""
    C, L, K, N, r = cfg["C"], cfg["L"], cfg["K"], cfg["N"], cfg["r"]
    M = C * 2 * L
    out = dict(x=_bf16(_rng(seed, _X), (M, K), 1.0), mask=extend_mask(C, L))
    if weights:
        out["w"] = _bf16(_rng(0, _W), (N, K), 0.02)
        out["a"] = _bf16(_rng(0, _A), (r, K), 1.0 / np.sqrt(K))
        out["b"] = _bf16(_rng(0, _B), (N, r), 0.02)
    return out


def gen_exact_head(M: int, K: int, N: int, seed: int = 0, which: str = "both") -> dict:
    """Hidden states and head weights whose products are exact in fp32: h in
    {-1, 0, 1} and W = k / 128 with integer k in [-16, 16], so every partial
    sum of a row is a multiple of 2^-7 below 2^9 (K <= 4096).  The bf16 logits
    are then the round-to-nearest-even of the exact product on any
    implementation.  wt is [N, K] (k-contiguous); bf16 bits."""
    out = {}
    if which in ("both", "h"):
        rng = _rng(seed, 10)
        out["h"] = f32_to_bf16_bits(rng.integers(-1, 2, size=(M, K)).astype(np.float32))
    if which in ("both", "w"):
        rng = _rng(0, 11)
        wt = np.empty((N, K), dtype=np.uint16)
        rows = max(1, (1 << 22) // K)
        for r0 in range(0, N, rows):
            r1 = min(N, r0 + rows)
            wt[r0:r1] = f32_to_bf16_bits(rng.integers(-16, 17, size=(r1 - r0, K)).astype(np.float32) / 128.0)
        out["wt"] = wt
    return out
