"""The seeded input generators: reproducibility, shapes, bf16 rounding and the
proposal sampler.  Workload statistics are measured and printed, not asserted
against any prose description of the workloads."""

import numpy as np
import pytest
from scipy import special, stats

from isd_inputs import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, gen_sequence, gen_step
from isd_inputs import gen as G


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                     -2.5, np.inf, -np.inf, 0.0, -0.0, 3.0e38], dtype=np.float32)
    bits = f32_to_bf16_bits(vals)
    back = bf16_bits_to_f32(bits)
    assert back[0] == one
    assert back[1] == one                    # exact tie rounds to even mantissa (1.0)
    assert back[2] == one + 2 * ulp          # tie between 1+ulp (odd) and 1+2ulp (even)
    assert back[3] == one + ulp              # just above the tie rounds up
    assert back[4] == -2.5
    assert np.isposinf(back[5]) and np.isneginf(back[6])
    assert bits[7] == 0x0000 and bits[8] == 0x8000
    assert np.isfinite(back[9]) or np.isposinf(back[9])


def test_bf16_rounding_error_bound(rng):
    a = rng.normal(0, 3, 100_000).astype(np.float32)
    back = bf16_bits_to_f32(f32_to_bf16_bits(a)).astype(np.float64)
    rel = np.abs(back - a) / np.abs(a)
    assert rel.max() <= 2.0 ** -8 * (1 + 1e-6)   # 8 significant bits: half-ulp <= 2^-8 relative


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 5])
def test_sequence_reproducible_and_shaped(cfg_id):
    cfg = CONFIGS[cfg_id]
    a = gen_sequence(cfg_id, 3, 1)
    b = gen_sequence(cfg_id, 3, 1)
    c = gen_sequence(cfg_id, 4, 1)
    L, V = cfg["L"], cfg["V"]
    ldt = np.uint16 if cfg["dtype"] == "bf16" else np.float32
    for key in ("p", "q", "qn"):
        assert a[key].shape == (L, V) and a[key].dtype == ldt
        np.testing.assert_array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])
    assert a["x"].shape == (L,) and a["x"].dtype == np.int32
    assert np.all((a["x"] >= 0) & (a["x"] < V))
    for key in ("ua", "ur", "up"):
        assert a[key].shape == (L,) and a[key].dtype == np.float32
        assert np.all((a[key] >= 0) & (a[key] < 1))


def test_gen_step_matches_per_sequence_and_pool():
    d1 = gen_step(2, 0, seqs=[5, 9])
    d2 = gen_step(2, 0, seqs=[5, 9], workers=2)
    s9 = gen_sequence(2, 0, 9)
    for key in ("p", "q", "qn", "x", "ua", "ur", "up"):
        np.testing.assert_array_equal(d1[key], d2[key])
        np.testing.assert_array_equal(d1[key][1], s9[key])


def test_greedy_proposals_are_argmax_of_rounded_q():
    s = gen_sequence(3, 0, 0)
    q = bf16_bits_to_f32(s["q"]).astype(np.float64)
    np.testing.assert_array_equal(s["x"], np.argmax(q, axis=-1))


def test_gumbel_proposals_follow_softmax():
    """The proposal sampler draws from softmax(q/T) (chi-square, tiny V)."""
    cfg = dict(CONFIGS[1], L=1, V=6, sigma_p=1.0, sigma_q=0.0, T=0.8)
    rng = np.random.default_rng(3)
    logits = rng.normal(0, 1, (1, 6))
    draws = np.concatenate([G._gumbel_argmax(np.broadcast_to(logits, (50_000, 6)), cfg["T"],
                                             np.random.default_rng(s)) for s in range(4)])
    counts = np.bincount(draws, minlength=6)
    _, pval = stats.chisquare(counts, len(draws) * special.softmax(logits[0] / cfg["T"]))
    assert pval > 1e-4


def test_workload_statistics_reported(capsys):
    """Print measured acceptance statistics of each sampled workload (context only)."""
    from oracle import isd_oracle as O
    for cfg_id in (1, 2):
        cfg = CONFIGS[cfg_id]
        d = gen_step(cfg_id, 0, seqs=range(min(4, cfg["C"])))
        p = O.decode_logits(d["p"], cfg["dtype"])
        q = O.decode_logits(d["q"], cfg["dtype"])
        beta = np.minimum(O.softmax(p), O.softmax(q)).sum(-1)
        with capsys.disabled():
            print(f"\nworkload {cfg['name']}: mean 1-TV(p,q) = {beta.mean():.3f}")
        assert 0.0 < beta.mean() < 1.0
