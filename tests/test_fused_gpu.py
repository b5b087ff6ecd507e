"""GPU parity of the statistics path: the LM head's epilogue partials
(isd_lm_head_stats) and the step fed by them (isd_step_fused).

Inputs come from gen_exact_head: h in {-1, 0, 1} and W on a grid of 2^-7, so
the fp32 accumulation is exact and the bf16 logits are the round-to-nearest-
even of the exact product on both sides.  The oracle computes those logits
itself (fp64 product, then the bf16 encoding) and runs the step on them; the
test also checks that the GPU wrote exactly those bits.

* tile partials: e = ceil(max * k2) equals the same fp32 computation; s
  matches sum 2^(x k2 - e) in fp64 to 1e-5, and so do the row denominators;
* the step: every output agrees with the oracle under the tolerance rule,
  and with isd_step on the same logits (the path that reads every row).
"""

import os

import numpy as np
import pytest

from isd_inputs import bf16_bits_to_f32, f32_to_bf16_bits, gen_exact_head
from oracle import isd_oracle as O
from tests.isd_testlib import compare, log, oracle_step, to_host

pytestmark = pytest.mark.gpu

WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module")
def isd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import speculative_verification_amd as isd_mod
    isd_mod.lib()
    return isd_mod


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_logits(h_bits, wt_bits, rows):
    """bf16 bits of the exact product for the given rows (in column blocks)."""
    h = bf16_bits_to_f32(h_bits[rows]).astype(np.float64)
    N = wt_bits.shape[0]
    out = np.empty((len(rows), N), dtype=np.uint16)
    for n0 in range(0, N, 16384):
        w = bf16_bits_to_f32(wt_bits[n0:n0 + 16384]).astype(np.float64)
        exact = O.lm_head(h, w.T)
        out[:, n0:n0 + 16384] = f32_to_bf16_bits(exact.astype(np.float32))   # exact in fp32
    return out


def _check_stats(logit_bits, stats, T):
    k2 = np.float32(LOG2E / T)
    x = bf16_bits_to_f32(logit_bits)
    M, N = x.shape
    nt = (N + 127) // 128
    pad = np.full((M, nt * 128), -np.inf, dtype=np.float32)
    pad[:, :N] = x
    tiles = pad.reshape(M, nt, 128)
    e = np.ceil(tiles.max(axis=-1) * k2)                 # fp32, as the kernel takes it
    np.testing.assert_array_equal(stats[..., 0], e)
    s = np.exp2(tiles.astype(np.float64) * np.float64(k2) - e[..., None].astype(np.float64)).sum(-1)
    np.testing.assert_allclose(stats[..., 1], s, rtol=1e-5)
    Z_tiles = (stats[..., 1].astype(np.float64) * np.exp2(stats[..., 0].astype(np.float64))).sum(-1)
    Z = np.exp2(x.astype(np.float64) * np.float64(k2)).sum(-1)
    np.testing.assert_allclose(Z_tiles, Z, rtol=1e-5)


def _run(isd, C, L, K, V, T, seed, check_rows=None, **variant):
    import torch
    M = C * 2 * L
    wt = gen_exact_head(M, K, V, which="w")["wt"]
    h_prev = gen_exact_head(M, K, V, seed=2 * seed, which="h")["h"]
    h_cur = gen_exact_head(M, K, V, seed=2 * seed + 1, which="h")["h"]
    wt_d = _dev(wt)
    lp, sp = isd.lm_head_stats(_dev(h_prev), wt_d, T)
    lc, sc = isd.lm_head_stats(_dev(h_cur), wt_d, T)
    base = isd.lm_head_packed(_dev(h_cur), wt_d)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(lc), _bits(base)), "stats epilogue changed the logits"
    nt = (V + 127) // 128
    ext_p, ext_c = lp.view(C, 2 * L, V), lc.view(C, 2 * L, V)
    st_p, st_c = sp.view(C, 2 * L, nt, 2), sc.view(C, 2 * L, nt, 2)
    p, qn, q = ext_c[:, :L], ext_c[:, L:], ext_p[:, L:]

    # oracle logits of the rows it checks (all, or the sequences in check_rows)
    seqs = np.arange(C) if check_rows is None else np.asarray(check_rows)
    rows_c = (seqs[:, None] * 2 * L + np.arange(2 * L)[None, :]).ravel()
    oc = _oracle_logits(h_cur, wt, rows_c).reshape(len(seqs), 2 * L, V)
    op = _oracle_logits(h_prev, wt, rows_c).reshape(len(seqs), 2 * L, V)
    assert np.array_equal(_bits(ext_c)[seqs], oc), "GPU logits differ from the exact product"
    assert np.array_equal(_bits(ext_p)[seqs], op)

    rng = np.random.default_rng(seed)
    ua, ur, up, u0 = (rng.random((C, L), dtype=np.float32) for _ in range(4))
    # proposals drawn from the previous mask rows (the q law), by the oracle
    x = np.zeros((C, L), dtype=np.int32)
    if variant.get("q_onehot"):
        x[seqs] = O.argmax_first(O.decode_logits(op[:, L:], "bf16"))
    else:
        x[seqs] = O.propose_sample(O.decode_logits(op[:, L:], "bf16"), u0[seqs], T)[0]
    if check_rows is not None:
        x[np.setdiff1d(np.arange(C), seqs)] = 7
    dv = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    args = (p, q, dv(x), dv(ua), dv(ur), qn, dv(up))
    qs = None if variant.get("q_onehot") else st_p[:, L:]
    fused = to_host(isd.step_fused(*args, st_c[:, :L], qs, st_c[:, L:], temperature=T, **variant))
    plain = to_host(isd.step(*args, temperature=T, **variant))
    torch.cuda.synchronize()

    d = dict(p=np.ascontiguousarray(oc[:, :L]), q=np.ascontiguousarray(op[:, L:]),
             qn=np.ascontiguousarray(oc[:, L:]), x=x[seqs], ua=ua[seqs], ur=ur[seqs], up=up[seqs])
    ref = oracle_step(d, "bf16", "sample", T, relax=variant.get("relax", 0.0),
                      q_onehot=variant.get("q_onehot", False), sampler=variant.get("sampler", "cdf"),
                      seq_ids=seqs, workers=WORKERS)
    sub = lambda o: {k: val[seqs] for k, val in o.items()}  # noqa: E731
    st1 = compare(sub(fused), ref, label="fused vs oracle")
    compare(sub(plain), ref, label="plain vs oracle")
    return fused, plain, ref, st1, (lp, sp, lc, sc)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_stats_and_fused_step_midsize(isd, T):
    """C=4, L=8 (M=64), K=256, V=20000: a ragged last stats tile."""
    fused, plain, ref, st, (lp, sp, lc, sc) = _run(isd, 4, 8, 256, 20000, T, seed=1 if T == 1.0 else 2)
    _check_stats(_bits(lc), sc.cpu().numpy(), T)
    _check_stats(_bits(lp), sp.cpu().numpy(), T)
    log(f"fused midsize T={T}: {st}")


@pytest.mark.parametrize("M,N", [(64, 20003), (300, 1029)])
def test_stats_ragged_width_and_rows(isd, M, N):
    """The statistics GEMM where N is not a multiple of 8 (element stores of the
    logits, a last 128-column tile of 35 or 5 columns) and, at M = 300, a ragged
    last row tile: the logits equal the exact product's bf16 bits and those of the
    packed head, and every (row, tile) partial matches the fp64 definition."""
    import torch
    K = 256
    d = gen_exact_head(M, K, N, seed=21)
    h, wt = _dev(d["h"]), _dev(d["wt"])
    logits, stats = isd.lm_head_stats(h, wt, 0.8)
    base = isd.lm_head_packed(h, wt)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(logits), _bits(base)), "statistics epilogue changed the logits"
    assert np.array_equal(_bits(logits), _oracle_logits(d["h"], d["wt"], np.arange(M)))
    _check_stats(_bits(logits), stats.cpu().numpy(), 0.8)
    log(f"statistics GEMM M={M} N={N}: logits exact, {stats.shape[1]} tiles per row checked")


def test_fused_step_serving_shape(isd):
    """The serving shape: C=64, L=8, V=151936 from an H=4096 head.  Every
    sequence of both paths (statistics and plain) against the oracle under
    the tolerance rule, with flagged cases validated; their probabilities
    agree with each other to 1e-5."""
    fused, plain, ref, st, _ = _run(isd, 64, 8, 4096, 151936, 1.0, seed=5)
    np.testing.assert_allclose(fused["p_x"], plain["p_x"], rtol=1e-5, atol=1e-30)
    np.testing.assert_allclose(fused["q_x"], plain["q_x"], rtol=1e-5, atol=1e-30)
    np.testing.assert_allclose(fused["alpha"], plain["alpha"], rtol=1e-5)
    log(f"fused serving shape, all 64 sequences against the oracle: {st}")


def test_fused_step_separate_launches(isd):
    """C = 200, L = 8: the decisions and proposals take 200 + 200 workgroups, more
    than fit on the CUs at once, so they run as two launches around the residual
    items instead of one.  Every sequence against the oracle."""
    fused, plain, ref, st, _ = _run(isd, 200, 8, 128, 3000, 0.9, seed=13)
    log(f"fused C=200 (separate decision and proposal launches): {st}")


@pytest.mark.parametrize("variant", [dict(sampler="gumbel"), dict(q_onehot=True, relax=0.5),
                                     dict(q_onehot=True, sampler="gumbel")])
def test_fused_step_variants(isd, variant):
    """One-hot proposals (no q statistics), relaxed acceptance and the
    Gumbel-max correction on the statistics path."""
    fused, plain, ref, st, _ = _run(isd, 4, 8, 256, 20000, 1.0, seed=9, **variant)
    log(f"fused {variant}: {st}")


@pytest.mark.parametrize("M,N", [(1000, 16389), (1024, 24576)])
def test_stats_k_split(isd, M, N):
    """The statistics GEMM with the GEMM workspace: the 256 x 256 tiles past the
    whole rounds over the CUs (4 of 260 with ragged rows and columns, 128 of 384)
    run as two halves of K, and the second half to arrive writes the logits and
    the partials.  The logits equal the exact product's bf16 bits and the packed
    head's with the same workspace, every partial matches the fp64 definition,
    a second call repeats the bits, and the counters return to zero."""
    import torch
    K = 256
    d = gen_exact_head(M, K, N, seed=23)
    h, wt = _dev(d["h"]), _dev(d["wt"])
    ws = isd.gemm_workspace(M, K, N)
    assert ws is not None
    logits, stats = isd.lm_head_stats(h, wt, 0.8, workspace=ws)
    logits2, stats2 = isd.lm_head_stats(h, wt, 0.8, workspace=ws)
    base = isd.lm_head_packed(h, wt, workspace=ws)
    torch.cuda.synchronize()
    per_tile = 128 + 2 * 256 * 256 * 4
    n_split = ws.numel() // per_tile
    assert int(ws[: n_split * 128].view(torch.int32).abs().sum()) == 0, "counters not returned to zero"
    assert np.array_equal(_bits(logits), _bits(logits2))
    assert torch.equal(stats, stats2)
    assert np.array_equal(_bits(logits), _bits(base)), "statistics epilogue changed the logits"
    assert np.array_equal(_bits(logits), _oracle_logits(d["h"], d["wt"], np.arange(M)))
    _check_stats(_bits(logits), stats.cpu().numpy(), 0.8)
    log(f"statistics GEMM with K split M={M} N={N}: {n_split} split tiles, logits exact, "
        f"{stats.shape[1]} tiles per row checked")
