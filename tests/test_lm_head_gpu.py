"""GPU parity of the LM-head projection (isd_lm_head) against the fp64 oracle.

The kernel accumulates in fp32 and rounds once to bf16 (nearest even).  Each
output must lie within half a bf16 ulp of the exact product plus the fp32
accumulation bound K * 2^-24 * sum_k |h_k w_k|, and almost every output must
equal the exact product rounded to bf16.
"""

import numpy as np
import pytest

from isd_inputs import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, gen_head_weights, gen_hidden
from oracle import isd_oracle as O
from tests.isd_testlib import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def isd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import speculative_verification_amd as isd_mod
    isd_mod.lib()
    return isd_mod


def _dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _check(gpu_bits, h_bits, w_bits, rows):
    """Compare output rows `rows` with the fp64 product."""
    h = bf16_bits_to_f32(h_bits[rows]).astype(np.float64)
    w = bf16_bits_to_f32(w_bits).astype(np.float64)
    exact = O.lm_head(h, w)
    absdot = np.abs(h) @ np.abs(w)
    got = bf16_bits_to_f32(gpu_bits[rows]).astype(np.float64)
    rne = bf16_bits_to_f32(f32_to_bf16_bits(exact.astype(np.float32))).astype(np.float64)
    mag = np.maximum(np.abs(exact), 1e-30)
    half_ulp = np.exp2(np.floor(np.log2(mag)) - 8)
    K = h.shape[1]
    bound = half_ulp + K * 2.0 ** -24 * absdot
    err = np.abs(got - exact)
    worst = np.max(err / bound)
    assert worst <= 1.0, f"max error / bound = {worst}"
    frac_rne = np.mean(got == rne)
    assert frac_rne >= 0.999, f"only {frac_rne:.5f} of outputs equal the rounded exact product"
    return worst, frac_rne


@pytest.mark.parametrize("M,K,N", [(300, 256, 1000), (64, 4096, 2048), (257, 128, 136)])
def test_lm_head_small_shapes(isd, M, K, N):
    import torch
    rng = np.random.default_rng(M * 7 + N)
    h_bits = f32_to_bf16_bits(rng.normal(0, 1, (M, K)).astype(np.float32))
    w_bits = f32_to_bf16_bits(rng.normal(0, 0.02, (K, N)).astype(np.float32))
    out = isd.lm_head(_dev_bf16(h_bits), _dev_bf16(w_bits))
    torch.cuda.synchronize()
    gpu = out.view(torch.int16).cpu().numpy().view(np.uint16)
    worst, frac = _check(gpu, h_bits, w_bits, np.arange(M))
    log(f"lm_head {M}x{K}x{N}: worst err/bound {worst:.3f}, exact-rounded fraction {frac:.5f}")


def test_lm_head_full_shape_sampled_rows(isd):
    """The LM-head workload: h [1024, 4096] x W [4096, 151936]."""
    import torch
    cfg = CONFIGS[4]
    log("lm_head full shape: generating W")
    w_bits = gen_head_weights(4)
    h_bits = gen_hidden(4, 0)
    out = isd.lm_head(_dev_bf16(h_bits), _dev_bf16(w_bits))
    torch.cuda.synchronize()
    gpu = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert gpu.shape == (cfg["C"] * 2 * cfg["L"], cfg["V"])
    rows = np.array([0, 1, 255, 256, 511, 700, 1022, 1023])
    worst, frac = _check(gpu, h_bits, w_bits, rows)
    log(f"lm_head full shape, rows {rows.tolist()}: worst err/bound {worst:.3f}, "
        f"exact-rounded fraction {frac:.5f}")


def test_lm_head_rejects_bad_shapes(isd):
    import torch
    h = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((100, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(isd.IsdError):
        isd.lm_head(h, w)


@pytest.mark.parametrize("M,K,N", [(300, 256, 1000), (64, 4096, 2048), (257, 128, 136), (5, 64, 7)])
def test_lm_head_packed_small_shapes(isd, M, K, N):
    """The pre-packed head: the pack is a bit-exact transpose, and the GEMM
    meets the same bound as the unpacked one."""
    import torch
    rng = np.random.default_rng(M * 11 + N)
    h_bits = f32_to_bf16_bits(rng.normal(0, 1, (M, K)).astype(np.float32))
    w_bits = f32_to_bf16_bits(rng.normal(0, 0.02, (K, N)).astype(np.float32))
    w = _dev_bf16(w_bits)
    wt = isd.lm_head_pack(w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(wt.view(torch.int16).cpu().numpy().view(np.uint16), w_bits.T)
    out = isd.lm_head_packed(_dev_bf16(h_bits), wt)
    torch.cuda.synchronize()
    gpu = out.view(torch.int16).cpu().numpy().view(np.uint16)
    worst, frac = _check(gpu, h_bits, w_bits, np.arange(M))
    log(f"lm_head_packed {M}x{K}x{N}: worst err/bound {worst:.3f}, exact-rounded fraction {frac:.5f}")


def test_lm_head_packed_full_shape_sampled_rows(isd):
    import torch
    cfg = CONFIGS[4]
    w_bits = gen_head_weights(4)
    h_bits = gen_hidden(4, 1)
    wt = isd.lm_head_pack(_dev_bf16(w_bits))
    out = isd.lm_head_packed(_dev_bf16(h_bits), wt)
    torch.cuda.synchronize()
    gpu = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert gpu.shape == (cfg["C"] * 2 * cfg["L"], cfg["V"])
    rows = np.array([0, 3, 255, 256, 600, 1023])
    worst, frac = _check(gpu, h_bits, w_bits, rows)
    log(f"lm_head_packed full shape, rows {rows.tolist()}: worst err/bound {worst:.3f}, "
        f"exact-rounded fraction {frac:.5f}")


@pytest.mark.parametrize("M,N", [(1024, 16128), (1024, 16384), (1000, 16392), (1000, 16389)])
def test_lm_head_packed_tile_width_threshold(isd, M, N):
    """1024 rows give four 256-row tiles; N = 16128 makes 252 tiles of 256 columns,
    fewer than the CUs (the packed head then runs on the 128-wide kernel), N = 16384
    exactly 256 (the 256-wide ping-pong kernel), and M = 1000 with N = 16392 or 16389
    takes the wide kernel with a ragged last row tile and a ragged last column tile.
    Every case must hold the oracle's bound on sampled rows and, where the unpacked
    kernel accepts the shape (N a multiple of 8), agree bit for bit with it: it
    accumulates in the same K order."""
    import torch
    K = 512
    rng = np.random.default_rng(N)
    h_bits = f32_to_bf16_bits(rng.normal(0, 1, (M, K)).astype(np.float32))
    w_bits = f32_to_bf16_bits(rng.normal(0, 0.02, (K, N)).astype(np.float32))
    w_dev = _dev_bf16(w_bits)
    h_dev = _dev_bf16(h_bits)
    packed = isd.lm_head_packed(h_dev, isd.lm_head_pack(w_dev))
    torch.cuda.synchronize()
    gp = packed.view(torch.int16).cpu().numpy().view(np.uint16)
    assert gp.shape == (M, N)
    rows = np.array([0, 1, 255, 256, 511, 767, 999, M - 1])
    worst, frac = _check(gp, h_bits, w_bits, rows)
    if N % 8 == 0:
        plain = isd.lm_head(h_dev, w_dev)
        torch.cuda.synchronize()
        gu = plain.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(gp, gu), "packed and unpacked heads differ"
    log(f"lm_head_packed M={M} K={K} N={N}: worst err/bound {worst:.3f}, "
        f"exact-rounded fraction {frac:.5f}" + (", equal to the unpacked kernel" if N % 8 == 0 else ""))


@pytest.mark.parametrize("M,K,N", [(1024, 512, 24576), (1000, 256, 24389), (1024, 256, 16640)])
def test_lm_head_packed_k_split(isd, M, K, N):
    """With a workspace, the 256 x 256 tiles past the whole rounds over the CUs
    are computed as two halves along K that meet in it: 128 of 384 tiles, 128
    of 384 with ragged rows and columns, 4 of 260.  Sampled rows (all columns,
    so every split tile is checked) hold the oracle's bound; the tiles of the
    whole rounds equal the call without a workspace bit for bit; a second call
    on the same workspace repeats the bits and leaves its counters zero."""
    import torch
    rng = np.random.default_rng(N + K)
    h_bits = f32_to_bf16_bits(rng.normal(0, 1, (M, K)).astype(np.float32))
    w_bits = f32_to_bf16_bits(rng.normal(0, 0.02, (K, N)).astype(np.float32))
    h_dev = _dev_bf16(h_bits)
    wt = isd.lm_head_pack(_dev_bf16(w_bits))
    ws = isd.gemm_workspace(M, K, N)
    assert ws is not None
    per_tile = 128 + 2 * 256 * 256 * 4
    n_split = ws.numel() // per_tile
    assert ws.numel() == n_split * per_tile and n_split > 0
    plain = isd.lm_head_packed(h_dev, wt)
    split = isd.lm_head_packed(h_dev, wt, workspace=ws)
    again = isd.lm_head_packed(h_dev, wt, workspace=ws)
    torch.cuda.synchronize()
    gp = plain.view(torch.int16).cpu().numpy().view(np.uint16)
    gs = split.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(gs, again.view(torch.int16).cpu().numpy().view(np.uint16))
    assert int(ws[: n_split * 128].view(torch.int32).abs().sum()) == 0, "counters not returned to zero"
    m_tiles = (M + 255) // 256
    n_tiles = (N + 255) // 256
    n_full = m_tiles * n_tiles - n_split
    tile = (np.arange(M)[:, None] // 256) + (np.arange(N)[None, :] // 256) * m_tiles
    whole = tile < n_full
    assert np.array_equal(gs[whole], gp[whole]), "tiles of the whole rounds changed"
    rows = np.array([0, 1, 255, 256, 511, 767, M - 2, M - 1])
    worst, frac = _check(gs, h_bits, w_bits, rows)
    differ = int(np.sum(gs[~whole] != gp[~whole]))
    log(f"lm_head_packed K split M={M} K={K} N={N}: {n_split} split tiles, worst err/bound "
        f"{worst:.3f}, exact-rounded fraction {frac:.5f}, {differ} of {int((~whole).sum())} split "
        f"outputs differ from the unsplit call")
