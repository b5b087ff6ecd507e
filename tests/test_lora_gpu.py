"""GPU parity of the segment-gated LoRA projection (isd_lora_gemm) against the
fp64 oracle: h_j = W x_j + [j is a mask position] B A x_j ("Introspective
Diffusion Language Models | Summary", appendix G; section 3.2).

Arithmetic of the kernels: t = A x accumulates in fp32 and is rounded once to
bf16 (zero on clean rows); h accumulates x W^T and t B^T in fp32 and is
rounded once to bf16.  So each output obeys

    |h - h_exact| <= half_ulp(h) + (K + r) 2^-24 (sum |W x| + sum |B t|)
                     + gate * sum_s |B_s| (half_ulp(t_s) + K 2^-24 sum |A_s x|)

and each adapter activation |t - t_exact| <= half_ulp(t) + K 2^-24 sum |A x|.
Clean rows must equal the base projection (isd_lm_head_packed on W alone)
exactly: the adapter segment adds exact zeros there.
"""

import numpy as np
import pytest

from isd_inputs import LORA_CONFIGS, bf16_bits_to_f32, gen_lora
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


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _half_ulp(v):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 1e-30))) - 8)


def _host(t):
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)


def _check(d, h_bits, t_bits, rows, mask):
    x, w, a, b = (_f64(d[k]) for k in ("x", "w", "a", "b"))
    x = x[rows]
    gate = (mask[rows] != 0).astype(np.float64)[:, None]
    K, r = x.shape[1], a.shape[0]
    t_exact = gate * (x @ a.T)
    t_bound = gate * (_half_ulp(t_exact) + K * 2.0 ** -24 * (np.abs(x) @ np.abs(a).T))
    t_got = _f64(t_bits[rows])
    assert np.all(t_got[gate[:, 0] == 0] == 0), "adapter activations on clean rows must be 0"
    t_worst = np.max(np.abs(t_got - t_exact) / np.maximum(t_bound, 1e-300) * gate)
    assert t_worst <= 1.0, f"t error / bound = {t_worst}"
    h_exact = O.lora_gemm(x, w, a, b, mask[rows])
    bound = (_half_ulp(h_exact)
             + (K + r) * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T + np.abs(t_exact) @ np.abs(b).T)
             + (t_bound) @ np.abs(b).T)
    err = np.abs(_f64(h_bits[rows]) - h_exact)
    worst = np.max(err / bound)
    assert worst <= 1.0, f"h error / bound = {worst}"
    return worst, t_worst


def test_lora_midsize_and_clean_rows_match_base(isd):
    import torch
    cfg = LORA_CONFIGS["mid"]
    d = gen_lora(cfg, seed=3)
    mask = d["mask"]
    x, a = _dev(d["x"]), _dev(d["a"])
    wcat = isd.lora_pack(_dev(d["w"]), _dev(d["b"]))
    h, t = isd.lora_gemm(x, a, wcat, torch.from_numpy(mask).cuda())
    base = isd.lm_head_packed(x, _dev(d["w"]))
    torch.cuda.synchronize()
    hb, tb = _host(h), _host(t)
    rows = np.arange(mask.size)
    worst, t_worst = _check(d, hb, tb, rows, mask)
    clean = mask == 0
    np.testing.assert_array_equal(_f64(hb[clean]), _f64(_host(base)[clean]))
    assert not np.array_equal(_f64(hb[~clean]), _f64(_host(base)[~clean]))
    log(f"lora mid: worst h err/bound {worst:.3f}, t err/bound {t_worst:.3f}")


def test_lora_no_mask_adapts_every_row(isd):
    import torch
    cfg = dict(LORA_CONFIGS["mid"], C=3, L=7, N=136, K=256, r=128)
    d = gen_lora(cfg, seed=4)
    x, a = _dev(d["x"]), _dev(d["a"])
    wcat = isd.lora_pack(_dev(d["w"]), _dev(d["b"]))
    h, t = isd.lora_gemm(x, a, wcat, None)
    torch.cuda.synchronize()
    ones = np.ones(d["x"].shape[0], np.int32)
    _check(d, _host(h), _host(t), np.arange(ones.size), ones)


def test_lora_split_shrink_ragged(isd):
    """An output buffer large enough for the shrink's fp32 partial sums (the
    split-K shrink): 42 rows (not a multiple of 64), K = 640 (three K slices,
    the last one partial), r = 128."""
    import torch
    cfg = dict(LORA_CONFIGS["mid"], C=3, L=7, N=2048, K=640, r=128)
    d = gen_lora(cfg, seed=6)
    mask = d["mask"]
    x, a = _dev(d["x"]), _dev(d["a"])
    wcat = isd.lora_pack(_dev(d["w"]), _dev(d["b"]))
    h, t = isd.lora_gemm(x, a, wcat, torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    worst, t_worst = _check(d, _host(h), _host(t), np.arange(mask.size), mask)
    log(f"lora split shrink: worst h err/bound {worst:.3f}, t err/bound {t_worst:.3f}")


@pytest.mark.parametrize("split", [False, True], ids=["whole", "k-split"])
def test_lora_wide_tiles_ragged(isd, split):
    """At least one 256 x 256 output tile per CU (4 x 65 here) takes the
    ping-pong kernel with its second K segment: 1000 rows (a ragged last row
    tile), N = 16389 (a ragged, odd last column tile), K = 256, r = 128; with
    a workspace, the 4 tiles past the first round are halved along K.
    Sampled rows meet the bound, and every clean row equals the base
    projection (given the same workspace) bit for bit."""
    import torch
    cfg = dict(LORA_CONFIGS["mid"], C=100, L=10, N=16389, K=256, r=128)
    d = gen_lora(cfg, seed=7)
    mask = d["mask"]
    x, a = _dev(d["x"]), _dev(d["a"])
    wcat = isd.lora_pack(_dev(d["w"]), _dev(d["b"]))
    ws = isd.gemm_workspace(x.shape[0], cfg["K"], cfg["N"]) if split else None
    assert (ws is not None) == split
    h, t = isd.lora_gemm(x, a, wcat, torch.from_numpy(mask).cuda(), workspace=ws)
    base = isd.lm_head_packed(x, _dev(d["w"]), workspace=ws)
    torch.cuda.synchronize()
    hb, tb = _host(h), _host(t)
    rows = np.unique(np.concatenate([np.arange(0, 1000, 37), [255, 256, 511, 512, 767, 768, 998, 999]]))
    worst, t_worst = _check(d, hb, tb, rows, mask)
    clean = mask == 0
    assert clean.any() and (~clean).any()
    np.testing.assert_array_equal(hb[clean], _host(base)[clean])
    log(f"lora wide tiles 1000 x 256 x 16389 (split {split}): worst h err/bound {worst:.3f}, "
        f"t err/bound {t_worst:.3f}, {int(clean.sum())} clean rows equal the base projection")


def test_lora_full_shape_sampled_rows(isd):
    """The MLP gate/up projection of an 8B model at the serving batch:
    M = 1024, K = 4096, N = 24576, r = 128; every adapter activation, the
    full output rows of a clean and a mask position of several sequences,
    and every clean row against the base projection, bit for bit; then the
    same with the K-split workspace."""
    import torch
    cfg = LORA_CONFIGS["mlp_up"]
    d = gen_lora(cfg, seed=0)
    mask = d["mask"]
    x, a = _dev(d["x"]), _dev(d["a"])
    wcat = isd.lora_pack(_dev(d["w"]), _dev(d["b"]))
    h, t = isd.lora_gemm(x, a, wcat, torch.from_numpy(mask).cuda())
    base = isd.lm_head_packed(x, _dev(d["w"]))
    torch.cuda.synchronize()
    hb, tb = _host(h), _host(t)
    clean = mask == 0
    np.testing.assert_array_equal(hb[clean], _host(base)[clean])
    # the same with a workspace: the 128 tiles past the first round (columns
    # 16384 on) are halved along K; the others keep their bits
    ws = isd.gemm_workspace(*d["x"].shape, cfg["N"])
    hs, ts = isd.lora_gemm(x, a, wcat, torch.from_numpy(mask).cuda(), workspace=ws)
    bs = isd.lm_head_packed(x, _dev(d["w"]), workspace=ws)
    torch.cuda.synchronize()
    hsb = _host(hs)
    np.testing.assert_array_equal(_host(ts), tb)
    np.testing.assert_array_equal(hsb[clean], _host(bs)[clean])
    np.testing.assert_array_equal(hsb[:, :16384], hb[:, :16384])
    split_worst, _ = _check(d, hsb, tb, np.array([3, 12, 700, 1019]), mask)
    rows = np.array([0, 7, 8, 15, 500, 511, 1016, 1023])
    worst, t_worst = _check(d, hb, tb, rows, mask)
    # all adapter activations
    all_rows = np.arange(mask.size)
    xa = _f64(d["x"]) @ _f64(d["a"]).T
    gate = (mask != 0)[:, None]
    tg = _f64(tb)
    assert np.all(tg[~gate[:, 0]] == 0)
    bound = _half_ulp(xa) + cfg["K"] * 2.0 ** -24 * (np.abs(_f64(d["x"])) @ np.abs(_f64(d["a"])).T)
    assert np.max((np.abs(tg - xa) / bound)[gate[:, 0]]) <= 1.0
    log(f"lora full shape rows {rows.tolist()}: worst h err/bound {worst:.3f}, "
        f"t err/bound {t_worst:.3f} ({all_rows.size} rows of t checked); with the K split "
        f"{split_worst:.3f}")
