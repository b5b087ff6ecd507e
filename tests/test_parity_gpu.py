"""GPU parity: libisd against the CPU oracle on the same seeded bytes.

Every call goes through the C ABI (ctypes binding).  Sizes: the tiny workload
(all 100 steps), a mid-size workload that spans several tiles with a ragged
tail, the serving and greedy workloads at full size (a few steps each, every
sequence checked), and the high-concurrency workload at full size (sampled
sequences checked against the oracle, invariants checked on all).
"""

import os

import numpy as np
import pytest

from isd_inputs import CONFIGS, f32_to_bf16_bits, gen_step
from tests.isd_testlib import compare, log, oracle_step, to_device, to_host

pytestmark = pytest.mark.gpu

WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module")
def isd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import speculative_verification_amd as isd_mod
    isd_mod.lib()
    isd_mod.set_tuning(0, 0, 0)
    yield isd_mod
    isd_mod.set_tuning(0, 0, 0)


def _run(isd, dd, cfg, api="step"):
    import torch
    mode, T = cfg["mode"], cfg["T"]
    if api == "step":
        o = isd.step(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"],
                     mode=mode, temperature=T)
    else:
        o = isd.verify_step(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], mode=mode,
                            temperature=T)
        o.update(isd.propose(dd["qn"], dd["up"], mode=mode, temperature=T))
    torch.cuda.synchronize()
    return to_host(o)


def _check_errors(isd):
    import torch
    dev = torch.device("cuda", 0)
    for key, ws in list(isd.isd._ws_cache.items()):
        if key[0] == dev:
            isd.check_device_error(ws)


def _totals(acc, st):
    for k, v in st.items():
        acc[k] = acc.get(k, 0) + v
    return acc


def test_tiny_workload_all_steps(isd):
    cfg = CONFIGS[1]
    totals = {}
    for step in range(cfg["steps"]):
        d = gen_step(1, step)
        dd = to_device(d, cfg["dtype"])
        ref = oracle_step(d, cfg["dtype"], cfg["mode"], cfg["T"])
        fused = _run(isd, dd, cfg, "step")
        split = _run(isd, dd, cfg, "split")
        for key in fused:
            np.testing.assert_array_equal(fused[key], split[key], err_msg=f"step {step} {key}")
        _totals(totals, compare(fused, ref, label=f"tiny step {step}"))
    _check_errors(isd)
    log(f"tiny workload, 100 steps: {totals}")


def test_alpha_entry_point(isd):
    import torch
    cfg = CONFIGS[1]
    for step in range(0, 100, 9):
        d = gen_step(1, step)
        dd = to_device(d, cfg["dtype"])
        o = to_host(isd.alpha(dd["p"], dd["q"], dd["x"]))
        torch.cuda.synchronize()
        ref = oracle_step(d, cfg["dtype"], cfg["mode"], cfg["T"])
        np.testing.assert_allclose(o["alpha"], ref["alpha"], rtol=1e-5)
        np.testing.assert_allclose(o["alpha_mean"][0], ref["alpha"].mean(), rtol=1e-5)


def _midsize_cfg(**kw):
    cfg = dict(CONFIGS[2], C=8, L=8, V=10000)
    cfg.update(kw)
    return cfg


@pytest.mark.parametrize("variant", ["default", "seg1", "seg3", "res1", "res5"])
def test_midsize_ragged_tiles(isd, variant):
    """V = 10000: four full 2048-element tiles and a ragged fifth; every
    decomposition choice must agree with the oracle."""
    tuning = dict(default=(0, 0), seg1=(1, 1), seg3=(3, 2), res1=(0, 1), res5=(2, 5))[variant]
    isd.set_tuning(tuning[0], tuning[1], 0)
    cfg = _midsize_cfg()
    totals = {}
    try:
        for step in range(12):
            d = gen_step(2, 1000 + step, cfg=cfg)
            dd = to_device(d, cfg["dtype"])
            ref = oracle_step(d, cfg["dtype"], cfg["mode"], cfg["T"])
            _totals(totals, compare(_run(isd, dd, cfg), ref, label=f"mid {variant} {step}"))
    finally:
        isd.set_tuning(0, 0, 0)
    _check_errors(isd)
    log(f"mid-size {variant}: {totals}")


def test_midsize_greedy(isd):
    cfg = dict(CONFIGS[3], C=8, L=8, V=10000)
    for step in range(6):
        d = gen_step(3, 1000 + step, cfg=cfg)
        dd = to_device(d, cfg["dtype"])
        ref = oracle_step(d, cfg["dtype"], "greedy", cfg["T"])
        compare(_run(isd, dd, cfg), ref, label=f"mid greedy {step}")
        compare(_run(isd, dd, cfg, "split"), ref, label=f"mid greedy split {step}")


# Full-size workloads: 20 fresh steps each, every sequence against the oracle.
# Steps are run in blocks so that each test stays around a minute.
_FULL_BLOCKS = [(2, 0, 10), (2, 10, 10), (3, 0, 10), (3, 10, 10),
                (5, 0, 5), (5, 5, 5), (5, 10, 5), (5, 15, 5)]


@pytest.mark.parametrize("cfg_id,first,n", _FULL_BLOCKS,
                         ids=[f"cfg{c}-steps{f}-{f + n - 1}" for c, f, n in _FULL_BLOCKS])
def test_full_size_workloads(isd, cfg_id, first, n):
    """Serving (C=64, L=8), strict/greedy (C=64, L=8) and high-concurrency
    (C=256, L=16) workloads at V=151936: steps first..first+n-1 of 20, every
    sequence of every step compared with the oracle; flagged cases are
    validated, and the output invariants hold for every sequence."""
    import torch
    cfg = CONFIGS[cfg_id]
    C, L = cfg["C"], cfg["L"]
    totals, hist = {}, np.zeros(L + 1, np.int64)
    for step in range(first, first + n):
        log(f"workload {cfg['name']} step {step}: generating")
        d = gen_step(cfg_id, step, workers=WORKERS)
        dd = to_device(d, cfg["dtype"])
        log(f"workload {cfg['name']} step {step}: running")
        gpu = _run(isd, dd, cfg)
        del dd
        al, out, ne = gpu["accept_len"], gpu["out_tokens"], gpu["n_emitted"]
        assert np.all((al >= 0) & (al <= L))
        np.testing.assert_array_equal(ne, al + (al < L))
        for c in range(C):
            np.testing.assert_array_equal(out[c, :al[c]], d["x"][c, :al[c]])
            assert np.all(out[c, ne[c]:] == -1)
        hist += np.bincount(al, minlength=L + 1)
        ref = oracle_step(d, cfg["dtype"], cfg["mode"], cfg["T"], workers=WORKERS)
        _totals(totals, compare(gpu, ref, label=f"{cfg['name']} step {step}"))
    torch.cuda.empty_cache()
    _check_errors(isd)
    log(f"workload {cfg['name']} steps {first}-{first + n - 1}: {totals}; "
        f"accept-length histogram {hist.tolist()}")


@pytest.mark.parametrize("sigma_q", [0.3, 0.1, 0.05])
def test_small_residual_mass_full_vocabulary(isd, sigma_q):
    """The serving construction with q = p + N(0, sigma_q^2), so the residual
    mass Z = sum max(0, P - Q) of a row falls to about 0.12, 0.04 and 0.02,
    and with every accept uniform just below 1, so that nearly every sequence
    rejects at its first position with P(x) < Q(x) and draws a correction
    from a small residual.  Every sequence of four steps is compared."""
    import torch
    cfg = dict(CONFIGS[2], sigma_q=sigma_q)
    below_one = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    totals = {}
    drawn = 0
    for step in range(4):
        d = gen_step(2, 2000 + step, cfg=cfg, workers=WORKERS)
        d["ua"][:] = below_one
        dd = to_device(d, cfg["dtype"])
        gpu = _run(isd, dd, cfg)
        del dd
        ref = oracle_step(d, cfg["dtype"], "sample", cfg["T"], workers=WORKERS)
        drawn += int((ref["accept_len"] < cfg["L"]).sum())
        _totals(totals, compare(gpu, ref, label=f"sigma_q={sigma_q} step {step}"))
    torch.cuda.empty_cache()
    _check_errors(isd)
    assert drawn >= 200, drawn
    log(f"small residual mass sigma_q={sigma_q}: {drawn} corrections drawn, {totals}")


def test_bounded_wait_gives_up_and_recovers(isd):
    """The residual items' wait for their sequence's decision is bounded.  With
    the bound set to one poll from the host, every residual item whose
    decision is not yet published gives up: the launch still ends normally
    and the device error word reports the expired wait.  The decisions that
    launch publishes late carry its epoch, so without re-zeroing the
    workspace the next launch (default bound) matches the oracle exactly and
    leaves the workspace zero; the binding's check re-zeroes it as well."""
    import ctypes

    import torch
    cfg = _midsize_cfg()
    d = gen_step(2, 3000, cfg=cfg)
    dd = to_device(d, cfg["dtype"])
    ref = oracle_step(d, cfg["dtype"], "sample", cfg["T"])
    ws = torch.zeros(isd.workspace_bytes(isd.make_shape(dd["p"])), dtype=torch.uint8,
                     device="cuda")
    args = (dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"])
    try:
        isd.set_tuning(spin_limit=1)
        isd.step(*args, ws=ws)
        torch.cuda.synchronize()
    finally:
        isd.set_tuning(0, 0, 0)
    st = isd.lib().isd_check_device_error(ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == isd.isd.ISD_ERR_DEVICE
    assert "wait expired" in isd.lib().isd_last_error().decode()
    # no re-zeroing: stale records of the expired launch must not leak into this one
    gpu = to_host(isd.step(*args, ws=ws))
    torch.cuda.synchronize()
    compare(gpu, ref, label="after an expired wait")
    isd.check_device_error(ws)
    assert int(torch.count_nonzero(ws)) == 0
    # the binding's check re-zeroes the workspace when it raises
    try:
        isd.set_tuning(spin_limit=1)
        isd.step(*args, ws=ws)
    finally:
        isd.set_tuning(0, 0, 0)
    with pytest.raises(isd.IsdError, match="wait expired"):
        isd.check_device_error(ws)
    assert int(torch.count_nonzero(ws)) == 0
    compare(to_host(isd.step(*args, ws=ws)), ref, label="after re-zeroing")
    isd.check_device_error(ws)


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

def _make_inputs(rng, C, L, V, dtype="bf16", sigma=3.0, noise=0.7, ld=None):
    ld = V if ld is None else ld
    p32 = (sigma * rng.standard_normal((C, L, V))).astype(np.float32)
    q32 = (p32 + noise * rng.standard_normal((C, L, V))).astype(np.float32)
    qn32 = (sigma * rng.standard_normal((C, L, V))).astype(np.float32)
    return _pack(rng, p32, q32, qn32, dtype, ld)


def _pack(rng, p32, q32, qn32, dtype, ld, x=None, ua=None, ur=None, up=None):
    C, L, V = p32.shape

    def enc(a):
        if dtype == "bf16":
            raw = f32_to_bf16_bits(a)
            buf = np.zeros((C, L, ld), np.uint16)
        else:
            raw = a.astype(np.float32)
            buf = np.zeros((C, L, ld), np.float32)
        buf[:, :, :V] = raw
        return raw, buf

    d, bufs = {}, {}
    for key, a in (("p", p32), ("q", q32), ("qn", qn32)):
        d[key], bufs[key] = enc(a)
    if x is None:
        qv = (d["q"].astype(np.uint32) << 16).view(np.float32) if dtype == "bf16" else d["q"]
        g = -np.log(-np.log(np.clip(rng.random((C, L, V)), 1e-300, 1 - 1e-16)))
        x = np.argmax(qv.astype(np.float64) + g, axis=-1).astype(np.int32)
    d["x"] = x.astype(np.int32)
    for key, u in (("ua", ua), ("ur", ur), ("up", up)):
        d[key] = (rng.random((C, L)).astype(np.float32) if u is None else
                  np.broadcast_to(np.asarray(u, np.float32), (C, L)).copy())
    return d, bufs


def _device_views(d, bufs, dtype, V):
    import torch
    dev = torch.device("cuda", 0)
    out = {}
    for key in ("p", "q", "qn"):
        b = bufs[key]
        if dtype == "bf16":
            t = torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            t = torch.from_numpy(b).to(dev)
        out[key] = t[:, :, :V]
    for key in ("x", "ua", "ur", "up"):
        out[key] = torch.from_numpy(np.ascontiguousarray(d[key])).to(dev)
    return out


@pytest.mark.parametrize("V", [1, 2, 7, 63, 64, 65, 511, 512, 1000, 2047, 2048, 2049, 4097, 151936])
@pytest.mark.parametrize("L", [1, 3, 16])
def test_fuzz_shapes(isd, V, L):
    rng = np.random.default_rng(V * 100 + L)
    C = 3
    for dtype in ("bf16", "f32"):
        d, bufs = _make_inputs(rng, C, L, V, dtype)
        dd = _device_views(d, bufs, dtype, V)
        cfg = dict(mode="sample", T=1.0)
        ref = oracle_step(d, dtype, "sample", 1.0)
        compare(_run(isd, dd, cfg), ref, label=f"fuzz V={V} L={L} {dtype}")
        refg = oracle_step(d, dtype, "greedy", 1.0)
        compare(_run(isd, dd, dict(mode="greedy", T=1.0)), refg, label=f"fuzz greedy V={V} L={L}")


@pytest.mark.parametrize("pad", [1, 3, 8, 13])
def test_fuzz_row_stride(isd, pad):
    """Rows padded to ld = V + pad elements (unaligned rows use element loads)."""
    rng = np.random.default_rng(pad)
    C, L, V = 4, 5, 5000
    for dtype in ("bf16", "f32"):
        d, bufs = _make_inputs(rng, C, L, V, dtype, ld=V + pad)
        dd = _device_views(d, bufs, dtype, V)
        ref = oracle_step(d, dtype, "sample", 0.8)
        compare(_run(isd, dd, dict(mode="sample", T=0.8)), ref, label=f"ld pad {pad} {dtype}")


def test_extreme_uniforms_and_temperature(isd):
    rng = np.random.default_rng(5)
    C, L, V = 4, 8, 6000
    for u in (0.0, float(np.nextafter(np.float32(1), np.float32(0)))):
        for T in (0.5, 1.0, 3.0):
            p32 = (3 * rng.standard_normal((C, L, V))).astype(np.float32)
            q32 = (p32 + 0.7 * rng.standard_normal((C, L, V))).astype(np.float32)
            qn32 = (3 * rng.standard_normal((C, L, V))).astype(np.float32)
            d, bufs = _pack(rng, p32, q32, qn32, "bf16", V, ua=u, ur=u, up=u)
            dd = _device_views(d, bufs, "bf16", V)
            ref = oracle_step(d, "bf16", "sample", T)
            compare(_run(isd, dd, dict(mode="sample", T=T)), ref, label=f"u={u} T={T}")


def test_one_hot_and_masked_rows(isd):
    """Rows that are -inf except at a few ids: P, Q of small support; the
    residual and the proposals must never pick a masked id."""
    rng = np.random.default_rng(9)
    C, L, V = 6, 4, 3000
    p32 = np.full((C, L, V), -np.inf, np.float32)
    q32 = np.full((C, L, V), -np.inf, np.float32)
    qn32 = np.full((C, L, V), -np.inf, np.float32)
    for c in range(C):
        for k in range(L):
            sp = rng.choice(V, size=1 + (c % 3), replace=False)
            sq = rng.choice(V, size=1 + (k % 2), replace=False)
            sn = rng.choice(V, size=3, replace=False)
            p32[c, k, sp] = rng.normal(0, 1, sp.size)
            q32[c, k, sq] = rng.normal(0, 1, sq.size)
            qn32[c, k, sn] = rng.normal(0, 1, sn.size)
    x = np.argmax(q32, axis=-1).astype(np.int32)
    d, bufs = _pack(rng, p32, q32, qn32, "bf16", V, x=x)
    dd = _device_views(d, bufs, "bf16", V)
    ref = oracle_step(d, "bf16", "sample", 1.0)
    gpu = _run(isd, dd, dict(mode="sample", T=1.0))
    compare(gpu, ref, label="one-hot")
    refg = oracle_step(d, "bf16", "greedy", 1.0)
    compare(_run(isd, dd, dict(mode="greedy", T=1.0)), refg, label="one-hot greedy")


def test_greedy_exact_ties(isd):
    """Equal maxima (including -0 and +0) resolve to the lowest index."""
    rng = np.random.default_rng(13)
    C, L, V = 4, 8, 9000
    p32 = np.round(rng.normal(0, 1, (C, L, V)) * 2).astype(np.float32) / 2
    top = p32.max(axis=-1, keepdims=True)
    for c in range(C):
        for k in range(L):
            idx = rng.choice(V, size=3, replace=False)
            p32[c, k, idx] = top[c, k] + 1.0
    p32[0, 0, :] = 0.0
    p32[0, 0, 7] = -0.0
    p32[0, 1, :] = -np.inf
    qn32 = p32[:, ::-1].copy()
    g = np.argmax(p32, axis=-1)
    x = np.where(rng.random((C, L)) < 0.8, g, 0).astype(np.int32)
    d, bufs = _pack(rng, p32, p32.copy(), qn32, "bf16", V, x=x)
    dd = _device_views(d, bufs, "bf16", V)
    refg = oracle_step(d, "bf16", "greedy", 1.0)
    compare(_run(isd, dd, dict(mode="greedy", T=1.0)), refg, label="ties")


def test_identical_rows_accept_all_and_determinism(isd):
    """p and q the same buffer: every ratio is exactly 1 and every proposal is
    kept; ten repeated launches give bitwise-identical outputs."""
    import torch
    rng = np.random.default_rng(21)
    C, L, V = 16, 8, 151936
    d, bufs = _make_inputs(rng, C, L, V, "bf16")
    dd = _device_views(d, bufs, "bf16", V)
    dd["ua"] = torch.full_like(dd["ua"], float(np.nextafter(np.float32(1), np.float32(0))))
    o = isd.step(dd["p"], dd["p"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"])
    torch.cuda.synchronize()
    h = to_host(o)
    assert np.all(h["accept_len"] == L) and np.all(h["n_emitted"] == L)
    np.testing.assert_array_equal(h["out_tokens"], d["x"])
    assert np.all(h["alpha"] == 1.0)
    np.testing.assert_array_equal(h["p_x"], h["q_x"])
    dd2 = _device_views(d, bufs, "bf16", V)
    first = _run(isd, dd2, dict(mode="sample", T=1.0))
    for _ in range(9):
        again = _run(isd, dd2, dict(mode="sample", T=1.0))
        for key in first:
            np.testing.assert_array_equal(first[key], again[key], err_msg=key)


def test_out_of_range_proposal_is_flagged_not_faulting(isd):
    import torch
    rng = np.random.default_rng(3)
    C, L, V = 2, 4, 4096
    d, bufs = _make_inputs(rng, C, L, V, "bf16")
    d["x"][1, 2] = V + 5
    d["x"][0, 0] = -3
    dd = _device_views(d, bufs, "bf16", V)
    ws = isd.workspace(isd.make_shape(dd["p"]))
    isd.step(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"], ws=ws)
    with pytest.raises(isd.IsdError, match="out of range"):
        isd.check_device_error(ws)
    isd.check_device_error(ws)      # the word was cleared
    torch.cuda.synchronize()
    ws.zero_()


def test_workspace_returns_to_zero_across_shapes(isd):
    """The workspace contract: zero-filled before first use, zero again after
    every call, whatever the shape, mode or entry point, so one workspace can
    serve calls of different shapes in turn.  (64, 8, 60000) makes 2304 step
    items, so its last 512 take tickets from the launch-wide counter, which
    must be re-armed to zero as well."""
    import torch
    rng = np.random.default_rng(17)
    shapes = [(8, 8, 10000), (64, 8, 4096), (3, 16, 151936), (1, 4, 1000), (64, 8, 30000),
              (64, 8, 60000)]
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    for C, L, V in shapes:
        d, bufs = _make_inputs(rng, C, L, V, "bf16")
        dd = _device_views(d, bufs, "bf16", V)
        for mode in ("sample", "greedy"):
            isd.step(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"],
                     mode=mode, ws=ws)
            isd.verify_step(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], mode=mode, ws=ws)
            isd.propose(dd["qn"], dd["up"], mode=mode, ws=ws)
            isd.alpha(dd["p"], dd["q"], dd["x"], mode=mode, ws=ws)
            torch.cuda.synchronize()
            nz = torch.nonzero(ws).flatten()[:8].tolist()
            assert not nz, f"workspace not zero after C={C} L={L} V={V} {mode}: bytes {nz}"


def test_extend_layout_matches_dense(isd):
    """Anchor and mask rows interleaved per sequence ([C, 2L, V], as one extend
    forward produces them) give bitwise the same results as dense tensors."""
    import torch
    rng = np.random.default_rng(31)
    C, L, V = 6, 8, 20000
    d, bufs = _make_inputs(rng, C, L, V, "bf16")
    dense = _device_views(d, bufs, "bf16", V)
    ext_bits = np.empty((C, 2 * L, V), np.uint16)
    ext_bits[:, :L] = d["p"]
    ext_bits[:, L:] = d["qn"]
    ext = torch.from_numpy(ext_bits.view(np.int16)).cuda().view(torch.bfloat16)
    prev_bits = np.zeros((C, 2 * L, V), np.uint16)   # the previous extend output's mask rows
    prev_bits[:, L:] = d["q"]
    prev = torch.from_numpy(prev_bits.view(np.int16)).cuda().view(torch.bfloat16)
    a = _run(isd, dense, dict(mode="sample", T=1.0))
    with pytest.raises(ValueError):
        isd.step(ext[:, :L], dense["q"], dense["x"], dense["ua"], dense["ur"], ext[:, L:],
                 dense["up"])
    o = isd.step(ext[:, :L], prev[:, L:], dense["x"], dense["ua"], dense["ur"], ext[:, L:],
                 dense["up"])
    torch.cuda.synchronize()
    b = to_host(o)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
    compare(b, oracle_step(d, "bf16", "sample", 1.0), label="extend layout")
