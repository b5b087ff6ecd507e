"""The allocation-free step (isd_step_noalloc) against isd_step with a
workspace, through the C ABI: two calls in a row on the library's device
scratch, the first at the serving shape and the second smaller, each
bitwise equal to the workspace path on the same inputs (the same kernels),
and the second also against the oracle.  The scratch is left zero-equivalent
between calls (the second, smaller call would otherwise read the first's
counters), and device errors come back through the error-word output."""

import numpy as np
import pytest

from tests.isd_testlib import compare, oracle_step, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def isd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import speculative_verification_amd as isd_mod
    isd_mod.lib()
    isd_mod.set_tuning(0, 0, 0)
    return isd_mod


def _inputs(rng, C, L, V):
    import torch
    from isd_inputs import f32_to_bf16_bits
    p32 = (3 * rng.standard_normal((C, L, V))).astype(np.float32)
    q32 = (p32 + 0.7 * rng.standard_normal((C, L, V))).astype(np.float32)
    qn32 = (3 * rng.standard_normal((C, L, V))).astype(np.float32)
    d = {k: f32_to_bf16_bits(a) for k, a in (("p", p32), ("q", q32), ("qn", qn32))}
    qv = (d["q"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g = -np.log(-np.log(np.clip(rng.random((C, L, V)), 1e-300, 1 - 1e-16)))
    d["x"] = np.argmax(qv + g, axis=-1).astype(np.int32)
    for k in ("ua", "ur", "up"):
        d[k] = rng.random((C, L)).astype(np.float32)
    dev = {}
    for k in ("p", "q", "qn"):
        dev[k] = torch.from_numpy(d[k].view(np.int16)).cuda().view(torch.bfloat16)
    for k in ("x", "ua", "ur", "up"):
        dev[k] = torch.from_numpy(d[k]).cuda()
    return d, dev


def _both(isd, dv):
    import torch
    args = (dv["p"], dv["q"], dv["x"], dv["ua"], dv["ur"], dv["qn"], dv["up"])
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    a = to_host(isd.step_noalloc(*args, device_error=err))
    torch.cuda.synchronize()
    b = to_host(isd.step(*args))
    torch.cuda.synchronize()
    return a, b, int(err.item())


def test_noalloc_matches_the_workspace_path_twice(isd):
    rng = np.random.default_rng(77)
    for C, L, V in ((64, 8, 151936), (4, 4, 5000)):
        d, dv = _inputs(rng, C, L, V)
        a, b, err = _both(isd, dv)
        assert err == 0
        for key in b:
            np.testing.assert_array_equal(a[key], b[key], err_msg=f"C={C} L={L} V={V} {key}")
        if C == 4:
            compare(a, oracle_step(d, "bf16", "sample", 1.0), label="noalloc small")


def test_noalloc_reports_device_errors(isd):
    import torch
    rng = np.random.default_rng(78)
    d, dv = _inputs(rng, 2, 4, 4096)
    dv["x"][1, 2] = 4096 + 5                 # an id out of range: flagged, never read
    err = torch.zeros((1,), dtype=torch.int32, device="cuda")
    isd.step_noalloc(dv["p"], dv["q"], dv["x"], dv["ua"], dv["ur"], dv["qn"], dv["up"],
                     device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    # the word was moved out and cleared: a clean call reports nothing
    dv["x"][1, 2] = 3
    isd.step_noalloc(dv["p"], dv["q"], dv["x"], dv["ua"], dv["ur"], dv["qn"], dv["up"],
                     device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
