"""The C ABI on the host: libisd loads, exports every function include/isd.h
declares, and rejects bad arguments synchronously with the documented
status codes.  No call here reaches a kernel launch, so no GPU is needed."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isd.h")

FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced on the host


@pytest.fixture(scope="module")
def isd():
    import speculative_verification_amd as m
    # test_abi_asan.py runs this file again against a build whose host code
    # carries AddressSanitizer
    if os.environ.get("ISD_TEST_LIBRARY"):
        m.isd.LIB_PATH = os.environ["ISD_TEST_LIBRARY"]
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(isd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("isd_verify_step", "isd_propose", "isd_alpha", "isd_step", "isd_lm_head",
                     "isd_workspace_bytes", "isd_last_error", "isd_check_device_error",
                     "isd_set_tuning"):
        assert required in names


def test_library_exports_every_declared_symbol(isd):
    lib = ctypes.CDLL(isd.isd.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def _shape(isd, **kw):
    base = dict(C=4, L=8, V=151936, ld=151936, dtype=0, mode=0, temperature=1.0)
    base.update(kw)
    return isd.Shape(base["C"], base["L"], base["V"], base["ld"], base["dtype"], base["mode"],
                     base["temperature"])


def _verify(isd, shape, ws_bytes=1 << 30, **ptrs):
    args = dict(p=FAKE, q=FAKE, x=FAKE, ua=FAKE, ur=FAKE, al=FAKE, out=FAKE, ne=FAKE)
    args.update(ptrs)
    return isd.lib().isd_verify_step(ctypes.byref(shape), args["p"], args["q"], args["x"],
                                     args["ua"], args["ur"], args["al"], args["out"], args["ne"],
                                     None, None, None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(C=0), 1, "C must be"),
    (dict(L=0), 1, "L must be"),
    (dict(L=65), 1, "L must be"),
    (dict(V=0), 1, "V must be"),
    (dict(ld=100), 1, "ld"),
    (dict(temperature=0.0), 1, "temperature"),
    (dict(temperature=float("nan")), 1, "temperature"),
    (dict(dtype=7), 2, "dtype"),
    (dict(mode=3), 2, "mode"),
])
def test_bad_shapes(isd, kw, status, msg):
    st = _verify(isd, _shape(isd, **kw))
    assert st == status
    assert msg in isd.lib().isd_last_error().decode()


@pytest.mark.parametrize("missing", ["p", "q", "x", "ua", "ur", "al", "out", "ne"])
def test_null_pointers(isd, missing):
    st = _verify(isd, _shape(isd), **{missing: None})
    assert st == 1
    assert "NULL" in isd.lib().isd_last_error().decode()


def test_greedy_ignores_q_and_uniforms(isd):
    # with q/ua/ur NULL in greedy mode the only remaining error is the workspace size
    st = _verify(isd, _shape(isd, mode=1), ws_bytes=16, q=None, ua=None, ur=None)
    assert st == 3


def test_misaligned_pointer(isd):
    st = _verify(isd, _shape(isd), p=ctypes.c_void_p(0x10001))
    assert st == 1 and "aligned" in isd.lib().isd_last_error().decode()


def test_workspace_too_small(isd):
    shape = _shape(isd)
    need = isd.lib().isd_workspace_bytes(ctypes.byref(shape))
    assert need > 0
    st = _verify(isd, shape, ws_bytes=need - 1)
    assert st == 3 and "workspace" in isd.lib().isd_last_error().decode()


def test_workspace_bytes(isd):
    lib = isd.lib()
    small = lib.isd_workspace_bytes(ctypes.byref(_shape(isd, C=1, L=4, V=1000, ld=1000)))
    big = lib.isd_workspace_bytes(ctypes.byref(_shape(isd, C=256, L=16)))
    assert 0 < small < big
    assert big % 256 == 0
    assert lib.isd_workspace_bytes(ctypes.byref(_shape(isd, C=0))) == 0
    assert lib.isd_workspace_bytes(None) == 0


def test_propose_alpha_step_validation(isd):
    lib = isd.lib()
    shape = _shape(isd)
    assert lib.isd_propose(ctypes.byref(shape), None, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.isd_alpha(ctypes.byref(shape), FAKE, FAKE, None, FAKE, None, FAKE, 1 << 30, None) == 1
    args = [FAKE] * 15
    args[5] = None                                   # qnext_logits
    assert lib.isd_step(ctypes.byref(shape), *args, FAKE, 1 << 30, None) == 1
    assert "qnext_logits" in lib.isd_last_error().decode()


def test_gemm_workspace_bytes(isd):
    """The K split of the ping-pong GEMM's last partial round (256 CUs): it
    applies when the 256 x 256 tiles past the whole rounds fill at most half a
    round and number a multiple of 4; the workspace holds a 128-byte counter
    and two fp32 256 x 256 halves per split tile."""
    f = isd.lib().isd_gemm_workspace_bytes
    per_tile = 128 + 2 * 256 * 256 * 4
    assert f(1024, 4096, 24576) == 128 * per_tile     # 384 tiles: 256 whole, 128 split
    assert f(1000, 256, 24389) == 128 * per_tile      # ragged rows and columns, same tiles
    assert f(1024, 4096, 151936) == 72 * per_tile     # 2376 tiles: 72 past nine rounds
    assert f(1024, 4096, 16384) == 0                  # exactly one round
    assert f(1024, 4096, 16640) == 4 * per_tile       # 260 tiles
    assert f(1024, 4096, 16448) == 4 * per_tile       # 260 tiles, the last one ragged
    assert f(1024, 4096, 8192) == 0                   # fewer tiles than CUs
    assert f(768, 4096, 22016) == 0                   # 258 tiles: 2 past the round
    assert f(1024, 4096, 26624) == 0                  # 416 tiles: 160 past, over half a round
    assert f(1024, 64, 24576) == 0                    # one K step cannot be halved
    assert f(0, 4096, 24576) == 0 and f(1024, 100, 24576) == 0


def test_gemm_workspace_alignment_is_checked(isd):
    lib = isd.lib()
    odd = ctypes.c_void_p(0x10080)                    # 128-byte, not 256-byte, aligned
    assert lib.isd_lm_head_packed(FAKE, FAKE, 1024, 4096, 24576, FAKE, odd, 1 << 30, None) == 1
    assert "workspace" in lib.isd_last_error().decode()
    assert lib.isd_lora_gemm(FAKE, FAKE, FAKE, None, 1024, 4096, 24576, 128, FAKE, FAKE, odd, 1 << 30,
                             None) == 1
    assert "workspace" in lib.isd_last_error().decode()


def test_lm_head_validation(isd):
    lib = isd.lib()
    assert lib.isd_lm_head(FAKE, FAKE, 16, 100, 64, FAKE, None, 0, None) == 1
    assert "multiple of 64" in lib.isd_last_error().decode()
    assert lib.isd_lm_head(FAKE, FAKE, 0, 64, 64, FAKE, None, 0, None) == 1
    assert lib.isd_lm_head(None, FAKE, 16, 64, 64, FAKE, None, 0, None) == 1


def test_tuning_validation(isd):
    lib = isd.lib()
    assert lib.isd_set_tuning(-1, 0, 0, 0) == 1
    assert lib.isd_set_tuning(0, 33, 0, 0) == 1
    assert lib.isd_set_tuning(0, 0, 1000, 0) == 1
    assert lib.isd_set_tuning(0, 0, 0, -5) == 1
    assert lib.isd_set_tuning(4, 2, 8, 100) == 0
    assert lib.isd_set_tuning(0, 0, 0, 0) == 0


def test_binding_layout_checks(isd):
    import torch
    t = torch.zeros((2, 3, 10), dtype=torch.bfloat16)
    s = isd.make_shape(t)
    assert (s.C, s.L, s.V, s.ld, s.dtype) == (2, 3, 10, 10, 0)
    padded = torch.zeros((2, 3, 16), dtype=torch.float32)[:, :, :10]
    s = isd.make_shape(padded)
    assert (s.V, s.ld, s.dtype) == (10, 16, 1)
    with pytest.raises(ValueError):
        isd.make_shape(torch.zeros((2, 3, 10), dtype=torch.float16))


def test_sequence_stride(isd):
    import torch
    lib = isd.lib()
    bad = _shape(isd, C=4, L=8, V=1000, ld=1000)
    bad.ldc = 7999                      # below L*ld: sequences would overlap
    assert _verify(isd, bad) == 1 and "ldc" in lib.isd_last_error().decode()
    ext = torch.zeros((3, 2 * 5, 64), dtype=torch.bfloat16)   # [C, 2L, V] extend output
    sp, sq = isd.make_shape(ext[:, :5]), isd.make_shape(ext[:, 5:])
    assert (sp.C, sp.L, sp.V, sp.ld, sp.ldc) == (3, 5, 64, 64, 640)
    assert (sq.ld, sq.ldc) == (64, 640)
    dense = torch.zeros((3, 5, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="same shape"):
        isd.isd._same_layout(sp, dense, "q", 0, 1.0)
    isd.isd._same_layout(sp, ext[:, 5:], "q", 0, 1.0)


def test_masked_and_loop_validation(isd):
    lib = isd.lib()
    shape = _shape(isd)
    # a misaligned mask is rejected before any launch
    args = [FAKE] * 15
    st = lib.isd_step_masked(ctypes.byref(shape), *args[:7], ctypes.c_void_p(0x10002), None,
                             *args[7:], FAKE, 1 << 30, None)
    assert st == 1 and "verify_mask" in lib.isd_last_error().decode()
    st = lib.isd_propose_masked(ctypes.byref(shape), FAKE, FAKE, ctypes.c_void_p(0x10001), FAKE,
                                None, FAKE, 1 << 30, None)
    assert st == 1 and "mask" in lib.isd_last_error().decode()
    assert lib.isd_decode_masks(0, 4, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.isd_decode_masks(4, 65, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.isd_decode_masks(4, 4, None, FAKE, FAKE, FAKE, None) == 1
    assert lib.isd_decode_commit(4, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, 8, FAKE, FAKE,
                                 None) == 1
    assert "history" in lib.isd_last_error().decode()
    assert lib.isd_decode_commit(4, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, -1, FAKE, FAKE,
                                 None) == 1
    assert lib.isd_decode_commit(4, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                                 ctypes.c_void_p(0x10004), FAKE, None) == 1


def test_variant_shape_validation(isd):
    lib = isd.lib()
    bad = _shape(isd)
    bad.relax = -0.5
    assert _verify(isd, bad) == 1 and "relax" in lib.isd_last_error().decode()
    bad = _shape(isd)
    bad.relax = float("inf")
    assert _verify(isd, bad) == 1
    bad = _shape(isd)
    bad.q_onehot = 2
    assert _verify(isd, bad) == 1 and "q_onehot" in lib.isd_last_error().decode()
    for v in (2, -1):
        bad = _shape(isd)
        bad.sampler = v
        assert _verify(isd, bad) == 1 and "sampler" in lib.isd_last_error().decode()
    # truncation: top_k in [0, 64]; top_p needs top_k; 0 or >= 1 turns top_p off
    for k, p_, status, word in ((65, 0.0, 2, "top_k"), (-1, 0.0, 1, "top_k"), (0, 0.9, 2, "top_p"),
                                (8, -0.5, 1, "top_p"), (8, float("nan"), 1, "top_p")):
        bad = _shape(isd)
        bad.top_k, bad.top_p = k, p_
        assert _verify(isd, bad) == status and word in lib.isd_last_error().decode(), (k, p_)
    plain = _shape(isd)
    trunc = _shape(isd)
    trunc.top_k, trunc.top_p = 50, 0.95
    assert lib.isd_workspace_bytes(ctypes.byref(trunc)) > lib.isd_workspace_bytes(ctypes.byref(plain))
    assert lib.isd_set_trunc_tuning(9) == 1 and lib.isd_set_trunc_tuning(0) == 0
    import torch
    s = isd.make_shape(torch.zeros(1, 1, 8), top_k=50, top_p=1.0)
    assert (s.top_k, s.top_p) == (50, 0.0)
    assert isd.make_shape(torch.zeros(1, 1, 8), sampler="gumbel").sampler == 1
    with pytest.raises(ValueError):
        isd.make_shape(torch.zeros(1, 1, 8), sampler="topk")
    # with one-hot proposals q may be NULL: the only remaining error is the workspace size
    ok = _shape(isd)
    ok.q_onehot = 1
    assert _verify(isd, ok, ws_bytes=16, q=None) == 3


def test_fused_and_stats_validation(isd):
    """The statistics path checks its arguments on the host (no compute)."""
    lib = isd.lib()
    sh = _shape(isd)
    args = [FAKE] * 10 + [ctypes.c_int64(1187), ctypes.c_int64(0)] + [FAKE] * 8 + [FAKE, 1 << 30, None]
    bad = list(args)
    bad[10] = ctypes.c_int64(1186)          # fewer than ceil(151936 / 128) entries per row
    assert lib.isd_step_fused(ctypes.byref(sh), *bad) == 1
    assert "stats_ld" in lib.isd_last_error().decode()
    greedy = _shape(isd, mode=1)
    assert lib.isd_step_fused(ctypes.byref(greedy), *args) == 2
    trunc = _shape(isd)
    trunc.top_k = 8
    assert lib.isd_step_fused(ctypes.byref(trunc), *args) == 2
    assert lib.isd_lm_head_stats(FAKE, FAKE, 8, 100, 64, ctypes.c_float(1.0), FAKE, FAKE, None, 0,
                                 None) == 1
    assert lib.isd_lm_head_stats(FAKE, FAKE, 8, 128, 64, ctypes.c_float(0.0), FAKE, FAKE, None, 0,
                                 None) == 1
    assert "temperature" in lib.isd_last_error().decode()
    odd = ctypes.c_void_p(0x10080)
    assert lib.isd_lm_head_stats(FAKE, FAKE, 1024, 4096, 24576, ctypes.c_float(1.0), FAKE, FAKE, odd,
                                 1 << 30, None) == 1
    assert "workspace" in lib.isd_last_error().decode()


@pytest.mark.parametrize("nbytes,tpg,msg", [
    (0, 38, "multiple of 4096"),
    (4095, 38, "multiple of 4096"),
    (4096 * 10 + 2, 38, "multiple of 4096"),
    (4096, 0, "tiles_per_group"),
    (4096, 5000, "tiles_per_group"),
])
def test_read_probe_rejects_bad_sizes(isd, nbytes, tpg, msg):
    st = isd.lib().isd_read_probe(FAKE, nbytes, tpg, FAKE, None)
    assert st == 1
    assert msg in isd.lib().isd_last_error().decode()


def test_read_probe_rejects_misaligned_or_null(isd):
    assert isd.lib().isd_read_probe(ctypes.c_void_p(0x10008), 4096, 38, FAKE, None) == 1
    assert "aligned" in isd.lib().isd_last_error().decode()
    assert isd.lib().isd_read_probe(FAKE, 4096, 38, None, None) == 1
    assert "NULL" in isd.lib().isd_last_error().decode()


def test_step_noalloc_rejects_shapes_beyond_its_scratch(isd):
    # C=256, L=16 with top-k 50 needs about 65 MiB of records: refused before any device call
    shape = isd.Shape(256, 16, 151936, 151936, 0, 0, 1.0, 0, 0.0, 0, 0, 50, 0.0)
    st = isd.lib().isd_step_noalloc(ctypes.byref(shape), *([FAKE] * 15), None, None)
    assert st == 3
    msg = isd.lib().isd_last_error().decode()
    assert "allocation-free" in msg and str(16 << 20) in msg


def test_step_noalloc_validates_pointers_first(isd):
    shape = _shape(isd)
    args = [FAKE] * 15
    args[8] = None                                   # out_tokens
    assert isd.lib().isd_step_noalloc(ctypes.byref(shape), *args, None, None) == 1
    assert "NULL" in isd.lib().isd_last_error().decode()
    args = [FAKE] * 15
    assert isd.lib().isd_step_noalloc(ctypes.byref(shape), *args, ctypes.c_void_p(0x10002),
                                      None) == 1
    assert "device_error" in isd.lib().isd_last_error().decode()
