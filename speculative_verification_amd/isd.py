"""ctypes binding of libisd (include/isd.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libisd.  Tensors are torch device tensors; the calls enqueue on
torch's current stream and return without synchronising.  A missing or
unloadable library raises immediately; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libisd.so")

ISD_OK, ISD_ERR_ARG, ISD_ERR_UNSUPPORTED, ISD_ERR_WORKSPACE, ISD_ERR_DEVICE = range(5)
DTYPE_BF16, DTYPE_F32 = 0, 1
MODE_SAMPLE, MODE_GREEDY = 0, 1
SAMPLER_CDF, SAMPLER_GUMBEL = 0, 1

_STATUS_NAMES = {ISD_ERR_ARG: "ISD_ERR_ARG", ISD_ERR_UNSUPPORTED: "ISD_ERR_UNSUPPORTED",
                 ISD_ERR_WORKSPACE: "ISD_ERR_WORKSPACE", ISD_ERR_DEVICE: "ISD_ERR_DEVICE"}


class IsdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("C", ctypes.c_int32), ("L", ctypes.c_int32), ("V", ctypes.c_int32),
                ("ld", ctypes.c_int64), ("dtype", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("temperature", ctypes.c_float), ("ldc", ctypes.c_int64),
                ("relax", ctypes.c_float), ("q_onehot", ctypes.c_int32),
                ("sampler", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_float)]


_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
_SIGS = {
    "isd_workspace_bytes": (_sz, [ctypes.POINTER(Shape)]),
    "isd_verify_step": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 11 + [_vp, _sz, _vp]),
    "isd_propose": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 4 + [_vp, _sz, _vp]),
    "isd_alpha": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 5 + [_vp, _sz, _vp]),
    "isd_step": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 15 + [_vp, _sz, _vp]),
    "isd_step_masked": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 17 + [_vp, _sz, _vp]),
    "isd_propose_masked": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 5 + [_vp, _sz, _vp]),
    "isd_decode_masks": (ctypes.c_int, [_i32, _i32] + [_vp] * 4 + [_vp]),
    "isd_decode_commit": (ctypes.c_int, [_i32, _i32] + [_vp] * 6 + [_i64, _vp, _vp, _vp]),
    "isd_lm_head": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "isd_lm_head_packed": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "isd_lm_head_pack": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "isd_check_device_error": (ctypes.c_int, [_vp, _sz, _vp]),
    "isd_set_tuning": (ctypes.c_int, [_i32, _i32, _i32, _i64]),
    "isd_set_trunc_tuning": (ctypes.c_int, [_i32]),
    "isd_lora_pack": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "isd_lm_head_stats": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, ctypes.c_float, _vp, _vp, _vp,
                                         _sz, _vp]),
    "isd_step_fused": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 10 + [_i64, _i64] +
                       [_vp] * 8 + [_vp, _sz, _vp]),
    "isd_lora_gemm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _sz,
                                     _vp]),
    "isd_gemm_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "isd_read_probe": (ctypes.c_int, [_vp, _sz, _i32, _vp, _vp]),
    "isd_step_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape)] + [_vp] * 16 + [_vp]),
    "isd_last_error": (ctypes.c_char_p, []),
}

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded libisd; raises if it is not built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"{LIB_PATH} is not built: run "
                                       "`python -m speculative_verification_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGS.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def _check(status: int):
    if status != ISD_OK:
        raise IsdError(status, lib().isd_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _logits_layout(t: torch.Tensor):
    """(C, L, V, ld, ldc, dtype code) of a [C, L, V] logits view whose rows are
    contiguous: row (c, k) starts at element c*stride(0) + k*stride(1)."""
    if t.dim() != 3:
        raise ValueError("logits must be [C, L, V]")
    if t.dtype == torch.bfloat16:
        code = DTYPE_BF16
    elif t.dtype == torch.float32:
        code = DTYPE_F32
    else:
        raise ValueError(f"unsupported logits dtype {t.dtype}")
    C, L, V = t.shape
    if t.stride(2) != 1 and V > 1:
        raise ValueError("logits rows must be contiguous")
    ld = int(t.stride(1)) if L > 1 else V
    ld = max(ld, V)
    ldc = int(t.stride(0)) if C > 1 else L * ld
    if ldc < L * ld:
        raise ValueError("sequences of a logits view must not overlap (stride(0) >= L*stride(1))")
    return C, L, V, ld, ldc, code


def _sampler_code(sampler) -> int:
    if sampler in ("cdf", SAMPLER_CDF):
        return SAMPLER_CDF
    if sampler in ("gumbel", SAMPLER_GUMBEL):
        return SAMPLER_GUMBEL
    raise ValueError(f"unknown sampler {sampler!r}")


def make_shape(logits: torch.Tensor, mode: int = MODE_SAMPLE, temperature: float = 1.0,
               relax: float = 0.0, q_onehot: bool = False, sampler="cdf", top_k: int = 0,
               top_p: float = 1.0) -> Shape:
    """Shape of a call on `logits` [C, L, V]; top_k = 0 and top_p >= 1 mean no
    truncation."""
    C, L, V, ld, ldc, code = _logits_layout(logits)
    tp = 0.0 if top_p >= 1.0 else float(top_p)
    return Shape(C, L, V, ld, code, mode, float(temperature), ldc, float(relax),
                 int(bool(q_onehot)), _sampler_code(sampler), int(top_k), tp)


def _same_layout(ref: Shape, t, name: str, mode: int, temperature: float):
    """Every logits tensor of a call is read with the layout of the first."""
    if t is None:
        return
    s = make_shape(t, mode, temperature)
    if (s.C, s.L, s.V, s.ld, s.ldc, s.dtype) != (ref.C, ref.L, ref.V, ref.ld, ref.ldc, ref.dtype):
        raise ValueError(f"{name} must have the same shape, dtype and strides as the anchor logits")


def _mode_code(mode) -> int:
    if mode in ("sample", MODE_SAMPLE):
        return MODE_SAMPLE
    if mode in ("greedy", MODE_GREEDY):
        return MODE_GREEDY
    raise ValueError(f"unknown mode {mode!r}")


def workspace_bytes(shape: Shape) -> int:
    n = lib().isd_workspace_bytes(ctypes.byref(shape))
    if n == 0:
        _check(ISD_ERR_ARG)
    return int(n)


_ws_cache: dict = {}


def workspace(shape: Shape, device=None) -> torch.Tensor:
    """A zero-filled workspace for `shape`, cached per device (one per thread of use)."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    need = workspace_bytes(shape)
    key = (device, threading.get_ident())
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _out(out, key, shape, dtype, device):
    t = None if out is None else out.get(key)
    if t is None:
        t = torch.empty(shape, dtype=dtype, device=device)
    return t


def verify_step(p, q, x, ua, ur, *, mode="sample", temperature=1.0, relax=0.0, q_onehot=False,
                sampler="cdf", top_k=0, top_p=1.0, out=None, ws=None):
    """Verify proposals x [C, L] against anchor rows p (and proposal rows q;
    None with q_onehot)."""
    m = _mode_code(mode)
    shape = make_shape(p, m, temperature, relax, q_onehot, sampler, top_k, top_p)
    if m == MODE_SAMPLE:
        _same_layout(shape, q, "q", m, temperature)
    C, L, dev = shape.C, shape.L, p.device
    o = dict(accept_len=_out(out, "accept_len", (C,), torch.int32, dev),
             out_tokens=_out(out, "out_tokens", (C, L), torch.int32, dev),
             n_emitted=_out(out, "n_emitted", (C,), torch.int32, dev),
             p_x=_out(out, "p_x", (C, L), torch.float32, dev),
             q_x=_out(out, "q_x", (C, L), torch.float32, dev),
             alpha=_out(out, "alpha", (C,), torch.float32, dev))
    ws = workspace(shape, dev) if ws is None else ws
    _check(lib().isd_verify_step(ctypes.byref(shape), _ptr(p), _ptr(q), _ptr(x), _ptr(ua), _ptr(ur),
                                 _ptr(o["accept_len"]), _ptr(o["out_tokens"]), _ptr(o["n_emitted"]),
                                 _ptr(o["p_x"]), _ptr(o["q_x"]), _ptr(o["alpha"]),
                                 _ptr(ws), ws.numel(), _stream()))
    return o


def propose(qn, up, *, mode="sample", temperature=1.0, top_k=0, top_p=1.0, out=None, ws=None):
    """Draw the next proposals [C, L] from the mask-position rows qn."""
    m = _mode_code(mode)
    shape = make_shape(qn, m, temperature, top_k=top_k, top_p=top_p)
    C, L, dev = shape.C, shape.L, qn.device
    o = dict(next_tokens=_out(out, "next_tokens", (C, L), torch.int32, dev),
             qnext_x=_out(out, "qnext_x", (C, L), torch.float32, dev))
    ws = workspace(shape, dev) if ws is None else ws
    _check(lib().isd_propose(ctypes.byref(shape), _ptr(qn), _ptr(up), _ptr(o["next_tokens"]),
                             _ptr(o["qnext_x"]), _ptr(ws), ws.numel(), _stream()))
    return o


def alpha(p, q, x, *, mode="sample", temperature=1.0, q_onehot=False, top_k=0, top_p=1.0,
          out=None, ws=None):
    """Introspective acceptance rate per sequence and its batch mean."""
    m = _mode_code(mode)
    shape = make_shape(p, m, temperature, 0.0, q_onehot, top_k=top_k, top_p=top_p)
    if m == MODE_SAMPLE:
        _same_layout(shape, q, "q", m, temperature)
    dev = p.device
    o = dict(alpha=_out(out, "alpha", (shape.C,), torch.float32, dev),
             alpha_mean=_out(out, "alpha_mean", (1,), torch.float32, dev))
    ws = workspace(shape, dev) if ws is None else ws
    _check(lib().isd_alpha(ctypes.byref(shape), _ptr(p), _ptr(q), _ptr(x), _ptr(o["alpha"]),
                           _ptr(o["alpha_mean"]), _ptr(ws), ws.numel(), _stream()))
    return o


class StepCall:
    """Pre-marshalled isd_step call: fixed shapes and output buffers, so that a
    timing loop pays one ctypes call per step."""

    def __init__(self, p, q, x, ua, ur, qn, up, *, mode="sample", temperature=1.0, relax=0.0,
                 q_onehot=False, sampler="cdf", top_k=0, top_p=1.0, out=None, ws=None):
        m = _mode_code(mode)
        self.shape = make_shape(p, m, temperature, relax, q_onehot, sampler, top_k, top_p)
        _same_layout(self.shape, qn, "qn", m, temperature)
        if m == MODE_SAMPLE:
            _same_layout(self.shape, q, "q", m, temperature)
        C, L, dev = self.shape.C, self.shape.L, p.device
        self.out = dict(accept_len=_out(out, "accept_len", (C,), torch.int32, dev),
                        out_tokens=_out(out, "out_tokens", (C, L), torch.int32, dev),
                        n_emitted=_out(out, "n_emitted", (C,), torch.int32, dev),
                        p_x=_out(out, "p_x", (C, L), torch.float32, dev),
                        q_x=_out(out, "q_x", (C, L), torch.float32, dev),
                        alpha=_out(out, "alpha", (C,), torch.float32, dev),
                        next_tokens=_out(out, "next_tokens", (C, L), torch.int32, dev),
                        qnext_x=_out(out, "qnext_x", (C, L), torch.float32, dev))
        self.ws = workspace(self.shape, dev) if ws is None else ws
        self._fn = lib().isd_step
        self._shape_ref = ctypes.byref(self.shape)
        self.bind_out(self.out)
        self.bind(p, q, x, ua, ur, qn, up)

    def bind(self, p, q, x, ua, ur, qn, up):
        """Point the call at new input tensors of the same shapes."""
        self._head = [_ptr(p), _ptr(q), _ptr(x), _ptr(ua), _ptr(ur), _ptr(qn), _ptr(up)]

    def bind_out(self, o: dict):
        """Point the call at other output tensors of the same shapes (every key
        of the constructor's outputs); later calls write there."""
        C, L = self.shape.C, self.shape.L
        for key, shape in (("accept_len", (C,)), ("out_tokens", (C, L)), ("n_emitted", (C,)),
                           ("p_x", (C, L)), ("q_x", (C, L)), ("alpha", (C,)),
                           ("next_tokens", (C, L)), ("qnext_x", (C, L))):
            if tuple(o[key].shape) != shape or not o[key].is_contiguous():
                raise ValueError(f"output {key} must be a contiguous {shape} tensor")
        self.out = o
        self._tail = [_ptr(o["accept_len"]), _ptr(o["out_tokens"]), _ptr(o["n_emitted"]),
                      _ptr(o["p_x"]), _ptr(o["q_x"]), _ptr(o["alpha"]), _ptr(o["next_tokens"]),
                      _ptr(o["qnext_x"]), _ptr(self.ws), self.ws.numel()]

    def __call__(self, stream=None):
        s = _stream() if stream is None else ctypes.c_void_p(stream)
        _check(self._fn(self._shape_ref, *self._head, *self._tail, s))
        return self.out


def step(p, q, x, ua, ur, qn, up, *, mode="sample", temperature=1.0, relax=0.0, q_onehot=False,
         sampler="cdf", top_k=0, top_p=1.0, out=None, ws=None):
    """One fused ISD step (verify + propose in one launch)."""
    return StepCall(p, q, x, ua, ur, qn, up, mode=mode, temperature=temperature, relax=relax,
                    q_onehot=q_onehot, sampler=sampler, top_k=top_k, top_p=top_p, out=out,
                    ws=ws)()


def step_noalloc(p, q, x, ua, ur, qn, up, *, mode="sample", temperature=1.0, relax=0.0,
                 q_onehot=False, sampler="cdf", top_k=0, top_p=1.0, out=None, device_error=None):
    """isd_step on the library's own device scratch (no workspace is passed
    or allocated by the library).  device_error: optional int32 [1] device
    tensor that receives the step's device error bits."""
    m = _mode_code(mode)
    shape = make_shape(p, m, temperature, relax, q_onehot, sampler, top_k, top_p)
    _same_layout(shape, qn, "qn", m, temperature)
    if m == MODE_SAMPLE:
        _same_layout(shape, q, "q", m, temperature)
    C, L, dev = shape.C, shape.L, p.device
    o = dict(accept_len=_out(out, "accept_len", (C,), torch.int32, dev),
             out_tokens=_out(out, "out_tokens", (C, L), torch.int32, dev),
             n_emitted=_out(out, "n_emitted", (C,), torch.int32, dev),
             p_x=_out(out, "p_x", (C, L), torch.float32, dev),
             q_x=_out(out, "q_x", (C, L), torch.float32, dev),
             alpha=_out(out, "alpha", (C,), torch.float32, dev),
             next_tokens=_out(out, "next_tokens", (C, L), torch.int32, dev),
             qnext_x=_out(out, "qnext_x", (C, L), torch.float32, dev))
    _check(lib().isd_step_noalloc(ctypes.byref(shape), _ptr(p), _ptr(q), _ptr(x), _ptr(ua),
                                  _ptr(ur), _ptr(qn), _ptr(up), _ptr(o["accept_len"]),
                                  _ptr(o["out_tokens"]), _ptr(o["n_emitted"]), _ptr(o["p_x"]),
                                  _ptr(o["q_x"]), _ptr(o["alpha"]), _ptr(o["next_tokens"]),
                                  _ptr(o["qnext_x"]), _ptr(device_error), _stream()))
    return o


def step_masked(p, q, x, ua, ur, qn, up, verify_mask=None, propose_mask=None, *, mode="sample",
                temperature=1.0, relax=0.0, q_onehot=False, sampler="cdf", top_k=0, top_p=1.0,
                out=None, ws=None):
    """isd_step with per-sequence verify / propose masks (int32 [C]; None = all)."""
    m = _mode_code(mode)
    shape = make_shape(p, m, temperature, relax, q_onehot, sampler, top_k, top_p)
    _same_layout(shape, qn, "qn", m, temperature)
    if m == MODE_SAMPLE:
        _same_layout(shape, q, "q", m, temperature)
    C, L, dev = shape.C, shape.L, p.device
    o = dict(accept_len=_out(out, "accept_len", (C,), torch.int32, dev),
             out_tokens=_out(out, "out_tokens", (C, L), torch.int32, dev),
             n_emitted=_out(out, "n_emitted", (C,), torch.int32, dev),
             p_x=_out(out, "p_x", (C, L), torch.float32, dev),
             q_x=_out(out, "q_x", (C, L), torch.float32, dev),
             alpha=_out(out, "alpha", (C,), torch.float32, dev),
             next_tokens=_out(out, "next_tokens", (C, L), torch.int32, dev),
             qnext_x=_out(out, "qnext_x", (C, L), torch.float32, dev))
    ws = workspace(shape, dev) if ws is None else ws
    _check(lib().isd_step_masked(
        ctypes.byref(shape), _ptr(p), _ptr(q), _ptr(x), _ptr(ua), _ptr(ur), _ptr(qn), _ptr(up),
        _ptr(verify_mask), _ptr(propose_mask), _ptr(o["accept_len"]), _ptr(o["out_tokens"]),
        _ptr(o["n_emitted"]), _ptr(o["p_x"]), _ptr(o["q_x"]), _ptr(o["alpha"]),
        _ptr(o["next_tokens"]), _ptr(o["qnext_x"]), _ptr(ws), ws.numel(), _stream()))
    return o


def propose_masked(rows, u, mask=None, *, mode="sample", temperature=1.0, top_k=0, top_p=1.0,
                   out=None, ws=None):
    """isd_propose with a per-sequence mask (int32 [C]; None = all)."""
    m = _mode_code(mode)
    shape = make_shape(rows, m, temperature, top_k=top_k, top_p=top_p)
    C, L, dev = shape.C, shape.L, rows.device
    o = dict(next_tokens=_out(out, "next_tokens", (C, L), torch.int32, dev),
             qnext_x=_out(out, "qnext_x", (C, L), torch.float32, dev))
    ws = workspace(shape, dev) if ws is None else ws
    _check(lib().isd_propose_masked(ctypes.byref(shape), _ptr(rows), _ptr(u), _ptr(mask),
                                    _ptr(o["next_tokens"]), _ptr(o["qnext_x"]), _ptr(ws),
                                    ws.numel(), _stream()))
    return o


def decode_masks(L, state, accept_len, bonus_mask, anchor_mask):
    """Bonus and anchor draw masks of one decoding-loop step."""
    _check(lib().isd_decode_masks(state.numel(), L, _ptr(state), _ptr(accept_len),
                                  _ptr(bonus_mask), _ptr(anchor_mask), _stream()))


def decode_commit(L, state, accept_len, out_tokens, bonus, anchor, tokens, forwards,
                  history=None):
    """Close one decoding-loop step: append tokens, count, advance the state."""
    cap = 0 if history is None else history.shape[1]
    _check(lib().isd_decode_commit(state.numel(), L, _ptr(state), _ptr(accept_len),
                                   _ptr(out_tokens), _ptr(bonus), _ptr(anchor), _ptr(history),
                                   cap, _ptr(tokens), _ptr(forwards), _stream()))


class Decoder:
    """Device-resident state of the multi-step decoding loop for C sequences
    with L proposals per step (stride L + 1).

    Every sequence starts in recovery (state 0).  ``step`` takes one
    forward's rows, all shaped [C, L + 1, V] with one layout: p (rows 0..L-1
    verify, row L is the bonus anchor, row 0 the anchor of a recovering
    sequence), q and qn (rows 0..L-1 used); and the uniforms ua, ur, up
    [C, L], ub, uz [C].  Each step is five library calls on the current
    stream and never synchronises."""

    def __init__(self, C, L, device, *, history=0, mode="sample", temperature=1.0):
        self.C, self.L, self.mode, self.temperature = C, L, mode, temperature
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)  # noqa: E731
        self.state = z((C,), torch.int32)
        self.x = z((C, L), torch.int32)
        self.tokens = z((C,), torch.int64)
        self.forwards = z((C,), torch.int64)
        self.history = z((C, history), torch.int32) if history else None
        self.bonus_mask = z((C,), torch.int32)
        self.anchor_mask = z((C,), torch.int32)
        self.last = None

    def step(self, p, q, qn, ua, ur, up, ub, uz):
        L, C = self.L, self.C
        kw = dict(mode=self.mode, temperature=self.temperature)
        o = step_masked(p[:, :L], q[:, :L], self.x, ua, ur, qn[:, :L], up,
                        verify_mask=self.state, **kw)
        state_before = self.state.clone()
        decode_masks(L, self.state, o["accept_len"], self.bonus_mask, self.anchor_mask)
        b = propose_masked(p[:, L:L + 1], ub.view(C, 1), self.bonus_mask, **kw)
        a = propose_masked(p[:, 0:1], uz.view(C, 1), self.anchor_mask, **kw)
        decode_commit(L, self.state, o["accept_len"], o["out_tokens"], b["next_tokens"],
                      a["next_tokens"], self.tokens, self.forwards, self.history)
        self.x.copy_(o["next_tokens"])
        self.last = dict(o, state_before=state_before, bonus=b["next_tokens"][:, 0],
                         anchor=a["next_tokens"][:, 0])
        return self.last


def lm_head(h, w, out=None):
    """logits [M, N] = h [M, K] @ w [K, N] (bf16, fp32 accumulation on MFMA)."""
    if h.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise ValueError("lm_head takes bf16 tensors")
    if not (h.is_contiguous() and w.is_contiguous()):
        raise ValueError("lm_head takes contiguous tensors")
    M, K = h.shape
    K2, N = w.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=h.device)
    _check(lib().isd_lm_head(_ptr(h), _ptr(w), M, K, N, _ptr(out), None, 0, _stream()))
    return out


def lm_head_pack(w):
    """wt [N, K] = w [K, N]^T, the head layout of lm_head_packed (a one-time pack)."""
    if w.dtype != torch.bfloat16 or not w.is_contiguous():
        raise ValueError("lm_head_pack takes a contiguous bf16 tensor")
    K, N = w.shape
    wt = torch.empty((N, K), dtype=torch.bfloat16, device=w.device)
    _check(lib().isd_lm_head_pack(_ptr(w), K, N, _ptr(wt), _stream()))
    return wt


def gemm_workspace(M: int, K: int, N: int, device="cuda"):
    """A zero-filled workspace for lm_head_packed / lora_gemm on an M x N output
    with a (first) K segment of K, or None when the K split does not apply."""
    n = lib().isd_gemm_workspace_bytes(M, K, N)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def _ws(ws):
    if ws is None:
        return None, 0
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    return _ptr(ws), ws.numel()


def lm_head_packed(h, wt, out=None, workspace=None):
    """logits [M, N] = h [M, K] @ wt [N, K]^T (bf16, fp32 accumulation on MFMA).
    `workspace` (from gemm_workspace) lets the GEMM halve its last partial round
    along K."""
    if h.dtype != torch.bfloat16 or wt.dtype != torch.bfloat16:
        raise ValueError("lm_head_packed takes bf16 tensors")
    if not (h.is_contiguous() and wt.is_contiguous()):
        raise ValueError("lm_head_packed takes contiguous tensors")
    M, K = h.shape
    N, K2 = wt.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=h.device)
    _check(lib().isd_lm_head_packed(_ptr(h), _ptr(wt), M, K, N, _ptr(out), *_ws(workspace), _stream()))
    return out


def check_device_error(ws: torch.Tensor):
    """Synchronise and raise IsdError if a kernel flagged undefined input or
    an expired wait.  A launch that flagged one may have left records in the
    workspace, so the workspace is zero-filled again before the error is
    raised (the library's contract for ISD_ERR_DEVICE)."""
    status = lib().isd_check_device_error(_ptr(ws), ws.numel(), _stream())
    if status == ISD_ERR_DEVICE:
        message = lib().isd_last_error().decode()
        ws.zero_()
        torch.cuda.current_stream().synchronize()
        raise IsdError(status, message)
    _check(status)


def read_probe(buf: torch.Tensor, sink: torch.Tensor, tiles_per_group: int = 38):
    """One streaming read of `buf` (a contiguous device tensor, 16-byte
    aligned, a multiple of 4096 bytes) with the step's tile loader."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().isd_read_probe(_ptr(buf), nbytes, tiles_per_group, _ptr(sink), _stream()))


def set_tuning(segments: int = 0, resid_segments: int = 0, spin_limit: int = 0,
               propose_segments: int = 0):
    """Process-wide decomposition knobs (0 = automatic)."""
    _check(lib().isd_set_tuning(segments, propose_segments, resid_segments, spin_limit))


def set_trunc_tuning(segments: int = 0):
    """Workgroups per row of the truncated (top-k) path (0 = automatic)."""
    _check(lib().isd_set_trunc_tuning(segments))


def lora_pack(w: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """(W [N, K] | B [N, r]) as one bf16 tensor [N, K + r] for lora_gemm."""
    if w.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise ValueError("w and b must be bf16")
    N, K = w.shape
    r = b.shape[1]
    if b.shape[0] != N or not (w.is_contiguous() and b.is_contiguous()):
        raise ValueError("w [N, K] and b [N, r] must be contiguous with the same N")
    wcat = torch.empty((N, K + r), dtype=torch.bfloat16, device=w.device)
    _check(lib().isd_lora_pack(_ptr(w), _ptr(b), N, K, r, _ptr(wcat), _stream()))
    return wcat


def lora_gemm(x: torch.Tensor, a: torch.Tensor, wcat: torch.Tensor, mask=None, *, out=None,
              t=None, workspace=None):
    """h = x W^T + [mask] (x A^T) B^T with wcat = lora_pack(W, B); returns (h, t).
    `workspace` (from gemm_workspace(M, K, N)) lets the GEMM halve its last
    partial round along K."""
    for name, v in (("x", x), ("a", a), ("wcat", wcat)):
        if v.dtype != torch.bfloat16 or not v.is_contiguous():
            raise ValueError(f"{name} must be contiguous bf16")
    M, K = x.shape
    r = a.shape[0]
    N = wcat.shape[0]
    if a.shape[1] != K or wcat.shape[1] != K + r:
        raise ValueError("shapes must be x [M, K], a [r, K], wcat [N, K + r]")
    if mask is not None and (mask.dtype != torch.int32 or mask.numel() != M):
        raise ValueError("mask must be int32 [M]")
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if out is None else out
    t = torch.empty((M, r), dtype=torch.bfloat16, device=x.device) if t is None else t
    _check(lib().isd_lora_gemm(_ptr(x), _ptr(a), _ptr(wcat), _ptr(mask), M, K, N, r, _ptr(t),
                               _ptr(out), *_ws(workspace), _stream()))
    return out, t


STATS_TILE = 128


def lm_head_stats(h, wt, temperature=1.0, out=None, stats=None, workspace=None):
    """logits [M, N] = h @ wt^T like lm_head_packed, plus the softmax partials
    of every (row, 128-column tile): stats [M, ceil(N / 128), 2] fp32 (e, s).
    `workspace` (from gemm_workspace) as for lm_head_packed."""
    if h.dtype != torch.bfloat16 or wt.dtype != torch.bfloat16:
        raise ValueError("lm_head_stats takes bf16 tensors")
    if not (h.is_contiguous() and wt.is_contiguous()):
        raise ValueError("lm_head_stats takes contiguous tensors")
    M, K = h.shape
    N, K2 = wt.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    nt = (N + STATS_TILE - 1) // STATS_TILE
    out = torch.empty((M, N), dtype=torch.bfloat16, device=h.device) if out is None else out
    stats = torch.empty((M, nt, 2), dtype=torch.float32, device=h.device) if stats is None else stats
    _check(lib().isd_lm_head_stats(_ptr(h), _ptr(wt), M, K, N, float(temperature), _ptr(out),
                                   _ptr(stats), *_ws(workspace), _stream()))
    return out, stats


def _stats_layout(st, C, L, nt, name):
    """(stats_ld, stats_ldc) in entries of a [C, L, nt, 2] fp32 view."""
    if st.dtype != torch.float32 or st.dim() != 4 or tuple(st.shape) != (C, L, nt, 2):
        raise ValueError(f"{name} must be fp32 [C, L, ceil(V / 128), 2]")
    if st.stride(3) != 1 or st.stride(2) != 2 or st.stride(1) % 2 or st.stride(0) % 2:
        raise ValueError(f"{name} must have contiguous (e, s) entries")
    return st.stride(1) // 2, st.stride(0) // 2


def step_fused(p, q, x, ua, ur, qn, up, p_stats, q_stats, qn_stats, *, temperature=1.0,
               relax=0.0, q_onehot=False, sampler="cdf", out=None, ws=None):
    """isd_step from the LM head's tile statistics (views [C, L, ceil(V / 128), 2])."""
    shape = make_shape(p, MODE_SAMPLE, temperature, relax, q_onehot, sampler)
    _same_layout(shape, qn, "qn", MODE_SAMPLE, temperature)
    if not q_onehot:
        _same_layout(shape, q, "q", MODE_SAMPLE, temperature)
    C, L, dev = shape.C, shape.L, p.device
    nt = (shape.V + STATS_TILE - 1) // STATS_TILE
    lay = _stats_layout(p_stats, C, L, nt, "p_stats")
    if _stats_layout(qn_stats, C, L, nt, "qn_stats") != lay or (
            not q_onehot and _stats_layout(q_stats, C, L, nt, "q_stats") != lay):
        raise ValueError("the statistics views must share one layout")
    o = dict(accept_len=_out(out, "accept_len", (C,), torch.int32, dev),
             out_tokens=_out(out, "out_tokens", (C, L), torch.int32, dev),
             n_emitted=_out(out, "n_emitted", (C,), torch.int32, dev),
             p_x=_out(out, "p_x", (C, L), torch.float32, dev),
             q_x=_out(out, "q_x", (C, L), torch.float32, dev),
             alpha=_out(out, "alpha", (C,), torch.float32, dev),
             next_tokens=_out(out, "next_tokens", (C, L), torch.int32, dev),
             qnext_x=_out(out, "qnext_x", (C, L), torch.float32, dev))
    ws = workspace(shape, dev) if ws is None else ws
    _check(lib().isd_step_fused(
        ctypes.byref(shape), _ptr(p), _ptr(q), _ptr(x), _ptr(ua), _ptr(ur), _ptr(qn), _ptr(up),
        _ptr(p_stats), _ptr(q_stats), _ptr(qn_stats), lay[0], lay[1], _ptr(o["accept_len"]),
        _ptr(o["out_tokens"]), _ptr(o["n_emitted"]), _ptr(o["p_x"]), _ptr(o["q_x"]),
        _ptr(o["alpha"]), _ptr(o["next_tokens"]), _ptr(o["qnext_x"]), _ptr(ws), ws.numel(),
        _stream()))
    return o
