"""Benchmark of the fused ISD verify-and-propose step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one isd_step launch over one batch: verification of C*L proposals
(anchor rows p and proposal rows q) plus the draw of the next C*L proposals
(mask rows qn).  The serving workload (C=64, L=8, V=151936, bf16 logits, T=1)
is the default.  Inputs are resident in HBM before timing; steps cycle over
`--sets` distinct logits sets (each larger than the 256 MB Infinity Cache)
with fresh uniforms every step (the tiny workload, --config 1, draws fresh
inputs for every step).  Prints one JSON line.

Order of work: inputs are generated and uploaded; the streaming-read probe
reads a 1 GiB buffer for about 0.4 s (its rate is reported, and the GPU clock
reaches its steady state meanwhile); W untimed steps; K timed steps, each
writing its own output buffers; then the CPU oracle recomputes every sequence
of the first timed steps from the same bytes and uniforms and the outputs of
those launches are compared with it.

Reported:
  value      verified positions per second = C*L / wall-clock time per step
             (the tiny workload reports microseconds per step instead)
  roofline   the step kernel against the HBM peak: algorithmic bytes per
             launch (every logit read once: 3*C*L*V*2 B) over the kernel's
             average duration (events on its stream around launches 2..K,
             which run back to back); `traffic` is the HBM bytes per launch
             from rocprofv3 FETCH_SIZE/WRITE_SIZE, calibrated on a plain copy,
             when profiles/ holds counters for the current kernel source
  read_probe the probe's read rate and the step's fraction of it
  check      the timed launches against the oracle: unflagged mismatches
             (must be 0), near-boundary flags, the largest relative error of
             the reported probabilities
  cpu_baseline  the CPU oracle's rate on that sample across the host's cores
             (process pool), with a one-core figure and the CPU model
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_isd_step_serving.json")
KERNEL_SOURCES = [os.path.join(ROOT, "speculative_verification_amd", "csrc", f)
                  for f in ("isd_step.hip", "isd_device.h", "isd_internal.h", "isd_api.hip")]
HEAD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_lm_head.json")
HEAD_SOURCES = [os.path.join(ROOT, "speculative_verification_amd", "csrc", f)
                for f in ("isd_lm_head.hip", "isd_internal.h", "isd_api.hip")]


def kernel_digest(sources=None) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES if sources is None else sources):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: the workload's own count: 100 tiny, 1000 serving "
                         "and greedy, 500 high concurrency, 200 otherwise)")
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps before the timed ones (the read probe before them has "
                         "already brought the GPU clock to its steady state)")
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5, 6],
                    help="1 tiny step (latency), 2 serving step, 3 greedy step, 4 LM head + step, "
                         "5 high concurrency, 6 segment-gated LoRA projection")
    ap.add_argument("--sets", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--segments", type=int, default=0)
    ap.add_argument("--resid-segments", type=int, default=0)
    ap.add_argument("--propose-segments", type=int, default=0)
    ap.add_argument("--sampler", choices=["cdf", "gumbel"], default="cdf",
                    help="correction draw: inverse CDF or Gumbel-max on Philox4x32-10")
    ap.add_argument("--top-k", type=int, default=0,
                    help="truncate P, Q and the proposal law to the top k entries (0: off)")
    ap.add_argument("--top-p", type=float, default=1.0, help="nucleus mass with --top-k (1: off)")
    ap.add_argument("--fused", action="store_true",
                    help="config 4: the LM head writes softmax statistics and the step reads them")
    ap.add_argument("--trunc-segments", type=int, default=0,
                    help="workgroups per row on the truncated path (0: automatic)")
    ap.add_argument("--probe", action="store_true",
                    help="only run the streaming-read probe (1 GiB, the step's tile loader)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = {1: 100, 2: 1000, 3: 1000, 5: 500}.get(args.config, 200)
    return args


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, five times: under rocprofv3
    counters its FETCH_SIZE and WRITE_SIZE per dispatch calibrate the counters
    against a known byte count."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_calibration_bytes=n, dispatches=5)), flush=True)


# ---------------------------------------------------------------------------
# Streaming-read probe (the device's practical read ceiling for the step's loop)
# ---------------------------------------------------------------------------

PROBE_BYTES = 1 << 30
PROBE_SETTLE_S = 0.4


def read_probe():
    """Streams a 1 GiB buffer with the step kernel's tile loader until about
    PROBE_SETTLE_S of device time has passed (which also brings the GPU clock
    to its steady state before any step is timed), then times 20 reads with
    two events.  Returns the read rate in GB/s."""
    import torch

    import speculative_verification_amd as isd
    buf = torch.empty(PROBE_BYTES, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < PROBE_SETTLE_S:
        for _ in range(50):
            isd.read_probe(buf, sink)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 20
    e0.record()
    for _ in range(n):
        isd.read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    del buf
    return PROBE_BYTES / (ms * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# CPU oracle on the timed steps (forked workers share the host inputs)
# ---------------------------------------------------------------------------

_HOST = {}


def _oracle_job(job):
    """Oracle outputs of sequence c of timed step i (the bytes and uniforms
    that launch consumed)."""
    os.environ["OMP_NUM_THREADS"] = "1"
    from oracle import isd_oracle as O
    i, c = job
    h = _HOST
    d = h["sets"][h["set_of"][i]]
    u = h["uni"][h["step_of"][i]]                      # [3, C, L]
    dt, mode, T, a = h["dtype"], h["mode"], h["T"], h["args"]
    p = O.decode_logits(d["p"][c:c + 1], dt)
    qn = O.decode_logits(d["qn"][c:c + 1], dt)
    x = d["x"][c:c + 1]
    if mode == "greedy":
        v = O.verify_greedy(p, x)
        g = v["argmax"]
        v.update(p_x=(x == g).astype(np.float64), q_x=np.ones(x.shape),
                 flagged=np.zeros(1, bool), resid_flagged=np.zeros(1, bool))
        tok, prob, nflag = O.propose_greedy(qn), np.ones(x.shape), np.zeros(x.shape, bool)
    else:
        q = O.decode_logits(d["q"][c:c + 1], dt)
        v = O.verify_sample(p, q, x, u[0, c:c + 1], u[1, c:c + 1], T, sampler=a["sampler"],
                            seq_ids=np.array([c]), top_k=a["top_k"], top_p=a["top_p"])
        tok, prob, _, nflag = O.propose_sample(qn, u[2, c:c + 1], T, top_k=a["top_k"],
                                               top_p=a["top_p"])
    return i, c, dict(accept_len=int(v["accept_len"][0]), out_tokens=v["out_tokens"][0],
                      n_emitted=int(v["n_emitted"][0]), p_x=v["p_x"][0], q_x=v["q_x"][0],
                      alpha=float(v["alpha"][0]), flagged=bool(v["flagged"][0]),
                      resid_flagged=bool(v["resid_flagged"][0]), next_tokens=tok[0],
                      qnext_x=prob[0], next_flagged=nflag[0])


def _rel(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    den = np.where(np.abs(o) > 0, np.abs(o), 1.0)
    return float(np.max(np.where(np.abs(o) > 0, np.abs(g - o) / den, np.abs(g - o)), initial=0.0))


def check_and_time_oracle(gpu, n_timed, cfg, target_s):
    """Runs the CPU oracle over every sequence of the first timed steps (as
    many as fit about target_s of wall time on the host's cores), compares
    each with the GPU outputs of the same launch, and times it.  Returns
    (cpu_baseline, check)."""
    import multiprocessing as mp
    C, L = cfg["C"], cfg["L"]
    cores = len(os.sched_getaffinity(0))
    _oracle_job((0, 0))                               # first call: imports and page-in
    t0 = time.perf_counter()
    n1 = min(C, 4)
    for c in range(n1):
        _oracle_job((0, c))
    per_seq = (time.perf_counter() - t0) / n1         # one sequence, one core, warm
    n_steps = int(max(1, min(n_timed, target_s * cores / max(per_seq * C, 1e-9))))
    jobs = [(i, c) for i in range(n_steps) for c in range(C)]
    pool = mp.get_context("fork").Pool(cores)
    try:
        t0 = time.perf_counter()
        res = list(pool.imap_unordered(_oracle_job, jobs, chunksize=1))
        wall = time.perf_counter() - t0
    finally:
        pool.close()
        pool.join()
    ck = dict(steps=n_steps, sequences=len(jobs), positions=len(jobs) * L, mismatches=0,
              decision_flags=0, resid_flags=0, propose_flags=0, max_rel_err_prob=0.0)
    for i, c, o in res:
        g = {k: v[i] for k, v in gpu.items()}
        ck["max_rel_err_prob"] = max(ck["max_rel_err_prob"], _rel(g["p_x"][c], o["p_x"]),
                                     _rel(g["q_x"][c], o["q_x"]), _rel(g["alpha"][c], o["alpha"]))
        ok_next = ~o["next_flagged"]
        ck["propose_flags"] += int((~ok_next).sum())
        ck["mismatches"] += int((g["next_tokens"][c][ok_next] != o["next_tokens"][ok_next]).sum())
        if ok_next.any():
            ck["max_rel_err_prob"] = max(ck["max_rel_err_prob"],
                                         _rel(g["qnext_x"][c][ok_next], o["qnext_x"][ok_next]))
        if o["flagged"]:
            ck["decision_flags"] += 1
            continue
        j = o["accept_len"]
        bad = g["accept_len"][c] != j or g["n_emitted"][c] != o["n_emitted"]
        keep = np.ones(L, bool)
        if j < L and o["resid_flagged"]:
            ck["resid_flags"] += 1
            keep[j] = False
        bad = bad or not np.array_equal(g["out_tokens"][c][keep], o["out_tokens"][keep])
        ck["mismatches"] += int(bad)
    ck["max_rel_err_prob"] = float(f"{ck['max_rel_err_prob']:.3g}")
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    base = dict(value=round(len(jobs) * L / wall, 3), unit="positions/s", cores=cores,
                kind="oracle",
                sample=f"every sequence of the first {n_steps} timed steps ({len(jobs)} sequences, "
                       f"{len(jobs) * L} positions, the launches' own inputs), fp64 numpy oracle, "
                       f"one process per core, {wall:.1f} s wall",
                value_1core=round(L / per_seq, 3), cpu_model=model)
    return base, ck


# ---------------------------------------------------------------------------

def lm_head_workload(args):
    """LM-head + ISD chain: per step, logits [C*2L, V] = h @ W on the matrix
    cores, then one fused step that verifies the previous step's proposals
    (q = the previous step's mask rows) against this step's anchor rows and
    draws the next proposals from this step's mask rows."""
    import torch

    import speculative_verification_amd as isd
    from isd_inputs import CONFIGS, gen_head_weights, gen_hidden, gen_uniforms

    cfg = CONFIGS[4]
    C, L, V, H, T = cfg["C"], cfg["L"], cfg["V"], cfg["H"], cfg["T"]
    M = C * 2 * L
    dev = torch.device("cuda", 0)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    t_gen = time.perf_counter()
    W = bf16(gen_head_weights(4))
    # one-time pack of the head into its k-contiguous layout (untimed)
    Wt = isd.lm_head_pack(W)
    del W
    hs = [bf16(gen_hidden(4, s)) for s in range(2)]
    total = args.warmup + args.steps + 1
    uni = torch.from_numpy(gen_uniforms(4, total)).to(dev)
    logits = [torch.empty((M, V), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    nt = (V + isd.isd.STATS_TILE - 1) // isd.isd.STATS_TILE
    stats = [torch.empty((M, nt, 2), dtype=torch.float32, device=dev) for _ in range(2)]
    xs = [torch.zeros((C, L), dtype=torch.int32, device=dev) for _ in range(2)]
    # the GEMM's workspace: the tiles of its last partial round are halved along K
    gws = isd.gemm_workspace(M, H, V)
    torch.cuda.synchronize()
    print(f"# W [{H}, {V}] and hidden states ready, {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    def views(i):
        ext = logits[i % 2].view(C, 2 * L, V)
        return ext[:, :L], ext[:, L:]

    def sviews(i):
        st = stats[i % 2].view(C, 2 * L, nt, 2)
        return st[:, :L], st[:, L:]

    def head(h, i):
        if args.fused:
            isd.lm_head_stats(h, Wt, T, out=logits[i % 2], stats=stats[i % 2], workspace=gws)
        else:
            isd.lm_head_packed(h, Wt, out=logits[i % 2], workspace=gws)

    def verify_propose(i):
        p, qn = views(i)
        _, q = views(i - 1)
        u = uni[i + 1]
        if args.fused:
            ps, qns = sviews(i)
            _, qs = sviews(i - 1)
            return isd.step_fused(p, q, xs[(i - 1) % 2], u[0], u[1], qn, u[2], ps, qs, qns,
                                  temperature=T, ws=ws, out=dict(next_tokens=xs[i % 2]))
        return isd.step(p, q, xs[(i - 1) % 2], u[0], u[1], qn, u[2], temperature=T, ws=ws,
                        out=dict(next_tokens=xs[i % 2]))

    # step -1: proposal-only bootstrap gives the first q and x
    head(hs[0], 1)
    _, qn0 = views(1)
    isd.propose(qn0, uni[0, 2], temperature=T, out=dict(next_tokens=xs[1]))
    ws = isd.workspace(isd.make_shape(views(0)[0]))
    outs = [None, None]

    def step(i):
        head(hs[i % 2], i)
        outs[i % 2] = verify_propose(i)

    probe_gbs = read_probe()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    isd.check_device_error(ws)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * args.steps)]
    t0 = time.perf_counter()
    for n in range(args.steps):
        i = args.warmup + n
        ev[3 * n].record(stream)
        head(hs[i % 2], i)
        ev[3 * n + 1].record(stream)
        outs[i % 2] = verify_propose(i)
        ev[3 * n + 2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    isd.check_device_error(ws)
    gemm_ms = np.mean([ev[3 * n].elapsed_time(ev[3 * n + 1]) for n in range(args.steps)])
    step_ms = np.mean([ev[3 * n + 1].elapsed_time(ev[3 * n + 2]) for n in range(args.steps)])
    flops = 2.0 * M * H * V
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    step_bytes = 3 * C * L * V * 2   # what the step would read without the statistics
    ms_per_step = wall * 1e3 / args.steps
    acc = outs[(args.warmup + args.steps - 1) % 2]["accept_len"].float().mean().item()
    counters = head_counters(M, H, V)
    print(json.dumps(dict(
        metric="ISD verified positions/sec with the LM-head projection (h @ W on MFMA) in the step",
        value=round(C * L / (ms_per_step * 1e-3), 1), unit="positions/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=round(ms_per_step, 4),
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=f"LM head + ISD step: h [{M}, {H}] x W [{H}, {V}] bf16, then "
                             f"C={C}, L={L} verify/propose", C=C, L=L, V=V, H=H,
                    head_layout="W packed once (untimed) to k-contiguous [V, H]",
                    k_split_workspace_bytes=0 if gws is None else gws.numel(),
                    step_input="LM-head tile statistics" if args.fused else "logits"),
        roofline=dict(bound="mfma", achieved=round(gemm_tflops, 1), peak=2500.0,
                      unit="TFLOP/s", frac=round(gemm_tflops / 2500.0, 4),
                      traffic=(counters or {}).get("bytes_per_launch") if not args.fused else None),
        gemm=dict(ms=round(float(gemm_ms), 4), tflops=round(gemm_tflops, 1),
                  flop_frac=round(gemm_tflops / 2500.0, 4), peak_tflops=2500.0,
                  mfma_busy=((counters or {}).get("mfma") or {}).get("busy_frac")
                  if not args.fused else None),
        step=(dict(us=round(float(step_ms) * 1e3, 2),
                   note="reads the residual rows and one 128-column tile per proposal")
              if args.fused else
              dict(us=round(float(step_ms) * 1e3, 2),
                   hbm_gbs=round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
                   frac=round(step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))),
        read_probe=dict(gbs=round(probe_gbs, 1)),
        accept_len_mean_last=round(acc, 3))), flush=True)


def head_counters(M, H, V):
    """rocprofv3 counters of the plain packed LM head, when profiles/ holds
    them for the current GEMM source and this shape, else None:
    bytes_per_launch (FETCH_SIZE / WRITE_SIZE, copy-calibrated) and mfma
    (SQ_VALU_MFMA_BUSY_CYCLES over the SIMD cycles GRBM_GUI_ACTIVE spans)."""
    if not os.path.exists(HEAD_TRAFFIC_FILE):
        return None
    with open(HEAD_TRAFFIC_FILE) as f:
        tr = json.load(f)
    if tr.get("kernel_digest") != kernel_digest(HEAD_SOURCES) or tr.get("shape") != [M, H, V]:
        return None
    return tr


def lora_workload(args):
    """Segment-gated LoRA projection of the residual ISD variant: per step,
    h = x W^T + [mask] (x A^T) B^T for the MLP gate/up projection of an 8B
    model at the serving batch (M = 64 sequences x 16 extend rows, K = 4096,
    N = 24576, rank 128, adapter on the 8 mask rows of each sequence).  The
    base projection alone is timed beside it."""
    import torch

    import speculative_verification_amd as isd
    from isd_inputs import LORA_CONFIGS, gen_lora

    cfg = LORA_CONFIGS["mlp_up"]
    dev = torch.device("cuda", 0)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    d = gen_lora(cfg, 0)
    x, a, w, b = bf16(d["x"]), bf16(d["a"]), bf16(d["w"]), bf16(d["b"])
    mask = torch.from_numpy(d["mask"]).to(dev)
    wcat = isd.lora_pack(w, b)    # once per adapter (untimed)
    M, K = x.shape
    N, r = w.shape[0], a.shape[0]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    t = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
    # the GEMM's workspace: the tiles of its last partial round are halved along K
    ws = isd.gemm_workspace(M, K, N)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps, (time.perf_counter() - t0) * 1e3 / args.steps

    read_probe()
    base_ms, _ = timed(lambda: isd.lm_head_packed(x, w, out=out, workspace=ws))
    lora_ms, wall_ms = timed(lambda: isd.lora_gemm(x, a, wcat, mask, out=out, t=t, workspace=ws))
    gated = int((d["mask"] != 0).sum())
    flops = 2.0 * M * K * N + 2.0 * gated * r * (K + N)
    tflops = flops / (lora_ms * 1e-3) / 1e12
    print(json.dumps(dict(
        metric="segment-gated LoRA projection TFLOP/s (h = W x + [mask] B A x)",
        value=round(tflops, 1), unit="TFLOP/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(wall_ms, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload=f"gated LoRA projection: x [{M}, {K}], W [{N}, {K}], rank {r}, "
                             f"adapter on {gated} mask rows", M=M, K=K, N=N, r=r),
        roofline=dict(bound="mfma", achieved=round(tflops, 1), peak=2500.0, unit="TFLOP/s",
                      frac=round(tflops / 2500.0, 4), traffic=None),
        kernel_us_avg=round(lora_ms * 1e3, 2), base_projection_us=round(base_ms * 1e3, 2),
        adapter_overhead=round(lora_ms / base_ms - 1.0, 4),
        k_split_workspace_bytes=0 if ws is None else ws.numel())), flush=True)


def step_workload(args):
    """Configs 1, 2, 3 and 5: the fused step over resident inputs."""
    import torch

    import speculative_verification_amd as isd
    from isd_inputs import CONFIGS, gen_step, gen_uniforms

    cfg = CONFIGS[args.config]
    C, L, V, mode, T = cfg["C"], cfg["L"], cfg["V"], cfg["mode"], cfg["T"]
    dt = cfg["dtype"]
    es = 2 if dt == "bf16" else 4
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    isd.set_tuning(args.segments, args.resid_segments, 0, args.propose_segments)
    isd.set_trunc_tuning(args.trunc_segments)

    total = args.warmup + args.steps
    # the tiny workload draws fresh inputs for every step; the large ones cycle
    # over a few resident sets, each larger than the 256 MB Infinity Cache
    tiny = args.config == 1
    nsets = total if tiny else max(1, args.sets)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t_gen = time.perf_counter()
    host_sets, dev_sets = [], []
    for s in range(nsets):
        d = gen_step(args.config, s, workers=1 if tiny else workers)
        host_sets.append(d)
        t = {}
        for key in ("p", "q", "qn"):
            a = np.ascontiguousarray(d[key])
            t[key] = (torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
                      if dt == "bf16" else torch.from_numpy(a).to(dev))
        t["x"] = torch.from_numpy(d["x"]).to(dev)
        dev_sets.append(t)
    uni_host = gen_uniforms(args.config, total)          # [steps, 3, C, L]
    uni = torch.from_numpy(uni_host).to(dev)

    def outputs():
        return dict(accept_len=torch.empty((C,), dtype=torch.int32, device=dev),
                    out_tokens=torch.empty((C, L), dtype=torch.int32, device=dev),
                    n_emitted=torch.empty((C,), dtype=torch.int32, device=dev),
                    p_x=torch.empty((C, L), dtype=torch.float32, device=dev),
                    q_x=torch.empty((C, L), dtype=torch.float32, device=dev),
                    alpha=torch.empty((C,), dtype=torch.float32, device=dev),
                    next_tokens=torch.empty((C, L), dtype=torch.int32, device=dev),
                    qnext_x=torch.empty((C, L), dtype=torch.float32, device=dev))

    timed_out = [outputs() for _ in range(args.steps)]   # every timed launch keeps its outputs
    torch.cuda.synchronize()
    print(f"# inputs ready: {nsets} sets x {3 * C * L * V * es / 1e6:.2f} MB, "
          f"{time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    probe_gbs = read_probe()

    d0 = dev_sets[0]
    call = isd.StepCall(d0["p"], d0["q"], d0["x"], uni[0, 0], uni[0, 1], d0["qn"], uni[0, 2],
                        mode=mode, temperature=T, sampler=args.sampler, top_k=args.top_k,
                        top_p=args.top_p)
    tails = []
    for o in timed_out:
        call.bind_out(o)
        tails.append(call._tail)

    # every step's input views, made before any timing: binding a step then
    # only swaps pointers
    step_inputs = [(dev_sets[i % nsets]["p"], dev_sets[i % nsets]["q"], dev_sets[i % nsets]["x"],
                    uni[i, 0], uni[i, 1], dev_sets[i % nsets]["qn"], uni[i, 2]) for i in range(total)]

    def bind(i):
        call.bind(*step_inputs[i])

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    call.bind_out(outputs())
    for i in range(args.warmup):
        bind(i)
        call(sh)
    torch.cuda.synchronize()
    isd.check_device_error(call.ws)

    # Events on the launch stream time the launches back to back.  The first
    # event follows the first launch: an event recorded before it would fire
    # at once and count the host's time to issue that launch as kernel time
    # (about 25 us, a microsecond per step over 20 steps).  So the kernel
    # average spans launches 2..K; the wall clock spans all K.
    ev_first = torch.cuda.Event(enable_timing=True)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_first.record(stream)
    for n in range(args.steps):
        bind(args.warmup + n)
        call._tail = tails[n]
        call(sh)
        if n == 0:
            ev0.record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    isd.check_device_error(call.ws)
    kernel_avg_ms = (ev0.elapsed_time(ev1) / (args.steps - 1) if args.steps > 1
                     else ev_first.elapsed_time(ev1))

    gpu = {k: np.stack([o[k].cpu().numpy() for o in timed_out]) for k in timed_out[0]}
    ms_per_step = wall * 1e3 / args.steps
    positions = C * L
    # rows the step reads once: anchor p, proposal q (sample mode only), mask qn
    bytes_alg = (2 if mode == "greedy" else 3) * C * L * V * es
    achieved = bytes_alg / (kernel_avg_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("kernel_digest") == kernel_digest() and tr.get("config") == args.config
                and tr.get("sampler", "cdf") == args.sampler and args.top_k == 0):
            traffic = tr.get("bytes_per_launch")

    hist = np.bincount(gpu["accept_len"].ravel().clip(0, L), minlength=L + 1)
    workload = (f"{cfg['name']} ISD step: C={C}, L={L}, V={V}, {dt} logits, "
                f"{'greedy' if mode == 'greedy' else f'T={T}'}")
    if tiny:
        us = ms_per_step * 1e3
        result = dict(metric="ISD step latency, tiny workload (C=1, L=4, V=1000, fp32 logits)",
                      value=round(us, 3), unit="us/step", higher_is_better=False)
    else:
        result = dict(metric="ISD verified positions/sec at C=64,L=8,V=151936 bf16; achieved HBM GB/s"
                      if args.config == 2 else f"ISD verified positions/sec ({cfg['name']} workload)",
                      value=round(positions / (ms_per_step * 1e-3), 1), unit="positions/s",
                      higher_is_better=True)
    result.update(
        n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=round(ms_per_step, 5),
        scaling="weak", vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload=workload, C=C, L=L, V=V, logits_dtype=dt, mode=mode,
                    sampler=args.sampler, top_k=args.top_k, top_p=args.top_p,
                    input_sets=nsets, parallelism="single GPU"),
        roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic),
        read_probe=dict(gbs=round(probe_gbs, 1), frac_of_peak=round(probe_gbs / HBM_PEAK_GBS, 4),
                        step_frac_of_probe=round(achieved / probe_gbs, 4)),
        hbm_gbs_wall=round(bytes_alg / (ms_per_step * 1e-3) / 1e9, 1),
        kernel_us_avg=round(kernel_avg_ms * 1e3, 2),
        bytes_per_step=bytes_alg,
        accept_len_mean=round(float(gpu["accept_len"].mean()), 4),
        accept_len_hist=hist.tolist(),
        alpha_mean=round(float(gpu["alpha"].mean()), 5),
    )
    if not args.no_cpu_baseline:
        print("# running the CPU oracle on the timed steps", file=sys.stderr, flush=True)
        _HOST.update(sets=host_sets, uni=uni_host, dtype=dt, mode=mode, T=T,
                     args=dict(sampler=args.sampler, top_k=args.top_k, top_p=args.top_p),
                     set_of=[(args.warmup + n) % nsets for n in range(args.steps)],
                     step_of=[args.warmup + n for n in range(args.steps)])
        result["cpu_baseline"], result["check"] = check_and_time_oracle(
            gpu, args.steps, cfg, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps(dict(error="this build runs on one GPU: the ISD step is measured "
                                    "on a single MI355X; multi-GPU runs are not supported",
                              n_gpus=args.gpus)))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.probe:
        gbs = read_probe()
        print(json.dumps(dict(metric="streaming read rate, step tile loader, 1 GiB",
                              value=round(gbs, 1), unit="GB/s",
                              frac_of_peak=round(gbs / HBM_PEAK_GBS, 4))), flush=True)
        return
    if args.config == 4:
        lm_head_workload(args)
        return
    if args.config == 6:
        lora_workload(args)
        return
    step_workload(args)


if __name__ == "__main__":
    main()
