"""Benchmark of the fused ISD verify-and-propose step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one isd_step launch over one batch: verification of C*L proposals
(anchor rows p and proposal rows q) plus the draw of the next C*L proposals
(mask rows qn).  The serving workload (C=64, L=8, V=151936, bf16 logits, T=1)
is the default.  Inputs are resident in HBM before timing; steps cycle over
`--sets` distinct logits sets (each larger than the 256 MB Infinity Cache)
with fresh uniforms every step.  Prints one JSON line.

Reported:
  value      verified positions per second = C*L / wall-clock time per step
  roofline   the step kernel against the HBM peak: algorithmic bytes per
             launch (every logit read once: 3*C*L*V*2 B) over the kernel's
             average duration (two events on its stream around the K
             back-to-back launches); `traffic` is the HBM bytes per launch
             from rocprofv3 FETCH_SIZE/WRITE_SIZE, calibrated on a plain copy,
             when profiles/ holds counters for the current kernel source
  cpu_baseline  the CPU oracle on a bounded sample of the same inputs,
             across the host's cores (process pool), in positions per second
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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000,
                    help="untimed steps first; about 0.2 s of the serving step, which brings the "
                         "GPU clock to its steady state (20 steps leave it ramping: +4-5%%)")
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5, 6],
                    help="2 serving step, 3 greedy step, 4 LM head + step, 5 high concurrency, "
                         "6 segment-gated LoRA projection")
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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


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
# CPU oracle baseline (forked workers share the host inputs copy-on-write)
# ---------------------------------------------------------------------------

_HOST = {}


def _oracle_seq(args):
    os.environ["OMP_NUM_THREADS"] = "1"
    from oracle import isd_oracle as O
    s, c, dtype, mode, T = args
    d = _HOST["sets"][s]
    p = O.decode_logits(d["p"][c:c + 1], dtype)
    qn = O.decode_logits(d["qn"][c:c + 1], dtype)
    if mode == "greedy":
        O.verify_greedy(p, d["x"][c:c + 1])
        O.propose_greedy(qn)
    else:
        q = O.decode_logits(d["q"][c:c + 1], dtype)
        O.verify_sample(p, q, d["x"][c:c + 1], d["ua"][c:c + 1], d["ur"][c:c + 1], T)
        O.propose_sample(qn, d["up"][c:c + 1], T)
    return 1


def cpu_baseline(host_sets, cfg, target_s):
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    _HOST["sets"] = host_sets
    C, L = cfg["C"], cfg["L"]
    jobs_all = [(s, c, cfg["dtype"], cfg["mode"], cfg["T"])
                for s in range(len(host_sets)) for c in range(C)]
    # calibrate on one sequence, then size the sample to about target_s of wall time
    t0 = time.perf_counter()
    _oracle_seq(jobs_all[0])
    per_seq = time.perf_counter() - t0
    n = int(max(cores, min(len(jobs_all) * 4, target_s * cores / max(per_seq, 1e-6))))
    jobs = [jobs_all[i % len(jobs_all)] for i in range(n)]
    pool = mp.get_context("fork").Pool(cores)
    try:
        t0 = time.perf_counter()
        done = sum(pool.imap_unordered(_oracle_seq, jobs, chunksize=1))
        wall = time.perf_counter() - t0
    finally:
        pool.close()
        pool.join()
    return dict(value=round(done * L / wall, 3), unit="positions/s", cores=cores, kind="oracle",
                sample=f"{done} sequences ({done * L} positions) of the timed workload's "
                       f"resident input sets, fp64 numpy oracle, one process per core, "
                       f"{wall:.1f} s wall")


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
            isd.lm_head_stats(h, Wt, T, out=logits[i % 2], stats=stats[i % 2])
        else:
            isd.lm_head_packed(h, Wt, out=logits[i % 2])

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
    print(json.dumps(dict(
        metric="ISD verified positions/sec with the LM-head projection (h @ W on MFMA) in the step",
        value=round(C * L / (ms_per_step * 1e-3), 1), unit="positions/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=round(ms_per_step, 4),
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=f"LM head + ISD step: h [{M}, {H}] x W [{H}, {V}] bf16, then "
                             f"C={C}, L={L} verify/propose", C=C, L=L, V=V, H=H,
                    head_layout="W packed once (untimed) to k-contiguous [V, H]",
                    step_input="LM-head tile statistics" if args.fused else "logits"),
        roofline=dict(bound="mfma", achieved=round(gemm_tflops, 1), peak=2500.0,
                      unit="TFLOP/s", frac=round(gemm_tflops / 2500.0, 4),
                      traffic=head_traffic(M, H, V) if not args.fused else None),
        gemm=dict(ms=round(float(gemm_ms), 4), tflops=round(gemm_tflops, 1),
                  mfma_util=round(gemm_tflops / 2500.0, 4), peak_tflops=2500.0),
        step=(dict(us=round(float(step_ms) * 1e3, 2),
                   note="reads the residual rows and one 128-column tile per proposal")
              if args.fused else
              dict(us=round(float(step_ms) * 1e3, 2),
                   hbm_gbs=round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
                   frac=round(step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))),
        accept_len_mean_last=round(acc, 3))), flush=True)


def head_traffic(M, H, V):
    """HBM bytes per launch of the plain packed LM head from rocprofv3
    FETCH_SIZE / WRITE_SIZE (copy-calibrated), when profiles/ holds counters
    for the current GEMM source and this shape; else None."""
    if not os.path.exists(HEAD_TRAFFIC_FILE):
        return None
    with open(HEAD_TRAFFIC_FILE) as f:
        tr = json.load(f)
    if tr.get("kernel_digest") != kernel_digest(HEAD_SOURCES) or tr.get("shape") != [M, H, V]:
        return None
    return tr.get("bytes_per_launch")


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

    base_ms, _ = timed(lambda: isd.lm_head_packed(x, w, out=out))
    lora_ms, wall_ms = timed(lambda: isd.lora_gemm(x, a, wcat, mask, out=out, t=t))
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
        adapter_overhead=round(lora_ms / base_ms - 1.0, 4))), flush=True)


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
    if args.config == 4:
        lm_head_workload(args)
        return
    if args.config == 6:
        lora_workload(args)
        return

    import torch

    import speculative_verification_amd as isd
    from isd_inputs import CONFIGS, gen_step, gen_uniforms

    cfg = CONFIGS[args.config]
    C, L, V, mode, T = cfg["C"], cfg["L"], cfg["V"], cfg["mode"], cfg["T"]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    isd.set_tuning(args.segments, args.resid_segments, 0, args.propose_segments)
    isd.set_trunc_tuning(args.trunc_segments)

    nsets = max(1, args.sets)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t_gen = time.perf_counter()
    host_sets, dev_sets = [], []
    for s in range(nsets):
        d = gen_step(args.config, s, workers=workers)
        host_sets.append(d)
        t = {}
        for key in ("p", "q", "qn"):
            t[key] = torch.from_numpy(d[key].view(np.int16)).to(dev).view(torch.bfloat16)
        t["x"] = torch.from_numpy(d["x"]).to(dev)
        dev_sets.append(t)
    total = args.warmup + args.steps
    uni = torch.from_numpy(gen_uniforms(args.config, total)).to(dev)   # [steps, 3, C, L]
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t_gen
    print(f"# inputs ready: {nsets} sets x {3 * C * L * V * 2 / 1e6:.1f} MB, {gen_s:.1f} s",
          file=sys.stderr, flush=True)

    d0 = dev_sets[0]
    call = isd.StepCall(d0["p"], d0["q"], d0["x"], uni[0, 0], uni[0, 1], d0["qn"], uni[0, 2],
                        mode=mode, temperature=T, sampler=args.sampler, top_k=args.top_k,
                        top_p=args.top_p)

    def bind(i):
        t = dev_sets[i % nsets]
        call.bind(t["p"], t["q"], t["x"], uni[i, 0], uni[i, 1], t["qn"], uni[i, 2])

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        bind(i)
        call()
    torch.cuda.synchronize()
    isd.check_device_error(call.ws)

    # two events on the launch stream bracket the K back-to-back launches
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        bind(args.warmup + i)
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    isd.check_device_error(call.ws)
    kernel_avg_ms = ev0.elapsed_time(ev1) / args.steps

    # untimed pass over the same steps for workload statistics
    n_stat = min(args.steps, 50)
    accept = torch.empty((n_stat, C), dtype=torch.int32, device=dev)
    alphas = torch.empty((n_stat, C), dtype=torch.float32, device=dev)
    for i in range(n_stat):
        bind(args.warmup + i)
        call()
        accept[i].copy_(call.out["accept_len"])
        alphas[i].copy_(call.out["alpha"])
    torch.cuda.synchronize()

    ms_per_step = wall * 1e3 / args.steps
    positions = C * L
    # rows the step reads once: anchor p, proposal q (sample mode only), mask qn
    bytes_alg = (2 if mode == "greedy" else 3) * C * L * V * 2
    achieved = bytes_alg / (kernel_avg_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("kernel_digest") == kernel_digest() and tr.get("config") == args.config
                and tr.get("sampler", "cdf") == args.sampler and args.top_k == 0):
            traffic = tr.get("bytes_per_launch")

    acc = accept.cpu().numpy()
    result = dict(
        metric="ISD verified positions/sec at C=64,L=8,V=151936 bf16; achieved HBM GB/s"
        if args.config == 2 else f"ISD verified positions/sec ({cfg['name']} workload)",
        value=round(positions / (ms_per_step * 1e-3), 1),
        unit="positions/s",
        n_gpus=1,
        steps=args.steps,
        warmup=args.warmup,
        ms_per_step=round(ms_per_step, 5),
        higher_is_better=True,
        scaling="weak",
        vs_baseline=None,
        dtype="f32",
        data="synthetic",
        config=dict(workload=f"{cfg['name']} ISD step: C={C}, L={L}, V={V}, bf16 logits, "
                             f"{'greedy' if mode == 'greedy' else f'T={T}'}",
                    C=C, L=L, V=V, logits_dtype="bf16", mode=mode, sampler=args.sampler,
                    top_k=args.top_k, top_p=args.top_p,
                    input_sets=nsets,
                    parallelism="single GPU"),
        roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic),
        hbm_gbs_wall=round(bytes_alg / (ms_per_step * 1e-3) / 1e9, 1),
        kernel_us_avg=round(kernel_avg_ms * 1e3, 2),
        bytes_per_step=bytes_alg,
        accept_len_mean=round(float(acc.mean()), 4),
        alpha_mean=round(float(alphas.mean().item()), 5),
    )
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(host_sets, cfg, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
