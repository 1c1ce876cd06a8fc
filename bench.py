"""Throughput of the In-Place TTT layer forward on one MI355X.

One step = the whole layer on one batch of synthetic input already resident
in HBM: ipttt_segments_device (the batch's segment descriptors, once) ->
ipttt_z -> ipttt_target -> ipttt_chunk_delta -> ipttt_scan_apply, all
enqueued on torch's current stream.  Default workload: the 4B-class layer at
32k context (d_model 2560, d_ff 9728, 1 x 32768 tokens, chunk 512, bf16,
eta 1e-3, clip 1e-5).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config 4b_32k]
                  [--no-cpu-baseline] [--cpu-seconds 15]

With --backward a step is a training step: the forward keeping what the
backward reuses (ipttt_z_save: the products before the gate;
ipttt_scan_apply_save: the chunk weights), then
ipttt_scan_apply_backward_saved -> ipttt_target_backward -> ipttt_z_backward_saved.

Timing: HIP events on the stream the kernels run on.  The K timed steps
carry one event at each step boundary and nothing else (`ms_per_step` is their
mean, `ms_per_step_median` the median).  K more steps then give the breakdown:
an event in front of every call and, through the library's launch hook
(ipttt_set_launch_hook), in front of every kernel, so each kernel is timed on
its own (mean and median over those steps); `roofline` is the dominant
kernel's, `kernels` every kernel's.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 bf16 FLOP/clk x 2.4 GHz (AMD's published 2.5 PFLOP/s dense)
PEAK_FP32_TFLOPS = 157.3    # fp32 matrix peak, for fp32 workloads
PEAK_HBM_GBS = 8000.0
METRIC = "TTT-MLP layer tokens/s at 4B shape, 32k ctx, C=512; % of bf16 MFMA peak"

# Sources of each profiled kernel: a committed traffic summary counts only
# while these files are unchanged.
KERNEL_SOURCES = {
    "gated_z_fast_kernel": ["gated_z.hip", "common.h", "epilogue.h", "launch.h", "mfma_core.h", "pingpong.h"],
    "scan_fast_kernel": ["delta.hip", "common.h", "epilogue.h", "launch.h", "mfma_core.h"],
    "apply_fast_kernel": ["apply.hip", "common.h", "epilogue.h", "launch.h", "mfma_core.h"],
}


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "test_weight_mlp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_of(kernel: str) -> dict:
    """The committed rocprofv3 counter summary of a kernel, or {} when its
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as fh:
        t = json.load(fh)
    return t if t.get("source_sha") == source_sha(kernel) else {}


def traffic_from_profile(kernel: str):
    """HBM bytes per launch from the committed counter summary (None when stale)."""
    return profile_of(kernel).get("bytes_per_launch")


def algorithmic_flops(cfg, target: str = "lm", carry: bool = False, backward: bool = False) -> float:
    """FLOPs of one step as the metric counts them: 8 T d f (Z: 4, the
    chunk deltas: 2, the apply: 2) + the target's own work (Conv1D 10 d and
    W_target 2 d^2 per token) + one d x f state add per chunk; without a
    carried-out state the last chunk's delta is never formed.  A training
    step counts three forwards (the backward's products are twice the
    forward's; recomputation inside it is not counted)."""
    tokens = cfg.rows * cfg.seq_len
    target_flops = {"lm": 2.0 * tokens * cfg.d_model ** 2 + 10.0 * tokens * cfg.d_model,
                    "no_conv": 2.0 * tokens * cfg.d_model ** 2,
                    "no_proj": 10.0 * tokens * cfg.d_model}[target]
    f = 8.0 * tokens * cfg.d_model * cfg.d_ff + target_flops + cfg.rows * cfg.n_chunks * cfg.d_model * cfg.d_ff
    if not carry:
        last = cfg.seq_len - (cfg.n_chunks - 1) * cfg.chunk
        f -= 2.0 * cfg.rows * last * cfg.d_model * cfg.d_ff
    return 3.0 * f if backward else f


def cpu_baseline(cfg, x, budget_s: float) -> dict:
    """The fp64 oracle on the first chunks of the same inputs, on host cores."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas_threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity count
        blas_threads = len(os.sched_getaffinity(0))
    C = cfg.chunk
    w = {k: x[k].double().cpu().numpy() for k in ("W_gate", "W_up", "W_down", "W_target", "conv_w")}

    def run(nch):
        n = nch * C
        H = x["H"][:n].double().cpu().numpy()
        X0 = x["X0"][:n].double().cpu().numpy()
        t0 = time.perf_counter()
        oracle.forward(H, X0, w["W_gate"], w["W_up"], w["W_down"], w["conv_w"], w["W_target"],
                       rows=1, T=n, C=C, eta=cfg.eta, tau=cfg.tau)
        return time.perf_counter() - t0

    t1 = run(1)
    nch = int(max(1, min(cfg.n_chunks, budget_s // max(t1, 1e-3))))
    t = run(nch) if nch > 1 else t1
    return {"value": nch * C / t, "unit": "tokens/s", "cores": int(blas_threads),
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"first {nch} chunks ({nch * C} tokens) of row 0 of the same inputs, "
                      f"fp64 numpy, sequential apply-then-update loop; {t:.1f} s"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="4b_32k")
    ap.add_argument("--target", default="lm", choices=["lm", "no_conv", "no_proj"],
                    help="the target V_hat: the method's (lm) or one of its ablations")
    ap.add_argument("--chunk", type=int, default=0, help="override the configuration's chunk size")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--backward", action="store_true",
                    help="time a training step: the forward, then the three backward calls "
                         "(gradients of every input for a random output cotangent)")
    ap.add_argument("--carry", action="store_true",
                    help="streamed reading: every row continues the document of the previous "
                         "step, whose fp32 state ipttt_scan_apply_carry takes in and hands out")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device-to-device tensor copy (the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the layer forward is built and timed on a single "
              "MI355X; runs on more than one GPU are not supported.", file=sys.stderr)
        return 2

    import torch
    import test_weight_mlp_amd as ip
    from test_weight_mlp_amd import inputs

    cfg = inputs.CONFIGS[args.config]
    if args.chunk:
        cfg = cfg.with_(chunk=args.chunk)
    x = inputs.make_inputs(cfg, args.seed, "cuda")
    dt = ip.IPTTT_F32 if cfg.dtype == "f32" else ip.IPTTT_BF16
    target = {"lm": ip.IPTTT_TARGET_LM, "no_conv": ip.IPTTT_TARGET_NO_CONV,
              "no_proj": ip.IPTTT_TARGET_NO_PROJ}[args.target]
    p = ip.Problem(cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.chunk, dt, x["doc_starts"], target=target,
                   continues=[1] * cfg.rows if args.carry else None)
    # a training step keeps the forward's chunk weights for the backward
    buf = ip.allocate(p, "cuda", save=args.backward)
    stream = torch.cuda.current_stream()
    # the batch's segment descriptors, built once per step by the step's first
    # call and read by every later one
    seg_table = torch.empty(p.rows * p.n_chunks * 3, dtype=torch.int32, device="cuda")
    seg_bytes = torch.empty(p.tokens, dtype=torch.uint8, device="cuda")
    p.use_segments(seg_table, seg_bytes)
    calls = ["ipttt_segments_device", "ipttt_z_save" if args.backward else "ipttt_z", "ipttt_target",
             "ipttt_chunk_delta",
             "ipttt_scan_apply_carry" if args.carry else
             "ipttt_scan_apply_save" if args.backward else "ipttt_scan_apply"]
    if args.backward:
        if args.carry:
            print("--backward differentiates the plain forward; drop --carry", file=sys.stderr)
            return 2
        calls += ["ipttt_scan_apply_backward_saved", "ipttt_target_backward", "ipttt_z_backward_saved"]
        grads = ip.Grads(p, "cuda")
        dO = inputs.make_cotangents(cfg, args.seed, "cuda")["dO"]
    # the carried state, updated in place by every step
    S = torch.zeros((cfg.rows, cfg.d_model, cfg.d_ff), dtype=torch.float32, device="cuda") if args.carry else None

    # Events of the step being timed, in stream order: ("call", name, ev) in
    # front of every call (and ("end", None, ev) after the last), ("kernel",
    # name, ev) from the library's launch hook in front of every kernel.
    seq = None

    def on_launch(name, stream_ptr):
        if seq is not None:
            if stream_ptr != stream.cuda_stream:
                raise RuntimeError(f"{name} launched on another stream")
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            seq.append(("kernel", name, ev))

    def mark(kind, name=None):
        if seq is not None:
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            seq.append((kind, name, ev))

    def step():
        mark("call", calls[0])
        ip.ipttt_segments_device(p, seg_table, seg_bytes)
        mark("call", calls[1])
        if args.backward:
            ip.ipttt_z_save(p, x["H"], x["W_gate"], x["W_up"], buf.Z, buf.GU)
        else:
            ip.ipttt_z(p, x["H"], x["W_gate"], x["W_up"], buf.Z)
        mark("call", calls[2])
        ip.ipttt_target(p, x["X0"], None if target == ip.IPTTT_TARGET_NO_CONV else x["conv_w"],
                        None if target == ip.IPTTT_TARGET_NO_PROJ else x["W_target"], buf.V, buf.ws)
        mark("call", calls[3])
        ip.ipttt_chunk_delta(p, buf.V, buf.Z, cfg.eta, cfg.tau, buf.alpha, None, buf.ws)
        mark("call", calls[4])
        if args.carry:
            ip.ipttt_scan_apply_carry(p, buf.Z, buf.V, x["W_down"], buf.alpha, cfg.eta, S, S, buf.O, buf.ws)
        elif args.backward:
            ip.ipttt_scan_apply_save(p, buf.Z, buf.V, x["W_down"], buf.alpha, cfg.eta, buf.O, buf.saved, buf.ws)
        else:
            ip.ipttt_scan_apply(p, buf.Z, buf.V, x["W_down"], buf.alpha, cfg.eta, buf.O, buf.ws)
        if args.backward:
            g = grads
            conv = None if target == ip.IPTTT_TARGET_NO_CONV else x["conv_w"]
            wt = None if target == ip.IPTTT_TARGET_NO_PROJ else x["W_target"]
            mark("call", calls[5])
            ip.ipttt_scan_apply_backward_saved(p, buf.Z, buf.V, x["W_down"], cfg.eta, cfg.tau, buf.alpha,
                                               buf.saved, dO, g.dZ, g.dV, g.dW_down, g.ws)
            mark("call", calls[6])
            ip.ipttt_target_backward(p, x["X0"], conv, wt, g.dV, g.dX0, g.dconv_w, g.dW_target, g.ws)
            mark("call", calls[7])
            ip.ipttt_z_backward_saved(p, x["H"], x["W_gate"], x["W_up"], buf.GU, g.dZ, g.dH, g.dW_gate, g.dW_up,
                                      g.ws)
        mark("end")

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed region: K steps with nothing but one event at each step
    # boundary on the stream (no per-call or per-kernel events).
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    bounds[0].record(stream)
    for s in range(args.steps):
        step()
        bounds[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = bounds[0].elapsed_time(bounds[-1]) / args.steps
    step_t = [bounds[s].elapsed_time(bounds[s + 1]) for s in range(args.steps)]
    # Then K more steps for the breakdown: an event in front of every call and,
    # through the library's launch hook, in front of every kernel.
    ip.ipttt_set_launch_hook(on_launch)
    steps_seq = []
    for s in range(args.steps):
        seq = []
        steps_seq.append(seq)
        step()
    seq = None
    torch.cuda.synchronize()
    ip.ipttt_set_launch_hook(None)
    # per step: each call's time (its mark to the next call's or the end), each
    # kernel's (its hook event to the next event of any kind)
    call_t = {c: [] for c in calls}
    kern_t, kern_n = {}, {}
    for sq in steps_seq:
        kt = {}
        for i, (kind, name, ev) in enumerate(sq[:-1]):
            dt_ms = ev.elapsed_time(sq[i + 1][2])
            if kind == "call":
                nxt = next(j for j in range(i + 1, len(sq)) if sq[j][0] in ("call", "end"))
                call_t[name].append(ev.elapsed_time(sq[nxt][2]))
            elif kind == "kernel":
                kt[name] = kt.get(name, 0.0) + dt_ms
                kern_n[name] = kern_n.get(name, 0) + 1
        for k, v in kt.items():
            kern_t.setdefault(k, []).append(v)
    per_call = {c: float(np.mean(v)) for c, v in call_t.items()}
    per_call_median = {c: float(np.median(v)) for c, v in call_t.items()}

    tokens = cfg.rows * cfg.seq_len
    f_alg = algorithmic_flops(cfg, args.target, args.carry, args.backward)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    tflops = f_alg / (ms * 1e-3) / 1e12
    # Algorithmic FLOPs per launch of the kernels that carry the method's
    # contractions; the scan forms the delta of every carried segment.
    M, d, f = tokens, cfg.d_model, cfg.d_ff
    tbl = ip.ipttt_segment_table(p)
    L = np.minimum(cfg.chunk, cfg.seq_len - np.arange(cfg.n_chunks) * cfg.chunk)
    carried = tbl[..., 2] != 0
    if args.carry:
        carried[:, -1] = True  # the last chunk's delta feeds the carried-out state
    carried_tokens = float(np.sum(np.where(carried, L[None, :] - tbl[..., 1], 0)))
    kflops = {"gated_z": 4.0 * M * d * f, "scan": 2.0 * d * f * carried_tokens, "apply": 2.0 * M * d * f,
              "target_gemm": 2.0 * M * d * d if target != ip.IPTTT_TARGET_NO_PROJ else None,
              "conv": 10.0 * M * d if target != ip.IPTTT_TARGET_NO_CONV else None}
    fast = cfg.dtype == "bf16" and cfg.d_model % 64 == 0 and cfg.d_ff % 64 == 0
    kernel_symbol = {"gated_z": "gated_z_fast_kernel" if fast else "gated_z_kernel",
                     "scan": "scan_fast_kernel" if fast else "scan_kernel",
                     "apply": "apply_fast_kernel" if fast else "apply_kernel",
                     "target_gemm": "target_fast_kernel" if fast else "target_kernel",
                     "gram": "gram_z_fast_kernel" if fast else "gram_kernel", "conv": "conv_kernel"}
    if fast:
        kernel_symbol["gram_v"] = "gram_v_fast_kernel"
    # The committed counter summaries were taken on the default workload only.
    profiled = (args.config == "4b_32k" and args.target == "lm" and not args.chunk and not args.carry and
                not args.backward)
    kernels = {}
    for name, v in kern_t.items():
        n_launch = kern_n[name] / args.steps
        e = {"launches_per_step": n_launch, "ms_per_step_mean": float(np.mean(v)),
             "ms_per_step_median": float(np.median(v))}
        fl = kflops.get(name)
        if fl and n_launch == 1:
            e.update(flop_per_launch=fl, avg_launch_ms=e["ms_per_step_mean"],
                     tflops=fl / (e["ms_per_step_mean"] * 1e-3) / 1e12)
            e["frac"] = e["tflops"] / peak
        if name in kernel_symbol:
            e["symbol"] = kernel_symbol[name]
            # HBM-side bytes per launch from the committed counter summary
            # (while the kernel's sources match it), against the 8 TB/s peak
            prof = profile_of(e["symbol"]) if (profiled and e["symbol"] in KERNEL_SOURCES and n_launch == 1) else {}
            if prof.get("bytes_per_launch"):
                e["traffic_bytes"] = prof["bytes_per_launch"]
                e["hbm_gbs"] = prof["bytes_per_launch"] / (e["ms_per_step_mean"] * 1e-3) / 1e9
                e["hbm_frac"] = e["hbm_gbs"] / PEAK_HBM_GBS
        kernels[name] = e
    # Dominant kernel: the gate/up dual GEMM, timed by its own hook event.
    # (The training step's Z kernel also writes G and U: other counters.)
    zk = kernel_symbol["gated_z"]
    z = kernels["gated_z"]
    prof = profile_of(zk) if profiled and zk in KERNEL_SOURCES else {}
    traffic = prof.get("bytes_per_launch")
    # The clock the kernel held in the counter run (GRBM_GUI_ACTIVE over its
    # time; the chip lowers it under sustained MFMA load) and the fraction of
    # the peak at that clock, from the same committed summary.
    clk = prof.get("clock_ghz")
    out = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": float(np.median(step_t)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name + ": " + cfg.description +
                   ("" if args.target == "lm" else f", target {args.target}") +
                   (f", chunk {cfg.chunk}" if args.chunk else "") +
                   (", streamed (fp32 state carried in and out)" if args.carry else "") +
                   (", forward + backward (training step)" if args.backward else ""), "rows": cfg.rows,
                   "seq_len": cfg.seq_len, "d_model": cfg.d_model, "d_ff": cfg.d_ff,
                   "chunk": cfg.chunk, "eta": cfg.eta, "tau": cfg.tau,
                   "doc_starts": int(len(x["doc_starts"])), "parallelism": "single GPU"},
        "tflops": tflops,
        "frac_of_peak": tflops / peak,
        "peak_tflops": peak,
        "peak_clock_mhz": 2400,
        "flop_per_step": f_alg,
        "per_call_ms": per_call,
        "per_call_ms_median": per_call_median,
        "kernels": kernels,
        "roofline": {"kernel": zk, "bound": "mfma", "achieved": z["tflops"], "peak": peak,
                     "unit": "TFLOP/s", "frac": z["tflops"] / peak, "traffic": traffic,
                     "flop_per_launch": z["flop_per_launch"], "avg_launch_ms": z["avg_launch_ms"],
                     "profiled_clock_ghz": clk, "profiled_mfma_busy": prof.get("mfma_busy"),
                     "frac_at_profiled_clock": (z["tflops"] / (256 * 4096 * clk * 1e9 / 1e12)) if clk else None},
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
