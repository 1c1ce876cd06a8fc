"""Throughput of the In-Place TTT layer forward on one MI355X.

One step = the whole layer on one batch of synthetic input already resident
in HBM: ipttt_z -> ipttt_target -> ipttt_chunk_delta -> ipttt_scan_apply, all
enqueued on torch's current stream.  Default workload: the 4B-class layer at
32k context (d_model 2560, d_ff 9728, 1 x 32768 tokens, chunk 512, bf16,
eta 1e-3, clip 1e-5).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config 4b_32k]
                  [--no-cpu-baseline] [--cpu-seconds 15]

With --backward a step is a training step: the forward keeping what the
backward reuses (ipttt_z_save: the products before the gate;
ipttt_scan_apply_save: the chunk weights), then
ipttt_scan_apply_backward_saved -> ipttt_target_backward -> ipttt_z_backward_saved.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

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
    "gated_z_fast_kernel": ["gated_z.hip", "common.h", "epilogue.h", "mfma_core.h"],
    "scan_fast_kernel": ["delta.hip", "common.h", "mfma_core.h"],
    "apply_fast_kernel": ["apply.hip", "common.h", "epilogue.h", "mfma_core.h"],
}


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "test_weight_mlp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def flops(cfg) -> dict:
    """Algorithmic FLOPs of one layer call, by call (no Gram-norm or re-applied work)."""
    B, T, d, f, N = cfg.rows, cfg.seq_len, cfg.d_model, cfg.d_ff, cfg.n_chunks
    return {
        "ipttt_z": 4.0 * B * T * d * f,
        "ipttt_target": 2.0 * B * T * d * d + 10.0 * B * T * d,  # the method's target
        "ipttt_chunk_delta": 0.0,
        "ipttt_scan_apply": 2.0 * B * T * d * f + 2.0 * B * T * d * f + 1.0 * B * N * d * f,
    }


def traffic_from_profile(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha") != source_sha(kernel):
        return None
    return t.get("bytes_per_launch")


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

    import numpy as np
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
    calls = ["ipttt_z_save" if args.backward else "ipttt_z", "ipttt_target", "ipttt_chunk_delta",
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

    def step(ev=None):
        def mark(k):
            if ev is not None:
                ev[k].record(stream)
        mark(0)
        if args.backward:
            ip.ipttt_z_save(p, x["H"], x["W_gate"], x["W_up"], buf.Z, buf.GU)
        else:
            ip.ipttt_z(p, x["H"], x["W_gate"], x["W_up"], buf.Z)
        mark(1)
        ip.ipttt_target(p, x["X0"], None if target == ip.IPTTT_TARGET_NO_CONV else x["conv_w"],
                        None if target == ip.IPTTT_TARGET_NO_PROJ else x["W_target"], buf.V, buf.ws)
        mark(2)
        ip.ipttt_chunk_delta(p, buf.V, buf.Z, cfg.eta, cfg.tau, buf.alpha, None, buf.ws)
        mark(3)
        if args.carry:
            ip.ipttt_scan_apply_carry(p, buf.Z, buf.V, x["W_down"], buf.alpha, cfg.eta, S, S, buf.O, buf.ws)
        elif args.backward:
            ip.ipttt_scan_apply_save(p, buf.Z, buf.V, x["W_down"], buf.alpha, cfg.eta, buf.O, buf.saved, buf.ws)
        else:
            ip.ipttt_scan_apply(p, buf.Z, buf.V, x["W_down"], buf.alpha, cfg.eta, buf.O, buf.ws)
        mark(4)
        if args.backward:
            g = grads
            conv = None if target == ip.IPTTT_TARGET_NO_CONV else x["conv_w"]
            wt = None if target == ip.IPTTT_TARGET_NO_PROJ else x["W_target"]
            ip.ipttt_scan_apply_backward_saved(p, buf.Z, buf.V, x["W_down"], cfg.eta, cfg.tau, buf.alpha,
                                               buf.saved, dO, g.dZ, g.dV, g.dW_down, g.ws)
            mark(5)
            ip.ipttt_target_backward(p, x["X0"], conv, wt, g.dV, g.dX0, g.dconv_w, g.dW_target, g.ws)
            mark(6)
            ip.ipttt_z_backward_saved(p, x["H"], x["W_gate"], x["W_up"], buf.GU, g.dZ, g.dH, g.dW_gate, g.dW_up,
                                      g.ws)
            mark(7)

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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / args.steps
    per_call = {c: float(np.mean([e[k].elapsed_time(e[k + 1]) for e in evs])) for k, c in enumerate(calls)}

    tokens = cfg.rows * cfg.seq_len
    F = flops(cfg)
    # algorithmic FLOPs: 8Tdf (Z, delta, apply) + the target's own work + the state adds
    target_flops = {"lm": 2.0 * tokens * cfg.d_model ** 2 + 10.0 * tokens * cfg.d_model,
                    "no_conv": 2.0 * tokens * cfg.d_model ** 2,
                    "no_proj": 10.0 * tokens * cfg.d_model}[args.target]
    f_alg = 8.0 * tokens * cfg.d_model * cfg.d_ff + target_flops + \
        cfg.rows * cfg.n_chunks * cfg.d_model * cfg.d_ff
    if not args.carry:
        # the last chunk's delta only feeds a carried-out state
        last = cfg.seq_len - (cfg.n_chunks - 1) * cfg.chunk
        f_alg -= 2.0 * cfg.rows * last * cfg.d_model * cfg.d_ff
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    if args.backward:
        # the usual convention for a training step: the backward's products
        # are twice the forward's (recomputation inside it is not counted)
        f_alg *= 3.0
    tflops = f_alg / (ms * 1e-3) / 1e12
    # Dominant kernel: the gate/up dual GEMM (ipttt_z launches exactly this one
    # kernel, so the events around the call time it on its own stream).
    zk = "gated_z_fast_kernel" if (cfg.dtype == "bf16" and cfg.d_model % 64 == 0) else "gated_z_kernel"
    z_ms = per_call[calls[0]]
    z_tf = F["ipttt_z"] / (z_ms * 1e-3) / 1e12
    # (the training step's Z kernel also writes G and U: its own counters)
    traffic = traffic_from_profile(zk) if zk in KERNEL_SOURCES and not args.backward else None
    out = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
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
        "flop_per_step": f_alg,
        "per_call_ms": per_call,
        "roofline": {"kernel": zk, "bound": "mfma", "achieved": z_tf, "peak": peak,
                     "unit": "TFLOP/s", "frac": z_tf / peak, "traffic": traffic,
                     "flop_per_launch": F["ipttt_z"], "avg_launch_ms": z_ms},
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
