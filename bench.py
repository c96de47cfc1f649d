"""Benchmark of the exact-attention forward on one MI355X.

One step = one fa_fwd launch (the whole forward path: tile schedule, Q/K/V
loads, QK^T and PV on MFMA, masking, online softmax, epilogue) over the
batch 4 / 32 heads / seqlen 4096 / head dim 128 causal bf16 workload, with
inputs resident in device memory. Throughput uses the FLOP convention
4*B*H*N^2*d, halved for causal.

Prints one JSON line. Also reports:
  roofline     - achieved TFLOP/s of the kernel against the bf16 dense MFMA
                 peak (kernel time from HIP events on the launch stream);
  cpu_baseline - the fp64 CPU oracle timed on a bounded sample of the same
                 workload (whole heads), in the same FLOP convention.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0


def fwd_flops(B, N, H, d, causal):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(w, x, target_s):
    """Time the fp64 oracle on whole heads of the workload (same inputs)."""
    import numpy as np
    import torch

    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    threads = max(1, min(threads, len(os.sched_getaffinity(0)), 16))
    qb, kb, vb = x["bf16"][:3]

    def head(b, h):
        return [oracle.bf16_bits_to_f64(z[b:b + 1, :, h:h + 1, :].contiguous()
                                        .view(torch.int16).numpy()) for z in (qb, kb, vb)]

    rng = np.random.default_rng(w.seed)
    order = [(int(b), int(h)) for b, h in zip(rng.integers(0, w.B, 4096),
                                              rng.integers(0, w.H, 4096))]
    done, elapsed, i = 0, 0.0, 0
    while i < len(order) and i < w.B * w.H:
        q1, k1, v1 = head(*order[i])
        t0 = time.perf_counter()
        oracle.attention_fwd(q1, k1, v1, w.scale, w.causal, threads=threads)
        elapsed += time.perf_counter() - t0
        done += 1
        i += 1
        if elapsed >= target_s:
            break
    flops = fwd_flops(1, w.N, 1, w.d, w.causal) * done
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d heads (b,h) of the %s workload, all rows, fp64, %.1f s" % (
                done, w.B * w.H, w.name, elapsed)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the timed region, launch one plain device copy of this many "
                         "MiB (a known-size kernel that calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the kernels shard over (batch, head) with no "
              "exchange, and no multi-GPU run is part of this build. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from exact_attention_117_amd import fa, inputs

    w = inputs.WORKLOADS[args.workload]
    if w.kind != "fwd":
        raise SystemExit("bench workload must be a fixed-length forward workload")
    x = inputs.make(w)
    q, k, v = (t.cuda() for t in x["bf16"][:3])
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)

    def step():
        fa.fa_fwd(q, k, v, scale=w.scale, causal=w.causal, o=o, lse=lse)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=q.device)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        log("copy probe: %d bytes read, %d bytes written" % (n, n))
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # per-launch durations (same stream) for median / min
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    med, mn = per[len(per) // 2], per[0]

    flops = fwd_flops(w.B, w.N, w.H, w.d, w.causal)
    tflops = flops / (ms * 1e-3) / 1e12
    algo_bytes = 4 * w.B * w.N * w.H * w.d * 2 + w.B * w.H * w.N * 4
    result = {
        "metric": "attention fwd TFLOP/s (bf16, causal, d=128) and % of MI355X MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d N=%d H=%d d=%d causal=%s bf16" % (
            w.name, w.B, w.N, w.H, w.d, w.causal), "B": w.B, "N": w.N, "H": w.H, "d": w.d,
            "causal": w.causal, "layout": "[B,N,H,d]", "parallelism": "single GPU"},
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "kernel": "fwd_kernel<128,causal>",
                     "algorithmic_bytes": algo_bytes,
                     "hbm_gbs_algorithmic": round(algo_bytes / (ms * 1e-3) / 1e9, 1)},
        "launch_ms": {"mean": round(ms, 5), "median": round(med, 5), "min": round(mn, 5)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
