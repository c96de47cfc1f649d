"""Benchmark of the exact-attention forward on one MI355X.

One step = one fa_fwd launch (the whole forward path: tile schedule, Q/K/V
loads, QK^T and PV on MFMA, masking, online softmax, epilogue) over the
batch 4 / 32 heads / seqlen 4096 / head dim 128 causal bf16 workload, with
inputs resident in device memory. Throughput uses the FLOP convention
4*B*H*N^2*d, halved for causal.

Other workloads of exact_attention_117_amd.inputs (--workload NAME) time the
same way: the page-1 and page-4 fixed-length shapes, the packed
variable-length batches (one fa_fwd_varlen launch), the backward (one
fa_bwd or fa_bwd_varlen call: three launches, with the forward's O and LSE as
inputs; FLOP convention 10*B*H*N^2*d, halved for causal) and the sliding
window (fa_fwd_window / fa_bwd_window; FLOPs 4*d (fwd) or 10*d (bwd) per
visible (query, key) pair, counted exactly). The decoding workload (one
fa_fwd_kvcache call over a paged cache) is HBM-bound and reports GB/s of its
algorithmic bytes (every cached key and value of every head read once, the
queries read and the outputs written) against the 8 TB/s HBM peak. Those
lines are reported beside the headline, not instead of it.

Prints one JSON line. Also reports:
  roofline     - achieved TFLOP/s of the kernel against the bf16 dense MFMA
                 peak (kernel time from HIP events on the launch stream);
  cpu_baseline - the fp64 CPU oracle timed on a bounded sample of the same
                 workload (whole heads), in the same FLOP convention.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Defaults: 300 warm-up steps, then 200 timed steps (the headline takes about
0.3 s in all).
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
PEAK_FP8_TFLOPS = 5033.2   # 256 CU x 2.4 GHz x 8192 dense fp8 FLOP/clk/CU
# The FP8 forward runs Q K^T (half of the convention FLOPs) on the FP8 matrix
# cores and P V on the bf16 ones, so its roofline is the time both halves take
# at their own peaks: 1 / (0.5 / fp8 peak + 0.5 / bf16 peak).
PEAK_FP8_MIXED_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch from the calibrated FETCH_SIZE/WRITE_SIZE passes
# summarised in a committed profile, per workload. Only reported while the
# kernel sources (and the build script, which holds the compiler flags) still
# hash to the value recorded there.
_COMMON = ["exact_attention_117_amd/csrc/fa_device.h",
           "exact_attention_117_amd/csrc/fa_launch.h",
           "exact_attention_117_amd/build.py"]
FWD_SOURCES = ["exact_attention_117_amd/csrc/fa_fwd.hip"] + _COMMON
DECODE_SOURCES = ["exact_attention_117_amd/csrc/fa_decode.hip"] + _COMMON
BWD_SOURCES = ["exact_attention_117_amd/csrc/fa_bwd.hip"] + _COMMON
TRAFFIC_PROFILES = {
    "headline": ("profiles/fwd_kernel_causal_b4_n4096_h32_d128.md", FWD_SOURCES),
    "decode_b16": ("profiles/decode_kernel_b16_paged64_h32_d128.md", DECODE_SOURCES),
    "d256_n8192": ("profiles/fwd_kernel_causal_b2_n8192_h16_d256.md", FWD_SOURCES),
    "bwd_n8192": ("profiles/bwd_kernels_causal_b2_n8192_h32_d128.md", BWD_SOURCES),
    "window_n16384": ("profiles/fwd_kernel_window4096_b2_n16384_h32_d128.md", FWD_SOURCES),
    "varlen64": ("profiles/fwd_kernel_varlen64_h32_d128.md", FWD_SOURCES),
    "headline_fp8": ("profiles/fwd_kernel_fp8_causal_b4_n4096_h32_d128.md", FWD_SOURCES),
    "p1_n4096": ("profiles/fwd_kernel_causal_b8_n4096_h16_d64.md", FWD_SOURCES),
    "p1_n1024": ("profiles/fwd_kernel_causal_b8_n1024_h16_d64.md", FWD_SOURCES),
    "window_bwd_n16384": ("profiles/bwd_kernels_window4096_b2_n16384_h32_d128.md", BWD_SOURCES),
}


def profiled_traffic(workload):
    """(bytes per launch, note) from the committed profile, or (None, why)."""
    import hashlib
    import re
    if workload not in TRAFFIC_PROFILES:
        return None, "not profiled"
    path, sources = TRAFFIC_PROFILES[workload]
    try:
        text = open(os.path.join(ROOT, path)).read()
    except OSError:
        return None, "no traffic profile"
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    m_sha = re.search(r"sha256: `([0-9a-f]{64})`", text)
    m_tr = re.search(r"^traffic_bytes_per_launch: (\d+)", text, re.M)
    if not m_sha or not m_tr:
        return None, "traffic profile unreadable"
    if m_sha.group(1) != h.hexdigest():
        return None, "kernel changed since the counters were taken"
    return int(m_tr.group(1)), "FETCH_SIZE + WRITE_SIZE, copy-calibrated (" + path + ")"


def fwd_flops(B, N, H, d, causal, window=None):
    if window is not None:
        return 4.0 * B * H * d * visible_pairs(N, causal, window)
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def visible_pairs(N, causal, window):
    """Number of (query, key) pairs with key i - left <= j <= i + right
    (j <= i if causal) in a sequence of N; -1 leaves a side unbounded."""
    import numpy as np
    wl, wr = window
    i = np.arange(N, dtype=np.int64)
    lo = np.zeros(N, np.int64) if wl < 0 else np.maximum(0, i - wl)
    hi = i + 1 if causal else (np.full(N, N, np.int64) if wr < 0 else np.minimum(N, i + wr + 1))
    return int((hi - lo).sum())


def algorithmic_bytes(w, lengths=None):
    """HBM bytes one step of workload w moves at least: every input read once
    and every output written once (lengths: the packed sequences' or cached
    keys' lengths of varlen and decode workloads)."""
    if w.kind == "decode":
        keys = sum(lengths)
        # every cached key and value row of every head once; q read, o and lse written
        return 2 * keys * w.H * w.d * 2 + 2 * w.B * w.nq * w.H * w.d * 2 + w.B * w.H * w.nq * 4
    rows = sum(lengths) if w.kind in ("varlen", "bwd_varlen") else w.B * w.N
    if w.kind in ("fwd", "varlen"):
        eb = 1 if w.dtype == "fp8" else 2  # bytes per q, k, v element (o is 16-bit)
        return rows * w.H * w.d * (3 * eb + 2) + rows * w.H * 4
    # backward: reads q, k, v, o, dO and LSE, writes dq, dk, dv and D
    return 8 * rows * w.H * w.d * 2 + 3 * rows * w.H * 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(w, x, target_s):
    """Time the fp64 oracle on whole heads of the workload (same inputs)."""
    import numpy as np

    import oracle
    # host cores this process may run on, and the OpenMP threads the oracle
    # uses: OMP_NUM_THREADS if set, else one per core, at most 16 (one GPU's
    # share of a shared host's cores)
    host_cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or host_cores
    threads = max(1, min(threads, host_cores, 16))
    qb, kb, vb = x["bf16"][:3]

    ds = x.get("descale", [1.0, 1.0, 1.0])  # FP8: codes times the per-tensor factors

    def head(b, h):  # exact fp64 copies of one head (bf16, fp16 and e4m3 widen exactly)
        return [z[b:b + 1, :, h:h + 1, :].double().numpy() * s for z, s in zip((qb, kb, vb), ds)]

    rng = np.random.default_rng(w.seed)
    order = [divmod(int(u), w.H) for u in rng.permutation(w.B * w.H)]  # distinct (b, h)
    done, elapsed, i = 0, 0.0, 0
    while i < len(order):
        q1, k1, v1 = head(*order[i])
        t0 = time.perf_counter()
        oracle.attention_fwd(q1, k1, v1, w.scale, w.causal, threads=threads,
                             window=w.window or (-1, -1))
        elapsed += time.perf_counter() - t0
        done += 1
        i += 1
        if elapsed >= target_s:
            break
    flops = fwd_flops(1, w.N, 1, w.d, w.causal, w.window) * done
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads,
            "threads": threads, "host_cores": host_cores, "kind": "oracle",
            "sample": "%d of %d heads (b,h) of the %s workload, all rows, fp64, %.1f s" % (
                done, w.B * w.H, w.name, elapsed)}


def make_step(w, x, fa, torch):
    """(step function, FLOPs per step, algorithmic HBM bytes per step, kernel)."""
    dev = torch.device("cuda")
    if w.kind == "fwd":
        q, k, v = (t.to(dev) for t in x["bf16"][:3])
        o = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "fp8" else q.dtype,
                        device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        if w.dtype == "fp8":
            def step():
                fa.fa_fwd_fp8(q, k, v, *x["descale"], scale=w.scale, causal=w.causal, o=o,
                              lse=lse, window=w.window)
        else:
            def step():
                fa.fa_fwd(q, k, v, scale=w.scale, causal=w.causal, o=o, lse=lse,
                          window=w.window)
        mask = "window" if w.window else "causal" if w.causal else "full"
        return (step, fwd_flops(w.B, w.N, w.H, w.d, w.causal, w.window), algorithmic_bytes(w),
                "fwd_kernel<%d,%s%s>" % (w.d, mask, ",fp8" if w.dtype == "fp8" else ""))
    if w.kind == "varlen":
        q, k, v = (t.to(dev) for t in x["bf16"][:3])
        cu = x["cu_seqlens"].to(dev)
        o = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "fp8" else q.dtype,
                        device=dev)
        lse = torch.empty((w.H, q.shape[0]), dtype=torch.float32, device=dev)

        if w.dtype == "fp8":
            def step():
                fa.fa_fwd_varlen_fp8(q, k, v, cu, x["max_seqlen"], *x["descale"], scale=w.scale,
                                     causal=w.causal, o=o, lse=lse)
        else:
            def step():
                fa.fa_fwd_varlen(q, k, v, cu, x["max_seqlen"], scale=w.scale, causal=w.causal,
                                 o=o, lse=lse)
        return (step, sum(fwd_flops(1, n, w.H, w.d, w.causal) for n in x["lengths"]),
                algorithmic_bytes(w, x["lengths"]),
                "fwd_kernel<%d,varlen%s>" % (w.d, ",fp8" if w.dtype == "fp8" else ""))
    if w.kind == "decode":
        q, kc, vc, bt, sl = (x[n].to(dev) for n in ("q", "k_cache", "v_cache", "block_table",
                                                     "cache_seqlens"))
        msk = max(x["lengths"])
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.nq), dtype=torch.float32, device=dev)
        ws = torch.empty(fa.fa_fwd_kvcache_workspace_size(w.B, w.nq, w.H, w.d, msk),
                         dtype=torch.uint8, device=dev)

        def step():
            fa.fa_fwd_kvcache(q, kc, vc, bt, sl, msk, scale=w.scale, causal=w.causal, o=o,
                              lse=lse, workspace=ws)
        flops = 4.0 * w.d * w.H * w.nq * sum(x["lengths"])
        return step, flops, algorithmic_bytes(w, x["lengths"]), "decode (split + merge)"
    # backward: the forward's O and LSE are inputs, computed once beforehand
    q, k, v, do = (t.to(dev) for t in x["bf16"][:4])
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    if w.kind == "bwd_varlen":
        cu = x["cu_seqlens"].to(dev)
        total = q.shape[0]
        o, lse = fa.fa_fwd_varlen(q, k, v, cu, x["max_seqlen"], scale=w.scale,
                                  causal=w.causal)
        ws = torch.empty(fa.fa_bwd_workspace_size(1, total, w.H, w.d), dtype=torch.uint8,
                         device=dev)

        def step():
            fa.fa_bwd_varlen(q, k, v, o, do, lse, cu, x["max_seqlen"], scale=w.scale,
                             causal=w.causal, dq=dq, dk=dk, dv=dv, workspace=ws)
        flops = 2.5 * sum(fwd_flops(1, n, w.H, w.d, w.causal) for n in x["lengths"])
    else:
        o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=w.causal, window=w.window)
        ws = torch.empty(fa.fa_bwd_workspace_size(w.B, w.N, w.H, w.d), dtype=torch.uint8,
                         device=dev)

        def step():
            fa.fa_bwd(q, k, v, o, do, lse, scale=w.scale, causal=w.causal, dq=dq, dk=dk, dv=dv,
                      workspace=ws, window=w.window)
        flops = 2.5 * fwd_flops(w.B, w.N, w.H, w.d, w.causal, w.window)
    # five N x N x d products (10*B*H*N^2*d), halved for causal
    return step, flops, algorithmic_bytes(w, x.get("lengths")), "bwd (pre + dkdv + dq)"


def phase_summary(a):
    """Per-iteration timing from clock stamps a[group, wavefront, iteration,
    6] (loop top, after the copy wait, after the barrier, after starting the
    copies, after phase 1, after phase 2; zeros where nothing was recorded),
    in shader-clock cycles: the median iteration period (barrier release to
    release), the median delay from the last wavefront's arrival at a
    barrier to its release, and per wavefront the means of its copy wait,
    barrier wait, copy issue, phase 1 and phase 2 (the phases over the
    iterations it ran)."""
    import numpy as np
    used = [wv for wv in range(a.shape[1]) if (a[:, wv, :, 0] > 0).any()]
    a = a[:, used]
    t0, ta, tb, tc, t2, t3 = (a[..., i] for i in range(6))
    valid = (t0 > 0).all(axis=1)
    ran = (t3 > 0) & valid[:, None, :]
    period = tb[:, 0, 1:] - tb[:, 0, :-1]
    pv = valid[:, 1:] & valid[:, :-1]
    release = (tb.min(axis=1) - ta.max(axis=1))[valid]
    slots = []
    for i, wv in enumerate(used):
        r = ran[:, i]
        slots.append({"wavefront": wv,
                      "copy_wait": round(float((ta - t0)[:, i][valid].mean()), 1),
                      "barrier_wait": round(float((tb - ta)[:, i][valid].mean()), 1),
                      "copy_issue": round(float((tc - tb)[:, i][valid].mean()), 1),
                      "phase1": round(float((t2 - tc)[:, i][r].mean()), 1),
                      "phase2": round(float((t3 - t2)[:, i][r].mean()), 1)})
    return {"unit": "shader clock cycles per iteration",
            "iterations": int(valid.sum()),
            "period_median": float(np.median(period[pv])),
            "last_arrival_to_release_median": float(np.median(release)),
            "per_wavefront": slots}


def trace_phases(fa, step, torch, warmup, backward, d):
    """Where the kernels' iterations spend their time, from the timing
    library's clock stamps (build(trace=True)), over one call after the
    warm-up: the plain forward kernel (the first 320 iterations of every
    wavefront of its first 256 workgroups), or the dK/dV and dQ kernels of a
    backward call (their first 260 and 160). At d = 128 the timing build of
    the dQ kernel spills its copy offsets to scratch (the product kernel
    fills its 256 vector registers, and the record needs more), so its dQ
    figures describe that build, not the product kernel; the summary says
    so."""
    import ctypes
    import numpy as np
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()

    def read(fn, waves, iters, *pre):
        n = 256 * waves * iters * 6
        buf = (ctypes.c_ulonglong * n)()
        rc = fn(*pre, buf, n)
        if rc != 0:
            raise RuntimeError("trace read failed: %d" % rc)
        return np.frombuffer(buf, dtype=np.uint64).reshape(256, waves, iters, 6).astype(np.int64)

    if backward:
        dq = phase_summary(read(fa.lib.fa_bwd_trace_read, 8, 160, 1))
        if d == 128:
            dq["note"] = ("the timing build of this kernel spills at d = 128: these figures "
                          "describe that build, not the product kernel")
        return {"dkdv_kernel": phase_summary(read(fa.lib.fa_bwd_trace_read, 4, 260, 0)),
                "dq_kernel": dq}
    return {"fwd_kernel": phase_summary(read(fa.lib.fa_fwd_trace_read, 8, 320))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks take a few hundred ms of sustained load to settle (a
    # launch trace shows the headline going 607 -> 767 -> 583 us over the
    # first 40 launches); the default warm-up covers that ramp
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="headline",
                    help="a name from exact_attention_117_amd.inputs.WORKLOADS")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the timed region, launch one plain device copy of this many "
                         "MiB (a known-size kernel that calibrates HBM byte counters)")
    ap.add_argument("--trace-phases", action="store_true",
                    help="with the timing library (python -m exact_attention_117_amd.build "
                         "--trace), print where the plain forward kernel's or the gradient "
                         "kernels' iterations spend their cycles instead of the benchmark line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only (--gpus 1): the kernels shard over (batch, head) "
              "with no exchange between GPUs, so N GPUs would run N independent copies of "
              "the one-GPU workload.", file=sys.stderr)
        sys.exit(2)

    if args.trace_phases:
        from exact_attention_117_amd import build as fa_build
        if not os.path.exists(fa_build.LIB_TRACE):
            print("the timing library is not built: python -m exact_attention_117_amd.build "
                  "--trace", file=sys.stderr)
            sys.exit(2)
        os.environ["FA_LIBRARY"] = fa_build.LIB_TRACE

    import torch
    from exact_attention_117_amd import fa, inputs

    w = inputs.WORKLOADS[args.workload]
    x = inputs.make(w)
    step, flops, algo_bytes, kernel = make_step(w, x, fa, torch)

    if args.trace_phases:
        if not ((w.kind == "fwd" and not w.window and w.dtype in ("bf16", "fp16"))
                or w.kind == "bwd"):
            print("--trace-phases times the fixed-length bf16/fp16 forward without a window, "
                  "or a fixed-length backward", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"workload": w.name,
                          "trace": trace_phases(fa, step, torch, args.warmup,
                                                backward=w.kind == "bwd", d=w.d)}))
        return

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        log("copy probe: %d bytes read, %d bytes written" % (n, n))
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the launches go to torch's current stream; the events are recorded on it
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

    tflops = flops / (ms * 1e-3) / 1e12
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    traffic, traffic_note = profiled_traffic(w.name)
    what = {"fwd": "attention fwd", "varlen": "attention varlen fwd", "bwd": "attention bwd",
            "bwd_varlen": "attention varlen bwd", "decode": "attention decode"}
    mask = "causal" if w.causal else "full"
    if w.window:
        mask += " window (%d, %d)" % tuple(w.window)
    metric = ("attention fwd TFLOP/s (bf16, causal, d=128) and % of MI355X MFMA peak"
              if w.name == "headline" else
              "%s TFLOP/s (%s, %s, d=%d)" % (what[w.kind], w.dtype, mask, w.d))
    config = {"workload": "%s: B=%d N=%d H=%d d=%d %s %s" % (
        w.name, w.B, w.N, w.H, w.d, mask, w.dtype), "B": w.B, "N": w.N, "H": w.H, "d": w.d,
        "causal": w.causal, "layout": "[B,N,H,d]", "parallelism": "single GPU"}
    if w.window:
        config["window"] = list(w.window)
    if w.kind in ("varlen", "bwd_varlen"):
        config.update(workload="%s: %d packed sequences, total %d, max %d, H=%d d=%d causal=%s "
                      "%s" % (w.name, len(x["lengths"]), sum(x["lengths"]), x["max_seqlen"],
                              w.H, w.d, w.causal, w.dtype), layout="[total,H,d]")
    if w.kind == "decode":
        metric = "attention decode HBM GB/s (bf16 paged KV cache, %d new query, d=%d)" % (
            w.nq, w.d)
        config.update(workload="%s: %d sequences of %d..%d cached keys (total %d), %d-key pages, "
                      "Nq=%d, H=%d d=%d causal bf16" % (
                          w.name, w.B, min(x["lengths"]), max(x["lengths"]), sum(x["lengths"]),
                          x["page"], w.nq, w.H, w.d), layout="cache [num_pages,page,H,d]",
                      N=max(x["lengths"]))
    if w.kind == "decode":
        value, unit = gbs, "GB/s"
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "tflops": round(tflops, 3)}
    else:
        value, unit = tflops, "TFLOP/s"
        peak = PEAK_FP8_MIXED_TFLOPS if w.dtype == "fp8" else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                "hbm_gbs_algorithmic": round(gbs, 1)}
        if w.dtype == "fp8":
            roof["peak_note"] = ("Q K^T on the FP8 matrix cores (5033.2), P V on the bf16 "
                                 "ones (2516.6): the time of both halves at their peaks")
            roof["frac_of_fp8_peak"] = round(tflops / PEAK_FP8_TFLOPS, 4)
    roof.update(traffic=traffic, traffic_note=traffic_note, kernel=kernel,
                algorithmic_bytes=algo_bytes)
    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": config,
        "pct_of_peak": round(100 * roof["frac"], 2),
        "roofline": roof,
        "launch_ms": {"mean": round(ms, 5), "median": round(med, 5), "min": round(mn, 5)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = (cpu_baseline(w, x, args.cpu_seconds) if w.kind == "fwd"
                                  else None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
