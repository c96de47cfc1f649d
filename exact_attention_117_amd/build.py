"""Build libfa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m exact_attention_117_amd.build           # or build() from Python
    python -m exact_attention_117_amd.build --trace   # libfa_trace.so, below

build(trace=True) writes a separate timing library, libfa_trace.so: the same
sources with per-iteration clock stamps in the plain forward kernels
(FA_FWD_TRACE) and the gradient kernels (FA_BWD_TRACE), read back by
`bench.py --trace-phases`.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
LIB_TRACE = os.path.join(HERE, "libfa_trace.so")
ARCH = "gfx950"

# (object, source, extra flags). fa_fwd.hip is compiled twice, one group of
# forward kernels per object, each with the machine-scheduler strategy that
# timed best for it on MI355X:
#  * FA_FWD_PLAIN, the fixed-length bf16 / fp16 kernels without a window:
#    max-ilp, 1.3-1.4% faster than the default strategy (causal B4 N4096 H32
#    d128, non-causal N8192, d256);
#  * without it, the window, packed-sequence and FP8 kernels: the default
#    strategy (at d = 128, iterative-ilp made the fixed-length windows 4-5%
#    slower, max-ilp 0.5%; iterative-ilp cost the others 1% to 11%).
OBJECTS = [
    ("fa_api", "fa_api.cpp", []),
    ("fa_fwd", "fa_fwd.hip", []),
    ("fa_fwd_plain", "fa_fwd.hip", ["-DFA_FWD_PLAIN", "-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
    ("fa_bwd", "fa_bwd.hip", []),
    ("fa_decode", "fa_decode.hip", []),
]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
# -fno-honor-nans (device code only): no NaN enters the kernels' max
# reductions, so fmaxf needs no NaN-quieting of its operands; host code keeps
# IEEE semantics (the argument checks test for non-finite scales).
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_device", "-fno-honor-nans",
               "-Wall", "-Wno-unused-command-line-argument"]


def _filtered(r: subprocess.CompletedProcess) -> str:
    return "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)


def build(verbose: bool = False, resource_usage: bool = False, trace: bool = False) -> str:
    """Compile each source to an object (in parallel), then link libfa.so
    (with trace, libfa_trace.so)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    if resource_usage:
        flags = ["-Rpass-analysis=kernel-resource-usage"] + flags
    tmpdir = tempfile.mkdtemp(prefix="fa_build_")
    try:
        objs, procs = [], []
        for name, src, extra in OBJECTS:
            if trace and name == "fa_fwd_plain":
                extra = extra + ["-DFA_FWD_TRACE"]
            if trace and name == "fa_bwd":
                extra = extra + ["-DFA_BWD_TRACE"]
            obj = os.path.join(tmpdir, name + ".o")
            cmd = [hipcc] + flags + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            objs.append(obj)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                          text=True))
        outs = []
        for p in procs:
            so, se = p.communicate()
            r = subprocess.CompletedProcess(p.args, p.returncode, so, se)
            outs.append(_filtered(r))
            if r.returncode != 0:
                raise RuntimeError("hipcc failed:\n" + outs[-1])
        out = LIB_TRACE if trace else LIB
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [hipcc] + HIPCC_FLAGS + objs + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        outs.append(_filtered(r))
        if r.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + outs[-1])
        if verbose or resource_usage:
            print("\n".join(o for o in outs if o))
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    build(verbose=True, resource_usage="--usage" in sys.argv, trace="--trace" in sys.argv)
