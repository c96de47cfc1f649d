"""Host sanitizers on the oracle: attn_oracle.c built with AddressSanitizer
and UndefinedBehaviorSanitizer (gcc, CPU only), then a subset of the pins run
against that build in a child process (the sanitizer runtime has to be the
first library the process loads). An out-of-bounds read or write, a use of
freed memory or undefined arithmetic in the oracle stops the child with a
report and fails the test; the pins must still pass under the sanitizers."""
import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "attn_oracle.c")

CHILD = """
import json, sys
import numpy as np
sys.path[:0] = [%r, %r]
import oracle
import test_oracle_mutants as m
with oracle.using(%r):
    failed = m.pins_fail()
    # the row-selection, column and varlen entry points as well
    r = np.random.default_rng(5)
    q, k, v, do = (r.standard_normal((2, 11, 3, 8)) for _ in range(4))
    for causal in (False, True):
        for win in ((-1, -1), (3, 2), (0, 0)):
            o, lse = oracle.attention_fwd(q, k, v, 0.3, causal, window=win)
            sel = np.array([[0, 0, 0], [1, 2, 10], [0, 1, 5]], np.int64)
            o_r, l_r = oracle.attention_fwd(q, k, v, 0.3, causal, rows=sel, window=win)
            if not np.allclose(o_r, o[sel[:, 0], sel[:, 2], sel[:, 1]], atol=1e-14, rtol=0):
                failed.append("rows")
            g = oracle.attention_bwd(q, k, v, do, 0.3, causal, window=win)
    cu = np.array([0, 4, 4, 11], np.int32)
    qp, kp, vp, dp = (t[0] for t in (q, k, v, do))
    oracle.attention_fwd_varlen(qp, kp, vp, cu, 0.3, True)
    oracle.attention_bwd_varlen(qp, kp, vp, dp, cu, 0.3, True)
print(json.dumps(sorted(set(failed))))
"""


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_pass_under_asan_and_ubsan(oracle_mod, tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Werror", SRC,
                           "-o", lib, "-lm"])
    env = dict(os.environ, LD_PRELOAD=asan, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD % (HERE, os.path.dirname(HERE), lib)],
                       capture_output=True, text=True, timeout=600, env=env)
    report = r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    assert json.loads(r.stdout.strip().splitlines()[-1]) == []
