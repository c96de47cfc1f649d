"""Sensitivity of the oracle pins: plant one plausible mistake at a time in a
copy of attn_oracle.c (a dropped term, a wrong sign, an off-by-one mask, a
swapped operand), build it on the CPU, and check that the pins reject it.
The unmutated oracle must pass the same checks. Each mutant runs in a child
process: a mutant that reads out of bounds and crashes counts as caught."""
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle

from test_oracle_bwd_pins import torch_reference_grads
from test_oracle_kvcache_pins import library_kvcache, paged
from test_oracle_pins import _parse, scipy_attention

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "attn_oracle.c")

MUTANTS = {
    "causal_excludes_diagonal": ("int64_t l = 0, h = causal ? i + 1 : N;",
                                 "int64_t l = 0, h = causal ? (i > 0 ? i : 1) : N;"),
    "scale_dropped": ("s[j - lo] = scale * dot(qi, k + IDX(", "s[j - lo] = dot(qi, k + IDX("),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "ds_sign": ("ds = s[j - lo] * (dp[j - lo] - D);", "ds = s[j - lo] * (dp[j - lo] + D);"),
    "D_without_p": ("D += s[j - lo] * dp[j - lo];", "D += dp[j - lo];"),
    "dq_scale_dropped": ("dq[c] += scale * ds * kj[c];", "dq[c] += ds * kj[c];"),
    "dk_wrong_operand": ("dk[c] += scale * ds * qi[c];", "dk[c] += scale * ds * doi[c];"),
    "dv_wrong_operand": ("dv[c] += p * doi[c];", "dv[c] += p * qi[c];"),
    "causal_cols_off_by_one": ("int64_t l = causal ? j : 0, h = N;",
                               "int64_t l = causal ? j + 1 : 0, h = N;"),
    "window_left_off_by_one": ("if (wl >= 0 && i - wl > l) l = i - wl;",
                               "if (wl >= 0 && i - wl + 1 > l) l = i - wl + 1;"),
    "window_cols_drop_right_bound": ("if (wr >= 0 && j - wr > l) l = j - wr;", ""),
    "cache_query_position_off_by_one": ("const int64_t pos = L - Nq + i;",
                                        "const int64_t pos = L - Nq + i + 1;"),
    "cache_page_and_slot_swapped": ("return block_table[b * max_pages + j / page] * page + j % page;",
                                    "return block_table[b * max_pages + j % page] * page + j / page;"),
}


def pins_fail() -> list:
    """A compact run of the pins; returns the names of those that fail."""
    failed = []
    ex = json.load(open(os.path.join(HERE, "golden", "hand_examples.json")))["examples"]
    for causal in (False, True):
        for e in ex:
            q, k, v = (np.array(_parse(e[n]))[None] for n in ("q", "k", "v"))
            o, lse = oracle.attention_fwd(q, k, v, e["scale"], causal)
            want = e["expect"]["causal" if causal else "noncausal"]
            if not (np.allclose(o, np.array(_parse(want["o"]))[None], atol=1e-12, rtol=0)
                    and np.allclose(lse, np.array(_parse(want["lse"]))[None], atol=1e-12,
                                    rtol=0)):
                failed.append("golden")
        r = np.random.default_rng(0)
        q, k, v, do = (r.standard_normal((1, 9, 2, 4)) for _ in range(4))
        o, lse = oracle.attention_fwd(q, k, v, 0.5, causal)
        o2, l2 = scipy_attention(q, k, v, 0.5, causal)
        if not (np.allclose(o, o2, atol=1e-12, rtol=0) and np.allclose(lse, l2, atol=1e-12,
                                                                        rtol=0)):
            failed.append("scipy")
        g = oracle.attention_bwd(q, k, v, do, 0.5, causal)
        ref = torch_reference_grads(q, k, v, do, 0.5, causal)
        if not all(np.allclose(g[n], ref[n], atol=1e-11, rtol=0) for n in ("dq", "dk", "dv")):
            failed.append("autograd")
        win = (2, 1)
        o, lse = oracle.attention_fwd(q, k, v, 0.5, causal, window=win)
        o2, l2 = scipy_attention(q, k, v, 0.5, causal, window=win)
        if not (np.allclose(o, o2, atol=1e-12, rtol=0) and np.allclose(lse, l2, atol=1e-12,
                                                                        rtol=0)):
            failed.append("scipy window")
        g = oracle.attention_bwd(q, k, v, do, 0.5, causal, window=win)
        ref = torch_reference_grads(q, k, v, do, 0.5, causal, window=win)
        if not all(np.allclose(g[n], ref[n], atol=1e-11, rtol=0) for n in ("dq", "dk", "dv")):
            failed.append("autograd window")
        rng = np.random.default_rng(3)
        lens, page = [13, 4, 9], 4
        kc, vc, bt = paged(rng, lens, 2, 4, page)
        qd = rng.standard_normal((3, 2, 2, 4))
        for win in ((-1, -1), (3, 1)):
            o, lse = oracle.attention_fwd_kvcache(qd, kc, vc, bt, lens, 0.5, causal, win)
            o2, l2 = library_kvcache(qd, kc, vc, bt, lens, page, 0.5, causal, win)
            if not (np.allclose(o, o2, atol=1e-12, rtol=0)
                    and np.allclose(lse, l2, atol=1e-12, rtol=0)):
                failed.append("kvcache")
    return sorted(set(failed))


def _build(src_text, path):
    c = path + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", c, "-o",
                           path + ".so", "-lm"])
    return path + ".so"


def test_unmutated_oracle_passes(oracle_mod):
    assert pins_fail() == []


CHILD = """
import json, sys
import numpy as np
sys.path[:0] = [%r, %r]
import oracle
import test_oracle_mutants as m
with oracle.using(%r):
    with np.errstate(all="ignore"):
        print(json.dumps(m.pins_fail()))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(oracle_mod, tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site not found exactly once: " + name
    lib = _build(text.replace(old, new), str(tmp_path / name))
    r = subprocess.run([sys.executable, "-c", CHILD % (HERE, os.path.dirname(HERE), lib)],
                       capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return  # the mutant crashed the checks: caught
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, "pins did not catch mutant " + name
