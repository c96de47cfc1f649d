"""GPU parity of fa_fwd against the fp64 CPU oracle, through the C ABI.

Small shapes are compared element by element over every output; the page
workloads (batch 8 / 16 heads / d 64 and batch 2 / 32 heads / d 128 at their
sequence lengths, plus batch 4 / 32 heads / 4096 / d 128) run in the same
launch configuration the benchmark times and are compared on sampled rows.
Structure tests catch errors the loose tolerances would let through (a causal
off-by-one changes an output by about 1/N).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_117_amd import inputs
from gpu_util import (LSE_ATOL, dev, f64, max_abs, o_excess, oracle_rows_one_head,
                      sample_rows, say, to_np)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_117_amd import fa as fa_mod
    return fa_mod


def run_fwd(fa, qb, kb, vb, scale, causal):
    q, k, v = dev(qb), dev(kb), dev(vb)
    o, lse = fa.fa_fwd(q, k, v, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o, lse


def full_compare(fa, qb, kb, vb, scale, causal, tag):
    say("fwd full compare", tag, tuple(qb.shape), "causal", causal)
    o, lse = run_fwd(fa, qb, kb, vb, scale, causal)
    o_ref, lse_ref = oracle.attention_fwd(f64(qb), f64(kb), f64(vb), scale, causal)
    eo, el = max_abs(to_np(o), o_ref), max_abs(to_np(lse), lse_ref)
    say("  O err %.3e  LSE err %.3e" % (eo, el))
    assert o_excess(to_np(o), o_ref) <= 0, tag
    assert el <= LSE_ATOL, tag
    return eo, el


def test_tiny_workload(fa):
    w = inputs.WORKLOADS["tiny"]
    x = inputs.make(w)
    eo, el = full_compare(fa, *x["bf16"], w.scale, w.causal, "tiny")
    # fp32-input oracle vs bf16-input oracle: the input quantisation effect,
    # reported only (the GPU path computes on the bf16 values)
    qf, kf, vf = (t.double().numpy() for t in x["f32"])
    o32, _ = oracle.attention_fwd(qf, kf, vf, w.scale, w.causal)
    ob, _ = oracle.attention_fwd(*(f64(t) for t in x["bf16"]), w.scale, w.causal)
    say("  input quantisation |O(fp32 in) - O(bf16 in)| max %.3e" % max_abs(o32, ob))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 64, 127, 128, 129, 200, 383, 512])
def test_small_shapes_full(fa, d, causal, N):
    B, H = 2, 3
    _, (qb, kb, vb) = inputs.qkv((B, N, H, d), seed=7000 + N * 2 + d + int(causal))
    full_compare(fa, qb, kb, vb, 1.0 / math.sqrt(d), causal, "N=%d d=%d" % (N, d))


@pytest.mark.parametrize("name", ["p1_n1024", "p1_n2048", "p1_n4096", "p4_n2048", "p4_n4096",
                                  "p4_n8192", "p4_n16384", "p4_n2048_nc", "p4_n4096_nc",
                                  "p4_n8192_nc", "p4_n16384_nc", "headline", "d256_n8192"])
def test_page_workloads_sampled(fa, name):
    w = inputs.WORKLOADS[name]
    say("fwd workload", name, (w.B, w.N, w.H, w.d), "causal", w.causal, "seed", w.seed)
    x = inputs.make(w)
    qb, kb, vb = x["bf16"]
    o, lse = run_fwd(fa, qb, kb, vb, w.scale, w.causal)
    o_c, lse_c = o.cpu(), lse.cpu()
    assert torch.isfinite(o_c.float()).all() and torch.isfinite(lse_c).all()
    rng = np.random.default_rng(w.seed)
    heads = {(0, 0), (w.B - 1, w.H - 1)}
    while len(heads) < 4:
        heads.add((int(rng.integers(w.B)), int(rng.integers(w.H))))
    worst_o = worst_l = 0.0
    excess = -1.0
    for (b, h) in sorted(heads):
        rows = sample_rows(w.N, 48, rng)
        o_ref, l_ref = oracle_rows_one_head(qb, kb, vb, b, h, rows, w.scale, w.causal)
        og = o_c[b, rows, h].double().numpy()
        lg = lse_c[b, h, rows].double().numpy()
        worst_o = max(worst_o, max_abs(og, o_ref))
        excess = max(excess, o_excess(og, o_ref))
        worst_l = max(worst_l, max_abs(lg, l_ref))
    say("  sampled O err %.3e  LSE err %.3e" % (worst_o, worst_l))
    assert excess <= 0 and worst_l <= LSE_ATOL


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [300, 4096])
def test_zero_q_gives_prefix_mean(fa, d, N):
    """Q = 0: every score is 0, so o_i is the mean of v_0..v_i and
    lse_i = ln(i+1) (causal). A causal off-by-one shifts lse_i by ~1/(i+1)."""
    B, H = 1, 2
    _, (qb, kb, vb) = inputs.qkv((B, N, H, d), seed=7100 + N + d)
    qb = torch.zeros_like(qb)
    say("zero-q prefix mean", N, d)
    o, lse = run_fwd(fa, qb, kb, vb, 1 / math.sqrt(d), True)
    lse_ref = np.log(np.arange(1, N + 1))
    assert max_abs(to_np(lse)[0, 0], lse_ref) < 2e-5
    v = f64(vb)
    mean = np.cumsum(v, axis=1) / np.arange(1, N + 1)[None, :, None, None]
    assert np.all(np.abs(to_np(o) - mean) <= 2.0 ** -8 * np.abs(mean) + 1e-5)
    # non-causal: lse = ln N everywhere
    o, lse = run_fwd(fa, qb, kb, vb, 1 / math.sqrt(d), False)
    assert max_abs(to_np(lse), math.log(N)) < 2e-5
    mean = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
    assert np.all(np.abs(to_np(o) - mean) <= 2.0 ** -8 * np.abs(mean) + 1e-5)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_causal_row0_is_v0_and_constant_v(fa, d):
    B, N, H = 2, 1000, 2
    _, (qb, kb, vb) = inputs.qkv((B, N, H, d), seed=7200 + d)
    o, lse = run_fwd(fa, qb, kb, vb, 1 / math.sqrt(d), True)
    assert torch.equal(o[:, 0].cpu(), vb[:, 0])
    s00 = (f64(qb)[:, 0] * f64(kb)[:, 0]).sum(-1) / math.sqrt(d)
    assert max_abs(to_np(lse)[:, :, 0], s00) < 1e-4
    c = torch.randn(d).to(torch.bfloat16)
    vc = c.expand(B, N, H, d).contiguous()
    o, _ = run_fwd(fa, qb, kb, vc, 1 / math.sqrt(d), True)
    cc = np.broadcast_to(c.double().numpy(), (B, N, H, d))
    assert np.all(np.abs(to_np(o) - cc) <= 2.0 ** -7 * np.abs(cc) + 1e-4)


def test_determinism_and_full_overwrite(fa):
    B, N, H, d = 2, 777, 4, 128
    _, (qb, kb, vb) = inputs.qkv((B, N, H, d), seed=7300)
    q, k, v = dev(qb), dev(kb), dev(vb)
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full((B, H, N), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, causal=True, o=o1, lse=l1)
    o2, l2 = fa.fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("shape", [(2, 8, 16384 - 37, 64), (2, 8, 16384 - 37, 128),
                                   (2, 8, 8192 - 37, 256), (8, 16, 3067, 128),
                                   (2, 8, 32768 - 5, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_persistent_schedule_matches_dispatched(fa, shape, causal):
    """A fixed-length launch with at least four query tiles per CU and heads
    that split evenly over the XCDs runs persistently (one workgroup per CU
    looping over its units). Its output equals, bit for bit, the packed
    variable-length call on the same sequences, which always launches one
    workgroup per unit; NaN-filled outputs show that every row is written.
    The lengths are ragged, so the last query and key tiles are partial; one
    shape has 12 query tiles per sequence, which do not divide a round of 32
    workgroups, and the last has 128, more than a round, over one unit per
    XCD."""
    B, H, N, d = shape
    say("persistent fwd", (B, N, H, d), "causal", causal)
    _, (qb, kb, vb) = inputs.qkv((B, N, H, d), seed=7500 + d + int(causal))
    q, k, v = dev(qb), dev(kb), dev(vb)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, causal=causal, o=o, lse=lse)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    o_v, l_v = fa.fa_fwd_varlen(q.view(B * N, H, d), k.view(B * N, H, d), v.view(B * N, H, d),
                                cu, N, causal=causal)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    assert torch.equal(o_v.view(B, N, H, d), o)
    assert torch.equal(l_v.view(H, B, N).permute(1, 0, 2), lse)


def test_guard_canaries(fa):
    """Outputs placed inside larger buffers: nothing outside them changes."""
    B, N, H, d = 1, 300, 2, 64
    _, (qb, kb, vb) = inputs.qkv((B, N, H, d), seed=7400)
    q, k, v = dev(qb), dev(kb), dev(vb)
    n = B * N * H * d
    pad = 4096
    big_o = torch.full((n + 2 * pad,), 3.0, dtype=torch.bfloat16, device="cuda")
    big_l = torch.full((B * H * N + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    o = big_o[pad:pad + n].view(B, N, H, d)
    lse = big_l[pad:pad + B * H * N].view(B, H, N)
    fa.fa_fwd(q, k, v, causal=True, o=o, lse=lse)
    torch.cuda.synchronize()
    assert (big_o[:pad] == 3.0).all() and (big_o[pad + n:] == 3.0).all()
    assert (big_l[:pad] == 7.0).all() and (big_l[pad + B * H * N:] == 7.0).all()


def test_lse_optional(fa):
    B, N, H, d = 1, 256, 2, 128
    _, (qb, kb, vb) = inputs.qkv((B, N, H, d), seed=7500)
    q, k, v = dev(qb), dev(kb), dev(vb)
    o1, _ = fa.fa_fwd(q, k, v, causal=True, need_lse=False)
    o2, _ = fa.fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_empty_problem_is_noop(fa):
    q = torch.empty((0, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fa_fwd(q, q, q, causal=True)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (0, 2, 16)
