"""GPU parity of the FP8 (e4m3) forward against the fp64 CPU oracle, through
the C ABI (fa_fwd_fp8, fa_fwd_varlen_fp8 and the FA_FP8_E4M3 typed calls).

The reference is the oracle's attention on the decoded codes times their
per-tensor descale factors (oracle.e4m3_to_f64), i.e. the same real inputs the
kernel sees; the kernel's own rounding (P and O in bf16, fp32 sums) is what
the bars bound, so they are those of the 16-bit path. Small shapes are
compared over every output, the page-shaped workloads on sampled rows of a
few heads in the launch configuration the benchmark times.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_117_amd import inputs
from gpu_util import LSE_ATOL, max_abs, o_excess, o_tolerance_bf16_p, sample_rows, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_117_amd import fa as fa_mod
    return fa_mod


def codes_f64(c, descale):
    return oracle.e4m3_to_f64(c.contiguous().view(torch.uint8).numpy()) * descale


def draw(shape, seed):
    g = torch.Generator().manual_seed(seed)
    out = [inputs.fp8_codes(torch.randn(shape, generator=g)) for _ in range(3)]
    return [c for c, _ in out], [d for _, d in out]


def check_full(fa, shape, causal, seed, window=None):
    B, N, H, d = shape
    (qc, kc, vc), ds = draw(shape, seed)
    scale = 1.0 / math.sqrt(d)
    say("fp8 fwd", shape, "causal", causal, "window", window)
    o, lse = fa.fa_fwd_fp8(qc.cuda(), kc.cuda(), vc.cuda(), *ds, scale=scale, causal=causal,
                           window=window)
    torch.cuda.synchronize()
    q, k, v = (codes_f64(c, s) for c, s in zip((qc, kc, vc), ds))
    o_ref, l_ref = oracle.attention_fwd(q, k, v, scale, causal,
                                        window=window if window else (-1, -1))
    og, lg = to_np(o), to_np(lse)
    if window:
        i = np.arange(N)
        keep = np.ones((N, N), bool)
        if causal:
            keep &= i[None, :] <= i[:, None]
        if window[0] >= 0:
            keep &= i[None, :] >= i[:, None] - window[0]
        if window[1] >= 0 and not causal:
            keep &= i[None, :] <= i[:, None] + window[1]
        tol = o_tolerance_bf16_p(q, k, v, o_ref, l_ref, scale, keep)
        assert np.all(np.abs(og - o_ref) <= tol)
    else:
        assert o_excess(og, o_ref) <= 0, max_abs(og, o_ref)
    assert max_abs(lg, l_ref) <= LSE_ATOL
    say("  O err %.3e LSE err %.3e" % (max_abs(og, o_ref), max_abs(lg, l_ref)))


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 64, 127, 129, 200, 383, 512])
def test_small_shapes_full(fa, d, causal, N):
    check_full(fa, (2, N, 3, d), causal, 12000 + 2 * N + d + int(causal))


@pytest.mark.parametrize("window", [(0, 0), (31, -1), (64, 40), (200, 0)])
def test_window_full(fa, window):
    check_full(fa, (1, 700, 2, 128), window[1] == 0, 12500 + window[0], window)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_ragged_and_empty_full(fa, d, causal):
    lens = [1, 127, 0, 129, 300, 0, 64, 5]
    g = torch.Generator().manual_seed(12600 + d + int(causal))
    total = sum(lens)
    codes = [inputs.fp8_codes(torch.randn((total, 3, d), generator=g)) for _ in range(3)]
    (qc, kc, vc), ds = [c for c, _ in codes], [s for _, s in codes]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    scale = 1 / math.sqrt(d)
    say("fp8 varlen", lens, d, causal)
    o, lse = fa.fa_fwd_varlen_fp8(qc.cuda(), kc.cuda(), vc.cuda(), cu.cuda(), max(lens), *ds,
                                  scale=scale, causal=causal)
    torch.cuda.synchronize()
    q, k, v = (codes_f64(c, s) for c, s in zip((qc, kc, vc), ds))
    o_ref, l_ref = oracle.attention_fwd_varlen(q, k, v, cu, scale, causal)
    assert o_excess(to_np(o), o_ref) <= 0
    assert max_abs(to_np(lse), l_ref) <= LSE_ATOL


@pytest.mark.parametrize("name", ["headline_fp8", "p4_n8192_fp8", "p4_n8192_nc_fp8",
                                  "d256_n8192_fp8"])
def test_page_workloads_sampled(fa, name):
    w = inputs.WORKLOADS[name]
    x = inputs.make(w)
    qc, kc, vc = x["bf16"]
    ds = x["descale"]
    say("fp8 workload", name, (w.B, w.N, w.H, w.d), "causal", w.causal, "seed", w.seed)
    o, lse = fa.fa_fwd_fp8(qc.cuda(), kc.cuda(), vc.cuda(), *ds, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    o_c, l_c = o.cpu(), lse.cpu()
    assert torch.isfinite(o_c.float()).all() and torch.isfinite(l_c).all()
    rng = np.random.default_rng(w.seed)
    heads = {(0, 0), (w.B - 1, w.H - 1)}
    while len(heads) < 4:
        heads.add((int(rng.integers(w.B)), int(rng.integers(w.H))))
    worst_o, worst_l, excess = 0.0, 0.0, -1.0
    for b, h in sorted(heads):
        rows = sample_rows(w.N, 64, rng)
        q1, k1, v1 = (codes_f64(t[b:b + 1, :, h:h + 1], s) for t, s in zip((qc, kc, vc), ds))
        sel = np.stack([np.zeros_like(rows), np.zeros_like(rows), rows], 1)
        o_ref, l_ref = oracle.attention_fwd(q1, k1, v1, w.scale, w.causal, rows=sel)
        og = o_c[b, rows, h].double().numpy()
        lg = l_c[b, h, rows].double().numpy()
        worst_o = max(worst_o, max_abs(og, o_ref))
        excess = max(excess, o_excess(og, o_ref))
        worst_l = max(worst_l, max_abs(lg, l_ref))
    say("  sampled O err %.3e LSE err %.3e" % (worst_o, worst_l))
    assert excess <= 0 and worst_l <= LSE_ATOL


def test_varlen64_sampled(fa):
    w = inputs.WORKLOADS["varlen64_fp8"]
    x = inputs.make(w)
    qc, kc, vc = x["bf16"]
    ds, lens, cu = x["descale"], x["lengths"], x["cu_seqlens"]
    say("fp8 varlen64 total", qc.shape[0])
    o, lse = fa.fa_fwd_varlen_fp8(qc.cuda(), kc.cuda(), vc.cuda(), cu.cuda(), x["max_seqlen"],
                                  *ds, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    o_c, l_c = o.cpu(), lse.cpu()
    rng = np.random.default_rng(w.seed)
    worst, worst_l = -1.0, 0.0
    for s in sorted({0, 63, int(np.argmax(lens))} | set(int(v) for v in rng.choice(64, 3))):
        a, L = int(cu[s]), lens[s]
        h = int(rng.integers(w.H))
        rows = np.unique(np.concatenate([[0, L - 1], rng.choice(L, min(L, 24), replace=False)]))
        q1, k1, v1 = (codes_f64(t[a:a + L, h:h + 1][None], sc) for t, sc in zip((qc, kc, vc), ds))
        sel = np.stack([np.zeros_like(rows), np.zeros_like(rows), rows], 1)
        o_ref, l_ref = oracle.attention_fwd(q1, k1, v1, w.scale, w.causal, rows=sel)
        worst = max(worst, o_excess(o_c[a + rows, h].double().numpy(), o_ref))
        worst_l = max(worst_l, max_abs(l_c[h, a + rows].double().numpy(), l_ref))
    assert worst <= 0 and worst_l <= LSE_ATOL


@pytest.mark.parametrize("shape", [(2, 8, 16384 - 37, 128), (2, 8, 8192 - 5, 256)])
@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, (1000, 0)),
                                           (False, (300, 200))])
def test_persistent_matches_dispatched_bitwise(fa, shape, causal, window):
    """Without a window the fixed-length FP8 launch runs persistently at these
    sizes (1024 work units, at least four per CU); with one it launches one
    workgroup per unit. Either way it equals the packed call (always one
    workgroup per unit) bit for bit."""
    B, H, N, d = shape
    (qc, kc, vc), ds = draw((B, N, H, d), 12700 + d + int(causal))
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    o = torch.full((B, N, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    fa.fa_fwd_fp8(q, k, v, *ds, causal=causal, o=o, lse=lse, window=window)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    o_v, l_v = fa.fa_fwd_varlen_fp8(q.view(B * N, H, d), k.view(B * N, H, d),
                                    v.view(B * N, H, d), cu, N, *ds, causal=causal,
                                    window=window)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    assert torch.equal(o_v.view(B, N, H, d), o)
    assert torch.equal(l_v.view(H, B, N).permute(1, 0, 2), lse)


def test_zero_q_gives_prefix_mean(fa):
    B, N, H, d = 1, 1000, 2, 128
    (qc, kc, vc), ds = draw((B, N, H, d), 12800)
    qc = torch.zeros_like(qc)
    o, lse = fa.fa_fwd_fp8(qc.cuda(), kc.cuda(), vc.cuda(), *ds, causal=True)
    torch.cuda.synchronize()
    assert max_abs(to_np(lse)[0, 0], np.log(np.arange(1, N + 1))) < 2e-5
    v = codes_f64(vc, ds[2])
    mean = np.cumsum(v, axis=1) / np.arange(1, N + 1)[None, :, None, None]
    assert np.all(np.abs(to_np(o) - mean) <= 2.0 ** -8 * np.abs(mean) + 1e-5)


def test_typed_call_with_unit_descales_is_the_fp8_call(fa):
    B, N, H, d = 2, 333, 4, 128
    (qc, kc, vc), _ = draw((B, N, H, d), 12900)
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    o1, l1 = fa.fa_fwd_fp8(q, k, v, 1.0, 1.0, 1.0, causal=True)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    st = fa.lib.fa_fwd_typed(fa.FA_FP8_E4M3, fa._ptr(q), fa._ptr(k), fa._ptr(v), fa._ptr(o2),
                             fa._ptr(l2), B, N, H, d, ctypes.c_float(1 / math.sqrt(d)), 1, -1, -1,
                             fa._stream(q.device))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
