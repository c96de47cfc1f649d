"""GPU parity of the float16 path (the *_typed entry points with FA_FP16)
against the fp64 CPU oracle, through the C ABI.

The page "FlashAttention-2" runs its usage examples in float16. The kernels are
the bfloat16 kernels over another element type: float16 operands on the
f16 MFMAs, P rounded to float16. The bars are the bfloat16 ones (float16
keeps more significant bits). Covered: small shapes in full (causal, full,
windowed), packed variable-length batches, the backward (fixed and packed),
decoding with an append, the headline shape sampled, and the typed calls with
bfloat16 tensors giving the plain calls' bits.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_117_amd import inputs
from gpu_util import GRAD_RELF, LSE_ATOL, dev, max_abs, o_excess, relf, sample_rows, say, to_np

pytestmark = pytest.mark.gpu
F16 = torch.float16


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_117_amd import fa as fa_mod
    return fa_mod


def w64(t):
    """Exact fp64 copy of a float16 CPU tensor."""
    return t.double().numpy()


def grads_ok(got, ref, tag):
    for n in ("dq", "dk", "dv"):
        g = to_np(got[n])
        if np.linalg.norm(ref[n]) < 1e-12:  # e.g. dq of a one-key sequence is exactly 0
            assert float(np.max(np.abs(g))) < 1e-3, (tag, n)
        else:
            e = relf(g, ref[n])
            assert e <= GRAD_RELF, (tag, n, e)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 63, 200, 513])
@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, (100, 0)),
                                           (False, (37, 5))])
def test_fwd_small_full(fa, d, N, causal, window):
    B, H = 2, 3
    _, (qh, kh, vh) = inputs.qkv((B, N, H, d), seed=12000 + N + d, dtype=F16)
    scale = 1 / math.sqrt(d)
    say("fp16 fwd", (B, N, H, d), causal, window)
    o, lse = fa.fa_fwd_typed(dev(qh), dev(kh), dev(vh), *(window or (-1, -1)), scale=scale,
                             causal=causal)
    torch.cuda.synchronize()
    assert o.dtype == F16
    o_ref, lse_ref = oracle.attention_fwd(w64(qh), w64(kh), w64(vh), scale, causal,
                                          window=window or (-1, -1))
    say("  O err %.3e  LSE err %.3e" % (max_abs(to_np(o), o_ref), max_abs(to_np(lse), lse_ref)))
    assert o_excess(to_np(o), o_ref) <= 0
    assert max_abs(to_np(lse), lse_ref) <= LSE_ATOL


def test_headline_shape_sampled(fa):
    B, N, H, d = 4, 4096, 32, 128
    _, (qh, kh, vh) = inputs.qkv((B, N, H, d), seed=12500, dtype=F16)
    o, lse = fa.fa_fwd(dev(qh), dev(kh), dev(vh), causal=True)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    assert torch.isfinite(o_c.float()).all() and torch.isfinite(lse_c).all()
    rng = np.random.default_rng(12500)
    for b, h in ((0, 0), (3, 31), (1, 17)):
        rows = sample_rows(N, 40, rng, tile=256)
        sel = np.stack([np.zeros_like(rows), np.zeros_like(rows), rows], 1)
        q1, k1, v1 = (w64(t[b:b + 1, :, h:h + 1, :]) for t in (qh, kh, vh))
        o_ref, l_ref = oracle.attention_fwd(q1, k1, v1, 1 / math.sqrt(d), True, rows=sel)
        assert o_excess(o_c[b, rows, h].double().numpy(), o_ref) <= 0
        assert max_abs(lse_c[b, h, rows].double().numpy(), l_ref) <= LSE_ATOL


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_fwd_bwd(fa, d, causal):
    lens = [1, 127, 0, 129, 300, 64, 5, 257]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    _, (qh, kh, vh, doh) = inputs.qkv((int(cu[-1]), 3, d), seed=12600 + d + int(causal), n=4,
                                      dtype=F16)
    scale = 1 / math.sqrt(d)
    q, k, v, do, c = dev(qh), dev(kh), dev(vh), dev(doh), dev(cu)
    o, lse = fa.fa_fwd_varlen(q, k, v, c, max(lens), scale=scale, causal=causal)
    dq, dk, dv = fa.fa_bwd_varlen(q, k, v, o, do, lse, c, max(lens), scale=scale,
                                  causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd_varlen(w64(qh), w64(kh), w64(vh), cu, scale, causal)
    assert o_excess(to_np(o), o_ref) <= 0
    assert max_abs(to_np(lse), lse_ref) <= LSE_ATOL
    ref = oracle.attention_bwd_varlen(w64(qh), w64(kh), w64(vh), w64(doh), cu, scale, causal)
    for s, L in enumerate(lens):
        if L == 0:
            continue
        a = int(cu[s])
        grads_ok({"dq": dq[a:a + L], "dk": dk[a:a + L], "dv": dv[a:a + L]},
                 {n: ref[n][a:a + L] for n in ("dq", "dk", "dv")}, ("seq", s))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [63, 300, 520])
@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, (64, 0))])
def test_bwd_small_full(fa, d, N, causal, window):
    B, H = 2, 2
    _, (qh, kh, vh, doh) = inputs.qkv((B, N, H, d), seed=12700 + N + d, n=4, dtype=F16)
    scale = 1 / math.sqrt(d)
    q, k, v, do = dev(qh), dev(kh), dev(vh), dev(doh)
    o, lse = fa.fa_fwd(q, k, v, scale=scale, causal=causal, window=window)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, scale=scale, causal=causal, window=window)
    torch.cuda.synchronize()
    assert dq.dtype == F16
    ref = oracle.attention_bwd(w64(qh), w64(kh), w64(vh), w64(doh), scale, causal,
                               window=window or (-1, -1))
    grads_ok({"dq": dq, "dk": dk, "dv": dv}, ref, (N, d, causal, window))


def test_bwd_workload_shape_sampled(fa):
    B, N, H, d = 2, 8192, 32, 128
    _, (qh, kh, vh, doh) = inputs.qkv((B, N, H, d), seed=12800, n=4, dtype=F16)
    q, k, v, do = dev(qh), dev(kh), dev(vh), dev(doh)
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    rng = np.random.default_rng(12800)
    keys = np.unique(np.concatenate([[0, 1, 127, 128, N - 1],
                                     rng.choice(N, 60, replace=False)])).astype(np.int64)
    for b, h in ((0, 0), (1, 31)):
        sl = lambda t: w64(t[b:b + 1, :, h:h + 1, :])  # noqa: E731
        r = oracle.attention_bwd_sampled(sl(qh), sl(kh), sl(vh), sl(doh), 1 / math.sqrt(d),
                                         True, heads=[(0, 0)], k_rows=keys)[(0, 0)]
        e = (relf(dq[b, :, h].double().numpy(), r["dq"]),
             relf(dk[b, keys, h].double().numpy(), r["dk"]),
             relf(dv[b, keys, h].double().numpy(), r["dv"]))
        say("  fp16 bwd head", (b, h), "dq %.2e dk %.2e dv %.2e" % e)
        assert max(e) <= GRAD_RELF


@pytest.mark.parametrize("d", [64, 128, 256])
def test_decode_with_append(fa, d):
    x = inputs.make_kvcache([0, 5, 300, 1111], H=4, d=d, page=16, nq=3, seed=12900 + d)
    for n in ("q", "k_new", "v_new", "k_cache", "v_cache"):
        x[n] = x[n].float().to(F16)
    xd = {n: t.cuda() for n, t in x.items() if isinstance(t, torch.Tensor)}
    total = [L + 3 for L in x["lengths"]]
    o, lse = fa.fa_fwd_kvcache(xd["q"], xd["k_cache"], xd["v_cache"], xd["block_table"],
                               xd["cache_seqlens"], max(total), k_new=xd["k_new"],
                               v_new=xd["v_new"], causal=True)
    torch.cuda.synchronize()
    bt = x["block_table"].numpy().astype(np.int64)
    kc, vc = oracle.kvcache_append(w64(x["k_cache"]), w64(x["v_cache"]), w64(x["k_new"]),
                                   w64(x["v_new"]), bt, x["cache_seqlens"].numpy())
    o_ref, lse_ref = oracle.attention_fwd_kvcache(w64(x["q"]), kc, vc, bt, total,
                                                  1 / math.sqrt(d), True)
    assert o_excess(to_np(o), o_ref) <= 0
    assert max_abs(lse.cpu().numpy().astype(np.float64), lse_ref) <= LSE_ATOL
    kc_bits = oracle.kvcache_append(x["k_cache"].view(torch.int16).numpy(),
                                    x["v_cache"].view(torch.int16).numpy(),
                                    x["k_new"].view(torch.int16).numpy(),
                                    x["v_new"].view(torch.int16).numpy(),
                                    x["block_table"].numpy(), x["cache_seqlens"].numpy())
    assert np.array_equal(xd["k_cache"].cpu().view(torch.int16).numpy(), kc_bits[0])


def test_typed_calls_with_bf16_equal_the_plain_calls(fa):
    B, N, H, d = 2, 333, 4, 128
    _, (qb, kb, vb, dob) = inputs.qkv((B, N, H, d), seed=12950, n=4)
    q, k, v, do = dev(qb), dev(kb), dev(vb), dev(dob)
    o1, l1 = fa.fa_fwd(q, k, v, causal=True)
    o2, l2 = fa.fa_fwd_typed(q, k, v, causal=True)
    g1 = fa.fa_bwd(q, k, v, o1, do, l1, causal=True)
    g2 = fa.fa_bwd_typed(q, k, v, o1, do, l1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_mixed_types_are_rejected(fa):
    q = torch.zeros((1, 8, 1, 64), dtype=F16, device="cuda")
    with pytest.raises(TypeError):
        fa.fa_fwd(q, q.to(torch.bfloat16), q)
