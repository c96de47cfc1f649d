"""GPU parity of fa_bwd against the fp64 CPU oracle, through the C ABI.

The GPU backward takes the GPU forward's O and LSE (as a caller would); the
oracle recomputes everything from the bf16 inputs in fp64. The bar is a
relative Frobenius error of at most 2e-2 on dQ, dK and dV.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from exact_attention_117_amd import inputs
from gpu_util import GRAD_RELF, dev, f64, relf, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_117_amd import fa as fa_mod
    return fa_mod


def fwd_bwd(fa, qb, kb, vb, dob, scale, causal):
    q, k, v, do = dev(qb), dev(kb), dev(vb), dev(dob)
    o, lse = fa.fa_fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 7, 64, 127, 128, 129, 200, 383, 512])
def test_small_shapes_full(fa, d, causal, N):
    B, H = 2, 3
    scale = 1 / math.sqrt(d)
    _, (qb, kb, vb, dob) = inputs.qkv((B, N, H, d), seed=9000 + 2 * N + d + int(causal), n=4)
    say("bwd full compare", (B, N, H, d), "causal", causal)
    dq, dk, dv = fwd_bwd(fa, qb, kb, vb, dob, scale, causal)
    g = oracle.attention_bwd(f64(qb), f64(kb), f64(vb), f64(dob), scale, causal)
    got = {"dq": to_np(dq), "dk": to_np(dk), "dv": to_np(dv)}
    errs = {n: relf(got[n], g[n]) for n in got}
    say("  rel-F errors", {n: "%.2e" % e for n, e in errs.items()})
    for n, e in errs.items():
        # N = 1: dq and dk are exactly zero in the definition; compare absolutely
        if np.linalg.norm(g[n]) < 1e-12:
            assert float(np.max(np.abs(got[n]))) < 1e-3, n
        else:
            assert e <= GRAD_RELF, (n, e)


@pytest.mark.parametrize("name", ["bwd_n8192", "bwd_d256_n8192"])
def test_backward_workload_sampled(fa, name):
    """Batch 2, seqlen 8192, causal: the backward workload (32 heads of d 128)
    and its d = 256 form (16 heads). Whole-head dQ for sampled heads and dK/dV
    on sampled keys of those heads are compared with the oracle."""
    w = inputs.WORKLOADS[name]
    x = inputs.make(w)
    qb, kb, vb, dob = x["bf16"]
    say("bwd workload", (w.B, w.N, w.H, w.d), "seed", w.seed)
    dq, dk, dv = fwd_bwd(fa, qb, kb, vb, dob, w.scale, w.causal)
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    rng = np.random.default_rng(w.seed)
    heads = [(0, 0), (1, w.H - 1), (int(rng.integers(2)), int(rng.integers(w.H)))]
    keys = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, w.N - 1, w.N - 128],
                                     rng.choice(w.N, 120, replace=False)])).astype(np.int64)
    for (b, h) in heads:
        sl = lambda t: f64(t[b:b + 1, :, h:h + 1, :])  # noqa: E731
        r = oracle.attention_bwd_sampled(sl(qb), sl(kb), sl(vb), sl(dob), w.scale, w.causal,
                                         heads=[(0, 0)], k_rows=keys)[(0, 0)]
        e_q = relf(dq[b, :, h].double().numpy(), r["dq"])
        e_k = relf(dk[b, keys, h].double().numpy(), r["dk"])
        e_v = relf(dv[b, keys, h].double().numpy(), r["dv"])
        say("  head", (b, h), "dq %.2e dk %.2e dv %.2e" % (e_q, e_k, e_v))
        assert max(e_q, e_k, e_v) <= GRAD_RELF


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(fa, causal, d):
    """sum_j dK_j = 0 (rows of dS sum to zero); sum_j dV_j = sum_i dO_i
    (rows of P sum to one)."""
    B, N, H = 2, 700, 4
    _, (qb, kb, vb, dob) = inputs.qkv((B, N, H, d), seed=9100 + int(causal), n=4)
    dq, dk, dv = fwd_bwd(fa, qb, kb, vb, dob, 1 / math.sqrt(d), causal)
    dk_sum = to_np(dk).sum(axis=1)
    dk_norm = np.linalg.norm(to_np(dk), axis=(1, 3)).max()
    assert np.max(np.abs(dk_sum)) <= 2e-2 * dk_norm
    dv_sum = to_np(dv).sum(axis=1)
    do_sum = f64(dob).sum(axis=1)
    assert np.max(np.abs(dv_sum - do_sum)) <= 2e-2 * np.max(np.abs(do_sum)) + 0.05


def test_constant_v_gives_zero_dq_dk(fa):
    B, N, H, d = 1, 300, 2, 64
    _, (qb, kb, _, dob) = inputs.qkv((B, N, H, d), seed=9200, n=4)
    c = torch.randn(d).to(torch.bfloat16)
    vb = c.expand(B, N, H, d).contiguous()
    dq, dk, dv = fwd_bwd(fa, qb, kb, vb, dob, 0.125, True)
    assert float(to_np(dq).__abs__().max()) < 1e-2
    assert float(to_np(dk).__abs__().max()) < 1e-2


def test_determinism(fa):
    B, N, H, d = 2, 555, 3, 128
    _, (qb, kb, vb, dob) = inputs.qkv((B, N, H, d), seed=9300, n=4)
    q, k, v, do = dev(qb), dev(kb), dev(vb), dev(dob)
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    r1 = fa.fa_bwd(q, k, v, o, do, lse, causal=True)
    ws = torch.full((fa.fa_bwd_workspace_size(B, N, H, d),), 255, dtype=torch.uint8,
                    device="cuda")
    nan = [torch.full_like(q, float("nan")) for _ in range(3)]
    r2 = fa.fa_bwd(q, k, v, o, do, lse, causal=True, dq=nan[0], dk=nan[1], dv=nan[2],
                   workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [128, 256])
def test_single_key_gradients(fa, d):
    """N = 1: P = 1, so dS = 0 (dQ = dK = 0) and dV = dO."""
    B, N, H = 3, 1, 2
    _, (qb, kb, vb, dob) = inputs.qkv((B, N, H, d), seed=9400, n=4)
    dq, dk, dv = fwd_bwd(fa, qb, kb, vb, dob, 0.1, True)
    assert torch.equal(dv.cpu(), dob)
    assert float(to_np(dq).__abs__().max()) < 1e-3 and float(to_np(dk).__abs__().max()) < 1e-3
