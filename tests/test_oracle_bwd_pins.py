"""Pins for the CPU oracle's backward: central finite differences of the
forward, a library autodiff (torch fp64 autograd of the plain definition),
and exact invariants. The pages only state that the backward recomputes the
forward (page "Flash Attention V3" section 3.2; page "FlashAttention-2",
backward section); the gradient formulas are the calculus of the definition.
"""
import math

import numpy as np
import pytest
import torch

from test_oracle_pins import band_mask


def rng(B, N, H, d, seed, n=4):
    r = np.random.default_rng(seed)
    return [r.standard_normal((B, N, H, d)) for _ in range(n)]


def loss(oracle_mod, q, k, v, do, scale, causal):
    o, _ = oracle_mod.attention_fwd(q, k, v, scale, causal, threads=1)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 3), (5, 2), (8, 4)])
def test_bwd_central_differences(oracle_mod, causal, N, d):
    B, H = 1, 2
    q, k, v, do = rng(B, N, H, d, seed=100 + N)
    scale = 0.7
    g = oracle_mod.attention_bwd(q, k, v, do, scale, causal)
    eps = 1e-5
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = loss(oracle_mod, q, k, v, do, scale, causal)
            x[idx] = old - eps
            lm = loss(oracle_mod, q, k, v, do, scale, causal)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=0, atol=1e-8, err_msg=name)


def torch_reference_grads(q, k, v, do, scale, causal, window=(-1, -1)):
    """Library autodiff of the plain definition, in fp64 on the CPU."""
    tq, tk, tv = (torch.tensor(np.transpose(x, (0, 2, 1, 3)), requires_grad=True)
                  for x in (q, k, v))
    s = scale * torch.matmul(tq, tk.transpose(-1, -2))
    if causal or window != (-1, -1):
        N = s.shape[-1]
        keep = torch.tensor(band_mask(N, causal, window))
        s = s.masked_fill(~keep, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(np.transpose(do, (0, 2, 1, 3))))
    return {n: np.transpose(t.grad.numpy(), (0, 2, 1, 3)) for n, t in
            (("dq", tq), ("dk", tk), ("dv", tv))}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 4), (2, 33, 3, 16), (1, 130, 2, 64)])
def test_bwd_vs_autograd(oracle_mod, causal, shape):
    q, k, v, do = rng(*shape, seed=sum(shape))
    scale = 1 / math.sqrt(shape[-1])
    g = oracle_mod.attention_bwd(q, k, v, do, scale, causal)
    ref = torch_reference_grads(q, k, v, do, scale, causal)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(g[n], ref[n], rtol=0, atol=1e-11, err_msg=n)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(oracle_mod, causal):
    B, N, H, d = 2, 41, 2, 8
    q, k, v, do = rng(B, N, H, d, seed=200)
    g = oracle_mod.attention_bwd(q, k, v, do, 0.35, causal)
    # every row of dS sums to zero  ->  sum_j dk_j = 0
    np.testing.assert_allclose(g["dk"].sum(axis=1), 0.0, rtol=0, atol=1e-11)
    # every row of P sums to one    ->  sum_j dv_j = sum_i dO_i
    np.testing.assert_allclose(g["dv"].sum(axis=1), do.sum(axis=1), rtol=0, atol=1e-11)
    # D_i = rowsum(dO_i * O_i), the form the GPU path uses
    o, lse = oracle_mod.attention_fwd(q, k, v, 0.35, causal)
    np.testing.assert_allclose(g["D"], np.einsum("bnhc,bnhc->bhn", do, o), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["lse"], lse, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_constant_v(oracle_mod, causal):
    B, N, H, d = 1, 30, 2, 8
    q, k, _, do = rng(B, N, H, d, seed=201)
    v = np.broadcast_to(np.arange(d, dtype=float), q.shape).copy()
    g = oracle_mod.attention_bwd(q, k, v, do, 0.5, causal)
    np.testing.assert_allclose(g["dq"], 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dk"], 0.0, rtol=0, atol=1e-12)


def test_bwd_causal_last_key(oracle_mod):
    # Under the causal mask key N-1 is seen only by row N-1:
    # dv_{N-1} = P_{N-1,N-1} dO_{N-1}.
    B, N, H, d = 1, 12, 1, 4
    q, k, v, do = rng(B, N, H, d, seed=202)
    g = oracle_mod.attention_bwd(q, k, v, do, 0.6, True)
    s = 0.6 * (q[0, N - 1, 0] @ k[0, N - 1, 0])
    p = math.exp(s - g["lse"][0, 0, N - 1])
    np.testing.assert_allclose(g["dv"][0, N - 1, 0], p * do[0, N - 1, 0], rtol=0, atol=1e-13)


def test_bwd_sampled_matches_full(oracle_mod):
    B, N, H, d = 2, 40, 2, 8
    q, k, v, do = rng(B, N, H, d, seed=203)
    for causal in (False, True):
        g = oracle_mod.attention_bwd(q, k, v, do, 0.4, causal)
        s = oracle_mod.attention_bwd_sampled(q, k, v, do, 0.4, causal, heads=[(1, 0), (0, 1)],
                                             q_rows=[0, 5, 39], k_rows=[39, 0, 17])
        for (b, h), r in s.items():
            np.testing.assert_array_equal(r["dq"], g["dq"][b, r["rows"], h])
            np.testing.assert_array_equal(r["dk"], g["dk"][b, r["keys"], h])
            np.testing.assert_array_equal(r["dv"], g["dv"][b, r["keys"], h])


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_equal_lengths_equals_fixed(oracle_mod, causal):
    """A packed batch of equal-length sequences is the fixed-length problem."""
    B, N, H, d = 3, 9, 2, 4
    r = np.random.default_rng(11)
    q, k, v, do = (r.standard_normal((B, N, H, d)) for _ in range(4))
    g = oracle_mod.attention_bwd(q, k, v, do, 0.4, causal)
    cu = np.arange(0, (B + 1) * N, N)
    gv = oracle_mod.attention_bwd_varlen(*(x.reshape(B * N, H, d) for x in (q, k, v, do)), cu,
                                         0.4, causal)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(gv[n].reshape(B, N, H, d), g[n], rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen_each_sequence_alone_and_empty(oracle_mod, causal):
    """Each sequence's gradients equal those of that sequence alone (no
    leakage across sequence bounds); empty sequences contribute nothing."""
    lens = [5, 0, 1, 7, 0]
    cu = np.concatenate([[0], np.cumsum(lens)])
    total, H, d = int(cu[-1]), 2, 3
    r = np.random.default_rng(12)
    q, k, v, do = (r.standard_normal((total, H, d)) for _ in range(4))
    gv = oracle_mod.attention_bwd_varlen(q, k, v, do, cu, 0.6, causal)
    for s, L in enumerate(lens):
        if L == 0:
            continue
        a = int(cu[s])
        g = oracle_mod.attention_bwd(*(x[a:a + L][None] for x in (q, k, v, do)), 0.6, causal)
        for n in ("dq", "dk", "dv"):
            np.testing.assert_allclose(gv[n][a:a + L], g[n][0], rtol=0, atol=1e-13)
    # a one-row sequence: P = 1, so dq = dk = 0 and dv = dO
    a = int(cu[2])
    np.testing.assert_allclose(gv["dv"][a], do[a], rtol=0, atol=1e-13)
    np.testing.assert_allclose(gv["dq"][a], 0, atol=1e-13)


@pytest.mark.parametrize("window", [(0, 0), (2, 0), (3, 1), (-1, 2), (1, -1)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_window_vs_autograd(oracle_mod, causal, window):
    """Backward of sliding-window attention against library autodiff of the
    banded definition."""
    q, k, v, do = rng(2, 13, 2, 5, seed=41)
    g = oracle_mod.attention_bwd(q, k, v, do, 0.45, causal, window=window)
    ref = torch_reference_grads(q, k, v, do, 0.45, causal, window=window)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(g[n], ref[n], rtol=0, atol=1e-11, err_msg=n)


def test_bwd_window_central_differences(oracle_mod):
    q, k, v, do = rng(1, 6, 1, 3, seed=42)
    win = (2, 1)
    g = oracle_mod.attention_bwd(q, k, v, do, 0.7, False, window=win)

    def loss(qq, kk, vv):
        o, _ = oracle_mod.attention_fwd(qq, kk, vv, 0.7, False, window=win)
        return float(np.sum(o * do))

    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g[name], num, rtol=0, atol=1e-7, err_msg=name)
