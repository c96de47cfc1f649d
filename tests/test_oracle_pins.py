"""Pins for the CPU oracle's forward, against things other than itself:
hand-derived closed forms (tests/golden), a library softmax (scipy), exact
invariants of the definition, and the online recurrence the tiled method uses.

The definition is that of page "FlashAttention-2" (standard attention
comparison section); causal masking j <= i follows causal=True on page
"FlashAttention实战" section 4.1.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

HERE = os.path.dirname(os.path.abspath(__file__))


def _parse(x):
    if isinstance(x, str) and x.startswith("ln:"):
        return math.log(float(x[3:]))
    if isinstance(x, list):
        return [_parse(y) for y in x]
    return float(x)


def rng_qkv(B, N, H, d, seed, scale_v=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, N, H, d)), r.standard_normal((B, N, H, d)),
            scale_v * r.standard_normal((B, N, H, d)))


def band_mask(N, causal, window=(-1, -1)):
    """visible[i, j] from the offset j - i: causal keeps offsets <= 0, a
    window keeps -wl <= offset <= wr (-1: that side unbounded)."""
    off = np.arange(N)[None, :] - np.arange(N)[:, None]
    keep = np.ones((N, N), bool)
    if causal:
        keep &= off <= 0
    wl, wr = window
    if wl >= 0:
        keep &= off >= -wl
    if wr >= 0:
        keep &= off <= wr
    return keep


def scipy_attention(q, k, v, scale, causal, window=(-1, -1)):
    """Independent expression: numpy matmul scores, masked with -inf, then the
    library's softmax and logsumexp."""
    B, N, H, d = q.shape
    qh, kh, vh = (np.transpose(x, (0, 2, 1, 3)) for x in (q, k, v))
    s = scale * np.matmul(qh, np.swapaxes(kh, -1, -2))
    if causal or window != (-1, -1):
        s = np.where(band_mask(N, causal, window), s, -np.inf)
    p = scipy.special.softmax(s, axis=-1)
    lse = scipy.special.logsumexp(s, axis=-1)
    o = np.matmul(p, vh)
    return np.transpose(o, (0, 2, 1, 3)), lse


@pytest.mark.parametrize("causal", [False, True])
def test_golden_hand_examples(oracle_mod, causal):
    data = json.load(open(os.path.join(HERE, "golden", "hand_examples.json")))
    for ex in data["examples"]:
        q, k, v = (np.array(_parse(ex[n]))[None] for n in ("q", "k", "v"))
        o, lse = oracle_mod.attention_fwd(q, k, v, ex["scale"], causal)
        exp = ex["expect"]["causal" if causal else "noncausal"]
        np.testing.assert_allclose(o, np.array(_parse(exp["o"]))[None], rtol=0, atol=1e-13,
                                   err_msg=ex["name"])
        np.testing.assert_allclose(lse, np.array(_parse(exp["lse"]))[None], rtol=0,
                                   atol=1e-13, err_msg=ex["name"])


@pytest.mark.parametrize("N,d", [(1, 4), (2, 4), (3, 4), (7, 4), (128, 64), (33, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_vs_library_softmax(oracle_mod, N, d, causal):
    q, k, v = rng_qkv(1, N, 2, d, seed=N * 10 + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle_mod.attention_fwd(q, k, v, scale, causal)
    o_ref, lse_ref = scipy_attention(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(oracle_mod, causal):
    # With v_j = e_j (d = N, one-hot values), o_i is exactly the row P_i.
    N = 24
    r = np.random.default_rng(1)
    q = r.standard_normal((1, N, 1, 8)) * 2
    k = r.standard_normal((1, N, 1, 8)) * 2
    qp = np.zeros((1, N, 1, N)); qp[..., :8] = q
    kp = np.zeros((1, N, 1, N)); kp[..., :8] = k
    v = np.eye(N)[None, :, None, :]
    o, _ = oracle_mod.attention_fwd(qp, kp, v, 0.7, causal)
    P = o[0, :, 0, :]
    assert np.all(P >= 0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    if causal:
        assert np.all(np.triu(P, 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(oracle_mod, causal):
    q, k, _ = rng_qkv(2, 40, 3, 16, seed=2)
    c = np.random.default_rng(3).standard_normal(16)
    v = np.broadcast_to(c, q.shape).copy()
    o, _ = oracle_mod.attention_fwd(q, k, v, 0.25, causal)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("zero", ["q", "k", "scale"])
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_give_mean_of_v(oracle_mod, zero, causal):
    B, N, H, d = 2, 37, 2, 8
    q, k, v = rng_qkv(B, N, H, d, seed=4)
    scale = 0.3
    if zero == "q":
        q[:] = 0
    elif zero == "k":
        k[:] = 0
    else:
        scale = 0.0
    o, lse = oracle_mod.attention_fwd(q, k, v, scale, causal)
    if causal:
        counts = np.arange(1, N + 1)
        mean = np.cumsum(v, axis=1) / counts[None, :, None, None]
        lse_ref = np.broadcast_to(np.log(counts), lse.shape)
    else:
        mean = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
        lse_ref = np.full(lse.shape, math.log(N))
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_causal_row0(oracle_mod):
    q, k, v = rng_qkv(2, 19, 3, 8, seed=5)
    o, lse = oracle_mod.attention_fwd(q, k, v, 0.4, True)
    np.testing.assert_array_equal(o[:, 0], v[:, 0])
    s00 = 0.4 * np.einsum("bhc,bhc->bh", q[:, 0], k[:, 0])
    np.testing.assert_allclose(lse[:, :, 0], s00, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(oracle_mod, causal):
    # s_ij -> s_ij + scale <q_i, u> is constant along each row: o unchanged,
    # lse_i shifted by scale <q_i, u>.
    q, k, v = rng_qkv(1, 50, 2, 16, seed=6)
    u = np.random.default_rng(7).standard_normal(16)
    o0, l0 = oracle_mod.attention_fwd(q, k, v, 0.25, causal)
    o1, l1 = oracle_mod.attention_fwd(q, k + u, v, 0.25, causal)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-11)
    shift = 0.25 * np.einsum("bnhc,c->bhn", q, u)
    np.testing.assert_allclose(l1, l0 + shift, rtol=0, atol=1e-11)


def test_joint_key_value_permutation(oracle_mod):
    q, k, v = rng_qkv(1, 45, 2, 8, seed=8)
    perm = np.random.default_rng(9).permutation(45)
    o0, l0 = oracle_mod.attention_fwd(q, k, v, 0.5, False)
    o1, l1 = oracle_mod.attention_fwd(q, k[:, perm], v[:, perm], 0.5, False)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-12)


def test_rows_independent_and_sampled_rows_match(oracle_mod):
    q, k, v = rng_qkv(2, 64, 3, 16, seed=10)
    for causal in (False, True):
        o, lse = oracle_mod.attention_fwd(q, k, v, 0.25, causal)
        sel = np.array([[0, 0, 0], [1, 2, 63], [0, 1, 31], [1, 0, 7]])
        os_, ls = oracle_mod.attention_fwd(q, k, v, 0.25, causal, rows=sel)
        for r, (b, h, i) in enumerate(sel):
            np.testing.assert_array_equal(os_[r], o[b, i, h])
            assert ls[r] == lse[b, h, i]


@pytest.mark.parametrize("tiles", ["1", "16", "64", "random"])
@pytest.mark.parametrize("causal", [False, True])
def test_online_merge_equals_one_shot(oracle_mod, tiles, causal):
    """The tiled recurrence (running max m, running sum l, rescaled partial
    output) reproduces the one-shot softmax of the definition."""
    N, d, scale = 200, 16, 0.9
    q, k, v = rng_qkv(1, N, 1, d, seed=11, scale_v=3.0)
    q *= 3.0  # wide score range, so the running max changes often
    o_ref, lse_ref = oracle_mod.attention_fwd(q, k, v, scale, causal)
    rng = np.random.default_rng(12)
    for i in (0, 1, 5, 99, N - 1):
        n = i + 1 if causal else N
        s = scale * k[0, :n, 0] @ q[0, i, 0]
        if tiles == "random":
            cuts = np.sort(rng.choice(np.arange(1, n), size=min(n - 1, 7), replace=False)) \
                if n > 1 else np.array([], int)
            bounds = [0] + list(cuts) + [n]
        else:
            t = int(tiles)
            bounds = list(range(0, n, t)) + [n]
        o, lse = oracle_mod.online_softmax_merge(s, v[0, :n, 0], bounds)
        np.testing.assert_allclose(o, o_ref[0, i, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref[0, 0, i], rtol=0, atol=1e-12)


def test_online_merge_without_rescale_is_wrong(oracle_mod):
    """Summing un-rescaled per-tile partial outputs (the accumulate-only
    reading of the kernel sketch on page 'FlashAttention实战' section 3.2)
    does not give the definition; the rescale is required."""
    N, d = 64, 4
    q, k, v = rng_qkv(1, N, 1, d, seed=13)
    s = 2.0 * k[0, :, 0] @ q[0, 0, 0]
    o_ref, _ = oracle_mod.attention_fwd(q, k, v, 2.0, False)
    parts = [np.exp(s[a:a + 16] - s[a:a + 16].max()) @ v[0, a:a + 16, 0] for a in range(0, N, 16)]
    ls = [np.exp(s[a:a + 16] - s[a:a + 16].max()).sum() for a in range(0, N, 16)]
    naive = sum(parts) / sum(ls)
    assert np.max(np.abs(naive - o_ref[0, 0, 0])) > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_equals_fixed(oracle_mod, causal):
    B, N, H, d = 3, 20, 2, 8
    q, k, v = rng_qkv(B, N, H, d, seed=14)
    o, lse = oracle_mod.attention_fwd(q, k, v, 0.3, causal)
    cu = np.arange(0, (B + 1) * N, N)
    ov, lv = oracle_mod.attention_fwd_varlen(q.reshape(B * N, H, d), k.reshape(B * N, H, d),
                                             v.reshape(B * N, H, d), cu, 0.3, causal)
    np.testing.assert_array_equal(ov, o.reshape(B * N, H, d))
    np.testing.assert_array_equal(lv, lse.transpose(1, 0, 2).reshape(H, B * N))


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_each_sequence_alone_and_empty(oracle_mod, causal):
    lens = [5, 0, 17, 1, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, d = int(cu[-1]), 2, 8
    r = np.random.default_rng(15)
    q, k, v = (r.standard_normal((T, H, d)) for _ in range(3))
    ov, lv = oracle_mod.attention_fwd_varlen(q, k, v, cu, 0.5, causal)
    for s, L in enumerate(lens):
        a = cu[s]
        if L == 0:
            continue
        o1, l1 = scipy_attention(q[a:a + L][None], k[a:a + L][None], v[a:a + L][None], 0.5,
                                 causal)
        np.testing.assert_allclose(ov[a:a + L], o1[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lv[:, a:a + L], l1[0], rtol=0, atol=1e-12)


def test_page_shapes(oracle_mod):
    """Shapes the pages print for their examples, on the oracle (head dim cut
    to keep the CPU run short where the shape check allows it)."""
    g = json.load(open(os.path.join(HERE, "golden", "page_shapes.json")))
    vl = g["varlen"]
    cu = np.concatenate([[0], np.cumsum(vl["lengths"])])
    assert list(cu) == vl["cu_seqlens"]
    assert max(vl["lengths"]) == vl["max_seqlen"]
    T = int(cu[-1])
    r = np.random.default_rng(16)
    q, k, v = (r.standard_normal((T, vl["H"], vl["d"])) for _ in range(3))
    o, lse = oracle_mod.attention_fwd_varlen(q, k, v, cu, 1 / math.sqrt(vl["d"]), vl["causal"])
    assert list(o.shape) == vl["output_shape"]
    assert lse.shape == (vl["H"], T)
    sm = g["score_matrix_bytes"]
    gib = sm["B"] * sm["H"] * sm["N"] ** 2 * sm["bytes_per_score"] / 2 ** 30
    assert gib == sm["approx_gb"]


def test_bf16_widening_is_exact(oracle_mod):
    import torch
    x = torch.randn(1000, dtype=torch.float32)
    b = x.to(torch.bfloat16)
    w = oracle_mod.bf16_bits_to_f64(b.view(torch.int16).numpy())
    np.testing.assert_array_equal(w, b.to(torch.float64).numpy())
    # bf16 keeps the top 16 bits of fp32 with round-to-nearest-even
    assert np.all(np.abs(w - x.numpy()) <= np.abs(x.numpy()) * 2.0 ** -8)


WINDOWS = [(0, 0), (3, 0), (2, 5), (0, -1), (7, -1), (-1, 4), (100, 100)]


@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("causal", [False, True])
def test_window_bruteforce_vs_library_softmax(oracle_mod, causal, window):
    """Sliding-window (local) attention against the library softmax of the
    banded mask (page "FlashAttention技术深度解析", attention variants)."""
    q, k, v = rng_qkv(2, 19, 2, 8, seed=31)
    o, lse = oracle_mod.attention_fwd(q, k, v, 0.35, causal, window=window)
    o_ref, lse_ref = scipy_attention(q, k, v, 0.35, causal, window)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_window_zero_is_identity(oracle_mod):
    """A window of width zero on both sides: row i sees only key i, so
    o_i = v_i and lse_i = s_ii exactly."""
    q, k, v = rng_qkv(1, 11, 3, 6, seed=32)
    o, lse = oracle_mod.attention_fwd(q, k, v, 0.5, False, window=(0, 0))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    s_ii = 0.5 * np.einsum("bnhd,bnhd->bhn", q, k)
    np.testing.assert_allclose(lse, s_ii, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_window_wider_than_sequence_is_no_window(oracle_mod, causal):
    q, k, v = rng_qkv(1, 16, 2, 4, seed=33)
    a = oracle_mod.attention_fwd(q, k, v, 0.5, causal)
    b = oracle_mod.attention_fwd(q, k, v, 0.5, causal, window=(16, 16))
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=0)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_window_uniform_scores_give_band_mean(oracle_mod, causal):
    """Q = 0: o_i is the mean of v over the visible band and lse_i is the log
    of the band's size."""
    N, wl, wr = 23, 4, 2
    q, k, v = rng_qkv(1, N, 2, 5, seed=34)
    q[:] = 0
    o, lse = oracle_mod.attention_fwd(q, k, v, 1.0, causal, window=(wl, wr))
    for i in range(N):
        lo, hi = max(0, i - wl), (i + 1 if causal else min(N, i + wr + 1))
        np.testing.assert_allclose(o[0, i], v[0, lo:hi].mean(axis=0), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[0, :, i], math.log(hi - lo), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_window_varlen_per_sequence(oracle_mod, causal):
    lens = [6, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    r = np.random.default_rng(35)
    q, k, v = (r.standard_normal((int(cu[-1]), 2, 4)) for _ in range(3))
    o, lse = oracle_mod.attention_fwd_varlen(q, k, v, cu, 0.5, causal, window=(2, 1))
    for s, L in enumerate(lens):
        a = int(cu[s])
        os_, ls = oracle_mod.attention_fwd(q[a:a + L][None], k[a:a + L][None],
                                           v[a:a + L][None], 0.5, causal, window=(2, 1))
        np.testing.assert_allclose(o[a:a + L], os_[0], rtol=0, atol=0)
        np.testing.assert_allclose(lse[:, a:a + L], ls[0], rtol=0, atol=0)
