"""Pins of the oracle's paged KV-cache forward (decoding new queries against
cached keys and values: page "FlashAttention技术深度解析", causal attention
with KV-cache incremental decoding, paged KV cache) to things other than
itself: library softmax over keys gathered with numpy indexing, the last rows
of ordinary (square) attention, invariance to where the pages physically
live, closed forms, and the append-then-attend identity."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from test_oracle_pins import scipy_attention


def paged(rng, lens, H, d, page, spare=3):
    """Random paged caches holding sequences of the given lengths: pages are
    handed out in a shuffled order, with `spare` unused pages mixed in."""
    need = [(L + page - 1) // page for L in lens]
    max_pages = max(need + [1])
    num_pages = sum(need) + spare
    order = rng.permutation(num_pages)
    bt = np.full((len(lens), max_pages), -7, np.int64)
    k = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[k:k + n]
        k += n
    kc = rng.standard_normal((num_pages, page, H, d))
    vc = rng.standard_normal((num_pages, page, H, d))
    return kc, vc, bt


def gather(cache, bt, b, L, page):
    """Logical rows 0..L-1 of sequence b, by numpy fancy indexing."""
    j = np.arange(L)
    return cache[bt[b, j // page], j % page]


def visible(pos, L, causal, window):
    wl, wr = window
    j = np.arange(L)
    keep = np.ones(L, bool)
    if causal:
        keep &= j <= pos
    if wl >= 0:
        keep &= j >= pos - wl
    if wr >= 0:
        keep &= j <= pos + wr
    return keep


def library_kvcache(q, kc, vc, bt, lens, page, scale, causal, window):
    B, Nq, H, d = q.shape
    o = np.zeros((B, Nq, H, d))
    lse = np.full((B, H, Nq), -np.inf)
    for b, L in enumerate(lens):
        K, V = gather(kc, bt, b, L, page), gather(vc, bt, b, L, page)
        for i in range(Nq):
            keep = visible(L - Nq + i, L, causal, window)
            if not keep.any():
                continue
            for h in range(H):
                s = np.where(keep, scale * K[:, h] @ q[b, i, h], -np.inf)
                o[b, i, h] = softmax(s) @ V[:, h]
                lse[b, h, i] = logsumexp(s)
    return o, lse


CASES = [(False, (-1, -1)), (True, (-1, -1)), (True, (5, 0)), (False, (3, 2)),
         (False, (-1, 0)), (True, (0, 0))]


@pytest.mark.parametrize("causal,window", CASES)
@pytest.mark.parametrize("page", [1, 4, 16])
@pytest.mark.parametrize("Nq", [1, 3])
def test_kvcache_vs_library_softmax(oracle_mod, causal, window, page, Nq):
    rng = np.random.default_rng(50 + page + Nq)
    lens = [37, Nq, 64, 5 + Nq]
    H, d = 2, 8
    kc, vc, bt = paged(rng, lens, H, d, page)
    q = rng.standard_normal((len(lens), Nq, H, d))
    o, lse = oracle_mod.attention_fwd_kvcache(q, kc, vc, bt, lens, 0.4, causal, window)
    o2, lse2 = library_kvcache(q, kc, vc, bt, lens, page, 0.4, causal, window)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (True, (9, 0)), (False, (-1, -1)),
                                           (False, (4, 6))])
def test_last_rows_of_square_attention(oracle_mod, causal, window):
    """Decoding the last Nq positions of a sequence gives the last Nq rows of
    ordinary attention over the whole sequence (fixes the query alignment)."""
    rng = np.random.default_rng(60)
    L, H, d, page, Nq = 45, 2, 8, 8, 4
    kc, vc, bt = paged(rng, [L], H, d, page)
    K, V = gather(kc, bt, 0, L, page)[None], gather(vc, bt, 0, L, page)[None]
    Q = rng.standard_normal((1, L, H, d))
    o_sq, lse_sq = scipy_attention(Q, K, V, 0.35, causal, window)
    o, lse = oracle_mod.attention_fwd_kvcache(Q[:, L - Nq:], kc, vc, bt, [L], 0.35, causal,
                                              window)
    np.testing.assert_allclose(o, o_sq[:, L - Nq:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_sq[:, :, L - Nq:], rtol=0, atol=1e-12)


def test_physical_page_order_does_not_matter(oracle_mod):
    """The same logical sequences stored in other physical pages give the
    same bits."""
    rng = np.random.default_rng(70)
    lens, H, d, page = [30, 17], 2, 8, 4
    kc, vc, bt = paged(rng, lens, H, d, page, spare=0)
    q = rng.standard_normal((2, 2, H, d))
    o, lse = oracle_mod.attention_fwd_kvcache(q, kc, vc, bt, lens, 0.5, True)
    perm = rng.permutation(kc.shape[0])       # physical page p moves to perm[p]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], bt)
    o2, lse2 = oracle_mod.attention_fwd_kvcache(q, kc2, vc2, bt2, lens, 0.5, True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (False, (-1, -1)), (True, (6, 0))])
def test_zero_query_gives_mean_of_visible_values(oracle_mod, causal, window):
    rng = np.random.default_rng(80)
    lens, H, d, page, Nq = [20, 33], 2, 4, 8, 3
    kc, vc, bt = paged(rng, lens, H, d, page)
    q = np.zeros((2, Nq, H, d))
    o, lse = oracle_mod.attention_fwd_kvcache(q, kc, vc, bt, lens, 1.0, causal, window)
    for b, L in enumerate(lens):
        V = gather(vc, bt, b, L, page)
        for i in range(Nq):
            keep = visible(L - Nq + i, L, causal, window)
            np.testing.assert_allclose(o[b, i], V[keep].mean(axis=0), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[b, :, i], math.log(keep.sum()), rtol=0, atol=1e-13)


def test_queries_that_see_no_key(oracle_mod):
    """An empty cache (non-causal) and queries placed before the first key
    (causal, fewer keys than queries): o = 0 and lse = -inf."""
    rng = np.random.default_rng(90)
    H, d, page = 2, 4, 4
    kc, vc, bt = paged(rng, [0, 2], H, d, page, spare=2)
    q = rng.standard_normal((2, 3, H, d))
    o, lse = oracle_mod.attention_fwd_kvcache(q, kc, vc, bt, [0, 2], 0.5, True)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(o[1, 0] == 0) and np.all(np.isneginf(lse[1, :, 0]))  # position -1
    V = gather(vc, bt, 1, 2, page)
    np.testing.assert_allclose(o[1, 1], V[0], rtol=0, atol=1e-15)       # position 0: key 0
    o, lse = oracle_mod.attention_fwd_kvcache(q, kc, vc, bt, [0, 2], 0.5, False)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


def test_append_then_attend_is_attention_on_the_longer_sequence(oracle_mod):
    """kvcache_append writes the new rows where logical positions
    cache_seqlens[b] .. +n-1 live; attending afterwards equals the library
    softmax over the old keys followed by the new ones."""
    rng = np.random.default_rng(100)
    old, n, H, d, page = [9, 16, 0], 3, 2, 8, 4
    kc, vc, bt = paged(rng, [L + n for L in old], H, d, page)
    k_new = rng.standard_normal((3, n, H, d))
    v_new = rng.standard_normal((3, n, H, d))
    kc2, vc2 = oracle_mod.kvcache_append(kc, vc, k_new, v_new, bt, old)
    for b, L in enumerate(old):
        np.testing.assert_array_equal(gather(kc2, bt, b, L + n, page)[L:], k_new[b])
        np.testing.assert_array_equal(gather(vc2, bt, b, L + n, page)[:L],
                                      gather(vc, bt, b, L, page))
    q = rng.standard_normal((3, n, H, d))
    o, lse = oracle_mod.attention_fwd_kvcache(q, kc2, vc2, bt, [L + n for L in old], 0.3, True)
    for b, L in enumerate(old):
        K = np.concatenate([gather(kc, bt, b, L, page), k_new[b]])[None]
        V = np.concatenate([gather(vc, bt, b, L, page), v_new[b]])[None]
        Q = np.concatenate([np.zeros((L, H, d)), q[b]])[None]
        o_sq, lse_sq = scipy_attention(Q, K, V, 0.3, True)
        np.testing.assert_allclose(o[b], o_sq[0, L:], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], lse_sq[0, :, L:], rtol=0, atol=1e-12)


def test_rejects_bad_tables(oracle_mod):
    rng = np.random.default_rng(110)
    kc, vc, bt = paged(rng, [8], 1, 4, 4, spare=0)
    q = rng.standard_normal((1, 1, 1, 4))
    with pytest.raises(RuntimeError):
        oracle_mod.attention_fwd_kvcache(q, kc, vc, bt, [9], 0.5, True)   # beyond the table
    bad = bt.copy()
    bad[0, 1] = kc.shape[0]
    with pytest.raises(RuntimeError):
        oracle_mod.attention_fwd_kvcache(q, kc, vc, bad, [8], 0.5, True)  # no such page
