"""Helpers for the GPU tests: device transfer, oracle comparisons, sampling."""
import sys

import numpy as np
import torch

import oracle

# Tolerances: max |GPU - oracle| on O and on LSE for bf16 N(0,1) inputs, and
# relative Frobenius error on the gradients.
O_ATOL = 1e-2
LSE_ATOL = 1e-3
GRAD_RELF = 2e-2


def o_excess(o, o_ref):
    """How far |o - o_ref| exceeds the O tolerance, elementwise max (<= 0 is a
    pass). The tolerance is O_ATOL absolute, widened where the reference's
    magnitude makes the bf16 rounding of the output alone (at most
    2^-8 |o|) approach it: tol = max(O_ATOL, 2^-8 |o_ref| + 1e-3)."""
    o, o_ref = np.asarray(o, np.float64), np.asarray(o_ref, np.float64)
    if o.size == 0:
        return -1.0
    tol = np.maximum(O_ATOL, 2.0 ** -8 * np.abs(o_ref) + 1e-3)
    return float(np.max(np.abs(o - o_ref) - tol))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(t):
    return t.to("cuda").contiguous()


def f64(t_bf16_cpu):
    """Exact fp64 copy of a bf16 CPU tensor (through its bit patterns)."""
    return oracle.bf16_bits_to_f64(t_bf16_cpu.contiguous().view(torch.int16).numpy())


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def relf(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def sample_rows(N, n, rng, tile=128):
    """Row indices covering the first/last rows, tile edges and random rows."""
    fixed = {0, 1, N - 1, N - 2}
    for t in range(0, N, tile):
        fixed.update({t, t + tile - 1})
    fixed = {i for i in fixed if 0 <= i < N}
    fixed = sorted(fixed)
    if len(fixed) > n // 2:
        fixed = list(rng.choice(fixed, n // 2, replace=False))
    extra = rng.choice(N, size=min(N, max(0, n - len(fixed))), replace=False)
    return np.unique(np.concatenate([np.array(fixed, int), extra])).astype(np.int64)


def oracle_rows_one_head(qb, kb, vb, b, h, rows, scale, causal):
    """Oracle O/LSE for rows of head (b, h) of bf16 CPU tensors [B,N,H,d],
    widening only that head to fp64."""
    q1 = f64(qb[b:b + 1, :, h:h + 1, :])
    k1 = f64(kb[b:b + 1, :, h:h + 1, :])
    v1 = f64(vb[b:b + 1, :, h:h + 1, :])
    sel = np.stack([np.zeros_like(rows), np.zeros_like(rows), rows], 1)
    return oracle.attention_fwd(q1, k1, v1, scale, causal, rows=sel)


def o_tolerance_bf16_p(q, k, v, o_ref, lse_ref, scale, keep):
    """Per-element O tolerance that also covers few-key rows.

    The kernels round each probability p_j to bf16 (p_j (1 + e_j), |e_j| <=
    2^-8) and normalise by the sum of the rounded values. To first order the
    output moves by sum_j w_ij e_j (v_j - o_i) (the shift of the normaliser
    multiplies sum_j w_ij (v_j - o_i) = 0), so
    |dO_i| <= 2^-8 sum_j w_ij |v_j - o_i|; the bf16 output adds 2^-8 |o_i|.
    With many keys the errors average out and the fixed bar of o_excess
    governs; with two or three keys this bound can exceed it. Returns
    max(fixed tolerance, 1e-3 + 2^-8 |o| + that bound). q, k, v: fp64 [B, N, H, d]; o_ref, lse_ref: the oracle's output;
    keep: boolean [N, N] visibility.
    """
    B, N, H, d = q.shape
    dev = np.zeros_like(o_ref)
    for b in range(B):
        for h in range(H):
            s = scale * q[b, :, h] @ k[b, :, h].T
            w = np.where(keep, np.exp(np.minimum(s - lse_ref[b, h][:, None], 0.0)), 0.0)
            for r0 in range(0, N, 64):
                r1 = min(N, r0 + 64)
                diff = np.abs(v[b, None, :, h] - o_ref[b, r0:r1, h][:, None, :])
                dev[b, r0:r1, h] = np.einsum("ij,ijc->ic", w[r0:r1], diff)
    derived = 1e-3 + 2.0 ** -8 * np.abs(o_ref) + 2.0 ** -8 * dev
    fixed = np.maximum(O_ATOL, 2.0 ** -8 * np.abs(o_ref) + 1e-3)
    return np.maximum(fixed, derived)
