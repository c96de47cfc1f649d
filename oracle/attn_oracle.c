/*
 * Plain fp64 CPU attention: the checker for the GPU library, and nothing else.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this file's library. It shares no code, header, table
 * or helper with the HIP library, and includes only libc, libm and OpenMP.
 *
 * What it computes is the plain definition of attention from the page
 * "FlashAttention-2" (section comparing it with standard attention, the
 * standard_attention listing): for one (batch, head) slice,
 *     s_ij = scale * <q_i, k_j>,
 *     P_i. = softmax over the keys j that row i may see,
 *     o_i  = sum_j P_ij v_j.
 * Row i may see every key (non-causal) or keys j <= i (causal=True, the
 * autoregressive mask that the pages enable with causal=True; queries and
 * keys have the same length here, so the mask is j <= i). A sliding window
 * (the local-attention variant the page "FlashAttention技术深度解析" lists
 * among its attention variants) further limits row i to keys
 * i - wl <= j <= i + wr; wl or wr = -1 leaves that side unbounded.
 *
 * Each score row is materialised in full and reduced in two passes (max, then
 * sum of exponentials). This is deliberately not the tiled online recurrence:
 * the pages state that the tiled method reaches this same result exactly.
 *
 * lse_i is the natural log of sum_j exp(s_ij), in the units of the scaled
 * scores; the pages do not define it, this is the plain reading.
 *
 * Backward (the pages only say the gradients are obtained by recomputation;
 * the formulas below are the calculus of the definition above, with
 * L a scalar loss and dO = dL/dO):
 *     P_ij  = exp(s_ij - lse_i)
 *     dP_ij = <dO_i, v_j>
 *     D_i   = sum_j P_ij dP_ij
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dq_i  = scale * sum_j dS_ij k_j
 *     dk_j  = scale * sum_i dS_ij q_i
 *     dv_j  = sum_i P_ij dO_i
 * dk_j and dv_j are computed as the sums over i that define them (one key at
 * a time), after the per-row lse_i and D_i are known.
 *
 * Decoding against a key/value cache (page "FlashAttention技术深度解析":
 * causal attention with incremental decoding over a KV cache, and the paged
 * KV cache among its inference optimisations): sequence b holds L_b keys and
 * values in fixed-size pages; logical key j lives in page
 * block_table[b][j / page], slot j % page. Its Nq newest queries are the
 * last Nq positions of the sequence: query i sits at position
 * L_b - Nq + i, and the visibility rules above (causal, window) apply to
 * that position. A query that sees no key (possible only when L_b < Nq or
 * L_b = 0) has o = 0 and lse = -inf.
 *
 * Layout: q, k, v, dout are [B][N][H][d] fp64, contiguous. Row selections are
 * lists of (b, h, i) triples (int64). The cache is [num_pages][page][H][d];
 * the block table is [B][max_pages] int64. Every function returns 0 on
 * success and a negative value on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

#define IDX(b, i, h, N, H, d) ((((int64_t)(b) * (N) + (i)) * (H) + (h)) * (d))

/* Keys row i may see: [*lo, *hi). */
static void key_range(int64_t i, int64_t N, int causal, int64_t wl, int64_t wr, int64_t *lo,
                      int64_t *hi) {
  int64_t l = 0, h = causal ? i + 1 : N;
  if (wl >= 0 && i - wl > l) l = i - wl;
  if (wr >= 0 && i + wr + 1 < h) h = i + wr + 1;
  *lo = l;
  *hi = h;
}

/* Rows that see key j: [*lo, *hi). */
static void row_range(int64_t j, int64_t N, int causal, int64_t wl, int64_t wr, int64_t *lo,
                      int64_t *hi) {
  int64_t l = causal ? j : 0, h = N;
  if (wr >= 0 && j - wr > l) l = j - wr;
  if (wl >= 0 && j + wl + 1 < h) h = j + wl + 1;
  *lo = l;
  *hi = h;
}

static double dot(const double *a, const double *b, int64_t d) {
  double s = 0.0;
  for (int64_t c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

/* Score row s[j - lo] = scale <q_i, k_j> for the visible keys lo <= j < hi,
 * then max and log-sum-exp in two passes. */
static void score_row(const double *q, const double *k, int64_t b, int64_t h, int64_t i,
                      int64_t N, int64_t H, int64_t d, double scale, int64_t lo, int64_t hi,
                      double *s, double *lse_out) {
  const double *qi = q + IDX(b, i, h, N, H, d);
  double m = -INFINITY;
  for (int64_t j = lo; j < hi; ++j) {
    s[j - lo] = scale * dot(qi, k + IDX(b, j, h, N, H, d), d);
    if (s[j - lo] > m) m = s[j - lo];
  }
  double l = 0.0;
  for (int64_t j = lo; j < hi; ++j) l += exp(s[j - lo] - m);
  *lse_out = m + log(l);
}

static int check_dims(int64_t B, int64_t N, int64_t H, int64_t d, int64_t wl, int64_t wr) {
  return (B >= 0 && N >= 0 && H >= 0 && d >= 1 && wl >= -1 && wr >= -1) ? 0 : -1;
}

static int check_sel(const int64_t *sel, int64_t n, int64_t B, int64_t N, int64_t H) {
  for (int64_t r = 0; r < n; ++r) {
    const int64_t b = sel[3 * r], h = sel[3 * r + 1], i = sel[3 * r + 2];
    if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N) return -2;
  }
  return 0;
}

/* Forward for the selected rows: o_sel is [nsel][d], lse_sel is [nsel]. */
int oracle_fwd_rows(const double *q, const double *k, const double *v, int64_t B, int64_t N,
                    int64_t H, int64_t d, double scale, int causal, int64_t wl, int64_t wr,
                    const int64_t *sel, int64_t nsel, double *o_sel, double *lse_sel,
                    int nthreads) {
  if (check_dims(B, N, H, d, wl, wr)) return -1;
  if (check_sel(sel, nsel, B, N, H)) return -2;
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!s) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nsel; ++r) {
      if (!s) continue;
      const int64_t b = sel[3 * r], h = sel[3 * r + 1], i = sel[3 * r + 2];
      double lse;
      int64_t lo, hi;
      key_range(i, N, causal, wl, wr, &lo, &hi);
      score_row(q, k, b, h, i, N, H, d, scale, lo, hi, s, &lse);
      double *o = o_sel + r * d;
      for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
      for (int64_t j = lo; j < hi; ++j) {
        const double p = exp(s[j - lo] - lse);
        const double *vj = v + IDX(b, j, h, N, H, d);
        for (int64_t c = 0; c < d; ++c) o[c] += p * vj[c];
      }
      lse_sel[r] = lse;
    }
    free(s);
  }
  return bad ? -3 : 0;
}

/* Backward, per-row part for the selected rows: lse_i, D_i and dq_i. */
int oracle_bwd_rows(const double *q, const double *k, const double *v, const double *dout,
                    int64_t B, int64_t N, int64_t H, int64_t d, double scale, int causal,
                    int64_t wl, int64_t wr, const int64_t *sel, int64_t nsel, double *dq_sel,
                    double *lse_sel, double *D_sel, int nthreads) {
  if (check_dims(B, N, H, d, wl, wr)) return -1;
  if (check_sel(sel, nsel, B, N, H)) return -2;
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double *s = (double *)malloc(sizeof(double) * 2 * (size_t)(N > 0 ? N : 1));
    if (!s) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nsel; ++r) {
      if (!s) continue;
      double *dp = s + N;
      const int64_t b = sel[3 * r], h = sel[3 * r + 1], i = sel[3 * r + 2];
      double lse;
      int64_t lo, hi;
      key_range(i, N, causal, wl, wr, &lo, &hi);
      score_row(q, k, b, h, i, N, H, d, scale, lo, hi, s, &lse);
      const double *doi = dout + IDX(b, i, h, N, H, d);
      double D = 0.0;
      for (int64_t j = lo; j < hi; ++j) {
        s[j - lo] = exp(s[j - lo] - lse); /* s now holds P_ij */
        dp[j - lo] = dot(doi, v + IDX(b, j, h, N, H, d), d);
        D += s[j - lo] * dp[j - lo];
      }
      double *dq = dq_sel + r * d;
      for (int64_t c = 0; c < d; ++c) dq[c] = 0.0;
      for (int64_t j = lo; j < hi; ++j) {
        const double ds = s[j - lo] * (dp[j - lo] - D);
        const double *kj = k + IDX(b, j, h, N, H, d);
        for (int64_t c = 0; c < d; ++c) dq[c] += scale * ds * kj[c];
      }
      lse_sel[r] = lse;
      D_sel[r] = D;
    }
    free(s);
  }
  return bad ? -3 : 0;
}

/* Backward, per-key part for the selected keys (b, h, j): dk_j and dv_j.
 * lse_all and D_all are [B][H][N] and must hold the per-row values of every
 * row of each selected head (from oracle_bwd_rows). */
int oracle_bwd_cols(const double *q, const double *k, const double *v, const double *dout,
                    int64_t B, int64_t N, int64_t H, int64_t d, double scale, int causal,
                    int64_t wl, int64_t wr, const double *lse_all, const double *D_all,
                    const int64_t *sel, int64_t nsel, double *dk_sel, double *dv_sel,
                    int nthreads) {
  if (check_dims(B, N, H, d, wl, wr)) return -1;
  if (check_sel(sel, nsel, B, N, H)) return -2;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads > 0 ? nthreads : 1)
  for (int64_t r = 0; r < nsel; ++r) {
    const int64_t b = sel[3 * r], h = sel[3 * r + 1], j = sel[3 * r + 2];
    const double *kj = k + IDX(b, j, h, N, H, d);
    const double *vj = v + IDX(b, j, h, N, H, d);
    const double *lse = lse_all + (b * H + h) * N;
    const double *Dr = D_all + (b * H + h) * N;
    double *dk = dk_sel + r * d, *dv = dv_sel + r * d;
    for (int64_t c = 0; c < d; ++c) dk[c] = dv[c] = 0.0;
    /* rows i that see key j */
    int64_t lo, hi;
    row_range(j, N, causal, wl, wr, &lo, &hi);
    for (int64_t i = lo; i < hi; ++i) {
      const double *qi = q + IDX(b, i, h, N, H, d);
      const double *doi = dout + IDX(b, i, h, N, H, d);
      const double p = exp(scale * dot(qi, kj, d) - lse[i]);
      const double ds = p * (dot(doi, vj, d) - Dr[i]);
      for (int64_t c = 0; c < d; ++c) {
        dv[c] += p * doi[c];
        dk[c] += scale * ds * qi[c];
      }
    }
  }
  return 0;
}

/* Row of the [num_pages * page] cache rows that holds logical key j of
 * sequence b. */
static int64_t cache_row(const int64_t *block_table, int64_t max_pages, int64_t page, int64_t b,
                         int64_t j) {
  return block_table[b * max_pages + j / page] * page + j % page;
}

/* Forward of Nq new queries per sequence against a paged key/value cache.
 * q: [B][Nq][H][d]; kc, vc: [num_pages][page][H][d]; block_table:
 * [B][max_pages]; seqlens: [B] keys held per sequence. o: [B][Nq][H][d],
 * lse: [B][H][Nq]. */
int oracle_fwd_cache(const double *q, const double *kc, const double *vc,
                     const int64_t *block_table, const int64_t *seqlens, int64_t B, int64_t Nq,
                     int64_t H, int64_t d, int64_t page, int64_t max_pages, int64_t num_pages,
                     double scale, int causal, int64_t wl, int64_t wr, double *o, double *lse,
                     int nthreads) {
  if (check_dims(B, Nq, H, d, wl, wr) || page < 1 || max_pages < 0 || num_pages < 0) return -1;
  for (int64_t b = 0; b < B; ++b) {
    if (seqlens[b] < 0 || seqlens[b] > page * max_pages) return -2;
    for (int64_t t = 0; t < (seqlens[b] + page - 1) / page; ++t)
      if (block_table[b * max_pages + t] < 0 || block_table[b * max_pages + t] >= num_pages)
        return -2;
  }
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    int64_t lmax = 1;
    for (int64_t b = 0; b < B; ++b)
      if (seqlens[b] > lmax) lmax = seqlens[b];
    double *s = (double *)malloc(sizeof(double) * (size_t)lmax);
    if (!s) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for collapse(3) schedule(dynamic, 4)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t i = 0; i < Nq; ++i)
        for (int64_t h = 0; h < H; ++h) {
          if (!s) continue;
          const int64_t L = seqlens[b];
          const int64_t pos = L - Nq + i; /* position of query i in its sequence */
          const double *qi = q + IDX(b, i, h, Nq, H, d);
          int64_t lo = 0, hi = 0;
          if (pos >= 0) {
            key_range(pos, L, causal, wl, wr, &lo, &hi);
          } else if (!causal) {
            /* a query before the sequence's first key: only a window can
               limit it */
            lo = 0;
            hi = L;
            if (wr >= 0 && pos + wr + 1 < hi) hi = pos + wr + 1 > 0 ? pos + wr + 1 : 0;
          }
          double m = -INFINITY;
          for (int64_t j = lo; j < hi; ++j) {
            const int64_t row = cache_row(block_table, max_pages, page, b, j);
            s[j - lo] = scale * dot(qi, kc + (row * H + h) * d, d);
            if (s[j - lo] > m) m = s[j - lo];
          }
          double l = 0.0;
          for (int64_t j = lo; j < hi; ++j) l += exp(s[j - lo] - m);
          double *oi = o + IDX(b, i, h, Nq, H, d);
          for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
          const double ls = (hi > lo) ? m + log(l) : -INFINITY;
          for (int64_t j = lo; j < hi; ++j) {
            const int64_t row = cache_row(block_table, max_pages, page, b, j);
            const double p = exp(s[j - lo] - ls);
            const double *vj = vc + (row * H + h) * d;
            for (int64_t c = 0; c < d; ++c) oi[c] += p * vj[c];
          }
          lse[(b * H + h) * Nq + i] = ls;
        }
    free(s);
  }
  return bad ? -3 : 0;
}

int oracle_max_threads(void) { return omp_get_max_threads(); }
