/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU oracle for block-sparse masked FlexAttention forward.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  The product path (the HIP library) never calls it, and this
 * file shares no code, header or constant with that library.
 *
 * What it computes, and where each piece comes from:
 *
 *  - Element masks (mask_true).  "[Inductor][Flex Attention] Add Subtiling
 *    Option for Alpha Scaling" names the mask_mod hook and the sliding-window
 *    use case (Summary); "Performance for templated attention strangely bad
 *    for a combination of causal + upper square mask" spells out the
 *    prefix-bidirectional-or-causal predicate with an inclusive bound of 1024
 *    and masked scores set to -inf (the bad.py -> bad2.py diff).  Causal is
 *    the q >= kv half of that same predicate.  The sliding window is the
 *    causal predicate further limited to q - kv <= window; window_min is an
 *    extra lower bound on q - kv (0 for the plain causal window).
 *    The document kinds stand for a mask_mod that closes over a tensor (the
 *    op's mask_mod_other_buffers slot, which the subtiling page's test hunks
 *    show holding a captured tensor): a per-token document id for queries
 *    and keys, a query seeing exactly the keys of its own document, and with
 *    DOCUMENT_CAUSAL only those at or before its own position.
 *
 *  - Scores.  s = scale * <q_i, k_j> from the exact input values widened to
 *    fp64, then the score modification is applied to the scaled score.  The
 *    identity modification leaves it alone; the relative-position bias
 *    subtracts slope_h * (i - j), slope_h = 2^(-bias_max * (h + 1) / H), or
 *    slope_h = slopes[h] when the caller passes a per-head table (a
 *    score_mod closing over a tensor, the op's score_mod_other_buffers).
 *
 *  - Softmax.  The online-softmax recurrence of forward_block_mn (the
 *    common.py.jinja hunk: running max, alpha rescale of the accumulator and
 *    of the row sum l_i) has the ordinary softmax as its fixed point, so the
 *    oracle is that definition written out densely: over every visible key,
 *    w_j = exp(s_j - max), out = sum_j w_j v_j / sum_j w_j,
 *    lse = max + ln(sum_j w_j).  A row that sees no key returns out = 0 and
 *    lse = -inf (the guarded case ROWS_GUARANTEED_SAFE=False leaves on).
 *
 *  - Block arrays (oracle_block_mask).  Brute force: every element of every
 *    Q_BLOCK x KV_BLOCK tile is evaluated; positions beyond q_len / kv_len
 *    count as masked.  A tile with every element visible is "full", one with
 *    some is "partial", one with none is skipped.  Each row of kv_indices
 *    (resp. full_kv_indices) lists its partial (resp. full) kv-blocks in
 *    ascending order, followed by every remaining kv-block in ascending
 *    order, so each row is a permutation of 0..n_kv_blocks-1.  The field
 *    names come from the block-mask tuple of the flex_attention
 *    higher-order-op call in the test hunks of the subtiling page.
 *
 *  - Transposed block arrays (oracle_block_mask_t).  The same tile classes,
 *    listed per kv-block column: q_num_blocks / q_indices and
 *    full_q_num_blocks / full_q_indices, the second half of the block-mask
 *    tuple in those test hunks (the arrays the backward pass walks).
 *
 *  - Backward (oracle_attention_backward).  The flex_attention_backward call
 *    in the same test hunks takes q, k, v, the forward output and
 *    log-sum-exp, the output gradient and a log-sum-exp gradient, and returns
 *    the gradients of q, k and v.  The oracle is the derivative of the
 *    forward definition above, written out with the chain rule for every
 *    visible pair (i, j):
 *      p_ij = exp(s_ij - lse_i)                     (the softmax weight)
 *      delta_i = <dout_i, out_i> - dlse_i
 *      ds_ij = p_ij * (<dout_i, v_j> - delta_i)     (gradient of s_ij)
 *      dq_i += scale * ds_ij * k_j,  dk_j += scale * ds_ij * q_i,
 *      dv_j += p_ij * dout_i.
 *    out and lse are the oracle's own fp64 forward values.  The score
 *    modification adds a term independent of q and k, so it changes p but
 *    not the two products.  Masked pairs and rows that see no key contribute
 *    nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MASK_NOOP 0
#define ORACLE_MASK_CAUSAL 1
#define ORACLE_MASK_SLIDING_WINDOW 2
#define ORACLE_MASK_PREFIX_CAUSAL 3
#define ORACLE_MASK_DOCUMENT 4
#define ORACLE_MASK_DOCUMENT_CAUSAL 5

#define ORACLE_SCORE_IDENTITY 0
#define ORACLE_SCORE_REL_BIAS 1

/* Is key j visible from query i?  Positions out of range are never visible.
 * The document kinds read a per-token document id for every query (q_doc)
 * and every key (kv_doc): a query sees the keys of its own document (and,
 * for DOCUMENT_CAUSAL, only those at or before it). */
static int mask_true(int kind, int64_t window, int64_t window_min,
                     int64_t prefix,
                     const int32_t* q_doc, const int32_t* kv_doc, int64_t i, int64_t j, int64_t q_len,
                     int64_t kv_len) {
  if (i < 0 || j < 0 || i >= q_len || j >= kv_len) return 0;
  switch (kind) {
    case ORACLE_MASK_NOOP:
      return 1;
    case ORACLE_MASK_CAUSAL:
      return i >= j;
    case ORACLE_MASK_SLIDING_WINDOW:
      return (i - j >= window_min) && (i - j <= window);
    case ORACLE_MASK_PREFIX_CAUSAL:
      return ((i <= prefix) && (j <= prefix)) || (i >= j);
    case ORACLE_MASK_DOCUMENT:
      if (!q_doc || !kv_doc) return -1;
      return q_doc[i] == kv_doc[j];
    case ORACLE_MASK_DOCUMENT_CAUSAL:
      if (!q_doc || !kv_doc) return -1;
      return (q_doc[i] == kv_doc[j]) && (i >= j);
    default:
      return -1;
  }
}

int oracle_mask_value(int kind, int64_t window, int64_t window_min,
                      int64_t prefix, const int32_t* q_doc, const int32_t* kv_doc,
                      int64_t i, int64_t j, int64_t q_len, int64_t kv_len) {
  return mask_true(kind, window, window_min, prefix, q_doc, kv_doc, i, j, q_len, kv_len);
}

/* Number of visible (i, j) pairs over the whole q_len x kv_len square. */
int64_t oracle_count_visible(int kind, int64_t window, int64_t window_min,
                             int64_t prefix, const int32_t* q_doc, const int32_t* kv_doc,
                             int64_t q_len, int64_t kv_len) {
  if (kind >= 4 && (!q_doc || !kv_doc)) return -1;
  int64_t n = 0;
  for (int64_t i = 0; i < q_len; ++i)
    for (int64_t j = 0; j < kv_len; ++j)
      n += mask_true(kind, window, window_min, prefix, q_doc, kv_doc, i, j, q_len, kv_len) == 1;
  return n;
}

/* Brute-force block arrays.  Returns 0, or -1 on a bad argument. */
int oracle_block_mask(int kind, int64_t window, int64_t window_min,
                      int64_t prefix,
                      const int32_t* q_doc, const int32_t* kv_doc, int64_t q_len, int64_t kv_len,
                      int64_t q_block, int64_t kv_block, int32_t* kv_num_blocks,
                      int32_t* kv_indices, int32_t* full_kv_num_blocks,
                      int32_t* full_kv_indices) {
  if (kind < 0 || kind > 5 || (kind >= 4 && (!q_doc || !kv_doc)) || q_len < 0 || kv_len < 0 || q_block <= 0 ||
      kv_block <= 0)
    return -1;
  int64_t nq = (q_len + q_block - 1) / q_block;
  int64_t nk = (kv_len + kv_block - 1) / kv_block;
  /* tile class: 0 empty, 1 partial, 2 full */
  int* cls = (int*)malloc(sizeof(int) * (size_t)(nk > 0 ? nk : 1));
  if (!cls) return -1;
  for (int64_t qb = 0; qb < nq; ++qb) {
    for (int64_t kb = 0; kb < nk; ++kb) {
      int64_t count = 0;
      for (int64_t i = qb * q_block; i < (qb + 1) * q_block; ++i)
        for (int64_t j = kb * kv_block; j < (kb + 1) * kv_block; ++j)
          count += mask_true(kind, window, window_min, prefix, q_doc, kv_doc, i, j, q_len,
                             kv_len) == 1;
      cls[kb] = count == 0 ? 0 : (count == q_block * kv_block ? 2 : 1);
    }
    for (int want = 1; want <= 2; ++want) {
      int32_t* num = want == 1 ? kv_num_blocks : full_kv_num_blocks;
      int32_t* idx = (want == 1 ? kv_indices : full_kv_indices) + qb * nk;
      int64_t w = 0;
      for (int64_t kb = 0; kb < nk; ++kb)
        if (cls[kb] == want) idx[w++] = (int32_t)kb;
      num[qb] = (int32_t)w;
      for (int64_t kb = 0; kb < nk; ++kb)
        if (cls[kb] != want) idx[w++] = (int32_t)kb;
    }
  }
  free(cls);
  return 0;
}

/*
 * Attention for a list of query rows.  q is [B, H, q_len, d], k is
 * [B, H, kv_len, d], v is [B, H, kv_len, dv], all contiguous float32 holding
 * the exact input values.  rows[r] is the flat row id (b * H + h) * q_len + i.
 * Writes out[r * dv + c] and lse[r] in fp64, and, when row_max is not NULL,
 * row_max[r] = the largest visible score of the row (after the score
 * modification; -inf when the row sees no key), the third output of the
 * flex_attention op in the subtiling page's test hunks (OUTPUT_MAX).
 * slopes: NULL, or [H] per-head slopes replacing the formula (REL_BIAS).
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attention_rows(const float* q, const float* k, const float* v,
                          int64_t B, int64_t H, int64_t q_len, int64_t kv_len,
                          int64_t d, int64_t dv, int mask_kind, int64_t window,
                          int64_t window_min, int64_t prefix, const int32_t* q_doc, const int32_t* kv_doc, int score_kind,
                          double bias_max, const double* slopes, double scale,
                          const int64_t* rows,
                          int64_t n_rows, double* out, double* lse, double* row_max) {
  if (B < 0 || H <= 0 || q_len < 0 || kv_len < 0 || d <= 0 || dv <= 0)
    return -1;
  if (mask_kind < 0 || mask_kind > 5) return -1;
  if (mask_kind >= 4 && (!q_doc || !kv_doc)) return -1;
  if (score_kind != ORACLE_SCORE_IDENTITY && score_kind != ORACLE_SCORE_REL_BIAS)
    return -1;
  double* s = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)dv);
  if (!s || !acc) {
    free(s);
    free(acc);
    return -1;
  }
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t id = rows[r];
    if (id < 0 || id >= B * H * q_len) {
      free(s);
      free(acc);
      return -1;
    }
    int64_t bh = id / q_len, i = id % q_len, h = bh % H;
    const float* qi = q + id * d;
    const float* kb = k + bh * kv_len * d;
    const float* vb = v + bh * kv_len * dv;
    double slope = slopes ? slopes[h] : pow(2.0, -bias_max * (double)(h + 1) / (double)H);

    /* scores for every key; masked ones are -inf */
    double mx = -INFINITY;
    int any = 0;
    for (int64_t j = 0; j < kv_len; ++j) {
      if (mask_true(mask_kind, window, window_min, prefix, q_doc, kv_doc, i, j, q_len,
                    kv_len) != 1) {
        s[j] = -INFINITY;
        continue;
      }
      double dot = 0.0;
      for (int64_t c = 0; c < d; ++c)
        dot += (double)qi[c] * (double)kb[j * d + c];
      double sj = scale * dot;
      if (score_kind == ORACLE_SCORE_REL_BIAS) sj -= slope * (double)(i - j);
      s[j] = sj;
      if (sj > mx) mx = sj;
      any = 1;
    }

    double* o = out + r * dv;
    if (row_max) row_max[r] = any ? mx : -INFINITY;
    if (!any) {
      for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
      lse[r] = -INFINITY;
      continue;
    }
    double l = 0.0;
    for (int64_t c = 0; c < dv; ++c) acc[c] = 0.0;
    for (int64_t j = 0; j < kv_len; ++j) {
      if (s[j] == -INFINITY) continue;
      double w = exp(s[j] - mx);
      l += w;
      for (int64_t c = 0; c < dv; ++c) acc[c] += w * (double)vb[j * dv + c];
    }
    for (int64_t c = 0; c < dv; ++c) o[c] = acc[c] / l;
    lse[r] = mx + log(l);
  }
  free(s);
  free(acc);
  return 0;
}

/* Brute-force transposed block arrays: per kv-block column, the partial and
 * full q-blocks ascending, then every other q-block ascending.  Shapes
 * [nKVB] and [nKVB, nQB].  Returns 0, or -1 on a bad argument. */
int oracle_block_mask_t(int kind, int64_t window, int64_t window_min,
                        int64_t prefix,
                        const int32_t* q_doc, const int32_t* kv_doc, int64_t q_len, int64_t kv_len,
                        int64_t q_block, int64_t kv_block, int32_t* q_num_blocks,
                        int32_t* q_indices, int32_t* full_q_num_blocks,
                        int32_t* full_q_indices) {
  if (kind < 0 || kind > 5 || (kind >= 4 && (!q_doc || !kv_doc)) || q_len < 0 || kv_len < 0 || q_block <= 0 ||
      kv_block <= 0)
    return -1;
  int64_t nq = (q_len + q_block - 1) / q_block;
  int64_t nk = (kv_len + kv_block - 1) / kv_block;
  int* cls = (int*)malloc(sizeof(int) * (size_t)(nq > 0 ? nq : 1));
  if (!cls) return -1;
  for (int64_t kb = 0; kb < nk; ++kb) {
    for (int64_t qb = 0; qb < nq; ++qb) {
      int64_t count = 0;
      for (int64_t i = qb * q_block; i < (qb + 1) * q_block; ++i)
        for (int64_t j = kb * kv_block; j < (kb + 1) * kv_block; ++j)
          count += mask_true(kind, window, window_min, prefix, q_doc, kv_doc, i, j, q_len,
                             kv_len) == 1;
      cls[qb] = count == 0 ? 0 : (count == q_block * kv_block ? 2 : 1);
    }
    for (int want = 1; want <= 2; ++want) {
      int32_t* num = want == 1 ? q_num_blocks : full_q_num_blocks;
      int32_t* idx = (want == 1 ? q_indices : full_q_indices) + kb * nq;
      int64_t w = 0;
      for (int64_t qb = 0; qb < nq; ++qb)
        if (cls[qb] == want) idx[w++] = (int32_t)qb;
      num[kb] = (int32_t)w;
      for (int64_t qb = 0; qb < nq; ++qb)
        if (cls[qb] != want) idx[w++] = (int32_t)qb;
    }
  }
  free(cls);
  return 0;
}

/*
 * Backward for a list of heads.  q, dout are [B, H, q_len, d] / [.., dv],
 * k, v are [B, H, kv_len, d] / [.., dv], all float32 holding the exact
 * values; dlse is [B, H, q_len] or NULL (zero).  heads[t] is the flat head
 * id b * H + h.  Writes the fp64 gradients of the listed heads into
 * dq [B*H*q_len*d], dk [B*H*kv_len*d], dv [B*H*kv_len*dv] (the slabs of
 * other heads are left alone).  Returns 0, or -1 on a bad argument or
 * allocation failure.
 */
int oracle_attention_backward(const float* q, const float* k, const float* v,
                              const float* dout, const float* dlse, int64_t B,
                              int64_t H, int64_t q_len, int64_t kv_len,
                              int64_t d, int64_t dv, int mask_kind,
                              int64_t window, int64_t window_min, int64_t prefix, const int32_t* q_doc, const int32_t* kv_doc,
                              int score_kind, double bias_max, const double* slopes,
                              double scale, const int64_t* heads, int64_t n_heads, double* dq,
                              double* dk, double* dvg) {
  if (B < 0 || H <= 0 || q_len < 0 || kv_len < 0 || d <= 0 || dv <= 0)
    return -1;
  if (mask_kind < 0 || mask_kind > 5) return -1;
  if (mask_kind >= 4 && (!q_doc || !kv_doc)) return -1;
  if (score_kind != ORACLE_SCORE_IDENTITY && score_kind != ORACLE_SCORE_REL_BIAS)
    return -1;
  size_t nk = (size_t)(kv_len > 0 ? kv_len : 1);
  double* s = (double*)malloc(sizeof(double) * nk);
  double* o = (double*)malloc(sizeof(double) * (size_t)dv);
  if (!s || !o) {
    free(s);
    free(o);
    return -1;
  }
  for (int64_t t = 0; t < n_heads; ++t) {
    int64_t bh = heads[t];
    if (bh < 0 || bh >= B * H) {
      free(s);
      free(o);
      return -1;
    }
    int64_t h = bh % H;
    double slope = slopes ? slopes[h] : pow(2.0, -bias_max * (double)(h + 1) / (double)H);
    const float* qh = q + bh * q_len * d;
    const float* kh = k + bh * kv_len * d;
    const float* vh = v + bh * kv_len * dv;
    const float* doh = dout + bh * q_len * dv;
    double* dqh = dq + bh * q_len * d;
    double* dkh = dk + bh * kv_len * d;
    double* dvh = dvg + bh * kv_len * dv;
    for (int64_t x = 0; x < q_len * d; ++x) dqh[x] = 0.0;
    for (int64_t x = 0; x < kv_len * d; ++x) dkh[x] = 0.0;
    for (int64_t x = 0; x < kv_len * dv; ++x) dvh[x] = 0.0;
    for (int64_t i = 0; i < q_len; ++i) {
      /* forward for row i: scores, max, sum, output, lse */
      double mx = -INFINITY;
      int any = 0;
      for (int64_t j = 0; j < kv_len; ++j) {
        if (mask_true(mask_kind, window, window_min, prefix, q_doc, kv_doc, i, j, q_len,
                      kv_len) != 1) {
          s[j] = -INFINITY;
          continue;
        }
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
          dot += (double)qh[i * d + c] * (double)kh[j * d + c];
        double sj = scale * dot;
        if (score_kind == ORACLE_SCORE_REL_BIAS) sj -= slope * (double)(i - j);
        s[j] = sj;
        if (sj > mx) mx = sj;
        any = 1;
      }
      if (!any) continue;
      double l = 0.0;
      for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
      for (int64_t j = 0; j < kv_len; ++j) {
        if (s[j] == -INFINITY) continue;
        double w = exp(s[j] - mx);
        l += w;
        for (int64_t c = 0; c < dv; ++c) o[c] += w * (double)vh[j * dv + c];
      }
      for (int64_t c = 0; c < dv; ++c) o[c] /= l;
      double lse = mx + log(l);
      /* delta_i = <dout_i, out_i> - dlse_i */
      double delta = 0.0;
      for (int64_t c = 0; c < dv; ++c) delta += (double)doh[i * dv + c] * o[c];
      if (dlse) delta -= (double)dlse[bh * q_len + i];
      for (int64_t j = 0; j < kv_len; ++j) {
        if (s[j] == -INFINITY) continue;
        double p = exp(s[j] - lse);
        double dp = 0.0;
        for (int64_t c = 0; c < dv; ++c)
          dp += (double)doh[i * dv + c] * (double)vh[j * dv + c];
        double ds = p * (dp - delta);
        for (int64_t c = 0; c < d; ++c) {
          dqh[i * d + c] += scale * ds * (double)kh[j * d + c];
          dkh[j * d + c] += scale * ds * (double)qh[i * d + c];
        }
        for (int64_t c = 0; c < dv; ++c) dvh[j * dv + c] += p * (double)doh[i * dv + c];
      }
    }
  }
  free(s);
  free(o);
  return 0;
}
