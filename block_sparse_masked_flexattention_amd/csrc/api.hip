// api.hip -- the extern "C" entry points of libflexattn.so (declared in
// include/flexattn.h).  Host-side validation, then one kernel launch on the
// caller's stream.  Nothing here allocates, synchronises or keeps state.
#include <math.h>
#include <stdlib.h>

#include "internal.hpp"

using namespace flexattn;

namespace {

// FLEXATTN_DEBUG_LDS_POISON set to anything but "0": read on every call, so
// that a test can switch it per call.
int32_t lds_poison_requested() {
  const char* e = getenv("FLEXATTN_DEBUG_LDS_POISON");
  return e != nullptr && e[0] != '\0' && !(e[0] == '0' && e[1] == '\0') ? 1 : 0;
}

bool mask_ok(const flex_mask_desc& m, int32_t* err) {
  switch (m.kind) {
    case FLEX_MASK_NOOP:
    case FLEX_MASK_CAUSAL:
      return true;
    case FLEX_MASK_SLIDING_WINDOW:
      if (m.window_min < 0 || m.window < m.window_min) {
        *err = FLEX_E_INVALID_ARG;
        return false;
      }
      return true;
    case FLEX_MASK_PREFIX_CAUSAL:
      if (m.prefix < 0) {
        *err = FLEX_E_INVALID_ARG;
        return false;
      }
      return true;
    case FLEX_MASK_DOCUMENT:
    case FLEX_MASK_DOCUMENT_CAUSAL:
      return true;
    default:
      *err = FLEX_E_UNSUPPORTED;
      return false;
  }
}

int32_t ceil_div(int32_t a, int32_t b) { return (int32_t)(((int64_t)a + b - 1) / b); }

}  // namespace

extern "C" {

int32_t flex_attn_abi_version(void) { return FLEXATTN_ABI_VERSION; }

const char* flex_attn_strerror(int32_t code) {
  switch (code) {
    case FLEX_OK:
      return "success";
    case FLEX_E_INVALID_ARG:
      return "invalid argument";
    case FLEX_E_UNSUPPORTED:
      return "unsupported configuration (no kernel instance for it)";
    case FLEX_E_HIP:
      return "HIP launch error";
    case FLEX_E_SCRATCH_LIMIT:
      return "too large for flex_attn_bwd_noalloc's scratch (2 * B * H * q_len floats)";
    default:
      return "unknown status code";
  }
}

int32_t flex_attn_block_mask_dims(int32_t q_len, int32_t kv_len, int32_t q_block,
                                  int32_t kv_block, int32_t* n_q_blocks,
                                  int32_t* n_kv_blocks) {
  if (!n_q_blocks || !n_kv_blocks || q_len < 0 || kv_len < 0 || q_block <= 0 ||
      kv_block <= 0)
    return FLEX_E_INVALID_ARG;
  *n_q_blocks = ceil_div(q_len, q_block);
  *n_kv_blocks = ceil_div(kv_len, kv_block);
  return FLEX_OK;
}

int32_t flex_attn_build_block_mask(const flex_mask_desc* mask, int32_t q_len,
                                   int32_t kv_len, int32_t q_block,
                                   int32_t kv_block, int32_t* kv_num_blocks,
                                   int32_t* kv_indices,
                                   int32_t* full_kv_num_blocks,
                                   int32_t* full_kv_indices, int32_t* row_bounds,
                                   void* stream) {
  if (!mask) return FLEX_E_INVALID_ARG;
  if (q_len < 0 || kv_len < 0 || q_block <= 0 || kv_block <= 0 ||
      q_block > 1024 || kv_block > 1024)
    return FLEX_E_INVALID_ARG;
  int32_t err = FLEX_OK;
  if (!mask_ok(*mask, &err)) return err;
  const int32_t nq = ceil_div(q_len, q_block), nk = ceil_div(kv_len, kv_block);
  if ((int64_t)nq * nk > INT32_MAX) return FLEX_E_INVALID_ARG;
  if (nq > 0 && (!kv_num_blocks || !full_kv_num_blocks)) return FLEX_E_INVALID_ARG;
  if (nq > 0 && nk > 0 && (!kv_indices || !full_kv_indices)) return FLEX_E_INVALID_ARG;
  const bool doc = is_document_mask(mask->kind);
  if (doc && q_len > 0 && (!row_bounds || !mask->q_doc)) return FLEX_E_INVALID_ARG;
  if (doc && kv_len > 0 && !mask->kv_doc) return FLEX_E_INVALID_ARG;
  if (nq == 0) return FLEX_OK;

  MaskBuildParams p;
  p.kind = mask->kind;
  p.window = mask->window;
  p.window_min = mask->window_min;
  p.prefix = mask->prefix;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.q_block = q_block;
  p.kv_block = kv_block;
  p.n_qb = nq;
  p.n_kb = nk;
  p.kv_num = kv_num_blocks;
  p.kv_idx = kv_indices;
  p.fkv_num = full_kv_num_blocks;
  p.fkv_idx = full_kv_indices;
  p.q_doc = mask->q_doc;
  p.kv_doc = mask->kv_doc;
  p.bounds = doc ? row_bounds : nullptr;
  return launch_block_mask(p, static_cast<hipStream_t>(stream)) == hipSuccess
             ? FLEX_OK
             : FLEX_E_HIP;
}

int32_t flex_attn_build_block_mask_t(const flex_mask_desc* mask, int32_t q_len,
                                     int32_t kv_len, int32_t q_block,
                                     int32_t kv_block, int32_t* q_num_blocks,
                                     int32_t* q_indices,
                                     int32_t* full_q_num_blocks,
                                     int32_t* full_q_indices, int32_t* col_bounds,
                                     void* stream) {
  if (!mask) return FLEX_E_INVALID_ARG;
  if (q_len < 0 || kv_len < 0 || q_block <= 0 || kv_block <= 0 ||
      q_block > 1024 || kv_block > 1024)
    return FLEX_E_INVALID_ARG;
  int32_t err = FLEX_OK;
  if (!mask_ok(*mask, &err)) return err;
  const int32_t nq = ceil_div(q_len, q_block), nk = ceil_div(kv_len, kv_block);
  if ((int64_t)nq * nk > INT32_MAX) return FLEX_E_INVALID_ARG;
  if (nk > 0 && (!q_num_blocks || !full_q_num_blocks)) return FLEX_E_INVALID_ARG;
  if (nq > 0 && nk > 0 && (!q_indices || !full_q_indices)) return FLEX_E_INVALID_ARG;
  const bool doc = is_document_mask(mask->kind);
  if (doc && kv_len > 0 && (!col_bounds || !mask->kv_doc)) return FLEX_E_INVALID_ARG;
  if (doc && q_len > 0 && !mask->q_doc) return FLEX_E_INVALID_ARG;
  if (nk == 0) return FLEX_OK;

  MaskBuildParams p;
  p.kind = mask->kind;
  p.window = mask->window;
  p.window_min = mask->window_min;
  p.prefix = mask->prefix;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.q_block = q_block;
  p.kv_block = kv_block;
  p.n_qb = nq;
  p.n_kb = nk;
  p.kv_num = q_num_blocks;
  p.kv_idx = q_indices;
  p.fkv_num = full_q_num_blocks;
  p.fkv_idx = full_q_indices;
  p.q_doc = mask->q_doc;
  p.kv_doc = mask->kv_doc;
  p.bounds = doc ? col_bounds : nullptr;
  return launch_block_mask_t(p, static_cast<hipStream_t>(stream)) == hipSuccess
             ? FLEX_OK
             : FLEX_E_HIP;
}

int32_t flex_attn_fwd(const void* q, const void* k, const void* v,
                      int32_t in_dtype, int32_t B, int32_t H, int32_t q_len,
                      int32_t kv_len, int32_t head_dim, int32_t v_head_dim,
                      const flex_block_mask* bm, const flex_score_desc* score,
                      float scale, void* out, int32_t out_dtype, float* lse,
                      float* max_out, const flex_fwd_options* opt, void* stream) {
  if (!bm) return FLEX_E_INVALID_ARG;
  if (B < 0 || H < 0 || q_len < 0 || kv_len < 0 || head_dim <= 0 || v_head_dim <= 0)
    return FLEX_E_INVALID_ARG;
  if (in_dtype != FLEX_DTYPE_BF16 && in_dtype != FLEX_DTYPE_FP32) return FLEX_E_INVALID_ARG;
  if (out_dtype != FLEX_DTYPE_BF16 && out_dtype != FLEX_DTYPE_FP32) return FLEX_E_INVALID_ARG;
  if (!isfinite(scale) || scale == 0.0f) return FLEX_E_UNSUPPORTED;
  if (bm->q_len != q_len || bm->kv_len != kv_len) return FLEX_E_INVALID_ARG;
  if (bm->q_block <= 0 || bm->kv_block <= 0) return FLEX_E_INVALID_ARG;
  if (bm->n_q_blocks != ceil_div(q_len, bm->q_block) ||
      bm->n_kv_blocks != ceil_div(kv_len, bm->kv_block))
    return FLEX_E_INVALID_ARG;
  int32_t err = FLEX_OK;
  if (!mask_ok(bm->mask, &err)) return err;
  int32_t score_kind = FLEX_SCORE_IDENTITY;
  float bias_max = 0.f;
  const float* slopes = nullptr;
  if (score) {
    score_kind = score->kind;
    if (score_kind != FLEX_SCORE_IDENTITY && score_kind != FLEX_SCORE_REL_BIAS)
      return FLEX_E_UNSUPPORTED;
    if (score_kind == FLEX_SCORE_REL_BIAS) {
      if (score->num_heads != H) return FLEX_E_INVALID_ARG;
      if (score->slopes == nullptr && !isfinite(score->bias_max)) return FLEX_E_INVALID_ARG;
      if (score->slopes != nullptr && (reinterpret_cast<uintptr_t>(score->slopes) & 3) != 0)
        return FLEX_E_INVALID_ARG;
      bias_max = score->bias_max;
      slopes = score->slopes;
    }
  }
  if (!fwd_supported(in_dtype, head_dim, v_head_dim, bm->q_block, bm->kv_block))
    return FLEX_E_UNSUPPORTED;

  const int64_t rows = (int64_t)B * H * q_len;
  const int64_t nwg = (int64_t)B * H * bm->n_q_blocks;
  const int64_t krows = (int64_t)B * H * kv_len;
  if (nwg > INT32_MAX || rows * head_dim > ((int64_t)1 << 40) ||
      rows * v_head_dim > ((int64_t)1 << 40) || krows * head_dim > ((int64_t)1 << 40) ||
      krows * v_head_dim > ((int64_t)1 << 40))
    return FLEX_E_INVALID_ARG;
  if (rows == 0) return FLEX_OK;  // nothing to write
  if (!q || !out) return FLEX_E_INVALID_ARG;
  if (kv_len > 0 && (!k || !v)) return FLEX_E_INVALID_ARG;
  if (!bm->kv_num_blocks || !bm->full_kv_num_blocks) return FLEX_E_INVALID_ARG;
  if (bm->n_kv_blocks > 0 && (!bm->kv_indices || !bm->full_kv_indices))
    return FLEX_E_INVALID_ARG;
  const uintptr_t align = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out;
  if (align & 15u) return FLEX_E_INVALID_ARG;
  if (((uintptr_t)lse | (uintptr_t)max_out) & 3u) return FLEX_E_INVALID_ARG;
  if (is_document_mask(bm->mask.kind) && !bm->row_bounds) return FLEX_E_INVALID_ARG;
  const flex_fwd_options o = opt ? *opt : flex_fwd_options{0, 0, 0, 0};

  FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.max_out = max_out;
  p.kv_num = bm->kv_num_blocks;
  p.kv_idx = bm->kv_indices;
  p.fkv_num = bm->full_kv_num_blocks;
  p.fkv_idx = bm->full_kv_indices;
  p.B = B;
  p.H = H;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.n_qb = bm->n_q_blocks;
  p.n_kb = bm->n_kv_blocks;
  p.window = bm->mask.window;
  p.window_min = bm->mask.window_min;
  p.prefix = bm->mask.prefix;
  p.c1 = fabsf(scale) * 1.44269504088896340736f;
  p.neg_q = scale < 0.f ? 1 : 0;
  p.bias_max = bias_max;
  p.slopes = slopes;
  p.out_bf16 = out_dtype == FLEX_DTYPE_BF16 ? 1 : 0;
  // PRESCALE_QK: q carries scale * log2 e (sign included); scores come out
  // of the product in base-2 units
  p.prescale = o.prescale_qk != 0 ? 1 : 0;
  p.qscale = (float)((double)scale * 1.44269504088896340736);
  if (p.prescale) {
    if (!isfinite(p.qscale) || p.qscale == 0.0f) return FLEX_E_UNSUPPORTED;
    p.c1 = 1.0f;
    p.neg_q = 0;
  }
  p.safe_rows = o.rows_guaranteed_safe != 0 ? 1 : 0;
  p.contig = o.blocks_are_contiguous != 0 ? 1 : 0;
  p.lds_poison = lds_poison_requested();
  p.bounds = bm->row_bounds;
  const int variant = (o.use_subtiling != 0 ? kFwdSubtile : 0) | (max_out ? kFwdExactMax : 0);
  return launch_fwd(p, in_dtype, head_dim, v_head_dim, bm->q_block, bm->kv_block,
                    bm->mask.kind, score_kind, variant,
                    static_cast<hipStream_t>(stream)) == hipSuccess
             ? FLEX_OK
             : FLEX_E_HIP;
}


int32_t flex_attn_bwd_workspace_floats(int32_t B, int32_t H, int32_t q_len,
                                       int64_t* n_floats) {
  if (!n_floats || B < 0 || H < 0 || q_len < 0) return FLEX_E_INVALID_ARG;
  *n_floats = 2 * (int64_t)B * H * q_len;
  return FLEX_OK;
}

int32_t flex_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, const float* dlse,
                      int32_t in_dtype, int32_t B, int32_t H, int32_t q_len,
                      int32_t kv_len, int32_t head_dim, int32_t v_head_dim,
                      const flex_block_mask* bm, const flex_block_mask_t* bmt,
                      const flex_score_desc* score, float scale, void* dq, void* dk,
                      void* dv, int32_t grad_dtype, float* workspace, void* stream) {
  if (!bm || !bmt) return FLEX_E_INVALID_ARG;
  if (B < 0 || H < 0 || q_len < 0 || kv_len < 0 || head_dim <= 0 || v_head_dim <= 0)
    return FLEX_E_INVALID_ARG;
  if (in_dtype != FLEX_DTYPE_BF16 && in_dtype != FLEX_DTYPE_FP32) return FLEX_E_INVALID_ARG;
  if (grad_dtype != FLEX_DTYPE_BF16 && grad_dtype != FLEX_DTYPE_FP32) return FLEX_E_INVALID_ARG;
  if (!isfinite(scale) || scale == 0.0f) return FLEX_E_UNSUPPORTED;
  if (bm->q_len != q_len || bm->kv_len != kv_len) return FLEX_E_INVALID_ARG;
  if (bm->q_block <= 0 || bm->kv_block <= 0) return FLEX_E_INVALID_ARG;
  if (bm->n_q_blocks != ceil_div(q_len, bm->q_block) ||
      bm->n_kv_blocks != ceil_div(kv_len, bm->kv_block))
    return FLEX_E_INVALID_ARG;
  if (bmt->q_block != bm->q_block || bmt->kv_block != bm->kv_block ||
      bmt->n_q_blocks != bm->n_q_blocks || bmt->n_kv_blocks != bm->n_kv_blocks)
    return FLEX_E_INVALID_ARG;
  int32_t err = FLEX_OK;
  if (!mask_ok(bm->mask, &err)) return err;
  int32_t score_kind = FLEX_SCORE_IDENTITY;
  float bias_max = 0.f;
  const float* slopes = nullptr;
  if (score) {
    score_kind = score->kind;
    if (score_kind != FLEX_SCORE_IDENTITY && score_kind != FLEX_SCORE_REL_BIAS)
      return FLEX_E_UNSUPPORTED;
    if (score_kind == FLEX_SCORE_REL_BIAS) {
      if (score->num_heads != H) return FLEX_E_INVALID_ARG;
      if (score->slopes == nullptr && !isfinite(score->bias_max)) return FLEX_E_INVALID_ARG;
      if (score->slopes != nullptr && (reinterpret_cast<uintptr_t>(score->slopes) & 3) != 0)
        return FLEX_E_INVALID_ARG;
      bias_max = score->bias_max;
      slopes = score->slopes;
    }
  }
  if (!bwd_supported(in_dtype, head_dim, v_head_dim, bm->q_block, bm->kv_block))
    return FLEX_E_UNSUPPORTED;

  const int64_t rows = (int64_t)B * H * q_len;
  const int64_t krows = (int64_t)B * H * kv_len;
  if ((int64_t)B * H * bm->n_q_blocks > INT32_MAX || (int64_t)B * H * bm->n_kv_blocks > INT32_MAX ||
      rows * head_dim > ((int64_t)1 << 40) || krows * head_dim > ((int64_t)1 << 40) ||
      rows * v_head_dim > ((int64_t)1 << 40) || krows * v_head_dim > ((int64_t)1 << 40))
    return FLEX_E_INVALID_ARG;
  if (rows == 0 && krows == 0) return FLEX_OK;  // nothing to write
  // dq may be NULL: WRITE_DQ off (dq is not computed)
  if (rows > 0 && (!q || !out || !dout || !lse || !workspace)) return FLEX_E_INVALID_ARG;
  if (krows > 0 && (!k || !v || !dk || !dv)) return FLEX_E_INVALID_ARG;
  if (bm->n_q_blocks > 0 && (!bm->kv_num_blocks || !bm->full_kv_num_blocks))
    return FLEX_E_INVALID_ARG;
  if (bm->n_q_blocks > 0 && bm->n_kv_blocks > 0 && (!bm->kv_indices || !bm->full_kv_indices))
    return FLEX_E_INVALID_ARG;
  if (bmt->n_kv_blocks > 0 && (!bmt->q_num_blocks || !bmt->full_q_num_blocks))
    return FLEX_E_INVALID_ARG;
  if (bmt->n_q_blocks > 0 && bmt->n_kv_blocks > 0 && (!bmt->q_indices || !bmt->full_q_indices))
    return FLEX_E_INVALID_ARG;
  const uintptr_t align = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out |
                          (uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv;
  if ((align & 15u) || ((uintptr_t)workspace & 3u)) return FLEX_E_INVALID_ARG;
  if (is_document_mask(bm->mask.kind) &&
      ((rows > 0 && !bm->row_bounds) || (krows > 0 && !bmt->col_bounds)))
    return FLEX_E_INVALID_ARG;

  BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.dout = dout;
  p.lse = lse;
  p.dlse = dlse;
  p.ws = workspace;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.kv_num = bm->kv_num_blocks;
  p.kv_idx = bm->kv_indices;
  p.fkv_num = bm->full_kv_num_blocks;
  p.fkv_idx = bm->full_kv_indices;
  p.q_num = bmt->q_num_blocks;
  p.q_idx = bmt->q_indices;
  p.fq_num = bmt->full_q_num_blocks;
  p.fq_idx = bmt->full_q_indices;
  p.bounds = bm->row_bounds;
  p.col_bounds = bmt->col_bounds;
  p.B = B;
  p.H = H;
  p.q_len = q_len;
  p.kv_len = kv_len;
  p.n_qb = bm->n_q_blocks;
  p.n_kb = bm->n_kv_blocks;
  p.window = bm->mask.window;
  p.window_min = bm->mask.window_min;
  p.prefix = bm->mask.prefix;
  p.c1 = fabsf(scale) * 1.44269504088896340736f;
  p.scale = scale;
  p.inv_abs_scale = 1.0f / fabsf(scale);
  p.neg = scale < 0.f ? 1 : 0;
  p.bias_max = bias_max;
  p.slopes = slopes;
  p.grad_bf16 = grad_dtype == FLEX_DTYPE_BF16 ? 1 : 0;
  return launch_bwd(p, in_dtype, head_dim, v_head_dim, bm->q_block, bm->kv_block,
                    bm->mask.kind, score_kind, static_cast<hipStream_t>(stream)) == hipSuccess
             ? FLEX_OK
             : FLEX_E_HIP;
}

}  // extern "C"
