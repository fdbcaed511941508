// internal.hpp -- shared between the C-ABI layer and the HIP kernels of
// libflexattn.so.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flexattn.h"

namespace flexattn {

// Document masks: the interval pair the builder writes for every row (and
// every key) when the ids are not non-decreasing.  Empty for the tile
// classification (first > last).
constexpr int kDocPoisonLo = 0x7fffffff;
constexpr int kDocPoisonHi = -0x7fffffff - 1;

// Everything the forward kernel reads, passed by value as the kernel argument.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;      // may be null
  float* max_out;  // may be null: the row max of the visible scores
  const int32_t* kv_num;
  const int32_t* kv_idx;
  const int32_t* fkv_num;
  const int32_t* fkv_idx;
  int32_t B, H, q_len, kv_len, n_qb, n_kb;
  int32_t window, window_min, prefix;  // mask parameters
  float c1;        // |scale| * log2(e): scores are kept in base-2 units
  int32_t neg_q;   // scale < 0: q is negated on load so c1 stays positive
  float bias_max;  // REL_BIAS: slope_h = 2^(-bias_max * (h + 1) / H)
  const float* slopes;  // REL_BIAS: slope_h = slopes[h] instead (may be null)
  int32_t out_bf16;
  // PRESCALE_QK: q is multiplied by qscale (= scale * log2 e) and rounded to
  // the input type on load; c1 is then 1 and neg_q 0
  int32_t prescale;
  float qscale;
  int32_t safe_rows;  // ROWS_GUARANTEED_SAFE: no fully masked-row guards
  int32_t contig;     // BLOCKS_ARE_CONTIGUOUS: list n is first + n
  const int32_t* bounds;  // document masks: [2 * q_len] visible key interval per row
  // debugging (FLEXATTN_DEBUG_LDS_POISON): the bf16 kernel fills each K/V
  // stage buffer with NaN before its next loads are issued
  int32_t lds_poison;
};

// Backward: gradients of q, k and v.  Both block masks are the forward's
// (kv-major, for dq) and its transpose (q-major, for dk and dv).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;   // the forward's output
  const void* dout;  // its gradient
  const float* lse;  // the forward's log-sum-exp (natural log)
  const float* dlse; // gradient of the log-sum-exp, may be null
  float* ws;         // [2 * B * H * q_len]: -delta per row, then a per row
  void* dq;
  void* dk;
  void* dv;
  const int32_t* kv_num;
  const int32_t* kv_idx;
  const int32_t* fkv_num;
  const int32_t* fkv_idx;
  const int32_t* q_num;
  const int32_t* q_idx;
  const int32_t* fq_num;
  const int32_t* fq_idx;
  const int32_t* bounds;      // document masks: [2 * q_len] key interval per query row
  const int32_t* col_bounds;  // document masks: [2 * kv_len] query interval per key
  int32_t B, H, q_len, kv_len, n_qb, n_kb;
  int32_t window, window_min, prefix;
  float c1;          // |scale| * log2(e)
  float scale;       // the signed scale (factor of dq and dk)
  float inv_abs_scale;
  int32_t neg;       // scale < 0: the sign goes onto q (dq kernel) or k (dk/dv kernel)
  float bias_max;
  const float* slopes;
  int32_t grad_bf16;
};

struct MaskBuildParams {
  int32_t kind, window, window_min, prefix;
  int32_t q_len, kv_len, q_block, kv_block, n_qb, n_kb;
  int32_t* kv_num;
  int32_t* kv_idx;
  int32_t* fkv_num;
  int32_t* fkv_idx;
  // document masks: the id arrays, and the interval array the builder
  // writes first (row bounds [2 * q_len] for the kv-major arrays, column
  // bounds [2 * kv_len] for the transposed ones) and then classifies from
  const int32_t* q_doc;
  const int32_t* kv_doc;
  int32_t* bounds;
};

// The forward and backward kernels have one instance for both document
// kinds: the intervals come from memory and the causal cut is already in
// them.
inline bool is_document_mask(int kind) {
  return kind == FLEX_MASK_DOCUMENT || kind == FLEX_MASK_DOCUMENT_CAUSAL;
}

hipError_t launch_block_mask(const MaskBuildParams& p, hipStream_t stream);
// The transposed arrays: kv_num / kv_idx / fkv_num / fkv_idx receive
// q_num_blocks [n_kb], q_indices [n_kb * n_qb], full_q_num_blocks,
// full_q_indices.
hipError_t launch_block_mask_t(const MaskBuildParams& p, hipStream_t stream);

// fwd_supported() decides FLEX_E_UNSUPPORTED before launch_fwd() is called;
// launch_fwd() returns hipErrorInvalidValue for an instance it does not have.
// Forward variant bits: subtiled alpha rescale, exact running max (taken
// when the row max is an output).
constexpr int kFwdSubtile = 1;
constexpr int kFwdExactMax = 2;
bool fwd_supported(int in_dtype, int head_dim, int v_head_dim, int q_block, int kv_block);
bool bwd_supported(int in_dtype, int head_dim, int v_head_dim, int q_block, int kv_block);
hipError_t launch_bwd(const BwdParams& p, int in_dtype, int head_dim, int v_head_dim,
                      int q_block, int kv_block, int mask_kind, int score_kind,
                      hipStream_t stream);
hipError_t launch_fwd(const FwdParams& p, int in_dtype, int head_dim, int v_head_dim,
                      int q_block, int kv_block, int mask_kind, int score_kind,
                      int variant, hipStream_t stream);

}  // namespace flexattn
