// internal.hpp -- shared between the C-ABI layer and the HIP kernels of
// libflexattn.so.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flexattn.h"

namespace flexattn {

// Everything the forward kernel reads, passed by value as the kernel argument.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;  // may be null
  const int32_t* kv_num;
  const int32_t* kv_idx;
  const int32_t* fkv_num;
  const int32_t* fkv_idx;
  int32_t B, H, q_len, kv_len, n_qb, n_kb;
  int32_t window, window_min, prefix;  // mask parameters
  float c1;        // |scale| * log2(e): scores are kept in base-2 units
  int32_t neg_q;   // scale < 0: q is negated on load so c1 stays positive
  float bias_max;  // REL_BIAS: slope_h = 2^(-bias_max * (h + 1) / H)
  int32_t out_bf16;
};

struct MaskBuildParams {
  int32_t kind, window, window_min, prefix;
  int32_t q_len, kv_len, q_block, kv_block, n_qb, n_kb;
  int32_t* kv_num;
  int32_t* kv_idx;
  int32_t* fkv_num;
  int32_t* fkv_idx;
};

hipError_t launch_block_mask(const MaskBuildParams& p, hipStream_t stream);

// fwd_supported() decides FLEX_E_UNSUPPORTED before launch_fwd() is called;
// launch_fwd() returns hipErrorInvalidValue for an instance it does not have.
bool fwd_supported(int in_dtype, int head_dim, int q_block, int kv_block);
hipError_t launch_fwd(const FwdParams& p, int in_dtype, int head_dim,
                      int q_block, int kv_block, int mask_kind, int score_kind,
                      bool subtile, hipStream_t stream);

}  // namespace flexattn
