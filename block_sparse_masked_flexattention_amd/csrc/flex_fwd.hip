// flex_fwd.hip -- dispatch of the forward kernel over its built instances
// (input dtype, head dim, q block, kv block); the instances themselves live
// in the fwd_*.hip units, the kernel in fwd_kernel.hpp.
#include "internal.hpp"

namespace flexattn {

hipError_t launch_fwd_bf16_d64_q64_k64(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_bf16_d64_q128_k64(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_bf16_d64_q128_k128(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_bf16_d128_q64_k64(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_bf16_d128_q128_k64(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_bf16_d128_q128_k128(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_fp32_d64_q64_k64(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_fp32_d64_q128_k64(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_fp32_d64_q128_k128(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_fp32_d128_q64_k64(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_fp32_d128_q128_k64(const FwdParams&, int, int, int, hipStream_t);
hipError_t launch_fwd_fp32_d128_q128_k128(const FwdParams&, int, int, int, hipStream_t);

bool fwd_supported(int in_dtype, int head_dim, int q_block, int kv_block) {
  if (in_dtype != FLEX_DTYPE_BF16 && in_dtype != FLEX_DTYPE_FP32) return false;
  if (head_dim != 64 && head_dim != 128) return false;
  return (q_block == 64 && kv_block == 64) || (q_block == 128 && kv_block == 64) ||
         (q_block == 128 && kv_block == 128);
}

hipError_t launch_fwd(const FwdParams& p, int in_dtype, int head_dim, int q_block,
                      int kv_block, int mask_kind, int score_kind, int variant,
                      hipStream_t stream) {
  if (in_dtype == FLEX_DTYPE_BF16 && head_dim == 64 && q_block == 64 && kv_block == 64)
    return launch_fwd_bf16_d64_q64_k64(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_BF16 && head_dim == 64 && q_block == 128 && kv_block == 64)
    return launch_fwd_bf16_d64_q128_k64(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_BF16 && head_dim == 64 && q_block == 128 && kv_block == 128)
    return launch_fwd_bf16_d64_q128_k128(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_BF16 && head_dim == 128 && q_block == 64 && kv_block == 64)
    return launch_fwd_bf16_d128_q64_k64(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_BF16 && head_dim == 128 && q_block == 128 && kv_block == 64)
    return launch_fwd_bf16_d128_q128_k64(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_BF16 && head_dim == 128 && q_block == 128 && kv_block == 128)
    return launch_fwd_bf16_d128_q128_k128(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_FP32 && head_dim == 64 && q_block == 64 && kv_block == 64)
    return launch_fwd_fp32_d64_q64_k64(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_FP32 && head_dim == 64 && q_block == 128 && kv_block == 64)
    return launch_fwd_fp32_d64_q128_k64(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_FP32 && head_dim == 64 && q_block == 128 && kv_block == 128)
    return launch_fwd_fp32_d64_q128_k128(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_FP32 && head_dim == 128 && q_block == 64 && kv_block == 64)
    return launch_fwd_fp32_d128_q64_k64(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_FP32 && head_dim == 128 && q_block == 128 && kv_block == 64)
    return launch_fwd_fp32_d128_q128_k64(p, mask_kind, score_kind, variant, stream);
  if (in_dtype == FLEX_DTYPE_FP32 && head_dim == 128 && q_block == 128 && kv_block == 128)
    return launch_fwd_fp32_d128_q128_k128(p, mask_kind, score_kind, variant, stream);
  return hipErrorInvalidValue;
}

}  // namespace flexattn
