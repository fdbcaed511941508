// flex_fwd.hip -- dispatch of the forward kernel over its built instances
// (input dtype, head dim, value head dim, q block, kv block); the instances
// themselves live in the fwd_*.hip units, the kernel in fwd_kernel.hpp.
#include "internal.hpp"

namespace flexattn {

typedef hipError_t (*FwdUnit)(const FwdParams&, int, int, int, hipStream_t);

#define FLEXATTN_DECLARE(NAME) hipError_t NAME(const FwdParams&, int, int, int, hipStream_t);
FLEXATTN_DECLARE(launch_fwd_bf16_d64_q64_k64)
FLEXATTN_DECLARE(launch_fwd_bf16_d64_q128_k64)
FLEXATTN_DECLARE(launch_fwd_bf16_d64_q128_k128)
FLEXATTN_DECLARE(launch_fwd_bf16_d128_q64_k64)
FLEXATTN_DECLARE(launch_fwd_bf16_d128_q128_k64)
FLEXATTN_DECLARE(launch_fwd_bf16_d128_q128_k128)
FLEXATTN_DECLARE(launch_fwd_bf16_d64v128_q64_k64)
FLEXATTN_DECLARE(launch_fwd_bf16_d64v128_q128_k64)
FLEXATTN_DECLARE(launch_fwd_bf16_d64v128_q128_k128)
FLEXATTN_DECLARE(launch_fwd_bf16_d128v64_q64_k64)
FLEXATTN_DECLARE(launch_fwd_bf16_d128v64_q128_k64)
FLEXATTN_DECLARE(launch_fwd_bf16_d128v64_q128_k128)
FLEXATTN_DECLARE(launch_fwd_fp32_d64_q64_k64)
FLEXATTN_DECLARE(launch_fwd_fp32_d64_q128_k64)
FLEXATTN_DECLARE(launch_fwd_fp32_d64_q128_k128)
FLEXATTN_DECLARE(launch_fwd_fp32_d128_q64_k64)
FLEXATTN_DECLARE(launch_fwd_fp32_d128_q128_k64)
FLEXATTN_DECLARE(launch_fwd_fp32_d128_q128_k128)
FLEXATTN_DECLARE(launch_fwd_fp32_d64v128_q64_k64)
FLEXATTN_DECLARE(launch_fwd_fp32_d64v128_q128_k64)
FLEXATTN_DECLARE(launch_fwd_fp32_d64v128_q128_k128)
FLEXATTN_DECLARE(launch_fwd_fp32_d128v64_q64_k64)
FLEXATTN_DECLARE(launch_fwd_fp32_d128v64_q128_k64)
FLEXATTN_DECLARE(launch_fwd_fp32_d128v64_q128_k128)
#undef FLEXATTN_DECLARE

namespace {

struct FwdInstance {
  int dtype, d, dv, qb, kb;
  FwdUnit fn;
};

const FwdInstance kFwdInstances[] = {
    {FLEX_DTYPE_BF16, 64, 64, 64, 64, launch_fwd_bf16_d64_q64_k64},
    {FLEX_DTYPE_BF16, 64, 64, 128, 64, launch_fwd_bf16_d64_q128_k64},
    {FLEX_DTYPE_BF16, 64, 64, 128, 128, launch_fwd_bf16_d64_q128_k128},
    {FLEX_DTYPE_BF16, 128, 128, 64, 64, launch_fwd_bf16_d128_q64_k64},
    {FLEX_DTYPE_BF16, 128, 128, 128, 64, launch_fwd_bf16_d128_q128_k64},
    {FLEX_DTYPE_BF16, 128, 128, 128, 128, launch_fwd_bf16_d128_q128_k128},
    {FLEX_DTYPE_BF16, 64, 128, 64, 64, launch_fwd_bf16_d64v128_q64_k64},
    {FLEX_DTYPE_BF16, 64, 128, 128, 64, launch_fwd_bf16_d64v128_q128_k64},
    {FLEX_DTYPE_BF16, 64, 128, 128, 128, launch_fwd_bf16_d64v128_q128_k128},
    {FLEX_DTYPE_BF16, 128, 64, 64, 64, launch_fwd_bf16_d128v64_q64_k64},
    {FLEX_DTYPE_BF16, 128, 64, 128, 64, launch_fwd_bf16_d128v64_q128_k64},
    {FLEX_DTYPE_BF16, 128, 64, 128, 128, launch_fwd_bf16_d128v64_q128_k128},
    {FLEX_DTYPE_FP32, 64, 64, 64, 64, launch_fwd_fp32_d64_q64_k64},
    {FLEX_DTYPE_FP32, 64, 64, 128, 64, launch_fwd_fp32_d64_q128_k64},
    {FLEX_DTYPE_FP32, 64, 64, 128, 128, launch_fwd_fp32_d64_q128_k128},
    {FLEX_DTYPE_FP32, 128, 128, 64, 64, launch_fwd_fp32_d128_q64_k64},
    {FLEX_DTYPE_FP32, 128, 128, 128, 64, launch_fwd_fp32_d128_q128_k64},
    {FLEX_DTYPE_FP32, 128, 128, 128, 128, launch_fwd_fp32_d128_q128_k128},
    {FLEX_DTYPE_FP32, 64, 128, 64, 64, launch_fwd_fp32_d64v128_q64_k64},
    {FLEX_DTYPE_FP32, 64, 128, 128, 64, launch_fwd_fp32_d64v128_q128_k64},
    {FLEX_DTYPE_FP32, 64, 128, 128, 128, launch_fwd_fp32_d64v128_q128_k128},
    {FLEX_DTYPE_FP32, 128, 64, 64, 64, launch_fwd_fp32_d128v64_q64_k64},
    {FLEX_DTYPE_FP32, 128, 64, 128, 64, launch_fwd_fp32_d128v64_q128_k64},
    {FLEX_DTYPE_FP32, 128, 64, 128, 128, launch_fwd_fp32_d128v64_q128_k128},
};

FwdUnit find_fwd(int in_dtype, int head_dim, int v_head_dim, int q_block, int kv_block) {
  for (const FwdInstance& f : kFwdInstances)
    if (f.dtype == in_dtype && f.d == head_dim && f.dv == v_head_dim && f.qb == q_block &&
        f.kb == kv_block)
      return f.fn;
  return nullptr;
}

}  // namespace

bool fwd_supported(int in_dtype, int head_dim, int v_head_dim, int q_block, int kv_block) {
  return find_fwd(in_dtype, head_dim, v_head_dim, q_block, kv_block) != nullptr;
}

hipError_t launch_fwd(const FwdParams& p, int in_dtype, int head_dim, int v_head_dim,
                      int q_block, int kv_block, int mask_kind, int score_kind, int variant,
                      hipStream_t stream) {
  const FwdUnit fn = find_fwd(in_dtype, head_dim, v_head_dim, q_block, kv_block);
  if (!fn) return hipErrorInvalidValue;
  return fn(p, mask_kind, score_kind, variant, stream);
}

}  // namespace flexattn
