// flex_bwd.hip -- dispatch of the backward over its built instances (input
// dtype, head dim, value head dim, q block, kv block); the instances live in
// the bwd_*.hip units, the kernels in bwd_bf16.hpp (bf16 inputs, any pair of
// head dims 64 / 128) and bwd_fp32.hpp (fp32 inputs, likewise).
#include "internal.hpp"

namespace flexattn {

typedef hipError_t (*BwdUnit)(const BwdParams&, int, int, hipStream_t);

hipError_t launch_bwd_bf16_d64_q64_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d64_q128_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d64_q128_k128(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d128_q64_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d128_q128_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d128_q128_k128(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d64v128_q64_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d64v128_q128_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d64v128_q128_k128(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d128v64_q64_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d128v64_q128_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d128v64_q128_k128(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d64_q64_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d64_q128_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d64_q128_k128(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d128_q64_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d128_q128_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d128_q128_k128(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d64v128_q64_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d64v128_q128_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d64v128_q128_k128(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d128v64_q64_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d128v64_q128_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_fp32_d128v64_q128_k128(const BwdParams&, int, int, hipStream_t);

namespace {

struct BwdInstance {
  int dtype, d, dv, qb, kb;
  BwdUnit fn;
};

const BwdInstance kBwdInstances[] = {
    {FLEX_DTYPE_BF16, 64, 64, 64, 64, launch_bwd_bf16_d64_q64_k64},
    {FLEX_DTYPE_BF16, 64, 64, 128, 64, launch_bwd_bf16_d64_q128_k64},
    {FLEX_DTYPE_BF16, 64, 64, 128, 128, launch_bwd_bf16_d64_q128_k128},
    {FLEX_DTYPE_BF16, 128, 128, 64, 64, launch_bwd_bf16_d128_q64_k64},
    {FLEX_DTYPE_BF16, 128, 128, 128, 64, launch_bwd_bf16_d128_q128_k64},
    {FLEX_DTYPE_BF16, 128, 128, 128, 128, launch_bwd_bf16_d128_q128_k128},
    {FLEX_DTYPE_BF16, 64, 128, 64, 64, launch_bwd_bf16_d64v128_q64_k64},
    {FLEX_DTYPE_BF16, 64, 128, 128, 64, launch_bwd_bf16_d64v128_q128_k64},
    {FLEX_DTYPE_BF16, 64, 128, 128, 128, launch_bwd_bf16_d64v128_q128_k128},
    {FLEX_DTYPE_BF16, 128, 64, 64, 64, launch_bwd_bf16_d128v64_q64_k64},
    {FLEX_DTYPE_BF16, 128, 64, 128, 64, launch_bwd_bf16_d128v64_q128_k64},
    {FLEX_DTYPE_BF16, 128, 64, 128, 128, launch_bwd_bf16_d128v64_q128_k128},
    {FLEX_DTYPE_FP32, 64, 64, 64, 64, launch_bwd_fp32_d64_q64_k64},
    {FLEX_DTYPE_FP32, 64, 64, 128, 64, launch_bwd_fp32_d64_q128_k64},
    {FLEX_DTYPE_FP32, 64, 64, 128, 128, launch_bwd_fp32_d64_q128_k128},
    {FLEX_DTYPE_FP32, 128, 128, 64, 64, launch_bwd_fp32_d128_q64_k64},
    {FLEX_DTYPE_FP32, 128, 128, 128, 64, launch_bwd_fp32_d128_q128_k64},
    {FLEX_DTYPE_FP32, 128, 128, 128, 128, launch_bwd_fp32_d128_q128_k128},
    {FLEX_DTYPE_FP32, 64, 128, 64, 64, launch_bwd_fp32_d64v128_q64_k64},
    {FLEX_DTYPE_FP32, 64, 128, 128, 64, launch_bwd_fp32_d64v128_q128_k64},
    {FLEX_DTYPE_FP32, 64, 128, 128, 128, launch_bwd_fp32_d64v128_q128_k128},
    {FLEX_DTYPE_FP32, 128, 64, 64, 64, launch_bwd_fp32_d128v64_q64_k64},
    {FLEX_DTYPE_FP32, 128, 64, 128, 64, launch_bwd_fp32_d128v64_q128_k64},
    {FLEX_DTYPE_FP32, 128, 64, 128, 128, launch_bwd_fp32_d128v64_q128_k128},
};

BwdUnit find_bwd(int in_dtype, int head_dim, int v_head_dim, int q_block, int kv_block) {
  for (const BwdInstance& b : kBwdInstances)
    if (b.dtype == in_dtype && b.d == head_dim && b.dv == v_head_dim && b.qb == q_block &&
        b.kb == kv_block)
      return b.fn;
  return nullptr;
}

}  // namespace

bool bwd_supported(int in_dtype, int head_dim, int v_head_dim, int q_block, int kv_block) {
  return find_bwd(in_dtype, head_dim, v_head_dim, q_block, kv_block) != nullptr;
}

hipError_t launch_bwd(const BwdParams& p, int in_dtype, int head_dim, int v_head_dim,
                      int q_block, int kv_block, int mask_kind, int score_kind,
                      hipStream_t stream) {
  const BwdUnit fn = find_bwd(in_dtype, head_dim, v_head_dim, q_block, kv_block);
  if (!fn) return hipErrorInvalidValue;
  return fn(p, mask_kind, score_kind, stream);
}

}  // namespace flexattn
