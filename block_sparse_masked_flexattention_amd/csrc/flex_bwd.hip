// flex_bwd.hip -- dispatch of the backward over its built instances (head
// dim, q block, kv block); the instances live in the bwd_*.hip units, the
// kernels in bwd_bf16.hpp.
#include "internal.hpp"

namespace flexattn {

hipError_t launch_bwd_bf16_d64_q64_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d64_q128_k64(const BwdParams&, int, int, hipStream_t);
hipError_t launch_bwd_bf16_d64_q128_k128(const BwdParams&, int, int, hipStream_t);

bool bwd_supported(int in_dtype, int head_dim, int q_block, int kv_block) {
  if (in_dtype != FLEX_DTYPE_BF16 || head_dim != 64) return false;
  return (q_block == 64 && kv_block == 64) || (q_block == 128 && kv_block == 64) ||
         (q_block == 128 && kv_block == 128);
}

hipError_t launch_bwd(const BwdParams& p, int head_dim, int q_block, int kv_block,
                      int mask_kind, int score_kind, hipStream_t stream) {
  if (head_dim == 64 && q_block == 64 && kv_block == 64)
    return launch_bwd_bf16_d64_q64_k64(p, mask_kind, score_kind, stream);
  if (head_dim == 64 && q_block == 128 && kv_block == 64)
    return launch_bwd_bf16_d64_q128_k64(p, mask_kind, score_kind, stream);
  if (head_dim == 64 && q_block == 128 && kv_block == 128)
    return launch_bwd_bf16_d64_q128_k128(p, mask_kind, score_kind, stream);
  return hipErrorInvalidValue;
}

}  // namespace flexattn
