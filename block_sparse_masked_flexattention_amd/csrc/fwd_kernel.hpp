// fwd_kernel.hpp -- kernel entry points and per-instance dispatch of the
// forward pass.  The kernels themselves are in fwd_bf16.hpp (bf16 inputs)
// and fwd_fp32.hpp (fp32 inputs); each fwd_*.hip unit instantiates one
// (dtype, head dim, q block, kv block) combination over every mask kind,
// score kind and subtiling setting.
#pragma once
#include "fwd_bf16.hpp"
#include "fwd_fp32.hpp"

namespace flexattn {
namespace fwd {

// (the clang attribute rather than the __launch_bounds__ macro: template
// arguments carry commas)
template <int D, int QB, int KB, int MASK, int SCORE, bool SUB>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Bf16Fwd<D, QB, KB, MASK, SCORE, SUB>::NT),
                          amdgpu_waves_per_eu(Bf16Fwd<D, QB, KB, MASK, SCORE, SUB>::WAVES_PER_SIMD)))
void bf16_fwd_kernel(FwdParams p) {
  Bf16Fwd<D, QB, KB, MASK, SCORE, SUB>::run(p);
}

template <int D, int QB, int KB, int MASK, int SCORE>
__global__ __attribute__((amdgpu_flat_work_group_size(
    1, Fp32Fwd<D, QB, KB, MASK, SCORE>::NT))) void fp32_fwd_kernel(FwdParams p) {
  Fp32Fwd<D, QB, KB, MASK, SCORE>::run(p);
}

template <bool BF16, int D, int QB, int KB, int MASK, int SCORE, bool SUB>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  const long long nwg = (long long)p.B * p.H * p.n_qb;
  if (nwg == 0) return hipSuccess;
  if constexpr (BF16) {
    hipLaunchKernelGGL((bf16_fwd_kernel<D, QB, KB, MASK, SCORE, SUB>), dim3((unsigned)nwg),
                       dim3(Bf16Fwd<D, QB, KB, MASK, SCORE, SUB>::NT), 0, stream, p);
  } else {
    hipLaunchKernelGGL((fp32_fwd_kernel<D, QB, KB, MASK, SCORE>), dim3((unsigned)nwg),
                       dim3(Fp32Fwd<D, QB, KB, MASK, SCORE>::NT), 0, stream, p);
  }
  return hipGetLastError();
}

template <bool BF16, int D, int QB, int KB, int MASK, int SCORE>
hipError_t pick_sub(const FwdParams& p, bool sub, hipStream_t s) {
  // fp32 inputs: the subtiled order is the same arithmetic; one instance.
  if constexpr (BF16) {
    if (sub) return launch_one<true, D, QB, KB, MASK, SCORE, true>(p, s);
    return launch_one<true, D, QB, KB, MASK, SCORE, false>(p, s);
  } else {
    return launch_one<false, D, QB, KB, MASK, SCORE, false>(p, s);
  }
}

template <bool BF16, int D, int QB, int KB, int MASK>
hipError_t pick_score(const FwdParams& p, int score, bool sub, hipStream_t s) {
  if (score == FLEX_SCORE_REL_BIAS)
    return pick_sub<BF16, D, QB, KB, MASK, FLEX_SCORE_REL_BIAS>(p, sub, s);
  return pick_sub<BF16, D, QB, KB, MASK, FLEX_SCORE_IDENTITY>(p, sub, s);
}

template <bool BF16, int D, int QB, int KB>
hipError_t pick_mask(const FwdParams& p, int mask, int score, bool sub, hipStream_t s) {
  switch (mask) {
    case FLEX_MASK_NOOP:
      return pick_score<BF16, D, QB, KB, FLEX_MASK_NOOP>(p, score, sub, s);
    case FLEX_MASK_CAUSAL:
      return pick_score<BF16, D, QB, KB, FLEX_MASK_CAUSAL>(p, score, sub, s);
    case FLEX_MASK_SLIDING_WINDOW:
      return pick_score<BF16, D, QB, KB, FLEX_MASK_SLIDING_WINDOW>(p, score, sub, s);
    default:
      return pick_score<BF16, D, QB, KB, FLEX_MASK_PREFIX_CAUSAL>(p, score, sub, s);
  }
}

}  // namespace fwd
}  // namespace flexattn

// One translation unit per (dtype, head dim, q block, kv block) keeps the
// builds parallel.
#define FLEXATTN_FWD_UNIT(NAME, BF16, D, QB, KB)                               \
  namespace flexattn {                                                       \
  hipError_t NAME(const FwdParams& p, int mask, int score, bool sub,         \
                  hipStream_t s) {                                           \
    return fwd::pick_mask<BF16, D, QB, KB>(p, mask, score, sub, s);          \
  }                                                                          \
  }
