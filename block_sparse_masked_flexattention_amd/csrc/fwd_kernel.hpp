// fwd_kernel.hpp -- kernel entry points and per-instance dispatch of the
// forward pass.  The kernels themselves are in fwd_bf16.hpp (bf16 inputs)
// and fwd_fp32.hpp (fp32 inputs); each fwd_*.hip unit instantiates one
// (dtype, head dim, q block, kv block) combination over every mask kind,
// score kind and variant (subtiled rescale, exact running max).
#pragma once
#include "fwd_bf16.hpp"
#include "fwd_fp32.hpp"

namespace flexattn {
namespace fwd {

// (the clang attribute rather than the __launch_bounds__ macro: template
// arguments carry commas)
template <int D, int DV, int QB, int KB, int MASK, int SCORE, bool SUB, bool XMAX>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Bf16Fwd<D, DV, QB, KB, MASK, SCORE, SUB, XMAX>::NT),
                          amdgpu_waves_per_eu(Bf16Fwd<D, DV, QB, KB, MASK, SCORE, SUB, XMAX>::WAVES_PER_SIMD)))
void bf16_fwd_kernel(FwdParams p) {
  Bf16Fwd<D, DV, QB, KB, MASK, SCORE, SUB, XMAX>::run(p);
}

template <int D, int DV, int QB, int KB, int MASK, int SCORE>
__global__ __attribute__((amdgpu_flat_work_group_size(
    1, Fp32Fwd<D, DV, QB, KB, MASK, SCORE>::NT))) void fp32_fwd_kernel(FwdParams p) {
  Fp32Fwd<D, DV, QB, KB, MASK, SCORE>::run(p);
}

template <bool BF16, int D, int DV, int QB, int KB, int MASK, int SCORE, bool SUB, bool XMAX>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  const long long nwg = (long long)p.B * p.H * p.n_qb;
  if (nwg == 0) return hipSuccess;
  if constexpr (BF16) {
    hipLaunchKernelGGL((bf16_fwd_kernel<D, DV, QB, KB, MASK, SCORE, SUB, XMAX>), dim3((unsigned)nwg),
                       dim3(Bf16Fwd<D, DV, QB, KB, MASK, SCORE, SUB, XMAX>::NT), 0, stream, p);
  } else {
    hipLaunchKernelGGL((fp32_fwd_kernel<D, DV, QB, KB, MASK, SCORE>), dim3((unsigned)nwg),
                       dim3(Fp32Fwd<D, DV, QB, KB, MASK, SCORE>::NT), 0, stream, p);
  }
  return hipGetLastError();
}

template <bool BF16, int D, int DV, int QB, int KB, int MASK, int SCORE>
hipError_t pick_variant(const FwdParams& p, int var, hipStream_t s) {
  // fp32 inputs: the running max is always exact and the subtiled order is
  // the same arithmetic; one instance.
  if constexpr (BF16) {
    const bool sub = (var & kFwdSubtile) != 0, xmax = (var & kFwdExactMax) != 0;
    if (xmax) {
      if (sub) return launch_one<true, D, DV, QB, KB, MASK, SCORE, true, true>(p, s);
      return launch_one<true, D, DV, QB, KB, MASK, SCORE, false, true>(p, s);
    }
    if (sub) return launch_one<true, D, DV, QB, KB, MASK, SCORE, true, false>(p, s);
    return launch_one<true, D, DV, QB, KB, MASK, SCORE, false, false>(p, s);
  } else {
    return launch_one<false, D, DV, QB, KB, MASK, SCORE, false, false>(p, s);
  }
}

template <bool BF16, int D, int DV, int QB, int KB, int MASK>
hipError_t pick_score(const FwdParams& p, int score, int var, hipStream_t s) {
  if (score == FLEX_SCORE_REL_BIAS)
    return pick_variant<BF16, D, DV, QB, KB, MASK, FLEX_SCORE_REL_BIAS>(p, var, s);
  return pick_variant<BF16, D, DV, QB, KB, MASK, FLEX_SCORE_IDENTITY>(p, var, s);
}

template <bool BF16, int D, int DV, int QB, int KB>
hipError_t pick_mask(const FwdParams& p, int mask, int score, int var, hipStream_t s) {
  switch (mask) {
    case FLEX_MASK_NOOP:
      return pick_score<BF16, D, DV, QB, KB, FLEX_MASK_NOOP>(p, score, var, s);
    case FLEX_MASK_CAUSAL:
      return pick_score<BF16, D, DV, QB, KB, FLEX_MASK_CAUSAL>(p, score, var, s);
    case FLEX_MASK_SLIDING_WINDOW:
      return pick_score<BF16, D, DV, QB, KB, FLEX_MASK_SLIDING_WINDOW>(p, score, var, s);
    case FLEX_MASK_DOCUMENT:
    case FLEX_MASK_DOCUMENT_CAUSAL:
      return pick_score<BF16, D, DV, QB, KB, FLEX_MASK_DOCUMENT>(p, score, var, s);
    default:
      return pick_score<BF16, D, DV, QB, KB, FLEX_MASK_PREFIX_CAUSAL>(p, score, var, s);
  }
}

}  // namespace fwd
}  // namespace flexattn

// One translation unit per (dtype, head dim, q block, kv block) keeps the
// builds parallel.
#define FLEXATTN_FWD_UNIT(NAME, BF16, D, DV, QB, KB)                           \
  namespace flexattn {                                                       \
  hipError_t NAME(const FwdParams& p, int mask, int score, int var,          \
                  hipStream_t s) {                                           \
    return fwd::pick_mask<BF16, D, DV, QB, KB>(p, mask, score, var, s);      \
  }                                                                          \
  }
