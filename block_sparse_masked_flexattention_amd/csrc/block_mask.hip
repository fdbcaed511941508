// block_mask.hip -- the integer block-mask builder.
//
// Produces the kv_num_blocks / kv_indices / full_kv_num_blocks /
// full_kv_indices fields of the FlexAttention block-mask tuple (the tuple
// passed to the flex_attention higher-order op in the test hunks of
// "[Inductor][Flex Attention] Add Subtiling Option for Alpha Scaling").
//
// Every supported mask kind sees, from query row i, one contiguous interval
// of keys [lo_i, hi_i] (possibly empty).  A tile is classified from those row
// intervals instead of from its q_block * kv_block elements:
//   full    every row of the tile is in range and its interval covers all of
//           the tile's columns (which must be in range too);
//   partial some row's interval meets the tile's in-range columns;
//   empty   otherwise.
// One work-group handles one q-block row of tiles: its threads classify the
// kv-blocks, then a block-wide prefix count over the 0/1 classes gives each
// kv-block its slot.  Rows are written in full: selected kv-blocks in
// ascending order, then the others in ascending order.
#include "internal.hpp"

namespace flexattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct RowInterval {
  int lo, hi;  // inclusive; empty when lo > hi
};

__device__ inline RowInterval visible_keys(const MaskBuildParams& p, int i) {
  int lo = 0, hi = p.kv_len - 1;
  switch (p.kind) {
    case FLEX_MASK_NOOP:
      break;
    case FLEX_MASK_CAUSAL:
      hi = min(hi, i);
      break;
    case FLEX_MASK_SLIDING_WINDOW: {
      // window_min <= i - j <= window; computed in 64 bits so that
      // i - window cannot overflow
      long long l = (long long)i - p.window;
      long long h = (long long)i - p.window_min;
      lo = (int)max(0LL, l);
      hi = (int)min((long long)hi, h);
      break;
    }
    case FLEX_MASK_PREFIX_CAUSAL:
      hi = min(hi, i <= p.prefix ? max(p.prefix, i) : i);
      break;
  }
  return {lo, hi};
}

// 0 empty, 1 partial, 2 full
__device__ inline int classify(const MaskBuildParams& p, int qb, int kb) {
  const int r0 = qb * p.q_block;
  const int r1 = min(r0 + p.q_block, p.q_len);  // exclusive
  const int c0 = kb * p.kv_block;
  const int c_end = c0 + p.kv_block - 1;         // last column of the tile
  const int c1 = min(c_end, p.kv_len - 1);       // last in-range column
  bool any = false;
  bool full = (r0 + p.q_block <= p.q_len) && (c_end < p.kv_len);
  for (int i = r0; i < r1; ++i) {
    RowInterval iv = visible_keys(p, i);
    const bool nonempty = iv.lo <= iv.hi;
    any |= nonempty && iv.lo <= c1 && iv.hi >= c0;
    full &= nonempty && iv.lo <= c0 && iv.hi >= c_end;
  }
  return full ? 2 : (any ? 1 : 0);
}

// Exclusive prefix count of a 0/1 flag over the work-group, plus the total.
// Uses wave ballots; `wave_tot` is LDS scratch of kWaves ints.
__device__ inline int block_prefix(bool flag, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int below = __popcll(bal & ((1ULL << lane) - 1ULL));
  __syncthreads();
  if (lane == 0) wave_tot[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = wave_tot[w];
    before += w < wave ? c : 0;
    tot += c;
  }
  *total = tot;
  return before + below;
}

__global__ __launch_bounds__(kThreads) void build_block_mask_kernel(MaskBuildParams p) {
  __shared__ int wave_tot[kWaves];
  const int qb = blockIdx.x;
  const int nk = p.n_kb;
  const int row = qb * nk;

  // pass 1: totals of partial and full tiles in this q-block row
  int n_part = 0, n_full = 0;
  for (int base = 0; base < nk; base += kThreads) {
    const int kb = base + threadIdx.x;
    const int c = kb < nk ? classify(p, qb, kb) : 0;
    int tp, tf;
    block_prefix(c == 1, wave_tot, &tp);
    block_prefix(c == 2, wave_tot, &tf);
    n_part += tp;
    n_full += tf;
  }
  if (threadIdx.x == 0) {
    p.kv_num[qb] = n_part;
    p.fkv_num[qb] = n_full;
  }

  // pass 2: slots.  A selected kv-block goes after the selected ones before
  // it; an unselected one goes after all selected ones and the unselected
  // ones before it.
  int seen_part = 0, seen_full = 0;
  for (int base = 0; base < nk; base += kThreads) {
    const int kb = base + threadIdx.x;
    const int c = kb < nk ? classify(p, qb, kb) : 0;
    int tp, tf;
    const int bp = seen_part + block_prefix(c == 1, wave_tot, &tp);
    const int bf = seen_full + block_prefix(c == 2, wave_tot, &tf);
    if (kb < nk) {
      p.kv_idx[row + (c == 1 ? bp : n_part + (kb - bp))] = kb;
      p.fkv_idx[row + (c == 2 ? bf : n_full + (kb - bf))] = kb;
    }
    seen_part += tp;
    seen_full += tf;
  }
}

}  // namespace

hipError_t launch_block_mask(const MaskBuildParams& p, hipStream_t stream) {
  if (p.n_qb == 0) return hipSuccess;
  hipLaunchKernelGGL(build_block_mask_kernel, dim3(p.n_qb), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace flexattn
