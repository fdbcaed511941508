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
//           the tile's columns (which must be in range too): with
//           LO = max_i lo_i and HI = min_i hi_i over the tile's rows, that is
//           LO <= first column and HI >= last column;
//   partial some row's interval meets the tile's columns, i.e. the tile lies
//           in the union over rows of the kv-block ranges
//           [lo_i / kv_block, hi_i / kv_block];
//   empty   otherwise.
// One work-group handles one q-block row of tiles.  Its threads take the
// rows (a block-wide max / min gives LO and HI; each row ORs its kv-block
// range into an LDS bitmask, 256 kv-blocks at a time) and then the kv-blocks
// (one per thread per chunk).  A block-wide prefix count over the 0/1 classes
// gives each kv-block its slot: selected kv-blocks in ascending order, then
// the others in ascending order.
#include <climits>

#include "internal.hpp"

namespace flexattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kChunk = kThreads;  // kv-blocks classified per pass

struct RowInterval {
  int lo, hi;  // inclusive, clipped to [0, kv_len - 1]; empty when lo > hi
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
      // window_min <= i - j <= window, in 64 bits so i - window cannot wrap
      const long long l = (long long)i - p.window;
      const long long h = (long long)i - p.window_min;
      lo = (int)max(0LL, l);
      hi = (int)min((long long)hi, h);
      break;
    }
    case FLEX_MASK_PREFIX_CAUSAL:
      hi = min(hi, i <= p.prefix ? max(p.prefix, i) : i);
      break;
    case FLEX_MASK_DOCUMENT:
    case FLEX_MASK_DOCUMENT_CAUSAL:
      // written by doc_bounds_kernel just before, on the same stream
      lo = p.bounds[2 * (size_t)i];
      hi = p.bounds[2 * (size_t)i + 1];
      break;
  }
  return {lo, hi};
}

// First index t in [0, n) with a[t] >= x (lower) or a[t] > x (upper), n if
// none, for a non-decreasing a.  On any other array it still ends after at
// most log2(n) + 1 halvings and reads only a[0 .. n - 1].
template <bool UPPER>
__device__ inline int search_i32(const int32_t* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = lo + ((hi - lo) >> 1);
    const int v = a[mid];
    if (UPPER ? v <= x : v < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Document masks: for each of the n_own positions, the interval of the other
// side's positions with the same document id, [lower, upper - 1]; with the
// causal kind cut at the position itself (keys j <= i for a row, queries
// i >= j for a column).  out[2t], out[2t + 1] = first, last (empty when
// first > last).
__global__ __launch_bounds__(256) void doc_bounds_kernel(const int32_t* own, int n_own,
                                                         const int32_t* other, int n_other,
                                                         int causal, int is_row,
                                                         int32_t* out) {
  const int t = blockIdx.x * 256 + (int)threadIdx.x;
  if (t >= n_own) return;
  const int id = own[t];
  int lo = search_i32<false>(other, n_other, id);
  int hi = search_i32<true>(other, n_other, id) - 1;
  if (causal) {
    if (is_row) hi = min(hi, t);
    else lo = max(lo, t);
  }
  out[2 * (size_t)t] = lo;
  out[2 * (size_t)t + 1] = hi;
}

// Block-wide reductions through wave shuffles and a small LDS array.
__device__ inline int block_max(int v, int* scratch) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = scratch[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = max(r, scratch[w]);
  return r;
}

__device__ inline int block_min(int v, int* scratch) {
  return -block_max(-v, scratch);
}

// Exclusive prefix count of a 0/1 flag over the work-group, plus the total.
__device__ inline int block_prefix(bool flag, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long bal = __ballot(flag);
  const int below = __popcll(bal & ((1ULL << lane) - 1ULL));
  __syncthreads();
  if (lane == 0) scratch[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = scratch[w];
    before += w < wave ? c : 0;
    tot += c;
  }
  *total = tot;
  return before + below;
}

// Classes of kv-blocks [k0, k0 + kChunk) of this q-block row: bit t of
// `touched` is set when some row's visible interval meets kv-block k0 + t.
__device__ inline void mark_touched(const MaskBuildParams& p, int r0, int r1, int k0,
                                    unsigned* touched) {
  if (threadIdx.x < kChunk / 32) touched[threadIdx.x] = 0u;
  __syncthreads();
  for (int i = r0 + (int)threadIdx.x; i < r1; i += kThreads) {
    const RowInterval iv = visible_keys(p, i);
    if (iv.lo > iv.hi) continue;
    const int first = max(iv.lo / p.kv_block, k0) - k0;
    const int last = min(iv.hi / p.kv_block, k0 + kChunk - 1) - k0;
    for (int w = first >> 5; w <= (last >> 5) && first <= last; ++w) {
      const int b0 = max(first, w * 32) - w * 32;
      const int b1 = min(last, w * 32 + 31) - w * 32;
      const unsigned bits = (b1 - b0 == 31) ? 0xffffffffu : (((1u << (b1 - b0 + 1)) - 1u) << b0);
      atomicOr(&touched[w], bits);
    }
  }
  __syncthreads();
}

// Document masks need non-decreasing ids on both sides (then every row sees
// one run of keys).  Each thread compares one id of each array with the
// next; a work-group that finds one below its predecessor overwrites every
// interval with the poison pair (kDocPoisonLo, kDocPoisonHi): empty for the
// classification below, so no tile is listed, and the forward and backward
// write NaN for every row and key, so that the broken precondition shows
// instead of giving plausible wrong numbers.  Runs after doc_bounds_kernel,
// on the same stream.
__global__ __launch_bounds__(256) void doc_order_check_kernel(const int32_t* a, int na,
                                                              const int32_t* b, int nb,
                                                              int32_t* out, int n_out) {
  const int t = blockIdx.x * 256 + (int)threadIdx.x;
  int bad = 0;
  if (t + 1 < na && a[t] > a[t + 1]) bad = 1;
  if (t + 1 < nb && b[t] > b[t + 1]) bad = 1;
  if (!__syncthreads_or(bad)) return;
  for (int i = (int)threadIdx.x; i < n_out; i += 256) {
    out[2 * (size_t)i] = kDocPoisonLo;
    out[2 * (size_t)i + 1] = kDocPoisonHi;
  }
}

__global__ __launch_bounds__(kThreads) void build_block_mask_kernel(MaskBuildParams p) {
  __shared__ int scratch[kWaves];
  __shared__ unsigned touched[kChunk / 32];
  const int qb = blockIdx.x;
  const int nk = p.n_kb;
  const size_t row = (size_t)qb * nk;
  const int r0 = qb * p.q_block;
  const int r1 = min(r0 + p.q_block, p.q_len);  // exclusive; r0 < r1 since qb < n_qb

  // LO = max lo_i, HI = min hi_i over the q-block's rows
  int lo_max = INT_MIN, hi_min = INT_MAX;
  for (int i = r0 + (int)threadIdx.x; i < r1; i += kThreads) {
    const RowInterval iv = visible_keys(p, i);
    lo_max = max(lo_max, iv.lo);
    hi_min = min(hi_min, iv.hi);
  }
  lo_max = block_max(lo_max, scratch);
  hi_min = block_min(hi_min, scratch);
  const bool rows_in_range = r0 + p.q_block <= p.q_len;

  // pass 0 counts, pass 1 writes; a row of at most kChunk kv-blocks is one
  // chunk, whose totals are known in the same pass that places it
  const bool one_chunk = nk <= kChunk;
  int n_part = 0, n_full = 0;
  for (int pass = one_chunk ? 1 : 0; pass < 2; ++pass) {
    int seen_part = 0, seen_full = 0;
    for (int k0 = 0; k0 < nk; k0 += kChunk) {
      mark_touched(p, r0, r1, k0, touched);
      const int kb = k0 + (int)threadIdx.x;
      int c = 0;  // 0 empty, 1 partial, 2 full
      if (kb < nk) {
        const int c0 = kb * p.kv_block;
        const int c_end = c0 + p.kv_block - 1;
        const bool full = rows_in_range && c_end < p.kv_len && lo_max <= c0 && hi_min >= c_end;
        const bool any = (touched[threadIdx.x >> 5] >> (threadIdx.x & 31)) & 1u;
        c = full ? 2 : (any ? 1 : 0);
      }
      int tp, tf;
      const int bp = seen_part + block_prefix(c == 1, scratch, &tp);
      const int bf = seen_full + block_prefix(c == 2, scratch, &tf);
      if (one_chunk) {
        n_part = tp;
        n_full = tf;
      }
      if (pass == 1 && kb < nk) {
        // selected: after the selected ones before it; otherwise after all
        // selected ones and the unselected ones before it
        p.kv_idx[row + (c == 1 ? bp : n_part + (kb - bp))] = kb;
        p.fkv_idx[row + (c == 2 ? bf : n_full + (kb - bf))] = kb;
      }
      seen_part += tp;
      seen_full += tf;
    }
    n_part = seen_part;
    n_full = seen_full;
  }
  if (threadIdx.x == 0) {
    p.kv_num[qb] = n_part;
    p.fkv_num[qb] = n_full;
  }
}

// Transposed arrays (q_num_blocks / q_indices / full_q_num_blocks /
// full_q_indices, the second half of the same block-mask tuple): one
// work-group per kv-block column, eight lanes per (q-block, kv-block) tile.
// The lanes classify their tile from the q-block's row intervals exactly as
// above (full: every row in range and its interval covering the in-range
// tile; partial: some row's interval meeting the tile's columns), then the
// same two-pass prefix count orders the column: selected q-blocks ascending,
// then the others ascending.  The kv_num / kv_idx / fkv_num / fkv_idx fields
// of the parameters carry the four transposed arrays here.
__global__ __launch_bounds__(kThreads) void build_block_mask_t_kernel(MaskBuildParams p) {
  // kLanes consecutive lanes share a tile and split its rows (or, for the
  // document kinds, its columns); their verdicts meet through shuffles
  constexpr int kLanes = 8;
  constexpr int kTiles = kThreads / kLanes;  // tiles per pass over the column
  // the first pass keeps each tile's class here for the second, when the
  // column has at most kMaxCached q-blocks; longer columns classify twice
  constexpr int kMaxCached = 4096;
  __shared__ int scratch[kWaves];
  __shared__ unsigned char cls[kMaxCached];
  const int kb = blockIdx.x;
  const int nq = p.n_qb;
  const size_t col = (size_t)kb * nq;
  const int c0 = kb * p.kv_block;
  const int c_end = c0 + p.kv_block - 1;
  const int c_last = min(c_end, p.kv_len - 1);  // c0 <= kv_len - 1 since kb < n_kb
  const int sub = (int)threadIdx.x % kLanes;
  const bool doc = p.kind == FLEX_MASK_DOCUMENT || p.kind == FLEX_MASK_DOCUMENT_CAUSAL;
  const bool cached = nq <= kMaxCached;
  int n_part = 0, n_full = 0;
  for (int pass = 0; pass < 2; ++pass) {
    int seen_part = 0, seen_full = 0;
    for (int q00 = 0; q00 < nq; q00 += kTiles) {
      const int qb = q00 + (int)threadIdx.x / kLanes;
      int all = 1, any = 0;
      if (pass == 1 && cached) {
        // (written in pass 0 before a barrier of its scans)
        const int c0c = qb < nq ? cls[qb] : 0;
        all = c0c == 2;
        any = c0c != 0;
      } else if (qb < nq) {
        const int r0 = qb * p.q_block;
        const int r1 = min(r0 + p.q_block, p.q_len);
        all = r0 + p.q_block <= p.q_len && c_end < p.kv_len;
        if (doc) {
          // the same classes from the columns' query intervals (p.bounds
          // holds the column bounds here)
          const int r_end = r0 + p.q_block - 1, r_last = r1 - 1;
          for (int j = c0 + sub; j <= c_last; j += kLanes) {
            const int clo = p.bounds[2 * (size_t)j], chi = p.bounds[2 * (size_t)j + 1];
            all = all && clo <= r0 && chi >= r_end;
            any = any || (clo <= chi && clo <= r_last && chi >= r0);
          }
        } else {
          for (int i = r0 + sub; i < r1; i += kLanes) {
            const RowInterval iv = visible_keys(p, i);
            all = all && iv.lo <= c0 && iv.hi >= c_end;
            any = any || (iv.lo <= iv.hi && iv.lo <= c_last && iv.hi >= c0);
          }
        }
      }
      if (pass == 0 || !cached) {
#pragma unroll
        for (int o = 1; o < kLanes; o <<= 1) {
          all &= __shfl_xor(all, o);
          any |= __shfl_xor(any, o);
        }
      }
      // one flag per tile, on its first lane: thread order is q-block order
      const int c = (qb < nq && sub == 0) ? (all ? 2 : (any ? 1 : 0)) : 0;
      if (pass == 0 && cached && qb < nq && sub == 0) cls[qb] = (unsigned char)c;
      int tp, tf;
      const int bp = seen_part + block_prefix(c == 1, scratch, &tp);
      const int bf = seen_full + block_prefix(c == 2, scratch, &tf);
      if (pass == 1 && qb < nq && sub == 0) {
        p.kv_idx[col + (c == 1 ? bp : n_part + (qb - bp))] = qb;
        p.fkv_idx[col + (c == 2 ? bf : n_full + (qb - bf))] = qb;
      }
      seen_part += tp;
      seen_full += tf;
    }
    n_part = seen_part;
    n_full = seen_full;
  }
  if (threadIdx.x == 0) {
    p.kv_num[kb] = n_part;
    p.fkv_num[kb] = n_full;
  }
}

}  // namespace

hipError_t launch_block_mask_t(const MaskBuildParams& p, hipStream_t stream) {
  if (p.n_kb == 0) return hipSuccess;
  if (is_document_mask(p.kind)) {
    hipLaunchKernelGGL(doc_bounds_kernel, dim3((unsigned)((p.kv_len + 255) / 256)), dim3(256), 0,
                       stream, p.kv_doc, p.kv_len, p.q_doc, p.q_len,
                       p.kind == FLEX_MASK_DOCUMENT_CAUSAL ? 1 : 0, 0, p.bounds);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nchk = max(p.q_len, p.kv_len);
    hipLaunchKernelGGL(doc_order_check_kernel, dim3((unsigned)((nchk + 255) / 256)), dim3(256), 0,
                       stream, p.q_doc, p.q_len, p.kv_doc, p.kv_len, p.bounds, p.kv_len);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(build_block_mask_t_kernel, dim3(p.n_kb), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_block_mask(const MaskBuildParams& p, hipStream_t stream) {
  if (p.n_qb == 0) return hipSuccess;
  if (is_document_mask(p.kind)) {
    hipLaunchKernelGGL(doc_bounds_kernel, dim3((unsigned)((p.q_len + 255) / 256)), dim3(256), 0,
                       stream, p.q_doc, p.q_len, p.kv_doc, p.kv_len,
                       p.kind == FLEX_MASK_DOCUMENT_CAUSAL ? 1 : 0, 1, p.bounds);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nchk = max(p.q_len, p.kv_len);
    hipLaunchKernelGGL(doc_order_check_kernel, dim3((unsigned)((nchk + 255) / 256)), dim3(256), 0,
                       stream, p.q_doc, p.q_len, p.kv_doc, p.kv_len, p.bounds, p.q_len);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(build_block_mask_kernel, dim3(p.n_qb), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace flexattn
