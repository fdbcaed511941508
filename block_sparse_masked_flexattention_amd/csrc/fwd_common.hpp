// fwd_common.hpp -- pieces shared by the bf16 and fp32 forward kernels.
#pragma once
#include "internal.hpp"

namespace flexattn {
namespace fwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kLdsBytes = 160 * 1024;
// Word 3 of a raw buffer resource on gfx9-family parts (no swizzle, no
// per-lane index, dword data): reads past the size return zero.
constexpr int kBufferRsrcWord3 = 0x00020000;

// value of lane l ^ 32
__device__ inline float xor32(float x) { return __shfl_xor(x, 32); }

// max over lanes l and l ^ 32, in every lane: v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second.
__device__ inline float max_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Three-input max; with NaNs not honoured the compiler emits one v_max3_f32.
// (Plain C rather than inline assembly: the compiler must see the
// instruction to insert the wait states a VALU read of a matrix-instruction
// result needs.)
__device__ inline float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

__device__ inline u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// PRESCALE_QK on a 16-byte piece of a bf16 row: each of the eight values
// times f in fp32, rounded back to bf16 (round to nearest even).  Word i
// holds elements 2i (low half) and 2i + 1 (high half).
__device__ inline u32x4 scale_bf16x8(u32x4 x, float f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(x[i] << 16) * f;
    const float hi = __uint_as_float(x[i] & 0xffff0000u) * f;
    r[i] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)lo, (__bf16)hi});
  }
  return r;
}

// swap bits 2 and 3 of a row index (an involution)
__device__ inline int swap23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Work items (head bh, q-block qb) split over the 8 XCDs, each of which has
// its own L2.  n_items = heads * n_qb; item k of XCD xcd (k = 0, 1, ...)
// maps to (bh, qb); returns false once k is past that XCD's items.
//  * When the number of heads is a multiple of 8, XCD x owns heads
//    [x H/8, (x+1) H/8) and orders their q-blocks last-to-first across all
//    of them: every head's last q-block, then every head's second-to-last,
//    ...  Under a causal-like mask the last q-blocks are the longest, so
//    long work starts first and the short blocks fill the tail, while each
//    head's K/V stay in one XCD's L2.
//  * Otherwise each XCD gets a contiguous range of (head, q-block) items,
//    q-blocks last-to-first within a head.
__device__ inline bool xcd_item(int n_items, int n_qb, int xcd, int k, int& bh, int& qb) {
  const int n_heads = n_items / n_qb;
  if ((n_heads & 7) == 0) {
    const int hx = n_heads >> 3;
    if (k >= hx * n_qb) return false;
    const int rank = k / hx;
    bh = xcd * hx + (k - rank * hx);
    qb = n_qb - 1 - rank;
    return true;
  }
  const int per = n_items >> 3, rem = n_items & 7;
  if (k >= per + (xcd < rem ? 1 : 0)) return false;
  const int r = xcd * per + min(xcd, rem) + k;
  bh = r / n_qb;
  qb = n_qb - 1 - (r - bh * n_qb);
  return true;
}

// One work-group per item: the dispatcher sends work-group w to XCD w % 8,
// so work-group w takes item w >> 3 of that XCD.
__device__ inline void wg_to_tile(int n_qb, int& bh, int& qb) {
  const int w = blockIdx.x;
  xcd_item(gridDim.x, n_qb, w & 7, w >> 3, bh, qb);
}

// The 32-row group a wave takes in a work-group of nw waves (a power of
// two), rotated by the work-group's item.  The waves of a work-group run
// their steps together (one barrier per step), and near the diagonal or a
// window edge the groups see unequal numbers of blocks per step; with wave w
// of every resident work-group on the same SIMD, equal groups would stack
// the same imbalance there.  The rotation differs between consecutive items
// of an XCD and between items 32 apart, the neighbours on one CU under
// either fill order.
__device__ inline int row_group(int wave, int nw) {
  const int item = (int)(blockIdx.x >> 3);
  return (wave + item + (item >> 5)) & (nw - 1);
}

// Keys visible from query row qi, as one interval [lo, hi] (empty when
// lo > hi), already clipped to the key range.
template <int MASK, typename P>
__device__ inline void row_interval(const P& p, int qi, int& lo, int& hi) {
  lo = 0;
  hi = p.kv_len - 1;
  if constexpr (MASK == FLEX_MASK_CAUSAL) {
    hi = min(hi, qi);
  } else if constexpr (MASK == FLEX_MASK_SLIDING_WINDOW) {
    lo = max(0, qi - p.window);
    hi = min(hi, qi - p.window_min);
  } else if constexpr (MASK == FLEX_MASK_PREFIX_CAUSAL) {
    hi = min(hi, qi <= p.prefix ? max(p.prefix, qi) : qi);
  } else if constexpr (MASK == FLEX_MASK_DOCUMENT) {
    // both document kinds: the builder's per-row interval (causal cut
    // included); rows past the end see nothing (they read the last row's
    // pair, with no branch around the loads, and drop it)
    const size_t qc = (size_t)min(qi, p.q_len - 1);
    lo = p.bounds[2 * qc];
    hi = p.bounds[2 * qc + 1];
    if (qi >= p.q_len) {
      lo = 1;
      hi = 0;
    }
  }
}

// REL_BIAS slope of head h: from the caller's per-head table when there is
// one (a score modification that closes over a tensor), else the formula.
template <typename P>
__device__ inline float head_slope(const P& p, int h) {
  return p.slopes != nullptr ? p.slopes[h] : exp2f(-p.bias_max * (float)(h + 1) / (float)p.H);
}

// Document masks: true for the interval pair (kDocPoisonLo, kDocPoisonHi)
// the builder writes when the ids are not non-decreasing; the forward and
// backward write NaN for such a row or key.
__device__ inline bool doc_poisoned(int lo, int hi) {
  return lo == kDocPoisonLo && hi == kDocPoisonHi;
}

// A quiet NaN the compiler cannot see as one: the library is built with
// -fno-honor-nans, under which a NaN constant lets it fold the arithmetic
// that carries it.
__device__ inline float opaque_nan() {
  float x;
  asm volatile("v_mov_b32 %0, 0x7fc00000" : "=v"(x));
  return x;
}

// Masks whose rows' intervals can start after key 0: partial tiles test both
// ends.
template <int MASK>
constexpr bool two_sided_mask() {
  return MASK == FLEX_MASK_SLIDING_WINDOW || MASK == FLEX_MASK_DOCUMENT;
}

// Store one query row of O^T accumulators (lane half g) scaled by inv.
// Accumulator register r of column block e holds d = 32e + 8(r/4) + 4g + r%4.
template <int NE>
__device__ inline void write_out_row(const FwdParams& p, size_t row, int D, int g,
                                     const f32x16 (&o)[NE], float inv) {
  char* og = static_cast<char*>(p.out) + row * (size_t)D * (p.out_bf16 ? 2 : 4);
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d = 32 * e + 8 * a + 4 * g;
      const float v0 = o[e][4 * a] * inv, v1 = o[e][4 * a + 1] * inv;
      const float v2 = o[e][4 * a + 2] * inv, v3 = o[e][4 * a + 3] * inv;
      if (p.out_bf16) {
        *reinterpret_cast<bf16x4*>(og + d * 2) =
            bf16x4{(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
      } else {
        *reinterpret_cast<f32x4*>(og + d * 4) = f32x4{v0, v1, v2, v3};
      }
    }
}

// Store the 32 rows of a wave's accumulators as bf16 through LDS.  The
// accumulators are laid out like O^T: lane (lq, g) holds, in register
// 4a + i of column block e, column 32e + 8a + 4g + i of row lq.  Each lane
// writes its 8-byte pieces into the wave's own region `reg` (32 * 64 * NE
// bytes, 16-byte chunks XOR-swizzled by row), then the wave stores the rows
// as 16-byte pieces, 64 lanes covering whole rows, to og + row * 64 * NE;
// rows at or past `nrows` are not written.  Directly from the accumulator
// layout every store instruction would write 8 bytes into each of 32 rows.
// The caller guarantees that no other wave touches `reg` meanwhile.
template <int NE>
__device__ inline void store_rows_bf16_lds(__attribute__((address_space(3))) char* reg, char* og,
                                           int nrows, const f32x16 (&a)[NE], float f, int lane) {
  constexpr int OROW = 64 * NE;  // bytes per row
  constexpr int OCH = OROW / 16;  // 16-byte chunks per row
  const int lq = lane & 31, g = lane >> 5;
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x4 w = {(__bf16)(a[e][4 * q] * f), (__bf16)(a[e][4 * q + 1] * f),
                        (__bf16)(a[e][4 * q + 2] * f), (__bf16)(a[e][4 * q + 3] * f)};
      *(__attribute__((address_space(3))) bf16x4*)(reg + lq * OROW +
                                                    (((4 * e + q) ^ (lq & 7)) << 4) + 8 * g) = w;
    }
  constexpr int RPI = 64 / OCH;  // rows per store instruction
  const int cc = lane % OCH;
#pragma unroll
  for (int j = 0; j < 32 / RPI; ++j) {
    const int r = j * RPI + lane / OCH;
    const u32x4 v =
        *(__attribute__((address_space(3))) u32x4*)(reg + r * OROW + ((cc ^ (r & 7)) << 4));
    if (r < nrows) *reinterpret_cast<u32x4*>(og + (size_t)r * OROW + cc * 16) = v;
  }
}

}  // namespace fwd
}  // namespace flexattn
