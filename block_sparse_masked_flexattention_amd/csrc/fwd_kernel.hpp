// fwd_kernel.hpp -- the block-sparse masked attention forward kernel for gfx950.
//
// What it computes follows the FlexAttention forward template: per Q_BLOCK
// rows of queries it walks the kv-blocks listed in the block mask (partial
// tiles first, then full tiles), forms S = scale * Q K^T per tile, applies the
// score modification on every tile and the mask only on partial tiles, then
// takes the online-softmax step of forward_block_mn ("[Inductor][Flex
// Attention] Add Subtiling Option for Alpha Scaling", common.py.jinja hunk):
//   m_new = max(m, rowmax S);  alpha = exp(m - m_new);  p = exp(S - m_new)
//   l = l * alpha + rowsum p;  acc = acc * alpha (optionally per D-half);
//   acc += p V  (p rounded to the input type first, accumulation inside the
//   matrix instruction, as in the acc = dot(p, v, acc) form discussed in
//   "Performance for templated attention strangely bad for a combination of
//   causal + upper square mask").
//
// How it maps onto CDNA4:
//  * One work-group per (batch, head, q-block); one wave per 32 query rows.
//  * Both products use v_mfma_f32_32x32x16_bf16 (v_mfma_f32_32x32x2_f32 for
//    fp32 inputs).  The first is computed transposed, S^T = K Q^T, so every
//    lane owns one query row: lane l holds row (l & 31) and half of that
//    row's keys; the row max needs one exchange between the lane halves and
//    the row sum none until the end.
//  * Q stays in registers for the whole kernel (B operand of S^T = K Q^T).
//  * K rows are stored in LDS with bits 2 and 3 of the row index swapped
//    inside each 32-row group.  With that permutation, the eight S^T values a
//    lane holds in registers 8h..8h+7 of a 32-key block are eight
//    consecutive keys, which is exactly the B operand of O^T = V^T P^T, so p
//    never leaves registers and V^T is read with one 16-byte LDS read per
//    instruction.
//  * V is transposed in registers on its way to LDS (4 keys x 8 columns per
//    thread), so LDS holds V^T.
//  * K and V^T tiles are double-buffered in LDS; the next tile's 128-bit
//    global loads are issued before the current tile's products.  LDS rows
//    are XOR-swizzled in 16-byte chunks so the wave's reads and writes hit
//    distinct banks.
//  * Scores are kept in base-2 units (scale * log2 e folded into one FMA) and
//    exponentiated with v_exp_f32.
//  * The mask of every supported kind is, for a fixed query row, one interval
//    of visible keys.  The interval is computed once per row (the q-side
//    predicate hoisted out of the key loop, the change the templated-attention
//    performance issue measured); on partial tiles each score then needs one
//    or two integer compares.
#pragma once
#include "internal.hpp"

namespace flexattn {
namespace fwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kLdsBytes = 160 * 1024;

__device__ inline float xor32(float x) { return __shfl_xor(x, 32); }

__device__ inline u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// swap bits 2 and 3 of a row index (an involution)
__device__ inline int swap23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <bool BF16, int D, int QB, int KB, int MASK, int SCORE, bool SUB>
struct FwdKernel {
  static constexpr int NW = QB / 32;  // waves per work-group
  static constexpr int NT = NW * 64;  // threads per work-group
  static constexpr int NB = KB / 32;  // 32-key blocks per tile
  static constexpr int NE = D / 32;   // 32-column blocks of the head dim
  static constexpr int ESZ = BF16 ? 2 : 4;
  static constexpr int TILE_BYTES = KB * D * ESZ;
  static constexpr int STAGES = (4 * TILE_BYTES <= kLdsBytes) ? 2 : 1;
  static constexpr int CPR = D * ESZ / 16;  // 16-byte chunks per row of K / V
  static constexpr int K_CHUNKS = KB * CPR;
  static constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
  // bf16 V goes through registers in blocks of 4 keys x 8 columns
  static constexpr int V_BLOCKS = BF16 ? (KB / 4) * (D / 8) : K_CHUNKS;
  static constexpr int V_PER_T = (V_BLOCKS + NT - 1) / NT;
  static constexpr int V_REGS = BF16 ? 4 : 1;  // 16-byte loads per V block
  static_assert(QB % 32 == 0 && KB % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(D >= 64 && KB >= 64, "swizzles need 8 chunks per row");

  // ---- LDS layouts ----
  // K: row m (swapped-bit order), 16-byte chunk c stored at chunk c ^ (m & 7)
  __device__ static inline int k_off(int m, int c) {
    return m * (D * ESZ) + ((c ^ (m & 7)) << 4);
  }
  // bf16 V^T: row d (head-dim column), 16-byte chunk c (8 keys) at c ^ swz(d)
  __device__ static inline int vt_off(int d, int c) {
    return d * (KB * 2) + ((c ^ ((d + (d >> 3)) & 7)) << 4);
  }
  // fp32 V: row-major [key][d]
  __device__ static inline int v_off(int kv, int d) { return (kv * D + d) * 4; }

  struct Stage {
    u32x4 k[K_PER_T];
    u32x4 v[V_PER_T][V_REGS];
  };

  __device__ static inline void load_tile(Stage& st, const char* kg,
                                          const char* vg, int kv0, int kv_len,
                                          bool ragged, int tid) {
#pragma unroll
    for (int it = 0; it < K_PER_T; ++it) {
      const int c = tid + it * NT;
      if (K_CHUNKS % NT == 0 || c < K_CHUNKS) {
        const int row = c / CPR, col = c % CPR;
        const size_t off = (size_t)(kv0 + row) * (D * ESZ) + col * 16;
        st.k[it] = (!ragged || kv0 + row < kv_len) ? ld_global16(kg + off)
                                                   : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int it = 0; it < V_PER_T; ++it) {
      const int blk = tid + it * NT;
      if (V_BLOCKS % NT == 0 || blk < V_BLOCKS) {
        if constexpr (BF16) {
          const int dg = ((blk >> 3) / (KB / 4)) * 8 + (blk & 7);
          const int kvg = (blk >> 3) % (KB / 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = 4 * kvg + j;
            const size_t off = (size_t)(kv0 + row) * (D * 2) + dg * 16;
            st.v[it][j] = (!ragged || kv0 + row < kv_len) ? ld_global16(vg + off)
                                                          : u32x4{0, 0, 0, 0};
          }
        } else {
          const int row = blk / CPR, col = blk % CPR;
          const size_t off = (size_t)(kv0 + row) * (D * 4) + col * 16;
          st.v[it][0] = (!ragged || kv0 + row < kv_len) ? ld_global16(vg + off)
                                                        : u32x4{0, 0, 0, 0};
        }
      }
    }
  }

  __device__ static inline void store_tile(const Stage& st, char* ks, char* vs,
                                           int tid) {
#pragma unroll
    for (int it = 0; it < K_PER_T; ++it) {
      const int c = tid + it * NT;
      if (K_CHUNKS % NT == 0 || c < K_CHUNKS) {
        const int row = c / CPR, col = c % CPR;
        const int m = (row & ~31) | swap23(row & 31);
        *reinterpret_cast<u32x4*>(ks + k_off(m, col)) = st.k[it];
      }
    }
#pragma unroll
    for (int it = 0; it < V_PER_T; ++it) {
      const int blk = tid + it * NT;
      if (V_BLOCKS % NT == 0 || blk < V_BLOCKS) {
        if constexpr (BF16) {
          const int dg = ((blk >> 3) / (KB / 4)) * 8 + (blk & 7);
          const int kvg = (blk >> 3) % (KB / 4);
          const u32x4* r = st.v[it];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            // column pair (8dg + 2w, 8dg + 2w + 1) of the four key rows
            const unsigned lo01 = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x05040100u);
            const unsigned lo23 = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x05040100u);
            const unsigned hi01 = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x07060302u);
            const unsigned hi23 = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x07060302u);
            const int d0 = dg * 8 + 2 * w;
            const int cc = kvg >> 1, half = (kvg & 1) * 8;
            *reinterpret_cast<u32x2*>(vs + vt_off(d0, cc) + half) = u32x2{lo01, lo23};
            *reinterpret_cast<u32x2*>(vs + vt_off(d0 + 1, cc) + half) = u32x2{hi01, hi23};
          }
        } else {
          const int row = blk / CPR, col = blk % CPR;
          *reinterpret_cast<u32x4*>(vs + v_off(row, col * 4)) = st.v[it][0];
        }
      }
    }
  }

  __device__ static void run(const FwdParams& p) {
    __shared__ __attribute__((aligned(16))) char lds[STAGES * 2 * TILE_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, g = lane >> 5;

    // ---- work-group -> (b, h, q-block): each XCD gets a contiguous range of
    // (head, q-block) work so a head's K/V stay in that XCD's L2; within a
    // head the q-blocks run last-to-first (the heaviest first under a
    // causal-like mask).
    const int nwg = gridDim.x, w = blockIdx.x;
    const int xcd = w & 7, per = nwg >> 3, rem = nwg & 7;
    const int r = xcd * per + min(xcd, rem) + (w >> 3);
    const int bh = r / p.n_qb;
    const int qb = p.n_qb - 1 - (r - bh * p.n_qb);
    const int h = bh % p.H;

    const int q0 = qb * QB;
    const int qi = q0 + wave * 32 + lq;  // this lane's query row
    const bool q_ok = qi < p.q_len;
    const bool q_ragged = q0 + QB > p.q_len;

    const size_t head_q = (size_t)bh * p.q_len;
    const size_t head_kv = (size_t)bh * p.kv_len;
    const char* qg = static_cast<const char*>(p.q) + head_q * D * ESZ;
    const char* kg = static_cast<const char*>(p.k) + head_kv * D * ESZ;
    const char* vg = static_cast<const char*>(p.v) + head_kv * D * ESZ;

    // ---- Q fragments: B operand of S^T = K Q^T ----
    constexpr int NQF = BF16 ? D / 16 : D / 8;
    u32x4 qf[NQF];
#pragma unroll
    for (int t = 0; t < NQF; ++t) {
      qf[t] = q_ok ? ld_global16(qg + ((size_t)qi * D) * ESZ + (2 * t + g) * 16)
                   : u32x4{0, 0, 0, 0};
      if (p.neg_q) qf[t] ^= (BF16 ? 0x80008000u : 0x80000000u);
    }

    // ---- this row's visible key interval [lo, hi] (mask kinds of the ABI)
    int lo = 0, hi = p.kv_len - 1;
    if constexpr (MASK == FLEX_MASK_CAUSAL) {
      hi = min(hi, qi);
    } else if constexpr (MASK == FLEX_MASK_SLIDING_WINDOW) {
      lo = max(0, qi - p.window);
      hi = min(hi, qi - p.window_min);
    } else if constexpr (MASK == FLEX_MASK_PREFIX_CAUSAL) {
      hi = min(hi, qi <= p.prefix ? max(p.prefix, qi) : qi);
    }

    float nsl2 = 0.f;  // -slope_h * log2(e)
    if constexpr (SCORE == FLEX_SCORE_REL_BIAS)
      nsl2 = -exp2f(-p.bias_max * (float)(h + 1) / (float)p.H) * kLog2e;

    // ---- tile list ----
    const int nk = p.n_kb;
    const int np = min(max(p.kv_num[qb], 0), nk);
    const int nf = min(max(p.fkv_num[qb], 0), nk);
    const int ntiles = np + nf;
    const int32_t* prow = p.kv_idx + (size_t)qb * nk;
    const int32_t* frow = p.fkv_idx + (size_t)qb * nk;
    auto tile_kb = [&](int n) {
      const int v = n < np ? prow[n] : frow[n - np];
      return min(max(v, 0), nk - 1);
    };

    float m_run = -INFINITY;  // running max, base-2 units
    float l_run = 0.f;        // this lane's half of the running row sum
    f32x16 o[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) o[e] = f32x16{};

    char* lds_k[STAGES];
    char* lds_v[STAGES];
#pragma unroll
    for (int s = 0; s < STAGES; ++s) {
      lds_k[s] = lds + s * 2 * TILE_BYTES;
      lds_v[s] = lds_k[s] + TILE_BYTES;
    }

    Stage st;
    int kb_cur = 0;
    if (ntiles > 0) {
      kb_cur = tile_kb(0);
      const int kv0 = kb_cur * KB;
      load_tile(st, kg, vg, kv0, p.kv_len, kv0 + KB > p.kv_len, tid);
      store_tile(st, lds_k[0], lds_v[0], tid);
    }
    __syncthreads();

    for (int n = 0; n < ntiles; ++n) {
      const int buf = STAGES == 2 ? (n & 1) : 0;
      const int kv0 = kb_cur * KB;
      const bool tile_ragged = kv0 + KB > p.kv_len;
      // a listed-full tile at a ragged edge is still handled as partial
      const bool partial = n < np || q_ragged || tile_ragged;

      int kb_next = 0;
      const bool has_next = n + 1 < ntiles;
      if (has_next) {
        kb_next = tile_kb(n + 1);
        const int kvn = kb_next * KB;
        if constexpr (STAGES == 2)
          load_tile(st, kg, vg, kvn, p.kv_len, kvn + KB > p.kv_len, tid);
      }

      const char* ks = lds_k[buf];
      const char* vs = lds_v[buf];

      // ---- S^T = K Q^T for the whole tile ----
      f32x16 s[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s[b] = f32x16{};
        const int m = 32 * b + lq;
        if constexpr (BF16) {
#pragma unroll
          for (int t = 0; t < D / 16; ++t) {
            const u32x4 kf = *reinterpret_cast<const u32x4*>(ks + k_off(m, 2 * t + g));
            s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qf[t]),
                s[b], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int u = 0; u < D / 8; ++u) {
            const f32x4 kf = *reinterpret_cast<const f32x4*>(ks + k_off(m, 2 * u + g));
            const f32x4 qv = __builtin_bit_cast(f32x4, qf[u]);
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
              s[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[e4], qv[e4], s[b], 0, 0, 0);
          }
        }
      }

      // ---- score modification, mask, online softmax ----
      // register r of block b holds key kv0 + 8g + 32b + 16(r >> 3) + (r & 7)
      const int kvl = kv0 + 8 * g;
      float m_use, alpha;
      {
        if constexpr (SCORE == FLEX_SCORE_REL_BIAS) {
          // t = c1 * qk - slope * log2(e) * (qi - kv)
          const float base = nsl2 * (float)(qi - kvl);
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int off = 32 * b + 16 * (rr >> 3) + (rr & 7);
              const float bias = fmaf(-nsl2, (float)off, base);
              s[b][rr] = fmaf(s[b][rr], p.c1, bias);
            }
        }
        if (partial) {
          const int lim_hi = hi - kvl, lim_lo = lo - kvl;
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int off = 32 * b + 16 * (rr >> 3) + (rr & 7);
              bool vis = off <= lim_hi;
              if constexpr (MASK == FLEX_MASK_SLIDING_WINDOW) vis = vis && off >= lim_lo;
              s[b][rr] = vis ? s[b][rr] : -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[b][rr]);
        mx = fmaxf(mx, xor32(mx));
        if constexpr (SCORE == FLEX_SCORE_IDENTITY) mx *= p.c1;
        const float m_new = fmaxf(m_run, mx);
        // a row with nothing visible so far keeps m = -inf; exponents then
        // use 0 so that exp2(-inf - 0) = 0 instead of NaN
        m_use = (partial && m_new == -INFINITY) ? 0.f : m_new;
        alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
      }

      float rowsum = 0.f;
      f32x16 pf[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          float x;
          if constexpr (SCORE == FLEX_SCORE_IDENTITY)
            x = fmaf(s[b][rr], p.c1, -m_use);
          else
            x = s[b][rr] - m_use;
          const float pv = __builtin_amdgcn_exp2f(x);
          pf[b][rr] = pv;
          rowsum += pv;
        }
      l_run = l_run * alpha + rowsum;

      // ---- O^T += V^T P^T, with the alpha rescale before it ----
      if constexpr (BF16) {
        bf16x8 pk[NB][2];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int i = 0; i < 8; ++i) pk[b][hh][i] = (__bf16)pf[b][8 * hh + i];

        constexpr int NHALF = SUB ? 2 : 1;
#pragma unroll
        for (int half = 0; half < NHALF; ++half) {
          constexpr int EPH = NE / NHALF;
#pragma unroll
          for (int e = half * EPH; e < (half + 1) * EPH; ++e) o[e] *= alpha;
#pragma unroll
          for (int e = half * EPH; e < (half + 1) * EPH; ++e) {
            const int d = 32 * e + lq;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
              for (int hh = 0; hh < 2; ++hh) {
                const u32x4 vf = *reinterpret_cast<const u32x4*>(
                    vs + vt_off(d, 4 * b + 2 * hh + g));
                o[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, vf), pk[b][hh], o[e], 0, 0, 0);
              }
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) o[e] *= alpha;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int d = 32 * e + lq;
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int kv = 32 * b + 16 * (rr >> 3) + 8 * g + (rr & 7);
              const float vv = *reinterpret_cast<const float*>(vs + v_off(kv, d));
              o[e] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, pf[b][rr], o[e], 0, 0, 0);
            }
        }
      }

      if (has_next) {
        if constexpr (STAGES == 2) {
          store_tile(st, lds_k[buf ^ 1], lds_v[buf ^ 1], tid);
        } else {
          __syncthreads();  // everyone is done reading the single buffer
          const int kvn = kb_next * KB;
          load_tile(st, kg, vg, kvn, p.kv_len, kvn + KB > p.kv_len, tid);
          store_tile(st, lds_k[0], lds_v[0], tid);
        }
      }
      __syncthreads();
      kb_cur = kb_next;
    }

    // ---- epilogue: out = acc / l, lse = m + ln l ----
    const float l_tot = l_run + xor32(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (q_ok) {
      char* og = static_cast<char*>(p.out) + (head_q + qi) * (size_t)D * (p.out_bf16 ? 2 : 4);
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = 32 * e + 8 * a + 4 * g;  // registers 4a..4a+3
          const float v0 = o[e][4 * a] * inv, v1 = o[e][4 * a + 1] * inv;
          const float v2 = o[e][4 * a + 2] * inv, v3 = o[e][4 * a + 3] * inv;
          if (p.out_bf16) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 ov = {(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
            *reinterpret_cast<bf16x4*>(og + d * 2) = ov;
          } else {
            *reinterpret_cast<f32x4*>(og + d * 4) = f32x4{v0, v1, v2, v3};
          }
        }
      if (p.lse != nullptr && g == 0)
        p.lse[head_q + qi] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
};

template <bool BF16, int D, int QB, int KB, int MASK, int SCORE, bool SUB>
__global__ __launch_bounds__(QB * 2) void flex_fwd_kernel(FwdParams p) {
  FwdKernel<BF16, D, QB, KB, MASK, SCORE, SUB>::run(p);
}

template <bool BF16, int D, int QB, int KB, int MASK, int SCORE, bool SUB>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  const long long nwg = (long long)p.B * p.H * p.n_qb;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL((flex_fwd_kernel<BF16, D, QB, KB, MASK, SCORE, SUB>),
                     dim3((unsigned)nwg), dim3(QB * 2), 0, stream, p);
  return hipGetLastError();
}

// ---- per-instance dispatch over mask kind, score kind and subtiling ----
template <bool BF16, int D, int QB, int KB, int MASK, int SCORE>
hipError_t pick_sub(const FwdParams& p, bool sub, hipStream_t s) {
  // fp32 inputs: the subtiled order is the same arithmetic; one instance.
  if (BF16 && sub) return launch_one<BF16, D, QB, KB, MASK, SCORE, true>(p, s);
  return launch_one<BF16, D, QB, KB, MASK, SCORE, false>(p, s);
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
#define FLEXATTN_FWD_UNIT(NAME, BF16, D, QB, KB)                                  \
  namespace flexattn {                                                          \
  hipError_t NAME(const FwdParams& p, int mask, int score, bool sub,            \
                  hipStream_t s) {                                              \
    return fwd::pick_mask<BF16, D, QB, KB>(p, mask, score, sub, s);             \
  }                                                                             \
  }
