// fwd_fp32.hpp -- the fp32-input forward kernel for gfx950.
//
// Same computation as the bf16 kernel (see fwd_bf16.hpp): the FlexAttention
// forward walking the block mask, online softmax as in forward_block_mn of
// "[Inductor][Flex Attention] Add Subtiling Option for Alpha Scaling".  With
// fp32 inputs everything stays in fp32: both products run on
// v_mfma_f32_32x32x2_f32 and p is not rounded before P V.  The lane layout is
// the bf16 kernel's (S^T = K Q^T, K rows with bits 2 and 3 swapped, one query
// row per lane); V stays row-major in LDS because an fp32 operand is one
// element per lane.  The running max is updated exactly every tile.  DV is
// the value head dim (V rows, the output), which may differ from D.
#pragma once
#include "fwd_common.hpp"

namespace flexattn {
namespace fwd {

template <int D, int DV, int QB, int KB, int MASK, int SCORE>
struct Fp32Fwd {
  static constexpr int NW = QB / 32;
  static constexpr int NT = NW * 64;
  static constexpr int NB = KB / 32;
  static constexpr int NE = DV / 32;
  static constexpr int ROWB = D * 4;         // bytes per K row
  static constexpr int ROWBV = DV * 4;       // bytes per V row
  static constexpr int TILE = KB * ROWB;     // K tile (V follows)
  static constexpr int TILEV = KB * ROWBV;
  static constexpr int STAGEB = TILE + TILEV;
  static constexpr int STAGES = (2 * STAGEB <= kLdsBytes) ? 2 : 1;
  static constexpr int CPR = ROWB / 16;
  static constexpr int CPRV = ROWBV / 16;
  static constexpr int LPT = KB * CPR / NT;
  static constexpr int LPTV = KB * CPRV / NT;
  static_assert(KB * CPR % NT == 0 && KB * CPRV % NT == 0, "tile load split");

  __device__ static inline int k_off(int m, int c) { return m * ROWB + ((c ^ (m & 7)) << 4); }

  __device__ static void run(const FwdParams& p) {
    __shared__ __attribute__((aligned(16))) char smem_raw[STAGES * STAGEB];
    typedef __attribute__((address_space(3))) char lds_t;
    lds_t* smem = (lds_t*)smem_raw;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, g = lane >> 5;

    int bh, qb;
    wg_to_tile(p.n_qb, bh, qb);
    const int h = bh % p.H;
    const int q0 = qb * QB;
    const int qi = q0 + wave * 32 + lq;
    const bool q_ragged = q0 + QB > p.q_len;
    const size_t head_q = (size_t)bh * p.q_len;
    const size_t head_kv = (size_t)bh * p.kv_len;
    const char* qg = static_cast<const char*>(p.q) + head_q * ROWB;
    const char* kg = static_cast<const char*>(p.k) + head_kv * ROWB;
    const char* vg = static_cast<const char*>(p.v) + head_kv * ROWBV;

    // Q fragments: lane group g holds d = 8u + 4g + e4
    f32x4 qf[D / 8];
#pragma unroll
    for (int u = 0; u < D / 8; ++u) {
      u32x4 raw = qi < p.q_len ? ld_global16(qg + (size_t)qi * ROWB + (2 * u + g) * 16)
                               : u32x4{0, 0, 0, 0};
      if (p.neg_q) raw ^= 0x80000000u;
      qf[u] = __builtin_bit_cast(f32x4, raw);
      if (p.prescale) qf[u] *= p.qscale;  // PRESCALE_QK (fp32: rounded to fp32)
    }
    int lo, hi;
    row_interval<MASK>(p, qi, lo, hi);
    float nsl2 = 0.f;
    if constexpr (SCORE == FLEX_SCORE_REL_BIAS)
      nsl2 = -head_slope(p, h) * kLog2e;

    const int nk = p.n_kb;
    const int np = min(max(p.kv_num[qb], 0), nk);
    const int nf = min(max(p.fkv_num[qb], 0), nk);
    const int ntiles = np + nf;
    const int32_t* prow = p.kv_idx + (size_t)qb * nk;
    const int32_t* frow = p.fkv_idx + (size_t)qb * nk;
    auto tile_kb = [&](int n) {
      const int v = p.contig ? (n < np ? prow[0] + n : frow[0] + (n - np))
                             : (n < np ? prow[n] : frow[n - np]);
      return __builtin_amdgcn_readfirstlane(min(max(v, 0), nk - 1));
    };

    u32x4 sk[LPT], sv[LPTV];
    auto fetch = [&](int kb) {
      const int kv0 = kb * KB;
      const bool ragged = kv0 + KB > p.kv_len;
#pragma unroll
      for (int it = 0; it < LPT; ++it) {
        const int id = tid + it * NT;
        const int row = id / CPR, col = id % CPR;
        const size_t off = (size_t)(kv0 + row) * ROWB + col * 16;
        const bool ok = !ragged || kv0 + row < p.kv_len;
        sk[it] = ok ? ld_global16(kg + off) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int it = 0; it < LPTV; ++it) {
        const int id = tid + it * NT;
        const int row = id / CPRV, col = id % CPRV;
        const size_t off = (size_t)(kv0 + row) * ROWBV + col * 16;
        const bool ok = !ragged || kv0 + row < p.kv_len;
        sv[it] = ok ? ld_global16(vg + off) : u32x4{0, 0, 0, 0};
      }
    };
    auto stash = [&](int buf) {
      const int base = buf * STAGEB;
#pragma unroll
      for (int it = 0; it < LPT; ++it) {
        const int id = tid + it * NT;
        const int row = id / CPR, col = id % CPR;
        const int m = (row & ~31) | swap23(row & 31);
        *(__attribute__((address_space(3))) u32x4*)(smem + base + k_off(m, col)) = sk[it];
      }
#pragma unroll
      for (int it = 0; it < LPTV; ++it) {
        const int id = tid + it * NT;
        const int row = id / CPRV, col = id % CPRV;
        *(__attribute__((address_space(3))) u32x4*)(smem + base + TILE + row * ROWBV + col * 16) =
            sv[it];
      }
    };

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) o[e] = f32x16{};

    int kb_cur = 0;
    if (ntiles > 0) {
      kb_cur = tile_kb(0);
      fetch(kb_cur);
      stash(0);
    }
    __syncthreads();

    for (int n = 0; n < ntiles; ++n) {
      const int base = STAGES == 2 ? (n & 1) * STAGEB : 0;
      const int kv0 = kb_cur * KB;
      const bool partial = n < np || q_ragged || kv0 + KB > p.kv_len;
      const bool has_next = n + 1 < ntiles;
      int kb_next = 0;
      if (has_next) {
        kb_next = tile_kb(n + 1);
        if constexpr (STAGES == 2) fetch(kb_next);
      }

      f32x16 s[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s[b] = f32x16{};
        const int m = 32 * b + lq;
#pragma unroll
        for (int u = 0; u < D / 8; ++u) {
          const f32x4 kf = *(__attribute__((address_space(3))) f32x4*)(
              smem + base + k_off(m, 2 * u + g));
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4)
            s[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[e4], qf[u][e4], s[b], 0, 0, 0);
        }
      }

      const int kvl = kv0 + 8 * g;
      if constexpr (SCORE == FLEX_SCORE_REL_BIAS) {
        const float bias0 = nsl2 * (float)(qi - kvl);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * b + 16 * (r >> 3) + (r & 7);
            s[b][r] = fmaf(s[b][r], p.c1, fmaf(-nsl2, (float)off, bias0));
          }
      }
      if (partial) {
        const int lim_hi = hi - kvl, lim_lo = lo - kvl;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 32 * b + 16 * (r >> 3) + (r & 7);
            bool vis = off <= lim_hi;
            if constexpr (two_sided_mask<MASK>()) vis = vis && off >= lim_lo;
            s[b][r] = vis ? s[b][r] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
      mx = max_halves(mx);
      if constexpr (SCORE == FLEX_SCORE_IDENTITY) mx *= p.c1;
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (partial && m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;

      float rowsum = 0.f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = SCORE == FLEX_SCORE_IDENTITY ? fmaf(s[b][r], p.c1, -m_use)
                                                       : s[b][r] - m_use;
          s[b][r] = __builtin_amdgcn_exp2f(x);
          rowsum += s[b][r];
        }
      l_run = l_run * alpha + rowsum;

#pragma unroll
      for (int e = 0; e < NE; ++e) o[e] *= alpha;
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kv = 32 * b + 16 * (r >> 3) + 8 * g + (r & 7);
            const float vv = *(__attribute__((address_space(3))) float*)(
                smem + base + TILE + kv * ROWBV + (32 * e + lq) * 4);
            o[e] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, s[b][r], o[e], 0, 0, 0);
          }

      if (has_next) {
        if constexpr (STAGES == 2) {
          stash((n + 1) & 1);
        } else {
          __syncthreads();  // everyone is done with the single buffer
          fetch(kb_next);
          stash(0);
        }
      }
      __syncthreads();
      kb_cur = kb_next;
    }

    // the running max is exact here, so the row max is m_run (base 2)
    const float l_tot = l_run + xor32(l_run);
    const bool live = p.safe_rows || l_tot > 0.f;
    float inv = live ? 1.0f / l_tot : 0.f;
    // document ids out of order: the builder poisoned every interval
    bool poison = false;
    if constexpr (MASK == FLEX_MASK_DOCUMENT) poison = doc_poisoned(lo, hi);
    if (poison) inv = opaque_nan();
    if (qi < p.q_len) {
      write_out_row<NE>(p, head_q + qi, DV, g, o, inv);
      if (p.lse != nullptr && g == 0)
        p.lse[head_q + qi] = poison ? opaque_nan()
                                    : live ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
      if (p.max_out != nullptr && g == 0) p.max_out[head_q + qi] = m_run * kLn2;
    }
  }
};

}  // namespace fwd
}  // namespace flexattn
