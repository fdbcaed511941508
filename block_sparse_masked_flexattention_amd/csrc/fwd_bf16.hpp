// fwd_bf16.hpp -- the bf16 forward kernel for gfx950 (CDNA4).
//
// What it computes is the FlexAttention forward: per Q_BLOCK rows of queries
// it walks the kv-blocks of the block mask (partial tiles first, then full
// tiles), forms S = scale * Q K^T, applies the score modification on every
// tile and the mask on partial tiles only, and takes the online-softmax step
// of forward_block_mn ("[Inductor][Flex Attention] Add Subtiling Option for
// Alpha Scaling", common.py.jinja hunk): running row max, alpha rescale of the
// accumulator and of the row sum, then acc += p V with p rounded to bf16 and
// the sum kept inside the matrix instruction ("Performance for templated
// attention strangely bad for a combination of causal + upper square mask",
// the acc = dot(p, v, acc) discussion).
//
// Mapping onto CDNA4:
//  * One work-group per (batch, head, q-block); each wave owns NQ sub-tiles
//    of 32 query rows.  Q stays in registers for the whole kernel.
//  * Both products run on v_mfma_f32_32x32x16_bf16.  The first is taken
//    transposed, S^T = K Q^T, so every lane owns one query row of each
//    sub-tile and half of that row's keys; the row max needs a single
//    v_permlane32_swap between the lane halves and the row sum nothing until
//    the epilogue.
//  * K rows sit in LDS with bits 2 and 3 of the row index swapped inside each
//    32-row group.  Then the eight S^T values a lane holds in accumulator
//    registers 8h..8h+7 of a 32-key block are eight consecutive keys: after
//    conversion to bf16 they are already the B operand of O^T = V^T P^T.
//  * V stays row-major in LDS; the V^T operand is read with
//    ds_read_b64_tr_b16, whose 16-lane transpose turns four 8-byte row
//    pieces into four keys of one column per lane.
//  * Both tiles are XOR-swizzled (K in 16-byte chunks, V in 8-byte units) so
//    that the wave's reads and writes hit distinct LDS banks.
//  * K and V move in steps of 64 keys (a 128-key block-mask tile is two
//    steps) through two LDS stage buffers.  The next step's tiles are loaded
//    straight from global memory into the other buffer with
//    global_load_lds_dwordx4 (no staging registers) while the current step
//    computes; one barrier per step.  The buffers are distinct LDS variables
//    and the step loop is unrolled by two, so the compiler can tell the
//    loads' destination from the buffer being read.
//  * Inside a step the keys go through in 32-key blocks (S^T, softmax, P V),
//    so only one block of scores is live and four waves fit on each SIMD;
//    the waves' matrix and vector work interleave on the SIMD.  (Issuing the
//    next block's S^T products ahead of the current softmax was measured
//    slower: its extra live registers either drop a wave per SIMD or spill.)
//  * Scores live in base-2 units (scale * log2 e folded into one FMA) and go
//    through v_exp_f32.  The running max used for exponentiation is only
//    raised when a row's max exceeds it by more than 2^8 (probabilities then
//    stay <= 256, exact in bf16's exponent range), so the accumulator rescale
//    runs only on tiles where some row of the wave needs it; the final
//    out = acc / l and lse = m + log2 l use that same max, so the result is
//    the softmax of the scores up to rounding.
//  * For every supported mask kind the keys a query row sees form one
//    interval; it is computed once per row (the q-side predicate hoisted out
//    of the key loop, as the templated-attention performance issue did by
//    hand), and a partial tile then costs one or two integer compares per
//    score.
#pragma once
#include "fwd_common.hpp"

namespace flexattn {
namespace fwd {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;
#define FLEXATTN_LDS(T, ptr) (*(__attribute__((address_space(3))) T*)(ptr))

// Query sub-tiles of 32 rows per wave.  Two sub-tiles halve the LDS reads
// per FLOP but need about twice the registers; on the 4096-long
// prefix-or-causal workload one sub-tile per wave (more waves in flight) was
// measured faster, 565 vs 467 TFLOP/s.
template <int D, int QB, int KB>
constexpr int bf16_nq() {
#ifdef FLEXATTN_NQ
  return (QB % (32 * FLEXATTN_NQ) == 0) ? FLEXATTN_NQ : 1;
#else
  return 1;
#endif
}

template <int V>
struct Int {
  static constexpr int value = V;
};

template <int D, int QB, int KB, int MASK, int SCORE, bool SUB>
struct Bf16Fwd {
  static constexpr int NQ = bf16_nq<D, QB, KB>();
  static constexpr int NW = QB / (32 * NQ);  // waves per work-group
  static constexpr int NT = 64 * NW;         // threads per work-group
  static constexpr int KS = 64;              // keys per step (one LDS stage)
  static constexpr int SPT = KB / KS;        // steps per block-mask tile
  static constexpr int NBS = KS / 32;        // 32-key blocks per step
  static constexpr int NE = D / 32;          // 32-column blocks of the head dim
  static constexpr int ROWB = D * 2;         // bytes per K / V row
  static constexpr int STAGE = KS * ROWB;    // bytes of K (or V) per step
  static constexpr int CPR = ROWB / 16;      // 16-byte chunks per row
  static constexpr int NDMA = KS * CPR / (64 * NW);  // 16-byte loads per lane per step (K or V)
  static constexpr float TAU = 8.0f;         // lazy-rescale threshold (log2 units)
  // Occupancy the register allocation aims for, in waves per SIMD: 4 for
  // head dim 64 (<= 128 VGPRs), 2 for 128, and never more than the LDS
  // allows (two stage buffers of K and V per work-group, 160 KiB per CU).
  static constexpr int LDS_WAVES = (kLdsBytes / (4 * STAGE)) * NW / 4;
  static constexpr int REG_WAVES = D == 64 ? 4 : 2;
  static constexpr int WAVES_PER_SIMD =
      LDS_WAVES < 1 ? 1 : (LDS_WAVES < REG_WAVES ? LDS_WAVES : REG_WAVES);
  static_assert(KB % KS == 0 && NDMA * 64 * NW == KS * CPR, "step split");
  static_assert(D == 64 || D == 128, "head dim");

  // K: row m, 16-byte chunk c at chunk c ^ kswz(m)
  __device__ static inline int kswz(int m) {
    return D == 64 ? ((m & 7) ^ ((m >> 3) & 1)) : (m & 15);
  }
  // V: row r, 8-byte unit u at unit u ^ vswz(r) (even, so 16-byte pieces stay whole)
  __device__ static inline int vswz(int r) {
    return D == 64 ? ((4 * (r & 1)) ^ (8 * ((r >> 1) & 1)))
                   : ((8 * (r & 1)) ^ (20 * ((r >> 1) & 1)));
  }

  __device__ static void run(const FwdParams& p) {
    __shared__ __attribute__((aligned(16))) char sbuf0[2 * STAGE];
    __shared__ __attribute__((aligned(16))) char sbuf1[2 * STAGE];
    lds_t* const buf[2] = {(lds_t*)sbuf0, (lds_t*)sbuf1};
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, g = lane >> 5;

    int bh, qb;
    wg_to_tile(p.n_qb, bh, qb);
    const int h = bh % p.H;
    const int q0 = qb * QB;
    const bool q_ragged = q0 + QB > p.q_len;

    const size_t head_q = (size_t)bh * p.q_len;
    const size_t head_kv = (size_t)bh * p.kv_len;
    const char* qg = static_cast<const char*>(p.q) + head_q * ROWB;
    const char* kg = static_cast<const char*>(p.k) + head_kv * ROWB;
    const char* vg = static_cast<const char*>(p.v) + head_kv * ROWB;

    // ---- per-lane constant offsets ----
    // K fragment reads: row 32b + lq, chunk 2t + g (kswz depends on lq only)
    int kro[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) kro[t] = lq * ROWB + (((2 * t + g) ^ kswz(lq)) << 4);
    // V^T fragment reads (transposing): in each 16-lane group lane j points
    // at row (.. + 4 t2 + j / 4), unit 8e + 4u + (j & 3)
    int vro[NE];
    {
      const int j = lane & 15, u = (lane >> 4) & 1;
      const int r0 = 8 * g + (j >> 2);
#pragma unroll
      for (int e = 0; e < NE; ++e)
        vro[e] = STAGE + r0 * ROWB + (((8 * e + 4 * u + (j & 3)) ^ vswz(r0)) << 3);
    }

    // ---- Q fragments: B operand of S^T = K Q^T ----
    int qi[NQ];
    u32x4 qf[NQ][D / 16];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      qi[c] = q0 + (wave * NQ + c) * 32 + lq;
      const bool ok = qi[c] < p.q_len;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        qf[c][t] = ok ? ld_global16(qg + (size_t)qi[c] * ROWB + (2 * t + g) * 16)
                      : u32x4{0, 0, 0, 0};
        if (p.neg_q) qf[c][t] ^= 0x80008000u;
      }
    }

    // ---- per-row visible key interval [lo, hi] ----
    int lo[NQ], hi[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) row_interval<MASK>(p, qi[c], lo[c], hi[c]);

    float nsl2 = 0.f;  // -slope_h * log2(e)
    if constexpr (SCORE == FLEX_SCORE_REL_BIAS)
      nsl2 = -exp2f(-p.bias_max * (float)(h + 1) / (float)p.H) * kLog2e;
    const float c1 = p.c1;

    // ---- step list: tile n / SPT, part n % SPT ----
    const int nk = p.n_kb;
    const int np = min(max(p.kv_num[qb], 0), nk);
    const int nf = min(max(p.fkv_num[qb], 0), nk);
    const int nsteps = (np + nf) * SPT;
    // the index rows are read-only for the kernel's lifetime: reading them
    // through the constant address space makes the loads scalar (s_load via
    // the scalar cache) rather than a vector load waited on at once
    typedef __attribute__((address_space(4))) const int32_t cint32;
    const cint32* prow = (const cint32*)(p.kv_idx + (size_t)qb * nk);
    const cint32* frow = (const cint32*)(p.fkv_idx + (size_t)qb * nk);
    auto tile_kb = [&](int t) {
      const int v = t < np ? prow[t] : frow[t - np];
      return min(max(v, 0), nk - 1);
    };

    // Load step (kb, part) into a stage buffer: K and V, 16 bytes per lane
    // per instruction straight into LDS.  The instruction's LDS slot for lane
    // i is fixed (base + 16 i), so the swizzle is applied on the global side:
    // slot s = (row m, position q) receives K row swap23(m), chunk q ^ kswz(m)
    // and V row m, chunk q ^ vswz(m) / 2.  Rows past the end of the keys are
    // clamped to the last key; the mask gives them zero weight.
    auto dma = [&](lds_t* dst, int kb, int part) {
      // a step may start past the last key (second half of a short ragged
      // tile): then every row reads the last key
      const int kv0 = min(kb * KB + part * KS, p.kv_len - 1);
      const int rows_left = min(KS, p.kv_len - kv0);  // >= 1
      const char* kt = kg + (size_t)kv0 * ROWB;
      const char* vt = vg + (size_t)kv0 * ROWB;
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        const int sl = (wave * NDMA + j) * 64 + lane;
        const int m = sl / CPR, q = sl % CPR;
        const int mk = min((m & ~31) | swap23(m & 31), rows_left - 1);
        const int mv = min(m, rows_left - 1);
        // 32-bit unsigned offsets from a uniform base: the SGPR-base form
        const unsigned ko = (unsigned)(mk * ROWB) + ((unsigned)(q ^ kswz(m)) << 4);
        const unsigned vo = (unsigned)(mv * ROWB) + ((unsigned)(q ^ (vswz(m) >> 1)) << 4);
        __builtin_amdgcn_global_load_lds(kt + ko,
                                         (__attribute__((address_space(3))) void*)(
                                             dst + (wave * NDMA + j) * 1024),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + vo,
                                         (__attribute__((address_space(3))) void*)(
                                             dst + STAGE + (wave * NDMA + j) * 1024),
                                         16, 0, 0);
      }
    };

    float m_run[NQ], l_run[NQ];
    f32x16 o[NQ][NE];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      m_run[c] = -INFINITY;
      l_run[c] = 0.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) o[c][e] = f32x16{};
    }

    // S^T block b (32 keys) of the step in `cur`, for every query sub-tile
    auto s_block = [&](const lds_t* cur, int b, f32x16 (&s)[NQ]) {
      u32x4 kf[D / 16];  // all K fragments of the block in flight at once
#pragma unroll
      for (int t = 0; t < D / 16; ++t) kf[t] = FLEXATTN_LDS(u32x4, cur + kro[t] + 32 * b * ROWB);
#pragma unroll
      for (int c = 0; c < NQ; ++c) s[c] = f32x16{};
#pragma unroll
      for (int t = 0; t < D / 16; ++t)
#pragma unroll
        for (int c = 0; c < NQ; ++c)
          s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, kf[t]), __builtin_bit_cast(bf16x8, qf[c][t]), s[c],
              0, 0, 0);
    };
    // V^T fragments of block b, half hh, column block e (two transposing reads)
    auto v_frag = [&](const lds_t* cur, int b, int hh, int e) {
      const lds_t* vp = cur + vro[e] + (32 * b + 16 * hh) * ROWB;
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)vp);
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vp + 4 * ROWB));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // One step: everything reads buf[BUF]; the next step is loaded into the
    // other buffer meanwhile.  Tile indices are fetched one tile ahead of
    // their use so that their load latency hides behind a whole tile.
    const int ntiles = np + nf;
    int kb_cur = 0, kb_nxt = 0;
    auto step = [&](auto buf_tag, int n) {
      constexpr int BUF = decltype(buf_tag)::value;
      lds_t* cur = buf[BUF];
      const int t = n / SPT, part = n % SPT;
      const int kv0 = kb_cur * KB + part * KS;
      // a listed-full tile at a ragged edge is still handled as partial
      const bool partial = t < np || q_ragged || kb_cur * KB + KB > p.kv_len;
      const bool last_part = part == SPT - 1;
      if (n + 1 < nsteps) dma(buf[BUF ^ 1], last_part ? kb_nxt : kb_cur, (n + 1) % SPT);
      int kb_after = kb_nxt;
      if (last_part && t + 2 < ntiles) kb_after = tile_kb(t + 2);

#pragma unroll
      for (int b = 0; b < NBS; ++b) {
        // On a partial tile, skip a 32-key block that no row of this wave
        // sees: its scores would all be -inf, i.e. weight exactly 0 and no
        // change to the running max.  (Diagonal tiles of a causal mask and
        // the window edges are mostly such blocks.)
        if (partial) {
          const int b0 = kv0 + 32 * b;
          bool any = false;
#pragma unroll
          for (int c = 0; c < NQ; ++c) any |= lo[c] <= b0 + 31 && hi[c] >= b0 && lo[c] <= hi[c];
          if (!__any(any)) continue;
        }
        f32x16 s[NQ];
        s_block(cur, b, s);

        // score modification, mask and running max; register r holds key
        // kv0 + 32b + 8g + 16(r >> 3) + (r & 7)
        const int kvl = kv0 + 32 * b + 8 * g;
        float alpha[NQ];
        bool need_any = false;
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          if constexpr (SCORE == FLEX_SCORE_REL_BIAS) {
            const float bias0 = nsl2 * (float)(qi[c] - kvl);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = 16 * (r >> 3) + (r & 7);
              s[c][r] = fmaf(s[c][r], c1, fmaf(-nsl2, (float)off, bias0));
            }
          }
          if (partial) {
            const int lim_hi = hi[c] - kvl, lim_lo = lo[c] - kvl;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = 16 * (r >> 3) + (r & 7);
              bool vis = off <= lim_hi;
              if constexpr (MASK == FLEX_MASK_SLIDING_WINDOW) vis = vis && off >= lim_lo;
              s[c][r] = vis ? s[c][r] : -INFINITY;
            }
          }
          // 16-way max as a v_max3 tree: 8 instructions, depth 3
          const float t0 = max3(s[c][0], s[c][1], s[c][2]);
          const float t1 = max3(s[c][3], s[c][4], s[c][5]);
          const float t2 = max3(s[c][6], s[c][7], s[c][8]);
          const float t3 = max3(s[c][9], s[c][10], s[c][11]);
          const float t4 = max3(s[c][12], s[c][13], s[c][14]);
          float mx = fmaxf(max3(t0, t1, t2), max3(t3, t4, s[c][15]));
          mx = max_halves(mx);
          if constexpr (SCORE == FLEX_SCORE_IDENTITY) mx *= c1;
          // raise the running max only when this block's max exceeds it by
          // more than TAU; alpha is exactly 1 otherwise (also at -inf)
          const bool need = mx > m_run[c] + TAU;
          alpha[c] = need ? __builtin_amdgcn_exp2f(m_run[c] - mx) : 1.0f;
          if (need) m_run[c] = mx;
          need_any |= need;
        }
        const bool rescale = __any(need_any);  // wave-uniform

        // the block's V^T fragments go out before the exponentials
        bf16x8 vf[NE][2];
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) vf[e][hh] = v_frag(cur, b, hh, e);

        bf16x8 pk[NQ][2];
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          // rows with nothing visible yet keep m = -inf; exponentiate against 0
          const float m_use = (partial && m_run[c] == -INFINITY) ? 0.f : m_run[c];
          float pv[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if constexpr (SCORE == FLEX_SCORE_IDENTITY)
              pv[r] = __builtin_amdgcn_exp2f(fmaf(s[c][r], c1, -m_use));
            else
              pv[r] = __builtin_amdgcn_exp2f(s[c][r] - m_use);
          }
          float rowsum = pv[0];  // fp32 sum: the LSE needs ~1e-4 relative accuracy
#pragma unroll
          for (int r = 1; r < 16; ++r) rowsum += pv[r];
          l_run[c] = fmaf(l_run[c], alpha[c], rowsum);
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            unsigned w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              w[i] = __builtin_bit_cast(
                  unsigned, bf16x2{(__bf16)pv[8 * hh + 2 * i], (__bf16)pv[8 * hh + 2 * i + 1]});
            pk[c][hh] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
          }
        }

        // O^T += V^T P^T; the alpha rescale first (per D-half with SUB)
        constexpr int NHALF = (SUB && NE >= 2) ? 2 : 1;
        constexpr int EPH = NE / NHALF;
#pragma unroll
        for (int half = 0; half < NHALF; ++half) {
          if (rescale) {
#pragma unroll
            for (int c = 0; c < NQ; ++c)
#pragma unroll
              for (int e = half * EPH; e < (half + 1) * EPH; ++e) o[c][e] *= alpha[c];
          }
#pragma unroll
          for (int e = half * EPH; e < (half + 1) * EPH; ++e)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int c = 0; c < NQ; ++c)
                o[c][e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[e][hh], pk[c][hh],
                                                                  o[c][e], 0, 0, 0);
        }
      }
      __syncthreads();  // the next step's loads have landed; this buffer is free
      if (last_part) {
        kb_cur = kb_nxt;
        kb_nxt = kb_after;
      }
    };

    if (nsteps > 0) {
      kb_cur = tile_kb(0);
      if (ntiles > 1) kb_nxt = tile_kb(1);
      dma(buf[0], kb_cur, 0);
    }
    __syncthreads();
    for (int n = 0; n < nsteps; n += 2) {
      step(Int<0>(), n);
      if (n + 1 < nsteps) step(Int<1>(), n + 1);
    }

    // ---- epilogue: out = acc / l, lse = (m + log2 l) ln 2 ----
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      const float l_tot = l_run[c] + xor32(l_run[c]);
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      if (qi[c] < p.q_len) {
        write_out_row<NE>(p, head_q + qi[c], D, g, o[c], inv);
        if (p.lse != nullptr && g == 0)
          p.lse[head_q + qi[c]] =
              l_tot > 0.f ? (m_run[c] + log2f(l_tot)) * kLn2 : -INFINITY;
      }
    }
  }
};

#undef FLEXATTN_LDS

}  // namespace fwd
}  // namespace flexattn
