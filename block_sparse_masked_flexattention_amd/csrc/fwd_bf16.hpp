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
//    through v_exp_f32.  Probabilities are taken against a per-row offset m
//    that may lag the row max: a block first exponentiates against the
//    current m and sums; only when some lane's sum exceeds 2^16 (a score rose
//    by more than 16 above m) or a row meets its first visible key does the
//    wave take the slow path, recompute the block's scores, raise m to the
//    block max, rescale the accumulator and row sum by alpha and
//    exponentiate again.  Most blocks thus cost no max reduction and no
//    rescale; out = acc / l and lse = m + log2 l use the same m, so the
//    result is the softmax of the scores up to rounding.
//  * The relative-position bias is linear in q - kv, so it enters as the
//    initial value of the S^T accumulators (two chains of adds of a uniform
//    step) and costs nothing per score after the product.
//  * s_setprio raises the wave's issue priority while it issues matrix
//    instructions, so a wave ready for the matrix unit goes ahead of the
//    other waves' vector work.
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

template <int V>
struct Int {
  static constexpr int value = V;
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// XMAX: the row max is an output (OUTPUT_MAX), so every block takes the
// exact running-max update of forward_block_mn instead of the lagging offset.
// DV: the value head dim (V_HEAD_DIM of the pages' kernel), which may differ
// from the query / key head dim D.
template <int D, int DV, int QB, int KB, int MASK, int SCORE, bool SUB, bool XMAX>
struct Bf16Fwd {
  // One 32-row query sub-tile per wave.  (Two sub-tiles per wave halve the
  // LDS reads per FLOP but need about twice the registers; on the 4096-long
  // prefix-or-causal workload one sub-tile per wave, with more waves in
  // flight, measured faster: 565 vs 467 TFLOP/s.)
  static constexpr int NQ = 1;
  static constexpr int NW = QB / (32 * NQ);  // waves per work-group
  static constexpr int NT = 64 * NW;         // threads per work-group
  // Keys per step (one LDS stage buffer) and stage buffers: a step's K and V
  // arrive one step ahead of their use.  (Three or four buffers, with 32- or
  // 64-key steps, measured flat or slower: at head dim 64 a third buffer
  // costs a work-group per CU.)
  static constexpr int KS = 64;
  static constexpr int NSTAGE = 2;
  static constexpr int SPT = KB / KS;        // steps per block-mask tile
  static constexpr int NBS = KS / 32;        // 32-key blocks per step
  static constexpr int NE = DV / 32;         // 32-column blocks of the value head dim
  static constexpr int ROWB = D * 2;         // bytes per K row
  static constexpr int ROWBV = DV * 2;       // bytes per V row
  static constexpr int STAGE = KS * ROWB;    // bytes of K per step (V follows at STAGE)
  static constexpr int STAGEV = KS * ROWBV;  // bytes of V per step
  static constexpr int CPR = ROWB / 16;      // 16-byte chunks per K row
  static constexpr int CPRV = ROWBV / 16;    // 16-byte chunks per V row
  static constexpr int NDMA = KS * CPR / (64 * NW);    // 16-byte K loads per lane per step
  static constexpr int NDMAV = KS * CPRV / (64 * NW);  // 16-byte V loads per lane per step
  // Probabilities are taken against a running offset that may lag the row
  // max; a block whose probabilities would exceed kPMax raises it.
  static constexpr float kPMax = 65536.0f;
  // Occupancy the register allocation aims for, in waves per SIMD: 4 for
  // head dim 64 (<= 128 VGPRs), 2 for 128, and never more than the LDS
  // allows (NSTAGE stage buffers of K and V per work-group, 160 KiB per CU).
  static constexpr int LDS_WAVES = (kLdsBytes / (NSTAGE * (STAGE + STAGEV))) * NW / 4;
  static constexpr int REG_WAVES = (D == 64 && DV == 64) ? 4 : 2;
  static constexpr int WAVES_PER_SIMD =
      LDS_WAVES < 1 ? 1 : (LDS_WAVES < REG_WAVES ? LDS_WAVES : REG_WAVES);
  static_assert(KB % KS == 0 && NDMA * 64 * NW == KS * CPR, "step split");
  static_assert(NDMAV * 64 * NW == KS * CPRV, "step split (V)");
  static_assert(D == 64 || D == 128, "head dim");
  static_assert((NW & (NW - 1)) == 0, "row-group rotation");
  static_assert((STAGE + STAGEV) % (16 * NT) == 0, "stage fill");
  static_assert(DV == 64 || DV == 128, "value head dim");

  // K: row m, 16-byte chunk c at chunk c ^ kswz(m)
  __device__ static inline int kswz(int m) {
    return D == 64 ? ((m & 7) ^ ((m >> 3) & 1)) : (m & 15);
  }
  // V: row r, 8-byte unit u at unit u ^ vswz(r) (even, so 16-byte pieces stay whole)
  __device__ static inline int vswz(int r) {
    return DV == 64 ? ((4 * (r & 1)) ^ (8 * ((r >> 1) & 1)))
                    : ((8 * (r & 1)) ^ (20 * ((r >> 1) & 1)));
  }

  // pairwise sum of 16 values (depth 4)
  __device__ static inline float sum16(const float (&x)[16]) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = x[2 * i] + x[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = a[2 * i] + a[2 * i + 1];
    return (a[0] + a[1]) + (a[2] + a[3]);
  }

  // End of a step: this wave's loads of the next step are complete, then
  // the work-group barrier (every wave's part of the next step is in LDS and
  // every wave is done reading the buffer the next step's loads overwrite).
  // The empty asm statements keep the compiler from moving memory accesses
  // across the barrier.
  __device__ static inline void step_barrier() {
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // Debugging (lds_poison): fill a stage buffer with NaN (all-ones bf16),
  // then the work-group barrier, so that the fill lands before the loads
  // that refill the buffer are issued.  A step that read a buffer before its
  // loads landed, or after the next step's loads began to overwrite it,
  // would then see NaN instead of plausible stale values.
  // (The thread index and the fill value are rebuilt here behind empty asm
  // statements, so that nothing of this rarely taken path is hoisted into
  // registers that stay live through the step loop.)
  __device__ static inline void poison_stage(lds_t* b) {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    unsigned ones = ~0u;
    asm volatile("" : "+v"(ones));
#pragma unroll
    for (int i = 0; i < (STAGE + STAGEV) / (16 * NT); ++i)
      FLEXATTN_LDS(u32x4, b + 16 * (t + i * NT)) = u32x4{ones, ones, ones, ones};
  }

  __device__ static void run(const FwdParams& p) {
    // one distinct LDS variable per stage buffer
    __shared__ __attribute__((aligned(16))) char sb0[STAGE + STAGEV];
    __shared__ __attribute__((aligned(16))) char sb1[STAGE + STAGEV];
    lds_t* const buf[2] = {(lds_t*)sb0, (lds_t*)sb1};
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, g = lane >> 5;

    int bh, qb;
    wg_to_tile(p.n_qb, bh, qb);
    const int h = bh % p.H;
    // this wave's 32 rows of the q-block: rotated under the sliding window,
    // where every q-block has the same uneven per-step block counts (under
    // the prefix-or-causal mask the rotation measured about 1% slower)
    const int rw = MASK == FLEX_MASK_SLIDING_WINDOW ? row_group(wave, NW) : wave;
    const int q0 = qb * QB;
    const bool q_ragged = q0 + QB > p.q_len;

    const size_t head_q = (size_t)bh * p.q_len;
    const size_t head_kv = (size_t)bh * p.kv_len;
    const char* qg = static_cast<const char*>(p.q) + head_q * ROWB;
    const char* kg = static_cast<const char*>(p.k) + head_kv * ROWB;
    const char* vg = static_cast<const char*>(p.v) + head_kv * ROWBV;

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
        vro[e] = STAGE + r0 * ROWBV + (((8 * e + 4 * u + (j & 3)) ^ vswz(r0)) << 3);
    }

    // ---- tile list (read first: the first step's loads wait for it, the
    // Q loads below do not): partial tiles, then full tiles, each list walked
    // from its last entry down.  Lists are ascending, so under causal-type
    // masks the nearest keys (the diagonal, the largest scores under a
    // decaying bias) come first, which keeps the lagging offset from being
    // raised again later; and under a sliding window every wave meets its
    // first visible keys in the same step, so the slow-path blocks of the
    // four waves overlap instead of following one another.  (Walking the
    // full tiles upwards instead, so that the q-blocks of a head that run
    // together would read key block 0 first at about the same time, measured
    // 1.5 times the HBM reads on the 4096-long prefix workload: descending,
    // q-block i + 1 reads each tile two steps before q-block i does, a short
    // and steady reuse distance.) ----
    const int nk = p.n_kb;
    const int np = min(max(p.kv_num[qb], 0), nk);
    const int nf = min(max(p.fkv_num[qb], 0), nk);
    const int ntiles = np + nf;
    const int nsteps = ntiles * SPT;
    const int32_t* prow = p.kv_idx + (size_t)qb * nk;
    const int32_t* frow = p.fkv_idx + (size_t)qb * nk;
    // Tile indices 64 at a time: lane i of `win` holds the kv-block of tile
    // win_base + i, lane i of `win_nx` that of tile win_base + 64 + i; a
    // tile's index is then one v_readlane.  The next window is loaded 64
    // tiles ahead of its use.
    auto load_window = [&](int base) {  // raw values; clamped when read
      // (one load per lane from inside the index rows whatever the count,
      // with no branch around it, so that the wait for it can leave the Q
      // loads issued after it in flight.  With no kv-blocks at all the index
      // rows are empty: the lane reads the q-block's count instead, a value
      // never used.)
      const int t = max(min(base + lane, ntiles - 1), 0);
      const bool in_p = t < np;
      const int j = in_p ? np - 1 - t : ntiles - 1 - t;  // entry of its list
      const int32_t* src = (in_p ? prow : frow) + (p.contig ? 0 : max(j, 0));
      const int v = *(nk > 0 ? src : p.kv_num + qb);
      return p.contig ? v + j : v;  // a contiguous list is first, first + 1, ...
    };
    int win_base = 0;
    int win = load_window(0);
    int win_nx = load_window(64);
    auto tile_kb = [&](int t) {  // t in [win_base, win_base + 128)
      const int i = t - win_base;
      const int v = i < 64 ? __builtin_amdgcn_readlane(win, i)
                           : __builtin_amdgcn_readlane(win_nx, i - 64);
      return min(max(v, 0), nk - 1);
    };

    // ---- Q fragments: B operand of S^T = K Q^T ----
    // q times -1 (negative scale) or scale * log2 e (PRESCALE_QK); times 1
    // otherwise.  Both signs and 1 are exact in bf16.
    const float qmul = p.prescale ? p.qscale : (p.neg_q ? -1.0f : 1.0f);
    int qi[NQ];
    u32x4 qf[NQ][D / 16];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      qi[c] = q0 + (rw * NQ + c) * 32 + lq;
      // rows past the end load the last row (zeroed below): no branch
      // around the loads
      const int qr = min(qi[c], p.q_len - 1);
#pragma unroll
      for (int t = 0; t < D / 16; ++t)
        qf[c][t] = ld_global16(qg + (size_t)qr * ROWB + (2 * t + g) * 16);
    }

    // ---- per-row visible key interval [lo, hi] ----
    int lo[NQ], hi[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) row_interval<MASK>(p, qi[c], lo[c], hi[c]);
    // the same ends and the row index less 8 g: a block's key offsets then
    // come from its first key kb0 alone, a wave-uniform value
    int lo_g[NQ], hi_g[NQ], qi_g[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      lo_g[c] = lo[c] - 8 * g;
      hi_g[c] = hi[c] - 8 * g;
      qi_g[c] = qi[c] - 8 * g;
    }

    const float c1 = p.c1;
    // Relative bias -slope_h (q - kv) in units of the raw score (c1 s + bias
    // in base 2 = c1 (s + bias / (|scale| ln 2 log2 e))): bias_u per unit
    // of q - kv.
    float bias_u = 0.f, bias_u16 = 0.f;
    if constexpr (SCORE == FLEX_SCORE_REL_BIAS) {
      bias_u = -head_slope(p, h) / (p.c1 * kLn2);
      bias_u16 = 16.0f * bias_u;
    }

    // Load step m into a stage buffer: K and V, 16 bytes per lane per
    // instruction straight into LDS.  The instruction's LDS slot for lane i
    // is fixed (base + 16 i), so the swizzle is applied on the global side:
    // slot s = (row r, position q) receives K row swap23(r), chunk
    // q ^ kswz(r) and V row r, chunk q ^ vswz(r) / 2.  The loads go through
    // buffer resources based at the step's first key whose size is the rows
    // that exist, so the per-lane offsets are the same for every step (set
    // once here) and rows past the end of the keys read as zero, with no
    // per-step clamp; the mask gives those keys zero weight.
    unsigned ko[NDMA], vo[NDMAV];
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int sl = (wave * NDMA + j) * 64 + lane;
      const int r = sl / CPR, q = sl % CPR;
      ko[j] = (unsigned)((((r & ~31) | swap23(r & 31))) * ROWB) + ((unsigned)(q ^ kswz(r)) << 4);
    }
#pragma unroll
    for (int j = 0; j < NDMAV; ++j) {
      const int sl = (wave * NDMAV + j) * 64 + lane;
      const int r = sl / CPRV, q = sl % CPRV;
      vo[j] = (unsigned)(r * ROWBV) + ((unsigned)(q ^ (vswz(r) >> 1)) << 4);
    }
    auto dma = [&](lds_t* dst, int m) {
      const int kb = tile_kb(m / SPT);
      // the second step of a short ragged tile may start past the last key:
      // then no row exists and every row reads as zero
      const int kv0 = kb * KB + (m % SPT) * KS;
      // (uniform; readfirstlane keeps the resource words in scalar
      // registers)
      const int rows = __builtin_amdgcn_readfirstlane(max(min(KS, p.kv_len - kv0), 0));
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(kg + (size_t)kv0 * ROWB), 0, rows * ROWB, kBufferRsrcWord3);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(vg + (size_t)kv0 * ROWBV), 0, rows * ROWBV, kBufferRsrcWord3);
      // (K and V loads alternate while both have one left: the same order
      // as one loop over both when the row widths match)
#pragma unroll
      for (int j = 0; j < (NDMA > NDMAV ? NDMA : NDMAV); ++j) {
        if (j < NDMA)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              kr, (__attribute__((address_space(3))) void*)(dst + (wave * NDMA + j) * 1024), 16,
              (int)ko[j], 0, 0, 0);
        if (j < NDMAV)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              vr, (__attribute__((address_space(3))) void*)(dst + STAGE + (wave * NDMAV + j) * 1024),
              16, (int)vo[j], 0, 0, 0);
      }
    };

    // Running state per query row: m_run is the offset the probabilities
    // are taken against (a lower bound of the row max, in base-2 units),
    // nm = -m_run (+inf before the row's first visible key), l_run the sum
    // of probabilities (per lane half), o the output accumulator.
    float m_run[NQ], nm[NQ], l_run[NQ];
    f32x16 o[NQ][NE];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      m_run[c] = -INFINITY;
      nm[c] = INFINITY;
      l_run[c] = 0.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) o[c][e] = f32x16{};
    }

    // S^T block b (32 keys) of the step in `cur`, for every query sub-tile,
    // keys from kb0 on (register r of lane half g: key
    // kb0 + 8 g + 16(r >> 3) + (r & 7)).  With
    // the relative bias the accumulators start at bias / c1, so that the
    // product leaves c1 s + bias in one FMA, as for the plain score.
    auto s_block = [&](const lds_t* cur, int b, int kb0, f32x16 (&s)[NQ]) {
      u32x4 kf[D / 16];  // all K fragments of the block in flight at once
#pragma unroll
      for (int t = 0; t < D / 16; ++t) kf[t] = FLEXATTN_LDS(u32x4, cur + kro[t] + 32 * b * ROWB);
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
        if constexpr (SCORE == FLEX_SCORE_REL_BIAS) {
          // bias_u (q - kv) for keys kb0 + 8 g + r and 16 more, r < 8, as two
          // chains of -bias_u steps (no per-register constants).  The empty
          // asm statement keeps the compiler from carrying one call's values
          // over to the next call in registers.
          float a = bias_u * (float)(qi_g[c] - kb0);
          asm volatile("" : "+v"(a));
          float x = a, y = a - bias_u16;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            s[c][r] = x;
            s[c][8 + r] = y;
            x -= bias_u;
            y -= bias_u;
          }
        } else {
          s[c] = f32x16{};
        }
      }
      __builtin_amdgcn_s_setprio(1);  // keep the matrix unit fed first
#pragma unroll
      for (int t = 0; t < D / 16; ++t)
#pragma unroll
        for (int c = 0; c < NQ; ++c)
          s[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, kf[t]), __builtin_bit_cast(bf16x8, qf[c][t]), s[c],
              0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    };
    // V^T fragments of block b, half hh, column block e (two transposing reads)
    auto v_frag = [&](const lds_t* cur, int b, int hh, int e) {
      const lds_t* vp = cur + vro[e] + (32 * b + 16 * hh) * ROWBV;
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)vp);
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vp + 4 * ROWBV));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // p = 2^(c1 s + offset)
    auto exp_score = [&](float sc, float nmc) { return __builtin_amdgcn_exp2f(fmaf(sc, c1, nmc)); };
    // set the keys row c does not see (partial tiles) to `fill`
    auto mask_block = [&](auto& x, int c, int kb0, float fill) {
      const int lim_hi = hi_g[c] - kb0, lim_lo = lo_g[c] - kb0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 16 * (r >> 3) + (r & 7);
        bool vis = off <= lim_hi;
        if constexpr (two_sided_mask<MASK>()) vis = vis && off >= lim_lo;
        x[r] = vis ? x[r] : fill;
      }
    };

    // One step: everything reads buf[B]; step n + 1 is loaded into the
    // other buffer (which step n - 1 used).
    auto step = [&](auto buf_tag, int n, auto exact_tag) {
      constexpr int B = decltype(buf_tag)::value;
      // EX: every block of this step takes the exact running-max update
      // (with XMAX always; otherwise on the first step, where no row has
      // met a key yet and the fast path could only fail)
      constexpr bool EX = XMAX || decltype(exact_tag)::value != 0;
      lds_t* cur = buf[B];
      const int t = n / SPT, part = n % SPT;
      if (t >= win_base + 64) {  // slide the index window
        win_base += 64;
        win = win_nx;
        if (win_base + 64 < ntiles) win_nx = load_window(win_base + 64);
      }
      const int kb = tile_kb(t);
      const int kv0 = kb * KB + part * KS;
      // a listed-full tile at a ragged edge is still handled as partial
      const bool partial = t < np || q_ragged || kb * KB + KB > p.kv_len;
      if (p.lds_poison) {  // (every wave is past the barrier that ended step n - 1)
        poison_stage(buf[B ^ 1]);
        __syncthreads();
      }
      if (n + 1 < nsteps) dma(buf[B ^ 1], n + 1);

#pragma unroll
      for (int b = 0; b < NBS; ++b) {
        // On a partial tile, skip a 32-key block that no row of this wave
        // sees: its scores would all be -inf, i.e. weight exactly 0 and no
        // change to the running max.  (Diagonal tiles of a causal mask and
        // the window edges are mostly such blocks.)  A block that every row
        // of the wave sees whole needs no mask either.
        bool masked = partial;
        if (partial) {
          const int b0 = kv0 + 32 * b;
          bool any = false, all = true;
#pragma unroll
          for (int c = 0; c < NQ; ++c) {
            any |= lo[c] <= b0 + 31 && hi[c] >= b0 && lo[c] <= hi[c];
            all = all && lo[c] <= b0 && hi[c] >= b0 + 31;
          }
          if (!__any(any)) continue;
          masked = !__all(all);
        }
        const int kb0 = kv0 + 32 * b;  // the block's first key
        f32x16 s[NQ];
        s_block(cur, b, kb0, s);

        // the block's V^T fragments go out before the exponentials
        bf16x8 vf[NE][2];
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) vf[e][hh] = v_frag(cur, b, hh, e);

        // Fast path: exponentiate against the stored offset, zero the masked
        // keys, and check that every probability stayed below kPMax (a row
        // that has not seen a key yet has offset +inf, so a visible key
        // gives +inf and fails the check).
        float pv[NQ][16], rs[NQ];
        bool bad = false;
        if constexpr (!EX) {
#pragma unroll
          for (int c = 0; c < NQ; ++c) {
#pragma unroll
            for (int r = 0; r < 16; ++r) pv[c][r] = exp_score(s[c][r], nm[c]);
            if (masked) mask_block(pv[c], c, kb0, 0.f);
            rs[c] = sum16(pv[c]);
            bad |= rs[c] > kPMax;
          }
        }
        float alpha[NQ];  // set and read only on the slow path
        const bool rescale = EX || __any(bad);  // wave-uniform
        // The mask flag again, recomputed rather than kept: carried through
        // the fast path it costs a copy through a vector register on every
        // block.  (The empty asm statement keeps the compiler from reusing
        // the first computation.)
        auto masked_again = [&]() {
          if constexpr (EX) return masked;
          int k0 = kb0;
          asm volatile("" : "+s"(k0));
          bool all = true;
#pragma unroll
          for (int c = 0; c < NQ; ++c) all = all && lo[c] <= k0 && hi[c] >= k0 + 31;
          return partial && !__all(all);
        };
        if (rescale) {
          // Slow path (a row's first visible keys, or scores that rose by
          // more than log2 kPMax; every block with XMAX): raise the running
          // max of every row of the wave to the block max, rescale by alpha
          // and exponentiate.  Coming from the fast path it first recomputes
          // the block's scores (the empty asm statement makes the compiler
          // read K from LDS again instead of keeping the fast path's
          // fragments live through it).
          if constexpr (!EX) {
            asm volatile("" ::: "memory");
            s_block(cur, b, kb0, s);
          }
#pragma unroll
          for (int c = 0; c < NQ; ++c) {
            if (masked_again()) mask_block(s[c], c, kb0, -INFINITY);
            // 16-way max as a v_max3 tree: 8 instructions, depth 3
            const float t0 = max3(s[c][0], s[c][1], s[c][2]);
            const float t1 = max3(s[c][3], s[c][4], s[c][5]);
            const float t2 = max3(s[c][6], s[c][7], s[c][8]);
            const float t3 = max3(s[c][9], s[c][10], s[c][11]);
            const float t4 = max3(s[c][12], s[c][13], s[c][14]);
            float mx = fmaxf(max3(t0, t1, t2), max3(t3, t4, s[c][15]));
            mx = max_halves(mx) * c1;
            const float m_new = fmaxf(m_run[c], mx);
            const bool seen = m_new != -INFINITY;
            // rows still at -inf keep alpha = 1 (their sum and output are 0)
            alpha[c] = seen ? __builtin_amdgcn_exp2f(m_run[c] - m_new) : 1.0f;
            l_run[c] *= alpha[c];
            m_run[c] = m_new;
            // masked scores are -inf here, so a finite offset zeroes them
            const float nm_now = seen ? -m_new : 0.f;
            nm[c] = seen ? -m_new : INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) pv[c][r] = exp_score(s[c][r], nm_now);
            rs[c] = sum16(pv[c]);
          }
        }

        bf16x8 pk[NQ][2];
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
          l_run[c] += rs[c];  // (rescaled by alpha in the slow path)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            unsigned w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              w[i] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)pv[c][8 * hh + 2 * i],
                                                         (__bf16)pv[c][8 * hh + 2 * i + 1]});
            pk[c][hh] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
          }
        }

        // O^T += V^T P^T; the alpha rescale first (per D-half with SUB)
        constexpr int NHALF = (SUB && NE >= 2) ? 2 : 1;
        constexpr int EPH = NE / NHALF;
        __builtin_amdgcn_s_setprio(1);
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
        __builtin_amdgcn_s_setprio(0);
      }
      step_barrier();
    };

    // prologue: step 0 in flight, then wait for it (the Q scaling, when
    // there is one, runs meanwhile)
    if (p.lds_poison) {
      poison_stage(buf[0]);
      poison_stage(buf[1]);
      __syncthreads();
    }
    if (nsteps > 0) dma(buf[0], 0);
    if (qmul != 1.0f || q_ragged) {
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
        const bool ok = qi[c] < p.q_len;
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
          qf[c][t] = ok ? scale_bf16x8(qf[c][t], qmul) : u32x4{0, 0, 0, 0};
      }
    }
    step_barrier();
    // pairs of steps, straight-line, then the remainder; the first step is
    // peeled off and takes the exact update: a row's first visible keys cost
    // one pass instead of a failed fast pass and a second one
    constexpr Int<0> FAST{};
    int n = 0;
    if (nsteps > 0) step(Int<0>(), 0, Int<1>());
    n = 1;
    for (; n + 2 <= nsteps; n += 2) {
      step(Int<1>(), n, FAST);
      step(Int<0>(), n + 1, FAST);
    }
    if (n < nsteps) step(Int<1>(), n, FAST);
    wait_vmcnt<0>();  // leave no load in flight behind the kernel

    // ---- epilogue: out = acc / l, lse = (m + log2 l) ln 2, max = m ln 2 ----
    // (with ROWS_GUARANTEED_SAFE the l = 0 guards are left out)
    // bf16 output goes through LDS: each wave writes its 32 rows into its
    // own region of the first stage buffer (free here: every wave is past
    // the last step barrier and no load is in flight, since each step's
    // barrier waits for all of its loads), then stores them as
    // whole 16-byte pieces, 64 lanes covering contiguous rows, instead of
    // 8-byte pieces scattered over 32 rows.
    constexpr int OROW = DV * 2;       // bytes per output row
    constexpr bool LDS_OUT = NQ == 1 && NW * 32 * OROW <= STAGE + STAGEV;
    const bool lds_out = LDS_OUT && p.out_bf16;
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      const float l_tot = l_run[c] + xor32(l_run[c]);
      const bool live = p.safe_rows || l_tot > 0.f;
      float inv = live ? 1.0f / l_tot : 0.f;
      // document ids out of order: the builder poisoned every interval
      bool poison = false;
      if constexpr (MASK == FLEX_MASK_DOCUMENT) poison = doc_poisoned(lo[c], hi[c]);
      if (poison) inv = opaque_nan();
      if (lds_out)
        store_rows_bf16_lds<NE>(buf[0] + wave * 32 * OROW,
                                static_cast<char*>(p.out) + (head_q + (size_t)(q0 + rw * 32)) * OROW,
                                p.q_len - (q0 + rw * 32), o[c], inv, lane);
      if (qi[c] < p.q_len) {
        if (!lds_out) write_out_row<NE>(p, head_q + qi[c], DV, g, o[c], inv);
        if (p.lse != nullptr && g == 0)
          p.lse[head_q + qi[c]] = poison ? opaque_nan()
                                         : live ? (m_run[c] + log2f(l_tot)) * kLn2 : -INFINITY;
        if constexpr (XMAX) {
          if (p.max_out != nullptr && g == 0) p.max_out[head_q + qi[c]] = m_run[c] * kLn2;
        }
      }
    }
  }
};

#undef FLEXATTN_LDS

}  // namespace fwd
}  // namespace flexattn
