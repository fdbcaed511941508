// bwd_bf16.hpp -- the backward pass (gradients of q, k and v) for bf16
// inputs on gfx950.
//
// What it computes is the derivative of the forward: the flex_attention
// backward higher-order op of "[Inductor][Flex Attention] Add Subtiling
// Option for Alpha Scaling" (test hunks) takes q, k, v, the forward output
// and log-sum-exp, the output gradient and a log-sum-exp gradient, and the
// block mask with its transposed q_num_blocks / q_indices / full_q_* arrays,
// and returns dq, dk and dv.  For every visible pair (i, j):
//   p_ij  = exp(s_ij - lse_i)
//   delta_i = <dout_i, out_i> - dlse_i
//   ds_ij = p_ij (<dout_i, v_j> - delta_i)
//   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
//   dv_j = sum_i p_ij dout_i.
// Three kernels:
//  * bwd_pre_kernel: per query row, -delta_i and a_i = -lse_i / |scale|
//    (the log-sum-exp in units of the raw score; -inf for a row that sees no
//    key), into the caller's workspace.
//  * Bf16BwdDq: one work-group per (batch, head, q-block), one wave per 32
//    query rows, walking the forward's tile list like the forward.  S^T and
//    dP^T = V dout^T are taken with K and V as the A operands and q, dout in
//    registers as B operands (lane = query row), p = 2^(c1 s + c1 a) needs no
//    row reduction, and dq^T += K^T ds^T reads K^T with the transposing LDS
//    read the forward uses for V^T.
//  * Bf16BwdDkv: one work-group per (batch, head, kv-block), one wave per 32
//    keys with that wave's K and V rows resident in registers as B operands
//    (lane = key), walking the transposed tile list in steps of 32 query
//    rows.  The S and dP accumulators start at a_i and -delta_i (read from
//    LDS straight into them), so p = 2^(c1 s) and ds = p dP; then
//    dv^T += dout^T p and dk^T += q^T ds read dout^T and q^T transposed.
// K, V, q and dout tiles sit in LDS in the forward's V layout with one more
// swizzle term (rows in order, 8-byte units XOR-swizzled by an even amount,
// so 16-byte pieces stay whole for the row reads; see vswz); a row read for
// an A operand takes row
// swap23(lane) so that accumulator registers 8h..8h+7 hold eight
// consecutive keys (queries), ready to be the next product's B operand.
#pragma once
#include "fwd_common.hpp"

namespace flexattn {
namespace bwd {

using fwd::bf16x2;
using fwd::bf16x4;
using fwd::bf16x8;
using fwd::f32x16;
using fwd::f32x4;
using fwd::u32x4;
using fwd::kLog2e;
using fwd::ld_global16;
using fwd::swap23;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;

template <int V>
struct Int {
  static constexpr int value = V;
};
#define FLEXATTN_LDS(T, ptr) (*(__attribute__((address_space(3))) T*)(ptr))

// Tile layout: row r, 8-byte unit u at unit u ^ vswz(r).  The backward reads
// its tiles two ways: transposing reads (ds_read_b64_tr_b16, rows r0 .. r0 + 3
// of a 4-row group at a time) and A-operand row reads (16 bytes per lane,
// rows swap23(lane)).  Bits 0 and 1 of the row (the forward's V swizzle)
// keep the transposing reads conflict-free; the term in bit 3 separates rows
// r and r + 8, which the row reads of one 16-lane group fetch together (with
// the forward's swizzle alone every such pair shared a bank).  Bank-conflict
// model checked on the host for 32 and 64 four-byte banks: the row reads
// drop from 48 to 16 extra cycles per 32-key block at head dim 64 (96 to 32
// at 128) with 64 banks and to none with 32; the transposing reads stay
// conflict-free.  The swizzle leaves bits 2, 4 and 5 alone, so the offsets
// of a group's second transposing read (4 rows on), of the second 16 rows
// and of the second 32-key block differ from the first by whole rows.
template <int D>
__device__ inline int vswz(int r) {
  return D == 64 ? ((4 * (r & 1)) ^ (8 * ((r >> 1) & 1)) ^ (2 * ((r >> 3) & 1)))
                 : ((8 * (r & 1)) ^ (20 * ((r >> 1) & 1)) ^ (2 * ((r >> 3) & 1)));
}

// The dk/dv kernel's q and dout tiles when both are 64 wide (FULL): a
// swizzle with a row-bit-2 term as well, conflict-free in the same model for
// both read patterns (32 or 64 banks).  The second transposing read of a
// 4-row group (rows r0 + 4 ..) then differs from the first in bit 2 only,
// which moves the 8-byte unit by 2: its offset is the first one's with bit 4
// flipped, plus 4 rows.  (Instances with a 128-wide tile keep vswz: their
// registers are already short and the variant spilled more.)
template <int D, bool FULL>
__device__ inline int vswz_q(int r) {
  return FULL ? (vswz<D>(r) ^ (2 * ((r >> 2) & 1)) ^ (4 * ((r >> 3) & 1))) : vswz<D>(r);
}

// Queries that see key kk, as one interval [lo, hi] (empty when lo > hi),
// clipped to the query range: the transpose of row_interval.
template <int MASK>
__device__ inline void col_interval(const BwdParams& p, int kk, int& lo, int& hi) {
  lo = 0;
  hi = p.q_len - 1;
  if (kk >= p.kv_len) {
    lo = 1;
    hi = 0;
    return;
  }
  if constexpr (MASK == FLEX_MASK_CAUSAL) {
    lo = kk;
  } else if constexpr (MASK == FLEX_MASK_SLIDING_WINDOW) {
    // window_min <= q - kk <= window, in 64 bits
    lo = (int)max(0LL, (long long)kk + p.window_min);
    hi = (int)min((long long)hi, (long long)kk + p.window);
  } else if constexpr (MASK == FLEX_MASK_PREFIX_CAUSAL) {
    // (q <= P and kk <= P) or q >= kk: every q when kk <= P
    lo = kk <= p.prefix ? 0 : kk;
  } else if constexpr (MASK == FLEX_MASK_DOCUMENT) {
    // the transposed builder's per-key interval (causal cut included)
    lo = p.col_bounds[2 * (size_t)kk];
    hi = p.col_bounds[2 * (size_t)kk + 1];
  }
}

__device__ inline void s_barrier_full() {
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Store one row of an accumulator transposed like the forward's O^T:
// register r of column block e holds column 32e + 8(r/4) + 4g + r%4.
template <int NE>
__device__ inline void write_row_t(void* base, bool bf16, size_t row, int D, int g,
                                   const f32x16 (&a)[NE], float f) {
  char* og = static_cast<char*>(base) + row * (size_t)D * (bf16 ? 2 : 4);
#pragma unroll
  for (int e = 0; e < NE; ++e)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * e + 8 * q + 4 * g;
      const float v0 = a[e][4 * q] * f, v1 = a[e][4 * q + 1] * f;
      const float v2 = a[e][4 * q + 2] * f, v3 = a[e][4 * q + 3] * f;
      if (bf16) {
        *reinterpret_cast<bf16x4*>(og + d * 2) =
            bf16x4{(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
      } else {
        *reinterpret_cast<f32x4*>(og + d * 4) = f32x4{v0, v1, v2, v3};
      }
    }
}

// bf16 B operands from 16 fp32 values: register 8h + 2i, 8h + 2i + 1 -> word i of pk[h]
__device__ inline void pack16(const float (&x)[16], bf16x8 (&pk)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    unsigned w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)x[8 * h + 2 * i], (__bf16)x[8 * h + 2 * i + 1]});
    pk[h] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
  }
}

// ---------------------------------------------------------------------------
// Per query row: ws[row] = -delta, ws[rows + row] = a.  DV / 8 lanes per row
// (DV the value head dim, the width of out and dout), each reading 8
// elements of out and dout.
// ---------------------------------------------------------------------------
template <int DV>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int LPR = DV / 8;
  const long long rows = (long long)p.B * p.H * p.q_len;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / LPR;
  const int part = (int)(t % LPR);
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = ld_global16(static_cast<const char*>(p.out) + (row * DV + part * 8) * 2);
    const u32x4 d = ld_global16(static_cast<const char*>(p.dout) + (row * DV + part * 8) * 2);
    const bf16x8 ob = __builtin_bit_cast(bf16x8, o), db = __builtin_bit_cast(bf16x8, d);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)ob[i], (float)db[i], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    const float delta = acc - (p.dlse != nullptr ? p.dlse[row] : 0.f);
    const float lse = p.lse[row];
    p.ws[row] = -delta;
    p.ws[rows + row] = lse == -INFINITY ? -INFINITY : -lse * p.inv_abs_scale;
  }
}

// ---------------------------------------------------------------------------
// dq
// ---------------------------------------------------------------------------
// D: head dim of q and k; DV: value head dim (width of v, out and dout)
template <int D, int DV, int QB, int KB, int MASK, int SCORE>
struct Bf16BwdDq {
  static constexpr int NW = QB / 32;
  static constexpr int NT = 64 * NW;
  static constexpr int KS = 64;             // keys per step
  static constexpr int SPT = KB / KS;
  static constexpr int NE = D / 32;
  static constexpr int ROWB = D * 2;        // bytes per K row
  static constexpr int ROWBV = DV * 2;      // bytes per V row
  static constexpr int STAGE = KS * ROWB;   // bytes of K per step (V follows)
  static constexpr int STAGEV = KS * ROWBV; // bytes of V per step
  static constexpr int CPR = ROWB / 16;
  static constexpr int CPRV = ROWBV / 16;
  static constexpr int NDMA = KS * CPR / (64 * NW);
  static constexpr int NDMAV = KS * CPRV / (64 * NW);
  // head dim 64: four waves per SIMD with 128-row tiles (128 VGPRs with 2-3
  // values spilled; 2-3% faster than three on the prefix and sliding-window
  // workloads), three with 64-row tiles, one fewer each when the dout rows
  // are 128 wide; head dim 128: two, or one with 64-row tiles (the two-wave
  // work-group's extra load addresses)
  static constexpr int WAVES_PER_SIMD =
      D == 64 ? (QB == 128 ? 4 : 3) - (DV == 64 ? 0 : 1) : (QB == 64 ? 1 : 2);
  static_assert(KB % KS == 0 && NDMA * 64 * NW == KS * CPR, "step split");
  static_assert(NDMAV * 64 * NW == KS * CPRV, "step split (V)");

  __device__ static void run(const BwdParams& p) {
    __shared__ __attribute__((aligned(16))) char sb0[STAGE + STAGEV];
    __shared__ __attribute__((aligned(16))) char sb1[STAGE + STAGEV];
    lds_t* const buf[2] = {(lds_t*)sb0, (lds_t*)sb1};
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, g = lane >> 5;

    int bh, qb;
    fwd::wg_to_tile(p.n_qb, bh, qb);
    const int h = bh % p.H;
    const int q0 = qb * QB;
    const bool q_ragged = q0 + QB > p.q_len;
    const long long rows = (long long)p.B * p.H * p.q_len;
    const size_t head_q = (size_t)bh * p.q_len;
    const char* qg = static_cast<const char*>(p.q) + head_q * ROWB;
    const char* dog = static_cast<const char*>(p.dout) + head_q * ROWBV;
    const char* kg = static_cast<const char*>(p.k) + (size_t)bh * p.kv_len * ROWB;
    const char* vg = static_cast<const char*>(p.v) + (size_t)bh * p.kv_len * ROWBV;

    // A-operand row reads: row swap23(lq), 16-byte piece 2t + g
    // (K rows D wide, V rows DV wide)
    const int ra = swap23(lq);
    int kra[D / 16], vra[DV / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      kra[t] = ra * ROWB + (((2 * t + g) ^ (vswz<D>(ra) >> 1)) << 4);
#pragma unroll
    for (int t = 0; t < DV / 16; ++t)
      vra[t] = ra * ROWBV + (((2 * t + g) ^ (vswz<DV>(ra) >> 1)) << 4);
    // transposing reads (the forward's V^T fragment offsets)
    int tro[NE];
    {
      const int j = lane & 15, u = (lane >> 4) & 1;
      const int r0 = 8 * g + (j >> 2);
#pragma unroll
      for (int e = 0; e < NE; ++e) tro[e] = r0 * ROWB + (((8 * e + 4 * u + (j & 3)) ^ vswz<D>(r0)) << 3);
    }

    // q and dout fragments (B operands), one query row per lane
    const int qi = q0 + wave * 32 + lq;
    const bool ok = qi < p.q_len;
    u32x4 qf[D / 16], dof[DV / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qf[t] = ok ? ld_global16(qg + (size_t)qi * ROWB + (2 * t + g) * 16) : u32x4{0, 0, 0, 0};
      if (p.neg) qf[t] ^= 0x80008000u;
    }
#pragma unroll
    for (int t = 0; t < DV / 16; ++t)
      dof[t] = ok ? ld_global16(dog + (size_t)qi * ROWBV + (2 * t + g) * 16) : u32x4{0, 0, 0, 0};
    const long long row = (long long)head_q + min(qi, max(p.q_len - 1, 0));
    const float ndelta = ok ? p.ws[row] : 0.f;
    const float nm = ok ? p.c1 * p.ws[rows + row] : -INFINITY;  // c1 a (-inf: no key)
    int lo, hi;
    fwd::row_interval<MASK>(p, qi, lo, hi);
    const float c1 = p.c1;
    float bias_u = 0.f, bias_u16 = 0.f;
    if constexpr (SCORE == FLEX_SCORE_REL_BIAS) {
      bias_u = -fwd::head_slope(p, h) / (p.c1 * fwd::kLn2);
      bias_u16 = 16.0f * bias_u;
    }

    // tile list
    const int nk = p.n_kb;
    const int np = min(max(p.kv_num[qb], 0), nk);
    const int nf = min(max(p.fkv_num[qb], 0), nk);
    const int ntiles = np + nf;
    const int nsteps = ntiles * SPT;
    const int32_t* prow = p.kv_idx + (size_t)qb * nk;
    const int32_t* frow = p.fkv_idx + (size_t)qb * nk;
    auto load_window = [&](int base) {
      const int t = min(base + lane, ntiles - 1);
      int v = 0;
      if (t >= 0) v = t < np ? prow[t] : frow[t - np];
      return v;
    };
    int win_base = 0;
    int win = load_window(0);
    int win_nx = ntiles > 64 ? load_window(64) : 0;
    auto tile_kb = [&](int t) {
      const int i = t - win_base;
      const int v = i < 64 ? __builtin_amdgcn_readlane(win, i) : __builtin_amdgcn_readlane(win_nx, i - 64);
      return min(max(v, 0), nk - 1);
    };

    // K and V of step m into a stage buffer, both in the tile layout, through
    // buffer resources based at the step's first key whose size is the rows
    // that exist: the per-lane offsets do not depend on the step, and rows
    // past the end of the keys read as zero (partial tiles mask them).
    // (The offsets are rebuilt per step from the lane index, behind an
    // empty asm statement so that they are not hoisted: kept in registers
    // across the loop they push the head-dim-64 instance into spills.)
    auto dma = [&](lds_t* dst, int m) {
      unsigned ln = (unsigned)lane;
      asm volatile("" : "+v"(ln));
      unsigned ko[NDMA], vo[NDMAV];
#pragma unroll
      for (int j = 0; j < NDMA; ++j) {
        const unsigned sl = (unsigned)((wave * NDMA + j) * 64) + ln;
        const int r = (int)(sl / CPR), q = (int)(sl % CPR);
        ko[j] = (unsigned)(r * ROWB) + ((unsigned)(q ^ (vswz<D>(r) >> 1)) << 4);
      }
#pragma unroll
      for (int j = 0; j < NDMAV; ++j) {
        const unsigned sl = (unsigned)((wave * NDMAV + j) * 64) + ln;
        const int r = (int)(sl / CPRV), q = (int)(sl % CPRV);
        vo[j] = (unsigned)(r * ROWBV) + ((unsigned)(q ^ (vswz<DV>(r) >> 1)) << 4);
      }
      const int kb = tile_kb(m / SPT);
      const int kv0 = kb * KB + (m % SPT) * KS;
      const int rows = __builtin_amdgcn_readfirstlane(max(min(KS, p.kv_len - kv0), 0));
      const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(kg + (size_t)kv0 * ROWB), 0, rows * ROWB, fwd::kBufferRsrcWord3);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(vg + (size_t)kv0 * ROWBV), 0, rows * ROWBV, fwd::kBufferRsrcWord3);
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

    f32x16 acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = f32x16{};

    auto block = [&](const lds_t* cur, int b, int kvl, bool partial) {
      // S^T = K q^T (accumulator starts at the bias for REL_BIAS)
      f32x16 s;
      if constexpr (SCORE == FLEX_SCORE_REL_BIAS) {
        float a0 = bias_u * (float)(qi - kvl);
        asm volatile("" : "+v"(a0));
        float x = a0, y = a0 - bias_u16;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          s[r] = x;
          s[8 + r] = y;
          x -= bias_u;
          y -= bias_u;
        }
      } else {
        s = f32x16{};
      }
      f32x16 dp = f32x16{};
      bf16x8 kf[D / 16], vf[DV / 16];
#pragma unroll
      for (int t = 0; t < D / 16; ++t)
        kf[t] = __builtin_bit_cast(bf16x8, FLEXATTN_LDS(u32x4, cur + kra[t] + 32 * b * ROWB));
#pragma unroll
      for (int t = 0; t < DV / 16; ++t)
        vf[t] = __builtin_bit_cast(bf16x8, FLEXATTN_LDS(u32x4, cur + STAGE + vra[t] + 32 * b * ROWBV));
#pragma unroll
      for (int t = 0; t < (D > DV ? D : DV) / 16; ++t) {
        if (t < D / 16)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], __builtin_bit_cast(bf16x8, qf[t]), s, 0, 0, 0);
        if (t < DV / 16)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t], __builtin_bit_cast(bf16x8, dof[t]), dp, 0, 0, 0);
      }
      // K^T fragments for dq^T += K^T ds^T
      bf16x8 ktf[NE][2];
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const lds_t* vp = cur + tro[e] + (32 * b + 16 * hh) * ROWB;
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)vp);
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(vp + 4 * ROWB));
          ktf[e][hh] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      // p = 2^(c1 s + c1 a), masked on partial tiles; ds = p (dP - delta)
      float ds[16];
      const int lim_hi = hi - kvl, lim_lo = lo - kvl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c1, nm));
        if (partial) {
          const int off = 16 * (r >> 3) + (r & 7);
          bool vis = off <= lim_hi;
          if constexpr (fwd::two_sided_mask<MASK>()) vis = vis && off >= lim_lo;
          pr = vis ? pr : 0.f;
        }
        ds[r] = pr * (dp[r] + ndelta);
      }
      bf16x8 pk[2];
      pack16(ds, pk);
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktf[e][hh], pk[hh], acc[e], 0, 0, 0);
    };

    auto step = [&](auto buf_tag, int n) {
      constexpr int B = decltype(buf_tag)::value;
      const lds_t* cur = buf[B];
      const int t = n / SPT, part = n % SPT;
      if (t >= win_base + 64) {
        win_base += 64;
        win = win_nx;
        if (win_base + 64 < ntiles) win_nx = load_window(win_base + 64);
      }
      const int kb = tile_kb(t);
      const int kv0 = kb * KB + part * KS;
      const bool partial = t < np || q_ragged || kb * KB + KB > p.kv_len;
      if (n + 1 < nsteps) dma(buf[(B + 1) % 2], n + 1);
#pragma unroll
      for (int b = 0; b < KS / 32; ++b) {
        // skip a 32-key block no row of the wave sees; mask only one that
        // some row sees in part
        bool masked = partial;
        if (partial) {
          const int b0 = kv0 + 32 * b;
          const bool any = lo <= b0 + 31 && hi >= b0 && lo <= hi;
          if (!__any(any)) continue;
          masked = !__all(lo <= b0 && hi >= b0 + 31);
        }
        block(cur, b, kv0 + 32 * b + 8 * g, masked);
      }
      s_barrier_full();
    };

    if (nsteps > 0) dma(buf[0], 0);
    s_barrier_full();
    int n = 0;
    for (; n + 2 <= nsteps; n += 2) {
      step(Int<0>(), n);
      step(Int<1>(), n + 1);
    }
    if (n < nsteps) step(Int<0>(), n);

    // bf16 dq goes through LDS (every wave is past the last step barrier,
    // no load in flight): whole 16-byte pieces over contiguous rows
    // (document ids out of order: the builder poisoned every interval, and
    // the row's gradient is NaN)
    float fq = p.scale;
    if constexpr (MASK == FLEX_MASK_DOCUMENT)
      if (fwd::doc_poisoned(lo, hi)) fq = fwd::opaque_nan();
    constexpr bool LDS_DQ = NW * 32 * ROWB <= STAGE + STAGEV;
    if (LDS_DQ && p.grad_bf16 != 0)
      fwd::store_rows_bf16_lds<NE>(buf[0] + wave * 32 * ROWB,
                                   static_cast<char*>(p.dq) + (head_q + (size_t)(q0 + wave * 32)) * ROWB,
                                   p.q_len - (q0 + wave * 32), acc, fq, lane);
    else if (ok)
      write_row_t<NE>(p.dq, p.grad_bf16 != 0, head_q + qi, D, g, acc, fq);
  }
};

// ---------------------------------------------------------------------------
// dk, dv
// ---------------------------------------------------------------------------
// D: head dim of q and k; DV: value head dim (width of v, out and dout)
template <int D, int DV, int QB, int KB, int MASK, int SCORE>
struct Bf16BwdDkv {
  static constexpr int NW = KB / 32;        // one wave per 32 keys
  static constexpr int NT = 64 * NW;
  static constexpr int QS = 32;             // query rows per step
  static constexpr int SPQ = QB / QS;       // steps per listed q-block
  static constexpr int NE = D / 32;         // dk accumulators
  static constexpr int NEV = DV / 32;       // dv accumulators
  static constexpr int ROWB = D * 2;        // bytes per q row
  static constexpr int ROWBV = DV * 2;      // bytes per dout row
  static constexpr bool QF = D == 64 && DV == 64;  // tile swizzle: see vswz_q
  static constexpr int TILE = QS * ROWB;    // bytes of q per step (dout follows)
  static constexpr int ARR = TILE + QS * ROWBV;  // offset of the per-row arrays
  static constexpr int STAGEB = ARR + 2 * QS * 4;
  static constexpr int CPR = ROWB / 16;
  static constexpr int CPRV = ROWBV / 16;
  static constexpr int NDMA = QS * CPR / (64 * NW);
  static constexpr int NDMAV = QS * CPRV / (64 * NW);
  // head dims 64/64: three waves per SIMD (168 VGPRs, with a few spilled; it
  // measured 4-17% faster than two); 128/128: two (the wave's K and V rows
  // and the dk and dv accumulators take ~275 registers, ~20 of them spilled;
  // 13-18% faster than one wave with no spill); 64/128 and 128/64: two
  static constexpr int WAVES_PER_SIMD = D == 64 && DV == 64 ? 3 : 2;
  static_assert(NDMA * 64 * NW == QS * CPR, "step split");
  static_assert(NDMAV * 64 * NW == QS * CPRV, "step split (dout)");

  __device__ static void run(const BwdParams& p) {
    __shared__ __attribute__((aligned(16))) char sb0[STAGEB];
    __shared__ __attribute__((aligned(16))) char sb1[STAGEB];
    lds_t* const buf[2] = {(lds_t*)sb0, (lds_t*)sb1};
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, g = lane >> 5;

    // (head, kv-block): the forward's order with the kv-block reversed, so the
    // kv-blocks the most q-blocks see (the first ones, under causal masks)
    // start first
    int bh, kbr;
    fwd::wg_to_tile(p.n_kb, bh, kbr);
    const int kb = p.n_kb - 1 - kbr;
    const int h = bh % p.H;
    const long long rows = (long long)p.B * p.H * p.q_len;
    const size_t head_q = (size_t)bh * p.q_len;
    const size_t head_kv = (size_t)bh * p.kv_len;
    const char* qg = static_cast<const char*>(p.q) + head_q * ROWB;
    const char* dog = static_cast<const char*>(p.dout) + head_q * ROWBV;
    const bool kv_ragged = kb * KB + KB > p.kv_len;

    // this lane's key, its K and V rows (B operands), its visible queries
    const int kk = kb * KB + wave * 32 + lq;
    const bool kok = kk < p.kv_len;
    const int kcl = min(kk, p.kv_len - 1);
    u32x4 kf[D / 16], vf[DV / 16];
    {
      const char* kr = static_cast<const char*>(p.k) + (head_kv + kcl) * ROWB;
      const char* vr = static_cast<const char*>(p.v) + (head_kv + kcl) * ROWBV;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        kf[t] = ld_global16(kr + (2 * t + g) * 16);
        if (p.neg) kf[t] ^= 0x80008000u;
      }
#pragma unroll
      for (int t = 0; t < DV / 16; ++t) vf[t] = ld_global16(vr + (2 * t + g) * 16);
    }
    int qlo, qhi;
    col_interval<MASK>(p, kk, qlo, qhi);
    const float c1 = p.c1;
    float bias_u = 0.f, bias_u16 = 0.f;
    if constexpr (SCORE == FLEX_SCORE_REL_BIAS) {
      bias_u = -fwd::head_slope(p, h) / (p.c1 * fwd::kLn2);
      bias_u16 = 16.0f * bias_u;
    }

    // A-operand row reads of the q / dout tiles, and transposing reads
    // (q rows D wide, dout rows DV wide)
    const int ra = swap23(lq);
    int qra[D / 16], dra[DV / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qra[t] = ra * ROWB + (((2 * t + g) ^ (vswz_q<D, QF>(ra) >> 1)) << 4);
#pragma unroll
    for (int t = 0; t < DV / 16; ++t)
      dra[t] = ra * ROWBV + (((2 * t + g) ^ (vswz_q<DV, QF>(ra) >> 1)) << 4);
    int tro[NE], trov[NEV];
    {
      const int j = lane & 15, u = (lane >> 4) & 1;
      const int r0 = 8 * g + (j >> 2);
#pragma unroll
      for (int e = 0; e < NE; ++e) tro[e] = r0 * ROWB + (((8 * e + 4 * u + (j & 3)) ^ vswz_q<D, QF>(r0)) << 3);
#pragma unroll
      for (int e = 0; e < NEV; ++e)
        trov[e] = r0 * ROWBV + (((8 * e + 4 * u + (j & 3)) ^ vswz_q<DV, QF>(r0)) << 3);
    }

    // transposed tile list of this kv-block
    const int nq = p.n_qb;
    const int np = min(max(p.q_num[kb], 0), nq);
    const int nf = min(max(p.fq_num[kb], 0), nq);
    const int ntiles = np + nf;
    const int nsteps = ntiles * SPQ;
    const int32_t* prow = p.q_idx + (size_t)kb * nq;
    const int32_t* frow = p.fq_idx + (size_t)kb * nq;
    auto load_window = [&](int base) {
      const int t = min(base + lane, ntiles - 1);
      int v = 0;
      if (t >= 0) v = t < np ? prow[t] : frow[t - np];
      return v;
    };
    int win_base = 0;
    int win = load_window(0);
    int win_nx = ntiles > 64 ? load_window(64) : 0;
    auto tile_qb = [&](int t) {
      const int i = t - win_base;
      const int v = i < 64 ? __builtin_amdgcn_readlane(win, i) : __builtin_amdgcn_readlane(win_nx, i - 64);
      return min(max(v, 0), nq - 1);
    };

    // q and dout rows of step m (32 query rows) in the tile layout, through buffer
    // resources as in the dq kernel (rows past the end of the queries read
    // as zero), then -delta and a of those rows (wave 0, one dword per lane,
    // clamped to the last row)
    unsigned qo[NDMA], dov[NDMAV];
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int sl = (wave * NDMA + j) * 64 + lane;
      const int r = sl / CPR, q = sl % CPR;
      qo[j] = (unsigned)(r * ROWB) + ((unsigned)(q ^ (vswz_q<D, QF>(r) >> 1)) << 4);
    }
#pragma unroll
    for (int j = 0; j < NDMAV; ++j) {
      const int sl = (wave * NDMAV + j) * 64 + lane;
      const int r = sl / CPRV, q = sl % CPRV;
      dov[j] = (unsigned)(r * ROWBV) + ((unsigned)(q ^ (vswz_q<DV, QF>(r) >> 1)) << 4);
    }
    auto dma = [&](lds_t* dst, int m) {
      const int qbm = tile_qb(m / SPQ);
      const int q0m = qbm * QB + (m % SPQ) * QS;
      const int rows_in = __builtin_amdgcn_readfirstlane(max(min(QS, p.q_len - q0m), 0));
      const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(qg + (size_t)q0m * ROWB), 0, rows_in * ROWB, fwd::kBufferRsrcWord3);
      const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(dog + (size_t)q0m * ROWBV), 0, rows_in * ROWBV, fwd::kBufferRsrcWord3);
#pragma unroll
      for (int j = 0; j < (NDMA > NDMAV ? NDMA : NDMAV); ++j) {
        if (j < NDMA)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              qr, (__attribute__((address_space(3))) void*)(dst + (wave * NDMA + j) * 1024), 16,
              (int)qo[j], 0, 0, 0);
        if (j < NDMAV)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              dr, (__attribute__((address_space(3))) void*)(dst + TILE + (wave * NDMAV + j) * 1024),
              16, (int)dov[j], 0, 0, 0);
      }
      const int r00 = min(q0m, p.q_len - 1);
      const int rows_left = min(QS, p.q_len - r00);
      if (wave == 0) {
        const int r = min(lq, rows_left - 1);
        const float* src = p.ws + (g == 0 ? 0 : rows) + (long long)head_q + r00 + r;
        // lanes 0..31: -delta, lanes 32..63: a
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst + ARR), 4, 0, 0);
      }
    };

    f32x16 dk[NE], dv[NEV];
#pragma unroll
    for (int e = 0; e < NE; ++e) dk[e] = f32x16{};
#pragma unroll
    for (int e = 0; e < NEV; ++e) dv[e] = f32x16{};

    // one step: 32 query rows q00.. against this wave's 32 keys
    auto block = [&](const lds_t* cur, int q00, bool partial) {
      // S = q K^T from a (the accumulator's start), + the bias for REL_BIAS;
      // register 8h + j holds query q00 + 16h + 8g + j
      f32x16 s, dp;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 a0 = FLEXATTN_LDS(f32x4, cur + ARR + 128 + (16 * hh + 8 * g) * 4);
        const f32x4 a1 = FLEXATTN_LDS(f32x4, cur + ARR + 128 + (16 * hh + 8 * g + 4) * 4);
        const f32x4 d0 = FLEXATTN_LDS(f32x4, cur + ARR + (16 * hh + 8 * g) * 4);
        const f32x4 d1 = FLEXATTN_LDS(f32x4, cur + ARR + (16 * hh + 8 * g + 4) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[8 * hh + i] = a0[i];
          s[8 * hh + 4 + i] = a1[i];
          dp[8 * hh + i] = d0[i];
          dp[8 * hh + 4 + i] = d1[i];
        }
      }
      if constexpr (SCORE == FLEX_SCORE_REL_BIAS) {
        float b0 = bias_u * (float)(q00 + 8 * g - kk);
        asm volatile("" : "+v"(b0));
        float x = b0, y = b0 + bias_u16;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          s[r] += x;
          s[8 + r] += y;
          x += bias_u;
          y += bias_u;
        }
      }
      bf16x8 qa[D / 16], da[DV / 16];
#pragma unroll
      for (int t = 0; t < D / 16; ++t) qa[t] = __builtin_bit_cast(bf16x8, FLEXATTN_LDS(u32x4, cur + qra[t]));
#pragma unroll
      for (int t = 0; t < DV / 16; ++t)
        da[t] = __builtin_bit_cast(bf16x8, FLEXATTN_LDS(u32x4, cur + TILE + dra[t]));
#pragma unroll
      for (int t = 0; t < (D > DV ? D : DV) / 16; ++t) {
        if (t < D / 16)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t], __builtin_bit_cast(bf16x8, kf[t]), s, 0, 0, 0);
        if (t < DV / 16)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[t], __builtin_bit_cast(bf16x8, vf[t]), dp, 0, 0, 0);
      }
      // transposed fragments of dout and q for the two accumulations
      // (the second read of each 4-row group: for 64-wide tiles the first
      // offset with bit 4 flipped (see vswz_q), rebuilt per block behind an
      // empty asm statement rather than kept in registers across the loop)
      bf16x8 dot[NEV][2], qt[NE][2];
#pragma unroll
      for (int e = 0; e < NEV; ++e) {
        int o2 = trov[e];
        if constexpr (QF) {
          o2 ^= 16;
          asm volatile("" : "+v"(o2));
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const lds_t* dp0 = cur + TILE + trov[e] + 16 * hh * ROWBV;
          const lds_t* dp1 = cur + TILE + o2 + (16 * hh + 4) * ROWBV;
          const i16x4 d0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)dp0);
          const i16x4 d1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)dp1);
          dot[e][hh] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(d0, d1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        int o2 = tro[e];
        if constexpr (QF) {
          o2 ^= 16;
          asm volatile("" : "+v"(o2));
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const lds_t* qp0 = cur + tro[e] + 16 * hh * ROWB;
          const lds_t* qp1 = cur + o2 + (16 * hh + 4) * ROWB;
          const i16x4 q0v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)qp0);
          const i16x4 q1v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)qp1);
          qt[e][hh] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(q0v, q1v, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
      // p = 2^(c1 s), masked on partial tiles; ds = p dP
      float pv[16], ds[16];
      const int lim_lo = qlo - q00 - 8 * g, lim_hi = qhi - q00 - 8 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = __builtin_amdgcn_exp2f(s[r] * c1);
        if (partial) {
          const int off = 16 * (r >> 3) + (r & 7);
          pr = (off >= lim_lo && off <= lim_hi) ? pr : 0.f;
        }
        pv[r] = pr;
        ds[r] = pr * dp[r];
      }
      bf16x8 pp[2], pd[2];
      pack16(pv, pp);
      pack16(ds, pd);
#pragma unroll
      for (int e = 0; e < (NE > NEV ? NE : NEV); ++e)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          if (e < NEV) dv[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dot[e][hh], pp[hh], dv[e], 0, 0, 0);
          if (e < NE) dk[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt[e][hh], pd[hh], dk[e], 0, 0, 0);
        }
    };

    auto step = [&](auto buf_tag, int n) {
      constexpr int B = decltype(buf_tag)::value;
      const lds_t* cur = buf[B];
      const int t = n / SPQ, part = n % SPQ;
      if (t >= win_base + 64) {
        win_base += 64;
        win = win_nx;
        if (win_base + 64 < ntiles) win_nx = load_window(win_base + 64);
      }
      const int qbt = tile_qb(t);
      const int q00 = qbt * QB + part * QS;
      // a listed-full tile at a ragged edge is still handled as partial
      const bool partial = t < np || kv_ragged || qbt * QB + QB > p.q_len;
      if (n + 1 < nsteps) dma(buf[(B + 1) % 2], n + 1);
      // skip a step no key of the wave is seen by; mask only one that some
      // key is seen in part by
      bool run_it = true, masked = partial;
      if (partial) {
        const bool any = qlo <= q00 + QS - 1 && qhi >= q00 && qlo <= qhi;
        run_it = __any(any);
        masked = !__all(qlo <= q00 && qhi >= q00 + QS - 1);
      }
      if (run_it) block(cur, q00, masked);
      s_barrier_full();
    };

    if (nsteps > 0) dma(buf[0], 0);
    s_barrier_full();
    int n = 0;
    for (; n + 2 <= nsteps; n += 2) {
      step(Int<0>(), n);
      step(Int<1>(), n + 1);
    }
    if (n < nsteps) step(Int<0>(), n);

    // bf16 dk and dv go through LDS like dq: wave w uses stage buffer w % 2
    // at region w / 2 (every wave is past the last step barrier)
    // (document ids out of order: the builder poisoned every interval, and
    // the key's gradients are NaN)
    float fk = p.scale, fv = 1.0f;
    if constexpr (MASK == FLEX_MASK_DOCUMENT)
      if (fwd::doc_poisoned(qlo, qhi)) fk = fv = fwd::opaque_nan();
    constexpr int REG = 32 * (ROWB > ROWBV ? ROWB : ROWBV);
    constexpr bool LDS_DKV = ((NW + 1) / 2) * REG <= STAGEB;
    if (LDS_DKV && p.grad_bf16 != 0) {
      lds_t* reg = ((wave & 1) ? buf[1] : buf[0]) + (wave >> 1) * REG;
      const int k0 = kb * KB + wave * 32;
      fwd::store_rows_bf16_lds<NE>(reg, static_cast<char*>(p.dk) + (head_kv + (size_t)k0) * ROWB,
                                   p.kv_len - k0, dk, fk, lane);
      fwd::store_rows_bf16_lds<NEV>(reg, static_cast<char*>(p.dv) + (head_kv + (size_t)k0) * ROWBV,
                                    p.kv_len - k0, dv, fv, lane);
    } else if (kok) {
      write_row_t<NE>(p.dk, p.grad_bf16 != 0, head_kv + kk, D, g, dk, fk);
      write_row_t<NEV>(p.dv, p.grad_bf16 != 0, head_kv + kk, DV, g, dv, fv);
    }
  }
};

#undef FLEXATTN_LDS

template <int D, int DV, int QB, int KB, int MASK, int SCORE>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Bf16BwdDq<D, DV, QB, KB, MASK, SCORE>::NT),
                          amdgpu_waves_per_eu(Bf16BwdDq<D, DV, QB, KB, MASK, SCORE>::WAVES_PER_SIMD)))
void bwd_dq_kernel(BwdParams p) {
  Bf16BwdDq<D, DV, QB, KB, MASK, SCORE>::run(p);
}

template <int D, int DV, int QB, int KB, int MASK, int SCORE>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Bf16BwdDkv<D, DV, QB, KB, MASK, SCORE>::NT),
                          amdgpu_waves_per_eu(Bf16BwdDkv<D, DV, QB, KB, MASK, SCORE>::WAVES_PER_SIMD)))
void bwd_dkv_kernel(BwdParams p) {
  Bf16BwdDkv<D, DV, QB, KB, MASK, SCORE>::run(p);
}

template <int D, int DV, int QB, int KB, int MASK, int SCORE>
hipError_t launch_bwd_one(const BwdParams& p, hipStream_t s) {
  const long long rows = (long long)p.B * p.H * p.q_len;
  if (rows > 0) {
    const long long threads = rows * (DV / 8);
    hipLaunchKernelGGL(bwd_pre_kernel<DV>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dq == nullptr: WRITE_DQ off, the dq kernel is skipped
  const long long nq = p.dq != nullptr ? (long long)p.B * p.H * p.n_qb : 0;
  if (nq > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, DV, QB, KB, MASK, SCORE>), dim3((unsigned)nq),
                       dim3(Bf16BwdDq<D, DV, QB, KB, MASK, SCORE>::NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long nkv = (long long)p.B * p.H * p.n_kb;
  if (nkv > 0) {
    hipLaunchKernelGGL((bwd_dkv_kernel<D, DV, QB, KB, MASK, SCORE>), dim3((unsigned)nkv),
                       dim3(Bf16BwdDkv<D, DV, QB, KB, MASK, SCORE>::NT), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D, int DV, int QB, int KB, int MASK>
hipError_t bwd_pick_score(const BwdParams& p, int score, hipStream_t s) {
  if (score == FLEX_SCORE_REL_BIAS) return launch_bwd_one<D, DV, QB, KB, MASK, FLEX_SCORE_REL_BIAS>(p, s);
  return launch_bwd_one<D, DV, QB, KB, MASK, FLEX_SCORE_IDENTITY>(p, s);
}

template <int D, int DV, int QB, int KB>
hipError_t bwd_pick_mask(const BwdParams& p, int mask, int score, hipStream_t s) {
  switch (mask) {
    case FLEX_MASK_NOOP:
      return bwd_pick_score<D, DV, QB, KB, FLEX_MASK_NOOP>(p, score, s);
    case FLEX_MASK_CAUSAL:
      return bwd_pick_score<D, DV, QB, KB, FLEX_MASK_CAUSAL>(p, score, s);
    case FLEX_MASK_SLIDING_WINDOW:
      return bwd_pick_score<D, DV, QB, KB, FLEX_MASK_SLIDING_WINDOW>(p, score, s);
    case FLEX_MASK_DOCUMENT:
    case FLEX_MASK_DOCUMENT_CAUSAL:
      return bwd_pick_score<D, DV, QB, KB, FLEX_MASK_DOCUMENT>(p, score, s);
    default:
      return bwd_pick_score<D, DV, QB, KB, FLEX_MASK_PREFIX_CAUSAL>(p, score, s);
  }
}

#undef FLEXATTN_LDS

}  // namespace bwd
}  // namespace flexattn

#define FLEXATTN_BWD_UNIT(NAME, D, DV, QB, KB)                                     \
  namespace flexattn {                                                           \
  hipError_t NAME(const BwdParams& p, int mask, int score, hipStream_t s) {      \
    return bwd::bwd_pick_mask<D, DV, QB, KB>(p, mask, score, s);                 \
  }                                                                              \
  }
