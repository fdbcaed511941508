// bwd_fp32.hpp -- the backward pass for fp32 inputs on gfx950.
//
// The gradients of bwd_bf16.hpp (the flex_attention backward op of
// "[Inductor][Flex Attention] Add Subtiling Option for Alpha Scaling", test
// hunks): for every visible pair (i, j)
//   p_ij = exp(s_ij - lse_i),  ds_ij = p_ij (<dout_i, v_j> - delta_i),
//   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
//   dv_j = sum_i p_ij dout_i,
// here with every operand and product in fp32 on the vector ALUs: the fp32
// path is the small parity workload's, where exactness matters more than
// rate.  Four lanes share a row (a query row in the dq kernel, a key in the
// dk/dv kernel), each holding a quarter of the head dim: lane u of a row owns
// the 16-byte chunks 4m + u of it, so that the four lanes of a row read four
// consecutive chunks of an LDS row (no bank conflicts) and every row of a
// wave reads the same ones (a broadcast).  A dot product is four partial
// sums and two lane exchanges.  Both kernels walk the block mask's tile lists
// (empty tiles are never visited; in a visited tile every pair is checked
// against the row's visible interval), staging the other side's tile in LDS
// 32 rows at a time.  DV is the value head dim (V, out, dout and dv rows),
// which may differ from D.
#pragma once
#include "bwd_bf16.hpp"

namespace flexattn {
namespace bwd32 {

using fwd::f32x4;
using fwd::u32x4;

typedef __attribute__((address_space(3))) char lds_t;
#define FLEXATTN_LDS(T, ptr) (*(__attribute__((address_space(3))) T*)(ptr))

// sum over the four lanes of a row (lanes 4r .. 4r + 3)
__device__ inline float sum4(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// Per query row: ws[row] = -delta = dlse_i - <dout_i, out_i>.  D / 4 lanes
// per row (D: the rows' width, the value head dim), each reading 4 elements
// of out and dout.
template <int D>
__global__ __launch_bounds__(256) void bwd32_pre_kernel(BwdParams p) {
  constexpr int LPR = D / 4;
  const long long rows = (long long)p.B * p.H * p.q_len;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / LPR;
  const int part = (int)(t % LPR);
  float acc = 0.f;
  if (row < rows) {
    const f32x4 o = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.out) + row * D + part * 4);
    const f32x4 d = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.dout) + row * D + part * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(o[i], d[i], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) p.ws[row] = (p.dlse != nullptr ? p.dlse[row] : 0.f) - acc;
}

// Load rows [r0, r0 + n) of a [*, D] fp32 matrix (from base) into an LDS
// tile of rows of D floats, 16 bytes per thread per instruction.
template <int D, int NT>
__device__ inline void stage_rows(lds_t* dst, const float* base, int r0, int n) {
  constexpr int CPR = D / 4;  // 16-byte chunks per row
  for (int c = (int)threadIdx.x; c < n * CPR; c += NT) {
    const int r = c / CPR, q = c % CPR;
    FLEXATTN_LDS(f32x4, dst + (r * D + 4 * q) * 4) =
        *reinterpret_cast<const f32x4*>(base + (size_t)(r0 + r) * D + 4 * q);
  }
}

// Store the D / 4 values a lane holds of one row (chunks 4m + u), times f.
template <int D>
__device__ inline void store_quarter(void* base, bool bf16, size_t row, int u, const f32x4 (&a)[D / 16],
                                     float f) {
#pragma unroll
  for (int m = 0; m < D / 16; ++m) {
    const int d = 16 * m + 4 * u;
    const f32x4 v = a[m] * f;
    if (bf16) {
      *reinterpret_cast<fwd::bf16x4*>(static_cast<char*>(base) + (row * D + d) * 2) =
          fwd::bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    } else {
      *reinterpret_cast<f32x4*>(static_cast<char*>(base) + (row * D + d) * 4) = v;
    }
  }
}

// ---------------------------------------------------------------------------
// dq: one work-group per (batch, head, q-block), four lanes per query row,
// walking the forward's tile list with each visited K and V tile in LDS.
// ---------------------------------------------------------------------------
template <int D, int DV, int QB, int KB, int MASK, int SCORE>
struct Fp32BwdDq {
  static constexpr int NT = 4 * QB;
  static constexpr int NM = D / 16;    // 16-byte chunks a lane holds of a q / K row
  static constexpr int NMV = DV / 16;  // ... of a dout / V row
  static constexpr int SUB = 32;       // keys staged at a time
  static constexpr int TILE = SUB * D * 4;
  static constexpr int TILEV = SUB * DV * 4;

  __device__ static void run(const BwdParams& p) {
    __shared__ __attribute__((aligned(16))) char smem[TILE + TILEV];
    lds_t* const kt = (lds_t*)smem;
    lds_t* const vt = kt + TILE;
    const int tid = threadIdx.x;
    const int r = tid >> 2, u = tid & 3;
    const int bh = blockIdx.x / p.n_qb, qb = blockIdx.x % p.n_qb;
    const int h = bh % p.H;
    const int qi = qb * QB + r;
    const bool row_ok = qi < p.q_len;
    const size_t head_q = (size_t)bh * p.q_len, head_kv = (size_t)bh * p.kv_len;
    const float* qg = static_cast<const float*>(p.q) + head_q * D;
    const float* dog = static_cast<const float*>(p.dout) + head_q * DV;
    const float* kg = static_cast<const float*>(p.k) + head_kv * D;
    const float* vg = static_cast<const float*>(p.v) + head_kv * DV;

    f32x4 qv[NM], dov[NMV], acc[NM];
    const int qr = min(qi, p.q_len - 1);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      qv[m] = *reinterpret_cast<const f32x4*>(qg + (size_t)qr * D + 16 * m + 4 * u);
      acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int m = 0; m < NMV; ++m)
      dov[m] = *reinterpret_cast<const f32x4*>(dog + (size_t)qr * DV + 16 * m + 4 * u);
    int lo, hi;
    fwd::row_interval<MASK>(p, qi, lo, hi);
    const float lse = row_ok ? p.lse[head_q + qi] : -INFINITY;
    const float ndelta = row_ok ? p.ws[head_q + qi] : 0.f;
    const bool live = row_ok && lse != -INFINITY && lo <= hi;
    float slope = 0.f;
    if constexpr (SCORE == FLEX_SCORE_REL_BIAS) slope = fwd::head_slope(p, h);

    const int nk = p.n_kb;
    const int np = min(max(p.kv_num[qb], 0), nk), nf = min(max(p.fkv_num[qb], 0), nk);
    const int32_t* prow = p.kv_idx + (size_t)qb * nk;
    const int32_t* frow = p.fkv_idx + (size_t)qb * nk;
    for (int t = 0; t < np + nf; ++t) {
      const int kb = min(max(t < np ? prow[t] : frow[t - np], 0), nk - 1);
      const int k0 = kb * KB, nkeys = min(KB, p.kv_len - k0);
      for (int c0 = 0; c0 < nkeys; c0 += SUB) {
      const int n = min(SUB, nkeys - c0);
      __syncthreads();  // every lane is done with the previous keys
      stage_rows<D, NT>(kt, kg, k0 + c0, n);
      stage_rows<DV, NT>(vt, vg, k0 + c0, n);
      __syncthreads();
      for (int j = 0; j < n; ++j) {
        f32x4 kq[NM];
        float sd = 0.f, sp = 0.f;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          kq[m] = FLEXATTN_LDS(f32x4, kt + (j * D + 16 * m + 4 * u) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sd = fmaf(qv[m][e], kq[m][e], sd);
        }
#pragma unroll
        for (int m = 0; m < NMV; ++m) {
          const f32x4 vq = FLEXATTN_LDS(f32x4, vt + (j * DV + 16 * m + 4 * u) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sp = fmaf(dov[m][e], vq[e], sp);
        }
        sd = sum4(sd);
        sp = sum4(sp);
        const int kk = k0 + c0 + j;
        float s = p.scale * sd;
        if constexpr (SCORE == FLEX_SCORE_REL_BIAS) s -= slope * (float)(qi - kk);
        const bool vis = live && kk >= lo && kk <= hi;
        const float pr = vis ? expf(s - lse) : 0.f;
        const float ds = pr * (sp + ndelta);
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] += ds * kq[m];
      }
      }
    }
    if (!row_ok) return;
    float f = p.scale;
    if constexpr (MASK == FLEX_MASK_DOCUMENT)
      if (fwd::doc_poisoned(lo, hi)) f = fwd::opaque_nan();
    store_quarter<D>(p.dq, p.grad_bf16 != 0, head_q + qi, u, acc, f);
  }
};

// ---------------------------------------------------------------------------
// dk, dv: one work-group per (batch, head, kv-block), four lanes per key,
// walking the transposed tile list with each visited q and dout tile (and
// its rows' lse and -delta) in LDS.
// ---------------------------------------------------------------------------
template <int D, int DV, int QB, int KB, int MASK, int SCORE>
struct Fp32BwdDkv {
  static constexpr int NT = 4 * KB;
  static constexpr int NM = D / 16;
  static constexpr int NMV = DV / 16;
  static constexpr int SUB = 32;  // query rows staged at a time
  static constexpr int TILE = SUB * D * 4;
  static constexpr int TILEV = SUB * DV * 4;

  __device__ static void run(const BwdParams& p) {
    __shared__ __attribute__((aligned(16))) char smem[TILE + TILEV + 2 * SUB * 4];
    lds_t* const qt = (lds_t*)smem;
    lds_t* const dt = qt + TILE;
    lds_t* const rt = dt + TILEV;  // lse, then -delta, of the tile's rows
    const int tid = threadIdx.x;
    const int r = tid >> 2, u = tid & 3;
    const int bh = blockIdx.x / p.n_kb, kb = blockIdx.x % p.n_kb;
    const int h = bh % p.H;
    const int kk = kb * KB + r;
    const bool key_ok = kk < p.kv_len;
    const size_t head_q = (size_t)bh * p.q_len, head_kv = (size_t)bh * p.kv_len;
    const float* qg = static_cast<const float*>(p.q) + head_q * D;
    const float* dog = static_cast<const float*>(p.dout) + head_q * DV;
    const float* kg = static_cast<const float*>(p.k) + head_kv * D;
    const float* vg = static_cast<const float*>(p.v) + head_kv * DV;

    f32x4 kv[NM], vv[NMV], dk[NM], dv[NMV];
    const int kr = min(kk, p.kv_len - 1);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      kv[m] = *reinterpret_cast<const f32x4*>(kg + (size_t)kr * D + 16 * m + 4 * u);
      dk[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int m = 0; m < NMV; ++m) {
      vv[m] = *reinterpret_cast<const f32x4*>(vg + (size_t)kr * DV + 16 * m + 4 * u);
      dv[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int qlo, qhi;
    bwd::col_interval<MASK>(p, kk, qlo, qhi);
    const bool live = key_ok && qlo <= qhi;
    float slope = 0.f;
    if constexpr (SCORE == FLEX_SCORE_REL_BIAS) slope = fwd::head_slope(p, h);

    const int nq = p.n_qb;
    const int np = min(max(p.q_num[kb], 0), nq), nf = min(max(p.fq_num[kb], 0), nq);
    const int32_t* pcol = p.q_idx + (size_t)kb * nq;
    const int32_t* fcol = p.fq_idx + (size_t)kb * nq;
    for (int t = 0; t < np + nf; ++t) {
      const int qb = min(max(t < np ? pcol[t] : fcol[t - np], 0), nq - 1);
      const int q0 = qb * QB, nrows = min(QB, p.q_len - q0);
      for (int c0 = 0; c0 < nrows; c0 += SUB) {
      const int n = min(SUB, nrows - c0), r0 = q0 + c0;
      __syncthreads();  // every lane is done with the previous rows
      stage_rows<D, NT>(qt, qg, r0, n);
      stage_rows<DV, NT>(dt, dog, r0, n);
      for (int i = tid; i < n; i += NT) {
        FLEXATTN_LDS(float, rt + 4 * i) = p.lse[head_q + r0 + i];
        FLEXATTN_LDS(float, rt + 4 * (SUB + i)) = p.ws[head_q + r0 + i];
      }
      __syncthreads();
      for (int i = 0; i < n; ++i) {
        f32x4 qq[NM], dd[NMV];
        float sd = 0.f, sp = 0.f;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          qq[m] = FLEXATTN_LDS(f32x4, qt + (i * D + 16 * m + 4 * u) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sd = fmaf(qq[m][e], kv[m][e], sd);
        }
#pragma unroll
        for (int m = 0; m < NMV; ++m) {
          dd[m] = FLEXATTN_LDS(f32x4, dt + (i * DV + 16 * m + 4 * u) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) sp = fmaf(dd[m][e], vv[m][e], sp);
        }
        sd = sum4(sd);
        sp = sum4(sp);
        const int qi = r0 + i;
        const float lse = FLEXATTN_LDS(float, rt + 4 * i);
        const float ndelta = FLEXATTN_LDS(float, rt + 4 * (SUB + i));
        float s = p.scale * sd;
        if constexpr (SCORE == FLEX_SCORE_REL_BIAS) s -= slope * (float)(qi - kk);
        const bool vis = live && qi >= qlo && qi <= qhi && lse != -INFINITY;
        const float pr = vis ? expf(s - lse) : 0.f;
        const float ds = pr * (sp + ndelta);
#pragma unroll
        for (int m = 0; m < NMV; ++m) dv[m] += pr * dd[m];
#pragma unroll
        for (int m = 0; m < NM; ++m) dk[m] += ds * qq[m];
      }
      }
    }
    if (!key_ok) return;
    float fk = p.scale, fv = 1.0f;
    if constexpr (MASK == FLEX_MASK_DOCUMENT)
      if (fwd::doc_poisoned(qlo, qhi)) fk = fv = fwd::opaque_nan();
    store_quarter<D>(p.dk, p.grad_bf16 != 0, head_kv + kk, u, dk, fk);
    store_quarter<DV>(p.dv, p.grad_bf16 != 0, head_kv + kk, u, dv, fv);
  }
};

#undef FLEXATTN_LDS

template <int D, int DV, int QB, int KB, int MASK, int SCORE>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Fp32BwdDq<D, DV, QB, KB, MASK, SCORE>::NT)))
void bwd32_dq_kernel(BwdParams p) {
  Fp32BwdDq<D, DV, QB, KB, MASK, SCORE>::run(p);
}

template <int D, int DV, int QB, int KB, int MASK, int SCORE>
__global__ __attribute__((amdgpu_flat_work_group_size(1, Fp32BwdDkv<D, DV, QB, KB, MASK, SCORE>::NT)))
void bwd32_dkv_kernel(BwdParams p) {
  Fp32BwdDkv<D, DV, QB, KB, MASK, SCORE>::run(p);
}

template <int D, int DV, int QB, int KB, int MASK, int SCORE>
hipError_t launch_bwd32_one(const BwdParams& p, hipStream_t s) {
  const long long rows = (long long)p.B * p.H * p.q_len;
  if (rows > 0) {
    const long long threads = rows * (DV / 4);
    hipLaunchKernelGGL(bwd32_pre_kernel<DV>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dq == nullptr: WRITE_DQ off, the dq kernel is skipped
  const long long nq = p.dq != nullptr ? (long long)p.B * p.H * p.n_qb : 0;
  if (nq > 0) {
    hipLaunchKernelGGL((bwd32_dq_kernel<D, DV, QB, KB, MASK, SCORE>), dim3((unsigned)nq),
                       dim3(Fp32BwdDq<D, DV, QB, KB, MASK, SCORE>::NT), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long nkv = (long long)p.B * p.H * p.n_kb;
  if (nkv > 0) {
    hipLaunchKernelGGL((bwd32_dkv_kernel<D, DV, QB, KB, MASK, SCORE>), dim3((unsigned)nkv),
                       dim3(Fp32BwdDkv<D, DV, QB, KB, MASK, SCORE>::NT), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D, int DV, int QB, int KB, int MASK>
hipError_t bwd32_pick_score(const BwdParams& p, int score, hipStream_t s) {
  if (score == FLEX_SCORE_REL_BIAS) return launch_bwd32_one<D, DV, QB, KB, MASK, FLEX_SCORE_REL_BIAS>(p, s);
  return launch_bwd32_one<D, DV, QB, KB, MASK, FLEX_SCORE_IDENTITY>(p, s);
}

template <int D, int DV, int QB, int KB>
hipError_t bwd32_pick_mask(const BwdParams& p, int mask, int score, hipStream_t s) {
  switch (mask) {
    case FLEX_MASK_NOOP:
      return bwd32_pick_score<D, DV, QB, KB, FLEX_MASK_NOOP>(p, score, s);
    case FLEX_MASK_CAUSAL:
      return bwd32_pick_score<D, DV, QB, KB, FLEX_MASK_CAUSAL>(p, score, s);
    case FLEX_MASK_SLIDING_WINDOW:
      return bwd32_pick_score<D, DV, QB, KB, FLEX_MASK_SLIDING_WINDOW>(p, score, s);
    case FLEX_MASK_DOCUMENT:
    case FLEX_MASK_DOCUMENT_CAUSAL:
      return bwd32_pick_score<D, DV, QB, KB, FLEX_MASK_DOCUMENT>(p, score, s);
    default:
      return bwd32_pick_score<D, DV, QB, KB, FLEX_MASK_PREFIX_CAUSAL>(p, score, s);
  }
}

}  // namespace bwd32
}  // namespace flexattn

#define FLEXATTN_BWD32_UNIT(NAME, D, DV, QB, KB)                              \
  namespace flexattn {                                                      \
  hipError_t NAME(const BwdParams& p, int mask, int score, hipStream_t s) { \
    return bwd32::bwd32_pick_mask<D, DV, QB, KB>(p, mask, score, s);        \
  }                                                                         \
  }
