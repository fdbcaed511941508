// noalloc.hip -- the backward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): flex_attn_bwd with its workspace taken from a
// file-scope device array instead of the caller.
#include <mutex>

#include "internal.hpp"

namespace flexattn {
namespace {

// The backward's per-row terms (-delta and the lse in raw-score units, two
// floats per query row) for every call of flex_attn_bwd_noalloc on a GPU.
// Each GPU the library runs on holds its own copy until the process ends.
constexpr int64_t kNoAllocScratchFloats = FLEX_NOALLOC_SCRATCH_FLOATS;
__device__ __align__(256) float scratch[kNoAllocScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's copy of `scratch`, looked up once per
// device with that device current.  (In host code the array's name is a
// host-side stand-in, not a device address.)
hipError_t scratch_for_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace flexattn

extern "C" int32_t flex_attn_bwd_noalloc(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, const float* dlse, int32_t in_dtype, int32_t B, int32_t H,
    int32_t q_len, int32_t kv_len, int32_t head_dim, int32_t v_head_dim,
    const flex_block_mask* bm, const flex_block_mask_t* bmt, const flex_score_desc* score,
    float scale, void* dq, void* dk, void* dv, int32_t grad_dtype, void* stream) {
  if (B < 0 || H < 0 || q_len < 0) return FLEX_E_INVALID_ARG;
  if (2 * (int64_t)B * H * q_len > flexattn::kNoAllocScratchFloats) return FLEX_E_SCRATCH_LIMIT;
  float* ws = nullptr;
  if (flexattn::scratch_for_current_device(&ws) != hipSuccess) return FLEX_E_HIP;
  return flex_attn_bwd(q, k, v, out, dout, lse, dlse, in_dtype, B, H, q_len, kv_len, head_dim,
                       v_head_dim, bm, bmt, score, scale, dq, dk, dv, grad_dtype, ws, stream);
}
