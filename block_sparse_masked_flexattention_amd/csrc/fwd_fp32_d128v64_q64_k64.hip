// fp32 inputs, head dim 128, value head dim 64, 64x64 tiles: kernel instances of
// fwd_kernel.hpp.
#include "fwd_kernel.hpp"

FLEXATTN_FWD_UNIT(launch_fwd_fp32_d128v64_q64_k64, false, 128, 64, 64, 64)
