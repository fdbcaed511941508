// fp32 inputs, head dim 64, value head dim 128, 64x64 tiles: backward kernel
// instances of bwd_fp32.hpp.
#include "bwd_fp32.hpp"

FLEXATTN_BWD32_UNIT(launch_bwd_fp32_d64v128_q64_k64, 64, 128, 64, 64)
