// fp32 inputs, head dim 64, value head dim 128, 128x128 tiles: backward kernel
// instances of bwd_fp32.hpp.
#include "bwd_fp32.hpp"

FLEXATTN_BWD32_UNIT(launch_bwd_fp32_d64v128_q128_k128, 64, 128, 128, 128)
