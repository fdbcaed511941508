// fp32 inputs, head dim 64, 128x128 tiles: backward kernel instances of bwd_fp32.hpp.
#include "bwd_fp32.hpp"

FLEXATTN_BWD32_UNIT(launch_bwd_fp32_d64_q128_k128, 64, 64, 128, 128)
