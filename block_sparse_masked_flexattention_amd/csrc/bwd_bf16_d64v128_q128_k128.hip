// bf16 inputs, head dim 64, value head dim 128, 128x128 tiles: backward kernel
// instances of bwd_bf16.hpp.
#include "bwd_bf16.hpp"

FLEXATTN_BWD_UNIT(launch_bwd_bf16_d64v128_q128_k128, 64, 128, 128, 128)
