// bf16 inputs, head dim 64, value head dim 128, 64x64 tiles: backward kernel
// instances of bwd_bf16.hpp.
#include "bwd_bf16.hpp"

FLEXATTN_BWD_UNIT(launch_bwd_bf16_d64v128_q64_k64, 64, 128, 64, 64)
