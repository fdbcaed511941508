// bf16 inputs, head dim 128, value head dim 64, 128x64 tiles: backward kernel
// instances of bwd_bf16.hpp.
#include "bwd_bf16.hpp"

FLEXATTN_BWD_UNIT(launch_bwd_bf16_d128v64_q128_k64, 128, 64, 128, 64)
