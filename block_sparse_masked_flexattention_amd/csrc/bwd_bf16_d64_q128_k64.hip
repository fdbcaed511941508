// bf16 inputs, head dim 64, 128x64 tiles: backward kernel instances of bwd_bf16.hpp.
#include "bwd_bf16.hpp"

FLEXATTN_BWD_UNIT(launch_bwd_bf16_d64_q128_k64, 64, 64, 128, 64)
