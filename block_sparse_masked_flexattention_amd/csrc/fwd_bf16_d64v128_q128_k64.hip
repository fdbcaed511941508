// bf16 inputs, head dim 64 with value head dim 128, 128x64 tiles: kernel
// instances of fwd_kernel.hpp.
#include "fwd_kernel.hpp"

FLEXATTN_FWD_UNIT(launch_fwd_bf16_d64v128_q128_k64, true, 64, 128, 128, 64)
