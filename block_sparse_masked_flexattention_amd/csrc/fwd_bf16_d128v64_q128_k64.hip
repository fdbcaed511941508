// bf16 inputs, head dim 128 with value head dim 64, 128x64 tiles: kernel
// instances of fwd_kernel.hpp.
#include "fwd_kernel.hpp"

FLEXATTN_FWD_UNIT(launch_fwd_bf16_d128v64_q128_k64, true, 128, 64, 128, 64)
