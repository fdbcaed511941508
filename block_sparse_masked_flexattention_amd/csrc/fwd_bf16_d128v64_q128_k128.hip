// bf16 inputs, head dim 128 with value head dim 64, 128x128 tiles: kernel
// instances of fwd_kernel.hpp.
#include "fwd_kernel.hpp"

FLEXATTN_FWD_UNIT(launch_fwd_bf16_d128v64_q128_k128, true, 128, 64, 128, 128)
