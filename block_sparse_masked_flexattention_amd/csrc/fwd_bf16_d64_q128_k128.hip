// bf16 inputs, head dim 64, 128x128 tiles: kernel instances of fwd_kernel.hpp.
#include "fwd_kernel.hpp"

FLEXATTN_FWD_UNIT(launch_fwd_bf16_d64_q128_k128, true, 64, 64, 128, 128)
