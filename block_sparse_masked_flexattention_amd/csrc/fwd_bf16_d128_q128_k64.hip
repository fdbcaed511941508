// bf16 inputs, head dim 128, 128x64 tiles: kernel instances of fwd_kernel.hpp.
#include "fwd_kernel.hpp"

FLEXATTN_FWD_UNIT(launch_fwd_bf16_d128_q128_k64, true, 128, 128, 128, 64)
