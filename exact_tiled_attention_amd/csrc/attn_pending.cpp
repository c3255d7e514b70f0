// attn_pending.cpp -- launchers whose kernels are not in this build yet report
// hipErrorNotSupported (surfaced as ATTN_ERR_HIP).
#include "attn_launch.h"

hipError_t attn_launch_fwd_fp8(const Fp8Args&, hipStream_t) { return hipErrorNotSupported; }
int attn_fp8_tile_keys() { return 64; }
