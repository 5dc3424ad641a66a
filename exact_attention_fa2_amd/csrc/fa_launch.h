// Host-side launchers shared by the C-ABI layer (arguments already validated).
#pragma once
#include <hip/hip_runtime.h>

#include "fa_fwd_kernel.h"

namespace fa {
// Picks the forward kernel variant for (d, dtype, causal, sequence length)
// and launches it on `st`. Returns FA_OK or FA_ERR_LAUNCH / FA_ERR_UNSUPPORTED.
int launch_fwd(FwdArgs a, int d, int dtype, bool causal, hipStream_t st);
}  // namespace fa
