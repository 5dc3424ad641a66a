// Host-side launchers shared by the C-ABI layer (arguments already validated).
#pragma once
#include <hip/hip_runtime.h>

#include "fa_fwd_kernel.h"

namespace fa {
// Picks the forward kernel variant for (d, dtype, causal, sequence length)
// and launches it on `st`. Returns FA_OK or FA_ERR_LAUNCH / FA_ERR_UNSUPPORTED.
int launch_fwd(FwdArgs a, int d, int dtype, bool causal, hipStream_t st);

// The small-grid forward kernels, built in a translation unit of their own
// (fa_fwd_small.hip) under another instruction-scheduling strategy:
//  * the key-split kernel with `ns` waves per 32-row unit (d = 64 or 128,
//    dt = DT_F16 or DT_BF16, ns = 4, or 8 at d = 64);
//  * the 8-wave bf16 d = 64 non-causal kernel that sums the weights by MFMA.
int launch_fwd_split(FwdArgs a, int d, int dt, bool causal, int ns, hipStream_t st);
int launch_fwd_mfma_sums(FwdArgs a, hipStream_t st);
}  // namespace fa
