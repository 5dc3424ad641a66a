// The small-grid forward kernels: the key-split kernel and the bf16 d = 64
// kernel with MFMA weight sums. The build compiles this file with the
// scheduler's max-ILP strategy. Against the default strategy, same GPU, four
// alternations each: N=400 x128 heads bf16 14.3-14.7 vs 15.3-15.6 us, N=400 x4
// heads fp16 7.93-7.95 vs 8.04-8.09 us. The large-grid kernels in fa_fwd.hip
// keep the default, which is faster there (N=8192 causal d=128: 562 vs
// 572-581 us; N=6400: 199 vs 202-204 us).
#include <hip/hip_runtime.h>

#include "fa.h"
#include "fa_fwd_launch.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D, int DT>
int split_c(FwdArgs a, bool causal, int ns, hipStream_t st) {
  if constexpr (D == 64) {
    if (ns == 8) return causal ? launch_split<D, DT, true, 8>(a, st) : launch_split<D, DT, false, 8>(a, st);
  }
  if (ns != 4) return FA_ERR_UNSUPPORTED;
  return causal ? launch_split<D, DT, true, 4>(a, st) : launch_split<D, DT, false, 4>(a, st);
}

template <int D>
int split_dt(FwdArgs a, int dt, bool causal, int ns, hipStream_t st) {
  return dt == DT_BF16 ? split_c<D, DT_BF16>(a, causal, ns, st) : split_c<D, DT_F16>(a, causal, ns, st);
}

}  // namespace

int launch_fwd_split(FwdArgs a, int d, int dt, bool causal, int ns, hipStream_t st) {
  switch (d) {
    case 64: return split_dt<64>(a, dt, causal, ns, st);
    case 96: return split_dt<96>(a, dt, causal, ns, st);
    case 128: return split_dt<128>(a, dt, causal, ns, st);
    case 256: return split_dt<256>(a, dt, causal, ns, st);
    default: return FA_ERR_UNSUPPORTED;
  }
}

int launch_fwd_mfma_sums(FwdArgs a, hipStream_t st) {
  return launch_one<64, DT_BF16, false, 8, 1, 64, k_prefetch<64, DT_BF16, 8>(), true>(a, st);
}

}  // namespace fa
