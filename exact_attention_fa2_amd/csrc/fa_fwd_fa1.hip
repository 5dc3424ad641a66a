// C ABI of the FlashAttention-1 loop-order ablation (fa_fwd_fa1_order).
#include <hip/hip_runtime.h>

#include "fa.h"
#include "fa_check.h"
#include "fa_fwd_fa1.h"

namespace fa {
namespace {

template <int D>
int64_t fa1_bytes(int B, int H, int N) {
  return Fa1Layout<D>::bytes(B, H, N);
}

int64_t fa1_workspace(int B, int H, int N, int d) {
  switch (d) {
    case 64: return fa1_bytes<64>(B, H, N);
    case 96: return fa1_bytes<96>(B, H, N);
    case 128: return fa1_bytes<128>(B, H, N);
    case 256: return fa1_bytes<256>(B, H, N);
    default: return -1;
  }
}

template <int D, int DT, bool CAUSAL>
int launch(const FwdArgs& a, float* ws, hipStream_t st) {
  (void)hipGetLastError();
  hipLaunchKernelGGL((fa_fwd_fa1_kernel<D, DT, CAUSAL>), dim3(a.B * a.H), dim3(256), 0, st, a, ws);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int D, int DT>
int pick_c(const FwdArgs& a, float* ws, bool causal, hipStream_t st) {
  return causal ? launch<D, DT, true>(a, ws, st) : launch<D, DT, false>(a, ws, st);
}

template <int DT>
int pick_d(const FwdArgs& a, float* ws, int d, bool causal, hipStream_t st) {
  switch (d) {
    case 64: return pick_c<64, DT>(a, ws, causal, st);
    case 96: return pick_c<96, DT>(a, ws, causal, st);
    case 128: return pick_c<128, DT>(a, ws, causal, st);
    case 256: return pick_c<256, DT>(a, ws, causal, st);
    default: return FA_ERR_UNSUPPORTED;
  }
}

}  // namespace
}  // namespace fa

using namespace fa;

extern "C" {

int64_t fa_fwd_fa1_workspace_bytes(int B, int H, int N, int d) {
  int64_t elems = 0;
  if (check_problem(B, H, N, d, 1.f, FA_F16, &elems) != FA_OK) return -1;
  if (elems == 0) return 0;
  return fa1_workspace(B, H, N, d);
}

int fa_fwd_fa1_order(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                     int B, int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  int64_t elems = 0;
  int rc = check_problem(B, H, N, d, scale, dtype, &elems);
  if (rc != FA_OK) return rc;
  if (elems == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace) ||
      (reinterpret_cast<uintptr_t>(lse) & 3))
    return FA_ERR_ALIGN;
  if ((int64_t)B * H > (INT64_C(1) << 30)) return FA_ERR_DIM;
  const int64_t nbytes = elems * 2, lbytes = (elems / d) * 4, wbytes = fa1_workspace(B, H, N, d);
  const void* ins[3] = {q, k, v};
  for (const void* in : ins)
    if (overlap(o, nbytes, in, nbytes) || overlap(lse, lbytes, in, nbytes) ||
        overlap(workspace, wbytes, in, nbytes))
      return FA_ERR_ALIAS;
  if (overlap(lse, lbytes, o, nbytes) || overlap(workspace, wbytes, o, nbytes) ||
      overlap(workspace, wbytes, lse, lbytes))
    return FA_ERR_ALIAS;
  if ((rc = device_ok()) != FA_OK) return rc;

  FwdArgs a = contiguous_args(q, k, v, o, lse, B, H, N, d, scale);
  return dtype == FA_BF16
             ? pick_d<DT_BF16>(a, static_cast<float*>(workspace), d, causal != 0, static_cast<hipStream_t>(stream))
             : pick_d<DT_F16>(a, static_cast<float*>(workspace), d, causal != 0, static_cast<hipStream_t>(stream));
}

}  // extern "C"
