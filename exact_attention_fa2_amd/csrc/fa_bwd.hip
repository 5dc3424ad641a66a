// C ABI of the backward pass (fa_bwd, fa_bwd_workspace_bytes).
#include <hip/hip_runtime.h>

#include <cmath>

#include "fa.h"
#include "fa_bwd_kernel.h"
#include "fa_check.h"

namespace fa {
namespace {

int64_t bwd_bytes(int B, int H, int N) {
  return ((int64_t)B * H * N * 4 + 255) / 256 * 256;  // D_i in fp32
}

// Kernels per head dim, each at the occupancy its registers allow:
//  * dK/dV in one pass with V fragments parked in LDS: d = 128 in 8-wave,
//    256-key blocks (two waves per SIMD), d = 64 in 4-wave, 128-key blocks
//    (three); d = 96 in two passes, dV then dK.
//  * dQ with K/V tiles by LDS-DMA: 8 waves at d = 128, 4 at d = 64 (dO
//    fragments in LDS, three waves per SIMD); the register-staged kernel at
//    d = 96.
// Every kernel orders its blocks key/query block major, head minor.
// Measured per backward, same GPU, against the earlier two-pass dK/dV
// (d = 128) or fused dK/dV with K/V fragments in registers (d = 64), the
// register-staged dQ and the head-major order: N=8192 causal bf16 d=128
// 4610 -> 1936 us, B4 H16 N4096 fp16 d=64 1203 -> 1048 us, N=400 x128 heads
// bf16 54.1 -> 49.3 us.
template <int D, int DT, bool CAUSAL>
int launch(const BwdArgs& a, hipStream_t st) {
  constexpr int QNW = D == 128 ? 8 : 4;
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const int64_t gdot = (rows * bwd_dot_lanes<D>() + 255) / 256;
  const int64_t gk = (int64_t)a.B * a.H * ((a.N + 127) / 128);
  const int64_t gq = (int64_t)a.B * a.H * ((a.N + 32 * QNW - 1) / (32 * QNW));
  if (gdot > (INT64_C(1) << 31) - 1 || gk > (INT64_C(1) << 31) - 1 || gq > (INT64_C(1) << 31) - 1)
    return FA_ERR_DIM;
  (void)hipGetLastError();
  if constexpr (D == 96) {
    hipLaunchKernelGGL((fa_bwd_dot_kernel<D, DT>), dim3((unsigned)gdot), dim3(256), 0, st, a);
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, DT, CAUSAL, BWD_DV>), dim3((unsigned)gk), dim3(256), 0, st, a);
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, DT, CAUSAL, BWD_DK>), dim3((unsigned)gk), dim3(256), 0, st, a);
    hipLaunchKernelGGL((fa_bwd_dq_staged_kernel<D, DT, CAUSAL, QNW>), dim3((unsigned)gq), dim3(QNW * 64), 0, st, a);
  } else {
    // dQ first: it also forms and stores D_i, which dK/dV reads
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, DT, CAUSAL, QNW>), dim3((unsigned)gq), dim3(QNW * 64), 0, st, a);
    if constexpr (D == 128) {
      const int64_t gw = (int64_t)a.B * a.H * ((a.N + 255) / 256);
      hipLaunchKernelGGL((fa_bwd_dkdv_wide_kernel<D, DT, CAUSAL, 8, 1>), dim3((unsigned)gw), dim3(512), 0, st, a);
    } else {
      hipLaunchKernelGGL((fa_bwd_dkdv_wide_kernel<D, DT, CAUSAL, 4, 3>), dim3((unsigned)gk), dim3(256), 0, st, a);
    }
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int D, int DT>
int pick_c(const BwdArgs& a, bool causal, hipStream_t st) {
  return causal ? launch<D, DT, true>(a, st) : launch<D, DT, false>(a, st);
}

template <int DT>
int pick_d(const BwdArgs& a, int d, bool causal, hipStream_t st) {
  switch (d) {
    case 64: return pick_c<64, DT>(a, causal, st);
    case 96: return pick_c<96, DT>(a, causal, st);
    case 128: return pick_c<128, DT>(a, causal, st);
    default: return FA_ERR_UNSUPPORTED;  // d = 256: the dK/dV accumulators do not fit
  }
}

}  // namespace
}  // namespace fa

using namespace fa;

extern "C" {

int64_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  int64_t elems = 0;
  if (check_problem(B, H, N, d, 1.f, FA_F16, &elems) != FA_OK) return -1;
  if (elems == 0) return 0;
  return bwd_bytes(B, H, N);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* do_, const float* lse,
           void* dq, void* dk, void* dv, void* workspace, int B, int H, int N, int d, float scale,
           int causal, int dtype, void* stream) {
  int64_t elems = 0;
  int rc = check_problem(B, H, N, d, scale, dtype, &elems);
  if (rc != FA_OK) return rc;
  if (d == 256) return FA_ERR_UNSUPPORTED;
  if (elems == 0) return FA_OK;
  if (!q || !k || !v || !o || !do_ || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
  const void* a16[8] = {q, k, v, o, do_, dq, dk, dv};
  for (const void* p : a16)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(lse) & 3)) return FA_ERR_ALIGN;
  const int64_t nb = elems * 2, lb = (elems / d) * 4, wb = bwd_bytes(B, H, N);
  const void* ins[6] = {q, k, v, o, do_, lse};
  const int64_t insz[6] = {nb, nb, nb, nb, nb, lb};
  void* outs[4] = {dq, dk, dv, workspace};
  const int64_t outsz[4] = {nb, nb, nb, wb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_ALIAS;
  }
  if ((rc = device_ok()) != FA_OK) return rc;

  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(do_);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.dvec = static_cast<float*>(workspace);
  a.B = B;
  a.H = H;
  a.N = N;
  a.c = std::fmax(std::fabs(scale) * kLog2e, 1e-30f);
  a.scale = scale;
  a.qsign = scale < 0.f ? 0x80008000u : 0u;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dtype == FA_BF16 ? pick_d<DT_BF16>(a, d, causal != 0, st) : pick_d<DT_F16>(a, d, causal != 0, st);
}

}  // extern "C"
