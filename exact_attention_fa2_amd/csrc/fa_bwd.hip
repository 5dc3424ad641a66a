// C ABI of the backward pass (fa_bwd, fa_bwd_workspace_bytes).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "fa.h"
#include "fa_bwd_kernel.h"
#include "fa_check.h"

namespace fa {
namespace {

int64_t bwd_bytes(int B, int H, int N) {
  return ((int64_t)B * H * N * 4 + 255) / 256 * 256;  // D_i in fp32
}

// Compute units of the current device, queried once (256 on MI355X; 0 if
// the query fails, which keeps the two-kernel sequence).
int cu_count() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    return cus;
  }();
  return n;
}

// Kernels per head dim, each at the occupancy its registers allow:
//  * dK/dV in one pass with V fragments parked in LDS: d = 128 in 8-wave,
//    256-key blocks (two waves per SIMD), d = 64 in 4-wave, 128-key blocks
//    (three); d = 96 in two passes, dV then dK.
//  * dQ with K/V tiles by LDS-DMA: 8 waves at d = 128, 4 at d = 64 (dO
//    fragments in LDS, three waves per SIMD); the register-staged kernel at
//    d = 96 and 256.
//  * d = 256 takes the d = 96 sequence at one wave per SIMD: the two dK/dV
//    passes and the dQ kernel each hold 128 accumulator registers.
//  * d = 96 and 256 with at most one block of each kind per CU: after D_i,
//    one joint grid of the dQ, dV-pass and dK-pass blocks (d = 96 B1 H4
//    N2048 139 -> 53 us, d = 256 B1 H4 N2048 382 -> 158 us, same GPU).
//  * d = 64 and 128 with at most one dQ block per CU (B*H*ceil(N/(32 QNW))
//    <= CUs): D_i by fa_bwd_dot_kernel, then one joint grid that interleaves
//    the dQ and dK/dV blocks, so both halves share the chip instead of each
//    leaving half of it idle. Kernel-only, warm, bf16 d = 64, same GPU: B1 H4
//    N4096 151 -> 107 us (causal 159 -> 104), B1 H2 N8192 297 -> 207, B2 H4
//    N400 24.7 -> 17.6, B1 H16 N1024 44.3 -> 31.5; 256 dQ blocks: B2 H8 N2048
//    83.9 -> 75.6, B4 H16 N512 29.9 -> 28.5; 512 (N=400 x128 heads): 35.5 ->
//    43.6, so the larger grids keep the sequence.
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
  if constexpr (D == 96 || D == 256) {
    hipLaunchKernelGGL((fa_bwd_dot_kernel<D, DT>), dim3((unsigned)gdot), dim3(256), 0, st, a);
    if (gk <= cu_count()) {
      // the dQ, dV-pass and dK-pass blocks side by side in one grid
      hipLaunchKernelGGL((fa_bwd_joint_staged_kernel<D, DT, CAUSAL>), dim3((unsigned)(3 * gk)), dim3(256), 0, st, a);
      return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
    }
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, DT, CAUSAL, BWD_DV>), dim3((unsigned)gk), dim3(256), 0, st, a);
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, DT, CAUSAL, BWD_DK>), dim3((unsigned)gk), dim3(256), 0, st, a);
    hipLaunchKernelGGL((fa_bwd_dq_staged_kernel<D, DT, CAUSAL, QNW>), dim3((unsigned)gq), dim3(QNW * 64), 0, st, a);
  } else {
    static_assert(QNW == bwd_joint_waves<D>(), "the joint grid pairs equal dQ and dK/dV grids");
    if (gq <= cu_count()) {
      // each half alone would fill at most one workgroup per CU: D_i first,
      // then the dQ and dK/dV blocks side by side in one grid
      hipLaunchKernelGGL((fa_bwd_dot_kernel<D, DT>), dim3((unsigned)gdot), dim3(256), 0, st, a);
      hipLaunchKernelGGL((fa_bwd_joint_kernel<D, DT, CAUSAL>), dim3((unsigned)(2 * gq)), dim3(QNW * 64), 0, st, a);
      return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
    }
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
    case 256: return pick_c<256, DT>(a, causal, st);
    default: return FA_ERR_UNSUPPORTED;
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

}  // extern "C"

// Scratch of fa_bwd_noalloc: the fp32 row terms D_i of at most
// FA_BWD_NOALLOC_MAX_ROWS rows (B*H*N), 16 MiB. Each device holds its own
// copy for the life of the process. Host code never passes `scratch` itself
// (a host-side stand-in): it takes the device address from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[FA_BWD_NOALLOC_MAX_ROWS];

namespace fa {
namespace {

// Device address of this device's `scratch`, looked up on the first call on
// each device (that device current) and kept; nullptr if the lookup fails.
void* scratch_address() {
  static std::atomic<void*> addr[64];
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = addr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  addr[dev].store(q, std::memory_order_release);
  return q;
}

// Checks shared by fa_bwd and fa_bwd_noalloc (everything but the workspace).
// max_rows > 0 bounds B*H*N (FA_ERR_TOO_LARGE), checked with the sizes,
// before any pointer.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* do_, const float* lse,
              void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int dtype,
              int64_t max_rows, int64_t* elems) {
  int rc = check_problem(B, H, N, d, scale, dtype, elems);
  if (rc != FA_OK) return rc;
  if (*elems == 0) return FA_OK;
  if (max_rows > 0 && *elems / d > max_rows) return FA_ERR_TOO_LARGE;
  if (!q || !k || !v || !o || !do_ || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  const void* a16[8] = {q, k, v, o, do_, dq, dk, dv};
  for (const void* p : a16)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(lse) & 3) return FA_ERR_ALIGN;
  const int64_t nb = *elems * 2, lb = (*elems / d) * 4;
  const void* ins[6] = {q, k, v, o, do_, lse};
  const int64_t insz[6] = {nb, nb, nb, nb, nb, lb};
  void* outs[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlap(outs[i], nb, ins[j], insz[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], nb, outs[j], nb)) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* do_, const float* lse,
            void* dq, void* dk, void* dv, float* dvec, int B, int H, int N, int d, float scale, int causal,
            int dtype, void* stream) {
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
  a.dvec = dvec;
  a.B = B;
  a.H = H;
  a.N = N;
  a.c = std::fmax(std::fabs(scale) * kLog2e, 1e-30f);
  a.scale = scale;
  a.qsign = scale < 0.f ? 0x80008000u : 0u;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return dtype == FA_BF16 ? pick_d<DT_BF16>(a, d, causal != 0, st) : pick_d<DT_F16>(a, d, causal != 0, st);
}

}  // namespace
}  // namespace fa

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* do_, const float* lse,
           void* dq, void* dk, void* dv, void* workspace, int B, int H, int N, int d, float scale,
           int causal, int dtype, void* stream) {
  int64_t elems = 0;
  int rc = check_bwd(q, k, v, o, do_, lse, dq, dk, dv, B, H, N, d, scale, dtype, 0, &elems);
  if (rc != FA_OK || elems == 0) return rc;
  if (!workspace) return FA_ERR_NULL;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  const int64_t nb = elems * 2, lb = (elems / d) * 4, wb = bwd_bytes(B, H, N);
  const void* other[9] = {q, k, v, o, do_, dq, dk, dv, lse};
  for (int j = 0; j < 9; ++j)
    if (overlap(workspace, wb, other[j], j == 8 ? lb : nb)) return FA_ERR_ALIAS;
  if ((rc = device_ok()) != FA_OK) return rc;
  return run_bwd(q, k, v, o, do_, lse, dq, dk, dv, static_cast<float*>(workspace), B, H, N, d, scale, causal,
                 dtype, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* do_,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                   int causal, int dtype, void* stream) {
  int64_t elems = 0;
  int rc = check_bwd(q, k, v, o, do_, lse, dq, dk, dv, B, H, N, d, scale, dtype, FA_BWD_NOALLOC_MAX_ROWS,
                     &elems);
  if (rc != FA_OK || elems == 0) return rc;
  if ((rc = device_ok()) != FA_OK) return rc;
  void* ws = scratch_address();
  if (ws == nullptr) return FA_ERR_DEVICE;
  // every D_i the kernels read is written first in the same call, so the
  // previous call's contents need no clearing
  return run_bwd(q, k, v, o, do_, lse, dq, dk, dv, static_cast<float*>(ws), B, H, N, d, scale, causal, dtype,
                 stream);
}

}  // extern "C"
