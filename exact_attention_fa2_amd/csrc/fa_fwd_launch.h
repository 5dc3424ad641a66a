// Host-side launch helpers of the forward kernels: blocks per head, the
// launch of one main-kernel variant, the launch of the key-split kernel.
// Internal linkage: each translation unit that includes this header
// instantiates its own kernels, so that no kernel is compiled twice under
// different code-generation options.
#pragma once
#include <hip/hip_runtime.h>

#include "fa.h"
#include "fa_fwd_kernel.h"
#include "fa_fwd16.h"
#include "fa_fwd_resident.h"
#include "fa_fwd_split.h"

namespace fa {
namespace {


// Blocks per head for `units` 32-row units over blocks of at most `nw`
// waves. The fewest blocks that cover the units, unless those workgroups
// fill the resident slots unevenly (some CUs holding one, some two): then
// more blocks of fewer units, as long as all stay resident at once, when that
// lowers the units the busiest CU holds, ceil(bh*n / cus) * units / n.
// N=6400 x16 heads d=64: 400 workgroups of 8 units for 512 slots (201 us)
// -> 512 of 6-7 units (193 us).
int balanced_blocks(int64_t bh, int units, int nw, int cus, int per_cu) {
  int best = (units + nw - 1) / nw;
  if (cus <= 0 || per_cu <= 0) return best;
  auto cost = [&](int n) { return (double)((bh * n + cus - 1) / cus) * units / n; };
  double best_cost = cost(best);
  for (int n = best + 1; n <= units && bh * n <= (int64_t)cus * per_cu; ++n)
    if (cost(n) < best_cost - 1e-9) {
      best = n;
      best_cost = cost(n);
    }
  return best;
}

template <int D, int DT, bool CAUSAL, int NW, int QB, int BC, int PF, bool LS = false>
int launch_one(FwdArgs a, hipStream_t st) {
  // 32-row units spread evenly over the blocks of a head (N = 400 on 4-wave
  // blocks: 3, 3, 3 and 4 units, not 4, 4, 4, 1)
  static_assert(QB == 1, "one 32-row unit per wave");
  a.units = (a.N + 31) / 32;
  a.nqb = (a.units + NW - 1) / NW;
  if (!CAUSAL && !a.cu_seqlens) {
    // CUs and resident workgroups per CU of this kernel, queried once
    static const int2 occ = [] {
      int dev = 0, cus = 0, per = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
          hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fa_fwd_kernel<D, DT, CAUSAL, NW, QB, BC, PF, LS>,
                                                       NW * 64, 0) != hipSuccess)
        return int2{0, 0};
      return int2{cus, per};
    }();
    a.nqb = balanced_blocks((int64_t)a.B * a.H, a.units, NW, occ.x, occ.y);
  }
  const int64_t total = (int64_t)a.B * a.H * a.nqb;
  if (total > (INT64_C(1) << 30)) return FA_ERR_DIM;
  a.total = (int)total;
  const int grid = (a.total + 7) / 8 * 8;  // a multiple of the 8 XCDs
  (void)hipGetLastError();
  hipLaunchKernelGGL((fa_fwd_kernel<D, DT, CAUSAL, NW, QB, BC, PF, LS>), dim3(grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// The head-packed kernel for equal-length maps of at most 32 * 8 / HP rows:
// HP heads per 8-wave workgroup.
template <int D, int DT, bool CAUSAL, int HP>
int launch_resident(FwdArgs a, hipStream_t st) {
  if (a.N > 32 * (8 / HP) || a.cu_seqlens) return FA_ERR_DIM;
  const int64_t groups = ((int64_t)a.B * a.H + HP - 1) / HP;
  if (groups > (INT64_C(1) << 30)) return FA_ERR_DIM;
  const int64_t lds = resident_lds_bytes<D, HP>(a.N);
  static const bool attr = hipFuncSetAttribute((const void*)fa_fwd_resident_kernel<D, DT, CAUSAL, HP>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)resident_lds_bytes<D, HP>(32 * (8 / HP))) == hipSuccess;
  (void)attr;
  (void)hipGetLastError();
  hipLaunchKernelGGL((fa_fwd_resident_kernel<D, DT, CAUSAL, HP>), dim3((unsigned)groups), dim3(512), (unsigned)lds,
                     st, a);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// The 16-row-unit kernel (causal, equal lengths): units of 16 query rows,
// at most NW a block, blocks by rank across heads.
template <int D, int DT, bool CAUSAL, int NW>
int launch_fwd16(FwdArgs a, hipStream_t st) {
  if (a.cu_seqlens || !CAUSAL) return FA_ERR_DIM;
  a.units = (a.N + 15) / 16;
  a.nqb = (a.units + NW - 1) / NW;
  const int64_t total = (int64_t)a.B * a.H * a.nqb;
  if (total > (INT64_C(1) << 30)) return FA_ERR_DIM;
  a.total = (int)total;
  (void)hipGetLastError();
  hipLaunchKernelGGL((fa_fwd16_kernel<D, DT, CAUSAL, NW>), dim3(a.total), dim3(NW * 64), 0, st, a);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Key-split kernel: one workgroup of NS waves per 32-row unit, the unit's
// keys split over the waves. Against 4 waves, 8 waves per unit at d=64
// (same GPU): N=2048 x4 heads 15.9 vs 19.9 us, N=4096 x2 heads causal 23.4
// vs 30.8 us, N=8192 x1 head 39.2 vs 56.7 us; but N=400 x4 heads 8.7 vs
// 8.1 us (7 tiles a row: one per wave, eight partials to merge) and N=400 x32
// heads 16.4 vs 10.4 us (416 workgroups of 128 KB: two rounds).
template <int D, int DT, bool CAUSAL, int NS>
int launch_split(FwdArgs a, hipStream_t st) {
  a.units = (a.N + 31) / 32;
  a.nqb = 1;
  const int64_t total = (int64_t)a.B * a.H * a.units;
  if (total > (INT64_C(1) << 30)) return FA_ERR_DIM;
  a.total = (int)total;
  const int grid = (a.total + 7) / 8 * 8;
  (void)hipGetLastError();
  hipLaunchKernelGGL((fa_fwd_split_kernel<D, DT, CAUSAL, NS, 1, 2>), dim3(grid), dim3(NS * 64), 0, st, a);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// K fragments are read two k-steps ahead of their MFMAs (PF = 2) wherever
// that costs no occupancy: N=400 x4 heads fp16 -2 %, N=8192 causal d128
// -1 %, N=400 x128 heads bf16 unchanged. The 8-wave fp16 d=64 kernel would
// need 135 VGPRs instead of 127 and drop from 4 to 3 waves per SIMD (N=4096:
// +7 %), so it keeps the compiler's schedule.
template <int D, int DT, int NW>
constexpr int k_prefetch() {
  return (D == 64 && DT == DT_F16 && NW == 8) ? 0 : 2;
}

}  // namespace
}  // namespace fa
