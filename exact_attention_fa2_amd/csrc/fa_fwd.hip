// Forward kernel instantiations and variant selection.
#include <hip/hip_runtime.h>

#include "fa.h"
#include "fa_fwd_launch.h"
#include "fa_launch.h"

namespace fa {
namespace {

// Variant choice, from same-run measurements on MI355X (kernel time per
// launch): 8 waves (256 query rows) per workgroup whenever the grid fills the
// chip (N=6400 d64: 206 us, N=4096 d64: 293 us, N=400 x128 heads: 15.5 us,
// N=8192 causal d128: 632 us); when B*H*ceil(N/256) is below the 256 CUs,
// 4 waves (128 rows) per workgroup for more parallelism (N=400 x4 heads:
// 9.8 us vs 11.8 us). d=96 uses 4 waves (its registers allow no more); d=256
// uses 4 waves and 32-key tiles.
//
// The key-split kernel (4 waves per 32-row unit, one K/V buffer per wave)
// runs while its B*H*ceil(N/32) workgroups all fit the chip at once: at most
// 512 at d=64 (64 KB of LDS each, two per CU), 256 at d=128 (128 KB, one per
// CU). Against the 4-wave kernel, same GPU: d=64 N=400 x4 heads 8.1 vs
// 9.8 us, N=4096 x2 heads 30.4 vs 56.6 us, N=512 x32 heads 11.0 vs 11.9 us;
// d=128 N=2048 x4 heads 33.2 vs 46.4 us, N=4096 x2 heads causal 52.2 vs
// 85.1 us, N=400 x8 heads 12.8 vs 14.2 us. Past that size it loses (d=64
// N=512 x64 heads 19.8 vs 13.5 us; d=128 N=1024 x16 heads 38.0 vs 27.4 us):
// each K/V tile is reused 4x less, and a second round of workgroups follows
// the first.
template <int D, int DT, bool CAUSAL>
int pick(FwdArgs a, hipStream_t st) {
  const int64_t wg256 = (int64_t)a.B * a.H * ((a.N + 255) / 256);
  if constexpr (D == 64 || D == 128) {
    // key-split kernel while all its workgroups fit the chip at once (64 KB
    // of LDS each at d=64: two per CU; 128 KB at d=128: one); at d=64 with
    // rows of 16 tiles or more, 8 waves per unit (128 KB: one per CU)
    const int64_t units = (int64_t)a.B * a.H * ((a.N + 31) / 32);
    if constexpr (D == 64)
      if (units <= 256 && a.N >= 1024) return launch_fwd_split(a, D, DT, CAUSAL, 8, st);
    constexpr int64_t kSplitMax = D == 64 ? 512 : 256;
    if (units <= kSplitMax) return launch_fwd_split(a, D, DT, CAUSAL, 4, st);
  }
  if constexpr (D == 96 || D == 256) {
    // key split over 4 waves, padded rows by LDS-DMA (100 / 140 KB of LDS:
    // one workgroup per CU), while every unit's workgroup fits the chip at once
    if ((int64_t)a.B * a.H * ((a.N + 31) / 32) <= 256) return launch_fwd_split(a, D, DT, CAUSAL, 4, st);
  }
  if constexpr (D == 64 || D == 128) {
    if (wg256 < 256) return launch_one<D, DT, CAUSAL, 4, 1, 64, k_prefetch<D, DT, 4>()>(a, st);
  }
  if constexpr (D == 64) {
    // maps of at most 128 rows: 2 heads (4 up to 64 rows) per workgroup, all
    // of their K and V loaded at once (B=64 x16 heads N=64 fp16: 10.4 vs
    // 13.3 us; B=64 x8 heads N=100 bf16: 10.8 vs 12.7 us). Longer maps keep
    // the kernels below: one head per workgroup with its whole K/V in LDS
    // lost at N=400 x128 heads (16.5 vs 14.6 us bf16, 16.1 vs 14.4 us fp16).
    if (a.cu_seqlens == nullptr && a.N <= 128)
      return a.N <= 64 ? launch_resident<D, DT, CAUSAL, 4>(a, st) : launch_resident<D, DT, CAUSAL, 2>(a, st);
  }
  if constexpr (D == 64 && CAUSAL) {
    // causal, at most 2048 units of 32 rows: 16-row units in 4-wave
    // workgroups (N=400 x128 heads bf16: 11.3 vs 14.9 us; N=256 x256 heads
    // fp16: 10.4 vs 12.7 us; N=1000 x64 heads fp16: 20.0 vs 25.2 us). With
    // more units they lose (N=400 x256 heads fp16: 19.3 vs 18.3 us); without
    // the mask the units are equal and the 32-row kernels are as fast or
    // faster (N=400 x128 heads: 14.8 vs 15.0 us; x256 fp16: 26.3 vs 24.8).
    if (a.cu_seqlens == nullptr && (int64_t)a.B * a.H * ((a.N + 31) / 32) <= 2048)
      return launch_fwd16<D, DT, CAUSAL, 4>(a, st);
  }
  if constexpr (D == 64 && DT == DT_BF16 && !CAUSAL) {
    // at most two 32-row units of work per SIMD (1024 SIMDs): the weight
    // sums by MFMA (N=400 x128 heads: 14.7-15.4 vs 15.0-15.8 us; with the
    // chip full they cost 1.5-5 %)
    if (a.cu_seqlens == nullptr && (int64_t)a.B * a.H * ((a.N + 31) / 32) <= 2048)
      return launch_fwd_mfma_sums(a, st);
  }
  if constexpr (D == 256)
    return launch_one<D, DT, CAUSAL, 4, 1, 32, k_prefetch<D, DT, 4>()>(a, st);
  else if constexpr (D == 96)
    return launch_one<D, DT, CAUSAL, 4, 1, 64, k_prefetch<D, DT, 4>()>(a, st);
  else
    return launch_one<D, DT, CAUSAL, 8, 1, 64, k_prefetch<D, DT, 8>()>(a, st);
}

template <int D, int DT>
int pick_causal(FwdArgs a, bool causal, hipStream_t st) {
  return causal ? pick<D, DT, true>(a, st) : pick<D, DT, false>(a, st);
}

template <int DT>
int pick_d(FwdArgs a, int d, bool causal, hipStream_t st) {
  switch (d) {
    case 64: return pick_causal<64, DT>(a, causal, st);
    case 96: return pick_causal<96, DT>(a, causal, st);
    case 128: return pick_causal<128, DT>(a, causal, st);
    case 256: return pick_causal<256, DT>(a, causal, st);
    default: return FA_ERR_UNSUPPORTED;
  }
}

}  // namespace

int launch_fwd(FwdArgs a, int d, int dtype, bool causal, hipStream_t st) {
  return dtype == FA_BF16 ? pick_d<DT_BF16>(a, d, causal, st) : pick_d<DT_F16>(a, d, causal, st);
}

}  // namespace fa
