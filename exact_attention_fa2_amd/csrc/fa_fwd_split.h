// Forward with the keys of each 32-row query unit split over the waves of a
// workgroup, for grids too small to fill the chip (a few heads of a short
// map, or a few heads of a long sequence).
//
// The mathematics is that of fa_fwd_kernel: tiles, the online softmax with a
// running max and sum ("FlashAttention explainer" (aitangshan.cn) sections
// 4.2-4.3). The split is the same rescale algebra applied once more: each
// wave ends with a partial (acc, m, l) over its own keys, and partials merge
// exactly as acc = sum_s 2^(m_s - m) acc_s, l = sum_s 2^(m_s - m) l_s with
// m = max_s m_s, the identity the online softmax itself rests on (section
// 4.3).
//
// MI355X mapping:
//  * One workgroup per (batch, head, 32-row unit); wave s takes a contiguous
//    run of the unit's 64-key tiles.
//  * Each wave moves its own K/V tiles HBM -> LDS with buffer_load ... lds
//    (LDS-DMA: no staging registers, no address VALU) into its own LDS region
//    (NB = 1 or 2 buffers) of unpadded, XOR-swizzled rows (d = 64, 128) or of
//    the main kernel's padded rows (d = 96). No other wave reads that region,
//    so a wave only waits for its own loads (vmcnt); the workgroup
//    synchronises once, for the merge.
//  * The tile step is the main kernel's (scores, online softmax, PV product).
#pragma once
#include "fa_fwd_kernel.h"

namespace fa {

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left at their maxima (gfx9
// encoding: vmcnt bits 3:0 and 15:14). The compiler does not track LDS-DMA
// writes, so the waits for them are explicit.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at their maxima: every LDS
// read this wave has issued has returned.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// LDS of the key-split kernel. d = 64 and 128: unpadded rows whose 16-byte
// chunks are XOR-swizzled (lds_off<D, 0>). d = 96 and 256, whose rows the
// swizzle does not cover: the main kernel's padded rows (K rows of D+8
// halves, V rows of fwd_vstr<D>; 32-key tiles at d = 256, as in the main
// kernel), which the LDS-DMA writes in 1 KB pieces of the padded tile, each
// padding slot a copy of its row's last chunk. A tile region is rounded up
// to whole pieces; the lanes past the tile's last row load rows outside the
// buffer descriptor, which arrive as zeros.
template <int D, int NS, int NB>
struct SplitSmem {
  static constexpr int BC = D == 256 ? 32 : 64;
  static constexpr bool PADDED = !(D == 64 || D == 128);
  static constexpr int KSTR = PADDED ? FwdSmem<D, BC>::KSTR : 0;  // 0: unpadded, swizzled
  static constexpr int VSTR = PADDED ? FwdSmem<D, BC>::VSTR : 0;
  static constexpr int KTILE = (BC * (PADDED ? KSTR : D) + 511) / 512 * 512;  // halves per K tile region
  static constexpr int VTILE = (BC * (PADDED ? VSTR : D) + 511) / 512 * 512;
  static constexpr int KJ = KTILE / 512, VJ = VTILE / 512;  // 1 KB pieces per tile
  static constexpr int WAVE = NB * (KTILE + VTILE);  // K then V, NB buffers each
  static constexpr int HALVES = NS * WAVE;
  // merge area (floats, reusing the tiles): per wave and lane DB*16
  // accumulators, m and the two sums, stored element-major
  static constexpr int PART = D / 32 * 16 + 3;
  static_assert(NS * PART * 64 * 2 <= HALVES, "partials must fit in the tile area");
};

template <int D, int DT, bool CAUSAL, int NS, int NB, int PF>
__global__ __launch_bounds__(NS * 64) void fa_fwd_split_kernel(const FwdArgs a) {
  using SM = SplitSmem<D, NS, NB>;
  constexpr int BC = SM::BC, KK = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int LOADS = BC * CPR / 64;  // DMA loads per wave per tensor per tile (unpadded rows)
  __shared__ __attribute__((aligned(16))) uint16_t smem[SM::HALVES];

  // ---- workgroup -> (batch, head, unit), XCD-aware as in fa_fwd_kernel ----
  const int per = gridDim.x >> 3;
  const int bid = blockIdx.x;
  const int lid = a.cu_seqlens ? bid : (bid & 7) * per + (bid >> 3);
  if (lid >= a.total) return;
  const int bh = lid / a.units;
  const int ui = lid - bh * a.units;
  const int u = CAUSAL ? a.units - 1 - ui : ui;  // causal: longest first
  const int b = bh / a.H, h = bh - b * a.H;

  int64_t row0 = 0;
  int Nb = a.N;
  if (a.cu_seqlens) {
    row0 = a.cu_seqlens[b];
    Nb = a.cu_seqlens[b + 1] - (int)row0;
  }
  const int qw0 = 32 * u;
  if (qw0 >= Nb) return;  // uniform over the workgroup

  const uint16_t* Qg = a.q + b * a.q_sb + h * a.q_sh + row0 * a.q_sr;
  const uint16_t* Kg = a.k + b * a.k_sb + h * a.k_sh + row0 * a.k_sr;
  const uint16_t* Vg = a.v + b * a.v_sb + h * a.v_sh + row0 * a.v_sr;
  uint16_t* Og = a.o + b * a.o_sb + h * a.o_sh + row0 * a.o_sr;
  float* Lg = a.lse + b * a.lse_sb + h * a.lse_sh + row0;

  const int tid = threadIdx.x;
  // The wave index, visibly uniform: each wave's key range, buffer
  // descriptors and LDS-DMA bases then sit in scalar registers, with no
  // per-lane loop around each DMA (N=400 x4 heads fp16 8.5 -> 7.7 us,
  // N=2048 x4 heads bf16 16.0 -> 14.0 us).
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  // this wave's tiles: a contiguous run of ceil(ntiles / NS)
  const int kv_end = CAUSAL ? min(Nb, qw0 + 32) : Nb;
  const int ntiles = (kv_end + BC - 1) / BC;
  const int tps = (ntiles + NS - 1) / NS;
  const int t_begin = w * tps;
  const int t_end = min(ntiles, t_begin + tps);

  uint16_t* wl = smem + w * SM::WAVE;  // this wave's LDS: K buffers, then V buffers
  auto ktile = [&](int buf) __attribute__((always_inline)) { return wl + buf * SM::KTILE; };
  auto vtile = [&](int buf) __attribute__((always_inline)) { return wl + NB * SM::KTILE + buf * SM::VTILE; };
  // padded rows: lane l of piece i carries the chunk at byte 1024 i + 16 l of
  // the padded tile (row, chunk), a padding slot the row's last chunk; the
  // per-lane byte offsets are the same for every tile
  [[maybe_unused]] uint32_t koff[SM::PADDED ? SM::KJ : 1], voff[SM::PADDED ? SM::VJ : 1];
  if constexpr (SM::PADDED) {
#pragma unroll
    for (int i = 0; i < SM::KJ; ++i) {
      const int o = 1024 * i + 16 * lane, r = o / (2 * SM::KSTR), ch = min(o % (2 * SM::KSTR) / 16, CPR - 1);
      koff[i] = (uint32_t)(r * (a.k_sr * 2) + ch * 16);
    }
#pragma unroll
    for (int i = 0; i < SM::VJ; ++i) {
      const int o = 1024 * i + 16 * lane, r = o / (2 * SM::VSTR), ch = min(o % (2 * SM::VSTR) / 16, CPR - 1);
      voff[i] = (uint32_t)(r * (a.v_sr * 2) + ch * 16);
    }
  }
  // DMA of tile t into buffer `buf`. Unpadded: chunk slot P = 64 i + lane of
  // the tile is row P / CPR, slot P % CPR, and receives that row's chunk
  // (slot ^ swizzle). Rows past kv_end lie outside the descriptor and arrive
  // as zeros.
  auto dma = [&](int t, int buf) __attribute__((always_inline)) {
    const int rows = min(kv_end - t * BC, BC);  // >= 1
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Kg + (int64_t)t * BC * a.k_sr), (short)0, (int)((rows - 1) * (a.k_sr * 2) + D * 2),
        kBufferDword3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Vg + (int64_t)t * BC * a.v_sr), (short)0, (int)((rows - 1) * (a.v_sr * 2) + D * 2),
        kBufferDword3);
    uint16_t* kd = ktile(buf);
    uint16_t* vd = vtile(buf);
    if constexpr (SM::PADDED) {
#pragma unroll
      for (int i = 0; i < SM::KJ; ++i) {
        const uint32_t o = koff[i];  // the builtin given koff[i] itself loses the host-side kernel stub
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(kd + 512 * i), 16,
                                                 o, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < SM::VJ; ++i) {
        const uint32_t o = voff[i];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(vd + 512 * i), 16,
                                                 o, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int P = 64 * i + lane;
        const int r = P / CPR, ch = (P % CPR) ^ lds_swz<D>(r);
        const uint32_t ko = (uint32_t)(r * (a.k_sr * 2) + ch * 16);
        const uint32_t vo = (uint32_t)(r * (a.v_sr * 2) + ch * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(kd + 64 * i * 8),
                                                 16, ko, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(vd + 64 * i * 8),
                                                 16, vo, 0, 0, 0);
      }
    }
  };

  // Q fragments (rows past the end are zero; a negative scale flips signs).
  // They are loaded raw and converted once the first tile's DMA has been
  // issued, so that the wait for Q does not hold back that DMA.
  u32x4 qf[1][KK];
  const int qr = qw0 + l32;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[0][kk] = *(const u32x4*)(Qg + min(qr, Nb - 1) * a.q_sr + 16 * kk + 8 * hh);

  f32x16 oacc[1][DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[0][db][r] = 0.f;
  float m_run[1] = {-INFINITY}, l_run[2][1] = {{0.f}, {0.f}};

  if (t_begin < t_end) {
    __builtin_amdgcn_sched_barrier(0);  // the Q loads stay ahead of the DMA
    dma(t_begin, 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[0][kk] = (qr < Nb ? qf[0][kk] : u32x4{0u, 0u, 0u, 0u}) ^ a.qsign;
    for (int t = t_begin; t < t_end; ++t) {
      const int buf = NB == 2 ? (t - t_begin) & 1 : 0;
      if (NB == 2 && t + 1 < t_end) {
        dma(t + 1, buf ^ 1);
        wait_vmcnt<SM::PADDED ? SM::KJ + SM::VJ : 2 * LOADS>();  // tile t has landed; tile t+1 may be in flight
      } else {
        wait_vmcnt<0>();
      }
      const int key0 = t * BC;
      const bool need_mask = (key0 + BC > Nb) || (CAUSAL && key0 + BC - 1 > qw0);
      tile_step_fwd<D, DT, CAUSAL, 1, BC, SM::KSTR, SM::VSTR, PF>(t == t_begin, need_mask, ktile(buf), vtile(buf),
                                                                  key0, Nb, qw0, lane, a.c, qf, oacc, m_run,
                                                                  l_run);
      // one buffer: the next tile's DMA writes the buffer this tile has just
      // read, so it waits until those LDS reads have returned (lgkmcnt 0),
      // and the fences keep the compiler from moving the reads below the wait or
      // the DMA above it
      if (NB == 1 && t + 1 < t_end) {
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkmcnt0();
        __builtin_amdgcn_sched_barrier(0);
        dma(t + 1, 0);
      }
    }
  }

  // ---- merge the NS partials, then O = acc / l and LSE = (m + log2 l) ln 2 ----
  __syncthreads();  // every wave is done with its tiles
  float* part = (float*)smem;
  auto pidx = [&](int s, int k) __attribute__((always_inline)) { return (s * SM::PART + k) * 64 + lane; };
  if (w != 0) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[pidx(w, 16 * db + r)] = oacc[0][db][r];
    part[pidx(w, DB * 16)] = m_run[0];
    part[pidx(w, DB * 16 + 1)] = l_run[0][0];
    part[pidx(w, DB * 16 + 2)] = l_run[1][0];
  }
  __syncthreads();
  if (w != 0) return;
  float m = m_run[0];
#pragma unroll
  for (int s = 1; s < NS; ++s) m = fmaxf(m, part[pidx(s, DB * 16)]);
  {
    // m is finite: wave 0's first tile holds key 0, which every row sees
    const float a0 = fast_exp2(m_run[0] - m);
    l_run[0][0] *= a0;
    l_run[1][0] *= a0;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[0][db][r] *= a0;
  }
#pragma unroll
  for (int s = 1; s < NS; ++s) {
    const float ms = part[pidx(s, DB * 16)];
    const float as = ms == -INFINITY ? 0.f : fast_exp2(ms - m);  // a wave without tiles adds nothing
    l_run[0][0] += as * part[pidx(s, DB * 16 + 1)];
    l_run[1][0] += as * part[pidx(s, DB * 16 + 2)];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[0][db][r] += as * part[pidx(s, 16 * db + r)];
  }

  // wave 0 turns its Oᵀ tile into row-major rows in LDS (after its own reads
  // of the partials, which the same wave's LDS ops complete in order) and
  // writes whole 16-byte row chunks
  constexpr int OSTR = D + 8;
  // past the partials where they leave room; else (d = 256) over the slots of
  // waves 1.. (slot 0 is unused), whose partials wave 0 has consumed: every
  // store below depends on the merged values
  constexpr bool OB_PAST = NS * SM::PART * 64 * 2 + 32 * OSTR <= SM::HALVES;
  uint16_t* ob = smem + (OB_PAST ? NS : 1) * SM::PART * 64 * 2;
  static_assert(SM::PART * 64 * 2 + 32 * OSTR <= SM::HALVES, "output staging must fit");
  if constexpr (!OB_PAST) wave_lds_sync();
  const float l_tot = l_run[0][0] + xor_lane32(l_run[0][0]);
  const float l_lse = DT == DT_F16 ? l_tot : l_run[1][0] + xor_lane32(l_run[1][0]);
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2 x;
      x[0] = pack2<DT>(oacc[0][db][4 * g4 + 0] * inv, oacc[0][db][4 * g4 + 1] * inv);
      x[1] = pack2<DT>(oacc[0][db][4 * g4 + 2] * inv, oacc[0][db][4 * g4 + 3] * inv);
      *(u32x2*)(ob + l32 * OSTR + db * 32 + 8 * g4 + 4 * hh) = x;
    }
  wave_lds_sync();  // the rows below were written by other lanes of this wave
  const int qrow = qw0 + l32;
  if (hh == 0 && qrow < Nb) Lg[qrow] = (m + fast_log2(l_lse)) * kLn2;
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int p = lane + 64 * i, r = p / CPR, ch = p % CPR;
    const u32x4 x = *(const u32x4*)(ob + r * OSTR + ch * 8);
    if (qw0 + r < Nb) *(u32x4*)(Og + (qw0 + r) * a.o_sr + ch * 8) = x;
  }
}

}  // namespace fa
