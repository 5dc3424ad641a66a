// Forward kernel for maps of at most 128 rows that packs several heads into
// one workgroup and holds their whole K and V in LDS.
//
// The mathematics is that of fa_fwd_kernel: K/V tiles through LDS and the
// online softmax ("FlashAttention explainer" (aitangshan.cn) sections 4.2,
// 4.3 and 5.2). The shapes are the smallest feature maps of "YOLO11 attention
// swapped for a FlashAttention-2-style implementation" (discosf.com),
// section 2.1 (deep detector layers: 8x8 to 11x11 maps), where a head holds
// at most two 64-key tiles.
//
// A head of at most 128 rows has at most four 32-row units, so an 8-wave
// workgroup of the main kernel (one unit per wave) leaves half of its waves
// or more without rows, and each head's K/V arrives one tile ahead of its
// use. Here an 8-wave workgroup takes HP heads (HP = 2 up to 128 rows, 4 up
// to 64): the 8 / HP waves of slot s own the units of head s. Every thread
// first issues the LDS-DMA loads of its wave's Q rows and of its share of the
// slot's K and V tiles (unpadded XOR-swizzled rows, no staging registers);
// then the waves take the tiles in order, each as soon as it has landed (a
// wait on this thread's outstanding loads plus one barrier). Q goes through
// LDS too: the compiler counts no LDS-DMA in its own waits for loaded
// registers, so a register load of Q issued before the DMAs would be waited
// for with every DMA behind it.
#pragma once
#include "fa_fwd_kernel.h"
#include "fa_fwd_split.h"

namespace fa {

// s_waitcnt vmcnt(n) for a wave-uniform n; a count above the largest case
// waits for that case, which is stronger and therefore also correct.
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break;
    case 19: wait_vmcnt<19>(); break;
    default: wait_vmcnt<20>(); break;
  }
}

// Workgroup barrier for LDS written by LDS-DMA whose completion each thread
// has already waited for (vmcnt). __syncthreads() would also make every wave
// wait for all of its LDS-DMA still in flight (its release fence covers LDS);
// wavefront-scope fences keep the compiler from moving LDS accesses across the
// barrier and add no waits.
__device__ __forceinline__ void barrier_after_dma() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS of the kernel, in halves: first the Q rows of the 8 waves (32 x D
// each), later the output staging of the epilogue (32 x (D + 8) each); then
// HP slots of 2 * ceil(n / 64) unpadded K and V tiles for maps of n rows
// (d=64: 100 KB with HP = 2 at n <= 128 or HP = 4 at n <= 64, one workgroup
// per CU).
template <int D>
constexpr int resident_q_halves() {
  return 8 * 32 * (D + 8);
}
template <int D, int HP>
constexpr int64_t resident_lds_bytes(int64_t n) {
  return 2 * (resident_q_halves<D>() + (int64_t)HP * 2 * ((n + 63) / 64) * 64 * D);
}

template <int D, int DT, bool CAUSAL, int HP>
__global__ __launch_bounds__(512) void fa_fwd_resident_kernel(const FwdArgs a) {
  constexpr int NW = 8, BC = 64, WPH = NW / HP;  // waves per head slot
  static_assert(HP == 2 || HP == 4, "two or four heads per workgroup");
  constexpr int TS = WPH * 64;  // threads per head slot
  constexpr int KK = D / 16, DB = D / 32;
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int LOADS = BC * CPR / TS;  // LDS-DMA loads per thread per tensor per tile
  static_assert(BC * CPR % TS == 0, "a tile must split evenly over a slot's threads");
  constexpr int TILE = BC * D;  // halves of an unpadded K or V tile
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_res[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int slot = w / WPH, ws = w - slot * WPH;  // head slot, wave inside the slot
  const int stid = tid - slot * TS;               // thread index inside the slot
  const int64_t bhs = (int64_t)blockIdx.x * HP + slot;
  const bool head_ok = bhs < (int64_t)a.B * a.H;
  const int b = head_ok ? (int)(bhs / a.H) : 0, h = head_ok ? (int)(bhs - (int64_t)b * a.H) : 0;
  const int Nb = a.N;  // equal lengths, at most 32 * WPH rows (host check)
  const int qw0 = 32 * ws;
  const bool wave_rows = head_ok && qw0 < Nb;
  const int ntl = (Nb + BC - 1) / BC;  // 1 or 2, the same for every slot

  const uint16_t* Qg = a.q + b * a.q_sb + h * a.q_sh;
  const uint16_t* Kg = a.k + b * a.k_sb + h * a.k_sh;
  const uint16_t* Vg = a.v + b * a.v_sb + h * a.v_sh;
  uint16_t* Og = a.o + b * a.o_sb + h * a.o_sh;
  float* Lg = a.lse + b * a.lse_sb + h * a.lse_sh;
  uint16_t* sq = smem_res + w * 32 * D;  // this wave's Q rows
  uint16_t* sl = smem_res + resident_q_halves<D>() + slot * 2 * ntl * TILE;  // K tiles, then V tiles

  // Q rows qw0.. of this wave: chunk slot P = 64*i + lane is row P / CPR,
  // position P % CPR, as for the K/V tiles; rows past the end arrive as zeros
  if (wave_rows) {
    const int rows = min(Nb - qw0, 32);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Qg + (int64_t)qw0 * a.q_sr), (short)0, (int)((rows - 1) * (a.q_sr * 2) + D * 2), kBufferDword3);
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int P = 64 * i + lane;
      const int r = P / CPR, ch = (P % CPR) ^ lds_swz<D>(r);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)(sq + 64 * i * 8), 16,
                                               (uint32_t)(r * (a.q_sr * 2) + ch * 16), 0, 0, 0);
    }
  }

  // Tile t of K into sl + t*TILE, of V into sl + (ntl + t)*TILE. Chunk slot
  // P = TS*i + stid of a tile is row P / CPR, position P % CPR, and receives
  // that row's chunk (position ^ swizzle); rows past the end arrive as zeros.
  // Each DMA writes 16 bytes per lane from the wave's base (lane 0's slot).
  auto dma = [&](int t) __attribute__((always_inline)) {
    const int rows = min(Nb - t * BC, BC);  // >= 1
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Kg + (int64_t)t * BC * a.k_sr), (short)0, (int)((rows - 1) * (a.k_sr * 2) + D * 2),
        kBufferDword3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Vg + (int64_t)t * BC * a.v_sr), (short)0, (int)((rows - 1) * (a.v_sr * 2) + D * 2),
        kBufferDword3);
    uint16_t* kd = sl + t * TILE;
    uint16_t* vd = sl + (ntl + t) * TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int P = TS * i + stid;
      const int r = P / CPR, ch = (P % CPR) ^ lds_swz<D>(r);
      const uint32_t ko = (uint32_t)(r * (a.k_sr * 2) + ch * 16);
      const uint32_t vo = (uint32_t)(r * (a.v_sr * 2) + ch * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(kd + (TS * i + 64 * ws) * 8), 16, ko, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)(vd + (TS * i + 64 * ws) * 8), 16, vo, 0, 0, 0);
    }
  };
  if (head_ok)
    for (int t = 0; t < ntl; ++t) dma(t);

  f32x16 oacc[1][DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[0][db][r] = 0.f;
  float m_run[1] = {-INFINITY}, l_run[2][1] = {{0.f}, {0.f}};

  // The tiles a wave's rows see (causal: up to its diagonal). A last tile of
  // at most 32 keys (the ragged end, or a causal diagonal at a 64-key
  // boundary) is a half step. Every wave takes all ntl barriers.
  const int wave_end = CAUSAL ? min(Nb, qw0 + 32) : Nb;
  const int wnt = wave_rows ? (wave_end + BC - 1) / BC : 0;
  const bool tail32 = wave_end - (wnt - 1) * BC <= 32;
  // Q and tile 0 have landed (this thread's loads, then every thread's)
  if (head_ok) wait_vmcnt_dyn((ntl - 1) * 2 * LOADS);
  barrier_after_dma();
  u32x4 qf[1][KK];  // a negative scale flips the signs
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[0][kk] = *(const u32x4*)(sq + lds_off<D, 0>(l32, 16 * kk + 8 * hh)) ^ a.qsign;
  for (int t = 0; t < ntl; ++t) {
    if (t > 0) {
      if (head_ok) wait_vmcnt_dyn((ntl - 1 - t) * 2 * LOADS);  // this thread's part of tile t has landed
      barrier_after_dma();                                      // and every thread's
    }
    if (t < wnt) {
      const uint16_t* sk = sl + t * TILE;
      const uint16_t* sv = sl + (ntl + t) * TILE;
      const int key0 = t * BC;
      const bool need_mask = (key0 + BC > Nb) || (CAUSAL && key0 + BC - 1 > qw0);
      if (t == wnt - 1 && tail32)
        tile_step_fwd<D, DT, CAUSAL, 1, 32, 0, 0, 2>(t == 0, true, sk, sv, key0, Nb, qw0, lane, a.c, qf, oacc,
                                                         m_run, l_run);
      else
        tile_step_fwd<D, DT, CAUSAL, 1, BC, 0, 0, 2>(t == 0, need_mask, sk, sv, key0, Nb, qw0, lane, a.c, qf,
                                                         oacc, m_run, l_run);
    }
  }

  // ---- epilogue (as in fa_fwd_kernel): each wave stages its rows in LDS ----
  constexpr int OSTR = D + 8;
  static_assert(8 * 32 * OSTR <= resident_q_halves<D>(), "output staging must fit in the Q area");
  __syncthreads();  // every wave is done with its Q rows and the K/V tiles
  if (!wave_rows) return;
  uint16_t* ob = smem_res + w * 32 * OSTR;
  {
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
    const int qrow = qw0 + l32;
    if (hh == 0 && qrow < Nb) Lg[qrow] = (m_run[0] + fast_log2(l_lse)) * kLn2;
  }
  wave_lds_sync();
#pragma unroll
  for (int k = 0; k < 32 * CPR / 64; ++k) {
    const int p = lane + 64 * k, r = p / CPR, ch = p % CPR;
    const u32x4 x = *(const u32x4*)(ob + r * OSTR + ch * 8);
    if (qw0 + r < Nb) *(u32x4*)(Og + (qw0 + r) * a.o_sr + ch * 8) = x;
  }
}

}  // namespace fa
