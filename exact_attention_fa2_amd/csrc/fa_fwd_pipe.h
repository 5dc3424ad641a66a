// Software-pipelined FlashAttention-2-style forward for gfx950 (d = 64, 128).
//
// Same mathematics as fa_fwd_kernel.h -- one workgroup per block of query
// rows, K/V tiles streamed through LDS, online softmax with running max and
// sum ("FlashAttention explainer" (aitangshan.cn) sections 4.1-4.3, 5.2) --
// with an MI355X-specific schedule:
//  * K/V tiles travel HBM -> LDS with buffer_load_dwordx4 ... lds (no
//    registers, no VALU address work); rows past the end of the sequence are
//    outside the buffer's range and arrive as zeros.
//  * LDS rows are unpadded; 16-byte chunk c of row r sits at chunk slot
//    c ^ f(r) (see swz), which keeps both the 16-byte K reads and the
//    transposing V reads free of bank conflicts.
//  * Iteration t computes the scores of tile t+1 (Sᵀ = K Qᵀ, MFMA) while the
//    softmax of tile t runs on the VALU and its P·V MFMAs follow, all in one
//    basic block the compiler may interleave; K runs one tile ahead of V,
//    each double-buffered, one barrier per tile.
//  * Tiles that need the ragged-tail or causal mask run a separate copy of
//    the loop body, so the common tiles carry no mask code.
#pragma once
#include <type_traits>

#include "fa_fwd_kernel.h"

namespace fa {

constexpr float kRescaleGap = 8.0f;  // raise the running max only when it grows by more than this (log2)

template <int D, int BC>
struct PipeSmem {
  static constexpr int TILE = BC * D;  // halves per K or V tile (unpadded)
  static constexpr int KOFF = 0;       // K stages 0, 1
  static constexpr int VOFF = 2 * TILE;  // V stages 0, 1
  static constexpr int HALVES = 4 * TILE;
};

// Issue the LDS-DMA loads of one BC x D tile starting at row `row0` into the
// LDS tile at `lds` (halves). Every wave covers NT/64 * 64-chunk slices.
template <int D, int BC, int NW>
__device__ __forceinline__ void tile_dma(__amdgpu_buffer_rsrc_t rs, int64_t row_bytes, int row0,
                                         uint16_t* lds, int w, int lane) {
  constexpr int CPR = D / 8;               // 16-byte chunks per row
  constexpr int ROUNDS = BC * CPR / (NW * 64);
  static_assert(BC * CPR % (NW * 64) == 0, "tile must split into whole wave loads");
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    const int slot0 = (i * NW + w) * 64;   // first chunk slot written by this wave
    const int P = slot0 + lane;
    const int r = P / CPR, p = P % CPR;
    const int c = p ^ swz<D>(r);
    const uint32_t voff = (uint32_t)((int64_t)(row0 + r) * row_bytes + c * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(lds + slot0 * 8), 16, voff, 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_dma_and_sync() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA loads have landed
  __syncthreads();
}

template <int D, int DT, int QB, int BC>
struct PipeWave {
  static constexpr int KK = D / 16, DB = D / 32, KB = BC / 32, CPR = D / 8;
  int lane, l32, hh;
  float c;

  // Sᵀ of one tile from the swizzled K tile in LDS
  __device__ __forceinline__ void scores(const uint16_t* sk, const u32x4 (&qf)[QB][KK],
                                         f32x16 (&s)[KB][QB]) const {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < QB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][j][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int r = kb * 32 + l32;
        const int ch = (2 * kk + hh) ^ swz<D>(r);
        const u32x4 ka = *(const u32x4*)(sk + r * D + ch * 8);
#pragma unroll
        for (int j = 0; j < QB; ++j) s[kb][j] = mfma32x32x16<DT>(ka, qf[j][kk], s[kb][j]);
      }
    }
  }

  template <bool CAUSAL>
  __device__ __forceinline__ void mask(f32x16 (&s)[KB][QB], int key0, int Nb, int qw0) const {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const int qrow = qw0 + 32 * j + l32;
        const int lim = CAUSAL ? min(Nb - 1, qrow) : Nb - 1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > lim) s[kb][j][r] = -INFINITY;
        }
      }
  }

  // row max of a score tile (log2 units), combined across the two lane halves
  __device__ __forceinline__ void rowmax(const f32x16 (&s)[KB][QB], float (&mx)[QB]) const {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      // four independent partial maxima keep the dependency chains short
      float mm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mm[r & 3] = fmaxf(mm[r & 3], s[kb][j][r]);
      float m = fmaxf(fmaxf(mm[0], mm[1]), fmaxf(mm[2], mm[3]));
      m = fmaxf(m, xor_lane32(m));
      mx[j] = m * c;
    }
  }

  // P = exp2(S c - m) packed to 16 bits. l[0] sums the packed weights (the
  // exact normaliser of the product they enter); l[1] is the fp32 sum the
  // bf16 LSE needs (fp16 weights are accurate enough for both).
  __device__ __forceinline__ void probs(const f32x16 (&s)[KB][QB], const float (&m_run)[QB],
                                        u32x4 (&pf)[QB][BC / 16], float (&l_run)[2][QB]) const {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const float mref = (m_run[j] == -INFINITY) ? 0.f : m_run[j];
      float lp[4] = {0.f, 0.f, 0.f, 0.f}, lf[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(__builtin_fmaf(s[kb][j][r], c, -mref));
          if constexpr (DT == DT_BF16) lf[r & 3] += p[r];
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          u32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = pack2<DT>(p[8 * c2 + 2 * e], p[8 * c2 + 2 * e + 1]);
            lp[e] = dot2_sum<DT>(x[e], lp[e]);
          }
          pf[j][2 * kb + c2] = x;
        }
      }
      l_run[0][j] += (lp[0] + lp[1]) + (lp[2] + lp[3]);
      if constexpr (DT == DT_BF16) l_run[1][j] += (lf[0] + lf[1]) + (lf[2] + lf[3]);
    }
  }

  // Oᵀ += Vᵀ Pᵀ from the swizzled V tile in LDS
  __device__ __forceinline__ void pv(const uint16_t* sv, const u32x4 (&pf)[QB][BC / 16],
                                     f32x16 (&oacc)[QB][DB]) const {
    const int g = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int ci = 0; ci < BC / 16; ++ci) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int colh = db * 32 + (g & 1) * 16 + 4 * (s16 & 3);  // column in halves
        const int cch = colh >> 3, cin = colh & 7;
        const int ra = 16 * ci + 4 * hh + (s16 >> 2), rb = ra + 8;
        const u32x2 lo = lds_read_tr4(sv + ra * D + ((cch ^ swz<D>(ra)) << 3) + cin);
        const u32x2 hi = lds_read_tr4(sv + rb * D + ((cch ^ swz<D>(rb)) << 3) + cin);
        const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int j = 0; j < QB; ++j) oacc[j][db] = mfma32x32x16<DT>(va, pf[j][ci], oacc[j][db]);
      }
    }
  }

  // raise the running max when it grew by more than kRescaleGap, rescaling
  // the accumulator and the running sum by exp2(m_old - m_new)
  __device__ __forceinline__ void update_max(const float (&mx)[QB], float (&m_run)[QB],
                                             float (&l_run)[2][QB], f32x16 (&oacc)[QB][DB]) const {
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const float m_new = fmaxf(m_run[j], mx[j]);
      if (wave_any(m_new > m_run[j] + kRescaleGap)) {
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[j] - m_new);
        l_run[0][j] *= alpha;
        l_run[1][j] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[j][db][r] *= alpha;
        m_run[j] = m_new;
      }
    }
  }
};


template <int D, int DT, bool CAUSAL, int NW, int QB, int BC, int MINW = 2>
__global__ __launch_bounds__(NW * 64, MINW) void fa_fwd_pipe_kernel(const FwdArgs a) {
  constexpr int QW = 32 * QB, BR = NW * QW;
  constexpr int KK = D / 16, DB = D / 32, KB = BC / 32;
  using SM = PipeSmem<D, BC>;
  using WV = PipeWave<D, DT, QB, BC>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SM::HALVES];

  // ---- workgroup -> (batch, head, query block), XCD-aware ----
  const int per = gridDim.x >> 3;
  const int bid = blockIdx.x;
  const int lid = (bid & 7) * per + (bid >> 3);
  if (lid >= a.total) return;
  const int bh = lid / a.nqb;
  const int qi = lid - bh * a.nqb;
  const int qblk = CAUSAL ? (a.nqb - 1 - qi) : qi;
  const int b = bh / a.H, h = bh - b * a.H;
  int64_t row0 = 0;
  int Nb = a.N;
  if (a.cu_seqlens) {
    row0 = a.cu_seqlens[b];
    Nb = a.cu_seqlens[b + 1] - (int)row0;
  }
  if (qblk * BR >= Nb) return;

  const uint16_t* Qg = a.q + b * a.q_sb + h * a.q_sh + row0 * a.q_sr;
  const uint16_t* Kg = a.k + b * a.k_sb + h * a.k_sh + row0 * a.k_sr;
  const uint16_t* Vg = a.v + b * a.v_sb + h * a.v_sh + row0 * a.v_sr;
  uint16_t* Og = a.o + b * a.o_sb + h * a.o_sh + row0 * a.o_sr;
  float* Lg = a.lse + b * a.lse_sb + h * a.lse_sh + row0;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  WV wv{lane, lane & 31, lane >> 5, a.c};
  const int qw0 = qblk * BR + w * QW;

  // buffer descriptors covering exactly the valid rows of K and V
  const int64_t kbytes = a.k_sr * 2, vbytes = a.v_sr * 2;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Kg, (short)0, (int)((Nb - 1) * kbytes + D * 2), kBufferDword3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Vg, (short)0, (int)((Nb - 1) * vbytes + D * 2), kBufferDword3);

  const int kv_end = CAUSAL ? min(Nb, (qblk + 1) * BR) : Nb;
  const int nt = (kv_end + BC - 1) / BC;

  // K and V stage i live at smem + KOFF/VOFF + i * TILE
  auto kst = [&](int i) __attribute__((always_inline)) { return smem + SM::KOFF + (i & 1) * SM::TILE; };
  auto vst = [&](int i) __attribute__((always_inline)) { return smem + SM::VOFF + (i & 1) * SM::TILE; };

  // prologue loads: K_0, V_0, K_1
  tile_dma<D, BC, NW>(rk, kbytes, 0, kst(0), w, lane);
  tile_dma<D, BC, NW>(rv, vbytes, 0, vst(0), w, lane);
  if (nt > 1) tile_dma<D, BC, NW>(rk, kbytes, BC, kst(1), w, lane);

  // Q fragments (B operand of Sᵀ = K Qᵀ) in registers
  u32x4 qf[QB][KK];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int r = qw0 + 32 * j + wv.l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      // rows past the end load row Nb-1 (in bounds) and are zeroed
      const u32x4 x = *(const u32x4*)(Qg + min(r, Nb - 1) * a.q_sr + 16 * kk + 8 * wv.hh);
      qf[j][kk] = (r < Nb ? x : u32x4{0u, 0u, 0u, 0u}) ^ a.qsign;
    }
  }

  f32x16 oacc[QB][DB];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[j][db][r] = 0.f;
  float m_run[QB], l_run[2][QB], mx[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) { m_run[j] = -INFINITY; l_run[0][j] = 0.f; l_run[1][j] = 0.f; }

  auto needs_mask = [&](int t) __attribute__((always_inline)) { return (t + 1) * BC > Nb || (CAUSAL && t * BC + BC - 1 > qw0); };

  // scores of tile 0
  f32x16 s0[KB][QB], s1[KB][QB];
  wait_dma_and_sync();
  wv.scores(kst(0), qf, s0);
  if (needs_mask(0)) wv.template mask<CAUSAL>(s0, 0, Nb, qw0);
  wv.rowmax(s0, mx);
  wv.update_max(mx, m_run, l_run, oacc);

  // one pipelined step: softmax + P·V of tile t from s_cur, scores of tile
  // t+1 into s_nxt
  auto step = [&](int t, f32x16(&s_cur)[KB][QB], f32x16(&s_nxt)[KB][QB], auto has_next,
                  auto mask_next) __attribute__((always_inline)) {
    constexpr bool HAS_NEXT = decltype(has_next)::value;
    constexpr bool MASK_NEXT = decltype(mask_next)::value;
    wait_dma_and_sync();
    if (t + 2 < nt) tile_dma<D, BC, NW>(rk, kbytes, (t + 2) * BC, kst(t), w, lane);
    if (t + 1 < nt) tile_dma<D, BC, NW>(rv, vbytes, (t + 1) * BC, vst(t + 1), w, lane);
    u32x4 pf[QB][BC / 16];
    wv.probs(s_cur, m_run, pf, l_run);
    if constexpr (HAS_NEXT) wv.scores(kst(t + 1), qf, s_nxt);
    wv.pv(vst(t), pf, oacc);
    if constexpr (HAS_NEXT) {
      if constexpr (MASK_NEXT) wv.template mask<CAUSAL>(s_nxt, (t + 1) * BC, Nb, qw0);
      wv.rowmax(s_nxt, mx);
      wv.update_max(mx, m_run, l_run, oacc);
    }
  };
  // run steps while cond(t) holds, alternating the two score arrays; the
  // current scores are left in s0
  int t = 0;
  auto phase = [&](auto mask_next, auto cond) __attribute__((always_inline)) {
    while (cond(t)) {
      step(t, s0, s1, std::true_type{}, mask_next);
      ++t;
      if (!cond(t)) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int j = 0; j < QB; ++j) s0[kb][j] = s1[kb][j];
        return;
      }
      step(t, s1, s0, std::true_type{}, mask_next);
      ++t;
    }
  };
  phase(std::false_type{}, [&](int u) { return u + 1 < nt && !needs_mask(u + 1); });
  phase(std::true_type{}, [&](int u) { return u + 1 < nt; });
  step(t, s0, s1, std::false_type{}, std::false_type{});

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float l_tot = l_run[0][j] + xor_lane32(l_run[0][j]);
    const float l_lse = DT == DT_F16 ? l_tot : l_run[1][j] + xor_lane32(l_run[1][j]);
    const float inv = 1.f / l_tot;
    const int qrow = qw0 + 32 * j + wv.l32;
    if (qrow < Nb) {
      uint16_t* orow = Og + qrow * a.o_sr;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 x;
          x[0] = pack2<DT>(oacc[j][db][4 * g4 + 0] * inv, oacc[j][db][4 * g4 + 1] * inv);
          x[1] = pack2<DT>(oacc[j][db][4 * g4 + 2] * inv, oacc[j][db][4 * g4 + 3] * inv);
          *(u32x2*)(orow + db * 32 + 8 * g4 + 4 * wv.hh) = x;
        }
      if (wv.hh == 0) Lg[qrow] = (m_run[j] + fast_log2(l_lse)) * kLn2;
    }
  }
}

}  // namespace fa
