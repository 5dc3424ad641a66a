// Attention forward with the FlashAttention-1 loop order, kept as an ablation
// of the FlashAttention-2 kernels ("FlashAttention explainer" (aitangshan.cn)
// sections 5.1 and 5.2; "YOLO11 attention swapped for a FlashAttention-2-style
// implementation" (discosf.com) section 2.4).
//
// One workgroup per (batch, head) -- the first version's parallelisation over
// batch and heads only. Its outer loop walks the K/V blocks; for each one the
// inner loop walks every query block, reads that block's running output
// accumulator, max and sum back from HBM (fp32 workspace), applies the same
// online-softmax update as the FA2 kernels (the per-wave tile step is shared),
// and writes them back. A query block's last visit writes O and LSE instead.
#pragma once
#include "fa_fwd_kernel.h"

namespace fa {

template <int D>
struct Fa1Layout {
  static constexpr int NW = 4, BC = 64, BR = NW * 32, DB = D / 32;
  // per wave: the Oᵀ accumulator registers plus m and the two sums, lane-major
  static constexpr int WAVE_FLOATS = (16 * DB + 3) * 64;
  static int64_t bytes(int B, int H, int N) {
    const int64_t nqb = (N + BR - 1) / BR;
    return (int64_t)B * H * nqb * NW * WAVE_FLOATS * 4;
  }
};

template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(256) void fa_fwd_fa1_kernel(const FwdArgs a, float* __restrict__ ws) {
  using L = Fa1Layout<D>;
  constexpr int NW = L::NW, BC = L::BC, BR = L::BR, QB = 1, NT = NW * 64;
  constexpr int KK = D / 16, DB = D / 32, CH = BC * D / 8 / NT;
  using SM = FwdSmem<D, BC>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SM::STAGE];

  const int bh = blockIdx.x;
  if (bh >= a.B * a.H) return;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Nb = a.N;
  const uint16_t* Qg = a.q + b * a.q_sb + h * a.q_sh;
  const uint16_t* Kg = a.k + b * a.k_sb + h * a.k_sh;
  const uint16_t* Vg = a.v + b * a.v_sb + h * a.v_sh;
  uint16_t* Og = a.o + b * a.o_sb + h * a.o_sh;
  float* Lg = a.lse + b * a.lse_sb + h * a.lse_sh;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int nqb = (Nb + BR - 1) / BR, ntk = (Nb + BC - 1) / BC;
  float* wsbh = ws + (int64_t)bh * nqb * NW * L::WAVE_FLOATS;
  uint16_t* sk = smem;
  uint16_t* sv = smem + SM::KTILE;

  for (int j = 0; j < ntk; ++j) {
    const int key0 = j * BC;
    // ---- outer step: K_j, V_j into LDS ----
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = tid + NT * c;
      const int r = ci / (D / 8), col = (ci % (D / 8)) * 8;
      const int gr = key0 + r;
      u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (gr < Nb) {
        xk = *(const u32x4*)(Kg + gr * a.k_sr + col);
        xv = *(const u32x4*)(Vg + gr * a.v_sr + col);
      }
      *(u32x4*)(sk + r * SM::KSTR + col) = xk;
      *(u32x4*)(sv + r * SM::VSTR + col) = xv;
    }
    __syncthreads();

    // ---- inner loop over every query block that sees this K/V block ----
    const int qb0 = CAUSAL ? max(0, (key0 - (BR - 1) + BR - 1) / BR) : 0;
    for (int qb = qb0; qb < nqb; ++qb) {
      const int qw0 = qb * BR + w * 32;
      u32x4 qf[QB][KK];
      {
        const int r = qw0 + l32;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 x = *(const u32x4*)(Qg + min(r, Nb - 1) * a.q_sr + 16 * kk + 8 * hh);
          qf[0][kk] = (r < Nb ? x : u32x4{0u, 0u, 0u, 0u}) ^ a.qsign;
        }
      }
      float* wsw = wsbh + ((int64_t)qb * NW + w) * L::WAVE_FLOATS;
      f32x16 oacc[QB][DB];
      float m_run[QB], l_run[2][QB];
      if (j == 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[0][db][r] = 0.f;
        m_run[0] = -INFINITY;
        l_run[0][0] = 0.f;
        l_run[1][0] = 0.f;
      } else {
        // read the running state back from HBM
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[0][db][r] = wsw[(db * 16 + r) * 64 + lane];
        m_run[0] = wsw[(DB * 16) * 64 + lane];
        l_run[0][0] = wsw[(DB * 16 + 1) * 64 + lane];
        l_run[1][0] = wsw[(DB * 16 + 2) * 64 + lane];
      }
      const bool need_mask = (key0 + BC > Nb) || (CAUSAL && key0 + BC - 1 > qw0);
      tile_step_fwd<D, DT, CAUSAL, QB, BC, SM::KSTR, SM::VSTR, 0>(j == 0, need_mask, sk, sv, key0, Nb, qw0,
                                                               lane, a.c, qf, oacc, m_run, l_run);
      const int last_j = CAUSAL ? min(ntk - 1, (qb * BR + BR - 1) / BC) : ntk - 1;
      if (j < last_j) {
        // write the running state back to HBM
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) wsw[(db * 16 + r) * 64 + lane] = oacc[0][db][r];
        wsw[(DB * 16) * 64 + lane] = m_run[0];
        wsw[(DB * 16 + 1) * 64 + lane] = l_run[0][0];
        wsw[(DB * 16 + 2) * 64 + lane] = l_run[1][0];
      } else if (j == last_j) {
        const float l_tot = l_run[0][0] + xor_lane32(l_run[0][0]);
        const float l_lse = DT == DT_F16 ? l_tot : l_run[1][0] + xor_lane32(l_run[1][0]);
        const float inv = 1.f / l_tot;
        const int qrow = qw0 + l32;
        if (qrow < Nb) {
          uint16_t* orow = Og + qrow * a.o_sr;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              u32x2 x;
              x[0] = pack2<DT>(oacc[0][db][4 * g4 + 0] * inv, oacc[0][db][4 * g4 + 1] * inv);
              x[1] = pack2<DT>(oacc[0][db][4 * g4 + 2] * inv, oacc[0][db][4 * g4 + 3] * inv);
              *(u32x2*)(orow + db * 32 + 8 * g4 + 4 * hh) = x;
            }
          if (hh == 0) Lg[qrow] = (m_run[0] + fast_log2(l_lse)) * kLn2;
        }
      }
    }
  }
}

}  // namespace fa
