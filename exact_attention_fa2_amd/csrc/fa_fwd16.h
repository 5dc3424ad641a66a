// Forward kernel with 16-row query units (16x16x32 MFMAs), for causal grids
// that give each SIMD only one or two 32-row units.
//
// The mathematics is that of fa_fwd_kernel: Q blocks per workgroup, K/V tiles
// through LDS, the online softmax with a reference max and a range check
// ("FlashAttention explainer" (aitangshan.cn) sections 4.2, 4.3 and 5.2).
// With 32-row units a grid such as N=400 x128 heads has 1664 units for 1024
// SIMDs: one or two waves per SIMD. Under the causal mask the units differ in
// length (unit u walks about u/2 tiles), and a workgroup of consecutive units
// lasts as long as its last one. Units of 16 rows in 4-wave workgroups double
// the waves over the same work and cut the rows a workgroup spans to 64, so
// the short units of a head finish early and the long ones spread over more
// SIMDs.
//
// Layout (16x16x32 MFMA, lane l: g = l/16, s = l%16):
//  * Sᵀ = K Qᵀ per 16-key block kb: A = K rows kb*16 + s at d = 32*kk + 8*g
//    (one 16-byte LDS read), B = Q row s at the same d (registers); lane l
//    holds the scores of query s with keys kb*16 + 4*g + r, r = 0..3.
//  * A query's 64 keys are spread over the four lanes s, s+16, s+32, s+48:
//    the row max and the row sums combine those lanes once per row (the
//    first tile and the epilogue), not per tile.
//  * Oᵀ += Vᵀ Pᵀ per 32-key step u: the lane's own weights of key blocks 2u
//    and 2u+1 form its B operand, so k-slot 8*g + t stands for key
//    32*u + 4*g + t (t < 4) or 32*u + 16 + 4*g + t - 4 (t >= 4); the A
//    operand is read with the same order by two transposing LDS reads (rows
//    32*u + 4*g.. and 32*u + 16 + 4*g..), so no weight moves between lanes.
//  * O accumulates as D/16 blocks of 16 d x 16 queries: lane l holds query s,
//    d = db*16 + 4*g + r.
#pragma once
#include "fa_fwd_kernel.h"

namespace fa {

template <int D, int DT, bool CAUSAL, int BC, int KSTR, int VSTR>
__device__ __forceinline__ void tile_step16(bool first, bool masked, const uint16_t* __restrict__ sk,
                                            const uint16_t* __restrict__ sv, int key0, int Nb, int qw0, int lane,
                                            float c, const u32x4 (&qf)[D / 32], f32x4 (&oacc)[D / 16],
                                            float& m_run, float (&l_run)[2]) {
  constexpr int KK = D / 32, DB = D / 16, KB = BC / 16;
  const int g = lane >> 4, s16 = lane & 15;

  f32x4 s[KB];
  auto scores = [&](int z) __attribute__((always_inline)) {
    const uint16_t* kt = sk + z;
    u32x4 ka[KB][KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        ka[kb][kk] = *(const u32x4*)(kt + lds_off<D, KSTR>(kb * 16 + s16, 32 * kk + 8 * g));
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) s[kb] = mfma16x16x32<DT>(ka[kb][kk], qf[kk], s[kb]);
    }
    if (masked) {
      // register r of block kb holds key key0 + 4*g + 16*kb + r: dead past
      // the end (key >= Nb) or, causal, after the query (key > qrow)
      const int base = key0 + 4 * g - z;
      int lim = Nb - 1 - base;
      if constexpr (CAUSAL) lim = min(lim, qw0 + s16 - base);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kb + r > lim) s[kb][r] = -INFINITY;
    }
  };
  scores(0);

  // weights p = exp2(s*c - mref) packed to 16 bits, key blocks 2u and 2u+1 in
  // pf[u]; lp: partial sums of the 16-bit weights; lf: fp32 sums (bf16 LSE)
  u32x4 pf[BC / 32];
  float lp[2], lf[2];
  auto probs = [&](float mref) __attribute__((always_inline)) {
    lp[0] = lp[1] = 0.f;
    lf[0] = lf[1] = 0.f;
#pragma unroll
    for (int u = 0; u < BC / 32; ++u) {
      float p[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        // c > 0 always (clamped on the host), so a masked -inf stays -inf
        p[t] = fast_exp2(__builtin_fmaf(s[2 * u + t / 4][t % 4], c, -mref));
        if constexpr (DT == DT_BF16) lf[t & 1] += p[t];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[u][e] = pack2<DT>(p[2 * e], p[2 * e + 1]);
        lp[e & 1] = dot2_sum<DT>(pf[u][e], lp[e & 1]);
      }
    }
  };
  auto tile_max = [&]() __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    return fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
  };
  if (first) m_run = tile_max() + ref_margin<DT>();
  probs(m_run == -INFINITY ? 0.f : m_run);
  const float pk = fmaxf(lp[0], lp[1]);
  if (wave_any(!(pk < partial_cap<DT>()))) {
    // some weight may have left the 16-bit range: raise the reference to the
    // true max, rescale what has been accumulated, redo the weights
    int zero = 0;
    asm volatile("" : "+s"(zero));
    scores(zero);
    const float m_new = fmaxf(m_run, tile_max());
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
    l_run[0] *= alpha;
    l_run[1] *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[db][r] *= alpha;
    m_run = m_new;
    probs(m_new == -INFINITY ? 0.f : m_new);
  }
  l_run[0] += lp[0] + lp[1];
  if constexpr (DT == DT_BF16) l_run[1] += lf[0] + lf[1];

  // Oᵀ += Vᵀ Pᵀ
#pragma unroll
  for (int u = 0; u < BC / 32; ++u) {
    const int row = 32 * u + 4 * g + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = db * 16 + 4 * (s16 & 3);
      const u32x2 lo = lds_read_tr4(sv + lds_off<D, VSTR>(row, col));
      const u32x2 hi = lds_read_tr4(sv + lds_off<D, VSTR>(row + 16, col));
      oacc[db] = mfma16x16x32<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[u], oacc[db]);
    }
  }
}

// NW waves x 16 query rows per workgroup, 64-key tiles staged as in
// fa_fwd_kernel (register loads one tile ahead, padded LDS rows, one barrier
// per tile). Causal, equal lengths (no cu_seqlens); a.units counts 16-row
// units.
template <int D, int DT, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) void fa_fwd16_kernel(const FwdArgs a) {
  static_assert(CAUSAL, "built for the causal mask");
  constexpr int NT = NW * 64, BC = 64;
  constexpr int KK = D / 32, DB = D / 16;
  constexpr int CH = BC * D / 8 / NT;  // 16-byte chunks per thread per tensor per tile
  static_assert(BC * D / 8 % NT == 0, "tile must split evenly over threads");
  // (V rows of D+16 halves: the 16-row step reads 8 consecutive rows 32 lanes
  // at a time, 8 banks each, which a stride of 40 or 72 banks keeps apart)
  using SM = FwdSmem<D, BC, D + 16>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SM::STAGE];

  // workgroup -> (batch*head, query block): blocks run by rank across heads,
  // longest first (as in fa_fwd_kernel)
  const int nbh = a.B * a.H;
  const int qi = blockIdx.x / nbh, bh = blockIdx.x - qi * nbh;
  if (qi >= a.nqb) return;
  const int qblk = a.nqb - 1 - qi;
  const int b = bh / a.H, h = bh - b * a.H;
  const int Nb = a.N;
  const int u0 = (int)((int64_t)qblk * a.units / a.nqb);
  const int u1 = (int)((int64_t)(qblk + 1) * a.units / a.nqb);

  const uint16_t* Qg = a.q + b * a.q_sb + h * a.q_sh;
  const uint16_t* Kg = a.k + b * a.k_sb + h * a.k_sh;
  const uint16_t* Vg = a.v + b * a.v_sb + h * a.v_sh;
  uint16_t* Og = a.o + b * a.o_sb + h * a.o_sh;
  float* Lg = a.lse + b * a.lse_sb + h * a.lse_sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, s16 = lane & 15;
  const int qw0 = 16 * (u0 + w);  // first query row of this wave
  const bool wave_rows = w < u1 - u0;

  // Q fragments (B operand of Sᵀ = K Qᵀ): row qw0 + s16, d = 32*kk + 8*g;
  // rows past the end load row Nb-1 and are zeroed below
  u32x4 qf[KK];
  {
    const int r = min(qw0 + s16, Nb - 1);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const u32x4*)(Qg + r * a.q_sr + 32 * kk + 8 * g);
  }

  const int kv_end = CAUSAL ? min(Nb, 16 * u1) : Nb;
  const int ntiles = (kv_end + BC - 1) / BC;

  u32x4 kst[CH], vst[CH];
  uint32_t koff[CH], voff[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ci = tid + NT * c;
    const int r = ci / (D / 8), col = (ci % (D / 8)) * 8;
    koff[c] = (uint32_t)(r * (a.k_sr * 2) + col * 2);
    voff[c] = (uint32_t)(r * (a.v_sr * 2) + col * 2);
  }
  auto fetch = [&](int t) __attribute__((always_inline)) {
    const int rows = min(kv_end - t * BC, BC);  // >= 1
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Kg + (int64_t)t * BC * a.k_sr), (short)0, (int)((rows - 1) * (a.k_sr * 2) + D * 2),
        kBufferDword3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Vg + (int64_t)t * BC * a.v_sr), (short)0, (int)((rows - 1) * (a.v_sr * 2) + D * 2),
        kBufferDword3);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      kst[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff[c], 0, 0));
      vst[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff[c], 0, 0));
    }
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
    uint16_t* sk = smem + buf * SM::STAGE;
    uint16_t* sv = sk + SM::KTILE;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = tid + NT * c;
      const int r = ci / (D / 8), col = (ci % (D / 8)) * 8;
      *(u32x4*)(sk + r * SM::KSTR + col) = kst[c];
      *(u32x4*)(sv + r * SM::VSTR + col) = vst[c];
    }
  };

  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run[2] = {0.f, 0.f};

  fetch(0);
  {
    const bool in = qw0 + s16 < Nb;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = (in ? qf[kk] : u32x4{0u, 0u, 0u, 0u}) ^ a.qsign;
  }
  stash(0);

  // as in fa_fwd_kernel: a wave's tiles end at the last key its rows see; a
  // last tile of at most 32 keys is a half step; waves past their tiles (or
  // without rows) keep loading until the workgroup's last tile
  if (wave_rows) {
    const int wave_end = CAUSAL ? min(kv_end, qw0 + 16) : kv_end;
    const int wnt = (wave_end + BC - 1) / BC;
    const bool tail32 = wave_end - (wnt - 1) * BC <= 32;
    const int nmain = tail32 ? wnt - 1 : wnt;
    int t = 0;
    for (; t < nmain; ++t) {
      __syncthreads();
      if (t + 1 < ntiles) fetch(t + 1);
      const int key0 = t * BC;
      const uint16_t* sk = smem + (t & 1) * SM::STAGE;
      const uint16_t* sv = sk + SM::KTILE;
      const bool need_mask = (key0 + BC > Nb) || (CAUSAL && key0 + BC - 1 > qw0);
      tile_step16<D, DT, CAUSAL, BC, SM::KSTR, SM::VSTR>(t == 0, need_mask, sk, sv, key0, Nb, qw0, lane, a.c, qf,
                                                             oacc, m_run, l_run);
      if (t + 1 < ntiles) stash((t + 1) & 1);
    }
    if (tail32) {
      __syncthreads();
      if (t + 1 < ntiles) fetch(t + 1);
      const uint16_t* sk = smem + (t & 1) * SM::STAGE;
      tile_step16<D, DT, CAUSAL, 32, SM::KSTR, SM::VSTR>(t == 0, true, sk, sk + SM::KTILE, t * BC, Nb, qw0, lane,
                                                             a.c, qf, oacc, m_run, l_run);
      if (t + 1 < ntiles) stash((t + 1) & 1);
      ++t;
    }
    for (; t < ntiles; ++t) {
      __syncthreads();
      if (t + 1 < ntiles) {
        fetch(t + 1);
        stash((t + 1) & 1);
      }
    }
  } else {
    for (int t = 0; t < ntiles; ++t) {
      __syncthreads();
      if (t + 1 < ntiles) {
        fetch(t + 1);
        stash((t + 1) & 1);
      }
    }
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2; rows staged in LDS ----
  constexpr int OSTR = D + 8;
  static_assert(NW * 16 * OSTR <= 2 * SM::STAGE, "output staging must fit in the K/V staging area");
  __syncthreads();  // every wave is done with the K/V tiles
  if (!wave_rows) return;
  uint16_t* ob = smem + w * 16 * OSTR;
  {
    float l_tot = l_run[0] + __shfl_xor(l_run[0], 16, 64), l_lse;
    l_tot += __shfl_xor(l_tot, 32, 64);
    if constexpr (DT == DT_F16) {
      l_lse = l_tot;
    } else {
      l_lse = l_run[1] + __shfl_xor(l_run[1], 16, 64);
      l_lse += __shfl_xor(l_lse, 32, 64);
    }
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      u32x2 x;
      x[0] = pack2<DT>(oacc[db][0] * inv, oacc[db][1] * inv);
      x[1] = pack2<DT>(oacc[db][2] * inv, oacc[db][3] * inv);
      *(u32x2*)(ob + s16 * OSTR + db * 16 + 4 * g) = x;
    }
    const int qrow = qw0 + s16;
    if (g == 0 && qrow < Nb) Lg[qrow] = (m_run + fast_log2(l_lse)) * kLn2;
  }
  wave_lds_sync();  // the rows below were written by other lanes of this wave
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < 16 * CPR / 64; ++i) {
    const int p = lane + 64 * i, r = p / CPR, ch = p % CPR;
    const u32x4 x = *(const u32x4*)(ob + r * OSTR + ch * 8);
    if (qw0 + r < Nb) *(u32x4*)(Og + (qw0 + r) * a.o_sr + ch * 8) = x;
  }
}

}  // namespace fa
