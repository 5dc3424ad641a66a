// Attention backward by recomputation for gfx950 ("FlashAttention explainer"
// (aitangshan.cn) section 6.2, first strategy; "YOLO11 attention swapped for a
// FlashAttention-2-style implementation" (discosf.com) section 2.3): only Q,
// K, V, O, dO and the forward's LSE are read; S and P are rebuilt tile by tile
// from LSE and never stored. With P = exp(s - LSE) and dP = dO Vᵀ:
//   dV = Pᵀ dO,  dS = P ∘ (dP - D),  D_i = <dO_i, O_i>,
//   dK = scale · dSᵀ Q,  dQ = scale · dS K.
//
// MI355X layout (our design), no atomics: two kernels at d = 64 and 128 (dQ,
// which also forms D_i, then dK/dV), four at d = 96 and 256. Blocks are
// ordered key or query block major, head minor.
//  * fa_bwd_dot_kernel (d = 96, 256): D_i in fp32. At d = 64 and 128 the dQ
//    kernel forms D_i for its own rows and stores it; it runs first.
//  * fa_bwd_dkdv_wide_kernel (d = 64, 128): one workgroup per block of keys,
//    each wave owning 32 keys; 64-query tiles of Q, dO, LSE and D stream
//    through LDS. S and dP are computed with the key in the lane (S = Q Kᵀ),
//    so P and dS are directly the B operand of dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS,
//    whose A operands (dOᵀ, Qᵀ) come from the row-major LDS tiles through the
//    transposing LDS read.
//  * fa_bwd_dkdv_kernel (d = 96, 256): the same as two passes, dV then dK,
//    with K and V fragments in registers.
//  * fa_bwd_dq_kernel (d = 64, 128): the mirror image with the query in the
//    lane (like the forward): Pᵀ = exp2(Sᵀ c - LSE log2 e), dPᵀ = V dOᵀ,
//    dQᵀ += Kᵀ dSᵀ; fa_bwd_dq_staged_kernel is the same for d = 96 and 256.
//  * fa_bwd_joint_kernel (d = 64, 128) and fa_bwd_joint_staged_kernel (d =
//    96, 256), for small grids: the blocks of the dQ and dK/dV kernels in one
//    launch, after fa_bwd_dot_kernel.
#pragma once
#include "fa_fwd_kernel.h"
#include "fa_fwd_split.h"

namespace fa {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dvec;   // D_i, [B, H, N] fp32 (workspace)
  int B, H, N;
  float c;       // |scale| * log2(e), > 0
  float scale;   // signed scale (multiplies dQ and dK)
  uint32_t qsign;  // 0x80008000 when scale < 0 (Q is read sign-flipped)
};

// ---- D_i = <dO_i, O_i> ----
// G consecutive lanes (a power of two) share a row, each taking D/8/G
// 16-byte chunks of O and dO, so a wave reads whole consecutive rows; the
// partial dots are then summed across those lanes.
template <int D>
constexpr int bwd_dot_lanes() {
  return (D / 8) % 16 == 0 ? 16 : (D / 8) % 8 == 0 ? 8 : 4;
}
template <int D, int DT>
__global__ __launch_bounds__(256) void fa_bwd_dot_kernel(const BwdArgs a) {
  constexpr int G = bwd_dot_lanes<D>();  // lanes per row
  constexpr int CPL = D / 8 / G;                                         // chunks per lane
  static_assert(CPL * G * 8 == D, "row must split evenly over its lanes");
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = t / G;
  const int ln = (int)(t % G);
  float acc = 0.f;
  if (r < rows) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int col = 8 * (ln + G * c);
      const u32x4 x = *(const u32x4*)(a.o + r * D + col);
      const u32x4 y = *(const u32x4*)(a.dout + r * D + col);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += to_f32<DT>((uint16_t)(x[e] & 0xFFFF)) * to_f32<DT>((uint16_t)(y[e] & 0xFFFF));
        acc += to_f32<DT>((uint16_t)(x[e] >> 16)) * to_f32<DT>((uint16_t)(y[e] >> 16));
      }
    }
  }
  // G divides 64 and each row starts at a multiple of G lanes, so a row's
  // lanes sit inside one wave
#pragma unroll
  for (int m = G / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (r < rows && ln == 0) a.dvec[r] = acc;
}

template <int D>
struct BwdSmem {
  // query rows per tile (two-pass dK/dV kernel); 32 at d = 256, which halves
  // the registers that stage the next tile (64 -> 32) and keeps the dK pass
  // free of spills at one wave per SIMD
  static constexpr int BQ = D == 256 ? 32 : 64;
  static constexpr int STR = D + 16;   // padded row (halves)
  static constexpr int TILE = BQ * STR;
  // per stage: Q tile, dO tile, LSE·log2e, D
  static constexpr int STAGE_HALVES = 2 * TILE + 2 * BQ * 2;
};

// 16 per-register row values for rows 8*(r/4) + 4*hh + r%4 of a 32-row block
// starting at `base` of an fp32 LDS vector (the row layout of an MFMA
// accumulator)
__device__ __forceinline__ f32x16 load_rowvals(const float* base, int hh) {
  f32x16 v;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 x = *(const f32x4*)(base + 8 * g + 4 * hh);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * g + e] = x[e];
  }
  return v;
}

// ---- dK, dV in two passes: one workgroup per 128 keys ----
// PART BWD_DV computes only dV (no V fragments, no dP), PART BWD_DK only dK.
// At d = 96 (whose 12 chunks per row do not split over the single-pass
// kernel's LDS-DMA) each pass then fits two waves per SIMD with the K and V
// fragments in registers. At d = 256 a pass holds 128 accumulator registers
// besides 64 of K (and 64 of V) fragments: one wave per SIMD, with the
// accumulation registers as overflow, and 69 KB of LDS per workgroup.
enum { BWD_DV = 1, BWD_DK = 2 };
template <int D>
constexpr int bwd_pass_min_blocks() {
  return D == 256 ? 1 : 2;
}
template <int D, int DT, bool CAUSAL, int PART>
__device__ __forceinline__ void dkdv_pass_body(const BwdArgs& a, const int bid, uint16_t* smem) {
  static_assert(PART == BWD_DV || PART == BWD_DK, "one of the two passes");
  constexpr bool WANT_DV = PART == BWD_DV, WANT_DK = PART == BWD_DK;
  constexpr int NW = 4, NT = 256, KK = D / 16, DB = D / 32;
  using SM = BwdSmem<D>;
  constexpr int BQ = SM::BQ, STR = SM::STR;
  constexpr int CH = BQ * D / 8 / NT;  // 16-byte chunks per thread per tile
  static_assert(BQ * D / 8 % NT == 0, "tile must split evenly");

  // block order as in fa_bwd_dkdv_wide_kernel: key block major, head minor
  const int nkb = (a.N + 127) / 128;
  const int BH = a.B * a.H;
  const int kblk = bid / BH, bh = bid - kblk * BH;
  if (kblk >= nkb) return;
  const int64_t off = (int64_t)bh * a.N * D;
  const uint16_t* Qg = a.q + off;
  const uint16_t* Kg = a.k + off;
  const uint16_t* Vg = a.v + off;
  const uint16_t* Gg = a.dout + off;
  const float* Lg = a.lse + (int64_t)bh * a.N;
  const float* Dg = a.dvec + (int64_t)bh * a.N;
  const int N = a.N;

  // the wave index read from the first lane, so that what derives from it
  // (tile ranges, buffer descriptors, LDS-DMA bases) is scalar: no per-lane
  // loop around loads (N=8192 causal d=128: 1875 -> 1785 us per backward)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int kw0 = kblk * 128 + w * 32;  // first key of this wave
  const int krow = kw0 + l32;

  // K and V fragments of this wave's keys (B operands: key in the lane)
  u32x4 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int rr = min(krow, N - 1);
    const u32x4 xk = *(const u32x4*)(Kg + (int64_t)rr * D + 16 * kk + 8 * hh);
    const u32x4 xv = *(const u32x4*)(Vg + (int64_t)rr * D + 16 * kk + 8 * hh);
    kf[kk] = krow < N ? xk : u32x4{0u, 0u, 0u, 0u};
    if constexpr (WANT_DK) vf[kk] = krow < N ? xv : u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 dk[WANT_DK ? DB : 1], dv[WANT_DV ? DB : 1];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (WANT_DK) dk[db][r] = 0.f;
      if constexpr (WANT_DV) dv[db][r] = 0.f;
    }

  // query tiles: causal blocks start at the tile holding the first key
  const int t0 = CAUSAL ? (kblk * 128) / BQ : 0;
  const int nt = (N + BQ - 1) / BQ;

  // The tile's Q and dO chunks and its rows' LSE and D_i are held raw in
  // registers from the loads to the stash at the end of the tile: any
  // arithmetic on them at the loads (sign flip, zeroing rows past the end)
  // would wait for each load right there.
  u32x4 qs[CH], gs[CH];
  float lraw = 0.f, draw = 0.f;
  int qf0 = 0;  // first query row of the fetched tile
  const float inv_c = 1.f / a.c;
  auto fetch = [&](int t) __attribute__((always_inline)) {
    qf0 = t * BQ;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = tid + NT * c;
      const int r = ci / (D / 8), col = (ci % (D / 8)) * 8;
      const int gr = min(qf0 + r, N - 1);
      qs[c] = *(const u32x4*)(Qg + (int64_t)gr * D + col);
      gs[c] = *(const u32x4*)(Gg + (int64_t)gr * D + col);
    }
    if (tid < BQ && qf0 + tid < N) {
      lraw = Lg[qf0 + tid];
      draw = Dg[qf0 + tid];
    }
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
    uint16_t* sq = smem + buf * SM::STAGE_HALVES;
    uint16_t* sg = sq + SM::TILE;
    float* sl = (float*)(sg + SM::TILE);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = tid + NT * c;
      const int r = ci / (D / 8), col = (ci % (D / 8)) * 8;
      const bool in = qf0 + r < N;
      *(u32x4*)(sq + r * STR + col) = in ? (qs[c] ^ a.qsign) : u32x4{0u, 0u, 0u, 0u};
      *(u32x4*)(sg + r * STR + col) = in ? gs[c] : u32x4{0u, 0u, 0u, 0u};
    }
    // per query row: -LSE log2(e) / c and -D_i, the starting values of the S
    // and dP accumulators; rows past the end start at -inf, which makes their
    // weights exactly zero
    if (tid < BQ) {
      const bool in = qf0 + tid < N;
      sl[tid] = in ? -lraw * kLog2e * inv_c : -INFINITY;
      sl[BQ + tid] = in ? -draw : 0.f;
    }
  };

  if (t0 < nt) {
    fetch(t0);
    stash(0);
  }
  const int g16 = lane >> 4, s16 = lane & 15;
  for (int t = t0; t < nt; ++t) {
    __syncthreads();
    if (t + 1 < nt) fetch(t + 1);
    const uint16_t* sq = smem + ((t - t0) & 1) * SM::STAGE_HALVES;
    const uint16_t* sg = sq + SM::TILE;
    const float* sl = (const float*)(sg + SM::TILE);
    const int q0 = t * BQ;
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int qr0 = q0 + 32 * qb;  // first query of this 32-row block
      if (CAUSAL && qr0 + 31 < kw0) continue;  // every query precedes every key
      // S = Q Kᵀ and dP = dO Vᵀ, key in the lane, queries in the registers.
      // The accumulators start at the row terms, so that they end as
      // S - LSE log2(e) / c (c times it is the log2 weight) and dP - D_i:
      // no registers hold the 16 row values of each beside them.
      f32x16 s = load_rowvals(sl + 32 * qb, hh), dp;
      if constexpr (WANT_DK) dp = load_rowvals(sl + BQ + 32 * qb, hh);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 qa = *(const u32x4*)(sq + (32 * qb + l32) * STR + 16 * kk + 8 * hh);
        s = mfma32x32x16<DT>(qa, kf[kk], s);
        if constexpr (WANT_DK) {
          const u32x4 ga = *(const u32x4*)(sg + (32 * qb + l32) * STR + 16 * kk + 8 * hh);
          dp = mfma32x32x16<DT>(ga, vf[kk], dp);
        }
      }
      // P and dS = P dP, packed; the causal mask of a diagonal block is a
      // second copy of the loop under a uniform branch (a test inside the one
      // loop became selects executed on every block)
      u32x4 pp[2], sp[2];
      auto weights = [&](bool mask) __attribute__((always_inline)) {
        // register r holds query qr0 + 8*(r/4) + 4*hh + r%4
        const int lim = krow - (qr0 + 4 * hh);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float pv[2], sv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = 8 * c2 + 2 * e + u;
              float p = fast_exp2(s[r] * a.c);
              if (mask && 8 * (r >> 2) + (r & 3) < lim) p = 0.f;
              pv[u] = p;
              if constexpr (WANT_DK) sv[u] = p * dp[r];
            }
            if constexpr (WANT_DV) pp[c2][e] = pack2<DT>(pv[0], pv[1]);
            if constexpr (WANT_DK) sp[c2][e] = pack2<DT>(sv[0], sv[1]);
          }
        }
      };
      if (CAUSAL && qr0 < kw0 + 31)
        weights(true);
      else
        weights(false);
      // dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS ; k-slot 8*hh + 4*rd + e of chunk c2 is
      // query 16*c2 + 8*rd + 4*hh + e of this block
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int ra = 32 * qb + 16 * c2 + 4 * hh + (s16 >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = db * 32 + (g16 & 1) * 16 + 4 * (s16 & 3);
          if constexpr (WANT_DV) {
            const u32x2 glo = lds_read_tr4(sg + ra * STR + col);
            const u32x2 ghi = lds_read_tr4(sg + (ra + 8) * STR + col);
            dv[db] = mfma32x32x16<DT>(u32x4{glo[0], glo[1], ghi[0], ghi[1]}, pp[c2], dv[db]);
          }
          if constexpr (WANT_DK) {
            const u32x2 qlo = lds_read_tr4(sq + ra * STR + col);
            const u32x2 qhi = lds_read_tr4(sq + (ra + 8) * STR + col);
            dk[db] = mfma32x32x16<DT>(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, sp[c2], dk[db]);
          }
        }
      }
    }
    if (t + 1 < nt) stash((t + 1 - t0) & 1);
  }

  // dK = scale dSᵀ Q = |scale| dSᵀ Q' (Q' is Q with its sign folded in for a
  // negative scale); dV = Pᵀ dO. Key row, 4 consecutive d per group.
  if (krow < N) {
    uint16_t* dkr = a.dk + off + (int64_t)krow * D;
    uint16_t* dvr = a.dv + off + (int64_t)krow * D;
    const float sk = fabsf(a.scale);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = db * 32 + 8 * g4 + 4 * hh;
        if constexpr (WANT_DK) {
          u32x2 x;
          x[0] = pack2<DT>(dk[db][4 * g4 + 0] * sk, dk[db][4 * g4 + 1] * sk);
          x[1] = pack2<DT>(dk[db][4 * g4 + 2] * sk, dk[db][4 * g4 + 3] * sk);
          *(u32x2*)(dkr + col) = x;
        }
        if constexpr (WANT_DV) {
          u32x2 y;
          y[0] = pack2<DT>(dv[db][4 * g4 + 0], dv[db][4 * g4 + 1]);
          y[1] = pack2<DT>(dv[db][4 * g4 + 2], dv[db][4 * g4 + 3]);
          *(u32x2*)(dvr + col) = y;
        }
      }
  }
}

template <int D, int DT, bool CAUSAL, int PART>
__global__ __launch_bounds__(256, (bwd_pass_min_blocks<D>())) void fa_bwd_dkdv_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * BwdSmem<D>::STAGE_HALVES];
  dkdv_pass_body<D, DT, CAUSAL, PART>(a, blockIdx.x, smem);
}

// ---- dK and dV in one pass: NW waves, 32 NW keys per workgroup ----
// Both accumulators in one pass, so S and the exponentials are computed once
// per (query, key) pair. What keeps the registers down (d = 128, 8 waves:
// two waves per SIMD; d = 64, 4 waves: three):
//  * each wave keeps only its K fragments in registers and parks its V
//    fragments in its own LDS slice, in fragment order (one conflict-free
//    16-byte read per lane and k-step);
//  * the 64-query Q and dO tiles arrive by LDS-DMA (buffer_load ... lds, no
//    staging registers) into unpadded rows whose 16-byte chunks are
//    XOR-swizzled (lds_off<D, 0>), double-buffered and shared by the NW waves.
// A negative scale flips the sign of K (so S keeps the sign of scale·q·k)
// and multiplies dK at the end; Q is used as stored.
template <int D, int NW>
constexpr int dkdv_wide_smem_halves() {
  return 2 * (2 * 64 * D + 2 * 64 * 2) + NW * (D / 16) * 64 * 8;
}
template <int D, int DT, bool CAUSAL, int NW>
__device__ __forceinline__ void dkdv_wide_body(const BwdArgs& a, const int bid, uint16_t* smem) {
  constexpr int KK = D / 16, DB = D / 32, KW = 32 * NW, BQ = 64, CPR = D / 8;
  constexpr int TILE = BQ * D;                   // halves per unpadded Q or dO tile
  constexpr int STAGE = 2 * TILE + 2 * BQ * 2;   // Q, dO, then the row terms (fp32)
  constexpr int LOADS = BQ * CPR / 64;           // wave loads (1 KB) per tensor per tile
  static_assert(LOADS % NW == 0, "tile loads split evenly over the waves");
  constexpr int LPW = LOADS / NW;
  constexpr int VFRAG = KK * 64;                 // u32x4 per wave
  static_assert(2 * STAGE + NW * VFRAG * 8 == dkdv_wide_smem_halves<D, NW>(), "LDS size");

  // block order: key block major, head minor. Causal blocks then start
  // longest first across all heads (a head-major order leaves the long
  // blocks of the last heads for the end), and with B*H a multiple of the 8
  // XCDs every block of a head lands on one XCD, sharing its Q/dO in L2.
  const int nkb = (a.N + KW - 1) / KW;
  const int BH = a.B * a.H;
  const int kblk = bid / BH, bh = bid - kblk * BH;
  if (kblk >= nkb) return;
  const int64_t off = (int64_t)bh * a.N * D;
  const uint16_t* Qg = a.q + off;
  const uint16_t* Kg = a.k + off;
  const uint16_t* Vg = a.v + off;
  const uint16_t* Gg = a.dout + off;
  const float* Lg = a.lse + (int64_t)bh * a.N;
  const float* Dg = a.dvec + (int64_t)bh * a.N;
  const int N = a.N;

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int kw0 = kblk * KW + w * 32;  // first key of this wave
  const int krow = kw0 + l32;

  // K fragments (sign of the scale folded in) in registers, V fragments in
  // this wave's LDS slice; keys past the end are zero
  u32x4 kf[KK];
  u32x4* vl = (u32x4*)(smem + 2 * STAGE) + w * VFRAG;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int rr = min(krow, N - 1);
    const u32x4 xk = *(const u32x4*)(Kg + (int64_t)rr * D + 16 * kk + 8 * hh);
    const u32x4 xv = *(const u32x4*)(Vg + (int64_t)rr * D + 16 * kk + 8 * hh);
    kf[kk] = krow < N ? (xk ^ a.qsign) : u32x4{0u, 0u, 0u, 0u};
    vl[kk * 64 + lane] = krow < N ? xv : u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[db][r] = 0.f;
      dv[db][r] = 0.f;
    }

  // query tiles: causal blocks start at the tile holding the block's first key
  const int t0 = CAUSAL ? (kblk * KW) / BQ : 0;
  const int nt = (N + BQ - 1) / BQ;

  // this wave's share of the Q and dO tiles of query tile t: chunk slot
  // P = 64 i + lane is row P / CPR, slot P % CPR, and receives that row's
  // chunk (slot ^ swizzle); rows past the end lie outside the descriptor and
  // arrive as zeros
  auto dma = [&](int t, int buf) __attribute__((always_inline)) {
    const int q0 = t * BQ;
    const int rows = min(N - q0, BQ);  // >= 1
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Qg + (int64_t)q0 * D), (short)0, rows * D * 2, kBufferDword3);
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Gg + (int64_t)q0 * D), (short)0, rows * D * 2, kBufferDword3);
    uint16_t* dq = smem + buf * STAGE;
    uint16_t* dg = dq + TILE;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int i = w * LPW + j;
      const int P = 64 * i + lane;
      const int r = P / CPR, ch = (P % CPR) ^ lds_swz<D>(r);
      const uint32_t o = (uint32_t)(r * D * 2 + ch * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)(dq + 64 * i * 8), 16,
                                               o, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (__attribute__((address_space(3))) void*)(dg + 64 * i * 8), 16,
                                               o, 0, 0, 0);
    }
  };
  // per query row: -LSE log2(e) / c and -D_i, the starting values of the S
  // and dP accumulators (rows past the end: -inf, so their weights are zero).
  // Wave 0 converts them at the load, and so waits there for the LDS-DMA it
  // has just issued; keeping them raw until the stash measured N=4096 0.5 %
  // faster and N=400 batched 1.5 % slower per backward.
  float ls = 0.f, ds = 0.f;
  const float inv_c = 1.f / a.c;
  auto fetch_rows = [&](int t) __attribute__((always_inline)) {
    if (tid < BQ) {
      const int gr = t * BQ + tid;
      ls = gr < N ? -Lg[gr] * kLog2e * inv_c : -INFINITY;
      ds = gr < N ? -Dg[gr] : 0.f;
    }
  };
  auto stash_rows = [&](int buf) __attribute__((always_inline)) {
    float* sl = (float*)(smem + buf * STAGE + 2 * TILE);
    if (tid < BQ) {
      sl[tid] = ls;
      sl[BQ + tid] = ds;
    }
  };

  if (t0 < nt) {
    dma(t0, 0);
    fetch_rows(t0);
    stash_rows(0);
  }
  const int g16 = lane >> 4, s16 = lane & 15;
  for (int t = t0; t < nt; ++t) {
    // tile t has landed (this wave's DMA, then everyone's), its row terms
    // are stored, and no wave still reads the other buffer
    wait_vmcnt<0>();
    __syncthreads();
    const int buf = (t - t0) & 1;
    if (t + 1 < nt) {
      dma(t + 1, buf ^ 1);
      fetch_rows(t + 1);
    }
    const uint16_t* sq = smem + buf * STAGE;
    const uint16_t* sg = sq + TILE;
    const float* sl = (const float*)(sg + TILE);
    const int q0 = t * BQ;
    // one 32-query block; the non-causal loop over blocks is unrolled, so that
    // the second block's LDS addresses are the first block's plus an immediate
    // offset (the swizzle depends only on the low 4 bits of a row) instead of
    // 31 address instructions a block; the causal one, with its masked copy of
    // the weights, would spill unrolled
    auto qblock = [&](int qb) __attribute__((always_inline)) {
      const int qr0 = q0 + 32 * qb;
      if (CAUSAL && qr0 + 31 < kw0) return;  // every query precedes every key
      f32x16 s = load_rowvals(sl + 32 * qb, hh), dp = load_rowvals(sl + BQ + 32 * qb, hh);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 qa = *(const u32x4*)(sq + lds_off<D, 0>(32 * qb + l32, 16 * kk + 8 * hh));
        const u32x4 ga = *(const u32x4*)(sg + lds_off<D, 0>(32 * qb + l32, 16 * kk + 8 * hh));
        s = mfma32x32x16<DT>(qa, kf[kk], s);
        dp = mfma32x32x16<DT>(ga, vl[kk * 64 + lane], dp);
      }
      // phase boundaries for the scheduler: LDS reads hoisted across them
      // would hold registers through the exponentials (48 spilled)
      __builtin_amdgcn_sched_barrier(0);
      // P and dS = P dP, packed; the causal mask of a diagonal block is a
      // second copy of the loop under a uniform branch (a test inside the one
      // loop became selects executed on every block)
      u32x4 pp[2], sp[2];
      auto weights = [&](bool mask) __attribute__((always_inline)) {
        // register r holds query qr0 + 8*(r/4) + 4*hh + r%4
        const int lim = krow - (qr0 + 4 * hh);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float pv[2], sv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = 8 * c2 + 2 * e + u;
              float p = fast_exp2(s[r] * a.c);
              if (mask && 8 * (r >> 2) + (r & 3) < lim) p = 0.f;
              pv[u] = p;
              sv[u] = p * dp[r];
            }
            pp[c2][e] = pack2<DT>(pv[0], pv[1]);
            sp[c2][e] = pack2<DT>(sv[0], sv[1]);
          }
        }
      };
      if (CAUSAL && qr0 < kw0 + 31)
        weights(true);
      else
        weights(false);
      __builtin_amdgcn_sched_barrier(0);
      // dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS ; k-slot 8*hh + 4*rd + e of chunk c2 is
      // query 16*c2 + 8*rd + 4*hh + e of this block
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int ra = 32 * qb + 16 * c2 + 4 * hh + (s16 >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = db * 32 + (g16 & 1) * 16 + 4 * (s16 & 3);
          const u32x2 glo = lds_read_tr4(sg + lds_off<D, 0>(ra, col));
          const u32x2 ghi = lds_read_tr4(sg + lds_off<D, 0>(ra + 8, col));
          dv[db] = mfma32x32x16<DT>(u32x4{glo[0], glo[1], ghi[0], ghi[1]}, pp[c2], dv[db]);
          const u32x2 qlo = lds_read_tr4(sq + lds_off<D, 0>(ra, col));
          const u32x2 qhi = lds_read_tr4(sq + lds_off<D, 0>(ra + 8, col));
          dk[db] = mfma32x32x16<DT>(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, sp[c2], dk[db]);
        }
      }
    };
    if constexpr (CAUSAL) {
#pragma unroll 1
      for (int qb = 0; qb < BQ / 32; ++qb) qblock(qb);
    } else {
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) qblock(qb);
    }
    if (t + 1 < nt) stash_rows(buf ^ 1);
  }

  // dK = scale dSᵀ Q, dV = Pᵀ dO; key row, 4 consecutive d per group
  if (krow < N) {
    uint16_t* dkr = a.dk + off + (int64_t)krow * D;
    uint16_t* dvr = a.dv + off + (int64_t)krow * D;
    const float sk = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = db * 32 + 8 * g4 + 4 * hh;
        u32x2 x, y;
        x[0] = pack2<DT>(dk[db][4 * g4 + 0] * sk, dk[db][4 * g4 + 1] * sk);
        x[1] = pack2<DT>(dk[db][4 * g4 + 2] * sk, dk[db][4 * g4 + 3] * sk);
        y[0] = pack2<DT>(dv[db][4 * g4 + 0], dv[db][4 * g4 + 1]);
        y[1] = pack2<DT>(dv[db][4 * g4 + 2], dv[db][4 * g4 + 3]);
        *(u32x2*)(dkr + col) = x;
        *(u32x2*)(dvr + col) = y;
      }
  }
}

template <int D, int DT, bool CAUSAL, int NW, int MINB>
__global__ __launch_bounds__(NW * 64, MINB) void fa_bwd_dkdv_wide_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[dkdv_wide_smem_halves<D, NW>()];
  dkdv_wide_body<D, DT, CAUSAL, NW>(a, blockIdx.x, smem);
}

// ---- dQ: one workgroup per NW*32 queries (query in the lane) ----
// NW waves of 32 query rows per workgroup (8 at d = 128, 4 at d = 64). K/V
// tiles arrive by LDS-DMA into unpadded, XOR-swizzled rows (no staging
// registers); at d = 64 each wave also parks its dO fragments in its own LDS
// slice, which brings the kernel to three waves per SIMD.
template <int D, int NW>
constexpr int dq_smem_halves() {
  return 4 * 64 * D + (D == 64 ? NW * (D / 16) * 64 * 8 : 0);
}
template <int D, int DT, bool CAUSAL, int NW, bool DI>
__device__ __forceinline__ void dq_body(const BwdArgs& a, const int bid, uint16_t* smem) {
  static_assert(D == 64 || D == 128, "swizzled LDS-DMA tiles: d = 64 or 128");
  constexpr int BR = NW * 32, BC = 64, KK = D / 16, DB = D / 32, KB = BC / 32, CPR = D / 8;
  constexpr int TILE = BC * D;                   // halves per unpadded K or V tile
  constexpr int LOADS = BC * CPR / 64;           // wave loads (1 KB) per tensor per tile
  static_assert(LOADS % NW == 0, "tile loads split evenly over the waves");
  constexpr int LPW = LOADS / NW;
  constexpr bool GL = D == 64;                   // dO fragments parked in LDS
  constexpr int GFRAG = KK * 64;                 // u32x4 per wave
  static_assert(4 * TILE + (GL ? NW * GFRAG * 8 : 0) == dq_smem_halves<D, NW>(), "LDS size");

  // block order: query block major (causal: longest first across all
  // heads), head minor, as in fa_bwd_dkdv_wide_kernel
  const int nqb = (a.N + BR - 1) / BR;
  const int BH = a.B * a.H;
  const int qblk0 = bid / BH, bh = bid - qblk0 * BH;
  if (qblk0 >= nqb) return;
  const int qblk = CAUSAL ? nqb - 1 - qblk0 : qblk0;
  const int64_t off = (int64_t)bh * a.N * D;
  const uint16_t* Qg = a.q + off;
  const uint16_t* Kg = a.k + off;
  const uint16_t* Vg = a.v + off;
  const uint16_t* Gg = a.dout + off;
  const int N = a.N;

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int qw0 = qblk * BR + w * 32;
  const int qrow = qw0 + l32;

  // Q and dO fragments of this lane's row (its half of the d columns), and
  // (DI) D_i = <dO_i, O_i> from the same half of O plus the partner lane's
  // half, stored for the dK/dV kernel, which runs after this one; without
  // DI, D_i is read from the row terms fa_bwd_dot_kernel wrote.
  u32x4 qf[KK], gf[GL ? 1 : KK];
  u32x4* gl = (u32x4*)(smem + 4 * TILE) + w * GFRAG;
  const uint16_t* Og = a.o + off;
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int rr = min(qrow, N - 1);
    const u32x4 x = *(const u32x4*)(Qg + (int64_t)rr * D + 16 * kk + 8 * hh);
    const u32x4 y = *(const u32x4*)(Gg + (int64_t)rr * D + 16 * kk + 8 * hh);
    const u32x4 ov = DI ? *(const u32x4*)(Og + (int64_t)rr * D + 16 * kk + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
    qf[kk] = (qrow < N ? x : u32x4{0u, 0u, 0u, 0u}) ^ a.qsign;
    const u32x4 g = qrow < N ? y : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dpart += to_f32<DT>((uint16_t)(g[e] & 0xFFFF)) * to_f32<DT>((uint16_t)(ov[e] & 0xFFFF));
      dpart += to_f32<DT>((uint16_t)(g[e] >> 16)) * to_f32<DT>((uint16_t)(ov[e] >> 16));
    }
    if constexpr (GL)
      gl[kk * 64 + lane] = g;
    else
      gf[kk] = g;
  }
  const float lq = qrow < N ? a.lse[(int64_t)bh * N + qrow] * kLog2e : INFINITY;
  float dq_row;
  if constexpr (DI) {
    dq_row = dpart + xor_lane32(dpart);
    if (hh == 0 && qrow < N) a.dvec[(int64_t)bh * N + qrow] = dq_row;
  } else {
    dq_row = qrow < N ? a.dvec[(int64_t)bh * N + qrow] : 0.f;
  }

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  const int kv_end = CAUSAL ? min(N, (qblk + 1) * BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;
  // tiles this wave computes: causal waves stop at their own diagonal (the
  // rest are fully masked) and then only help with the loads; waves with no
  // rows only help with the loads
  const int wave_end = qw0 >= N ? 0 : (CAUSAL ? min(kv_end, qw0 + 32) : kv_end);
  const int wnt = (wave_end + BC - 1) / BC;
  // this wave's share of K/V tile t into buffer `buf`: chunk slot P = 64 i +
  // lane is row P / CPR, slot P % CPR, and receives that row's chunk (slot ^
  // swizzle); rows past kv_end lie outside the descriptor and arrive as zeros
  auto dma = [&](int t, int buf) __attribute__((always_inline)) {
    const int rows = min(kv_end - t * BC, BC);  // >= 1
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Kg + (int64_t)t * BC * D), (short)0, rows * D * 2, kBufferDword3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Vg + (int64_t)t * BC * D), (short)0, rows * D * 2, kBufferDword3);
    uint16_t* kd = smem + buf * 2 * TILE;
    uint16_t* vd = kd + TILE;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int i = w * LPW + j;
      const int P = 64 * i + lane;
      const int r = P / CPR, ch = (P % CPR) ^ lds_swz<D>(r);
      const uint32_t o = (uint32_t)(r * D * 2 + ch * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(kd + 64 * i * 8), 16,
                                               o, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(vd + 64 * i * 8), 16,
                                               o, 0, 0, 0);
    }
  };
  // tile t has landed (this wave's DMA, then everyone's) and no wave still
  // reads the buffer the next tile goes to
  auto arrive = [&](int t) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    __syncthreads();
    if (t + 1 < ntiles) dma(t + 1, (t + 1) & 1);
  };

  dma(0, 0);
  const int g16 = lane >> 4, s16 = lane & 15;
  int t = 0;
  for (; t < wnt; ++t) {
    arrive(t);
    const uint16_t* sk = smem + (t & 1) * 2 * TILE;
    const uint16_t* sv = sk + TILE;
    const int key0 = t * BC;
    // Sᵀ = K Qᵀ and dPᵀ - D = V dOᵀ - D: query in the lane, keys in the
    // registers (the dP accumulators start at -D of the lane's row)
    f32x16 s[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[kb][r] = -dq_row;
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 g;
      if constexpr (GL)
        g = gl[kk * 64 + lane];
      else
        g = gf[kk];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 ka = *(const u32x4*)(sk + lds_off<D, 0>(kb * 32 + l32, 16 * kk + 8 * hh));
        const u32x4 va = *(const u32x4*)(sv + lds_off<D, 0>(kb * 32 + l32, 16 * kk + 8 * hh));
        s[kb] = mfma32x32x16<DT>(ka, qf[kk], s[kb]);
        dp[kb] = mfma32x32x16<DT>(va, g, dp[kb]);
      }
    }
    // phase boundaries for the scheduler (LDS reads hoisted across them
    // would hold registers through the exponentials)
    __builtin_amdgcn_sched_barrier(0);
    // P in place of S; the mask runs as a loop of its own under a uniform
    // branch (inside the loop above the compiler turned it into selects
    // executed on every tile: 95 of the tile's 252 VALU instructions at d=64)
    const bool masked = key0 + BC > N || (CAUSAL && key0 + BC - 1 > qw0);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], a.c, -lq));
    if (masked) {
      // register r of block kb holds key key0 + 32*kb + 8*(r/4) + 4*hh + r%4
      int lim = N - 1 - (key0 + 4 * hh);
      if constexpr (CAUSAL) lim = min(lim, qrow - (key0 + 4 * hh));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = 0.f;
    }
    u32x4 sf[BC / 16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * c2 + 2 * e;
          x[e] = pack2<DT>(s[kb][r] * dp[kb][r], s[kb][r + 1] * dp[kb][r + 1]);
        }
        sf[2 * kb + c2] = x;
      }
    __builtin_amdgcn_sched_barrier(0);
    // dQᵀ += Kᵀ dSᵀ ; k-slot 8*hh + 4*rd + e of chunk ci is key 16*ci + 8*rd + 4*hh + e
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ci = 0; ci < BC / 16; ++ci) {
        const int col = db * 32 + (g16 & 1) * 16 + 4 * (s16 & 3);
        const int ra = 16 * ci + 4 * hh + (s16 >> 2);
        const u32x2 lo = lds_read_tr4(sk + lds_off<D, 0>(ra, col));
        const u32x2 hi = lds_read_tr4(sk + lds_off<D, 0>(ra + 8, col));
        dqacc[db] = mfma32x32x16<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, sf[ci], dqacc[db]);
      }
  }
  for (; t < ntiles; ++t) arrive(t);

  if (qrow < N) {
    uint16_t* dqr = a.dq + off + (int64_t)qrow * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 x;
        x[0] = pack2<DT>(dqacc[db][4 * g4 + 0] * sc, dqacc[db][4 * g4 + 1] * sc);
        x[1] = pack2<DT>(dqacc[db][4 * g4 + 2] * sc, dqacc[db][4 * g4 + 3] * sc);
        *(u32x2*)(dqr + db * 32 + 8 * g4 + 4 * hh) = x;
      }
  }
}

template <int D, int DT, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64, D == 64 ? 3 : 1) void fa_bwd_dq_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[dq_smem_halves<D, NW>()];
  dq_body<D, DT, CAUSAL, NW, true>(a, blockIdx.x, smem);
}

// ---- dQ and dK/dV blocks in one grid (d = 64, 128) ----
// For grids that leave the chip half empty: block 2i is dQ block i (D_i read
// from fa_bwd_dot_kernel, which runs first), block 2i + 1 is dK/dV block i,
// so the two halves of the backward run side by side instead of one after
// the other. NW waves per workgroup as in the separate kernels (the dQ and
// dK/dV grids then have the same number of blocks), LDS the larger of the two.
template <int D>
constexpr int bwd_joint_waves() {
  return D == 128 ? 8 : 4;
}
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(bwd_joint_waves<D>() * 64, D == 64 ? 3 : 1)
void fa_bwd_joint_kernel(const BwdArgs a) {
  constexpr int NW = bwd_joint_waves<D>();
  constexpr int H1 = dq_smem_halves<D, NW>(), H2 = dkdv_wide_smem_halves<D, NW>();
  __shared__ __attribute__((aligned(16))) uint16_t smem[H1 > H2 ? H1 : H2];
  const int bid = blockIdx.x;
  if (bid & 1)
    dkdv_wide_body<D, DT, CAUSAL, NW>(a, bid >> 1, smem);
  else
    dq_body<D, DT, CAUSAL, NW, false>(a, bid >> 1, smem);
}

// ---- dQ at d = 96 and 256: K/V tiles staged through registers into padded
// rows (96 halves per row split into 12 chunks, which the XOR swizzle of the
// LDS-DMA layout does not cover; at 256 the swizzle is not laid out either).
// Otherwise as fa_bwd_dq_kernel. At d = 256 it runs at one wave per SIMD
// (Q and dO fragments 128 registers, the dQ accumulator 128).
template <int D, int DT, bool CAUSAL, int NW>
__device__ __forceinline__ void dq_staged_body(const BwdArgs& a, const int bid, uint16_t* smem) {
  constexpr int NT = NW * 64, BR = NW * 32, BC = 64, KK = D / 16, DB = D / 32, KB = BC / 32;
  constexpr int CH = BC * D / 8 / NT;
  static_assert(BC * D / 8 % NT == 0, "tile must split evenly");
  using SM = FwdSmem<D, BC>;

  const int nqb = (a.N + BR - 1) / BR;
  const int BH = a.B * a.H;
  const int qblk0 = bid / BH, bh = bid - qblk0 * BH;
  if (qblk0 >= nqb) return;
  const int qblk = CAUSAL ? nqb - 1 - qblk0 : qblk0;  // longest first
  const int64_t off = (int64_t)bh * a.N * D;
  const uint16_t* Qg = a.q + off;
  const uint16_t* Kg = a.k + off;
  const uint16_t* Vg = a.v + off;
  const uint16_t* Gg = a.dout + off;
  const int N = a.N;

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int qw0 = qblk * BR + w * 32;
  const int qrow = qw0 + l32;

  u32x4 qf[KK], gf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int rr = min(qrow, N - 1);
    const u32x4 x = *(const u32x4*)(Qg + (int64_t)rr * D + 16 * kk + 8 * hh);
    const u32x4 y = *(const u32x4*)(Gg + (int64_t)rr * D + 16 * kk + 8 * hh);
    qf[kk] = (qrow < N ? x : u32x4{0u, 0u, 0u, 0u}) ^ a.qsign;
    gf[kk] = qrow < N ? y : u32x4{0u, 0u, 0u, 0u};
  }
  const float lq = qrow < N ? a.lse[(int64_t)bh * N + qrow] * kLog2e : INFINITY;
  const float dq_row = qrow < N ? a.dvec[(int64_t)bh * N + qrow] : 0.f;

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  const int kv_end = CAUSAL ? min(N, (qblk + 1) * BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;
  // tiles this wave computes: causal waves stop at their own diagonal (the
  // rest are fully masked) and then only help with the loads; waves with no
  // rows only help with the loads
  const int wave_end = qw0 >= N ? 0 : (CAUSAL ? min(kv_end, qw0 + 32) : kv_end);
  const int wnt = (wave_end + BC - 1) / BC;
  // K/V chunks stay raw from the loads to the stash (zeroing rows past the
  // end at the loads would wait for each load right there)
  u32x4 kst[CH], vst[CH];
  int kf0 = 0;  // first key row of the fetched tile
  auto fetch = [&](int t) __attribute__((always_inline)) {
    kf0 = t * BC;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = tid + NT * c;
      const int r = ci / (D / 8), col = (ci % (D / 8)) * 8;
      const int rr = min(kf0 + r, N - 1);
      kst[c] = *(const u32x4*)(Kg + (int64_t)rr * D + col);
      vst[c] = *(const u32x4*)(Vg + (int64_t)rr * D + col);
    }
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
    uint16_t* sk = smem + buf * SM::STAGE;
    uint16_t* sv = sk + SM::KTILE;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ci = tid + NT * c;
      const int r = ci / (D / 8), col = (ci % (D / 8)) * 8;
      const bool in = kf0 + r < kv_end;
      *(u32x4*)(sk + r * SM::KSTR + col) = in ? kst[c] : u32x4{0u, 0u, 0u, 0u};
      *(u32x4*)(sv + r * SM::VSTR + col) = in ? vst[c] : u32x4{0u, 0u, 0u, 0u};
    }
  };

  fetch(0);
  stash(0);
  const int g16 = lane >> 4, s16 = lane & 15;
  int t = 0;
  for (; t < wnt; ++t) {
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);
    const uint16_t* sk = smem + (t & 1) * SM::STAGE;
    const uint16_t* sv = sk + SM::KTILE;
    const int key0 = t * BC;
    // Sᵀ = K Qᵀ and dPᵀ = V dOᵀ: query in the lane, keys in the registers
    f32x16 s[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const u32x4 ka = *(const u32x4*)(sk + (kb * 32 + l32) * SM::KSTR + 16 * kk + 8 * hh);
        const u32x4 va = *(const u32x4*)(sv + (kb * 32 + l32) * SM::VSTR + 16 * kk + 8 * hh);
        s[kb] = mfma32x32x16<DT>(ka, qf[kk], s[kb]);
        dp[kb] = mfma32x32x16<DT>(va, gf[kk], dp[kb]);
      }
    // P in place of S; the mask as a loop of its own under a uniform branch
    // (folded into the exponentials' loop it became selects on every tile)
    const bool masked = key0 + BC > N || (CAUSAL && key0 + BC - 1 > qw0);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(__builtin_fmaf(s[kb][r], a.c, -lq));
    if (masked) {
      // register r of block kb holds key key0 + 32*kb + 8*(r/4) + 4*hh + r%4
      int lim = N - 1 - (key0 + 4 * hh);
      if constexpr (CAUSAL) lim = min(lim, qrow - (key0 + 4 * hh));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = 0.f;
    }
    u32x4 sf[BC / 16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * c2 + 2 * e;
          x[e] = pack2<DT>(s[kb][r] * (dp[kb][r] - dq_row), s[kb][r + 1] * (dp[kb][r + 1] - dq_row));
        }
        sf[2 * kb + c2] = x;
      }
    // dQᵀ += Kᵀ dSᵀ ; k-slot 8*hh + 4*rd + e of chunk ci is key 16*ci + 8*rd + 4*hh + e
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ci = 0; ci < BC / 16; ++ci) {
        const int col = db * 32 + (g16 & 1) * 16 + 4 * (s16 & 3);
        const int ra = 16 * ci + 4 * hh + (s16 >> 2);
        const u32x2 lo = lds_read_tr4(sk + ra * SM::KSTR + col);
        const u32x2 hi = lds_read_tr4(sk + (ra + 8) * SM::KSTR + col);
        dqacc[db] = mfma32x32x16<DT>(u32x4{lo[0], lo[1], hi[0], hi[1]}, sf[ci], dqacc[db]);
      }
    if (t + 1 < ntiles) stash((t + 1) & 1);
  }
  for (; t < ntiles; ++t) {
    __syncthreads();
    if (t + 1 < ntiles) {
      fetch(t + 1);
      stash((t + 1) & 1);
    }
  }

  if (qrow < N) {
    uint16_t* dqr = a.dq + off + (int64_t)qrow * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 x;
        x[0] = pack2<DT>(dqacc[db][4 * g4 + 0] * sc, dqacc[db][4 * g4 + 1] * sc);
        x[1] = pack2<DT>(dqacc[db][4 * g4 + 2] * sc, dqacc[db][4 * g4 + 3] * sc);
        *(u32x2*)(dqr + db * 32 + 8 * g4 + 4 * hh) = x;
      }
  }
}

// two workgroups per CU at d = 96 (228-236 VGPRs; left to itself the
// compiler may take more and halve the occupancy), one at d = 256
template <int D, int DT, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64, (bwd_pass_min_blocks<D>())) void fa_bwd_dq_staged_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * FwdSmem<D, 64>::STAGE];
  dq_staged_body<D, DT, CAUSAL, NW>(a, blockIdx.x, smem);
}

// ---- the d = 96 and 256 sequence in one grid, for small grids ----
// Block 3i is dQ block i, 3i + 1 dV-pass block i, 3i + 2 dK-pass block i
// (128 queries or keys each, 4 waves), after fa_bwd_dot_kernel; LDS the
// largest of the three.
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(256, (bwd_pass_min_blocks<D>())) void fa_bwd_joint_staged_kernel(const BwdArgs a) {
  constexpr int H1 = 2 * FwdSmem<D, 64>::STAGE, H2 = 2 * BwdSmem<D>::STAGE_HALVES;
  __shared__ __attribute__((aligned(16))) uint16_t smem[H1 > H2 ? H1 : H2];
  const int bid = blockIdx.x, i = bid / 3, kind = bid - 3 * i;
  if (kind == 0)
    dq_staged_body<D, DT, CAUSAL, 4>(a, i, smem);
  else if (kind == 1)
    dkdv_pass_body<D, DT, CAUSAL, BWD_DV>(a, i, smem);
  else
    dkdv_pass_body<D, DT, CAUSAL, BWD_DK>(a, i, smem);
}

}  // namespace fa
