// FlashAttention-2-style exact attention forward for gfx950.
//
// What it computes: O = softmax(scale * Q Kᵀ) V and LSE per row, with the
// optional causal mask ("FlashAttention explainer" (aitangshan.cn) sections
// 1 and 7.1). How: one workgroup owns a block of BR query rows (the outer
// loop over Q blocks of section 5.2); it streams K/V tiles of BC rows
// through LDS (tiling, section 4.2) and keeps the running row max m and sum l
// of the online softmax in registers, rescaling the partial output whenever
// the max moves (section 4.3; "YOLO11 attention swapped for a
// FlashAttention-2-style implementation" (discosf.com) section 2.2). Only O
// and LSE are written, once ("FlashAttention explainer" section 5.2).
//
// MI355X mapping (our design, not the pages'):
//  * Each wave owns QW = 32*QB query rows and computes the TRANSPOSED score
//    tile Sᵀ = K Qᵀ with v_mfma_f32_32x32x16: the query index then sits in
//    the lane (lane % 32) and the keys in the accumulator registers, so the
//    row max / row sum are in-register reductions plus one exchange with
//    lane ^ 32, and the same layout feeds Oᵀ = Vᵀ Pᵀ as its B operand with
//    no data movement. Oᵀ keeps the query in the lane too, so the rescale by
//    exp2(m_old - m_new) is a per-lane scalar.
//  * Vᵀ (the A operand of Oᵀ += Vᵀ Pᵀ) is read from the row-major V tile
//    with ds_read_b64_tr_b16, the gfx950 LDS transpose read.
//  * Softmax runs in the log2 domain: c = |scale|*log2(e), p = exp2(s*c - m).
//    A negative scale is folded into Q by flipping its sign bits (exact).
//  * The reference m of a row is its first tile's max (raised by 16 log2
//    units for bf16, see ref_margin). Later tiles skip the max entirely:
//    their weights p = exp2(s*c - m) are formed with the standing m and
//    only their partial sums are checked; a tile whose
//    partial sums reach partial_cap (so some weight could leave the 16-bit
//    range) is redone with the true max and a rescale of the output
//    accumulator. In the bf16 kernel for small grids the sum of the 16-bit
//    weights comes from the MFMA units (an all-ones block of V). O = acc / l and LSE = (m + log2 l) ln 2 are exact for any
//    reference m, so only the range of p matters, not which m is used.
//  * K/V for tile t+1 are fetched into registers (buffer loads whose
//    descriptor covers only the tile's valid rows: rows past the end read
//    as zero with no per-lane test) while tile t is computed from the other
//    half of a double-buffered LDS, one barrier per tile.
//  * Workgroup ids are remapped so that each XCD (workgroups are dealt
//    round-robin over the 8 XCDs) walks whole heads, sharing K/V in its L2
//    (packed batches of unequal sequences keep the plain order); causal
//    blocks run by rank across all heads, longest first.
//  * A head's 32-row units are spread evenly over its blocks, one unit per
//    wave; waves without a unit only help with the K/V loads.
#pragma once
#include <type_traits>

#include "fa_device.h"

namespace fa {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t q_sb, q_sh, q_sr;  // element strides (batch, head, row)
  int64_t k_sb, k_sh, k_sr;
  int64_t v_sb, v_sh, v_sr;
  int64_t o_sb, o_sh, o_sr;
  int64_t lse_sb, lse_sh;    // lse index = b*lse_sb + h*lse_sh + (row offset) + i
  const int32_t* cu_seqlens; // null: every sequence has N rows
  int B, H, N;               // N: rows per sequence (an upper bound with cu_seqlens)
  int nqb;                   // query blocks per (batch, head)
  int units;                 // 32-row units of a sequence of N rows, ceil(N / 32); block q
                             // owns units [q*units/nqb, (q+1)*units/nqb), at most one per wave
  int total;                 // B * H * nqb
  float c;                   // max(|scale| * log2(e), 1e-30): strictly positive
  uint32_t qsign;            // 0x80008000 when scale < 0, else 0
};

// A weight tile is accepted when each lane's partial sums of its 16-bit
// weights (at most 8 weights each) stay below this cap. fp16: every weight is
// then below 2^15, inside the fp16 range. bf16 weights keep their relative
// precision at any magnitude, so their cap is 2^32: a row's sum then grows by
// less than 2^35 per 64-key tile and stays below 2^60 even for 2^31 keys, and
// the unnormalised output stays finite for |v| < 2^67. A redo then needs a
// score 32 (log2) units above the row's reference, which large-logit inputs
// rarely reach.
template <int DT>
constexpr float partial_cap() {
  return DT == DT_BF16 ? 4294967296.0f : 32768.0f;
}

// A row's reference max is its first tile's max raised by this many log2
// units. bf16 weights keep their relative precision far below 1 (8 exponent
// bits), so the first tile's weights may start at 2^-16 and later tiles need
// a score 16 + 32 units above the first tile's max before the range check
// redoes a tile; large-logit rows then almost never redo. fp16 weights would
// lose precision below 2^-14, so they keep the first tile's max.
template <int DT>
constexpr float ref_margin() {
  return DT == DT_BF16 ? 16.0f : 0.0f;
}

// dword 3 of a raw buffer descriptor on gfx950 (32-bit data format, raw
// addressing; loads past num_records return zero)
constexpr int kBufferDword3 = 0x00020000;

// Padded V row (halves) of the 32-row tile step. Its transposing reads are
// served 32 lanes at a time over 64 banks of 4 bytes: 4 consecutive rows at
// 8-byte steps across 64 bytes of columns, so each row covers 16 banks, and
// the 4 rows are conflict-free when the row stride is 16 or 48 banks (mod 64),
// i.e. VSTR = 32 or 96 halves (mod 128). d=64 and 96: 96; d=128 and 256: D+32.
template <int D>
constexpr int fwd_vstr() {
  return D <= 96 ? 96 : D + 32;
}
static_assert(fwd_vstr<64>() % 128 == 96 && fwd_vstr<96>() % 128 == 96 && fwd_vstr<128>() % 128 == 32 &&
                  fwd_vstr<256>() % 128 == 32,
              "V rows at 16 or 48 banks");

template <int D, int BC, int VS = fwd_vstr<D>()>
struct FwdSmem {
  static constexpr int KSTR = D + 8;  // padded K row (halves): conflict-free 16-byte reads
  static constexpr int VSTR = VS;     // padded V row (halves)
  static constexpr int KTILE = BC * KSTR;
  static constexpr int VTILE = BC * VSTR;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int BYTES = 2 * STAGE * 2;
};

// XOR swizzle of the 16-byte chunk slot of row r in an unpadded LDS tile
// (rows of D halves). LDS has 64 banks; a 16-byte read is served 16 lanes at
// a time and an 8-byte transposing read 32 lanes at a time, so the slot must
// (a) differ over 16 consecutive rows read at the same chunk (the K operand)
// and (b) spread 4 aligned rows x 4 aligned chunks over 16 distinct bank
// groups (the V operand). With 256-byte rows (d=128) the bank group is the
// slot itself; with 128-byte rows (d=64) it is the slot plus 8 for odd rows.
template <int D>
__device__ __forceinline__ int lds_swz(int r) {
  static_assert(D == 64 || D == 128, "swizzled tiles are laid out for d = 64 and 128");
  if constexpr (D == 128)
    return 4 * (r & 3) + ((r >> 2) & 3);
  else
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Offset (halves) of (row, col) in an LDS K or V tile: rows padded to STR
// halves, or, with STR = 0, unpadded rows of D halves whose 16-byte chunks
// are XOR-swizzled (the layout that whole-row LDS-DMA writes can produce).
template <int D, int STR>
__device__ __forceinline__ int lds_off(int row, int col) {
  if constexpr (STR == 0)
    return row * D + (((col >> 3) ^ lds_swz<D>(row)) << 3) + (col & 7);
  else
    return row * STR + col;
}

// One K/V tile for one wave: Sᵀ = K Qᵀ, online-softmax update, Oᵀ += Vᵀ Pᵀ.
// Masked tiles (wave-uniform flag) apply the ragged-tail and causal masks;
// `first` (wave-uniform) marks the first tile of the wave's rows.
// LS (bf16 only): the sum of the 16-bit weights is accumulated by MFMA as an
// extra all-ones block of V, oacc[j][D/32] (every register of it holds the
// row's full sum), instead of by dot2 instructions; the range check then uses
// the fp32 sums. It trades 20 VALU instructions a tile for 4 MFMAs, which
// pays only where the MFMA units have slack.
template <int D, int DT, bool CAUSAL, int QB, int BC, int KSTR, int VSTR, int PF, bool LS = false>
__device__ __forceinline__ void tile_step_fwd(bool first, bool masked, const uint16_t* __restrict__ sk,
                                               const uint16_t* __restrict__ sv, int key0, int Nb,
                                               int qw0, int lane, float c, const u32x4 (&qf)[QB][D / 16],
                                               f32x16 (&oacc)[QB][D / 32 + LS], float (&m_run)[QB],
                                               float (&l_run)[2][QB]) {
  static_assert(!LS || DT == DT_BF16, "MFMA weight sums rely on the fp32 sums of the bf16 path");
  constexpr int KK = D / 16, DB = D / 32, KB = BC / 32;
  const int l32 = lane & 31, hh = lane >> 5;

  // Sᵀ = K_t Qᵀ : s[kb][j] covers keys kb*32.. and queries 32j.. (a redone
  // tile computes it again from LDS rather than keeping it live)
  f32x16 s[KB][QB];
  auto scores = [&](int z) __attribute__((always_inline)) {
    const uint16_t* kt = sk + z;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < QB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][j][r] = 0.f;
    if constexpr (PF > 0) {
      // K fragments read PF k-steps ahead of the MFMAs that use them, with a
      // scheduling fence per k-step so that the reads stay ahead (left to
      // itself the compiler keeps about one step in flight and each MFMA pair
      // waits out an LDS round trip)
      u32x4 kfp[PF][KB];
#pragma unroll
      for (int i = 0; i < PF; ++i)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          kfp[i][kb] = *(const u32x4*)(kt + lds_off<D, KSTR>(kb * 32 + l32, 16 * i + 8 * hh));
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int j = 0; j < QB; ++j) s[kb][j] = mfma32x32x16<DT>(kfp[kk % PF][kb], qf[j][kk], s[kb][j]);
        if (kk + PF < KK) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
            kfp[kk % PF][kb] = *(const u32x4*)(kt + lds_off<D, KSTR>(kb * 32 + l32, 16 * (kk + PF) + 8 * hh));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x4 ka = *(const u32x4*)(kt + lds_off<D, KSTR>(kb * 32 + l32, 16 * kk + 8 * hh));
#pragma unroll
          for (int j = 0; j < QB; ++j) s[kb][j] = mfma32x32x16<DT>(ka, qf[j][kk], s[kb][j]);
        }
      }
    }
    if (masked) {
      // register r of block kb holds key key0 + 4*hh + off, off = 32*kb +
      // 8*(r/4) + r%4; it is dead when past the end (key >= Nb) or, causal,
      // after the query (key > qrow): off > lim with one per-lane limit
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const int base = key0 + 4 * hh - z;
        int lim = Nb - 1 - base;
        if constexpr (CAUSAL) lim = min(lim, qw0 + 32 * j + l32 - base);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][j][r] = -INFINITY;
      }
    }
  };
  scores(0);

  // online softmax (log2 domain)
  u32x4 pf[QB][BC / 16];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    // weights p = exp2(s*c - mref) packed to 16 bits; lp: 4 partial sums of
    // the 16-bit weights (the ones that multiply V, so O is normalised by
    // exactly what it accumulates); lf: fp32 sums for the bf16 LSE
    float lp[4], lf[4];
    auto probs = [&](float mref) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) lp[e] = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // c > 0 always (clamped on the host), so a masked -inf stays -inf
          p[r] = fast_exp2(__builtin_fmaf(s[kb][j][r], c, -mref));
          if constexpr (DT == DT_BF16) {
            if (kb == 0 && r < 4) lf[r] = p[r];
            else lf[r & 3] += p[r];
          }
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          u32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = pack2<DT>(p[8 * c2 + 2 * e], p[8 * c2 + 2 * e + 1]);
            if constexpr (!LS) lp[e] = dot2_sum<DT>(x[e], lp[e]);
          }
          pf[j][2 * kb + c2] = x;
        }
      }
    };
    auto tile_max = [&]() __attribute__((always_inline)) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][j][r]);
      return fmaxf(mx, xor_lane32(mx)) * c;
    };
    // the first tile of a row sets its reference max (the accumulator is
    // still zero, so nothing needs rescaling)
    if (first) m_run[j] = tile_max() + ref_margin<DT>();
    probs(m_run[j] == -INFINITY ? 0.f : m_run[j]);
    const float pk = LS ? fmaxf(fmaxf(lf[0], lf[1]), fmaxf(lf[2], lf[3]))
                        : fmaxf(fmaxf(lp[0], lp[1]), fmaxf(lp[2], lp[3]));
    if (wave_any(!(pk < partial_cap<DT>()))) {
      // some weight may have left the 16-bit range: raise the reference to
      // the true max, rescale what has been accumulated, redo the weights
      // (through an offset the compiler cannot see is zero, so that K and
      // the mask are formed again rather than kept live across the fast path)
      int zero = 0;
      asm volatile("" : "+s"(zero));
      scores(zero);
      const float m_new = fmaxf(m_run[j], tile_max());
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[j] - m_new);
      l_run[0][j] *= alpha;
      l_run[1][j] *= alpha;
#pragma unroll
      for (int db = 0; db < DB + LS; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[j][db][r] *= alpha;
      m_run[j] = m_new;
      probs(m_new == -INFINITY ? 0.f : m_new);
    }
    if constexpr (!LS) l_run[0][j] += (lp[0] + lp[1]) + (lp[2] + lp[3]);
    if constexpr (DT == DT_BF16) l_run[1][j] += (lf[0] + lf[1]) + (lf[2] + lf[3]);
  }

  // Oᵀ += Vᵀ Pᵀ ; k-slot 8*hh + 4*rd + e of chunk ci is key 16*ci + 8*rd + 4*hh + e
  const int g = lane >> 4, s16 = lane & 15;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int ci = 0; ci < BC / 16; ++ci) {
      const int col = db * 32 + (g & 1) * 16 + 4 * (s16 & 3);
      const int rowa = 16 * ci + 4 * hh + (s16 >> 2);
      const u32x2 lo = lds_read_tr4(sv + lds_off<D, VSTR>(rowa, col));
      const u32x2 hi = lds_read_tr4(sv + lds_off<D, VSTR>(rowa + 8, col));
      const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int j = 0; j < QB; ++j) oacc[j][db] = mfma32x32x16<DT>(va, pf[j][ci], oacc[j][db]);
    }
  }
  if constexpr (LS) {
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
#pragma unroll
    for (int ci = 0; ci < BC / 16; ++ci)
#pragma unroll
      for (int j = 0; j < QB; ++j) oacc[j][DB] = mfma32x32x16<DT>(ones, pf[j][ci], oacc[j][DB]);
  }
}

// Waves per SIMD the compiler is to fit (the second launch bound). The
// 4-wave d=96 kernel left to itself takes 276-280 VGPRs (one wave per SIMD);
// held to two it fits 184-191 without spills (B4 H16 N4096 fp16: 454 vs
// 459 us); three spill.
template <int D, int NW>
constexpr int fwd_min_waves() {
  return D == 96 && NW == 4 ? 2 : 1;
}

// Whether the main tile loop runs in pairs of tiles, so that the LDS stage
// is a constant in each copy of the tile step. Two kernels keep the
// single-tile loop, because in pairs they lose occupancy or spill: the 4-wave
// d=128 kernels (fp16 causal: more than 256 VGPRs) and the 8-wave d=64 fp16
// causal kernel (131 VGPRs, 3 waves per SIMD instead of 4; held to 128 it
// spills).
template <int D, int DT, bool CAUSAL, int NW>
constexpr bool fwd_pair_loop() {
  return !(D == 128 && NW == 4) && !(D == 64 && DT == DT_F16 && CAUSAL && NW == 8);
}

template <int D, int DT, bool CAUSAL, int NW, int QB, int BC, int PF, bool LS = false>
__global__ __launch_bounds__(NW * 64, (fwd_min_waves<D, NW>())) void fa_fwd_kernel(const FwdArgs a) {
  static_assert(QB == 1, "one 32-row unit per wave");
  constexpr int NT = NW * 64;
  constexpr int QW = 32 * QB;          // query rows per wave
  constexpr int BR = NW * QW;          // query rows per workgroup
  constexpr int KK = D / 16;           // k-steps of Sᵀ = K Qᵀ
  constexpr int DB = D / 32;           // 32-row blocks of Oᵀ
  constexpr int KB = BC / 32;          // 32-key blocks of Sᵀ per tile
  constexpr int CH = BC * D / 8 / NT;  // 16-byte chunks per thread per tensor per tile
  static_assert(BC * D / 8 % NT == 0, "tile must split evenly over threads");
  using SM = FwdSmem<D, BC>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SM::STAGE];

  // ---- workgroup -> (batch, head, query block), XCD-aware ----
  // Workgroups are dealt round-robin over the 8 XCDs and dispatched in
  // order. Equal-length sequences:
  //  * non-causal: each XCD takes a contiguous run of whole heads, whose
  //    blocks then share K/V in that XCD's L2;
  //  * causal: block rank major, head minor, so that the longest blocks of
  //    every head start first (a head-major order leaves long blocks of the
  //    last heads for the end), and with B*H a multiple of 8 every block of
  //    a head still lands on one XCD. With long rows (32 or more blocks a
  //    head) and B*H a multiple of 16, each XCD takes its heads in pairs,
  //    rank major within a pair: as fast, with two heads' K/V in flight per
  //    XCD instead of all of them (N=8192 x32 heads: 0.63x the fetched bytes).
  // Packed sequences of different lengths keep the plain order: a contiguous
  // run would hand the long sequences to a few XCDs, while the plain order
  // spreads every sequence's blocks over all eight (re-reads of K/V across
  // XCDs hit the shared Infinity Cache).
  const int bid = blockIdx.x;
  int bh, qi;
  if (CAUSAL && !a.cu_seqlens) {
    const int nbh = a.B * a.H;
    if ((nbh & 15) == 0 && a.nqb >= 32) {
      const int x = bid & 7, j = bid >> 3;  // XCD, position in its order
      const int grp = j / (2 * a.nqb), r = j - grp * 2 * a.nqb;
      qi = r >> 1;
      bh = x + 8 * (2 * grp + (r & 1));
      if (bh >= nbh) return;
    } else {
      qi = bid / nbh;
      bh = bid - qi * nbh;
      if (qi >= a.nqb) return;
    }
  } else {
    const int per = gridDim.x >> 3;
    const int lid = a.cu_seqlens ? bid : (bid & 7) * per + (bid >> 3);
    if (lid >= a.total) return;
    bh = lid / a.nqb;
    qi = lid - bh * a.nqb;
  }
  const int qblk = CAUSAL ? (a.nqb - 1 - qi) : qi;
  const int b = bh / a.H, h = bh - b * a.H;

  int64_t row0 = 0;
  int Nb = a.N;
  if (a.cu_seqlens) {
    row0 = a.cu_seqlens[b];
    Nb = a.cu_seqlens[b + 1] - (int)row0;
  }
  // this block's rows: units spread evenly over the blocks of a head
  const int u0 = (int)((int64_t)qblk * a.units / a.nqb);
  const int u1 = (int)((int64_t)(qblk + 1) * a.units / a.nqb);
  if (32 * u0 >= Nb) return;  // uniform over the workgroup

  const uint16_t* Qg = a.q + b * a.q_sb + h * a.q_sh + row0 * a.q_sr;
  const uint16_t* Kg = a.k + b * a.k_sb + h * a.k_sh + row0 * a.k_sr;
  const uint16_t* Vg = a.v + b * a.v_sb + h * a.v_sh + row0 * a.v_sr;
  uint16_t* Og = a.o + b * a.o_sb + h * a.o_sh + row0 * a.o_sr;
  float* Lg = a.lse + b * a.lse_sb + h * a.lse_sh + row0;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qw0 = 32 * u0 + w * QW;         // first query row of this wave
  const bool wave_rows = w < u1 - u0;       // waves past the block only help with the loads

  // ---- Q fragments (B operand of Sᵀ = K Qᵀ), kept in registers; rows past
  // the end load row Nb-1 (in bounds) and are zeroed once the first K/V
  // tile's loads are in flight too ----
  u32x4 qf[QB][KK];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int r = qw0 + 32 * j + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[j][kk] = *(const u32x4*)(Qg + min(r, Nb - 1) * a.q_sr + 16 * kk + 8 * hh);
  }

  const int kv_end = CAUSAL ? min(Nb, 32 * u1) : Nb;
  const int ntiles = (kv_end + BC - 1) / BC;

  // ---- global -> register staging of one K/V tile ----
  // Per tile, a buffer descriptor based at the tile's first row whose size
  // ends with the last valid row (host guarantee: BC row strides < 2^31
  // bytes); each lane's byte offset inside the tile is fixed.
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

  // ---- running state ----
  f32x16 oacc[QB][DB + LS];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int db = 0; db < DB + LS; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[j][db][r] = 0.f;
  float m_run[QB], l_run[2][QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) { m_run[j] = -INFINITY; l_run[0][j] = 0.f; l_run[1][j] = 0.f; }

  fetch(0);
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const bool in = qw0 + 32 * j + l32 < Nb;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[j][kk] = (in ? qf[j][kk] : u32x4{0u, 0u, 0u, 0u}) ^ a.qsign;
  }
  stash(0);


  // The tiles a wave computes end with the last key any of its rows sees
  // (causal: its own diagonal; tiles past that are fully masked and are
  // skipped). A ragged last tile that fits in 32 keys -- the ragged end of
  // a sequence, or a causal diagonal block of a wave whose rows start on a
  // 64-key boundary -- runs as a half-width step. After its last tile a wave
  // keeps helping with the loads until the workgroup's last tile (same
  // barriers), and waves with no rows only help with the loads. Keeping each
  // loop body a single path lets the output accumulator stay in place.
  if (wave_rows && qw0 < Nb) {
    const int wave_end = CAUSAL ? min(kv_end, qw0 + QW) : kv_end;
    const int wnt = (wave_end + BC - 1) / BC;
    const bool tail32 = BC == 64 && wave_end - (wnt - 1) * BC <= 32;
    const int nmain = tail32 ? wnt - 1 : wnt;
    // tile t computes from LDS stage P = t % 2; taken in pairs from t = 0,
    // P is a constant in each copy of the step and the stage's LDS addresses
    // are immediate offsets from fixed bases
    auto main_step = [&](int t, auto stage) __attribute__((always_inline)) {
      const int P = stage;
      __syncthreads();
      if (t + 1 < ntiles) fetch(t + 1);
      const int key0 = t * BC;
      const uint16_t* sk = smem + P * SM::STAGE;
      const uint16_t* sv = sk + SM::KTILE;
      // ragged last tile, or (causal) keys after some query of this wave
      const bool need_mask = (key0 + BC > Nb) || (CAUSAL && key0 + BC - 1 > qw0);
      tile_step_fwd<D, DT, CAUSAL, QB, BC, SM::KSTR, SM::VSTR, PF, LS>(P == 0 && t == 0, need_mask, sk, sv, key0, Nb,
                                                               qw0, lane, a.c, qf, oacc, m_run, l_run);
      if (t + 1 < ntiles) stash(P ^ 1);
    };
    int t = 0;
    if constexpr (fwd_pair_loop<D, DT, CAUSAL, NW>()) {
      for (; t + 1 < nmain; t += 2) {
        main_step(t, std::integral_constant<int, 0>{});
        main_step(t + 1, std::integral_constant<int, 1>{});
      }
      if (t < nmain) {
        main_step(t, std::integral_constant<int, 0>{});
        ++t;
      }
    } else {
      for (; t < nmain; ++t) main_step(t, t & 1);
    }
    if constexpr (BC == 64) {
      if (tail32) {
        __syncthreads();
        if (t + 1 < ntiles) fetch(t + 1);
        const uint16_t* sk = smem + (t & 1) * SM::STAGE;
        tile_step_fwd<D, DT, CAUSAL, QB, 32, SM::KSTR, SM::VSTR, PF, LS>(t == 0, true, sk, sk + SM::KTILE, t * BC,
                                                                 Nb, qw0, lane, a.c, qf, oacc, m_run, l_run);
        if (t + 1 < ntiles) stash((t + 1) & 1);
        ++t;
      }
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

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
  // Each wave turns its Oᵀ tile (query in the lane) into row-major rows in
  // LDS and writes whole 16-byte row chunks from there: 64 lanes then cover
  // 1 KB of consecutive rows per store instead of 16 bytes of 32 rows.
  constexpr int OSTR = D + 8;  // padded output row in LDS (halves)
  static_assert(NW * QW * OSTR <= 2 * SM::STAGE, "output staging must fit in the K/V staging area");
  __syncthreads();  // every wave is done with the K/V tiles
  if (!(wave_rows && qw0 < Nb)) return;
  uint16_t* ob = smem + w * QW * OSTR;
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float l_tot = LS ? oacc[j][DB][0] : l_run[0][j] + xor_lane32(l_run[0][j]);
    const float l_lse = DT == DT_F16 ? l_tot : l_run[1][j] + xor_lane32(l_run[1][j]);
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 x;
        x[0] = pack2<DT>(oacc[j][db][4 * g4 + 0] * inv, oacc[j][db][4 * g4 + 1] * inv);
        x[1] = pack2<DT>(oacc[j][db][4 * g4 + 2] * inv, oacc[j][db][4 * g4 + 3] * inv);
        *(u32x2*)(ob + (32 * j + l32) * OSTR + db * 32 + 8 * g4 + 4 * hh) = x;
      }
    const int qrow = qw0 + 32 * j + l32;
    if (hh == 0 && qrow < Nb) Lg[qrow] = (m_run[j] + fast_log2(l_lse)) * kLn2;
  }
  wave_lds_sync();  // the rows below were written by other lanes of this wave
  constexpr int CPR = D / 8;  // 16-byte chunks per output row
#pragma unroll
  for (int i = 0; i < QW * CPR / 64; ++i) {
    const int p = lane + 64 * i, r = p / CPR, ch = p % CPR;
    const u32x4 x = *(const u32x4*)(ob + r * OSTR + ch * 8);
    if (qw0 + r < Nb) *(u32x4*)(Og + (qw0 + r) * a.o_sr + ch * 8) = x;
  }
}

}  // namespace fa
