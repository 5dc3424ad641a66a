// Device-side building blocks for the gfx950 attention kernels: vector
// types, the 16-bit MFMA wrappers, LDS transpose reads and fp32 -> 16-bit
// packing. gfx950 (CDNA4) only; wave64.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 b16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16) * B(16x32); each lane holds 8 16-bit values of A
// (row lane%32, k = 8*(lane/32)..+7) and of B (column lane%32, same k), and
// 16 fp32 of D (row 8*(r/4) + 4*(lane/32) + r%4, column lane%32).
template <int DT>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h16x8, a),
                                                  __builtin_bit_cast(h16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b16x8, a),
                                                   __builtin_bit_cast(b16x8, b), c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32) * B(32x16); each lane holds 8 16-bit values of A
// (row lane%16, k = 8*(lane/16)..+7) and of B (column lane%16, same k), and
// 4 fp32 of D (row 4*(lane/16) + r, column lane%16).
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8, a),
                                                  __builtin_bit_cast(h16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b16x8, a),
                                                   __builtin_bit_cast(b16x8, b), c, 0, 0, 0);
}

// Two fp32 -> one dword of two 16-bit values (round to nearest even); `lo`
// lands in the low half.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == DT_F16) {
    h16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    b16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// acc + lo + hi of a packed pair of 16-bit values, with fp32 accumulation
// (v_dot2_f32_f16 / v_dot2_f32_bf16 against (1, 1))
template <int DT>
__device__ __forceinline__ float dot2_sum(uint32_t packed, float acc) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h16x2, packed), h16x2{(_Float16)1.f, (_Float16)1.f},
                                  acc, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b16x2, packed),
                                           b16x2{(__bf16)1.f, (__bf16)1.f}, acc, false);
}

template <int DT>
__device__ __forceinline__ float to_f32(uint16_t x) {
  if constexpr (DT == DT_F16)
    return (float)__builtin_bit_cast(_Float16, x);
  else
    return __builtin_bit_cast(float, (uint32_t)x << 16);
}

// LDS transpose read of 4 x 16-bit per lane (ds_read_b64_tr_b16). Inside each
// group of 16 lanes, lane i receives element (i % 4) of the 8-byte words
// addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12 of its group, in that
// order. Pointing lane s at row r0 + s/4, column c0 + 4*(s%4) of a row-major
// 16-bit matrix therefore hands lane i the column c0 + i of rows r0..r0+3.
// The __restrict__ gives the read alias-scope information. Without it the
// compiler cannot tell that the read does not touch LDS being filled by an
// LDS-DMA load in flight, and makes it wait for every such load. The kernels
// order DMA-filled tiles and their reads with their own waits and barriers.
__device__ __forceinline__ u32x2 lds_read_tr4(const uint16_t* __restrict__ p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float xor_lane32(float x) {
  return __shfl_xor(x, 32, 64);
}

// Orders this wave's LDS writes before its later LDS reads of what other
// lanes wrote (wave-scope release/acquire; the LDS executes one wave's
// operations in order, so no wait instruction is needed, only that the
// compiler keeps the order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

}  // namespace fa
