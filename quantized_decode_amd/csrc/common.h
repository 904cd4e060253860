// Device-side helpers shared by the libqkdec kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qkdec.h"

namespace qk {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(half_t, (uint16_t)bits16);
}
__device__ __forceinline__ uint16_t f2h_bits(float x) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (half_t)x);
}
__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ __forceinline__ uint32_t h2_bits(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ half2_t pack_h2(float lo, float hi) {
  // exact for the small integers and power-of-two fractions used here
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// 2^k as a float, k clamped to the normal range
// storage format of one cache tensor (keys or values)
enum : int { kFmtF16 = 0, kFmtQ8 = 1, kFmtF8 = 2 };

__device__ __forceinline__ float exp2i(int k) {
  k = k < -126 ? -126 : (k > 127 ? 127 : k);
  return __builtin_bit_cast(float, (uint32_t)(k + 127) << 23);
}

__device__ __forceinline__ floatx4 mfma16x16x32(const half8_t& a, const half8_t& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Round a double to the nearest-even fp16 bit pattern (one rounding, with
// subnormals and overflow to infinity).
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
  uint64_t u = __builtin_bit_cast(uint64_t, x);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  uint64_t a = u & 0x7fffffffffffffffull;
  if (a >= 0x7ff0000000000000ull) {                         // inf or nan
    return sign | (a > 0x7ff0000000000000ull ? 0x7e00 : 0x7c00);
  }
  int e = (int)(a >> 52) - 1023;                             // unbiased exponent
  uint64_t mant = (a & 0xfffffffffffffull) | (1ull << 52);   // 53-bit significand
  if (e > 15) return sign | 0x7c00;
  if (a == 0) return sign;
  // fp16 value = m * 2^(qexp) with m integer; normal: e >= -14 -> 11-bit m, qexp = e-10
  int qexp = (e >= -14) ? (e - 10) : -24;
  int shift = 52 - e + qexp;        // bits of mant to drop: mant*2^(e-52) = m * 2^qexp
  uint64_t m;
  if (shift >= 64) {
    m = 0;
    // value < 2^-25 * ...: rounds to zero unless exactly above half of 2^-24
    // (cannot be, since shift >= 64 means value < 2^(qexp-11))
    return sign;
  }
  m = mant >> shift;
  uint64_t rem = mant & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (m & 1))) ++m;
  // m may now be 2048 (normal overflow into next exponent) or 1024 (subnormal -> normal)
  uint32_t bits;
  if (qexp == -24) {
    bits = (uint32_t)m;              // subnormal (or 0x400 = smallest normal)
  } else {
    int ee = e;
    if (m == 2048) { m = 1024; ++ee; }
    if (ee > 15) return sign | 0x7c00;
    bits = ((uint32_t)(ee + 15) << 10) | (uint32_t)(m & 0x3ff);
  }
  return sign | (uint16_t)bits;
}



// ---- sum-of-squares slots for the fused RMSNorm.
// A residual-stream row of width H is covered by H/16 slots of 16 columns
// (one matrix-core tile of outputs, so one wave finishes a slot); slot s of
// row b is ss[s * 16 + b].  The kernel that writes a row also writes its
// slots; a consumer folds them in a fixed order (deterministic).
constexpr int kSsCols = 16;
constexpr int kSsMaxSlots = 512;   // H <= 8192

// Fold of the slots by all NT threads of a work-group, in two halves so that
// the loads can be issued early and the adds done later.  Thread t loads the
// float4 of rows 4q..4q+3 (q = t % 4) of slots t/4, t/4 + NT/4, ... (at most
// SMAX slots: the register array is sized for it); load() then fold() leaves
// one partial per (wave, row) in red[NT/64][16]; after a barrier rms_inv()
// adds the waves' partials in order (deterministic).
template <int NT, int SMAX>
struct SsFold {
  static constexpr int G = NT / 4;
  static constexpr int J = SMAX > 0 ? (SMAX + G - 1) / G : 1;   // SMAX = 0: a caller that never folds
  floatx4 v[J];
  __device__ __forceinline__ void load(const float* __restrict__ ss, int n_slots) {
    const int q = threadIdx.x & 3, s0 = threadIdx.x >> 2;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      // unconditional load of an in-range slot, then a select: no branch
      // around a load (a branch would make later load waits conservative)
      const int s = s0 + G * j;
      const floatx4 w = *reinterpret_cast<const floatx4*>(ss + (size_t)(s < n_slots ? s : 0) * 16 + 4 * q);
      v[j] = s < n_slots ? w : floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __device__ __forceinline__ void fold(float (*red)[16]) const {
    floatx4 p = v[0];
#pragma unroll
    for (int j = 1; j < J; ++j) p += v[j];
    // lanes with the same q (lane % 4) hold the same rows
#pragma unroll
    for (int o = 4; o < 64; o <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] += __shfl_xor(p[i], o);
    const int lane = threadIdx.x & 63;
    if (lane < 4)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[threadIdx.x >> 6][4 * lane + i] = p[i];
  }
};

template <int NW>
__device__ __forceinline__ float rms_inv(const float (*red)[16], int b, float inv_h, float eps) {
  float tot = red[0][b];
#pragma unroll
  for (int w = 1; w < NW; ++w) tot += red[w][b];
  return 1.0f / sqrtf(tot * inv_h + eps);
}

// h = f16(x * rinv * gamma), the one RMSNorm rounding used everywhere
__device__ __forceinline__ half_t norm_apply(float x, float rinv, float gamma) { return (half_t)((x * rinv) * gamma); }

__device__ __forceinline__ double f16_bits_to_f64(uint16_t b) {
  return (double)__builtin_bit_cast(half_t, b);
}

}  // namespace qk
