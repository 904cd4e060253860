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



// ---- device-scope (cross-work-group) access within one launch.  The L2 of
// each XCD is not coherent with the others: data that another work-group of
// the same launch wrote is read with sc1 loads (fetched from memory, never a
// stale L2 line) and such data is written with sc1 stores (written through).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
__device__ __forceinline__ u32x4 dev_load_b128(const void* base, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(dev_rsrc(base), byte_off, 0, 16));
}
__device__ __forceinline__ float dev_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void dev_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// load that is device-scope when DEV
template <bool DEV>
__device__ __forceinline__ float ld(const float* p) {
  if constexpr (DEV) return dev_load(p);
  else return *p;
}
template <bool DEV>
__device__ __forceinline__ void st(float* p, float v) {
  if constexpr (DEV) dev_store(p, v);
  else *p = v;
}

// ---- sum-of-squares slots for the fused RMSNorm.
// A residual-stream row of width H is covered by H/64 slots of 64 columns;
// slot s of row b is ss[s * 16 + b].  The kernel that writes a row also
// writes its slots; a consumer folds them in a fixed order (deterministic).
constexpr int kSsCols = 64;
constexpr int kSsMaxSlots = 128;   // H <= 8192

// Per-thread share of the fold in two halves, so that the loads can be
// issued early and the adds done later: thread t of a 256-thread block covers
// row t % 16 and slots t/16, t/16 + 16, ...
template <bool DEV = false>
__device__ __forceinline__ void ss_thread_load(const float* __restrict__ ss, int n_slots,
                                               float (&v)[kSsMaxSlots / 16]) {
  const int b = threadIdx.x & 15, s0 = threadIdx.x >> 4;
#pragma unroll
  for (int j = 0; j < kSsMaxSlots / 16; ++j) {
    const int s = s0 + 16 * j;
    v[j] = ld<DEV>(ss + (s < n_slots ? s : n_slots - 1) * 16 + b);
  }
}
__device__ __forceinline__ float ss_thread_sum(const float (&v)[kSsMaxSlots / 16], int n_slots) {
  const int s0 = threadIdx.x >> 4;
  float p = 0.f;
#pragma unroll
  for (int j = 0; j < kSsMaxSlots / 16; ++j) p += (s0 + 16 * j < n_slots) ? v[j] : 0.f;
  return p;
}

// Second half of the fold: combine the 16 thread parts of each row within a
// wave, then write one value per (wave, row) to red[4][16].  The caller
// synchronizes the block before rms_inv().
__device__ __forceinline__ void ss_wave_fold(float p, float (*red)[16]) {
  p += __shfl_xor(p, 16);
  p += __shfl_xor(p, 32);
  const int lane = threadIdx.x & 63;
  if (lane < 16) red[threadIdx.x >> 6][lane] = p;
}

__device__ __forceinline__ float rms_inv(const float (*red)[16], int b, float inv_h, float eps) {
  const float tot = (red[0][b] + red[1][b]) + (red[2][b] + red[3][b]);
  return 1.0f / sqrtf(tot * inv_h + eps);
}

// h = f16(x * rinv * gamma), the one RMSNorm rounding used everywhere
__device__ __forceinline__ half_t norm_apply(float x, float rinv, float gamma) { return (half_t)((x * rinv) * gamma); }

__device__ __forceinline__ double f16_bits_to_f64(uint16_t b) {
  return (double)__builtin_bit_cast(half_t, b);
}

}  // namespace qk
