// Device code of the KV-cache store shared by the append kernels and the QKV
// projection's finishing step: fp16 rounding, the Q8_0 quantizer of one
// 32-value block or the E4M3 rounding (the arithmetic is described at the top
// of kv_append.hip).
#pragma once

#include "common.h"

namespace qk {

// max over aligned groups of 32 lanes
__device__ __forceinline__ double amax32(double v) {
  for (int o = 16; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 32));
  return v;
}

__device__ __forceinline__ int8_t q8_code(double x, double d) {
  if (d == 0.0) return 0;
  const double y = x / d;
  const double t = trunc(y);
  double r = t;
  if (fabs(y - t) >= 0.5) r += (y > 0.0) ? 1.0 : -1.0;
  if (r > 127.0) r = 127.0;
  if (r < -127.0) r = -127.0;
  return (int8_t)r;
}

struct CacheRef {
  uint8_t* k;
  uint8_t* v;
  uint16_t* ks;
  uint16_t* vs;
  int n_kv, cap, D, n_slots;
  int kf, vf;   // key / value format (kFmtF16, kFmtQ8, kFmtF8)
};

// Element stores of dim d of (slot s, kv head g, position p), into K
// (is_v = false) or into V, which is transposed within 32-token blocks
// ([cap/32][D][32] per head): fp16 bits, or a Q8_0 code with its block scale
// (written by the block's dim 0).
__device__ __forceinline__ size_t v_index(const CacheRef& c, size_t head, int p, int d) {
  return ((head * (c.cap >> 5) + (p >> 5)) * c.D + d) * 32 + (p & 31);
}
__device__ __forceinline__ void store_f16(const CacheRef& c, bool is_v, int s, int g, int p, int d, float x) {
  const size_t head = (size_t)s * c.n_kv + g;
  const uint16_t h = f2h_bits(x);
  if (!is_v) reinterpret_cast<uint16_t*>(c.k)[(head * c.cap + p) * c.D + d] = h;
  else reinterpret_cast<uint16_t*>(c.v)[v_index(c, head, p, d)] = h;
}
__device__ __forceinline__ void store_q8(const CacheRef& c, bool is_v, int s, int g, int p, int d, int8_t q,
                                         uint16_t dbits) {
  const size_t head = (size_t)s * c.n_kv + g;
  if (!is_v) {
    reinterpret_cast<int8_t*>(c.k)[(head * c.cap + p) * c.D + d] = q;
    if ((d & 31) == 0) c.ks[(head * c.cap + p) * (c.D / 32) + d / 32] = dbits;
  } else {
    reinterpret_cast<int8_t*>(c.v)[v_index(c, head, p, d)] = q;
    if ((d & 31) == 0) c.vs[(head * c.cap + p) * (c.D / 32) + d / 32] = dbits;
  }
}

// OCP E4M3 code of x: nearest (ties to even), magnitudes above 448 to +-448,
// NaN to 0x7F (sign kept).  In binade e = floor(log2 |x|) >= -6 the step is
// 2^(e-3) and below 2^-6 the subnormal step 2^-9; |x| * 2^(3-e) is exact and
// rintf rounds it to even, and a result of 16 carries into the exponent
// field (the next binade's first code).
__device__ __forceinline__ uint8_t f8_code(float x) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u;
  if (x != x) return (uint8_t)(sign | 0x7Fu);
  const float a = fminf(fabsf(x), 448.f);
  int e = (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 255u) - 127;
  e = e < -6 ? -6 : e;
  const int q = (int)rintf(a * exp2i(3 - e));
  return (uint8_t)(sign | (uint32_t)(((e + 7) << 3) + q - 8));
}
__device__ __forceinline__ void store_f8(const CacheRef& c, bool is_v, int s, int g, int p, int d, float x) {
  const size_t head = (size_t)s * c.n_kv + g;
  const uint8_t q = f8_code(x);
  if (!is_v) c.k[(head * c.cap + p) * c.D + d] = q;
  else c.v[v_index(c, head, p, d)] = q;
}
// Element-wise formats (fp16, E4M3): one value, no block reduction.
__device__ __forceinline__ void store_point(const CacheRef& c, bool is_v, int s, int g, int p, int d, float x) {
  if ((is_v ? c.vf : c.kf) == kFmtF8) store_f8(c, is_v, s, g, p, d, x);
  else store_f16(c, is_v, s, g, p, d, x);
}

// One Q8_0 block value: code of x for the block maximum amax (both fp64).
__device__ __forceinline__ void q8_encode(double x, double amax, int8_t& q, uint16_t& dbits) {
  dbits = f64_to_f16_bits(amax / 127.0);
  q = q8_code(x, f16_bits_to_f64(dbits));
}

// Store value `x` of dim d of (slot, kv head g, pos) into K (is_v = false) or V.
// For Q8_0 all 32 lanes of the dim's block must call this together.
__device__ __forceinline__ void store_elem(const CacheRef& c, bool is_v, int s, int g, int p, int d, float x,
                                           bool ok) {
  if ((is_v ? c.vf : c.kf) != kFmtQ8) {
    if (ok) store_point(c, is_v, s, g, p, d, x);
  } else {
    const double xd = (double)x;
    int8_t q;
    uint16_t dbits;
    q8_encode(xd, amax32(fabs(xd)), q, dbits);
    if (ok) store_q8(c, is_v, s, g, p, d, q, dbits);
  }
}

// Where logical position p of sequence b is stored.  Slot arena (pages ==
// nullptr): slot s as given, position p.  Paged pool (slots are pages of cap
// tokens, cap = 2^page_shift): s = pages[b * max_pages + p / cap], p % cap.
// On return s and p address the store; false if it lies outside the cache.
__device__ __forceinline__ bool kv_locate(const int32_t* pages, int max_pages, int page_shift, int n_slots, int cap,
                                          int b, int& s, int& p) {
  if (pages) {
    const bool in = p >= 0 && p < (max_pages << page_shift);
    s = in ? pages[(size_t)b * max_pages + (p >> page_shift)] : -1;
    p &= cap - 1;
    return in && s >= 0 && s < n_slots;
  }
  return s >= 0 && s < n_slots && p >= 0 && p < cap;
}

// Rotary position embedding, rotate-half pairs (i, i + D/2): the angle of
// pair i at position p, p * base^(-2i/D), is formed in fp64; cos and sin are
// rounded once to fp32 and the rotation itself is fp32.
__device__ __forceinline__ void rope_cos_sin(int p, int i, int D, float base, float& cs, float& sn) {
  const double theta = pow((double)base, -2.0 * (double)i / (double)D);
  const double ang = (double)p * theta;
  cs = (float)cos(ang);
  sn = (float)sin(ang);
}

__device__ __forceinline__ CacheRef cache_ref(const qkdec_kv_layer& kv) {
  CacheRef c;
  c.k = reinterpret_cast<uint8_t*>(kv.k);
  c.v = reinterpret_cast<uint8_t*>(kv.v);
  c.ks = reinterpret_cast<uint16_t*>(kv.k_scale);
  c.vs = reinterpret_cast<uint16_t*>(kv.v_scale);
  c.n_kv = kv.n_kv_heads;
  c.cap = kv.capacity;
  c.D = kv.head_dim;
  c.n_slots = kv.n_slots;
  c.kf = kv.type == QKDEC_KV_FP8_E4M3 ? kFmtF8
         : (kv.type == QKDEC_KV_Q8_0 || kv.type == QKDEC_KV_Q8_0_K_F16_V) ? kFmtQ8 : kFmtF16;
  c.vf = kv.type == QKDEC_KV_FP8_E4M3 ? kFmtF8
         : (kv.type == QKDEC_KV_Q8_0 || kv.type == QKDEC_KV_F16_K_Q8_0_V) ? kFmtQ8 : kFmtF16;
  return c;
}

}  // namespace qk
