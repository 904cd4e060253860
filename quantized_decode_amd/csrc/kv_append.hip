// KV-cache append (fp16 / Q8_0) and the fused RoPE + append of a decode step.
// (P1, P2, P3: the three pages listed, with their titles, at the top of include/qkdec.h.)
//
// P3 "Why Q8 is close to free and where the sharp edges are": the quantized
// cache stores one byte per element plus a per-block scale.  The Q8_0
// quantizer of one block of 32 values (one token, one KV head) runs in fp64:
// d = RN_fp16(amax / 127), q = x / d rounded half away from zero, clamped to
// [-127, 127], q = 0 where d = 0.  A thread owns one or two dims; the block
// amax is a max-reduction over the 32 lanes holding one block.
//
// Rotary position embedding (rotate-half pairs (i, i + D/2), angle
// pos * base^(-2i/D)): the angle is formed in fp64, cos/sin are rounded once
// to fp32 and the rotation is fp32.
#include "common.h"
#include "internal.h"

namespace qk {

__device__ __forceinline__ double amax32(double v) {
  // max over aligned groups of 32 lanes
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
  bool q8;
};

// Store value `x` of dim d of (slot, kv head g, pos) into K (is_v = false) or V.
// For Q8_0 all 32 lanes of the dim's block must call this together.
__device__ __forceinline__ void store_elem(const CacheRef& c, bool is_v, int s, int g, int p, int d, float x,
                                           bool ok) {
  const size_t head = (size_t)s * c.n_kv + g;
  if (!c.q8) {
    if (!ok) return;
    const uint16_t h = f2h_bits(x);
    if (!is_v) reinterpret_cast<uint16_t*>(c.k)[(head * c.cap + p) * c.D + d] = h;
    else reinterpret_cast<uint16_t*>(c.v)[(head * c.D + d) * c.cap + p] = h;
  } else {
    const double xd = (double)x;
    const double amax = amax32(fabs(xd));
    const uint16_t dbits = f64_to_f16_bits(amax / 127.0);
    const int8_t q = q8_code(xd, f16_bits_to_f64(dbits));
    if (!ok) return;
    if (!is_v) {
      reinterpret_cast<int8_t*>(c.k)[(head * c.cap + p) * c.D + d] = q;
      if ((d & 31) == 0) c.ks[(head * c.cap + p) * (c.D / 32) + d / 32] = dbits;
    } else {
      reinterpret_cast<int8_t*>(c.v)[(head * c.D + d) * c.cap + p] = q;
      if ((d & 31) == 0) c.vs[(head * c.cap + p) * (c.D / 32) + d / 32] = dbits;
    }
  }
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
  c.q8 = kv.type == QKDEC_KV_Q8_0;
  return c;
}

// grid (n_kv, B), block D threads: thread d stores dim d of k and v.
__global__ void kv_append_kernel(qkdec_kv_layer kv, const int32_t* slot, const int32_t* pos, const float* k,
                                 const float* v, int32_t* err) {
  const CacheRef c = cache_ref(kv);
  const int g = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int s = slot[b], p = pos[b];
  const bool ok = s >= 0 && s < c.n_slots && p >= 0 && p < c.cap;
  if (!ok && d == 0 && err) *err = QKDEC_E_CAPACITY;
  const size_t src = ((size_t)b * c.n_kv + g) * c.D + d;
  store_elem(c, false, s, g, p, d, k[src], ok);
  store_elem(c, true, s, g, p, d, v[src], ok);
}

// Fused step kernel.  grid (Hq + Hkv, B), block D/2 threads; thread i owns the
// rotate-half pair (i, i + D/2).  Blocks h < Hq rotate query head h and write
// it as fp16; blocks Hq + g rotate key head g and append key and value head g.
__global__ void rope_append_kernel(qkdec_kv_layer kv, const int32_t* slot, const int32_t* pos, const float* qkv,
                                   int Hq, float rope_base, half_t* q16, int32_t* err) {
  const CacheRef c = cache_ref(kv);
  const int hb = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
  const int D = c.D, half = D / 2, Hkv = c.n_kv;
  const int p = pos[b];
  const int s = slot[b];
  const size_t row = (size_t)b * (Hq + 2 * Hkv) * D;
  const double theta = pow((double)rope_base, -2.0 * (double)i / (double)D);
  const double ang = (double)p * theta;
  const float cs = (float)cos(ang), sn = (float)sin(ang);
  if (hb < Hq) {
    const float* x = qkv + row + (size_t)hb * D;
    const float x1 = x[i], x2 = x[i + half];
    half_t* o = q16 + ((size_t)b * Hq + hb) * D;
    o[i] = (half_t)(x1 * cs - x2 * sn);
    o[i + half] = (half_t)(x2 * cs + x1 * sn);
  } else {
    const int g = hb - Hq;
    const bool ok = s >= 0 && s < c.n_slots && p >= 0 && p < c.cap;
    if (!ok && i == 0 && err) *err = QKDEC_E_CAPACITY;
    const float* xk = qkv + row + (size_t)(Hq + g) * D;
    const float* xv = qkv + row + (size_t)(Hq + Hkv + g) * D;
    const float k1 = xk[i], k2 = xk[i + half];
    store_elem(c, false, s, g, p, i, k1 * cs - k2 * sn, ok);
    store_elem(c, false, s, g, p, i + half, k2 * cs + k1 * sn, ok);
    store_elem(c, true, s, g, p, i, xv[i], ok);
    store_elem(c, true, s, g, p, i + half, xv[i + half], ok);
  }
}

hipError_t launch_kv_append(const qkdec_kv_layer& kv, const int32_t* slot, const int32_t* pos, const float* k,
                            const float* v, int B, int32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(kv.n_kv_heads, B), dim3(kv.head_dim), 0, st, kv, slot, pos, k, v, err);
  return hipGetLastError();
}

hipError_t launch_rope_append(const qkdec_kv_layer& kv, const int32_t* slot, const int32_t* pos, const float* qkv,
                              int B, int n_q_heads, float rope_base, uint16_t* q16, int32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(rope_append_kernel, dim3(n_q_heads + kv.n_kv_heads, B), dim3(kv.head_dim / 2), 0, st, kv, slot,
                     pos, qkv, n_q_heads, rope_base, reinterpret_cast<half_t*>(q16), err);
  return hipGetLastError();
}

}  // namespace qk
