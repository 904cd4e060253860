// KV-cache append (fp16 / Q8_0 / E4M3).  Within a decode step the append (with the
// rotary embedding of k) is done by the QKV projection's finishing work-group
// (gemm_q4k.hip, MODE 2) with the same store helpers (kv_dev.h).
// (P1, P2, P3: the three pages listed, with their titles, at the top of include/qkdec.h.)
//
// P3 "Why Q8 is close to free and where the sharp edges are": the quantized
// cache stores one byte per element plus a per-block scale.  The Q8_0
// quantizer of one block of 32 values (one token, one KV head) runs in fp64:
// d = RN_fp16(amax / 127), q = x / d rounded half away from zero, clamped to
// [-127, 127], q = 0 where d = 0.  A thread owns one or two dims; the block
// amax is a max-reduction over the 32 lanes holding one block.
//
// P2 "What a long-running swarm should actually tune": an 8-bit float cache
// (read here as OCP E4M3, unscaled) stores each value as its nearest code,
// ties to even, saturating at +-448 (f8_code in kv_dev.h); no reduction.
#include "common.h"
#include "internal.h"
#include "kv_dev.h"

namespace qk {

// grid (n_kv, B), block D threads: thread d stores dim d of k and v.  With a
// page table (pages != NULL) the cache layer is a pool of pages of cap tokens
// (a power of two, 2^page_shift) and position pos[b] of sequence b goes to
// page pages[b * max_pages + pos / cap] at pos % cap.
__global__ void kv_append_kernel(qkdec_kv_layer kv, const int32_t* slot, const int32_t* pos, const float* k,
                                 const float* v, int32_t* err, const int32_t* pages, int max_pages, int page_shift) {
  const CacheRef c = cache_ref(kv);
  const int g = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  int s = pages ? 0 : slot[b], p = pos[b];
  const bool ok = kv_locate(pages, max_pages, page_shift, c.n_slots, c.cap, b, s, p);
  if (!ok && d == 0 && err) *err = QKDEC_E_CAPACITY;
  const size_t src = ((size_t)b * c.n_kv + g) * c.D + d;
  store_elem(c, false, s, g, p, d, k[src], ok);
  store_elem(c, true, s, g, p, d, v[src], ok);
}

// The QKV projection's finish as its own launch (after a projection kernel
// that only stores the fp32 rows Y = [q heads; k heads; v heads] per
// sequence): grid (Hq + 2 n_kv, B), block D threads; thread d of head h rotates
// dims (d, d +- D/2) of q and k at pos[b] (rope_cos_sin), q goes out as fp16,
// k and v are appended to the cache at (slot[b], spos[b]) (spos: pos, or the
// position within the page a paged step located).
__global__ void rope_append_kernel(qkdec_kv_layer kv, const float* __restrict__ Y, int64_t ldy, int Hq,
                                   const int32_t* slot, const int32_t* pos, float rope_base, uint16_t* q16,
                                   int32_t* err, const int32_t* spos, const float2* rope) {
  const CacheRef c = cache_ref(kv);
  const int head = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int D = c.D, half = D / 2;
  const bool is_q = head < Hq, is_v = head >= Hq + c.n_kv;
  const float* yr = Y + (size_t)b * ldy + (size_t)head * D;
  const float x = yr[d];
  const int p = pos[b];
  float out = x;
  if (!is_v) {
    const float other = yr[d < half ? d + half : d - half];
    float cs, sn;
    if (rope) {
      const float2 c = rope[(size_t)b * half + d % half];
      cs = c.x;
      sn = c.y;
    } else {
      rope_cos_sin(p, d % half, D, rope_base, cs, sn);
    }
    // d < D/2: x_i cos - x_{i+D/2} sin; d >= D/2: x_{i+D/2} cos + x_i sin
    out = d < half ? x * cs - other * sn : x * cs + other * sn;
  }
  if (is_q) {
    q16[((size_t)b * Hq + head) * D + d] = f2h_bits(out);
    return;
  }
  const int s = slot[b], pp = spos[b];
  const bool ok = s >= 0 && s < c.n_slots && pp >= 0 && pp < c.cap;
  if (!ok && d == 0 && err) *err = QKDEC_E_CAPACITY;
  const int g = is_v ? head - Hq - c.n_kv : head - Hq;
  store_elem(c, is_v, s, g, pp, d, out, ok);
}

hipError_t launch_rope_append(const qkdec_kv_layer& kv, const float* Y, int64_t ldy, int Hq, int B,
                              const int32_t* slot, const int32_t* pos, float rope_base, uint16_t* q16, int32_t* err,
                              hipStream_t st, const int32_t* spos, const float2* rope) {
  hipLaunchKernelGGL(rope_append_kernel, dim3(Hq + 2 * kv.n_kv_heads, B), dim3(kv.head_dim), 0, st, kv, Y, ldy, Hq,
                     slot, pos, rope_base, q16, err, spos ? spos : pos, rope);
  return hipGetLastError();
}

__global__ void rope_table_kernel(const int32_t* pos, int D, float rope_base, float2* table) {
  const int b = blockIdx.x, i = threadIdx.x;
  float cs, sn;
  rope_cos_sin(pos[b], i, D, rope_base, cs, sn);
  table[(size_t)b * (D / 2) + i] = make_float2(cs, sn);
}

hipError_t launch_rope_table(const int32_t* pos, int B, int D, float rope_base, float2* table, hipStream_t st) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(B), dim3(D / 2), 0, st, pos, D, rope_base, table);
  return hipGetLastError();
}

// one thread per sequence: page and position within it of pos[b]
__global__ void page_locate_kernel(const int32_t* pages, int max_pages, int page_shift, int n_pages,
                                   const int32_t* pos, int B, int32_t* page, int32_t* page_pos) {
  const int b = threadIdx.x;
  if (b >= B) return;
  int s = 0, p = pos[b];
  const bool ok = kv_locate(pages, max_pages, page_shift, n_pages, 1 << page_shift, b, s, p);
  page[b] = ok ? s : -1;
  page_pos[b] = p;
}

hipError_t launch_page_locate(const int32_t* pages, int max_pages, int page_tokens, int n_pages, const int32_t* pos,
                              int B, int32_t* page, int32_t* page_pos, hipStream_t st) {
  int shift = 0;
  while ((1 << shift) < page_tokens) ++shift;
  hipLaunchKernelGGL(page_locate_kernel, dim3(1), dim3(64), 0, st, pages, max_pages, shift, n_pages, pos, B, page,
                     page_pos);
  return hipGetLastError();
}

hipError_t launch_kv_append(const qkdec_kv_layer& kv, const int32_t* slot, const int32_t* pos, const float* k,
                            const float* v, int B, int32_t* err, hipStream_t st, const int32_t* pages,
                            int max_pages) {
  int shift = 0;
  while (pages && (1 << shift) < kv.capacity) ++shift;
  hipLaunchKernelGGL(kv_append_kernel, dim3(kv.n_kv_heads, B), dim3(kv.head_dim), 0, st, kv, slot, pos, k, v, err,
                     pages, pages ? max_pages : 0, shift);
  return hipGetLastError();
}

}  // namespace qk
