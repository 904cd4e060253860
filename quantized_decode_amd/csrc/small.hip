// Embedding gather (with the row statistics for the fused RMSNorm), the final
// RMSNorm -> fp16, and the fp16 LM head with fused argmax.
// (P1, P2, P3: the three pages listed, with their titles, at the top of include/qkdec.h.)
//
// P1 "The weight read is the only term that does not scale": the norms run
// over one row per sequence; reading the output embedding is shared by the
// batch while the matmul against it and the sampling are per sequence.
#include "common.h"
#include "internal.h"

namespace qk {

// x[b] = E[tok[b]] in fp32 (a token outside [0, vocab) reads row 0), and the
// sum-of-squares slots of x (16 lanes per 16-column slot): hidden % 256 == 0.
__global__ void __launch_bounds__(256) embed_kernel(const half_t* __restrict__ E, int hidden, int vocab,
                                                    const int32_t* tok, float* x, float* ss) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  int t = tok[b];
  if (t < 0 || t >= vocab) t = 0;
  const float v = (float)E[(size_t)t * hidden + i];
  x[(size_t)b * hidden + i] = v;
  float q = v * v;
  for (int o = 8; o >= 1; o >>= 1) q += __shfl_xor(q, o);
  if ((threadIdx.x & 15) == 0) ss[(blockIdx.x * 16 + (threadIdx.x >> 4)) * 16 + b] = q;
}

// h = f16(x * rinv * gamma) with rinv from the sum-of-squares slots of x;
// one 256-column block per work-group.
__global__ void __launch_bounds__(256) rmsnorm_f16_kernel(const float* __restrict__ x, const float* __restrict__ gamma,
                                                          const float* __restrict__ ss, int hidden, float eps,
                                                          half_t* __restrict__ h) {
  __shared__ float red[4][16];
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  SsFold<256, kSsMaxSlots> f;
  f.load(ss, hidden / kSsCols);
  const float xv = x[(size_t)b * hidden + i];
  const float gv = gamma[i];
  f.fold(red);
  __syncthreads();
  h[(size_t)b * hidden + i] = norm_apply(xv, rms_inv<4>(red, b, 1.0f / (float)hidden, eps), gv);
}

// ------------------------------------------------------------------ LM head
// Tiles of 16 vocabulary rows; v_mfma_f32_16x16x32_f16 with A = hidden states
// (sequence rows, staged once per work-group in LDS) and B = W_lm^T.  Lane
// (g, r) reads row r of the tile, 8 values at 32j + 8g of each 256-wide chunk.
// Every wave keeps a running (max, lowest index) per sequence; the work-group
// result goes to a partials buffer that lm_argmax_reduce_kernel folds.
constexpr int kLmWaves = 8;
constexpr int kLmGroups = 512;   // work-groups of the LM head launch (grid-stride over tiles)

__device__ __forceinline__ void better(float& v, int& ix, float v2, int ix2) {
  if (v2 > v || (v2 == v && ix2 < ix)) { v = v2; ix = ix2; }
}

__global__ void __launch_bounds__(64 * kLmWaves) lm_head_kernel(const half_t* __restrict__ W, int n_tiles, int H,
                                                      const half_t* __restrict__ X, int B, float* logits, int64_t V,
                                                      float* part_v, int32_t* part_i) {
  extern __shared__ half_t xs[];                 // [B][H + 8]
  const int ldsx = H + 8;
  for (int idx = threadIdx.x; idx < B * (H / 8); idx += 64 * kLmWaves) {
    const int b = idx / (H / 8), c = idx % (H / 8);
    *reinterpret_cast<half8_t*>(xs + b * ldsx + 8 * c) = *reinterpret_cast<const half8_t*>(X + (size_t)b * H + 8 * c);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const bool act = r < B;
  float bestv[4];
  int besti[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { bestv[i] = -__builtin_inff(); besti[i] = 0x7fffffff; }

  const int nchunks = H / 256;
  for (int tile = blockIdx.x * kLmWaves + wave; tile < n_tiles; tile += gridDim.x * kLmWaves) {
    const half_t* wrow = W + ((size_t)tile * 16 + r) * H + 8 * g;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    half8_t wb[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wb[0][j] = *reinterpret_cast<const half8_t*>(wrow + 32 * j);
    for (int c0 = 0; c0 < nchunks; c0 += 2) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int c = c0 + p;
        if (c < nchunks) {
          const int nx = (c + 1 < nchunks) ? c + 1 : c;
#pragma unroll
          for (int j = 0; j < 8; ++j) wb[p ^ 1][j] = *reinterpret_cast<const half8_t*>(wrow + 256 * nx + 32 * j);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            half8_t a = act ? *reinterpret_cast<const half8_t*>(xs + r * ldsx + 256 * c + 32 * j + 8 * g)
                            : half8_t{0, 0, 0, 0, 0, 0, 0, 0};
            acc = mfma16x16x32(a, wb[p][j], acc);
          }
        }
      }
    }
    const int v = tile * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * g + i;
      if (b < B) {
        if (logits) logits[(size_t)b * V + v] = acc[i];
        better(bestv[i], besti[i], acc[i], v);
      }
    }
  }
  // reduce over the 16 rows (lanes r) of each lane group
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    for (int o = 8; o >= 1; o >>= 1) {
      const float v2 = __shfl_xor(bestv[i], o, 16);
      const int i2 = __shfl_xor(besti[i], o, 16);
      better(bestv[i], besti[i], v2, i2);
    }
  }
  __shared__ float sv[kLmWaves][16];
  __shared__ int si[kLmWaves][16];
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { sv[wave][4 * g + i] = bestv[i]; si[wave][4 * g + i] = besti[i]; }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int b = threadIdx.x;
    float v = sv[0][b];
    int ix = si[0][b];
    for (int w = 1; w < kLmWaves; ++w) better(v, ix, sv[w][b], si[w][b]);
    part_v[blockIdx.x * 16 + b] = v;
    part_i[blockIdx.x * 16 + b] = ix;
  }
}

// tok[b] = index of the best partial; pos[b] += 1 when pos is given.
__global__ void lm_argmax_reduce_kernel(const float* part_v, const int32_t* part_i, int n_parts, int B,
                                        int32_t* tok, int32_t* pos_inc) {
  const int b = blockIdx.x;
  float v = -__builtin_inff();
  int ix = 0x7fffffff;
  for (int j = threadIdx.x; j < n_parts; j += 64) better(v, ix, part_v[j * 16 + b], part_i[j * 16 + b]);
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = __shfl_xor(v, o);
    const int i2 = __shfl_xor(ix, o);
    better(v, ix, v2, i2);
  }
  if (threadIdx.x == 0) {
    tok[b] = (ix == 0x7fffffff) ? 0 : ix;
    if (pos_inc) pos_inc[b] += 1;
  }
}

__global__ void fill_zero_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_embed(const uint16_t* E, int hidden, int vocab, const int32_t* tok, int B, float* x, float* ss,
                        hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(hidden / 256, B), dim3(256), 0, st, reinterpret_cast<const half_t*>(E), hidden,
                     vocab, tok, x, ss);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_f16(const float* x, const float* gamma, const float* ss, int hidden, int B, float eps,
                              uint16_t* h, hipStream_t st) {
  hipLaunchKernelGGL(rmsnorm_f16_kernel, dim3(hidden / 256, B), dim3(256), 0, st, x, gamma, ss, hidden, eps,
                     reinterpret_cast<half_t*>(h));
  return hipGetLastError();
}

size_t lm_head_partials_bytes(int64_t V, int B) {
  (void)V;
  (void)B;
  return (size_t)kLmGroups * 16 * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_lm_head_argmax(const uint16_t* Wlm, int64_t V, int64_t H, const uint16_t* X, int B, float* logits,
                                 int32_t* tok, void* partials, int32_t* pos_inc, hipStream_t st) {
  const int n_tiles = (int)(V / 16);
  int groups = (n_tiles + kLmWaves - 1) / kLmWaves;
  if (groups > kLmGroups) groups = kLmGroups;
  float* pv = reinterpret_cast<float*>(partials);
  int32_t* pi = reinterpret_cast<int32_t*>(pv + (size_t)kLmGroups * 16);
  const size_t lds = (size_t)B * (H + 8) * sizeof(half_t);
  hipLaunchKernelGGL(lm_head_kernel, dim3(groups), dim3(64 * kLmWaves), lds, st, reinterpret_cast<const half_t*>(Wlm), n_tiles,
                     (int)H, reinterpret_cast<const half_t*>(X), B, logits, V, pv, pi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lm_argmax_reduce_kernel, dim3(B), dim3(64), 0, st, pv, pi, groups, B, tok, pos_inc);
  return hipGetLastError();
}

__global__ void prefill_rows_kernel(int s, int start, const int32_t* tokens, int rows, int32_t* slot, int32_t* pos,
                                    int32_t* tok) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= rows) return;
  slot[b] = s;
  pos[b] = start + b;
  tok[b] = tokens[b];
}

hipError_t launch_prefill_rows(int s, int start, const int32_t* tokens, int rows, int32_t* slot, int32_t* pos,
                               int32_t* tok, hipStream_t st) {
  hipLaunchKernelGGL(prefill_rows_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, s, start, tokens, rows, slot, pos,
                     tok);
  return hipGetLastError();
}

// the rows of one prefill chunk of a sequence in a paged pool (page table
// row `pages`, max_pages entries, pages of 2^page_shift tokens): pos[b] =
// start + b, page[b] = the page holding it (-1 outside the table or the
// pool), page_pos[b] = its position in the page, tok[b] = tokens[b]
__global__ void prefill_page_rows_kernel(const int32_t* pages, int max_pages, int page_shift, int n_pages, int start,
                                         const int32_t* tokens, int rows, int32_t* page, int32_t* pos,
                                         int32_t* page_pos, int32_t* tok) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= rows) return;
  const int p = start + b;
  const int pi = p >> page_shift;
  const int pg = pi < max_pages ? pages[pi] : -1;
  page[b] = (pg >= 0 && pg < n_pages) ? pg : -1;
  pos[b] = p;
  page_pos[b] = p & ((1 << page_shift) - 1);
  tok[b] = tokens[b];
}

hipError_t launch_prefill_page_rows(const int32_t* pages, int max_pages, int page_tokens, int n_pages, int start,
                                    const int32_t* tokens, int rows, int32_t* page, int32_t* pos, int32_t* page_pos,
                                    int32_t* tok, hipStream_t st) {
  int shift = 0;
  while ((1 << shift) < page_tokens) ++shift;
  hipLaunchKernelGGL(prefill_page_rows_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, pages, max_pages, shift,
                     n_pages, start, tokens, rows, page, pos, page_pos, tok);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, reinterpret_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace qk
