// Device code of the Q4_K dequant-GEMM shared by both GEMM kernels (split-K
// in gemm_q4k.hip, K split over waves in gemm_wk.hip): fragment loads, the
// exact nibble decode and the MFMA pair of one super-block (the layout and
// the arithmetic are described at the top of gemm_q4k.hip).
#pragma once

#include "common.h"
#include "internal.h"

namespace qk {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

struct Q4Frag {
  u32x4 hdr;   // bytes 0-15 of the lane's block: d, dmin, scale groups
  u32x4 q0;    // quant bytes 16+32g .. +15
  u32x4 q1;    // quant bytes 32+32g .. +15
};

__device__ __forceinline__ void load_frag(Q4Frag& f, const uint8_t* __restrict__ blk, int g) {
  f.hdr = *reinterpret_cast<const u32x4*>(blk);
  f.q0 = *reinterpret_cast<const u32x4*>(blk + 16 + 32 * g);
  f.q1 = *reinterpret_cast<const u32x4*>(blk + 32 + 32 * g);
}

// keep a constant in a VGPR so the mask-and-or pairs fuse into v_and_or_b32
__device__ __forceinline__ uint32_t in_vgpr(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

struct NibbleMasks {
  uint32_t lo, hi, magic;
};

// Decoded B operand for one MFMA: weights 8j..8j+7 of one 32-bit quant word,
// times the sub-block scale.
__device__ __forceinline__ half8_t decode_word(uint32_t w, const NibbleMasks& k, half2_t s1, half2_t c1, half2_t s16,
                                              half2_t c16) {
  const uint32_t w8 = w >> 8;
  half2_t v0 = as_h2((w & k.lo) | k.magic);
  half2_t v1 = as_h2((w & k.hi) | k.magic);
  half2_t v2 = as_h2((w8 & k.lo) | k.magic);
  half2_t v3 = as_h2((w8 & k.hi) | k.magic);
  v0 = __builtin_elementwise_fma(v0, s1, c1);
  v1 = __builtin_elementwise_fma(v1, s16, c16);
  v2 = __builtin_elementwise_fma(v2, s1, c1);
  v3 = __builtin_elementwise_fma(v3, s16, c16);
  half8_t b;
  b[0] = v0[0]; b[1] = v0[1]; b[2] = v1[0]; b[3] = v1[1];
  b[4] = v2[0]; b[5] = v2[1]; b[6] = v3[0]; b[7] = v3[1];
  return b;
}

// The block header fields lane (g, r) needs: d, dmin, the mins m0, m1 of its
// sub-blocks 2g, 2g+1, and the packed constants that turn a nibble expanded
// to 1024 + q (or 1024 + 16q) into sc * q exactly (decode_word).
struct Q4Header {
  float d, dmin, m0, m1;
  half2_t s1a, c1a, s16a, c16a, s1b, c1b, s16b, c16b;
};

__device__ __forceinline__ Q4Header q4_header(const Q4Frag& f, int g) {
  Q4Header h;
  const uint32_t h0 = f.hdr[0], h1 = f.hdr[1], h2 = f.hdr[2], h3 = f.hdr[3];
  h.d = h2f(h0 & 0xffffu);
  h.dmin = h2f(h0 >> 16);
  // the 24-bit scale group of sub-blocks 2g, 2g+1 sits at bit 24g of bytes 4..15
  const uint32_t lo = (g < 2) ? h1 : (g == 2 ? h2 : h3);
  const uint32_t hi = (g < 2) ? h2 : h3;
  const uint32_t grp = __builtin_amdgcn_alignbit(hi, lo, (24u * (uint32_t)g) & 31u);
  const float sc0 = (float)(grp & 63u), sc1 = (float)((grp >> 6) & 63u);
  h.m0 = (float)((grp >> 12) & 63u);
  h.m1 = (float)((grp >> 18) & 63u);
  h.s1a = pack_h2(sc0, sc0); h.c1a = pack_h2(-1024.f * sc0, -1024.f * sc0);
  h.s16a = pack_h2(sc0 * 0.0625f, sc0 * 0.0625f); h.c16a = pack_h2(-64.f * sc0, -64.f * sc0);
  h.s1b = pack_h2(sc1, sc1); h.c1b = pack_h2(-1024.f * sc1, -1024.f * sc1);
  h.s16b = pack_h2(sc1 * 0.0625f, sc1 * 0.0625f); h.c16b = pack_h2(-64.f * sc1, -64.f * sc1);
  return h;
}

// Weights 8j..8j+7 of the lane's 64 (sub-block 2g for j < 4, 2g+1 after), as
// sc * q in fp16.
__device__ __forceinline__ half8_t q4_word(const Q4Frag& f, const Q4Header& h, int j, const NibbleMasks& k) {
  const uint32_t w = j < 4 ? f.q0[j] : f.q1[j - 4];
  return j < 4 ? decode_word(w, k, h.s1a, h.c1a, h.s16a, h.c16a) : decode_word(w, k, h.s1b, h.c1b, h.s16b, h.c16b);
}

// One super-block of one 16-row tile: sq = X . (sc*q), sm = xsums . m (per
// sequence row), with d and dmin returned for the deferred accumulation.
__device__ __forceinline__ void q4_superblock(const Q4Frag& f, const half8_t (&a)[8], const half4_t& axs, int g,
                                              const NibbleMasks& k, floatx4& sq, floatx4& sm, float& d,
                                              float& dmin) {
  const Q4Header h = q4_header(f, g);
  d = h.d;
  dmin = h.dmin;
  const half2_t mm = pack_h2(h.m0, h.m1);
  half4_t bm;
  bm[0] = mm[0]; bm[1] = mm[1]; bm[2] = mm[0]; bm[3] = mm[1];
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
  sm = __builtin_amdgcn_mfma_f32_16x16x16f16(axs, bm, zero, 0, 0, 0);
  sq = zero;
#pragma unroll
  for (int j = 0; j < 8; ++j) sq = mfma16x16x32(a[j], q4_word(f, h, j, k), sq);
}

// The same super-block on the vector ALU for NB <= 2 sequences (the
// small-batch matvec): the lane decodes exactly the weights it decodes for
// the MFMA (row r, weights 64g..64g+63) and forms, per sequence b, the packed
// fp16 dot products sq[b] = sum_k x_b[k] sc q_k (fp32 accumulation; every
// product exact) and sm[b] = m0 X_b,2g + m1 X_b,2g+1 from the sub-block sums
// xs[b] (fp32).  No matrix-core instruction and no padding of the batch.
template <int NB>
__device__ __forceinline__ void q4_superblock_mv(const Q4Frag& f, const half8_t (&x)[NB][8], const float (&xs)[NB][2],
                                                 int g, const NibbleMasks& k, float (&sq)[NB], float (&sm)[NB],
                                                 float& d, float& dmin) {
  const Q4Header h = q4_header(f, g);
  d = h.d;
  dmin = h.dmin;
#pragma unroll
  for (int b = 0; b < NB; ++b) sq[b] = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const half8_t w = q4_word(f, h, j, k);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        sq[b] = __builtin_amdgcn_fdot2(half2_t{x[b][j][e], x[b][j][e + 1]}, half2_t{w[e], w[e + 1]}, sq[b], false);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) sm[b] = __builtin_fmaf(h.m0, xs[b][0], h.m1 * xs[b][1]);
}


// The hi/lo sums of sub-blocks 2g (pieces 0..3) and 2g+1 (pieces 4..7) of av
// and the row's dmin factor; fdr is the row's d factor.
__device__ __forceinline__ void a_sums(const half8_t (&av)[8], float fdr, half4_t& axs, float& fmr) {
  // pairs of fp16 values added into fp32 accumulators (v_dot2_f32_f16 against
  // (1, 1)): half the instructions of a convert and an add per value
  const half2_t one = {(half_t)1.f, (half_t)1.f};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      s0 = __builtin_amdgcn_fdot2(half2_t{av[j][e], av[j][e + 1]}, one, s0, false);
      s1 = __builtin_amdgcn_fdot2(half2_t{av[4 + j][e], av[4 + j][e + 1]}, one, s1, false);
    }
  // a super-block whose sub-block sums leave fp16's range stages them divided
  // by 32 (32 values of at most 65504 then fit); dmin is multiplied back
  float ms = fmaxf(fabsf(s0), fabsf(s1));
  ms = fmaxf(ms, __shfl_xor(ms, 16));
  ms = fmaxf(ms, __shfl_xor(ms, 32));
  const bool big = ms > 65504.f;
  if (big) {
    s0 *= 0.03125f;
    s1 *= 0.03125f;
  }
  fmr = big ? 32.f * fdr : fdr;
  const half_t h0 = (half_t)s0, h1 = (half_t)s1;
  axs[0] = h0;
  axs[1] = h1;
  axs[2] = (half_t)(s0 - (float)h0);
  axs[3] = (half_t)(s1 - (float)h1);
}

// smallest s >= 0 with amax * 2^-s <= 65504 (the largest finite fp16)
__device__ __forceinline__ int f16_block_shift(float amax) {
  const int e = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 255u) - 127;
  int sh = e - 15 > 0 ? e - 15 : 0;
  if (amax * exp2i(-sh) > 65504.f) ++sh;
  return sh;
}

// Tile of wave w in row group rg (WPB waves per work-group).
//   MODE 0 and 2: tiles WPB*rg .. WPB*rg + WPB - 1 (one per wave).
//   MODE 1 (SwiGLU): waves 0 .. H-1 (H = WPB/2) take gate tiles H*rg + w, waves
//   H .. WPB-1 the up tiles F/16 later, so one work-group holds both halves of
//   16*H outputs.
template <int MODE, int WPB>
__device__ __forceinline__ int tile_of(int rg, int w, int f_tiles) {
  constexpr int H = WPB / 2;
  if (MODE != 1) return rg * WPB + w;
  return (w < H) ? (rg * H + w) : (f_tiles + rg * H + (w - H));
}
template <int MODE, int WPB>
__device__ __forceinline__ bool tile_valid(int rg, int w, int n_tiles, int f_tiles) {
  constexpr int H = WPB / 2;
  if (MODE != 1) return rg * WPB + w < n_tiles;
  return rg * H + (w % H) < f_tiles;
}

// How the activations arrive.
enum XMode : int {
  kXF16 = 0,         // fp16, used as they are
  kXF32Blocked = 1,  // fp32, rounded to fp16 with one power-of-two offset per row and 256 values
  kXNorm = 2,        // fp32 residual stream, RMSNorm applied while staging: f16(x * rinv * gamma)
};

struct GemmArgs {
  const uint8_t* W;
  const void* X;
  const float* gamma;    // kXNorm: gains of the K inputs
  const float* ss_in;    // kXNorm: sum-of-squares slots of the rows of X
  float* Y;              // MODE 0 output (may alias residual)
  const float* residual;
  float* ss_out;         // MODE 0: sum-of-squares slots of Y (one slot per work-group), or null
  float* A;              // MODE 1 output
  float* part;           // split-K partial sums
  unsigned* counters;    // split-K arrival counters (one per row group)
  int64_t ldx, ldy, ldr, lda;
  int n_tiles, kb, B, f_tiles, ss_slots;
  float eps, inv_k;
  RopeAppendArgs ra;     // MODE 2 only
};

// LDS scratch of one GEMM work item besides its staged activations; MODE 2
// adds the rotary (cos, sin) table.
template <int WPB, int MODE = 0>
struct GemmSmem {
  float fac_d[16 * 16], fac_m[16 * 16];   // per (super-block i, row b) at i * 16 + b: factors of d and dmin
  float s_red[WPB][16];                   // per-wave partial row statistics
  floatx4 fin[WPB][64];                   // SwiGLU: gate and up accumulators exchanged between waves
  int s_last;
};
template <int WPB>
struct GemmSmem<WPB, 2> : GemmSmem<WPB, 0> {
  float2 rope[16][64];                    // (cos, sin) per (sequence, pair), head_dim <= 128
};

}  // namespace qk
