// Q4_K dequant-GEMM for a decode batch of 1..16 sequences on CDNA4 MFMA.
//
// P1 "The weight read is the only term that does not scale": the step streams
// each weight once and multiplies all sequences' hidden states against it.
// P1 "RDNA4 pads the batch dimension to 16 whether you fill it or not": the
// sequences are the M dimension of a 16-row matrix-core tile, so B = 1 and
// B = 16 issue the same instructions.  On gfx950 the tile is
// v_mfma_f32_16x16x32_f16 with A = activations (16 sequence rows, zero padded)
// and B = decoded weights (16 weight rows).
//
// Exactness: a Q4_K weight is d*sc*q - dmin*m.  The MFMA consumes the integer
// sc*q (<= 945, exact in fp16) against fp16 x, so every product is exact and
// accumulates in fp32.  The min term sum_s m_s * (sum of x over sub-block s)
// is one v_mfma_f32_16x16x16_f16 per super-block whose A operand holds the
// eight sub-block sums of x, each split into an fp16 hi + lo pair (about 22
// significant bits; a super-block whose sums exceed fp16's range has them
// divided by 32 and dmin multiplied by 32), and whose B operand holds the
// integer mins.  Per
// super-block and weight row the two results are scaled by d and dmin in fp32.
// No weight is ever rounded.
//
// Lane mapping (wave64, lane = 16*g + r, g = lane group 0..3, r = 0..15):
//   main MFMA j (0..7): B = weight row r, weights 64g + 8j + e (e = 0..7), i.e.
//     the lane's 32 contiguous quant bytes (16 + 32g) cover sub-blocks 2g (j < 4)
//     and 2g+1; A = sequence row r, x[sb*256 + 64g + 8j .. +7].
//   min MFMA: k-slots 4g..4g+3 = (hi_2g, hi_2g+1, lo_2g, lo_2g+1) of the x sums
//     against (m_2g, m_2g+1, m_2g, m_2g+1): each lane needs only its own scale group.
//   D: lane holds Y[4g + i][tile*16 + r], i = 0..3.
// The nibble layout puts weights 8j..8j+7 of a 32-bit word in slot order
// after two masks and one shift: (w & 0x000F000F) -> weights 8j, 8j+1;
// (w & 0x00F000F0) -> 8j+2, 8j+3 (times 16); the same on w >> 8 -> 8j+4..8j+7.
// OR-ing 0x6400 makes each half the fp16 value 1024 + q (or 1024 + 16q); one
// packed FMA with (sc, -1024 sc) (or (sc/16, -64 sc)) yields sc*q exactly.
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

// One super-block of one 16-row tile: sq = X . (sc*q), sm = xsums . m (per
// sequence row), with d and dmin returned for the deferred accumulation.
__device__ __forceinline__ void q4_superblock(const Q4Frag& f, const half8_t (&a)[8], const half4_t& axs, int g,
                                              const NibbleMasks& k, floatx4& sq, floatx4& sm, float& d,
                                              float& dmin) {
  const uint32_t h0 = f.hdr[0], h1 = f.hdr[1], h2 = f.hdr[2], h3 = f.hdr[3];
  d = h2f(h0 & 0xffffu);
  dmin = h2f(h0 >> 16);
  // the 24-bit scale group of sub-blocks 2g, 2g+1 sits at bit 24g of bytes 4..15
  const uint32_t lo = (g < 2) ? h1 : (g == 2 ? h2 : h3);
  const uint32_t hi = (g < 2) ? h2 : h3;
  const uint32_t grp = __builtin_amdgcn_alignbit(hi, lo, (24u * (uint32_t)g) & 31u);
  const float sc0 = (float)(grp & 63u), sc1 = (float)((grp >> 6) & 63u);
  const float m0 = (float)((grp >> 12) & 63u), m1 = (float)((grp >> 18) & 63u);
  const half2_t s1a = pack_h2(sc0, sc0), c1a = pack_h2(-1024.f * sc0, -1024.f * sc0);
  const half2_t s16a = pack_h2(sc0 * 0.0625f, sc0 * 0.0625f), c16a = pack_h2(-64.f * sc0, -64.f * sc0);
  const half2_t s1b = pack_h2(sc1, sc1), c1b = pack_h2(-1024.f * sc1, -1024.f * sc1);
  const half2_t s16b = pack_h2(sc1 * 0.0625f, sc1 * 0.0625f), c16b = pack_h2(-64.f * sc1, -64.f * sc1);
  const half2_t mm = pack_h2(m0, m1);
  half4_t bm;
  bm[0] = mm[0]; bm[1] = mm[1]; bm[2] = mm[0]; bm[3] = mm[1];
  const uint32_t words[8] = {f.q0[0], f.q0[1], f.q0[2], f.q0[3], f.q1[0], f.q1[1], f.q1[2], f.q1[3]};
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
  sm = __builtin_amdgcn_mfma_f32_16x16x16f16(axs, bm, zero, 0, 0, 0);
  sq = zero;
#pragma unroll
  for (int j = 0; j < 4; ++j) sq = mfma16x16x32(a[j], decode_word(words[j], k, s1a, c1a, s16a, c16a), sq);
#pragma unroll
  for (int j = 4; j < 8; ++j) sq = mfma16x16x32(a[j], decode_word(words[j], k, s1b, c1b, s16b, c16b), sq);
}

// 2^k as a float, k clamped to the normal range
__device__ __forceinline__ float exp2i(int k) {
  k = k < -126 ? -126 : (k > 127 ? 127 : k);
  return __builtin_bit_cast(float, (uint32_t)(k + 127) << 23);
}

// smallest s >= 0 with amax * 2^-s <= 65504 (the largest finite fp16)
__device__ __forceinline__ int f16_block_shift(float amax) {
  const int e = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 255u) - 127;
  int sh = e - 15 > 0 ? e - 15 : 0;
  if (amax * exp2i(-sh) > 65504.f) ++sh;
  return sh;
}

// Tile handled by slot t (0..TW-1) of wave w in row group rg.
//   MODE 0: consecutive tiles, 4*TW per work-group.
//   MODE 1 (SwiGLU), TW = 2: slot 0 = gate tile 4rg + w, slot 1 = the up tile F/16 later.
//   MODE 1, TW = 1: waves 0, 1 = gate tiles 2rg, 2rg + 1; waves 2, 3 = their up tiles.
template <int MODE, int TW>
__device__ __forceinline__ int tile_of(int rg, int w, int t, int f_tiles) {
  if (MODE == 0) return (rg * 4 + w) * TW + t;
  if (TW == 2) return (t == 0) ? (rg * 4 + w) : (f_tiles + rg * 4 + w);
  return (w < 2) ? (rg * 2 + w) : (f_tiles + rg * 2 + (w - 2));
}
template <int MODE, int TW>
__device__ __forceinline__ bool tile_valid(int rg, int w, int t, int n_tiles, int f_tiles) {
  if (MODE == 0) return tile_of<MODE, TW>(rg, w, t, f_tiles) < n_tiles;
  if (TW == 2) return rg * 4 + w < f_tiles;
  return rg * 2 + (w & 1) < f_tiles;
}

// Work-group: 4 waves, TW 16-row tiles each, covering super-blocks
// [c*KC, c*KC + KC) of K (c = blockIdx.y).  The work-group's activations
// (and their sub-block sums) are staged once in LDS and shared by its tiles.
// Each wave streams its tiles' super-blocks (2304 contiguous bytes each) with
// P - 1 of them in flight; a super-block's products are accumulated one
// super-block later, so the wave keeps issuing while its MFMAs finish.  With
// several K chunks every work-group writes its partial sums with write-through
// stores and the last one to arrive for a row group adds the chunks in chunk
// order (so the result does not depend on arrival order).
//
// XF32: the activations arrive in fp32 and are rounded to fp16 while staged,
// per row and 256-value block with the smallest power-of-two offset that
// keeps the block inside fp16's range (0 whenever plain fp16 fits); the
// offsets are multiplied back exactly per super-block.
template <int KC, int MODE, bool XF32, int TW>
__global__ void __launch_bounds__(256) gemm_q4k_kernel(
    const uint8_t* __restrict__ W, int n_tiles, int kb, const void* __restrict__ Xv, int64_t ldx, int B,
    float* Y, int64_t ldy, const float* residual, int64_t ldr, float* __restrict__ A, int64_t lda, int f_tiles,
    float* part, unsigned* counters) {
  constexpr int P = KC < 4 ? KC : 4;   // super-blocks resident per wave (P - 1 in flight)
  extern __shared__ half_t xs[];        // [B][KC*256 + 8] activations, then [B][KC][16] x sums
  // per (super-block i, row b) at i * 16 + b: the factors that d and dmin are
  // multiplied by (XF32 block offset; 32 where the x sums were staged divided by 32)
  __shared__ float fac_d[16 * 16], fac_m[16 * 16];
  const int ldsx = KC * 256 + 8;
  half_t* xsum = xs + B * ldsx;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r = lane & 15;
  const int rg = blockIdx.x;
  const int c = blockIdx.y;
  const int n_chunks = gridDim.y;
  const int sb0 = c * KC;

  const uint8_t* tbase[TW];
  bool tok[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    tok[t] = tile_valid<MODE, TW>(rg, wave, t, n_tiles, f_tiles);
    const int tl = tok[t] ? tile_of<MODE, TW>(rg, wave, t, f_tiles) : 0;   // keep addresses in bounds
    tbase[t] = W + ((size_t)tl * kb + sb0) * 2304 + (size_t)r * 144;
  }
  Q4Frag fr[P][TW];
#pragma unroll
  for (int p = 0; p < P - 1; ++p)
#pragma unroll
    for (int t = 0; t < TW; ++t) load_frag(fr[p][t], tbase[t] + (size_t)p * 2304, g);

  // ---- activations of this chunk -> LDS (fp16), with the fp32 sum of every
  // 32-value sub-block split into an fp16 hi/lo pair for the min-term MFMA.
  const int n_pieces = B * KC * 32;   // 8-value pieces
  for (int base = 0; base < n_pieces; base += 1024) {
    half8_t hv[4];
    float xfk[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (!XF32) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = base + threadIdx.x + 256 * k;
        if (idx < n_pieces) {
          const int b = idx / (KC * 32), col = idx % (KC * 32);
          hv[k] = *reinterpret_cast<const half8_t*>(reinterpret_cast<const half_t*>(Xv) + (size_t)b * ldx +
                                                    (size_t)sb0 * 256 + 8 * col);
        }
      }
    } else {
      floatx4 v[4][2];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int idx = base + threadIdx.x + 256 * k;
        if (idx < n_pieces) {
          const int b = idx / (KC * 32), col = idx % (KC * 32);
          const float* src = reinterpret_cast<const float*>(Xv) + (size_t)b * ldx + (size_t)sb0 * 256 + 8 * col;
          v[k][0] = *reinterpret_cast<const floatx4*>(src);
          v[k][1] = *reinterpret_cast<const floatx4*>(src + 4);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // the 32 pieces of one (row, super-block) are 32 consecutive threads
        const int idx = base + threadIdx.x + 256 * k;
        const int b = idx / (KC * 32), col = idx % (KC * 32);
        float am = 0.f;
        if (idx < n_pieces) {
#pragma unroll
          for (int e = 0; e < 4; ++e) am = fmaxf(am, fmaxf(fabsf(v[k][0][e]), fabsf(v[k][1][e])));
        }
        for (int o = 16; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 32));
        const int sh = f16_block_shift(am);
        const float inv = exp2i(-sh);
        xfk[k] = exp2i(sh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[k][e] = (half_t)(v[k][0][e] * inv);
          hv[k][4 + e] = (half_t)(v[k][1][e] * inv);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = base + threadIdx.x + 256 * k;
      const int b = idx / (KC * 32), col = idx % (KC * 32);
      float ps = 0.f;
      if (idx < n_pieces) {
        *reinterpret_cast<half8_t*>(xs + b * ldsx + 8 * col) = hv[k];
#pragma unroll
        for (int e = 0; e < 8; ++e) ps += (float)hv[k][e];
      }
      // a 32-value sub-block is 4 consecutive pieces = 4 consecutive threads,
      // a super-block 32 consecutive threads
      ps += __shfl_xor(ps, 1);
      ps += __shfl_xor(ps, 2);
      float ms = fabsf(ps);
      ms = fmaxf(ms, __shfl_xor(ms, 4, 32));
      ms = fmaxf(ms, __shfl_xor(ms, 8, 32));
      ms = fmaxf(ms, __shfl_xor(ms, 16, 32));
      // a super-block whose sub-block sums leave fp16's range stages them divided
      // by 32 (32 values of at most 65504 then fit); dmin is multiplied back
      const bool big = ms > 65504.f;
      const float pss = big ? ps * 0.03125f : ps;
      if (idx < n_pieces && (col & 3) == 0) {
        const int sbl = col >> 5, sub = (col & 31) >> 2;   // super-block in chunk, sub-block 0..7
        const half_t hs = (half_t)pss;
        const half_t ls = (half_t)(pss - (float)hs);
        half_t* dst = xsum + (b * KC + sbl) * 16 + 4 * (sub >> 1) + (sub & 1);
        dst[0] = hs;
        dst[2] = ls;
        if ((col & 31) == 0) {
          fac_d[sbl * 16 + b] = xfk[k];
          fac_m[sbl * 16 + b] = big ? 32.f * xfk[k] : xfk[k];
        }
      }
    }
  }
  for (int t = threadIdx.x; t < (16 - B) * KC; t += 256) {
    const int i = t / (16 - B), b = B + t % (16 - B);
    fac_d[i * 16 + b] = 1.f;
    fac_m[i * 16 + b] = 1.f;
  }
  __syncthreads();

  const NibbleMasks km = {in_vgpr(0x000F000Fu), in_vgpr(0x00F000F0u), in_vgpr(0x64006400u)};
  const int xrow = r < B ? r : B - 1;
  const half_t* xr = xs + xrow * ldsx + 64 * g;
  floatx4 acc[TW], psq[TW], psm[TW];
  float pd[TW], pdm[TW];
  floatx4 pfd = {1.f, 1.f, 1.f, 1.f}, pfm = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
  for (int t = 0; t < TW; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    // issue the loads of super-block i + P - 1 before decoding super-block i
    if (i + P - 1 < KC)
#pragma unroll
      for (int t = 0; t < TW; ++t) load_frag(fr[(i + P - 1) % P][t], tbase[t] + (size_t)(i + P - 1) * 2304, g);
    __builtin_amdgcn_sched_barrier(0);
    half8_t av[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) av[j] = *reinterpret_cast<const half8_t*>(xr + 256 * i + 8 * j);
    const half4_t axs = *reinterpret_cast<const half4_t*>(xsum + (xrow * KC + i) * 16 + 4 * g);
    const floatx4 fm = *reinterpret_cast<const floatx4*>(fac_m + i * 16 + 4 * g);
    floatx4 fd = {1.f, 1.f, 1.f, 1.f};
    if constexpr (XF32) fd = *reinterpret_cast<const floatx4*>(fac_d + i * 16 + 4 * g);
    floatx4 sq[TW], sm[TW];
    float d[TW], dm[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) q4_superblock(fr[i % P][t], av, axs, g, km, sq[t], sm[t], d[t], dm[t]);
    // accumulate the previous super-block now that its MFMAs are long done;
    // d * fd and dmin * fm are exact (the factors are powers of two)
    if (i > 0) {
#pragma unroll
      for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          acc[t][ii] = __builtin_fmaf(pd[t] * pfd[ii], psq[t][ii], __builtin_fmaf(-pdm[t] * pfm[ii], psm[t][ii], acc[t][ii]));
    }
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      psq[t] = sq[t];
      psm[t] = sm[t];
      pd[t] = d[t];
      pdm[t] = dm[t];
    }
    pfd = fd;
    pfm = fm;
  }
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      acc[t][ii] = __builtin_fmaf(pd[t] * pfd[ii], psq[t][ii], __builtin_fmaf(-pdm[t] * pfm[ii], psm[t][ii], acc[t][ii]));

  __shared__ int s_last;
  if (n_chunks > 1) {
    // write-through partial sums; the arrival counter is a relaxed device-scope
    // atomic issued after every thread's stores completed
    const int n_total = n_tiles * 16;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      if (!tok[t]) continue;
      const int n = tile_of<MODE, TW>(rg, wave, t, f_tiles) * 16 + r;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        if (b < B)
          __hip_atomic_store(&part[((size_t)c * B + b) * n_total + n], acc[t][ii], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      s_last = (__hip_atomic_fetch_add(&counters[rg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (unsigned)(n_chunks - 1));
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      if (!tok[t]) continue;
      const int n = tile_of<MODE, TW>(rg, wave, t, f_tiles) * 16 + r;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        float v = 0.f;
        if (b < B)
          for (int cc = 0; cc < n_chunks; ++cc)
            v += __hip_atomic_load(&part[((size_t)cc * B + b) * n_total + n], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        acc[t][ii] = v;
      }
    }
    if (threadIdx.x == 0) counters[rg] = 0u;
  }

  if (MODE == 0) {
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      if (!tok[t]) continue;
      const int n = tile_of<MODE, TW>(rg, wave, t, f_tiles) * 16 + r;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        if (b < B) {
          float v = acc[t][ii];
          if (residual) v += residual[(size_t)b * ldr + n];
          Y[(size_t)b * ldy + n] = v;
        }
      }
    }
  } else {
    floatx4 gv, uv;
    bool write;
    int n;
    if constexpr (TW == 2) {
      gv = acc[0];
      uv = acc[1];
      write = tok[0];
      n = tile_of<MODE, TW>(rg, wave, 0, f_tiles) * 16 + r;
    } else {
      __shared__ floatx4 fin[4][64];
      fin[wave][lane] = acc[0];
      __syncthreads();
      gv = fin[wave & 1][lane];
      uv = fin[(wave & 1) + 2][lane];
      write = wave < 2 && tok[0];
      n = tile_of<MODE, TW>(rg, wave & 1, 0, f_tiles) * 16 + r;
    }
    if (write) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        if (b < B) {
          const float z = gv[ii];
          float sil;
          if (z >= 0.f) {
            sil = z / (1.f + expf(-z));
          } else {
            const float ez = expf(z);
            sil = z * ez / (1.f + ez);
          }
          A[(size_t)b * lda + n] = sil * uv[ii];
        }
      }
    }
  }
}

// Bit-exact dequantization of blocks in storage order (test export).
__global__ void dequant_q4k_kernel(const uint8_t* __restrict__ W, int64_t n_blocks, float* __restrict__ out) {
  const int64_t blk = blockIdx.x;
  if (blk >= n_blocks) return;
  const uint8_t* p = W + blk * 144;
  const int k = threadIdx.x;  // 0..255
  const uint32_t h0 = *reinterpret_cast<const uint32_t*>(p);
  const float d = h2f(h0 & 0xffffu), dmin = h2f(h0 >> 16);
  const int sub = k >> 5;
  const int grp_i = sub >> 1;
  const uint32_t grp = (uint32_t)p[4 + 3 * grp_i] | ((uint32_t)p[5 + 3 * grp_i] << 8) | ((uint32_t)p[6 + 3 * grp_i] << 16);
  const uint32_t sc = (grp >> (6 * (sub & 1))) & 63u;
  const uint32_t m = (grp >> (12 + 6 * (sub & 1))) & 63u;
  const int word = k >> 3, rr = k & 7;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p + 16 + 4 * word);
  const uint32_t q = (w >> (16 * (rr & 1) + 4 * (rr >> 1))) & 15u;
  // d*sc and dmin*m are exact in fp32; one fused rounding of d*sc*q - dmin*m
  out[blk * 256 + k] = __builtin_fmaf(d * (float)sc, (float)q, -(dmin * (float)m));
}

// ---------------------------------------------------------------- launchers
// Tiles per wave (TW) and K chunk (KC) of one launch.  One tile per wave; KC
// is the largest divisor of kb up to 12 that keeps the staged activations
// within ~48 KB of LDS and still gives at least 192 work-groups (measured on
// MI355X for the 6144x4096, 4096x4096, 24576x4096 and 4096x12288 shapes).
struct GemmShape {
  int tw, kc;
};

static size_t lds_bytes(int B, int kc) { return (size_t)B * (kc * 256 + 8) * 2 + (size_t)B * kc * 32; }

static int64_t n_groups_of(int64_t n_tiles, int tw, bool swiglu) {
  if (swiglu) return tw == 2 ? (n_tiles / 2 + 3) / 4 : (n_tiles / 2 + 1) / 2;
  return (n_tiles + 4 * tw - 1) / (4 * tw);
}

GemmShape gemm_shape(int64_t n_tiles, int64_t kb, int B, bool swiglu) {
  static const int cands[] = {12, 8, 6, 4, 2, 1};
  const int tw = 1;
  const int64_t groups = n_groups_of(n_tiles, tw, swiglu);
  for (int kc : cands) {
    if (kb % kc) continue;
    // sized for max(B, 8) so that every batch of up to 8 sequences uses the same
    // K chunking: a sequence's outputs then do not depend on its batch-mates
    if (lds_bytes(B > 8 ? B : 8, kc) > 48 * 1024) continue;
    if (groups * (kb / kc) < 192 && kc > 1) continue;
    return {tw, kc};
  }
  return {tw, 1};
}

// The split-K arrival counters occupy a fixed area at the start of the
// workspace, so that calls of different shapes can share one workspace (each
// last arriver returns its counter to zero; the partial sums of one call then
// never land on another call's counters).
static size_t counters_bytes() { return (size_t)kGemmMaxGroups * 4; }

size_t gemm_workspace_bytes(int64_t n_rows, int64_t K, int B, bool swiglu) {
  const int64_t kb = K / 256;
  const int64_t n_tiles = n_rows / 16;
  const GemmShape gs = gemm_shape(n_tiles, kb, B, swiglu);
  const int64_t chunks = kb / gs.kc;
  size_t bytes = counters_bytes();
  if (chunks > 1) bytes += (size_t)chunks * B * n_rows * 4;
  return bytes;
}

template <int MODE, bool XF32, int TW>
static hipError_t launch_chunked(int kc, dim3 grid, size_t lds, hipStream_t st, const uint8_t* w, int n_tiles, int kb,
                                 const void* x, int64_t ldx, int B, float* Y, int64_t ldy, const float* residual,
                                 int64_t ldr, float* a, int64_t lda, int f_tiles, float* part, unsigned* counters) {
#define QK_GEMM_CASE(KC)                                                                                           \
  case KC:                                                                                                         \
    hipLaunchKernelGGL((gemm_q4k_kernel<KC, MODE, XF32, TW>), grid, dim3(256), lds, st, w, n_tiles, kb, x, ldx, B,  \
                       Y, ldy, residual, ldr, a, lda, f_tiles, part, counters);                                  \
    break;
  switch (kc) {
    QK_GEMM_CASE(1)
    QK_GEMM_CASE(2)
    QK_GEMM_CASE(4)
    QK_GEMM_CASE(6)
    QK_GEMM_CASE(8)
    QK_GEMM_CASE(12)
    QK_GEMM_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef QK_GEMM_CASE
  return hipGetLastError();
}

static void carve(void* ws, unsigned** counters, float** part) {
  char* p = reinterpret_cast<char*>(ws);
  *counters = reinterpret_cast<unsigned*>(p);
  *part = reinterpret_cast<float*>(p + counters_bytes());
}

static hipError_t gemm_run(const void* W, int64_t n_tiles, int64_t K, const void* X, bool x_f32, int64_t ldx, int B,
                           float* Y, int64_t ldy, const float* residual, int64_t ldr, float* Aout, int64_t lda,
                           bool swiglu, void* ws, hipStream_t st, GemmShape force) {
  const int kb = (int)(K / 256);
  GemmShape gs = gemm_shape(n_tiles, kb, B, swiglu);
  if (force.kc) gs = force;
  const int64_t n_groups = n_groups_of(n_tiles, gs.tw, swiglu);
  unsigned* counters;
  float* part;
  carve(ws, &counters, &part);
  const dim3 grid((unsigned)n_groups, (unsigned)(kb / gs.kc));
  const size_t lds = lds_bytes(B, gs.kc);
  const uint8_t* w = reinterpret_cast<const uint8_t*>(W);
  const int nt = (int)n_tiles, ft = (int)(n_tiles / 2);
  if (swiglu) {
    if (gs.tw == 2)
      return launch_chunked<1, false, 2>(gs.kc, grid, lds, st, w, nt, kb, X, ldx, B, nullptr, 0, nullptr, 0, Aout,
                                         lda, ft, part, counters);
    return launch_chunked<1, false, 1>(gs.kc, grid, lds, st, w, nt, kb, X, ldx, B, nullptr, 0, nullptr, 0, Aout, lda,
                                       ft, part, counters);
  }
  if (x_f32) {
    if (gs.tw == 2)
      return launch_chunked<0, true, 2>(gs.kc, grid, lds, st, w, nt, kb, X, ldx, B, Y, ldy, residual, ldr, nullptr, 0,
                                        0, part, counters);
    return launch_chunked<0, true, 1>(gs.kc, grid, lds, st, w, nt, kb, X, ldx, B, Y, ldy, residual, ldr, nullptr, 0, 0,
                                      part, counters);
  }
  if (gs.tw == 2)
    return launch_chunked<0, false, 2>(gs.kc, grid, lds, st, w, nt, kb, X, ldx, B, Y, ldy, residual, ldr, nullptr, 0,
                                       0, part, counters);
  return launch_chunked<0, false, 1>(gs.kc, grid, lds, st, w, nt, kb, X, ldx, B, Y, ldy, residual, ldr, nullptr, 0, 0,
                                     part, counters);
}

hipError_t launch_gemm_q4k(const void* W, int64_t N, int64_t K, const uint16_t* X, int64_t ldx, int B, float* Y,
                           int64_t ldy, const float* residual, int64_t ldr, void* ws, hipStream_t st, int force_tw,
                           int force_kc) {
  return gemm_run(W, N / 16, K, X, false, ldx, B, Y, ldy, residual, ldr, nullptr, 0, false, ws, st,
                  {force_tw, force_kc});
}

hipError_t launch_gemm_q4k_xf32(const void* W, int64_t N, int64_t K, const float* X, int64_t ldx, int B, float* Y,
                                int64_t ldy, const float* residual, int64_t ldr, void* ws, hipStream_t st,
                                int force_tw, int force_kc) {
  return gemm_run(W, N / 16, K, X, true, ldx, B, Y, ldy, residual, ldr, nullptr, 0, false, ws, st,
                  {force_tw, force_kc});
}

hipError_t launch_gemm_q4k_swiglu(const void* W, int64_t F, int64_t K, const uint16_t* X, int64_t ldx, int B,
                                  float* A, int64_t lda, void* ws, hipStream_t st, int force_tw, int force_kc) {
  return gemm_run(W, 2 * (F / 16), K, X, false, ldx, B, nullptr, 0, nullptr, 0, A, lda, true, ws, st,
                  {force_tw, force_kc});
}

hipError_t launch_dequant_q4k(const void* W, int64_t n_blocks, float* out, hipStream_t st) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_q4k_kernel, dim3((unsigned)n_blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint8_t*>(W), n_blocks, out);
  return hipGetLastError();
}

}  // namespace qk
