// The projections and their finishing kernels of prompt ingestion
// (qkdec_prefill), on MFMA tiles of 64 prompt tokens.
// (P1, P2, P3: the three pages listed, with their titles, at the top of include/qkdec.h.)
//
// P2 "This is the mirror image of the prefill story": unlike decode, a prompt
// has many rows per weight, so one weight read serves all of them and the
// products, not the bytes, set the pace.  A pass of up to kPfChunk tokens of
// one sequence goes through the layers at once.  Each projection is
//
//   gemm_pf_kernel   64 prompt rows (one row tile, the grid's third
//                    dimension) x 64 * NTW weight rows per work-group over a
//                    range of K super-blocks (split-K across work-groups when
//                    the rows alone do not fill the chip).
//                    The 64 x 256 fp16 activation tile of a super-block, its
//                    sub-block sums and row factors are staged in LDS once
//                    per work-group (double-buffered); each wave decodes NTW
//                    weight tiles of 16 rows exactly (sc*q, as in the decode
//                    GEMM) and runs them against the four 16-row activation
//                    tiles read from LDS.  Partial sums go to part[ks][t][n].
//   pf_finish_kernel one wave per (256 columns, prompt row): the K ranges'
//                    partial sums added in order (+ the residual, and each
//                    block's sum of squares), or the SwiGLU output rounded
//                    per 256 values with a power-of-two offset (the decode
//                    step's f16b staging) and its sub-block sums.
//   pf_norm_kernel   the same blocks: h = f16(x rinv gamma) with rinv from the
//                    row's block sums of squares, and its sub-block sums.
//
// The min term of Q4_K (dmin * m * sum x) uses the fp16 hi/lo split of each
// 32-value sub-block sum, formed once per row and super-block by the kernel
// that writes the activations.  The sums are always staged divided by 32 (a
// power of two: any sum of 32 fp16 values then fits fp16), so the factor
// that brings them back is 32 for every row and folds into -32 dmin once
// per weight row and super-block; the decode GEMM divides only the row
// super-blocks that need it (a_sums in q4k_dev.h).  A projection whose
// input has a power-of-two factor per row and super-block (the SwiGLU
// output, f16b) scales each product by it; the others (UNIT) do not.
//
// RoPE and the KV append are the decode kernels with the pass's tokens as
// rows, and the attention is launch_attn_prefill (attn_decode.hip); the
// append lands before any row attends, and row i attends over start + i + 1
// tokens.
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "q4k_dev.h"

namespace qk {

struct PfGemmArgs {
  const uint8_t* W;      // Q4_K tiles [N/16][kb][16][144]
  const half_t* X;       // [T][ldx] fp16 activations
  int64_t ldx;
  const half4_t* xs;     // [T][kb][4] sub-block sums of X / 32 (pf_block_sums)
  const float* fd;       // [T][kb] power-of-two factor of each row super-block of X (read unless UNIT)
  float* part;           // [ksplit][T][N] partial sums
  int kb, T, N, ksplit;
};

template <int NTW, bool UNIT>
__global__ void __launch_bounds__(256, 2) gemm_pf_kernel(const PfGemmArgs a) {
  // activation tile: row t's 16-byte chunk c at slot c ^ (t & 15) of the row
  // (512 bytes), so the 16 rows a read instruction touches hit 16 distinct slots
  // (two buffers as separate objects, so the compiler can tell the tile being
  // read from the one being filled and need not wait for the fill)
  __shared__ __attribute__((aligned(16))) half_t s_x0[kPfRows * 256];
  __shared__ __attribute__((aligned(16))) half_t s_x1[kPfRows * 256];
  __shared__ half4_t s_xs[2][kPfRows][4];   // sub-block sums of lane group g: hi 2g, hi 2g+1, lo 2g, lo 2g+1
  __shared__ float s_f[2][kPfRows];         // factor of each row (not UNIT)
  const int tx = threadIdx.x, lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int ks = blockIdx.y;
  const int b0 = (int)((int64_t)ks * a.kb / a.ksplit), b1 = (int)((int64_t)(ks + 1) * a.kb / a.ksplit);
  const int tile0 = (blockIdx.x * 4 + wave) * NTW;
  // rows row0 .. row0 + rows - 1 of the a.T rows
  const int row0 = kPfRows * blockIdx.z;
  const int rows = min(kPfRows, a.T - row0);

  // ---- activation staging.  The tile goes from global memory straight to LDS:
  // wave w moves rows 16 w .. 16 w + 15, two rows (1 KB) per instruction, lane
  // l filling slot l & 31 of row 2 q + (l >> 5) (rows past T repeat row T - 1,
  // whose products are never stored).  The sums of row tx >> 2, group tx & 3
  // and (tx < 64) the factor of row tx pass through registers.
  half4_t xsr;
  float fr1 = 1.f;
  auto load_x = [&](int sb, half_t* dst) {
    // the addresses are formed anew at every call (kept out of registers
    // between super-blocks)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = wave * 8 + i, row = 2 * q + (ln >> 5), slot = ln & 31;
      const int srow = row0 + (row < rows ? row : rows - 1);
      const half_t* src = a.X + (size_t)srow * a.ldx + (size_t)sb * 256 + (size_t)((slot ^ (row & 15)) * 8);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&dst[q * 512], 16, 0, 0);
    }
    const int srow = tx >> 2;
    xsr = half4_t{0, 0, 0, 0};
    if (srow < rows) xsr = a.xs[((size_t)(row0 + srow) * a.kb + sb) * 4 + (tx & 3)];
    if constexpr (!UNIT) {
      fr1 = 1.f;
      if (tx < rows) fr1 = a.fd[(size_t)(row0 + tx) * a.kb + sb];
    }
  };
  auto store_x = [&](int buf) {
    s_xs[buf][tx >> 2][tx & 3] = xsr;
    if constexpr (!UNIT)
      if (tx < kPfRows) s_f[buf][tx] = fr1;
  };
  // every wave's tile loads have landed in LDS before the barrier that
  // publishes them (vmcnt(0); expcnt and lgkmcnt left at their maxima)
  auto wait_loads = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };

  auto wsrc = [&](int tt, int sb) { return a.W + ((size_t)(tile0 + tt) * a.kb + sb) * 2304 + (size_t)r * 144; };
  const NibbleMasks km = {in_vgpr(0x000F000Fu), in_vgpr(0x00F000F0u), in_vgpr(0x64006400u)};
  floatx4 acc[NTW][4];
#pragma unroll
  for (int tt = 0; tt < NTW; ++tt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[tt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  Q4Frag fr[NTW], fn[NTW];
  load_x(b0, s_x0);
#pragma unroll
  for (int tt = 0; tt < NTW; ++tt) load_frag(fn[tt], wsrc(tt, b0), g);
  store_x(0);
  wait_loads();
  __syncthreads();
  // one super-block: multiply the tile in buffer BUF while the next one is
  // loaded into the other
  auto step = [&](auto bufc, int sb) {
    constexpr int BUF = decltype(bufc)::value;
    half_t* const cur = BUF == 0 ? s_x0 : s_x1;
    half_t* const nxt = BUF == 0 ? s_x1 : s_x0;
    const bool more = sb + 1 < b1;
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) fr[tt] = fn[tt];
    if (more) {
      load_x(sb + 1, nxt);
#pragma unroll
      for (int tt = 0; tt < NTW; ++tt) load_frag(fn[tt], wsrc(tt, sb + 1), g);
    }
    float d[NTW], dm[NTW];
    half4_t bm[NTW];
    half8_t bq[NTW][8];
#pragma unroll
    for (int tt = 0; tt < NTW; ++tt) {
      const Q4Header h = q4_header(fr[tt], g);
      d[tt] = h.d;
      dm[tt] = -32.f * h.dmin;   // the sums are staged divided by 32
      const half2_t mm = pack_h2(h.m0, h.m1);
      bm[tt][0] = mm[0]; bm[tt][1] = mm[1]; bm[tt][2] = mm[0]; bm[tt][3] = mm[1];
#pragma unroll
      for (int j = 0; j < 8; ++j) bq[tt][j] = q4_word(fr[tt], h, j, km);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const half_t* xs = &cur[(mt * 16 + r) * 256];
      half8_t av[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) av[j] = *reinterpret_cast<const half8_t*>(xs + ((8 * g + j) ^ r) * 8);
      const half4_t axs = s_xs[BUF][mt * 16 + r][g];
      float fd[4];
      if constexpr (!UNIT)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) fd[ii] = s_f[BUF][mt * 16 + 4 * g + ii];
      const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < NTW; ++tt) {
        const floatx4 sm = __builtin_amdgcn_mfma_f32_16x16x16f16(axs, bm[tt], zero, 0, 0, 0);
        floatx4 sq = zero;
#pragma unroll
        for (int j = 0; j < 8; ++j) sq = mfma16x16x32(av[j], bq[tt][j], sq);
        // d * fd and -32 dmin * fd are exact (the factors are powers of two)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          if constexpr (UNIT)
            acc[tt][mt][ii] = __builtin_fmaf(d[tt], sq[ii], __builtin_fmaf(dm[tt], sm[ii], acc[tt][mt][ii]));
          else
            acc[tt][mt][ii] =
                __builtin_fmaf(d[tt] * fd[ii], sq[ii], __builtin_fmaf(dm[tt] * fd[ii], sm[ii], acc[tt][mt][ii]));
        }
      }
    }
    if (more) store_x(BUF ^ 1);
    wait_loads();
    __syncthreads();
  };
  for (int sb = b0;;) {
    step(std::integral_constant<int, 0>{}, sb);
    if (++sb >= b1) break;
    step(std::integral_constant<int, 1>{}, sb);
    if (++sb >= b1) break;
  }

  // lane (g, r) holds rows mt * 16 + 4g + ii of output column 16 tile + r
  float* dst = a.part + (size_t)ks * a.T * a.N;
#pragma unroll
  for (int tt = 0; tt < NTW; ++tt) {
    const int n = (tile0 + tt) * 16 + r;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int t = mt * 16 + 4 * g + ii;
        if (t < rows) dst[(size_t)(row0 + t) * a.N + n] = acc[tt][mt][ii];
      }
  }
}

// ---- finish of a projection and staging of the next one's input: one
// wave per 256-column block c of row t (lane l owns columns 256 c + 4 l ..
// + 3), four blocks per work-group; no barriers.
constexpr int kPfBlocksPerGroup = 4;

// The staged fp16 values hv of this lane (super-block c of row t): the
// 32-value sub-block sums of the block (fp32 over the fp16 values, 8 lanes
// each) divided by 32, as hi/lo fp16 pairs per lane group g of the GEMM, and
// the block's factor fd.
__device__ void pf_block_sums(const half_t (&hv)[4], float fd, int kb, int t, int c, half4_t* xs, float* fdv,
                              int lane) {
  float s = (((float)hv[0] + (float)hv[1]) + (float)hv[2]) + (float)hv[3];
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);                // lanes 8 j ..: sub-block j = lane >> 3
  const float s1 = __shfl_xor(s, 8);    // at lane 16 g: sub-block 2 g + 1
  if ((lane & 15) == 0) {
    const float a0 = s * 0.03125f, a1 = s1 * 0.03125f;
    const half_t h0 = (half_t)a0, h1 = (half_t)a1;
    half4_t q;
    q[0] = h0; q[1] = h1; q[2] = (half_t)(a0 - (float)h0); q[3] = (half_t)(a1 - (float)h1);
    xs[((size_t)t * kb + c) * 4 + (lane >> 4)] = q;
  }
  if (lane == 0) fdv[(size_t)t * kb + c] = fd;
}

struct PfFinishArgs {
  const float* part;     // [ksplit][T][N] (ksplit may be 0)
  int ksplit, T, N;
  const float* res;      // [T][ldo] added to the sums, or null (may alias out)
  float* out;            // kPfOut, kPfNorm: [T][ldo]
  int64_t ldo;
  int mode;
  float* ssq;            // kPfNorm: [T][N / 256] sum of squares of each block of out
  half_t* h;             // kPfSwiglu: [T][N / 2] fp16 input of the down projection
  half4_t* xs;           // and its sums and factors (pf_block_sums)
  float* fd;
};

__global__ void __launch_bounds__(256) pf_finish_kernel(const PfFinishArgs a) {
  const int tx = threadIdx.x, lane = tx & 63, wave = tx >> 6;
  const int c = blockIdx.x * kPfBlocksPerGroup + wave, t = blockIdx.y;
  const size_t plane = (size_t)a.T * a.N;
  const float* pr = a.part + (size_t)t * a.N;
  auto psum = [&](int k) {
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < a.ksplit; ++q) s += *reinterpret_cast<const floatx4*>(pr + q * plane + k);
    return s;
  };
  if (a.mode == kPfSwiglu) {
    // gate in columns [0, F), up in [F, 2F); silu(gate) * up rounded to fp16
    // with the smallest power-of-two offset that keeps the block finite
    const int F = a.N / 2;
    if (c >= F / 256) return;
    const int k = c * 256 + 4 * lane;
    const floatx4 z = psum(k), u = psum(F + k);
    float v[4], am = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sil;
      if (z[i] >= 0.f) {
        sil = z[i] / (1.f + expf(-z[i]));
      } else {
        const float ez = expf(z[i]);
        sil = z[i] * ez / (1.f + ez);
      }
      v[i] = sil * u[i];
      am = fmaxf(am, fabsf(v[i]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
    const int sh = f16_block_shift(am);
    const float inv = exp2i(-sh);
    half_t hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = (half_t)(v[i] * inv);
    half4_t h4;
    h4[0] = hv[0]; h4[1] = hv[1]; h4[2] = hv[2]; h4[3] = hv[3];
    *reinterpret_cast<half4_t*>(a.h + (size_t)t * F + k) = h4;
    pf_block_sums(hv, exp2i(sh), F / 256, t, c, a.xs, a.fd, lane);
    return;
  }
  if (c >= (a.N + 255) / 256) return;
  const int k = c * 256 + 4 * lane;
  float q = 0.f;
  if (k < a.N) {   // kPfOut only: kPfNorm widths are whole blocks
    floatx4 y = psum(k);
    if (a.res) y += *reinterpret_cast<const floatx4*>(a.res + (size_t)t * a.ldo + k);
    *reinterpret_cast<floatx4*>(a.out + (size_t)t * a.ldo + k) = y;
    q = ((y[0] * y[0] + y[1] * y[1]) + y[2] * y[2]) + y[3] * y[3];
  }
  if (a.mode != kPfNorm) return;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) q += __shfl_xor(q, o);
  if (lane == 0) a.ssq[(size_t)t * (a.N / 256) + c] = q;
}

// h = f16(x rinv gamma) for block c of row t, rinv from the row's block sums
// of squares; then its sub-block sums.  x = null: h is already staged (the
// attention output), only the sums are formed.
__global__ void __launch_bounds__(256) pf_norm_kernel(const float* __restrict__ x, const float* __restrict__ ssq,
                                                      const float* __restrict__ gamma, float eps, int K, half_t* h,
                                                      half4_t* xs, float* fdv) {
  const int tx = threadIdx.x, lane = tx & 63, wave = tx >> 6;
  const int c = blockIdx.x * kPfBlocksPerGroup + wave, t = blockIdx.y, nb = K / 256;
  if (c >= nb) return;
  const int k = c * 256 + 4 * lane;
  half_t hv[4];
  if (x) {
    float tot = 0.f;
    for (int b = lane; b < nb; b += 64) tot += ssq[(size_t)t * nb + b];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
    const float rinv = 1.0f / sqrtf(tot * (1.0f / (float)K) + eps);
    const floatx4 xv = *reinterpret_cast<const floatx4*>(x + (size_t)t * K + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = norm_apply(xv[i], rinv, gamma[k + i]);
    half4_t h4;
    h4[0] = hv[0]; h4[1] = hv[1]; h4[2] = hv[2]; h4[3] = hv[3];
    *reinterpret_cast<half4_t*>(h + (size_t)t * K + k) = h4;
  } else {
    const half4_t h4 = *reinterpret_cast<const half4_t*>(h + (size_t)t * K + k);
    hv[0] = h4[0]; hv[1] = h4[1]; hv[2] = h4[2]; hv[3] = h4[3];
  }
  pf_block_sums(hv, 1.f, nb, t, c, xs, fdv, lane);
}

int pf_ksplit(int64_t n_rows, int64_t K, int T) {
  const int64_t groups = n_rows / (16 * 4 * kPfTilesPerWave) * ((T + kPfRows - 1) / kPfRows);
  const int kb = (int)(K / 256);
  int64_t s = (kPfTargetGroups + groups - 1) / groups;
  if (s > kb) s = kb;
  return s < 1 ? 1 : (int)s;
}

hipError_t launch_gemm_pf(const void* W, int64_t n_rows, int64_t K, const uint16_t* X, int64_t ldx, const void* xs,
                          const float* fd, int T, float* part, int ksplit, hipStream_t st) {
  if (n_rows % (64 * kPfTilesPerWave) != 0 || K % 256 != 0 || T < 1 || T > kPfChunk || ksplit < 1 ||
      ksplit > K / 256)
    return hipErrorInvalidValue;
  PfGemmArgs a{};
  a.W = reinterpret_cast<const uint8_t*>(W);
  a.X = reinterpret_cast<const half_t*>(X);
  a.ldx = ldx;
  a.xs = reinterpret_cast<const half4_t*>(xs);
  a.fd = fd;
  a.part = part;
  a.kb = (int)(K / 256);
  a.T = T;
  a.N = (int)n_rows;
  a.ksplit = ksplit;
  const dim3 grid((unsigned)(n_rows / (64 * kPfTilesPerWave)), (unsigned)ksplit, (unsigned)((T + kPfRows - 1) / kPfRows));
  if (fd)
    hipLaunchKernelGGL((gemm_pf_kernel<kPfTilesPerWave, false>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_pf_kernel<kPfTilesPerWave, true>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pf_finish(const float* part, int ksplit, int T, int N, const float* res, float* out, int64_t ldo,
                            int mode, float* ssq, uint16_t* h, void* xs, float* fd, hipStream_t st) {
  if (T < 1 || T > kPfChunk || N < 1 || ksplit < 0 || (mode == kPfNorm && N % 256 != 0) ||
      (mode == kPfSwiglu && N % 512 != 0))
    return hipErrorInvalidValue;
  PfFinishArgs a{};
  a.part = part;
  a.ksplit = ksplit;
  a.T = T;
  a.N = N;
  a.res = res;
  a.out = out;
  a.ldo = ldo;
  a.mode = mode;
  a.ssq = ssq;
  a.h = reinterpret_cast<half_t*>(h);
  a.xs = reinterpret_cast<half4_t*>(xs);
  a.fd = fd;
  const int blocks = mode == kPfSwiglu ? N / 512 : (N + 255) / 256;
  hipLaunchKernelGGL(pf_finish_kernel, dim3((blocks + kPfBlocksPerGroup - 1) / kPfBlocksPerGroup, T), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_pf_norm(const float* x, const float* ssq, const float* gamma, float eps, int K, int T, uint16_t* h,
                          void* xs, float* fd, hipStream_t st) {
  if (T < 1 || T > kPfChunk || K < 256 || K % 256 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pf_norm_kernel, dim3((K / 256 + kPfBlocksPerGroup - 1) / kPfBlocksPerGroup, T), dim3(256), 0,
                     st, x, ssq, gamma, eps, K,
                     reinterpret_cast<half_t*>(h), reinterpret_cast<half4_t*>(xs), fd);
  return hipGetLastError();
}

}  // namespace qk
