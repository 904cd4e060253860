// Q4_K dequant-GEMM with K split over the waves of one work-group: the decode
// step's projections.
// (P1, P2, P3: the three pages listed, with their titles, at the top of include/qkdec.h.)
//
// P1 "The weight read is the only term that does not scale": every weight is
// read once per step and multiplied against all B sequences' hidden states.
// P1 "RDNA4 pads the batch dimension to 16 whether you fill it or not": the
// sequences are the 16 rows of the matrix-core tile (v_mfma_f32_16x16x32_f16,
// A = activations, B = decoded weights; the exact decode and the min-term MFMA
// are those of gemm_q4k.hip, in q4k_dev.h).
//
// Work decomposition.  One work-group computes one output item: a tile of 16
// weight rows (MODE 0), or the gate tile and the up tile of 16 SwiGLU outputs
// (MODE 1).  Its S waves split the item's K super-blocks into S contiguous
// ranges; their partial sums are added in LDS in wave order.  No item is split
// across work-groups, so a launch needs no workspace, no arrival counters and
// no second pass: the latency from the last weight load to the stored output
// is one LDS exchange.  The price is that every work-group reads the whole
// activation vector, from L2 (it was written by an earlier launch).
//
// Activations are built per wave and per super-block directly in the MFMA A
// layout: lane (g, r) needs x[r][256 sb + 64 g .. + 63], i.e. 64 consecutive
// values of one sequence row, which cover its two 32-value sub-blocks 2g and
// 2g+1 (so the min-term sums need no exchange).  Modes:
//   kXF16        fp16 activations as they are;
//   kXNorm       fp32 residual-stream rows, RMSNorm applied on the fly
//                (statistics folded once per work-group from the 16-column
//                sum-of-squares slots);
//   kXF32Blocked fp32 rows rounded to fp16 with one power-of-two offset per row
//                and super-block (the offset is a factor of d and dmin).
#include "common.h"
#include "internal.h"
#include "kv_dev.h"
#include "q4k_dev.h"

namespace qk {

struct WkArgs {
  const uint8_t* W;
  const void* X;         // [B][ldx] fp16 (kXF16) or fp32
  const float* gamma;    // kXNorm: gains of the K inputs
  const float* ss_in;    // kXNorm: 16-column sum-of-squares slots of the rows of X
  float* Y;              // MODE 0 output (may alias residual)
  const float* residual;
  float* ss_out;         // MODE 0: slot of each output tile, or null
  float* A;              // MODE 1 output
  int64_t ldx, ldy, ldr, lda;
  int kb, B, f_tiles, ss_slots;
  float eps, inv_k;
  RopeAppendArgs ra;     // MODE 2 (gemm_wi_kernel): QKV finish, fp16 cache
  int qh;                // MODE 2: tiles per half head (head_dim / 32)
  float* part;           // K split over work-groups (gemm_wi_kernel): partial sums [chunk][B][N]
  unsigned* counters;    // ... and one arrival counter per row group (zero between launches)
};

// The A operand of super-block sb for lane (g, r): av (8 MFMA pieces), the
// hi/lo sub-block sums axs, and this row's factors of d (fdr) and dmin (fmr).
template <int XMODE>
__device__ __forceinline__ void build_a(const WkArgs& a, int sb, int g, int r, float rinv, half8_t (&av)[8],
                                        half4_t& axs, float& fdr, float& fmr) {
  const bool live = r < a.B;
  const size_t k0 = (size_t)sb * 256 + 64 * g;
  fdr = 1.f;
  if constexpr (XMODE == kXF16) {
    const half_t* src = reinterpret_cast<const half_t*>(a.X) + (size_t)r * a.ldx + k0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      half8_t v = {};
      if (live) v = *reinterpret_cast<const half8_t*>(src + 8 * j);
      av[j] = v;
    }
  } else if constexpr (XMODE == kXNorm) {
    const float* src = reinterpret_cast<const float*>(a.X) + (size_t)r * a.ldx + k0;
    const float* gm = a.gamma + k0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // two halves of 32 values keep fewer registers in flight
      floatx4 xv[8], gv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        xv[q] = live ? *reinterpret_cast<const floatx4*>(src + 32 * h + 4 * q) : floatx4{0.f, 0.f, 0.f, 0.f};
        gv[q] = *reinterpret_cast<const floatx4*>(gm + 32 * h + 4 * q);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = norm_apply(xv[2 * j + e / 4][e % 4], rinv, gv[2 * j + e / 4][e % 4]);
        av[4 * h + j] = v;
      }
    }
  } else {
    const float* src = reinterpret_cast<const float*>(a.X) + (size_t)r * a.ldx + k0;
    floatx4 xv[16];
    float am = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      xv[q] = live ? *reinterpret_cast<const floatx4*>(src + 4 * q) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) am = fmaxf(am, fabsf(xv[q][e]));
    }
    // the row's 256 values of this super-block are held by lanes r, r+16, r+32, r+48
    am = fmaxf(am, __shfl_xor(am, 16));
    am = fmaxf(am, __shfl_xor(am, 32));
    const int sh = f16_block_shift(am);
    const float inv = exp2i(-sh);
    fdr = exp2i(sh);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      half8_t v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (half_t)(xv[2 * j + e / 4][e % 4] * inv);
      av[j] = v;
    }
  }
  a_sums(av, fdr, axs, fmr);
}

// Waves per SIMD: fp16 activations fit 128 registers (four waves per SIMD);
// fp32 activations (64 values, and 64 gains for the RMSNorm, per lane and
// super-block in flight) take up to 256 (two waves per SIMD).
template <int XMODE>
constexpr int wk_waves_per_simd() {
  return XMODE == kXF16 ? 4 : 2;
}

template <int MODE, int XMODE, int S, int P>
__global__ void __launch_bounds__(64 * S, wk_waves_per_simd<XMODE>()) gemm_wk_kernel(const WkArgs a) {
  constexpr int T = MODE == 1 ? 2 : 1;   // weight tiles per item
  __shared__ floatx4 red[S][T][64];
  __shared__ float s_part[4 * S][16];
  __shared__ float s_rinv[16];
  const int item = blockIdx.x;
  const int tx = threadIdx.x, lane = tx & 63, wave = tx >> 6, g = lane >> 4, r = lane & 15;
  const int kb = a.kb;
  const int sb_begin = wave * kb / S, sb_end = (wave + 1) * kb / S;
  const int nsb = sb_end - sb_begin;
  int tile[T];
  tile[0] = item;
  if constexpr (T == 2) tile[1] = item + a.f_tiles;
  auto wptr = [&](int tt, int sb) { return a.W + ((size_t)tile[tt] * kb + sb) * 2304 + (size_t)r * 144; };

  // ---- weights of the first P super-blocks, then the row statistics
  Q4Frag fr[P][T];
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < nsb)
#pragma unroll
      for (int tt = 0; tt < T; ++tt) load_frag(fr[p][tt], wptr(tt, sb_begin + p), g);
  float rinv = 1.f;
  if constexpr (XMODE == kXNorm) {
    // thread (j, b) adds slots j, j + 4S, ... of row b; then 16 threads add the
    // 4S parts in order
    const int b = tx & 15, j = tx >> 4;
    float p = 0.f;
    for (int s = j; s < a.ss_slots; s += 4 * S) p += a.ss_in[(size_t)s * 16 + b];
    s_part[j][b] = p;
    __syncthreads();
    if (tx < 16) {
      float tot = 0.f;
      for (int k = 0; k < 4 * S; ++k) tot += s_part[k][tx];
      s_rinv[tx] = 1.0f / sqrtf(tot * a.inv_k + a.eps);
    }
    __syncthreads();
    rinv = r < a.B ? s_rinv[r] : 0.f;   // rows past B stay zero
  }

  // the residual of wave 0's outputs, loaded now rather than after the sum
  float resv[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (MODE == 0) {
    if (wave == 0 && a.residual) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        if (b < a.B) resv[ii] = a.residual[(size_t)b * a.ldr + item * 16 + r];
      }
    }
  }

  // ---- main loop: one super-block per step, P weight loads in flight
  const NibbleMasks km = {in_vgpr(0x000F000Fu), in_vgpr(0x00F000F0u), in_vgpr(0x64006400u)};
  floatx4 acc[T];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) acc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < nsb; i0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int i = i0 + p;
      // one super-block at a time: its activation loads are not hoisted into
      // the previous step (they would need another 32-64 registers)
      __builtin_amdgcn_sched_barrier(0);
      if (i < nsb) {
        half8_t av[8];
        half4_t axs;
        float fdr, fmr;
        build_a<XMODE>(a, sb_begin + i, g, r, rinv, av, axs, fdr, fmr);
        // factors of the D rows 4g + ii come from lanes 4g + ii (g = 0)
        floatx4 fd, fm;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          fd[ii] = __shfl(fdr, 4 * g + ii);
          fm[ii] = __shfl(fmr, 4 * g + ii);
        }
#pragma unroll
        for (int tt = 0; tt < T; ++tt) {
          floatx4 sq, sm;
          float d, dm;
          q4_superblock(fr[p][tt], av, axs, g, km, sq, sm, d, dm);
          if (i + P < nsb) load_frag(fr[p][tt], wptr(tt, sb_begin + i + P), g);
          // d * fd and dmin * fm are exact (the factors are powers of two)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            acc[tt][ii] = __builtin_fmaf(d * fd[ii], sq[ii], __builtin_fmaf(-dm * fm[ii], sm[ii], acc[tt][ii]));
        }
      }
    }
  }

  // ---- the S partial sums, added in wave order by wave 0
#pragma unroll
  for (int tt = 0; tt < T; ++tt) red[wave][tt][lane] = acc[tt];
  __syncthreads();
  if (wave != 0) return;
  floatx4 v[T];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    v[tt] = red[0][tt][lane];
#pragma unroll
    for (int w = 1; w < S; ++w) v[tt] += red[w][tt][lane];
  }
  // lane (g, r) holds outputs (sequence 4g + ii, row 16 item + r)
  const int n = item * 16 + r;
  if constexpr (MODE == 0) {
    float sq[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii;
      float y = v[0][ii];
      if (b < a.B) {
        if (a.residual) y += resv[ii];
        a.Y[(size_t)b * a.ldy + n] = y;
      }
      sq[ii] = b < a.B ? y * y : 0.f;
    }
    if (a.ss_out) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        float t = sq[ii];
        t += __shfl_xor(t, 1);
        t += __shfl_xor(t, 2);
        t += __shfl_xor(t, 4);
        t += __shfl_xor(t, 8);
        if (r == 0) a.ss_out[(size_t)item * 16 + 4 * g + ii] = t;
      }
    }
  } else {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii;
      if (b < a.B) {
        const float z = v[0][ii];
        float sil;
        if (z >= 0.f) {
          sil = z / (1.f + expf(-z));
        } else {
          const float ez = expf(z);
          sil = z * ez / (1.f + ez);
        }
        a.A[(size_t)b * a.lda + n] = sil * v[1][ii];
      }
    }
  }
}

// MODE 2 finish of gemm_wi_kernel (all waves call it after the partial sums
// are in LDS): waves 0 and 1 add the partial sums of tiles hj and hj + D/32 of
// the head, store the fp32 rows, exchange them for the rotation, then store q
// as fp16 and append k, v to an fp16 or E4M3 cache, or stage a Q8_0 part.
template <int S, typename Red>
__device__ void qkv_finish(const WkArgs& a, Red red, int wave, int lane, int g, int r, int head, int hj,
                           const int (&sl)[4], const int (&ps)[4], const float2* s_rope) {
  __shared__ floatx4 s_fin[2][64];
  const RopeAppendArgs& ra = a.ra;
  const int D = 32 * a.qh, HALF = D / 2;
  floatx4 v = {0.f, 0.f, 0.f, 0.f};
  if (wave < 2) {
    v = red[wave][0][0][lane];
#pragma unroll
    for (int w = 1; w < S; ++w) v += red[wave][0][w][lane];
    const int n = (head * 2 * a.qh + hj + a.qh * wave) * 16 + r;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      if (4 * g + ii < a.B) a.Y[(size_t)(4 * g + ii) * a.ldy + n] = v[ii];
    s_fin[wave][lane] = v;
  }
  __syncthreads();
  if (wave >= 2) return;
  const bool is_q = head < ra.Hq, is_v = head >= ra.Hq + ra.n_kv;
  const int d = 16 * (hj + a.qh * wave) + r;   // dim within the head
  float out[4];
  if (!is_v) {
    const floatx4 other = s_fin[wave ^ 1][lane];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii < a.B ? 4 * g + ii : 0;
      const float2 c = s_rope[b * 16 + r];
      // d < D/2: x_i cos - x_{i+D/2} sin; d >= D/2: x_{i+D/2} cos + x_i sin
      out[ii] = d < HALF ? v[ii] * c.x - other[ii] * c.y : v[ii] * c.x + other[ii] * c.y;
    }
  } else {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) out[ii] = v[ii];
  }
  if (is_q) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii;
      if (b < a.B) ra.q16[((size_t)b * ra.Hq + head) * D + d] = f2h_bits(out[ii]);
    }
    return;
  }
  CacheRef c;
  c.k = ra.k; c.v = ra.v; c.ks = ra.ks; c.vs = ra.vs;
  c.n_kv = ra.n_kv; c.cap = ra.cap; c.D = D; c.n_slots = ra.n_slots; c.kf = ra.kf; c.vf = ra.vf;
  const int kvh = is_v ? head - ra.Hq - ra.n_kv : head - ra.Hq;
  // with a Q8_0 part (kv_new set) both parts are staged for the attention
  // kernel, which quantizes and stores the Q8_0 one (its 32-dim blocks span
  // two work-groups here); an fp16 part is stored here as well
  const bool q8 = (is_v ? ra.vf : ra.kf) == kFmtQ8;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int b = 4 * g + ii;
    if (b >= a.B) continue;
    const bool ok = sl[ii] >= 0 && sl[ii] < ra.n_slots && ps[ii] >= 0 && ps[ii] < ra.cap;
    if (ra.kv_new) ra.kv_new[(((size_t)b * 2 + (is_v ? 1 : 0)) * ra.n_kv + kvh) * D + d] = out[ii];
    if (ok && !q8) store_point(c, is_v, sl[ii], kvh, ps[ii], d, out[ii]);
    if (!ok && r == 0) *ra.err = QKDEC_E_CAPACITY;
  }
}

// Several output items per work-group.  Wave w owns super-blocks
// [KW w, KW w + KW) of K (kb = S * KW) for every item, so it builds the A
// operands of its K slice once and keeps them in registers; the weights of
// PD items are in flight at a time, issued before anything else.  Each item's
// S partial sums go to LDS; after one barrier wave i adds item i's partials in
// wave order and finishes it (no split-K round trips, no workspace).  With
// IPW items per work-group a launch of ceil(items / IPW) work-groups can be
// resident on the chip at once.
// MODE 2 (the QKV projection of a decode step): a work-group owns tiles j and
// j + D/32 of one head (dims 16 j + r and 16 j + r + D/2, the rotate-half
// pairs), so it finishes the head slice itself: the fp32 rows go to Y, q and
// k are rotated at pos, q is stored as fp16 and k, v are appended (fp16 or
// E4M3) or staged for the attention kernel (Q8_0).
// KSPLIT > 1 (MODE 0): K is cut into KSPLIT chunks of S KW super-blocks;
// work-group i takes chunk i / (grid / KSPLIT), and the last of a tile's
// chunks to arrive adds the chunks' partial sums in chunk order.
// MV > 0 (the small-batch matvec, B = MV <= 2 sequences): the same items,
// staging and finishes, with each super-block's products formed on the vector
// ALU (q4_superblock_mv) for the live sequences only instead of on the
// matrix cores for a tile padded to 16; lane (g, r) then holds the sums of
// row r over its K slice for every sequence, which two lane exchanges add
// over g and which are laid out as the MFMA's results for the finish.
template <int MODE, int XMODE, int S, int KW, int IPW, int PD, int KSPLIT = 1, int MV = 0>
__global__ void __launch_bounds__(64 * S, 1) gemm_wi_kernel(const WkArgs a) {
  constexpr int T = MODE == 1 ? 2 : 1;   // weight tiles per item
  static_assert(KSPLIT == 1 || MODE == 0, "K split: plain outputs only");
  static_assert(MV >= 0 && MV <= 2, "matvec: one or two sequences");
  constexpr int NM = MV > 0 ? MV : 1;
  static_assert(IPW <= S && PD <= IPW, "one finishing wave per item");
  static_assert(MODE != 2 || (IPW == 2 && XMODE == kXNorm), "QKV finish: a tile pair, RMSNorm fused");
  // LDS: kXNorm first holds the normalized activations h [16][K + 8] (fp16),
  // then, after a barrier, the partial sums red[IPW][T][S][64]
  constexpr size_t kRedBytes = sizeof(floatx4) * IPW * T * S * 64;
  constexpr size_t kHBytes = XMODE != kXF16 ? (size_t)16 * (S * KW * 256 + 8) * 2 : 0;
  __shared__ __align__(16) char smem[kRedBytes > kHBytes ? kRedBytes : kHBytes];
  auto red = reinterpret_cast<floatx4(*)[T][S][64]>(smem);
  __shared__ float s_part[4 * S][16];
  __shared__ float s_rinv[16];
  // the wave index as a wave-uniform value (scalar registers, uniform branches)
  const int tx = threadIdx.x, lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int kb = a.kb;
  const int n_groups = (int)gridDim.x / KSPLIT;
  const int kc = KSPLIT > 1 ? (int)blockIdx.x / n_groups : 0;   // K chunk
  const int item0 = (KSPLIT > 1 ? (int)blockIdx.x % n_groups : (int)blockIdx.x) * IPW;
  const int n_items = MODE == 2 ? 2 : (a.f_tiles - item0 < IPW ? a.f_tiles - item0 : IPW);
  // MODE 2: head and half-head tile of this work-group
  const int head = MODE == 2 ? (int)blockIdx.x / a.qh : 0, hj = MODE == 2 ? (int)blockIdx.x % a.qh : 0;
  auto tile_of_item = [&](int it) {
    if constexpr (MODE == 2) return head * 2 * a.qh + hj + a.qh * it;
    return item0 + (it < n_items ? it : n_items - 1);
  };
  const int sbl = wave * KW;                 // first super-block of this wave in the chunk
  const int sb0 = kc * S * KW + sbl;         // ... in the row
  // items past the launch's last one read the last one's weights again: every
  // weight load is unconditional, so the compiler's in-order load counting
  // never has to assume a shorter path and wait for the whole stream
  auto wptr = [&](int it, int tt, int sb) {
    const int tile = tile_of_item(it) + (tt ? a.f_tiles : 0);
    return a.W + ((size_t)tile * kb + sb) * 2304 + (size_t)r * 144;
  };

  // Vector memory loads return in order, so everything small that the
  // prologue waits on (RMSNorm statistics, gains, activations) is issued
  // before the weight stream: waiting on it never waits on the weights.
  constexpr int K = S * KW * 256, LDH = K + 8;   // K of one chunk
  const int cbase = kc * (K / 4);                // the chunk's first float4 column
  half8_t av[KW][8];
  half4_t axs[KW];
  floatx4 fd[KW], fm[KW];
  // MV: the K slice's activations of every sequence (lane (g, r): values
  // 64g..64g+63 of each super-block), their sub-block sums and d factors
  half8_t xm[KW][NM][8];
  float xs[KW][NM][2], fdm[KW][NM];
  // sums of the two sub-blocks (pieces 0..3, 4..7) of one row's 64 values
  auto mv_sums = [&](int p, int b) {
    const half2_t one = {(half_t)1.f, (half_t)1.f};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        s0 = __builtin_amdgcn_fdot2(half2_t{xm[p][b][j][e], xm[p][b][j][e + 1]}, one, s0, false);
        s1 = __builtin_amdgcn_fdot2(half2_t{xm[p][b][4 + j][e], xm[p][b][4 + j][e + 1]}, one, s1, false);
      }
    xs[p][b][0] = s0;
    xs[p][b][1] = s1;
  };
  // kXNorm: slots of the sum-of-squares fold, gains and x rows 0..7 of the
  // thread's float4 columns tx + 64 S c (c < KW)
  SsFold<64 * S, (XMODE == kXNorm ? K / kSsCols : 0)> ssf;   // the K inputs have K / 16 slots
  floatx4 gv[XMODE == kXNorm ? KW : 1], xv[XMODE != kXF16 ? KW : 1][8];
  const float* X32 = reinterpret_cast<const float*>(a.X);
  if constexpr (XMODE == kXNorm) {
    ssf.load(a.ss_in, a.ss_slots);
#pragma unroll
    for (int c = 0; c < KW; ++c) {
      const int c4 = tx + 64 * S * c;
      gv[c] = *reinterpret_cast<const floatx4*>(a.gamma + 4 * c4);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int bb = u < a.B ? u : a.B - 1;
        xv[c][u] = *reinterpret_cast<const floatx4*>(X32 + (size_t)bb * a.ldx + 4 * c4);
      }
    }
  } else if constexpr (XMODE == kXF32Blocked) {
#pragma unroll
    for (int c = 0; c < KW; ++c) {
      const int c4 = cbase + tx + 64 * S * c;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int bb = u < a.B ? u : a.B - 1;
        xv[c][u] = *reinterpret_cast<const floatx4*>(X32 + (size_t)bb * a.ldx + 4 * c4);
      }
    }
  } else if constexpr (XMODE == kXF16) {
    const half_t* X16 = reinterpret_cast<const half_t*>(a.X);
    if constexpr (MV > 0) {
#pragma unroll
      for (int p = 0; p < KW; ++p)
#pragma unroll
        for (int b = 0; b < MV; ++b)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            xm[p][b][j] =
                *reinterpret_cast<const half8_t*>(X16 + (size_t)b * a.ldx + (sb0 + p) * 256 + 64 * g + 8 * j);
    } else {
      const int rr = r < a.B ? r : a.B - 1;
#pragma unroll
      for (int p = 0; p < KW; ++p)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          av[p][j] = *reinterpret_cast<const half8_t*>(X16 + (size_t)rr * a.ldx + (sb0 + p) * 256 + 64 * g + 8 * j);
    }
  }
  // MODE 2: slot and position of the lane's rows 4g + ii, and of row tx / 16
  // for the rotary table
  int sl[4] = {0, 0, 0, 0}, ps[4] = {0, 0, 0, 0}, pos_t = 0;
  if constexpr (MODE == 2) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii < a.B ? 4 * g + ii : a.B - 1;
      sl[ii] = a.ra.slot[b];
      ps[ii] = a.ra.spos[b];
    }
    pos_t = (tx >> 4) < a.B ? (tx >> 4) : a.B - 1;   // the row whose rotary pair this thread stages
  }
  // the residual of the item this wave finishes
  float resv[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (MODE == 0) {
    // unconditional (no branch around a load): a missing residual reads Y and
    // is replaced by zero
    const float* rp = a.residual ? a.residual : a.Y;
    const int64_t ld = a.residual ? a.ldr : a.ldy;
    const int it = wave < n_items ? wave : n_items - 1;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii < a.B ? 4 * g + ii : a.B - 1;
      const float v = rp[(size_t)b * ld + (item0 + it) * 16 + r];
      resv[ii] = a.residual ? v : 0.f;
    }
  }

  // ---- weights of the first PD items.  fp32 activations: issued only once
  // the activations are staged in LDS (the first item), then once they are
  // built (the rest): 16 waves' weight loads issued during the staging held
  // it up (0.3-0.7 us per launch) and the x rows would share the registers
  Q4Frag fr[PD][KW][T];
  constexpr int PD0 = XMODE != kXF16 ? 1 : PD;
  __builtin_amdgcn_sched_barrier(0);
  // fp32 activations: every wave's small loads come home before any wave's
  // weight stream starts (phase stamps: with weights issued per wave as soon
  // as its own small loads were home, the last wave's small loads took 3.2 us
  // against 1.2 us for the first, queued behind the other waves' streams);
  // the statistics fold is done on the way
  if constexpr (XMODE != kXF16) {
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (XMODE == kXNorm) ssf.fold(s_part);
    __syncthreads();
  }
  if constexpr (XMODE == kXF16) {
#pragma unroll
  for (int q = 0; q < PD0; ++q)
#pragma unroll
      for (int p = 0; p < KW; ++p)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) load_frag(fr[q][p][tt], wptr(q, tt, sb0 + p), g);
  }
  __builtin_amdgcn_sched_barrier(0);

  // MODE 2: (cos, sin) of pair 16 hj + (tx % 16) at the position of row tx / 16
  // (pos_t), from the step's rotary table
  __shared__ float2 s_rope[MODE == 2 ? 16 * 16 : 1];
  if constexpr (MODE == 2) {
    if (tx < 16 * 16) s_rope[tx] = a.ra.rope[(size_t)pos_t * (16 * a.qh) + 16 * hj + (tx & 15)];
  }

  // ---- A operands of this wave's K slice, kept for every item
  if constexpr (XMODE == kXNorm) {
    if (tx < 16) s_rinv[tx] = rms_inv<S>(s_part, tx, a.inv_k, a.eps);
    __syncthreads();
    // h = f16(x * rinv * gamma) of the rows < B into LDS
    half_t* hs = reinterpret_cast<half_t*>(smem);
#pragma unroll
    for (int c = 0; c < KW; ++c) {
      const int c4 = tx + 64 * S * c;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u < a.B) {
          const float ri = s_rinv[u];
          half4_t h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = norm_apply(xv[c][u][e], ri, gv[c][e]);
          *reinterpret_cast<half4_t*>(hs + u * LDH + 4 * c4) = h;
        }
      }
      // rows 8..15 (B > 8) are loaded only now
      for (int b0 = 8; b0 < a.B; b0 += 8) {
        floatx4 xw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int bb = b0 + u < a.B ? b0 + u : a.B - 1;
          xw[u] = *reinterpret_cast<const floatx4*>(X32 + (size_t)bb * a.ldx + 4 * c4);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (b0 + u < a.B) {
            const float ri = s_rinv[b0 + u];
            half4_t h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = norm_apply(xw[u][e], ri, gv[c][e]);
            *reinterpret_cast<half4_t*>(hs + (b0 + u) * LDH + 4 * c4) = h;
          }
        }
      }
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < PD0; ++q)
#pragma unroll
      for (int p = 0; p < KW; ++p)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) load_frag(fr[q][p][tt], wptr(q, tt, sb0 + p), g);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < KW; ++p) {
      if constexpr (MV > 0) {
#pragma unroll
        for (int b = 0; b < MV; ++b) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            xm[p][b][j] = *reinterpret_cast<const half8_t*>(hs + b * LDH + (sbl + p) * 256 + 64 * g + 8 * j);
          mv_sums(p, b);
          fdm[p][b] = 1.f;
        }
        continue;
      }
      const half_t* src = hs + (r < a.B ? r : 0) * LDH + (sbl + p) * 256 + 64 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        half8_t v = *reinterpret_cast<const half8_t*>(src + 8 * j);
        if (r >= a.B) v = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
        av[p][j] = v;
      }
      float fmr;
      a_sums(av[p], 1.f, axs[p], fmr);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        fd[p][ii] = 1.f;
        fm[p][ii] = __shfl(fmr, 4 * g + ii);
      }
    }
    __syncthreads();   // the h area becomes the partial-sum area
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = PD0; q < PD; ++q)
#pragma unroll
        for (int p = 0; p < KW; ++p)
#pragma unroll
          for (int tt = 0; tt < T; ++tt) load_frag(fr[q][p][tt], wptr(q, tt, sb0 + p), g);
    __builtin_amdgcn_sched_barrier(0);
  } else if constexpr (XMODE == kXF32Blocked) {
    // f16b: row u's 256 values of super-block w + S c (the 64 float4 columns of
    // wave w) are rounded to fp16 after a shift by 2^-sh, sh the smallest
    // exponent that keeps their maximum finite; 2^sh is the factor of d and dmin
    __shared__ float s_fac[S * KW][16];
    half_t* hs = reinterpret_cast<half_t*>(smem);
    auto stage_row = [&](const floatx4& x4, int u, int c) {
      float am = fmaxf(fmaxf(fabsf(x4[0]), fabsf(x4[1])), fmaxf(fabsf(x4[2]), fabsf(x4[3])));
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
      const int sh = f16_block_shift(am);
      const float inv = exp2i(-sh);
      half4_t h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (half_t)(x4[e] * inv);
      const int c4 = tx + 64 * S * c;
      *reinterpret_cast<half4_t*>(hs + u * LDH + 4 * c4) = h;
      if (lane == 0) s_fac[wave + S * c][u] = exp2i(sh);
    };
#pragma unroll
    for (int c = 0; c < KW; ++c) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < a.B) stage_row(xv[c][u], u, c);
      for (int b0 = 8; b0 < a.B; b0 += 8) {
        floatx4 xw[8];
        const int c4 = cbase + tx + 64 * S * c;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int bb = b0 + u < a.B ? b0 + u : a.B - 1;
          xw[u] = *reinterpret_cast<const floatx4*>(X32 + (size_t)bb * a.ldx + 4 * c4);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (b0 + u < a.B) stage_row(xw[u], b0 + u, c);
      }
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < PD0; ++q)
#pragma unroll
      for (int p = 0; p < KW; ++p)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) load_frag(fr[q][p][tt], wptr(q, tt, sb0 + p), g);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < KW; ++p) {
      if constexpr (MV > 0) {
#pragma unroll
        for (int b = 0; b < MV; ++b) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            xm[p][b][j] = *reinterpret_cast<const half8_t*>(hs + b * LDH + (sbl + p) * 256 + 64 * g + 8 * j);
          mv_sums(p, b);
          fdm[p][b] = s_fac[sbl + p][b];
        }
        continue;
      }
      const half_t* src = hs + (r < a.B ? r : 0) * LDH + (sbl + p) * 256 + 64 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        half8_t v = *reinterpret_cast<const half8_t*>(src + 8 * j);
        if (r >= a.B) v = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
        av[p][j] = v;
      }
      const float fdr = r < a.B ? s_fac[sbl + p][r] : 1.f;
      float fmr;
      a_sums(av[p], fdr, axs[p], fmr);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        fd[p][ii] = __shfl(fdr, 4 * g + ii);
        fm[p][ii] = __shfl(fmr, 4 * g + ii);
      }
    }
    __syncthreads();   // the activation area becomes the partial-sum area
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = PD0; q < PD; ++q)
#pragma unroll
        for (int p = 0; p < KW; ++p)
#pragma unroll
          for (int tt = 0; tt < T; ++tt) load_frag(fr[q][p][tt], wptr(q, tt, sb0 + p), g);
    __builtin_amdgcn_sched_barrier(0);
  } else {
    static_assert(XMODE == kXF16, "fp16 or fp32 activations");
#pragma unroll
    for (int p = 0; p < KW; ++p) {
      if constexpr (MV > 0) {
#pragma unroll
        for (int b = 0; b < MV; ++b) {
          mv_sums(p, b);
          fdm[p][b] = 1.f;
        }
        continue;
      }
      if (r >= a.B)
#pragma unroll
        for (int j = 0; j < 8; ++j) av[p][j] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
      float fmr;
      a_sums(av[p], 1.f, axs[p], fmr);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        fd[p][ii] = 1.f;
        fm[p][ii] = __shfl(fmr, 4 * g + ii);
      }
    }
  }

  // ---- items: products of the slice, next weights issued into the freed slot
  const NibbleMasks km = {in_vgpr(0x000F000Fu), in_vgpr(0x00F000F0u), in_vgpr(0x64006400u)};
#pragma unroll
  for (int it = 0; it < IPW; ++it) {
    {
      floatx4 acc[T];
#pragma unroll
      for (int tt = 0; tt < T; ++tt) acc[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
      if constexpr (MV > 0) {
        float accm[T][MV];
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
#pragma unroll
          for (int b = 0; b < MV; ++b) accm[tt][b] = 0.f;
#pragma unroll
        for (int p = 0; p < KW; ++p)
#pragma unroll
          for (int tt = 0; tt < T; ++tt) {
            float sq[MV], sm[MV];
            float d, dm;
            q4_superblock_mv<MV>(fr[it % PD][p][tt], xm[p], xs[p], g, km, sq, sm, d, dm);
#pragma unroll
            for (int b = 0; b < MV; ++b)
              accm[tt][b] = __builtin_fmaf(d * fdm[p][b], sq[b], __builtin_fmaf(-dm * fdm[p][b], sm[b], accm[tt][b]));
          }
        // lanes r, r + 16, r + 32, r + 48 hold the four 64-value pieces of
        // row r; their sum, for sequence b, goes where the MFMA would leave
        // it: lane (0, r), element b
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
#pragma unroll
          for (int b = 0; b < MV; ++b) {
            float v = accm[tt][b];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[tt][b] = g == 0 ? v : 0.f;
          }
      } else {
#pragma unroll
        for (int p = 0; p < KW; ++p)
#pragma unroll
          for (int tt = 0; tt < T; ++tt) {
            floatx4 sq, sm;
            float d, dm;
            q4_superblock(fr[it % PD][p][tt], av[p], axs[p], g, km, sq, sm, d, dm);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
              acc[tt][ii] =
                  __builtin_fmaf(d * fd[p][ii], sq[ii], __builtin_fmaf(-dm * fm[p][ii], sm[ii], acc[tt][ii]));
          }
      }
      if (it + PD < IPW) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < KW; ++p)
#pragma unroll
          for (int tt = 0; tt < T; ++tt) load_frag(fr[it % PD][p][tt], wptr(it + PD, tt, sb0 + p), g);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int tt = 0; tt < T; ++tt) red[it][tt][wave][lane] = acc[tt];
    }
  }
  __syncthreads();

  // ---- wave i finishes item i: the S partial sums in wave order
  if constexpr (MODE == 2) {
    qkv_finish<S>(a, red, wave, lane, g, r, head, hj, sl, ps, s_rope);
    return;
  }
  // (with K split across work-groups every wave takes part in the arrival
  // below, so the waves without an item leave only after it)
  if (KSPLIT == 1 && wave >= n_items) return;
  floatx4 v[T];
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    v[tt] = red[0][tt][0][lane];
  }
#pragma unroll
  for (int it = 0; it < IPW; ++it) {
    if (it == wave) {
#pragma unroll
      for (int tt = 0; tt < T; ++tt) {
        v[tt] = red[it][tt][0][lane];
#pragma unroll
        for (int w = 1; w < S; ++w) v[tt] += red[it][tt][w][lane];
      }
    }
  }
  const int item = item0 + wave;
  const int n = item * 16 + r;
  if constexpr (MODE == 0 && KSPLIT > 1) {
    // this chunk's partial sums of the work-group's items (wave i: item i);
    // the last of the row group's KSPLIT work-groups to arrive adds the
    // chunks of every item in chunk order.  One arrival per work-group: the
    // barrier orders every wave's stores before thread 0's agent-scope
    // release, which publishes them ahead of the count; the last arriver's
    // acquire orders the reloads after it.
    __shared__ int s_last;
    const int n_total = a.f_tiles * 16;
    const int grp = (int)blockIdx.x % n_groups;
    if (wave < n_items) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        if (b < a.B)
          __hip_atomic_store(&a.part[((size_t)kc * a.B + b) * n_total + n], v[0][ii], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (tx == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const unsigned prev = __hip_atomic_fetch_add(&a.counters[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (unsigned)(KSPLIT - 1);
      if (s_last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __hip_atomic_store(&a.counters[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (!s_last || wave >= n_items) return;
    float pv[KSPLIT][4];
#pragma unroll
    for (int cc = 0; cc < KSPLIT; ++cc)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii < a.B ? 4 * g + ii : a.B - 1;
        pv[cc][ii] = __hip_atomic_load(&a.part[((size_t)cc * a.B + b) * n_total + n], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float t = pv[0][ii];
#pragma unroll
      for (int cc = 1; cc < KSPLIT; ++cc) t += pv[cc][ii];
      v[0][ii] = t;
    }
  }
  if constexpr (MODE == 0) {
    float sq[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii;
      float y = v[0][ii];
      if (b < a.B) {
        if (a.residual) y += resv[ii];
        a.Y[(size_t)b * a.ldy + n] = y;
      }
      sq[ii] = b < a.B ? y * y : 0.f;
    }
    if (a.ss_out) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        float t = sq[ii];
        t += __shfl_xor(t, 1);
        t += __shfl_xor(t, 2);
        t += __shfl_xor(t, 4);
        t += __shfl_xor(t, 8);
        if (r == 0) a.ss_out[(size_t)item * 16 + 4 * g + ii] = t;
      }
    }
  } else {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii;
      if (b < a.B) {
        const float z = v[0][ii];
        float sil;
        if (z >= 0.f) {
          sil = z / (1.f + expf(-z));
        } else {
          const float ez = expf(z);
          sil = z * ez / (1.f + ez);
        }
        a.A[(size_t)b * a.lda + n] = sil * v[1][ii];
      }
    }
  }
}

// ---------------------------------------------------------------- launcher
// Waves per work-group and super-blocks in flight per wave, by shape and
// activation mode (MI355X, B = 8, the 6144x4096, 4096x4096, 2x12288x4096 and
// 4096x12288 projections): fp16 activations take 8 waves (two work-groups per
// CU at 128 registers); the fp32 modes, at up to 256 registers, 4 waves (two
// work-groups per CU), or 8 for a long K (one work-group per CU, 6 super-
// blocks per wave at K = 12288).
WkConfig wk_config(int kb, bool swiglu, int xmode) {
  WkConfig c{4, 2};
  if (!swiglu && xmode == kXF16 && kb >= 8) c.s = 8;
  if (!swiglu && xmode == kXF16 && kb >= 16) c = {16, 1};
  if (!swiglu && xmode == kXF32Blocked && kb >= 32) c.s = 8;
  return c;
}

template <int MODE, int XMODE>
static void launch_mode(int s, int items, const WkArgs& a, hipStream_t st) {
  if constexpr (XMODE == kXF16 && MODE == 0) {
    if (s == 16) {
      hipLaunchKernelGGL((gemm_wk_kernel<MODE, XMODE, 16, 1>), dim3(items), dim3(1024), 0, st, a);
      return;
    }
  }
  if (s == 8)
    hipLaunchKernelGGL((gemm_wk_kernel<MODE, XMODE, 8, 2>), dim3(items), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_wk_kernel<MODE, XMODE, 4, 2>), dim3(items), dim3(256), 0, st, a);
}

// One configuration of the multi-item kernel, as the MFMA tiles (mv = 0) or
// the matvec for mv = B in {1, 2} sequences.
// SwiGLU items hold two weight tiles each: with two items in flight the
// matvec of two sequences spills, so that combination is never built (the
// caller takes one item in flight for it)
template <int MODE, int PD>
constexpr bool wi_mv2_fits() {
  return !(MODE == 1 && PD > 1);
}
template <int MODE, int XMODE, int S, int KW, int IPW, int PD, int KSPLIT = 1>
static void launch_wi(int mv, dim3 grid, const WkArgs& a, hipStream_t st) {
  if (mv == 1) {
    hipLaunchKernelGGL((gemm_wi_kernel<MODE, XMODE, S, KW, IPW, PD, KSPLIT, 1>), grid, dim3(64 * S), 0, st, a);
  } else if (mv == 2) {
    if constexpr (wi_mv2_fits<MODE, PD>())
      hipLaunchKernelGGL((gemm_wi_kernel<MODE, XMODE, S, KW, IPW, PD, KSPLIT, 2>), grid, dim3(64 * S), 0, st, a);
  } else {
    hipLaunchKernelGGL((gemm_wi_kernel<MODE, XMODE, S, KW, IPW, PD, KSPLIT, 0>), grid, dim3(64 * S), 0, st, a);
  }
}

// The kernel arguments of one launch (the K-split partials and arrival
// counters from the workspace, used where the shape splits K).
static WkArgs wk_args(const GemmLaunch& L) {
  WkArgs a{};
  a.W = reinterpret_cast<const uint8_t*>(L.W);
  a.X = L.X;
  a.gamma = L.gamma;
  a.ss_in = L.ss_in;
  a.Y = L.Y;
  a.residual = L.residual;
  a.ss_out = L.ss_out;
  a.A = L.A;
  a.ldx = L.ldx;
  a.ldy = L.ldy;
  a.ldr = L.ldr;
  a.lda = L.lda;
  a.kb = (int)(L.K / 256);
  a.B = L.B;
  a.f_tiles = (int)(L.n_rows / 16);
  a.ss_slots = (int)(L.K / kSsCols);
  a.eps = L.eps;
  a.inv_k = 1.0f / (float)L.K;
  char* p = reinterpret_cast<char*>(L.ws);
  a.counters = reinterpret_cast<unsigned*>(p);
  a.part = p ? reinterpret_cast<float*>(p + (size_t)kGemmMaxGroups * 4) : nullptr;
  return a;
}

// Multi-item launch for the shapes it is built for; hipErrorNotSupported
// otherwise (the caller then uses another kernel).  K = 4096 (16 waves of
// one super-block each):
//   SwiGLU: three gate/up tile pairs per work-group, two in flight (768 pairs
//     for F = 12288: 256 work-groups);
//   plain, RMSNorm fused: two tiles per work-group (6144 rows: 192);
//   plain, fp16 activations: one tile per work-group up to 4096 rows, else two.
// K = 12288, plain (fp32 activations with the blocked fp16 rounding, or fp16):
// four K chunks of 3072 (12 waves), four tiles per work-group.
hipError_t launch_gemm_wi(const GemmLaunch& L, hipStream_t st) {
  const int kb = (int)(L.K / 256);
  const int64_t items = L.n_rows / 16;
  const int xmode = L.x_f32 ? (L.gamma ? kXNorm : kXF32Blocked) : kXF16;
  if (kb != 16 && !(kb == 48 && xmode != kXNorm && !L.swiglu)) return hipErrorNotSupported;
  const int mv = gemm_matvec_rows(L.kernel, L.B);
  const WkArgs a = wk_args(L);
  if (kb == 48) {
    // K = 12288: four K chunks of 3072 (12 waves of one super-block), four
    // tiles per work-group: 256 work-groups for N = 4096, one round on the chip
    const dim3 grid((unsigned)((items + 3) / 4) * 4);
    if (xmode == kXF32Blocked) launch_wi<0, kXF32Blocked, 12, 1, 4, 2, 4>(mv, grid, a, st);
    else launch_wi<0, kXF16, 12, 1, 4, 2, 4>(mv, grid, a, st);
    return hipGetLastError();
  }
  if (L.swiglu) {
    // two sequences on the vector ALU hold one item's weights in flight (two
    // would spill)
    const dim3 grid((unsigned)((items + 2) / 3));
    if (xmode == kXNorm) {
      if (mv == 2) launch_wi<1, kXNorm, 16, 1, 3, 1>(mv, grid, a, st);
      else launch_wi<1, kXNorm, 16, 1, 3, 2>(mv, grid, a, st);
    } else {
      if (mv == 2) launch_wi<1, kXF16, 16, 1, 3, 1>(mv, grid, a, st);
      else launch_wi<1, kXF16, 16, 1, 3, 2>(mv, grid, a, st);
    }
  } else if (xmode == kXNorm) {
    launch_wi<0, kXNorm, 16, 1, 2, 2>(mv, dim3((unsigned)((items + 1) / 2)), a, st);
  } else if (items <= 256) {
    launch_wi<0, kXF16, 16, 1, 1, 1>(mv, dim3((unsigned)items), a, st);
  } else {
    launch_wi<0, kXF16, 16, 1, 2, 2>(mv, dim3((unsigned)((items + 1) / 2)), a, st);
  }
  return hipGetLastError();
}

// The QKV projection of a decode step with its RoPE / append finish: K =
// 4096, RMSNorm fused, fp16 or E4M3 cache (element-wise stores), head_dim 64
// or 128; one work-group per
// (head, half-head tile).  hipErrorNotSupported for any other case.
hipError_t launch_gemm_wi_qkv(const GemmLaunch& L, const RopeAppendArgs& ra, int head_dim, hipStream_t st) {
  const int kb = (int)(L.K / 256);
  if (kb != 16 || !L.x_f32 || !L.gamma || ((ra.kf == kFmtQ8 || ra.vf == kFmtQ8) && !ra.kv_new) ||
      (head_dim != 64 && head_dim != 128) || L.residual || L.ss_out || !ra.rope)
    return hipErrorNotSupported;
  WkArgs a = wk_args(L);
  a.ra = ra;
  a.qh = head_dim / 32;
  const int n_heads = (int)(L.n_rows / head_dim);
  launch_wi<2, kXNorm, 16, 1, 2, 2>(gemm_matvec_rows(L.kernel, L.B), dim3((unsigned)(n_heads * a.qh)), a, st);
  return hipGetLastError();
}

hipError_t launch_gemm_wk(const GemmLaunch& L, hipStream_t st) {
  const int kb = (int)(L.K / 256);
  const int64_t items = L.n_rows / 16;   // SwiGLU: n_rows = F, one item per gate/up tile pair
  const int xmode = L.x_f32 ? (L.gamma ? kXNorm : kXF32Blocked) : kXF16;
  const WkConfig c = wk_config(kb, L.swiglu, xmode);
  const WkArgs a = wk_args(L);
  if (L.swiglu) {
    if (xmode == kXNorm) launch_mode<1, kXNorm>(c.s, (int)items, a, st);
    else launch_mode<1, kXF16>(c.s, (int)items, a, st);
  } else if (xmode == kXNorm) {
    launch_mode<0, kXNorm>(c.s, (int)items, a, st);
  } else if (xmode == kXF32Blocked) {
    launch_mode<0, kXF32Blocked>(c.s, (int)items, a, st);
  } else {
    launch_mode<0, kXF16>(c.s, (int)items, a, st);
  }
  return hipGetLastError();
}

}  // namespace qk
