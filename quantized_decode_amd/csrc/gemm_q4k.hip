// Q4_K dequant-GEMM for a decode batch of 1..16 sequences on CDNA4 MFMA.
// (P1, P2, P3: the three pages listed, with their titles, at the top of include/qkdec.h.)
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
#include <algorithm>

#include "common.h"
#include "internal.h"
#include "kv_dev.h"
#include "q4k_dev.h"

namespace qk {

// Work-group: WPB waves, one 16-row tile each, covering super-blocks
// [c*KC, c*KC + KC) of K (c = blockIdx.y).  More waves per work-group share
// one staged copy of the activations: each work-group reads B*KC*256
// activations for 16*WPB*KC*256 weights.
//
// The prologue issues every load the work-group can hold before waiting on
// any: the RMSNorm statistics and gains (kXNorm), the first round of
// activations, then the weights of the first P super-blocks of each wave's
// tile (2304 contiguous bytes each; P = min(KC, 8), 4 with 16 waves).
// Activations are staged once in LDS as fp16 together with the fp32 sum of
// every 32-value sub-block (split hi/lo for the min-term MFMA) and shared by
// the work-group's tiles.  The main loop decodes and multiplies one
// super-block per step and accumulates the previous step's products, so MFMA
// results are never waited on.  With
// several K chunks every work-group writes its partial sums with write-through
// stores and the last one to arrive for a row group adds the chunks in chunk
// order (so the result does not depend on arrival order).
// One work item (row group rg, K chunk c).  SMAX: most sum-of-squares slots
// the kXNorm statistics fold holds (sizes its registers).
template <int KC, int MODE, int XMODE, int WPB, int SMAX>
__device__ void gemm_item(const GemmArgs& a, int rg, int c, int n_chunks, half_t* xs, GemmSmem<WPB, MODE>& sm) {
  constexpr int NT = 64 * WPB;                           // threads
  // super-blocks in flight per wave: 8 with 8-wave work-groups, 4 otherwise
  // (16 waves, and 4-wave work-groups packed four to a CU, leave 128 registers per lane)
  constexpr int PMAX = WPB == 8 ? 8 : 4;
  constexpr int P = KC < PMAX ? KC : PMAX;
  constexpr int XB = WPB == 16 ? 2 : (XMODE == kXF16 ? 8 : 4);   // activation pieces (8 values) per thread and round
  constexpr int GL = (KC * 64 + NT - 1) / NT;            // kXNorm: float4 of gains per thread
  // xs: [B][KC*256 + 8] fp16 activations, [B][KC][16] x sums, kXNorm: [KC*256] fp32 gains
  float* fac_d = sm.fac_d;
  float* fac_m = sm.fac_m;
  auto& s_red = sm.s_red;
  const int B = a.B;
  const int ldsx = KC * 256 + 8;
  half_t* xsum = xs + B * ldsx;
  float* gls = reinterpret_cast<float*>(xsum + B * KC * 16);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int r = lane & 15;
  const int sb0 = c * KC;
  const int n_pieces = B * KC * 32;

  const bool tok = tile_valid<MODE, WPB>(rg, wave, a.n_tiles, a.f_tiles);
  const int tl = tok ? tile_of<MODE, WPB>(rg, wave, a.f_tiles) : 0;   // keep addresses in bounds
  const uint8_t* tbase = a.W + ((size_t)tl * a.kb + sb0) * 2304 + (size_t)r * 144;

  // ---- prologue: loads in the order they are needed
  Q4Frag fr[P];
  SsFold<NT, SMAX> ssf;
  floatx4 gv[GL];
  if constexpr (XMODE == kXNorm) {
    ssf.load(a.ss_in, a.ss_slots);
#pragma unroll
    for (int k = 0; k < GL; ++k) {
      const int idx = threadIdx.x + NT * k;
      const int idc = idx < KC * 64 ? idx : KC * 64 - 1;
      gv[k] = *reinterpret_cast<const floatx4*>(a.gamma + (size_t)sb0 * 256 + 4 * idc);
    }
  }
  half8_t hv[XB];
  floatx4 xv[XB][2];
  auto load_round = [&](int base) {
#pragma unroll
    for (int k = 0; k < XB; ++k) {
      int idx = base + threadIdx.x + NT * k;
      idx = idx < n_pieces ? idx : n_pieces - 1;
      const int b = idx / (KC * 32), col = idx % (KC * 32);
      const size_t e0 = (size_t)b * a.ldx + (size_t)sb0 * 256 + 8 * col;   // element offset
      if constexpr (XMODE == kXF16) {
        hv[k] = *reinterpret_cast<const half8_t*>(reinterpret_cast<const half_t*>(a.X) + e0);
      } else {
        const float* src = reinterpret_cast<const float*>(a.X) + e0;
        xv[k][0] = *reinterpret_cast<const floatx4*>(src);
        xv[k][1] = *reinterpret_cast<const floatx4*>(src + 4);
      }
    }
  };
  load_round(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < P; ++p) load_frag(fr[p], tbase + (size_t)p * 2304, g);
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (XMODE == kXNorm) {
    ssf.fold(s_red);
#pragma unroll
    for (int k = 0; k < GL; ++k) {
      const int idx = threadIdx.x + NT * k;
      if (idx < KC * 64) *reinterpret_cast<floatx4*>(gls + 4 * idx) = gv[k];
    }
    __syncthreads();
  }

  // ---- activations -> LDS (fp16) with the sub-block sums
  for (int base = 0; base < n_pieces; base += NT * XB) {
    if (base > 0) load_round(base);
#pragma unroll
    for (int k = 0; k < XB; ++k) {
      const int idx = base + threadIdx.x + NT * k;
      const bool valid = idx < n_pieces;
      const int idc = valid ? idx : n_pieces - 1;
      const int b = idc / (KC * 32), col = idc % (KC * 32);
      half8_t h;
      float xfk = 1.f;
      if constexpr (XMODE == kXF16) {
        h = hv[k];
      } else if constexpr (XMODE == kXNorm) {
        const float rinv = rms_inv<WPB>(s_red, b, a.inv_k, a.eps);
        const float* gr = gls + 8 * col;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[e] = norm_apply(xv[k][0][e], rinv, gr[e]);
          h[4 + e] = norm_apply(xv[k][1][e], rinv, gr[4 + e]);
        }
      } else {
        // the 32 pieces of one (row, super-block) are 32 consecutive threads
        float am = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) am = fmaxf(am, fmaxf(fabsf(xv[k][0][e]), fabsf(xv[k][1][e])));
        for (int o = 16; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 32));
        const int sh = f16_block_shift(am);
        const float inv = exp2i(-sh);
        xfk = exp2i(sh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          h[e] = (half_t)(xv[k][0][e] * inv);
          h[4 + e] = (half_t)(xv[k][1][e] * inv);
        }
      }
      float ps = 0.f;
      if (valid) {
        *reinterpret_cast<half8_t*>(xs + b * ldsx + 8 * col) = h;
#pragma unroll
        for (int e = 0; e < 8; ++e) ps += (float)h[e];
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
      if (valid && (col & 3) == 0) {
        const int sbl = col >> 5, sub = (col & 31) >> 2;   // super-block in chunk, sub-block 0..7
        const half_t hs = (half_t)pss;
        const half_t ls = (half_t)(pss - (float)hs);
        half_t* dst = xsum + (b * KC + sbl) * 16 + 4 * (sub >> 1) + (sub & 1);
        dst[0] = hs;
        dst[2] = ls;
        if ((col & 31) == 0) {
          fac_d[sbl * 16 + b] = xfk;
          fac_m[sbl * 16 + b] = big ? 32.f * xfk : xfk;
        }
      }
    }
  }
  for (int t = threadIdx.x; t < (16 - B) * KC; t += NT) {
    const int i = t / (16 - B), b = B + t % (16 - B);
    fac_d[i * 16 + b] = 1.f;
    fac_m[i * 16 + b] = 1.f;
  }
  __syncthreads();

  // ---- main loop
  const NibbleMasks km = {in_vgpr(0x000F000Fu), in_vgpr(0x00F000F0u), in_vgpr(0x64006400u)};
  const int xrow = r < B ? r : B - 1;
  const half_t* xr = xs + xrow * ldsx + 64 * g;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  floatx4 psq, psm;
  float pd = 0.f, pdm = 0.f;
  floatx4 pfd = {1.f, 1.f, 1.f, 1.f}, pfm = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    half8_t av[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) av[j] = *reinterpret_cast<const half8_t*>(xr + 256 * i + 8 * j);
    const half4_t axs = *reinterpret_cast<const half4_t*>(xsum + (xrow * KC + i) * 16 + 4 * g);
    const floatx4 fm = *reinterpret_cast<const floatx4*>(fac_m + i * 16 + 4 * g);
    floatx4 fd = {1.f, 1.f, 1.f, 1.f};
    if constexpr (XMODE == kXF32Blocked) fd = *reinterpret_cast<const floatx4*>(fac_d + i * 16 + 4 * g);
    floatx4 sq, sm;
    float d, dm;
    q4_superblock(fr[i % P], av, axs, g, km, sq, sm, d, dm);
    if (i + P < KC) {
      __builtin_amdgcn_sched_barrier(0);
      load_frag(fr[i % P], tbase + (size_t)(i + P) * 2304, g);
      __builtin_amdgcn_sched_barrier(0);
    }
    // accumulate the previous super-block now that its MFMAs are long done;
    // d * fd and dmin * fm are exact (the factors are powers of two)
    if (i > 0) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        acc[ii] = __builtin_fmaf(pd * pfd[ii], psq[ii], __builtin_fmaf(-pdm * pfm[ii], psm[ii], acc[ii]));
    }
    psq = sq;
    psm = sm;
    pd = d;
    pdm = dm;
    pfd = fd;
    pfm = fm;
  }
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
    acc[ii] = __builtin_fmaf(pd * pfd[ii], psq[ii], __builtin_fmaf(-pdm * pfm[ii], psm[ii], acc[ii]));

  // ---- split-K: the last work-group of a row group to arrive finishes it
  const int n = tile_of<MODE, WPB>(rg, wave, a.f_tiles) * 16 + r;   // this lane's output row
  const int n_total = a.n_tiles * 16;
  float res[4] = {0.f, 0.f, 0.f, 0.f};
  if (n_chunks > 1) {
    if (tok) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        if (b < B)
          __hip_atomic_store(&a.part[((size_t)c * B + b) * n_total + n], acc[ii], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    // every wave's partial stores happen before thread 0's release (the
    // barrier), which publishes them at device scope before the arrival count;
    // the last arriver's acquire orders its partial loads after the count
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const unsigned prev = __hip_atomic_fetch_add(&a.counters[rg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.s_last = prev == (unsigned)(n_chunks - 1);
      if (sm.s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (!sm.s_last) return;
    // all chunks' partials (and the residual) in one batch of loads, then the
    // sum in chunk order
    const int nc = tok ? n : 0;
    float pv[8][4];
    if (n_chunks <= 8) {
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        if (cc < n_chunks) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int b = 4 * g + ii < B ? 4 * g + ii : B - 1;
            pv[cc][ii] = __hip_atomic_load(&a.part[((size_t)cc * B + b) * n_total + nc], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      if (MODE != 1 && a.residual) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int b = 4 * g + ii < B ? 4 * g + ii : B - 1;
          res[ii] = a.residual[(size_t)b * a.ldr + nc];
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        float v = pv[0][ii];
#pragma unroll
        for (int cc = 1; cc < 8; ++cc)
          if (cc < n_chunks) v += pv[cc][ii];
        acc[ii] = v;
      }
    } else {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii < B ? 4 * g + ii : B - 1;
        float v = 0.f;
        for (int cc = 0; cc < n_chunks; ++cc)
          v += __hip_atomic_load(&a.part[((size_t)cc * B + b) * n_total + nc], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        acc[ii] = v;
      }
      if (MODE != 1 && a.residual) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int b = 4 * g + ii < B ? 4 * g + ii : B - 1;
          res[ii] = a.residual[(size_t)b * a.ldr + nc];
        }
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&a.counters[rg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (MODE != 1 && a.residual) {
    const int nc = tok ? n : 0;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii < B ? 4 * g + ii : B - 1;
      res[ii] = a.residual[(size_t)b * a.ldr + nc];
    }
  }

  if constexpr (MODE == 2) {
    // One head (WPB = head_dim / 16 tiles); wave w holds dims 16w + r of rows
    // 4g + ii.  The fp32 projection is stored as it is (workspace views), then
    // q and k are rotated (pair (i, i + D/2) sits in waves w and w ^ WPB/2),
    // q goes out as fp16 and k, v are appended to the cache at pos.
    const RopeAppendArgs& ra = a.ra;
    constexpr int D = 16 * WPB, HALF = D / 2;
    const int head = rg, d = 16 * wave + r;
    const int n_kv = ra.n_kv;
    const bool is_q = head < ra.Hq, is_v = head >= ra.Hq + n_kv;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      if (4 * g + ii < B) a.Y[(size_t)(4 * g + ii) * a.ldy + n] = acc[ii];
    if (!is_v) {
      for (int t = threadIdx.x; t < B * HALF; t += NT) {
        const int b = t / HALF, i = t % HALF;
        float2 c;
        if (ra.rope) {
          c = ra.rope[(size_t)b * HALF + i];
        } else {
          rope_cos_sin(ra.pos[b], i, D, ra.rope_base, c.x, c.y);
        }
        sm.rope[b][i] = c;
      }
    }
    sm.fin[wave][lane] = acc;
    __syncthreads();
    float out[4];
    if (!is_v) {
      const floatx4 other = sm.fin[wave ^ (WPB / 2)][lane];
      const int i = d % HALF;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float2 c = sm.rope[4 * g + ii < B ? 4 * g + ii : 0][i];
        // d < D/2: x_i cos - x_{i+D/2} sin; d >= D/2: x_{i+D/2} cos + x_i sin
        out[ii] = d < HALF ? acc[ii] * c.x - other[ii] * c.y : acc[ii] * c.x + other[ii] * c.y;
      }
    } else {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) out[ii] = acc[ii];
    }
    if (is_q) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        if (b < B) ra.q16[((size_t)b * ra.Hq + head) * D + d] = f2h_bits(out[ii]);
      }
    } else {
      const int kvh = is_v ? head - ra.Hq - n_kv : head - ra.Hq;
      CacheRef c;
      c.k = ra.k; c.v = ra.v; c.ks = ra.ks; c.vs = ra.vs;
      c.n_kv = n_kv; c.cap = ra.cap; c.D = D; c.n_slots = ra.n_slots; c.kf = ra.kf; c.vf = ra.vf;
      int sl[4], ps[4];
      bool ok[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        sl[ii] = b < B ? ra.slot[b] : 0;
        ps[ii] = b < B ? ra.spos[b] : 0;
        ok[ii] = b < B && sl[ii] >= 0 && sl[ii] < ra.n_slots && ps[ii] >= 0 && ps[ii] < ra.cap;
        if (b < B && !ok[ii] && wave == 0 && r == 0) *ra.err = QKDEC_E_CAPACITY;
      }
      if ((is_v ? ra.vf : ra.kf) != kFmtQ8) {   // uniform: one head per work-group
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          if (ok[ii]) store_point(c, is_v, sl[ii], kvh, ps[ii], d, out[ii]);
      } else {
        // a Q8_0 block is 32 dims: the 16 lanes of this wave's row group and
        // the same lanes of the partner wave w ^ 1
        double am[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          float m = fabsf(out[ii]);
          m = fmaxf(m, __shfl_xor(m, 1));
          m = fmaxf(m, __shfl_xor(m, 2));
          m = fmaxf(m, __shfl_xor(m, 4));
          m = fmaxf(m, __shfl_xor(m, 8));
          if (r == 0) sm.s_red[wave][4 * g + ii] = m;
        }
        __syncthreads();
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int b = 4 * g + ii;
          am[ii] = (double)fmaxf(sm.s_red[wave][b], sm.s_red[wave ^ 1][b]);
          int8_t q;
          uint16_t dbits;
          q8_encode((double)out[ii], am[ii], q, dbits);
          if (ok[ii]) store_q8(c, is_v, sl[ii], kvh, ps[ii], d, q, dbits);
        }
      }
    }
  } else if constexpr (MODE == 0) {
    float sq[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int b = 4 * g + ii;
      const float v = acc[ii] + res[ii];
      sq[ii] = (tok && b < B) ? v * v : 0.f;
      if (tok && b < B) a.Y[(size_t)b * a.ldy + n] = v;
    }
    if (a.ss_out && tok) {
      // each wave's 16 columns make one sum-of-squares slot (zero for rows >= B)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        float t = sq[ii];
        t += __shfl_xor(t, 1);
        t += __shfl_xor(t, 2);
        t += __shfl_xor(t, 4);
        t += __shfl_xor(t, 8);
        if (r == 0) a.ss_out[(size_t)(n >> 4) * 16 + 4 * g + ii] = t;
      }
    }
  } else {
    constexpr int H = WPB / 2;
    auto& fin = sm.fin;
    fin[wave][lane] = acc;
    __syncthreads();
    const floatx4 gvv = fin[wave % H][lane];
    const floatx4 uvv = fin[wave % H + H][lane];
    const int nf = tile_of<MODE, WPB>(rg, wave % H, a.f_tiles) * 16 + r;
    if (wave < H && tok) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int b = 4 * g + ii;
        if (b < B) {
          const float z = gvv[ii];
          float sil;
          if (z >= 0.f) {
            sil = z / (1.f + expf(-z));
          } else {
            const float ez = expf(z);
            sil = z * ez / (1.f + ez);
          }
          a.A[(size_t)b * a.lda + nf] = sil * uvv[ii];
        }
      }
    }
  }
}

template <int KC, int MODE, int XMODE, int WPB, int SMAX>
__global__ void __launch_bounds__(64 * WPB) gemm_q4k_kernel(const GemmArgs a) {
  extern __shared__ half_t xs[];
  __shared__ GemmSmem<WPB, MODE> sm;
  gemm_item<KC, MODE, XMODE, WPB, SMAX>(a, blockIdx.x, blockIdx.y, gridDim.y, xs, sm);
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
static size_t lds_bytes(int B, int kc, int xmode) {
  size_t n = (size_t)B * (kc * 256 + 8) * 2 + (size_t)B * kc * 32;
  if (xmode == kXNorm) n += (size_t)kc * 256 * 4;
  return n;
}

static int64_t n_groups_of(int64_t n_tiles, bool swiglu, int wpb) {
  if (swiglu) return (n_tiles / 2 + wpb / 2 - 1) / (wpb / 2);
  return (n_tiles + wpb - 1) / wpb;
}

// Launch shape: K chunk (super-blocks per work-group) and waves per
// work-group.  Eight waves share one staged copy of the activations where the
// launch is large (many tiles, or a long K); the chunk is the smallest divisor
// of kb that keeps at most 8 chunks and at most 1024 work-groups and whose
// staged activations fit the LDS budget.  The budget is sized for max(B, 8),
// so every batch of up to 8 sequences uses the same chunking and a sequence's
// outputs do not depend on its batch-mates.  (Chosen from sweeps on MI355X of
// the 6144x4096, 4096x4096, 2x12288x4096 and 4096x12288 shapes at B = 8.)
struct GemmConfig {
  int kc, wpb;
};

// The K chunk for a given number of waves per work-group.
static int gemm_kc(int64_t n_tiles, int64_t kb, int B, bool swiglu, int xmode, int wpb) {
  static const int cands[] = {1, 2, 4, 6, 8, 12, 16};
  const int64_t groups = n_groups_of(n_tiles, swiglu, wpb);
  const int bb = B > 8 ? B : 8;
  int best = 0;
  for (int kc : cands) {
    if (kb % kc) continue;
    if (lds_bytes(bb, kc, xmode) > 64 * 1024) break;
    best = kc;
    if (kb / kc <= 8 && groups * (kb / kc) <= 1024) break;
  }
  return best ? best : 1;
}

GemmConfig gemm_config(int64_t n_tiles, int64_t kb, int B, bool swiglu, int xmode) {
  const int wpb = (n_tiles >= 1024 || kb > 32) ? 8 : 4;
  return {gemm_kc(n_tiles, kb, B, swiglu, xmode, wpb), wpb};
}

// The split-K arrival counters occupy a fixed area at the start of the
// workspace, so that calls of different shapes can share one workspace (each
// last arriver returns its counter to zero; the partial sums of one call then
// never land on another call's counters).
static size_t counters_bytes() { return (size_t)kGemmMaxGroups * 4; }

size_t gemm_workspace_bytes(int64_t n_rows, int64_t K, int B, bool swiglu) {
  const int64_t kb = K / 256;
  const int64_t n_tiles = n_rows / 16;
  int64_t chunks = 1;
  for (int xmode : {(int)kXF16, (int)kXF32Blocked, (int)kXNorm})
    chunks = std::max<int64_t>(chunks, kb / gemm_config(n_tiles, kb, B, swiglu, xmode).kc);
  if (kb == 48 && !swiglu) chunks = std::max<int64_t>(chunks, 4);   // the multi-item kernel's K split
  size_t bytes = counters_bytes();
  if (chunks > 1) bytes += (size_t)chunks * B * n_rows * 4;
  return bytes;
}

// 16-wave work-groups leave 128 registers per lane: K chunks up to 4 only.
template <int MODE, int XMODE, int WPB, int SMAX>
static hipError_t launch_kc(int kc, dim3 grid, size_t lds, hipStream_t st, const GemmArgs& a) {
#define QK_GEMM_CASE(KC)                                                                                \
  case KC:                                                                                              \
    hipLaunchKernelGGL((gemm_q4k_kernel<KC, MODE, XMODE, WPB, SMAX>), grid, dim3(64 * WPB), lds, st, a); \
    break;
  if constexpr (WPB == 16) {
    switch (kc) {
      QK_GEMM_CASE(1)
      QK_GEMM_CASE(2)
      QK_GEMM_CASE(4)
      default: return hipErrorInvalidValue;
    }
  } else {
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
  }
#undef QK_GEMM_CASE
  return hipGetLastError();
}

template <int MODE, int XMODE, int SMAX>
static hipError_t launch_wpb(int wpb, int kc, dim3 grid, size_t lds, hipStream_t st, const GemmArgs& a) {
  switch (wpb) {
    case 4: return launch_kc<MODE, XMODE, 4, SMAX>(kc, grid, lds, st, a);
    case 8: return launch_kc<MODE, XMODE, 8, SMAX>(kc, grid, lds, st, a);
    case 16: return launch_kc<MODE, XMODE, 16, SMAX>(kc, grid, lds, st, a);
    default: return hipErrorInvalidValue;
  }
}

// kXNorm: the statistics fold sized for H <= 4096 (256 slots) or for the
// largest H (kSsMaxSlots); the other modes do not fold.
template <int MODE>
static hipError_t launch_norm(int wpb, int kc, dim3 grid, size_t lds, hipStream_t st, const GemmArgs& a) {
  if (a.ss_slots <= 256) return launch_wpb<MODE, kXNorm, 256>(wpb, kc, grid, lds, st, a);
  return launch_wpb<MODE, kXNorm, kSsMaxSlots>(wpb, kc, grid, lds, st, a);
}

static GemmArgs gemm_args(const GemmLaunch& L, int64_t n_tiles, int kb) {
  GemmArgs a{};
  a.W = reinterpret_cast<const uint8_t*>(L.W);
  a.X = L.X;
  a.gamma = L.gamma;
  a.ss_in = L.ss_in;
  a.Y = L.Y;
  a.residual = L.residual;
  a.ss_out = L.ss_out;
  a.A = L.A;
  char* p = reinterpret_cast<char*>(L.ws);
  a.counters = reinterpret_cast<unsigned*>(p);
  a.part = reinterpret_cast<float*>(p + counters_bytes());
  a.ldx = L.ldx;
  a.ldy = L.ldy;
  a.ldr = L.ldr;
  a.lda = L.lda;
  a.n_tiles = (int)n_tiles;
  a.kb = kb;
  a.B = L.B;
  a.f_tiles = (int)(n_tiles / 2);
  a.ss_slots = (int)(L.K / kSsCols);
  a.eps = L.eps;
  a.inv_k = 1.0f / (float)L.K;
  return a;
}

hipError_t launch_gemm(const GemmLaunch& L, hipStream_t st) {
  // fp16 activations without SwiGLU: one work-group per tile, K over its waves
  if (!L.force_kc && !L.force_wpb) {
    const hipError_t e = launch_gemm_wi(L, st);
    if (e != hipErrorNotSupported) return e;
  }
  if (!L.x_f32 && !L.swiglu) return launch_gemm_wk(L, st);
  const int64_t n_tiles = L.swiglu ? 2 * (L.n_rows / 16) : L.n_rows / 16;
  const int kb = (int)(L.K / 256);
  const int xmode = L.x_f32 ? (L.gamma ? kXNorm : kXF32Blocked) : kXF16;
  GemmConfig cfg = gemm_config(n_tiles, kb, L.B, L.swiglu, xmode);
  if (L.force_kc) cfg.kc = L.force_kc;
  if (L.force_wpb) cfg.wpb = L.force_wpb;
  const GemmArgs a = gemm_args(L, n_tiles, kb);
  const dim3 grid((unsigned)n_groups_of(n_tiles, L.swiglu, cfg.wpb), (unsigned)(kb / cfg.kc));
  const size_t lds = lds_bytes(L.B, cfg.kc, xmode);
  if (lds > 150 * 1024) return hipErrorInvalidValue;
  if (L.swiglu) {
    if (xmode == kXNorm) return launch_norm<1>(cfg.wpb, cfg.kc, grid, lds, st, a);
    return launch_wpb<1, kXF16, 0>(cfg.wpb, cfg.kc, grid, lds, st, a);
  }
  if (xmode == kXNorm) return launch_norm<0>(cfg.wpb, cfg.kc, grid, lds, st, a);
  return launch_wpb<0, kXF32Blocked, 0>(cfg.wpb, cfg.kc, grid, lds, st, a);
}


// QKV projection with the RoPE / append finish (MODE 2): one head per row
// group, so head_dim / 16 waves per work-group; K chunks 1, 2 or 4.
template <int WPB, int SMAX>
static hipError_t launch_qkv_kc(int kc, dim3 grid, size_t lds, hipStream_t st, const GemmArgs& a) {
  switch (kc) {
    case 1: hipLaunchKernelGGL((gemm_q4k_kernel<1, 2, kXNorm, WPB, SMAX>), grid, dim3(64 * WPB), lds, st, a); break;
    case 2: hipLaunchKernelGGL((gemm_q4k_kernel<2, 2, kXNorm, WPB, SMAX>), grid, dim3(64 * WPB), lds, st, a); break;
    case 4: hipLaunchKernelGGL((gemm_q4k_kernel<4, 2, kXNorm, WPB, SMAX>), grid, dim3(64 * WPB), lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_qkv_rope(const GemmLaunch& L, const RopeAppendArgs& ra, int head_dim, hipStream_t st) {
  const int64_t n_tiles = L.n_rows / 16;
  const int kb = (int)(L.K / 256);
  const int wpb = head_dim / 16;
  if (!L.x_f32 || !L.gamma || L.residual || L.ss_out || (wpb != 4 && wpb != 8)) return hipErrorInvalidValue;
  int kc = gemm_kc(n_tiles, kb, L.B, false, kXNorm, wpb);
  if (kc > 4 || kb % kc) kc = kb % 4 == 0 ? 4 : (kb % 2 == 0 ? 2 : 1);
  GemmArgs a = gemm_args(L, n_tiles, kb);
  a.ra = ra;
  const dim3 grid((unsigned)n_groups_of(n_tiles, false, wpb), (unsigned)(kb / kc));
  const size_t lds = lds_bytes(L.B, kc, kXNorm);
  const bool wide = a.ss_slots > 256;
  if (wpb == 8) return wide ? launch_qkv_kc<8, kSsMaxSlots>(kc, grid, lds, st, a) : launch_qkv_kc<8, 256>(kc, grid, lds, st, a);
  return wide ? launch_qkv_kc<4, kSsMaxSlots>(kc, grid, lds, st, a) : launch_qkv_kc<4, 256>(kc, grid, lds, st, a);
}

hipError_t launch_gemm_q4k_xf32(const void* W, int64_t N, int64_t K, const float* X, int64_t ldx, int B, float* Y,
                                int64_t ldy, const float* residual, int64_t ldr, void* ws, hipStream_t st,
                                int force_kc) {
  GemmLaunch L{};
  L.W = W; L.n_rows = N; L.K = K; L.X = X; L.x_f32 = true; L.ldx = ldx; L.B = B;
  L.Y = Y; L.ldy = ldy; L.residual = residual; L.ldr = ldr; L.ws = ws; L.force_kc = force_kc;
  return launch_gemm(L, st);
}

hipError_t launch_gemm_q4k_swiglu(const void* W, int64_t F, int64_t K, const uint16_t* X, int64_t ldx, int B,
                                  float* A, int64_t lda, void* ws, hipStream_t st, int force_kc) {
  GemmLaunch L{};
  L.W = W; L.n_rows = F; L.K = K; L.X = X; L.ldx = ldx; L.B = B; L.swiglu = true;
  L.A = A; L.lda = lda; L.ws = ws; L.force_kc = force_kc;
  return launch_gemm(L, st);
}

hipError_t launch_dequant_q4k(const void* W, int64_t n_blocks, float* out, hipStream_t st) {
  if (n_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_q4k_kernel, dim3((unsigned)n_blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint8_t*>(W), n_blocks, out);
  return hipGetLastError();
}

}  // namespace qk
