// Device code of the flash-decode attention: KV tile loads (fp16, Q8_0 or E4M3),
// the online softmax state and one 32-token tile on MFMA (described at the
// top of attn_decode.hip).
#pragma once

#include "common.h"
#include "internal.h"

namespace qk {

template <int D>
struct DimMap {
  static constexpr int NQK = D / 32;   // QK MFMAs per 16-row set
  static constexpr int NPV = D / 16;   // PV MFMAs (16-dim output tiles)
};

// int8 x 4 (one dword) -> two half2 (exact)
__device__ __forceinline__ void i8x4_to_h2x2(uint32_t w, half2_t& lo, half2_t& hi) {
  const uint32_t u = w ^ 0x80808080u;                              // b + 128
  const uint32_t plo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t phi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const half2_t off = {(half_t)-1152.f, (half_t)-1152.f};
  lo = as_h2(plo) + off;
  hi = as_h2(phi) + off;
}

__device__ __forceinline__ half8_t i8x8_to_h8(uint32_t w0, uint32_t w1) {
  half2_t a, b, c, d;
  i8x4_to_h2x2(w0, a, b);
  i8x4_to_h2x2(w1, c, d);
  half8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// E4M3 x 8 (two dwords, byte i = element i) -> fp16 x 8: exact (every E4M3
// value is an fp16 normal or zero), one conversion per two codes
__device__ __forceinline__ half8_t f8x8_to_h8(uint32_t w0, uint32_t w1) {
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  half8_t r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// One 32-token tile of keys and values held by a lane; keys and values each
// in their own cache format (kFmtF16, kFmtQ8, kFmtF8).
template <int D, int F>
struct KPart;
template <int D>
struct KPart<D, kFmtF16> {
  half8_t k[2][D / 32];
};
template <int D>
struct KPart<D, kFmtQ8> {
  uint32_t k[2][D / 32][2];
  uint32_t ks[D / 8];   // fp16 scales of tokens 8lg..8lg+7, D/32 blocks each (2 per dword)
};
template <int D>
struct KPart<D, kFmtF8> {
  uint32_t k[2][D / 32][2];
};
template <int D, int F>
struct VPart;
template <int D>
struct VPart<D, kFmtF16> {
  half8_t v[D / 16];
};
template <int D>
struct VPart<D, kFmtQ8> {
  uint32_t v[D / 16][2];
  uint32_t vs[D / 8];
};
template <int D>
struct VPart<D, kFmtF8> {
  uint32_t v[D / 16][2];
};
template <int D, int KF, int VF>
struct KVFrag : KPart<D, KF>, VPart<D, VF> {};

struct AttnArgs {
  const uint8_t* k;
  const uint8_t* v;
  const uint16_t* ks;
  const uint16_t* vs;
  int n_kv, cap, n_slots;
  const int32_t* slot;
  const int32_t* n_ctx;
  int n_ctx_add;
  const half_t* Q;
  int Hq;
  float scale_log2;
  float* part_o;
  float* part_ml;
  int n_splits;      // partial-result rows per (b, q head): the most runs a sequence can have
  int runs_wanted;   // runs per sequence this call aims at (see attn_runs)
  // paged pool (slot = page, cap = page size, a power of two): token t of
  // sequence b is in page pages[b * max_pages + (t >> page_shift)]
  const int32_t* pages;
  int max_pages, page_shift;
  int seq_cap;       // most tokens a sequence can hold: cap, or max_pages * page size
  // prompt rows (attn_split_kernel MULTI): tok rows per work item, nrows rows
  int tok, nrows;
  // decode step with a Q8_0 part: the new token's rotated fp32 k and v
  // ([B][2][n_kv][D], staged by the QKV projection), quantized and stored
  // into the cache by the sequence's last run; null otherwise
  const float* kv_new;
};

// Runs of a sequence with n cached tokens (same in the split and merge
// kernels): ceil(n / kAttnChunk) rounded up to a multiple of the wanted
// count, at most one per 5 tiles but never fewer than ceil(n / kAttnChunk),
// and at most max_runs; 0 for n <= 0.
__host__ __device__ __forceinline__ int attn_runs(int n, int wanted, int max_runs) {
  if (n <= 0) return 0;
  const int tiles = (n + 31) / 32;
  const int need = (n + kAttnChunk - 1) / kAttnChunk;   // never more than kAttnChunk tokens per run
  int r = (need + wanted - 1) / wanted * wanted;
  const int by_tiles = tiles / 5 > 1 ? tiles / 5 : 1;
  if (r > by_tiles) r = by_tiles;
  if (r < need) r = need;
  if (r > max_runs) r = max_runs;
  return r;
}

// O[b][h] = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j over the splits, j in
// run order.  Up to kMergeBatch runs' (m, l, o) are loaded in one batch, so
// the merge costs one memory round trip (the running maximum is rescaled
// between batches).
constexpr int kMergeBatch = 8;
// Output element (b, h, d).  Paged: slot holds no slots (any readable
// int32[B]; its values are ignored).
__device__ __forceinline__ void attn_merge_elem(const MergeArgs& mg, int b, int h, int d) {
  const float* __restrict__ part_o = mg.part_o;
  const float* __restrict__ part_ml = mg.part_ml;
  const int n_splits = mg.n_splits, runs_wanted = mg.runs_wanted, paged = mg.paged, n_ctx_add = mg.n_ctx_add;
  const int cap = mg.cap, n_slots = mg.n_slots, Hq = mg.Hq, D = mg.D;
  const int32_t* slot = mg.slot;
  const int32_t* n_ctx = mg.n_ctx;
  float* O = mg.O;
  half_t* O16 = mg.O16;
  const size_t row0 = ((size_t)b * Hq + h) * n_splits;
  // The first batch of run states is loaded before the run count is known
  // (rows row0 .. row0 + min(kMergeBatch, n_splits) - 1 always lie in the
  // partial area; rows past the count are never used), so the count's loads
  // and the states' loads make one memory round trip, not two.
  float m[kMergeBatch], l[kMergeBatch], o[kMergeBatch];
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j) {
    const size_t row = row0 + (j < n_splits ? j : 0);
    m[j] = part_ml[2 * row];
    l[j] = part_ml[2 * row + 1];
    o[j] = part_o[row * D + d];
  }
  __asm__ volatile("" ::: "memory");   // keep the loads above ahead of the run count's
  const int bn = mg.tok > 1 ? min(b / mg.tok * mg.tok + mg.tok - 1, mg.nrows - 1) : b;
  int n = n_ctx[bn] + n_ctx_add;
  if (n > cap) n = cap;               // cap: the most tokens a sequence holds
  const int s = slot[b];   // unconditional: no branch ahead of the loads above
  if (n < 0 || (!paged && (s < 0 || s >= n_slots))) n = 0;
  const int ns = attn_runs(n, runs_wanted, n_splits);
  // first batch: selects rather than branches, so that its loads stay
  // unconditional and go out together with those of the run count (the
  // values equal the branchy form: fmax with -inf and additions of +0)
  float big = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j) big = fmaxf(big, j < ns ? m[j] : -__builtin_inff());
  // runs without a valid token (all their tiles on unmapped pages) carry
  // m = -inf, l = 0; a reference of 0 while no run has a finite maximum keeps
  // their weights at 0 rather than NaN
  float num = 0.f, den = 0.f;
  float bref = big == -__builtin_inff() ? 0.f : big;
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j) {
    const float w = exp2f(m[j] - bref);
    den += j < ns ? w * l[j] : 0.f;
    num += j < ns ? w * o[j] : 0.f;
  }
  for (int j0 = kMergeBatch; j0 < ns; j0 += kMergeBatch) {
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const size_t row = row0 + (j0 + j < ns ? j0 + j : j0);
      m[j] = part_ml[2 * row];
      l[j] = part_ml[2 * row + 1];
      o[j] = part_o[row * D + d];
    }
    float nb = big;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      if (j0 + j < ns) nb = fmaxf(nb, m[j]);
    const float nref = nb == -__builtin_inff() ? 0.f : nb;
    const float fr = exp2f(bref - nref);
    num *= fr;
    den *= fr;
    big = nb;
    bref = nref;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      if (j0 + j < ns) {
        const float w = exp2f(m[j] - bref);
        den += w * l[j];
        num += w * o[j];
      }
  }
  // no run with a valid token (or no token at all): O = 0
  const float out = den > 0.f ? num / den : 0.f;
  const size_t oi = ((size_t)b * Hq + h) * D + d;
  if (O) O[oi] = out;
  if (O16) O16[oi] = (half_t)out;
}

// Keys (and their Q8_0 scales) of the 32-token tile at t0; head_row0 =
// (slot * n_kv + g) * cap is the index of token 0 of this head.  fp16 and
// E4M3 lanes hold dims (D/4) lg + 8j .. +7 of their tokens, Q8_0 lanes dims
// 32j + 8lg .. +7 (one MFMA per 32-dim block and scale).
template <int D, int KF, int VF>
__device__ __forceinline__ void load_k(KVFrag<D, KF, VF>& f, const AttnArgs& a, size_t head_row0, int t0, int lg,
                                       int m) {
  if constexpr (KF == kFmtF8) {
    const uint8_t* kb = a.k + head_row0 * D;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int tok = t0 + 8 * (m >> 2) + 4 * hf + (m & 3);
      const uint8_t* row = kb + (size_t)tok * D + (D / 4) * lg;
#pragma unroll
      for (int j2 = 0; j2 < D / 64; ++j2) {
        const uint4 w = *reinterpret_cast<const uint4*>(row + 16 * j2);
        f.k[hf][2 * j2][0] = w.x;
        f.k[hf][2 * j2][1] = w.y;
        f.k[hf][2 * j2 + 1][0] = w.z;
        f.k[hf][2 * j2 + 1][1] = w.w;
      }
    }
  } else if constexpr (KF == kFmtF16) {
    const half_t* kb = reinterpret_cast<const half_t*>(a.k) + head_row0 * D;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int tok = t0 + 8 * (m >> 2) + 4 * hf + (m & 3);
      const half_t* row = kb + (size_t)tok * D + (D / 4) * lg;
#pragma unroll
      for (int j = 0; j < D / 32; ++j) f.k[hf][j] = *reinterpret_cast<const half8_t*>(row + 8 * j);
    }
  } else {
    const uint8_t* kb = a.k + head_row0 * D;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int tok = t0 + 8 * (m >> 2) + 4 * hf + (m & 3);
      const uint8_t* row = kb + (size_t)tok * D + 8 * lg;
#pragma unroll
      for (int j = 0; j < D / 32; ++j) {
        const uint2 w = *reinterpret_cast<const uint2*>(row + 32 * j);
        f.k[hf][j][0] = w.x;
        f.k[hf][j][1] = w.y;
      }
    }
    const uint32_t* ksb = reinterpret_cast<const uint32_t*>(a.ks + (head_row0 + t0 + 8 * lg) * (D / 32));
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const u32x4 x = reinterpret_cast<const u32x4*>(ksb)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) f.ks[4 * i + e] = x[e];
    }
  }
}

// Values (and their Q8_0 scales) of the same tile, from the value cache
// transposed within 32-token blocks ([cap/32][D][32] per head: the tile at t0
// is one contiguous run; lane (lg, m) reads tokens 8lg..8lg+7 of dim 16i + m).
template <int D, int KF, int VF>
__device__ __forceinline__ void load_v(KVFrag<D, KF, VF>& f, const AttnArgs& a, size_t head_row0, int t0, int lg,
                                       int m) {
  if constexpr (VF == kFmtF8) {
    const uint8_t* vb = a.v + head_row0 * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const uint2 w = *reinterpret_cast<const uint2*>(vb + ((size_t)(t0 >> 5) * D + 16 * i + m) * 32 + 8 * lg);
      f.v[i][0] = w.x;
      f.v[i][1] = w.y;
    }
  } else if constexpr (VF == kFmtF16) {
    const half_t* vb = reinterpret_cast<const half_t*>(a.v) + head_row0 * D;  // [D][cap] of this head
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      f.v[i] = *reinterpret_cast<const half8_t*>(vb + ((size_t)(t0 >> 5) * D + 16 * i + m) * 32 + 8 * lg);
  } else {
    const uint8_t* vb = a.v + head_row0 * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const uint2 w = *reinterpret_cast<const uint2*>(vb + ((size_t)(t0 >> 5) * D + 16 * i + m) * 32 + 8 * lg);
      f.v[i][0] = w.x;
      f.v[i][1] = w.y;
    }
    const uint32_t* vsb = reinterpret_cast<const uint32_t*>(a.vs + (head_row0 + t0 + 8 * lg) * (D / 32));
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const u32x4 y = reinterpret_cast<const u32x4*>(vsb)[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) f.vs[4 * i + e] = y[e];
    }
  }
}

// fp16 scale of local token e (0..7) and block j from the packed scale words
template <int D>
__device__ __forceinline__ float scale_at(const uint32_t (&w)[D / 8], int e, int j) {
  const int idx = e * (D / 32) + j;  // fp16 index
  const uint32_t word = w[idx >> 1];
  return h2f((idx & 1) ? (word >> 16) : (word & 0xffffu));
}

template <int D, bool Q8>
struct AttnState {
  floatx4 o[D / 16];
  float m;   // running max (log2 units), same in the 4 lane groups
  float l;   // this lane group's share of the running denominator
  int ex;   // Q8_0: o is kept multiplied by 2^ex (never increases)
};


// fp16 hi/lo operands of the value MFMA are formed from p * 2^kPScale so that
// they stay clear of fp16 subnormals; the result is scaled back at the end
constexpr int kPScale = 14;

// One 32-token tile.  mid() is called once the scores and the softmax update
// are done, before the value products (the caller issues the next tile's
// value loads there, into registers this tile's keys no longer need).  The
// fp16 values of out-of-range tokens are zeroed in place in f.
// PERCOL: the columns are different query tokens of one sequence (prompt
// rows), and vcol (this lane's column, <= valid) is the number of the tile's
// tokens that column may attend to; scores past it are masked.  Otherwise
// every column sees the same valid tokens (vcol unused).
// PLO = false: the value products take p rounded to fp16 alone (no low half),
// for a caller that rounds O to fp16 right after.
template <int D, int KF, int VF, bool PERCOL = false, bool PLO = true, typename Mid>
__device__ __forceinline__ void attn_tile(AttnState<D, VF == kFmtQ8>& st, KVFrag<D, KF, VF>& f,
                                          const half8_t (&qf)[D / 32], float scale_log2, int valid, int lg,
                                          const Mid& mid, int vcol = 0) {
  // valid = number of tokens of this 32-token tile that are in range (0..32;
  // 0 for a tile on an unmapped page of a paged pool): data past it is never
  // used
  float sc[8];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KF == kFmtF16) {
#pragma unroll
      for (int j = 0; j < D / 32; ++j) acc = mfma16x16x32(f.k[hf][j], qf[j], acc);
    } else if constexpr (KF == kFmtF8) {
#pragma unroll
      for (int j = 0; j < D / 32; ++j) acc = mfma16x16x32(f8x8_to_h8(f.k[hf][j][0], f.k[hf][j][1]), qf[j], acc);
    } else {
#pragma unroll
      for (int j = 0; j < D / 32; ++j) {
        const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
        const floatx4 part = mfma16x16x32(i8x8_to_h8(f.k[hf][j][0], f.k[hf][j][1]), qf[j], zero);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(scale_at<D>(f.ks, 4 * hf + i, j), part[i], acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[4 * hf + i] = acc[i] * scale_log2;
  }
  if constexpr (PERCOL) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sc[e] = (8 * lg + e < vcol) ? sc[e] : -__builtin_inff();
  } else if (valid < 32) {   // uniform branch; selects inside
#pragma unroll
    for (int e = 0; e < 8; ++e) sc[e] = (8 * lg + e < valid) ? sc[e] : -__builtin_inff();
  }
  float tmax = sc[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, sc[e]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float mnew = fmaxf(st.m, tmax);
  // while no valid token has been seen (a masked tile, valid = 0, first) the
  // maximum stays -inf; a reference of 0 then keeps corr and p at 0, not NaN
  const float mref = mnew == -__builtin_inff() ? 0.f : mnew;
  const float corr = exp2f(st.m - mref);   // 0 on the first tile (m = -inf)
  st.m = mnew;
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = exp2f(sc[e] - mref);
    psum += p[e];
  }
  st.l = st.l * corr + psum;
  // Q8_0 values: p * scale is brought near 2^13..2^14 by an exact power of
  // two taken from the largest value scale of the tile's in-range tokens (over
  // all blocks), so the fp16 hi/lo pair keeps ~22 bits instead of sinking into
  // fp16 subnormals; the exponent never increases, and a smaller one rescales
  // o by fr together with the softmax correction.  A tile whose 32 tokens are
  // all in range (every tile but a run's last) takes the maximum with packed
  // fp16 instructions over the scale words; in a partial tile an out-of-range
  // token's scale may hold any bits and is selected away, never multiplied in.
  float ocorr = corr;
  if constexpr (VF == kFmtQ8) {
    const int lim = valid - 8 * lg;
    float vmax = 0.f;
    if (valid == 32) {   // uniform across the wave
      half2_t m2 = __builtin_elementwise_abs(as_h2(f.vs[0]));
#pragma unroll
      for (int w = 1; w < D / 8; ++w) m2 = __builtin_elementwise_max(m2, __builtin_elementwise_abs(as_h2(f.vs[w])));
      vmax = fmaxf((float)m2[0], (float)m2[1]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) vmax = fmaxf(vmax, e < lim ? fabsf(scale_at<D>(f.vs, e, c)) : 0.f);
    }
    vmax = fmaxf(vmax, __shfl_xor(vmax, 16));
    vmax = fmaxf(vmax, __shfl_xor(vmax, 32));
    const int exv = 13 - ((int)((__builtin_bit_cast(uint32_t, vmax) >> 23) & 255u) - 127);
    const int exn = (vmax > 0.f && exv < st.ex) ? exv : st.ex;
    ocorr = corr * exp2i(exn - st.ex);   // the power of two is 1 when the exponent stays
    st.ex = exn;
  }
  // once the running maxima settle most tiles change none of them: the
  // rescale by 1 is skipped (same values) when no lane of the wave needs it
  if (__ballot(ocorr != 1.f) != 0) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      st.o[i][0] *= ocorr; st.o[i][1] *= ocorr; st.o[i][2] *= ocorr; st.o[i][3] *= ocorr;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  mid();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (VF == kFmtF8) {
    half8_t phi;
    [[maybe_unused]] half8_t plo;
    const float ps = exp2i(kPScale);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = p[e] * ps;
      const half_t h = (half_t)pe;
      phi[e] = h;
      if constexpr (PLO) plo[e] = (half_t)(pe - (float)h);
    }
    const int lim = valid - 8 * lg;   // codes past the end may be NaN codes: never reach the MFMA
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      half8_t vf = f8x8_to_h8(f.v[i][0], f.v[i][1]);
      if (valid < 32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = e < lim ? vf[e] : (half_t)0.f;
      }
      st.o[i] = mfma16x16x32(vf, phi, st.o[i]);
      if constexpr (PLO) st.o[i] = mfma16x16x32(vf, plo, st.o[i]);
    }
  } else if constexpr (VF == kFmtF16) {
    half8_t phi;
    [[maybe_unused]] half8_t plo;
    const float ps = exp2i(kPScale);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = p[e] * ps;
      const half_t h = (half_t)pe;
      phi[e] = h;
      if constexpr (PLO) plo[e] = (half_t)(pe - (float)h);
    }
    if (valid < 32) {  // never let values past the end reach the MFMA (0 * NaN)
      const int lim = valid - 8 * lg;
#pragma unroll
      for (int i = 0; i < D / 16; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= lim) f.v[i][e] = (half_t)0.f;
    }
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      st.o[i] = mfma16x16x32(f.v[i], phi, st.o[i]);
      if constexpr (PLO) st.o[i] = mfma16x16x32(f.v[i], plo, st.o[i]);
    }
  } else {
    const int lim = valid - 8 * lg;   // tokens of this lane at or past lim are out of range
    const bool full = valid == 32;    // uniform across the wave
    const float fc = exp2i(st.ex);
    float pf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = p[e] * fc;   // exact (a power of two)
    // -1 in a register the compiler cannot see through, so that hi * -1 + pv
    // stays one mixed-precision fused operation on the fp16 hi
    float m1 = -1.f;
    asm volatile("" : "+v"(m1));
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      // hi = pv rounded to the nearest fp16, lo = the exact remainder pv - hi
      // rounded likewise: hi + lo is pv to 2^-22 relative.  pv and the
      // remainder are single fused operations on the fp16 scale and hi
      half8_t phi;
      [[maybe_unused]] half8_t plo;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float pv0 = __builtin_fmaf(pf[e], scale_at<D>(f.vs, e, c), 0.f);
        float pv1 = __builtin_fmaf(pf[e + 1], scale_at<D>(f.vs, e + 1, c), 0.f);
        if (!full) {
          pv0 = e < lim ? pv0 : 0.f;
          pv1 = e + 1 < lim ? pv1 : 0.f;
        }
        const half_t h0 = (half_t)pv0, h1 = (half_t)pv1;
        phi[e] = h0;
        phi[e + 1] = h1;
        if constexpr (PLO) {
          plo[e] = (half_t)__builtin_fmaf((float)h0, m1, pv0);
          plo[e + 1] = (half_t)__builtin_fmaf((float)h1, m1, pv1);
        }
      }
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * c + ii;
        half8_t vf = i8x8_to_h8(f.v[i][0], f.v[i][1]);
        st.o[i] = mfma16x16x32(vf, phi, st.o[i]);
        if constexpr (PLO) st.o[i] = mfma16x16x32(vf, plo, st.o[i]);
      }
    }
  }
}

}  // namespace qk
