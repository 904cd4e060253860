// Split-K flash-decode GQA attention over a slot-arena KV cache or a paged
// pool: fp16, Q8_0, mixed, or E4M3 keys and values.
// (P1, P2, P3: the three pages listed, with their titles, at the top of include/qkdec.h.)
//
// P2 "The two halves of a decode-step memory bill": each sequence reads its
// whole private cache every step; P3 FAQ "Is KV cache quantization a kernel
// change or a storage change?": a quantized cache is dequantized inside the
// fused attention kernel.  One work-group of 4 waves handles one work item
// (sequence b, KV head g, run c of the sequence's 32-token tiles; the runs
// split the tiles evenly, as many as fill the chip: attn_runs): wave w takes
// the run's tiles w, w + 4, ...; the four waves' states are merged in LDS and
// the merge of the runs uses their log-sum-exp weights (attn_combine_kernel).
//
// Both contractions run on MFMA v_mfma_f32_16x16x32_f16 with the G <= 16
// query heads of the group as the N columns (zero padded):
//   S^T = K Q^T:  A = 16 cached keys (rows) x 32 dims, B = q^T.
//     Two MFMA row sets per 32-token tile: set hf takes tokens
//     8*(m>>2) + 4*hf + (m&3) as row m, so lane (lg, h) ends up holding the
//     scores of tokens 8*lg .. 8*lg+7 of head h.
//   O^T = V^T P^T: A = 16 dims x 32 tokens of the transposed V cache (each
//     lane reads 8 consecutive tokens of one dim), B = P^T, which is exactly
//     the score layout above.  Lane (lg, h) accumulates O[h][16i + 4lg + rr].
// P is carried as an fp16 hi/lo pair (p ~ hi + lo to 2^-22) so the value sum
// keeps fp32-level accuracy.  Scores are kept in log2 units (exp2).
//
// Q8_0: keys are int8 + one fp16 scale per (token, 32 dims).  Each QK MFMA
// covers exactly one 32-dim block; its fp32 result is multiplied by the
// token's block scale.  Values: the per-(token, block) scale is folded into P
// before the hi/lo split, with one power-of-two exponent per tile and head
// (from the tile's largest value scale) keeping the pair clear of fp16
// subnormals.  int8 -> fp16 is exact (byte permute into the
// mantissa of 1024+128+x, then one packed subtract).
//
// E4M3 (no scale): each pair of codes becomes two fp16 values in one hardware
// conversion (exact), after which keys and values take the fp16 path.
//
// Paged pool (PAGED): the cache layer's slots are fixed-size pages and each
// 32-token tile's page comes from the sequence's row of the page table (the
// run's entries staged in LDS at the start); everything else is the arena
// kernel.
#include <algorithm>
#include <type_traits>

#include "attn_dev.h"
#include "common.h"
#include "internal.h"
#include "kv_dev.h"

namespace qk {

constexpr int kAttnWaves = 4;

// Two waves per SIMD: with the split key / value prefetch the fp16 kernel
// fits 256 registers without spilling (see the run targets next to kAttnChunk)
//
// MULTI (prompt rows, arena only): work item z covers rows z * tok .. + tok - 1
// of one sequence (consecutive positions); column r is head r % G of row
// z * tok + r / G.  The runs are those of the item's last row, and each
// column masks the keys past its own row's length.
template <int D, int KF, int VF, bool PAGED, bool MULTI = false>
__global__ void __launch_bounds__(64 * kAttnWaves, 2) attn_split_kernel(AttnArgs a) {
  const int c = blockIdx.x, g = blockIdx.y;
  const int G = a.Hq / a.n_kv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lg = lane >> 4, r = lane & 15;
  // bl: the row whose length sets the runs; (b, hcol): this lane's column
  int bl, b, hcol;
  bool colv;
  if constexpr (MULTI) {
    const int z = blockIdx.z, u = r / G;
    bl = min(z * a.tok + a.tok - 1, a.nrows - 1);
    hcol = r - u * G;
    colv = u < a.tok && z * a.tok + u < a.nrows;
    b = colv ? z * a.tok + u : bl;
  } else {
    bl = b = blockIdx.z;
    hcol = r;
    colv = r < G;
  }
  const int s = PAGED ? 0 : a.slot[bl];
  int n = a.n_ctx[bl] + a.n_ctx_add;
  if (n > a.seq_cap) n = a.seq_cap;
  if (n < 0 || (!PAGED && (s < 0 || s >= a.n_slots))) n = 0;
  const int runs = attn_runs(n, a.runs_wanted, a.n_splits);
  if (c >= runs) return;
  const int tiles = (n + 31) / 32;
  const int t_begin = 32 * (c * tiles / runs);
  const int t_end = min(32 * ((c + 1) * tiles / runs), n);
  // MULTI: this column's length (at most the item's)
  int ncol = n;
  if constexpr (MULTI) ncol = colv ? min(max(a.n_ctx[b] + a.n_ctx_add, 0), n) : 0;

  half8_t qf[D / 32];
  {
    const bool hv = colv;
    const half_t* qrow = a.Q + ((size_t)b * a.Hq + g * G + (hv ? hcol : 0)) * D;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const int d0 = KF == kFmtQ8 ? (32 * j + 8 * lg) : ((D / 4) * lg + 8 * j);
      qf[j] = hv ? *reinterpret_cast<const half8_t*>(qrow + d0) : half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  const size_t head_row0 = ((size_t)s * a.n_kv + g) * a.cap;
  // Paged: the run's page entries (a run is at most kAttnChunk tokens, so at
  // most kAttnChunk / 32 + 1 pages) are staged in LDS once, so a tile's lookup
  // is an LDS read rather than a global load.  An entry outside the pool (a
  // page not handed out, -1) is staged as -1: its tiles are loaded from page 0
  // (never outside the pool) and masked out of the softmax entirely.
  __shared__ int s_pg[PAGED ? kAttnChunk / 32 + 1 : 1];
  const int pg0 = t_begin >> a.page_shift;
  if constexpr (PAGED) {
    const int npg = ((t_end - 1) >> a.page_shift) - pg0 + 1;
    if ((int)threadIdx.x < npg && (int)threadIdx.x < kAttnChunk / 32 + 1) {
      const int pg = a.pages[(size_t)b * a.max_pages + pg0 + threadIdx.x];
      s_pg[threadIdx.x] = (pg < 0 || pg >= a.n_slots) ? -1 : pg;
    }
    __syncthreads();
  }
  // (row of token 0 of this head, position within it) of the tile at t; false
  // for a tile on an unmapped page
  auto tile_at = [&](int t, size_t& row0, int& tt) -> bool {
    if constexpr (PAGED) {
      const int pg = __builtin_amdgcn_readfirstlane(s_pg[(t >> a.page_shift) - pg0]);
      row0 = ((size_t)(pg < 0 ? 0 : pg) * a.n_kv + g) * a.cap;
      tt = t & (a.cap - 1);
      return pg >= 0;
    } else {
      row0 = head_row0;
      tt = t;
      return true;
    }
  };

  AttnState<D, VF == kFmtQ8> st;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) st.o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  st.m = -__builtin_inff();
  st.l = 0.f;
  st.ex = 127;

  // The new token of a decode step with a Q8_0 part (kv_new): its 32-dim
  // blocks were split over two work-groups of the QKV projection, so the
  // sequence's last run quantizes it here.  The tile loop leaves the token
  // out (its cache bytes are not written yet); after its tiles the last wave,
  // which has the fewest, reads the staged fp32 key and value, forms them
  // (the appends' Q8_0 arithmetic, or fp16 rounding for an fp16 part),
  // stores the Q8_0 codes and scales into the cache and adds the token to its
  // state.  (Its load is issued only then: a load issued before the loop on
  // one wave's path alone makes the compiler wait for every tile load.)
  constexpr bool kStage = !MULTI && (KF == kFmtQ8 || VF == kFmtQ8);
  constexpr int kSubWave = kAttnWaves - 1;
  __shared__ float s_new[kStage ? 2 * D : 1];   // k, then v
  bool sub = false;
  size_t nrow0 = 0;
  int ntt = 0;
  if constexpr (kStage) {
    const int tn = a.n_ctx[bl] + a.n_ctx_add - 1;   // its position (n - 1 unless n was clamped)
    sub = a.kv_new && c == runs - 1 && tn == n - 1 && tile_at(tn, nrow0, ntt);
  }

  // this wave's tiles: wave, wave + 4, ...  The next tile's keys are issued
  // before the current tile is processed, its values once the current tile's
  // softmax is done (two tiles of keys and values are never held at once)
  const int ntiles = (t_end - t_begin + 31) / 32;
  if (wave < ntiles) {
    KVFrag<D, KF, VF> buf[2];
    size_t row0;
    int tt;
    bool mapped = tile_at(t_begin + 32 * wave, row0, tt);
    load_k(buf[0], a, row0, tt, lg, r);
    load_v(buf[0], a, row0, tt, lg, r);
    for (int it = wave; it < ntiles; it += 2 * kAttnWaves) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int i = it + p * kAttnWaves;
        if (i < ntiles) {
          const int nx = (i + kAttnWaves < ntiles) ? i + kAttnWaves : i;
          const bool cur_mapped = mapped;
          mapped = tile_at(t_begin + 32 * nx, row0, tt);
          load_k(buf[p ^ 1], a, row0, tt, lg, r);
          const int t0 = t_begin + 32 * i;
          // a tile on an unmapped page has no valid token (every score -inf);
          // the staged new token (sub: the run's last token) is added later
          const int valid = cur_mapped ? min(32, t_end - t0) - (sub && t0 + 32 >= t_end ? 1 : 0) : 0;
          if constexpr (MULTI)
            attn_tile<D, KF, VF, true>(st, buf[p], qf, a.scale_log2, valid, lg,
                                       [&]() { load_v(buf[p ^ 1], a, row0, tt, lg, r); },
                                       min(max(ncol - t0, 0), valid));
          else
            attn_tile(st, buf[p], qf, a.scale_log2, valid, lg, [&]() { load_v(buf[p ^ 1], a, row0, tt, lg, r); });
        }
      }
    }
  }

  // undo the operand scaling of the value products (exact powers of two)
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const float un = VF == kFmtQ8 ? exp2i(-st.ex) : exp2i(-kPScale);
    st.o[i][0] *= un; st.o[i][1] *= un; st.o[i][2] *= un; st.o[i][3] *= un;
  }
  if constexpr (kStage) {
    if (sub && wave == kSubWave) {
      // lane: dims 2 lane, 2 lane + 1 of each part
      const bool has = 2 * lane < D;
      float2 xs[2];
#pragma unroll
      for (int part = 0; part < 2; ++part)
        xs[part] = has ? *reinterpret_cast<const float2*>(a.kv_new + (((size_t)b * 2 + part) * a.n_kv + g) * D +
                                                         2 * lane)
                       : make_float2(0.f, 0.f);
      float y[2][2];
#pragma unroll
      for (int part = 0; part < 2; ++part) {
        const float x0 = xs[part].x, x1 = xs[part].y;
        if ((part == 0 ? KF : VF) == kFmtQ8) {
          // block maximum over the 16 lanes of one 32-dim block (exact in fp32)
          float am = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
          for (int o = 8; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
          int8_t q0, q1;
          uint16_t db;
          q8_encode((double)x0, (double)am, q0, db);
          q8_encode((double)x1, (double)am, q1, db);
          const float dd = h2f(db);
          y[part][0] = (float)q0 * dd;
          y[part][1] = (float)q1 * dd;
          if (has) {
            const int d0 = 2 * lane;
            if (part == 0) {
              *reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(a.k) + (nrow0 + ntt) * D + d0) =
                  (uint16_t)((uint8_t)q0 | ((uint16_t)(uint8_t)q1 << 8));
              if ((lane & 15) == 0) const_cast<uint16_t*>(a.ks)[(nrow0 + ntt) * (D / 32) + d0 / 32] = db;
            } else {
              // values transposed within 32-token blocks ([cap/32][D][32] per head)
              uint8_t* vc = const_cast<uint8_t*>(a.v) + nrow0 * D;
              const size_t base = ((size_t)(ntt >> 5) * D + d0) * 32 + (ntt & 31);
              vc[base] = (uint8_t)q0;
              vc[base + 32] = (uint8_t)q1;
              if ((lane & 15) == 0) const_cast<uint16_t*>(a.vs)[(nrow0 + ntt) * (D / 32) + d0 / 32] = db;
            }
          }
        } else {
          // an fp16 part: the projection stored it; its cached value
          y[part][0] = h2f(f2h_bits(x0));
          y[part][1] = h2f(f2h_bits(x1));
        }
      }
      if (has) {
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          s_new[part * D + 2 * lane] = y[part][0];
          s_new[part * D + 2 * lane + 1] = y[part][1];
        }
      }
      // its score for this lane's column over this lane's dims of q (the
      // tile step's layout), summed over the lane groups
      float sp = 0.f;
#pragma unroll
      for (int j = 0; j < D / 32; ++j) {
        const int d0 = KF == kFmtQ8 ? (32 * j + 8 * lg) : ((D / 4) * lg + 8 * j);
#pragma unroll
        for (int k = 0; k < 8; ++k) sp = __builtin_fmaf((float)qf[j][k], s_new[d0 + k], sp);
      }
      sp += __shfl_xor(sp, 16);
      sp += __shfl_xor(sp, 32);
      const float sc = sp * a.scale_log2;
      const float mnew = fmaxf(st.m, sc);
      const float co = exp2f(st.m - mnew);   // 0 while the wave saw no token (m = -inf)
      const float pn = exp2f(sc - mnew);
      st.l = st.l * co + (lg == 0 ? pn : 0.f);   // one lane group's share carries it
#pragma unroll
      for (int i = 0; i < D / 16; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          st.o[i][rr] = __builtin_fmaf(pn, s_new[D + 16 * i + 4 * lg + rr], st.o[i][rr] * co);
      st.m = mnew;
    }
  }
  // merge the four waves' states (same lane layout in every wave) in LDS;
  // a wave without tiles has m = -inf, l = 0, o = 0 and weighs nothing
  __shared__ float s_m[kAttnWaves][64], s_l[kAttnWaves][64];
  __shared__ floatx4 s_o[kAttnWaves][D / 16][64];
  s_m[wave][lane] = st.m;
  s_l[wave][lane] = st.l;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) s_o[wave][i][lane] = st.o[i];
  __syncthreads();
  if (wave != 0) return;
  float mm = s_m[0][lane];
#pragma unroll
  for (int w = 1; w < kAttnWaves; ++w) mm = fmaxf(mm, s_m[w][lane]);
  // every wave without a valid token (m = -inf): weights 0, not NaN
  const float mref = mm == -__builtin_inff() ? 0.f : mm;
  float wt[kAttnWaves];
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) wt[w] = exp2f(s_m[w][lane] - mref);
  st.m = mm;
  st.l = 0.f;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) st.l += wt[w] * s_l[w][lane];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const floatx4 ow = s_o[w][i][lane];
      acc[0] += wt[w] * ow[0]; acc[1] += wt[w] * ow[1]; acc[2] += wt[w] * ow[2]; acc[3] += wt[w] * ow[3];
    }
    st.o[i] = acc;
  }
  const float ltot = st.l + __shfl_xor(st.l, 16);
  const float lsum = ltot + __shfl_xor(ltot, 32);
  if (colv) {
    const size_t row = ((size_t)b * a.Hq + g * G + hcol) * a.n_splits + c;
    float* po = a.part_o + row * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) *reinterpret_cast<floatx4*>(po + 16 * i + 4 * lg) = st.o[i];
    if (lg == 0) {
      a.part_ml[2 * row] = st.m;
      a.part_ml[2 * row + 1] = lsum;
    }
  }
}

__global__ void attn_combine_kernel(const MergeArgs m) { attn_merge_elem(m, blockIdx.y, blockIdx.x, threadIdx.x); }

hipError_t launch_attn_decode(const qkdec_kv_layer& kv, const int32_t* slot, const int32_t* n_ctx, int B,
                              const uint16_t* Q, int n_q_heads, float scale, float* O, uint16_t* O16,
                              float* partials, int n_ctx_add, hipStream_t st, const int32_t* pages, int max_pages,
                              const float* kv_new) {
  AttnArgs a;
  a.kv_new = kv_new;
  a.k = reinterpret_cast<const uint8_t*>(kv.k);
  a.v = reinterpret_cast<const uint8_t*>(kv.v);
  a.ks = reinterpret_cast<const uint16_t*>(kv.k_scale);
  a.vs = reinterpret_cast<const uint16_t*>(kv.v_scale);
  a.n_kv = kv.n_kv_heads;
  a.cap = kv.capacity;
  a.n_slots = kv.n_slots;
  a.slot = slot;
  a.n_ctx = n_ctx;
  a.n_ctx_add = n_ctx_add;
  a.Q = reinterpret_cast<const half_t*>(Q);
  a.Hq = n_q_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.pages = pages;
  a.max_pages = pages ? max_pages : 0;
  a.page_shift = 0;
  while (pages && (1 << a.page_shift) < kv.capacity) ++a.page_shift;
  a.seq_cap = (int)attn_seq_cap(kv, pages ? max_pages : 0);   // at most 2^30 (checked by the entry points)
  a.tok = 1;
  a.nrows = B;
  a.n_splits = attn_max_runs(a.seq_cap, kv.n_kv_heads);
  a.runs_wanted = attn_runs_wanted(B, kv.n_kv_heads);
  const int D = kv.head_dim;
  const size_t n_rows = (size_t)B * n_q_heads * a.n_splits;
  a.part_o = partials;
  a.part_ml = partials + n_rows * D;
  // runs past a sequence's own count return at once
  const int max_runs = attn_runs(a.seq_cap, a.runs_wanted, a.n_splits);
  const dim3 grid(max_runs, kv.n_kv_heads, B);
  const dim3 blk(64 * kAttnWaves);
#define QK_ATTN(DD, KF, VF, PG) hipLaunchKernelGGL((attn_split_kernel<DD, KF, VF, PG>), grid, blk, 0, st, a)
#define QK_ATTN_D(DD, PG)                                                      \
  do {                                                                         \
    if (kf == kFmtF8) QK_ATTN(DD, kFmtF8, kFmtF8, PG);                         \
    else if (kf == kFmtQ8 && vf == kFmtQ8) QK_ATTN(DD, kFmtQ8, kFmtQ8, PG);    \
    else if (kf == kFmtQ8) QK_ATTN(DD, kFmtQ8, kFmtF16, PG);                   \
    else if (vf == kFmtQ8) QK_ATTN(DD, kFmtF16, kFmtQ8, PG);                   \
    else QK_ATTN(DD, kFmtF16, kFmtF16, PG);                                    \
  } while (0)
  const int kf = kv_k_fmt(kv.type), vf = kv_v_fmt(kv.type);
  if (pages) {
    if (D == 128) QK_ATTN_D(128, true);
    else QK_ATTN_D(64, true);
  } else {
    if (D == 128) QK_ATTN_D(128, false);
    else QK_ATTN_D(64, false);
  }
#undef QK_ATTN_D
#undef QK_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeArgs mg;
  mg.part_o = a.part_o;
  mg.part_ml = a.part_ml;
  mg.n_splits = a.n_splits;
  mg.runs_wanted = a.runs_wanted;
  mg.slot = pages ? n_ctx : slot;
  mg.paged = pages ? 1 : 0;
  mg.n_ctx = n_ctx;
  mg.n_ctx_add = n_ctx_add;
  mg.cap = a.seq_cap;
  mg.n_slots = kv.n_slots;
  mg.Hq = n_q_heads;
  mg.D = D;
  mg.tok = 1;
  mg.nrows = B;
  mg.O = O;
  mg.O16 = reinterpret_cast<half_t*>(O16);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(n_q_heads, B), dim3(D), 0, st, mg);
  return hipGetLastError();
}

// rows per work item of the prompt-row attention (1: the decode kernel)
static int attn_prefill_tok(int n_q_heads, int n_kv) {
  const int G = n_q_heads / n_kv;
  return (16 % G != 0 || G == 16) ? 1 : 16 / G;
}

int attn_prefill_splits(int B, int n_q_heads, const qkdec_kv_layer& kv) {
  const int tok = attn_prefill_tok(n_q_heads, kv.n_kv_heads);
  if (tok == 1) return attn_max_runs(kv.capacity, kv.n_kv_heads);
  const int groups = (B + tok - 1) / tok;
  const int by_len = (int)(((int64_t)kv.capacity + kAttnChunk - 1) / kAttnChunk);
  const int wanted = attn_runs_wanted(groups, kv.n_kv_heads);
  return (by_len + wanted - 1) / wanted * wanted;   // the most attn_runs gives (by_len >= 1)
}

size_t attn_prefill_partials_bytes(int max_rows, int n_q_heads, const qkdec_kv_layer& kv) {
  size_t most = 0;
  for (int b = 1; b <= max_rows; ++b) {
    const size_t rows = (size_t)b * n_q_heads * attn_prefill_splits(b, n_q_heads, kv);
    if (rows > most) most = rows;
  }
  return most * (size_t)(kv.head_dim + 2) * sizeof(float);
}

// ---- prompt rows: flash attention without a key split.  A work-group holds
// 64 query columns that share one KV head: H4 = min(G, 4) heads of the group
// times 64 / H4 consecutive prompt rows; wave w takes head w % H4 of 16 rows.
// Each 32-token key and value tile (codes, and for Q8_0 the block scales) is
// DMA'd to LDS once for all four waves, double-buffered, with the 16-byte
// chunks XOR-swizzled so the waves' fragment reads spread over the banks;
// every wave builds the decode kernel's fragments from LDS and runs its tile
// step (attn_tile, per-column causal masks) over all the keys its rows see,
// so the softmax state is final at the end: no partial results, no merge.
struct FlashArgs {
  const uint8_t* k;      // keys [slots][n_kv][cap][D] (fp16 or 8-bit codes)
  const uint8_t* v;      // values [slots][n_kv][cap/32][D][32]
  const uint16_t* ks;    // Q8_0 key scales [slots][n_kv][cap][D/32]
  const uint16_t* vs;    // Q8_0 value scales, the same shape
  int n_kv, cap, n_slots;
  const int32_t* slot;   // [rows] (one sequence: the first row's slot)
  const int32_t* pos;    // [rows] ascending; row r attends over pos[r] + n_add tokens
  int n_add, rows;
  const half_t* Q;       // [rows][Hq][D]
  int Hq, h4;
  float scale_log2;
  half_t* O16;           // [rows][Hq][D]
  // paged pool (PAGED): the sequence's page table row, pages of 2^page_shift
  // (= cap) tokens; a tile on an entry outside the pool is masked out
  const int32_t* pages;
  int max_pages, page_shift;
};

// Swizzle of the LDS tiles: the 16-byte chunk c of key row t (CK chunks a
// row) sits at slot fk_slot(t, c); chunk c of value row d at fv_slot(d, c).
template <int CK>
__device__ __forceinline__ int fk_slot(int t, int c) {
  return (c ^ (((t >> 1) & 12) | (t & 3))) & (CK - 1);
}
template <int CV>
__device__ __forceinline__ int fv_slot(int d, int c) {
  return CV == 4 ? c ^ ((d >> 2) & 3) : c ^ ((d >> 3) & 1);
}

template <int D, int KF, int VF, bool PAGED>
__global__ void __launch_bounds__(256, 2) attn_prefill_kernel(const FlashArgs a) {
  constexpr int KB = KF == kFmtF16 ? 2 : 1, VB = VF == kFmtF16 ? 2 : 1;   // bytes per element
  constexpr int CK = D * KB / 16, CV = 32 * VB / 16;                       // 16-byte chunks per row
  constexpr int NK = 32 * D * KB / 1024, NV = 32 * D * VB / 1024;          // 1 KB copies per tile
  constexpr bool KQ = KF == kFmtQ8, VQ = VF == kFmtQ8;
  __shared__ __attribute__((aligned(16))) uint8_t s_k0[32 * D * KB], s_k1[32 * D * KB];
  __shared__ __attribute__((aligned(16))) uint8_t s_v0[32 * D * VB], s_v1[32 * D * VB];
  // Q8_0 scales of the tile's 32 tokens, [32][D/32] fp16 as in the cache
  __shared__ __attribute__((aligned(16))) uint8_t s_ks0[KQ ? 2 * D : 16], s_ks1[KQ ? 2 * D : 16];
  __shared__ __attribute__((aligned(16))) uint8_t s_vs0[VQ ? 2 * D : 16], s_vs1[VQ ? 2 * D : 16];
  const int tx = threadIdx.x, lane = tx & 63, wave = __builtin_amdgcn_readfirstlane(tx >> 6);
  const int lg = lane >> 4, r = lane & 15;
  const int g = blockIdx.y, G = a.Hq / a.n_kv, h4 = a.h4, tb = 64 / h4;
  const int row_first = blockIdx.x * tb;
  const int head = g * G + blockIdx.z * h4 + wave % h4;
  const int row = row_first + (wave / h4) * 16 + r;   // this lane's column
  const bool colv = row < a.rows;
  const int last = min(row_first + tb - 1, a.rows - 1);
  const int s = PAGED ? 0 : a.slot[row_first];
  const int seq_cap = PAGED ? (a.max_pages << a.page_shift) : a.cap;
  int n = a.pos[last] + a.n_add;
  if (n > seq_cap) n = seq_cap;
  if (s < 0 || s >= a.n_slots || n < 0) n = 0;
  const int ncol = colv ? min(max(a.pos[row] + a.n_add, 0), n) : 0;
  // (row of token 0 of this head, position in it) of the tile at t0, and
  // whether the tile is on a page of the pool
  auto tile_at = [&](int t0, size_t& row0, int& tt) -> bool {
    if constexpr (PAGED) {
      const int pg = a.pages[t0 >> a.page_shift];
      const bool ok = pg >= 0 && pg < a.n_slots;
      row0 = ((size_t)(ok ? pg : 0) * a.n_kv + g) * a.cap;
      tt = t0 & (a.cap - 1);
      return ok;
    } else {
      row0 = ((size_t)s * a.n_kv + g) * a.cap;
      tt = t0;
      return true;
    }
  };

  half8_t qf[D / 32];
  {
    const half_t* qrow = a.Q + ((size_t)(colv ? row : last) * a.Hq + head) * D;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const int d0 = KQ ? (32 * j + 8 * lg) : ((D / 4) * lg + 8 * j);
      qf[j] = colv ? *reinterpret_cast<const half8_t*>(qrow + d0) : half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // the tile at t0 to LDS: NK + NV copies of 1 KB spread over the waves, then
  // the Q8_0 scales (2 D bytes each) by waves 0 and 1
  auto load_tile = [&](int t0l, uint8_t* sk, uint8_t* sv, uint8_t* sks, uint8_t* svs) {
    size_t head_row0;
    int t0;
    tile_at(t0l, head_row0, t0);
    const uint8_t* kh = a.k + head_row0 * D * KB;
    const uint8_t* vh = a.v + head_row0 * D * VB;
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int p = 0; p < (NK + NV + 3) / 4; ++p) {
      const int q = wave + 4 * p;
      if (q < NK) {
        const int kt = q * (1024 / (D * KB)) + ln / CK, sl = ln % CK;   // key row and slot of this lane
        const uint8_t* src = kh + ((size_t)(t0 + kt) * D * KB) + fk_slot<CK>(kt, sl) * 16;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&sk[q * 1024], 16, 0, 0);
      } else if (q < NK + NV) {
        const int i = q - NK;
        const int vd = i * (1024 / (32 * VB)) + ln / CV, sl = ln % CV;  // value row (dim) and slot
        const uint8_t* src = vh + ((size_t)(t0 >> 5) * D + vd) * 32 * VB + fv_slot<CV>(vd, sl) * 16;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&sv[i * 1024], 16, 0, 0);
      }
    }
    if constexpr (KQ) {
      if (wave == 0 && ln < D / 8) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.ks + (head_row0 + t0) * (D / 32)) + ln * 16;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)sks, 16, 0, 0);
      }
    }
    if constexpr (VQ) {
      if (wave == 1 && ln < D / 8) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.vs + (head_row0 + t0) * (D / 32)) + ln * 16;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)svs, 16, 0, 0);
      }
    }
  };
  auto wait_loads = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

  AttnState<D, VQ> st;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) st.o[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  st.m = -__builtin_inff();
  st.l = 0.f;
  st.ex = 127;
  const int ntiles = (n + 31) / 32;
  if (ntiles > 0) {
    load_tile(0, s_k0, s_v0, s_ks0, s_vs0);
    wait_loads();
    __syncthreads();
  }
  auto step = [&](auto bufc, int it) {
    constexpr int BUF = decltype(bufc)::value;
    const uint8_t* sk = BUF == 0 ? s_k0 : s_k1;
    const uint8_t* sv = BUF == 0 ? s_v0 : s_v1;
    const uint8_t* sks = BUF == 0 ? s_ks0 : s_ks1;
    const uint8_t* svs = BUF == 0 ? s_vs0 : s_vs1;
    const int t0 = 32 * it;
    if (it + 1 < ntiles)
      load_tile(t0 + 32, BUF == 0 ? s_k1 : s_k0, BUF == 0 ? s_v1 : s_v0, BUF == 0 ? s_ks1 : s_ks0,
                BUF == 0 ? s_vs1 : s_vs0);
    KVFrag<D, KF, VF> f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int kt = 8 * (r >> 2) + 4 * hf + (r & 3);
      const uint8_t* krow = sk + kt * D * KB;
      if constexpr (KF == kFmtF16) {
#pragma unroll
        for (int j = 0; j < D / 32; ++j)
          f.k[hf][j] = *reinterpret_cast<const half8_t*>(krow + fk_slot<CK>(kt, (D / 32) * lg + j) * 16);
      } else if constexpr (KF == kFmtQ8) {
#pragma unroll
        for (int j = 0; j < D / 32; ++j) {   // bytes 32 j + 8 lg .. + 7
          const uint2 w = *reinterpret_cast<const uint2*>(krow + fk_slot<CK>(kt, 2 * j + (lg >> 1)) * 16 + 8 * (lg & 1));
          f.k[hf][j][0] = w.x;
          f.k[hf][j][1] = w.y;
        }
      } else {
#pragma unroll
        for (int j2 = 0; j2 < D / 64; ++j2) {   // bytes (D / 4) lg + 16 j2 .. + 15
          const uint4 w = *reinterpret_cast<const uint4*>(krow + fk_slot<CK>(kt, (D / 64) * lg + j2) * 16);
          f.k[hf][2 * j2][0] = w.x;
          f.k[hf][2 * j2][1] = w.y;
          f.k[hf][2 * j2 + 1][0] = w.z;
          f.k[hf][2 * j2 + 1][1] = w.w;
        }
      }
    }
    if constexpr (KQ) {
      // scales of tokens 8 lg .. 8 lg + 7
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(sks + 16 * lg * (D / 32) + 16 * i);
#pragma unroll
        for (int e = 0; e < 4; ++e) f.ks[4 * i + e] = x[e];
      }
    }
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int vd = 16 * i + r;
      const uint8_t* vrow = sv + vd * 32 * VB;
      if constexpr (VF == kFmtF16) {
        f.v[i] = *reinterpret_cast<const half8_t*>(vrow + fv_slot<CV>(vd, lg) * 16);
      } else {   // tokens 8 lg .. 8 lg + 7
        const uint2 w = *reinterpret_cast<const uint2*>(vrow + fv_slot<CV>(vd, lg >> 1) * 16 + 8 * (lg & 1));
        f.v[i][0] = w.x;
        f.v[i][1] = w.y;
      }
    }
    if constexpr (VQ) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        const u32x4 y = *reinterpret_cast<const u32x4*>(svs + 16 * lg * (D / 32) + 16 * i);
#pragma unroll
        for (int e = 0; e < 4; ++e) f.vs[4 * i + e] = y[e];
      }
    }
    size_t row0_unused;
    int tt_unused;
    // a tile on a page outside the pool has no valid token (every score -inf)
    const int valid = tile_at(t0, row0_unused, tt_unused) ? min(32, n - t0) : 0;
    // O is rounded to fp16 at the end: p is taken to fp16 alone (no low half)
    attn_tile<D, KF, VF, true, false>(st, f, qf, a.scale_log2, valid, lg, [] {}, min(max(ncol - t0, 0), valid));
    wait_loads();
    __syncthreads();
  };
  for (int it = 0; it < ntiles;) {
    step(std::integral_constant<int, 0>{}, it);
    if (++it >= ntiles) break;
    step(std::integral_constant<int, 1>{}, it);
    ++it;
  }

  // O = o / l (the value products carry p * 2^kPScale, or p * 2^ex for Q8_0 values)
  const float ltot = st.l + __shfl_xor(st.l, 16);
  const float lsum = ltot + __shfl_xor(ltot, 32);
  if (colv) {
    const float inv = (VQ ? exp2i(-st.ex) : exp2i(-kPScale)) / lsum;
    half_t* orow = a.O16 + ((size_t)row * a.Hq + head) * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      // rounded to nearest, as the merge of the split-K kernel stores O16
      const half2_t lo = {(half_t)(st.o[i][0] * inv), (half_t)(st.o[i][1] * inv)};
      const half2_t hi = {(half_t)(st.o[i][2] * inv), (half_t)(st.o[i][3] * inv)};
      *reinterpret_cast<uint2*>(orow + 16 * i + 4 * lg) = make_uint2(h2_bits(lo), h2_bits(hi));
    }
  }
}

hipError_t launch_attn_prefill(const qkdec_kv_layer& kv, const int32_t* slot, const int32_t* n_ctx, int B,
                               const uint16_t* Q, int n_q_heads, float scale, uint16_t* O16, float* partials,
                               int n_ctx_add, hipStream_t st, const int32_t* pages, int max_pages) {
  const int G = n_q_heads / kv.n_kv_heads;
  if (pages && !(G <= 16 && (G & (G - 1)) == 0)) return hipErrorInvalidValue;
  if (G <= 16 && (G & (G - 1)) == 0) {
    FlashArgs f;
    f.k = reinterpret_cast<const uint8_t*>(kv.k);
    f.v = reinterpret_cast<const uint8_t*>(kv.v);
    f.ks = reinterpret_cast<const uint16_t*>(kv.k_scale);
    f.vs = reinterpret_cast<const uint16_t*>(kv.v_scale);
    f.n_kv = kv.n_kv_heads;
    f.cap = kv.capacity;
    f.n_slots = kv.n_slots;
    f.slot = slot;
    f.pos = n_ctx;
    f.n_add = n_ctx_add;
    f.rows = B;
    f.Q = reinterpret_cast<const half_t*>(Q);
    f.Hq = n_q_heads;
    f.h4 = G < 4 ? G : 4;
    f.scale_log2 = scale * 1.4426950408889634f;
    f.O16 = reinterpret_cast<half_t*>(O16);
    f.pages = pages;
    f.max_pages = pages ? max_pages : 0;
    f.page_shift = 0;
    while (pages && (1 << f.page_shift) < kv.capacity) ++f.page_shift;
    const dim3 grid((unsigned)((B + 64 / f.h4 - 1) / (64 / f.h4)), kv.n_kv_heads, G / f.h4);
#define QK_FA(DD, KF, VF)                                                                                     \
  do {                                                                                                        \
    if (pages) hipLaunchKernelGGL((attn_prefill_kernel<DD, KF, VF, true>), grid, dim3(256), 0, st, f);      \
    else hipLaunchKernelGGL((attn_prefill_kernel<DD, KF, VF, false>), grid, dim3(256), 0, st, f);           \
  } while (0)
#define QK_FA_D(DD)                                                      \
  do {                                                                   \
    if (kf == kFmtF8) QK_FA(DD, kFmtF8, kFmtF8);                         \
    else if (kf == kFmtQ8 && vf == kFmtQ8) QK_FA(DD, kFmtQ8, kFmtQ8);    \
    else if (kf == kFmtQ8) QK_FA(DD, kFmtQ8, kFmtF16);                   \
    else if (vf == kFmtQ8) QK_FA(DD, kFmtF16, kFmtQ8);                   \
    else QK_FA(DD, kFmtF16, kFmtF16);                                    \
  } while (0)
    const int kf = kv_k_fmt(kv.type), vf = kv_v_fmt(kv.type);
    if (kv.head_dim == 128) QK_FA_D(128);
    else QK_FA_D(64);
#undef QK_FA_D
#undef QK_FA
    return hipGetLastError();
  }
  // other caches: the split-K kernel, at most kPfAttnRows rows per call
  if (B > kPfAttnRows) {
    for (int r0 = 0; r0 < B; r0 += kPfAttnRows) {
      const hipError_t e = launch_attn_prefill(kv, slot + r0, n_ctx + r0, std::min(kPfAttnRows, B - r0),
                                               Q + (size_t)r0 * n_q_heads * kv.head_dim, n_q_heads, scale,
                                               O16 + (size_t)r0 * n_q_heads * kv.head_dim, partials, n_ctx_add, st);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int tok = attn_prefill_tok(n_q_heads, kv.n_kv_heads);
  if (tok == 1)
    return launch_attn_decode(kv, slot, n_ctx, B, Q, n_q_heads, scale, nullptr, O16, partials, n_ctx_add, st);
  const int groups = (B + tok - 1) / tok;
  AttnArgs a;
  a.k = reinterpret_cast<const uint8_t*>(kv.k);
  a.v = reinterpret_cast<const uint8_t*>(kv.v);
  a.ks = reinterpret_cast<const uint16_t*>(kv.k_scale);
  a.vs = reinterpret_cast<const uint16_t*>(kv.v_scale);
  a.n_kv = kv.n_kv_heads;
  a.cap = kv.capacity;
  a.n_slots = kv.n_slots;
  a.slot = slot;
  a.n_ctx = n_ctx;
  a.n_ctx_add = n_ctx_add;
  a.Q = reinterpret_cast<const half_t*>(Q);
  a.Hq = n_q_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.pages = nullptr;
  a.max_pages = 0;
  a.page_shift = 0;
  a.seq_cap = kv.capacity;
  a.tok = tok;
  a.kv_new = nullptr;
  a.nrows = B;
  a.n_splits = attn_prefill_splits(B, n_q_heads, kv);
  a.runs_wanted = attn_runs_wanted(groups, kv.n_kv_heads);
  const int D = kv.head_dim;
  const size_t n_rows = (size_t)B * n_q_heads * a.n_splits;
  a.part_o = partials;
  a.part_ml = partials + n_rows * D;
  const int max_runs = attn_runs(a.seq_cap, a.runs_wanted, a.n_splits);
  const dim3 grid(max_runs, kv.n_kv_heads, groups);
  const dim3 blk(64 * kAttnWaves);
#define QK_ATTN(DD, KF, VF) hipLaunchKernelGGL((attn_split_kernel<DD, KF, VF, false, true>), grid, blk, 0, st, a)
#define QK_ATTN_D(DD)                                                      \
  do {                                                                     \
    if (kf == kFmtF8) QK_ATTN(DD, kFmtF8, kFmtF8);                         \
    else if (kf == kFmtQ8 && vf == kFmtQ8) QK_ATTN(DD, kFmtQ8, kFmtQ8);    \
    else if (kf == kFmtQ8) QK_ATTN(DD, kFmtQ8, kFmtF16);                   \
    else if (vf == kFmtQ8) QK_ATTN(DD, kFmtF16, kFmtQ8);                   \
    else QK_ATTN(DD, kFmtF16, kFmtF16);                                    \
  } while (0)
  const int kf = kv_k_fmt(kv.type), vf = kv_v_fmt(kv.type);
  if (D == 128) QK_ATTN_D(128);
  else QK_ATTN_D(64);
#undef QK_ATTN_D
#undef QK_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeArgs mg;
  mg.part_o = a.part_o;
  mg.part_ml = a.part_ml;
  mg.n_splits = a.n_splits;
  mg.runs_wanted = a.runs_wanted;
  mg.slot = slot;
  mg.paged = 0;
  mg.n_ctx = n_ctx;
  mg.n_ctx_add = n_ctx_add;
  mg.cap = a.seq_cap;
  mg.n_slots = kv.n_slots;
  mg.Hq = n_q_heads;
  mg.D = D;
  mg.tok = tok;
  mg.nrows = B;
  mg.O = nullptr;
  mg.O16 = reinterpret_cast<half_t*>(O16);
  hipLaunchKernelGGL(attn_combine_kernel, dim3(n_q_heads, B), dim3(D), 0, st, mg);
  return hipGetLastError();
}

}  // namespace qk
