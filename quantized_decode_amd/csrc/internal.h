// Host-side launchers shared between the translation units of libqkdec.
// Every launcher assumes its arguments were validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qkdec.h"

namespace qk {

// ---- Q4_K GEMM (gemm_q4k.hip); force_kc = 0 picks the K chunk by shape.
// ws: device workspace of gemm_workspace_bytes(); its counters must be zero
// before the first launch (every launch leaves them zero again).
size_t gemm_workspace_bytes(int64_t n_rows, int64_t K, int B, bool swiglu);

// One launch of the general kernel.  Activations: fp16 X, or fp32 X (x_f32)
// rounded per 256-value block, or fp32 residual-stream rows normalized while
// staged when gamma is set (RMSNorm with the sum-of-squares slots ss_in, see
// common.h).  Output: Y (+ residual) and optionally ss_out (one slot per 64
// rows of Y), or, for swiglu, A = silu(gate) * up with n_rows = F.
struct GemmLaunch {
  const void* W = nullptr;
  int64_t n_rows = 0, K = 0;
  const void* X = nullptr;
  bool x_f32 = false;
  int64_t ldx = 0;
  int B = 0;
  const float* gamma = nullptr;
  const float* ss_in = nullptr;
  float eps = 0.f;
  float* Y = nullptr;
  int64_t ldy = 0;
  const float* residual = nullptr;
  int64_t ldr = 0;
  float* ss_out = nullptr;
  bool swiglu = false;
  float* A = nullptr;
  int64_t lda = 0;
  void* ws = nullptr;
  int force_kc = 0;    // 0: K chunk chosen by shape
  int force_wpb = 0;   // 0: waves per work-group chosen by shape (4, 8 or 16)
  int kernel = 0;      // QKDEC_GEMM_AUTO / _MFMA / _MATVEC (multi-item shapes)
};
// Whether a multi-item launch of B sequences runs the vector-ALU matvec
// (gemm_wi_kernel MV = B) rather than the MFMA tiles: on request, or for
// QKDEC_GEMM_AUTO at B <= QKDEC_MATVEC_AUTO_MAX_B.
inline int gemm_matvec_rows(int kernel, int B) {
  const bool want = kernel == QKDEC_GEMM_MATVEC || (kernel == QKDEC_GEMM_AUTO && B <= QKDEC_MATVEC_AUTO_MAX_B);
  return want && B <= QKDEC_MATVEC_MAX_B ? B : 0;
}
hipError_t launch_gemm(const GemmLaunch& L, hipStream_t st);
// The QKV projection of a decode step (RMSNorm fused, L.x_f32 + L.gamma),
// finished per head: Y gets the fp32 projection, then q and k are rotated
// (RoPE at pos), q is written as fp16 to q16 [B][Hq][head_dim] and k, v are
// appended to the cache at (slot, pos).  One work-group row per head.
struct RopeAppendArgs {
  const int32_t* slot;   // [B] cache slot of each sequence
  const int32_t* pos;    // [B] position of the new token
  uint8_t *k, *v;        // cache of this layer (fp16 or Q8_0 codes)
  uint16_t *ks, *vs;     // Q8_0 block scales
  int n_kv, cap, n_slots, Hq;
  // where the new token is stored: (slot[b], spos[b]); spos = pos for a slot
  // arena, the page and the position within it for a paged pool
  // (launch_page_locate)
  const int32_t* spos;
  int kf, vf;             // key / value format (kFmtF16, kFmtQ8, kFmtF8)
  float rope_base;
  // (cos, sin) of every pair at each row's position, [B][head_dim/2]
  // (launch_rope_table), or null to form them in place
  const float2* rope;
  uint16_t* q16;         // rotated queries, fp16 bits
  int32_t* err;          // set to QKDEC_E_CAPACITY for a position outside the cache
  // Q8_0 keys or values of a decode step (multi-item QKV projection only):
  // the rotated fp32 k (part 0) and v (part 1) of the new token go to
  // kv_new[B][2][n_kv][head_dim] instead of the cache, and the attention
  // kernel (launch_attn_decode's kv_new) quantizes and stores them; null
  // otherwise
  float* kv_new;
};
hipError_t launch_gemm_qkv_rope(const GemmLaunch& L, const RopeAppendArgs& ra, int head_dim, hipStream_t st);
// The same product with K split over the waves of one work-group per output
// tile (gemm_wk.hip): no workspace.  Waves per work-group (s) and super-blocks
// in flight per wave (p) by shape.
struct WkConfig {
  int s, p;
};
WkConfig wk_config(int kb, bool swiglu, int xmode);
hipError_t launch_gemm_wk(const GemmLaunch& L, hipStream_t st);
// Several output items per work-group (gemm_wk.hip), for the shapes it covers;
// returns hipErrorNotSupported for any other.
hipError_t launch_gemm_wi(const GemmLaunch& L, hipStream_t st);
// The decode step's QKV projection with its RoPE and append finish on the
// multi-item kernel (K = 4096, fp16 or E4M3 cache); hipErrorNotSupported
// otherwise.
hipError_t launch_gemm_wi_qkv(const GemmLaunch& L, const RopeAppendArgs& ra, int head_dim, hipStream_t st);
hipError_t launch_gemm_q4k_xf32(const void* W, int64_t N, int64_t K, const float* X, int64_t ldx, int B,
                                float* Y, int64_t ldy, const float* residual, int64_t ldr, void* ws, hipStream_t st,
                                int force_kc = 0);
hipError_t launch_gemm_q4k_swiglu(const void* W, int64_t F, int64_t K, const uint16_t* X, int64_t ldx, int B,
                                  float* A, int64_t lda, void* ws, hipStream_t st, int force_kc = 0);
hipError_t launch_dequant_q4k(const void* W, int64_t n_blocks, float* out, hipStream_t st);

// Largest number of row groups (work-groups along N) of one Q4_K GEMM launch:
// at least 4 tiles of 16 rows per group, so N <= 16 * 4 * kGemmMaxGroups =
// 2^20 rows (a SwiGLU launch covers gate and up: 2F <= 2^20).
constexpr int kGemmMaxGroups = 16384;
constexpr int64_t kGemmMaxRows = 16 * 4 * (int64_t)kGemmMaxGroups;

// ---- cache formats: the key / value format of a cache type
inline int kv_k_fmt(int type) {
  return type == QKDEC_KV_FP8_E4M3 ? kFmtF8
         : (type == QKDEC_KV_Q8_0 || type == QKDEC_KV_Q8_0_K_F16_V) ? kFmtQ8 : kFmtF16;
}
inline int kv_v_fmt(int type) {
  return type == QKDEC_KV_FP8_E4M3 ? kFmtF8
         : (type == QKDEC_KV_Q8_0 || type == QKDEC_KV_F16_K_Q8_0_V) ? kFmtQ8 : kFmtF16;
}
inline bool kv_k_q8(int type) { return kv_k_fmt(type) == kFmtQ8; }
inline bool kv_v_q8(int type) { return kv_v_fmt(type) == kFmtQ8; }

// ---- attention (attn_decode.hip)
// A sequence's n cached tokens (ceil(n/32) tiles of 32) are cut into runs of
// whole tiles, spread evenly, one work item each.  Runs per sequence: the
// count w that makes the B * n_kv * w work items reach kAttnTarget (one per
// CU of MI355X), or, when n needs more than w runs of at most kAttnChunk
// tokens, the next multiple of w, so that a uniform batch's work items fill
// whole rounds of the chip (B = 8, n_kv = 8: 4, 8, 12, ... runs; 5 runs
// would leave the second round three quarters empty); at most one run per 5
// tiles (where this binds, one or two sequences, one per 5 measured faster
// than one per 4, 6 or 8), never fewer than ceil(n / kAttnChunk), and at
// most attn_max_runs (the partial-result stride).
// kAttnChunk = 4096: runs of up to 4096 tokens were faster than runs of up to
// 1024 or 2048 at every long context measured (B = 8 at L = 6900 to 32000,
// B = 16 at L = 32000) and as fast as 8192 or 16384; below ~4k tokens the
// limit does not bind at B = 8.
constexpr int kAttnChunk = 4096;
constexpr int kAttnTarget = 256;
constexpr int kAttnMaxBatch = 16;   // most sequences of a decode attention call
// runs wanted per sequence for a call with B sequences (before the per-
// sequence rounding and limits)
inline int attn_runs_wanted(int B, int n_kv) {
  const int w = (kAttnTarget + B * n_kv - 1) / (B * n_kv);
  return w > 1 ? w : 1;
}
// partial-result rows per (b, q head): the most runs any call of 1 ..
// kAttnMaxBatch sequences gives a sequence of this capacity, so a workspace
// sized for one batch serves any smaller one (capacity: most tokens of one
// sequence, at most 2^31 - 1; n_kv >= 1)
inline int attn_max_runs(int64_t capacity, int n_kv) {
  const int by_len = (int)((capacity + kAttnChunk - 1) / kAttnChunk);
  int most = by_len;
  for (int B = 1; B <= kAttnMaxBatch; ++B) {
    const int w = attn_runs_wanted(B, n_kv);
    const int r = (by_len + w - 1) / w * w;
    most = r > most ? r : most;
  }
  return most;
}
// partial results per (b, q head, run): m, l, then head_dim values of o
inline size_t attn_partials_bytes(int B, int n_q_heads, int head_dim, int64_t capacity, int n_kv) {
  return (size_t)B * n_q_heads * attn_max_runs(capacity, n_kv) * (size_t)(head_dim + 2) * sizeof(float);
}
// most tokens one sequence can hold: the slot capacity, or for a paged pool
// (max_pages > 0) max_pages pages of kv.capacity tokens
inline int64_t attn_seq_cap(const qkdec_kv_layer& kv, int max_pages) {
  return max_pages > 0 ? (int64_t)max_pages * kv.capacity : kv.capacity;
}
// The merge of the runs' partial results into O / O16 (attn_merge_elem, one
// output element per call)
struct MergeArgs {
  const float* part_o;
  const float* part_ml;
  int n_splits, runs_wanted;
  const int32_t* slot;   // paged: any readable int32 [B] (unused)
  int paged;
  const int32_t* n_ctx;
  int n_ctx_add, cap, n_slots, Hq, D;
  // prompt rows taken tok at a time (launch_attn_prefill): a row's runs are
  // those of the last of its tok rows (at most nrows - 1); 1 otherwise
  int tok, nrows;
  float* O;
  _Float16* O16;
};

// pages != NULL: kv is a pool of n_slots pages of capacity tokens (a power of
// two) and sequence b's pages are pages[b * max_pages ...]; slot is unused.
// kv_new (decode step, a cache with a Q8_0 part, n_ctx_add = 1): the new
// tokens' rotated k and v staged by the QKV projection (RopeAppendArgs
// kv_new); each sequence's last run quantizes and stores them and attends to
// them.  Null: every token is read from the cache.
hipError_t launch_attn_decode(const qkdec_kv_layer& kv, const int32_t* slot, const int32_t* n_ctx, int B,
                              const uint16_t* Q, int n_q_heads, float scale, float* O, uint16_t* O16,
                              float* partials, int n_ctx_add, hipStream_t st, const int32_t* pages = nullptr,
                              int max_pages = 0, const float* kv_new = nullptr);
// The same attention for B consecutive prompt rows of one sequence (row b:
// slot[b], n_ctx[b] + n_ctx_add tokens, ascending by one).  An fp16 cache
// with G a power of two up to 16: flash attention, 64 query columns per
// work-group sharing each key and value tile, no key split (partials unused).
// Other caches: the split-K kernel, kPfAttnRows rows per launch, 16 / G rows
// per work item with their (row, head) pairs as the MFMA columns and scores
// past a row's own length masked (for G not dividing 16, launch_attn_decode).
// Its partial-result rows per (row, head) for a call of B rows: enough runs
// for the longest sequence (one per kAttnChunk tokens) and for the wanted
// count, which falls as B grows.
int attn_prefill_splits(int B, int n_q_heads, const qkdec_kv_layer& kv);
// Partial-result bytes for any call of 1 .. max_rows rows.
size_t attn_prefill_partials_bytes(int max_rows, int n_q_heads, const qkdec_kv_layer& kv);
// pages != NULL: kv is a paged pool (pages of kv.capacity tokens, a power of
// two) and the sequence's page table row is pages[0 .. max_pages - 1]; slot is
// unused, and G must be a power of two (hipErrorInvalidValue otherwise).
hipError_t launch_attn_prefill(const qkdec_kv_layer& kv, const int32_t* slot, const int32_t* n_ctx, int B,
                               const uint16_t* Q, int n_q_heads, float scale, uint16_t* O16, float* partials,
                               int n_ctx_add, hipStream_t st, const int32_t* pages = nullptr, int max_pages = 0);

// ---- KV append and RoPE (kv_append.hip)
// RoPE of q and k, q -> fp16 and the KV append, from the fp32 QKV rows Y
// (row b: [q heads; k heads; v heads], head_dim each)
hipError_t launch_rope_append(const qkdec_kv_layer& kv, const float* Y, int64_t ldy, int Hq, int B,
                              const int32_t* slot, const int32_t* pos, float rope_base, uint16_t* q16, int32_t* err,
                              hipStream_t st, const int32_t* spos = nullptr, const float2* rope = nullptr);
// The rotary (cos, sin) of pair i of head_dim D at position pos[b], for every
// row b < B: table[b * D/2 + i] (angle in fp64, rounded once to fp32); the
// positions are the same in every layer of a step, so one table serves them all.
hipError_t launch_rope_table(const int32_t* pos, int B, int D, float rope_base, float2* table, hipStream_t st);
// Paged step: page[b] and the position within it of logical position pos[b]
// of sequence b (page -1 when outside the table or the pool), once per step
// for every layer's stores.
hipError_t launch_page_locate(const int32_t* pages, int max_pages, int page_tokens, int n_pages, const int32_t* pos,
                              int B, int32_t* page, int32_t* page_pos, hipStream_t st);
hipError_t launch_kv_append(const qkdec_kv_layer& kv, const int32_t* slot, const int32_t* pos, const float* k,
                            const float* v, int B, int32_t* err, hipStream_t st, const int32_t* pages = nullptr,
                            int max_pages = 0);


// ---- small kernels (small.hip)
// x = E[tok] and its sum-of-squares slots ss (common.h); hidden % 256 == 0
hipError_t launch_embed(const uint16_t* E, int hidden, int vocab, const int32_t* tok, int B, float* x, float* ss,
                        hipStream_t st);
// h = f16(RMSNorm(x)) with the sum-of-squares slots of x
hipError_t launch_rmsnorm_f16(const float* x, const float* gamma, const float* ss, int hidden, int B, float eps,
                              uint16_t* h, hipStream_t st);
size_t lm_head_partials_bytes(int64_t V, int B);
// bytes of LDS the LM head kernel needs for B sequences of width H
inline size_t lm_head_lds_bytes(int64_t H, int B) { return (size_t)B * (size_t)(H + 8) * 2; }
hipError_t launch_lm_head_argmax(const uint16_t* Wlm, int64_t V, int64_t H, const uint16_t* X, int B,
                                 float* logits, int32_t* tok, void* partials, int32_t* pos_inc, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// the rows of one prefill chunk: slot[b] = s, pos[b] = start + b,
// tok[b] = tokens[b] for b < rows (tokens: device int32)
hipError_t launch_prefill_rows(int s, int start, const int32_t* tokens, int rows, int32_t* slot, int32_t* pos,
                               int32_t* tok, hipStream_t st);
// the same for one sequence in a paged pool: page[b] (-1 outside the table or
// the pool of n_pages pages), pos[b] = start + b, page_pos[b] within the page
hipError_t launch_prefill_page_rows(const int32_t* pages, int max_pages, int page_tokens, int n_pages, int start,
                                    const int32_t* tokens, int rows, int32_t* page, int32_t* pos, int32_t* page_pos,
                                    int32_t* tok, hipStream_t st);

// ---- prompt ingestion (prefill.hip): chunks of up to kPfRows prompt tokens
// of one sequence.  A projection is gemm_pf (partial sums of ksplit K ranges,
// part[ks][T][n_rows]) and pf_finish (their sum); a projection's fp16 input
// comes with its 32-value sub-block sums / 32, xs [T][K/256][4] (half4), and
// the power-of-two factor fd [T][K/256] of each row super-block (pf_norm: 1,
// or pf_finish for the SwiGLU output).
constexpr int kPfChunk = 2048;        // prompt rows per pass of the layers
constexpr int kPfAttnRows = 256;      // prompt rows per attention call
constexpr int kPfRows = 64;           // prompt rows per GEMM work-group
constexpr int kPfTilesPerWave = 2;    // weight tiles of 16 rows per wave: 128 rows per work-group
constexpr int kPfTargetGroups = 256;  // work-groups per projection launch aimed at
// K ranges (1 .. K / 256) of a projection with n_rows weight rows over T prompt rows
int pf_ksplit(int64_t n_rows, int64_t K, int T);
// n_rows % 128 == 0, K % 256 == 0, 1 <= T <= kPfChunk; fd = null: every
// factor is 1 (inputs staged by pf_norm)
hipError_t launch_gemm_pf(const void* W, int64_t n_rows, int64_t K, const uint16_t* X, int64_t ldx, const void* xs,
                          const float* fd, int T, float* part, int ksplit, hipStream_t st);
enum PfFinishMode {
  kPfOut = 0,     // out = res + sum of the partials
  kPfNorm = 1,    // and ssq [T][N/256]: the sum of squares of each 256 values of out
  kPfSwiglu = 2,  // h [T][N/2] = f16b(silu(gate) up) with its xs, fd (gate: columns [0, N/2), up: [N/2, N))
};
hipError_t launch_pf_finish(const float* part, int ksplit, int T, int N, const float* res, float* out, int64_t ldo,
                            int mode, float* ssq, uint16_t* h, void* xs, float* fd, hipStream_t st);
// h [T][K] = f16(RMSNorm(x) gamma) from the block sums of squares ssq, with its
// xs, fd; x = null: only the sums of the fp16 rows already in h
hipError_t launch_pf_norm(const float* x, const float* ssq, const float* gamma, float eps, int K, int T, uint16_t* h,
                          void* xs, float* fd, hipStream_t st);

}  // namespace qk
