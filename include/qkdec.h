/*
 * qkdec.h - C ABI of libqkdec: one batched LLM decode step with Q4_K weights
 * and an fp16, Q8_0, mixed or 8-bit float KV cache, for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources (three pages of one blog series on batched decode on one GPU):
 *   P1 "Batch One Is the Local LLM Assumption Agent Workloads Break on RDNA4"
 *   P2 "Why a Batched Local Agent Swarm's Speedup Erodes With Context on RDNA4"
 *   P3 "KV Cache Quantization on RDNA4: Moving the Weight-vs-KV Crossover for a
 *       Local Agent Swarm"
 * The problem these entry points take is the pages' own: B sequences, each
 * with its own context length L and private KV cache, sharing one set of
 * weights W that a step reads once (P2 "The two halves of a decode-step memory
 * bill").
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes in these calls (except the plan
 *     calls, which own a HIP graph), never reads device data on the host, and
 *     only launches kernels on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream).  Calls other than the plan calls may be captured
 *     into a HIP graph.
 *   - fp16 values are passed as uint16_t bit patterns.
 *   - Every call returns a qkdec_status.  Arguments are validated before any
 *     launch: on error nothing is launched and nothing is written.  A launch
 *     failure reported by HIP returns QKDEC_E_HIP.
 *   - Calls keep no mutable global state and are safe to issue from several
 *     host threads on different streams; two calls that share an output or a
 *     workspace must be ordered by the caller.
 *
 * Q4_K matrix format (N rows = outputs, K columns = inputs, K % 256 == 0,
 * N % 16 == 0; base address 16-byte aligned).  A super-block holds 256
 * consecutive weights of one row in 144 bytes:
 *   bytes 0-1    fp16 d         (little-endian)
 *   bytes 2-3    fp16 dmin
 *   bytes 4-15   four 24-bit little-endian groups; group p (bytes 4+3p..6+3p)
 *                holds sc[2p], sc[2p+1], m[2p], m[2p+1] (6 bits each, from the
 *                least significant bit); sub-block s covers weights 32s..32s+31
 *   bytes 16-143 32 little-endian 32-bit words; word j covers weights 8j..8j+7:
 *                weight 8j+2i+par is the 4-bit field at bit 16*par + 4*i
 *   weight = d*sc[s]*q - dmin*m[s]
 * Blocks are stored in row tiles of 16 rows: [N/16][K/256][16][144] (tile,
 * super-block column, row in tile).  A tile's 16 blocks of one super-block
 * column are therefore one contiguous, 128-byte-aligned 2304-byte run.
 *
 * KV cache formats (one layer; see qkdec_kv_layer).  Blocks of Q8_0 are 32
 * consecutive head_dim values of one token and KV head; value = d*q.
 */
#ifndef QKDEC_H
#define QKDEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKDEC_ABI_VERSION 1

typedef int32_t qkdec_status;
enum {
  QKDEC_OK = 0,
  QKDEC_E_ARG = -1,         /* NULL pointer, bad enum, non-positive size      */
  QKDEC_E_SHAPE = -2,       /* unsupported or inconsistent dimensions        */
  QKDEC_E_ALIGN = -3,       /* pointer or leading dimension misaligned       */
  QKDEC_E_WORKSPACE = -4,   /* workspace missing or smaller than required    */
  QKDEC_E_CAPACITY = -5,    /* a position reached the cache capacity         */
  QKDEC_E_UNSUPPORTED = -6, /* valid request this build does not implement   */
  QKDEC_E_HIP = -7          /* the HIP runtime reported an error             */
};

enum {
  QKDEC_KV_F16 = 0,
  QKDEC_KV_Q8_0 = 1,
  QKDEC_KV_Q8_0_K_F16_V = 2,
  QKDEC_KV_F16_K_Q8_0_V = 3,
  QKDEC_KV_FP8_E4M3 = 4
};

/* Human-readable name of a status code (static string). */
const char* qkdec_status_str(qkdec_status s);
/* QKDEC_ABI_VERSION of the built library. */
int32_t qkdec_abi_version(void);
/* Identifier of the sources the library was built from (a hash of its HIP
 * sources, headers and compiler flags; static string), so that a measurement
 * recorded with one build is recognised as stale under another. */
const char* qkdec_build_id(void);

/* ------------------------------------------------------------------ GEMM ---
 * Y[b][n] = residual[b][n] + sum_k W[n][k] * X[b][k]   for b < B, n < N.
 *
 * P1 "The weight read is the only term that does not scale": a step streams
 * the weights once and multiplies every sequence's hidden state against each
 * weight tile; P1 "RDNA4 pads the batch dimension to 16 whether you fill it or
 * not": the matrix cores take the sequences as the M dimension of a tile of
 * 16.  Here every B in 1..16 runs the same MFMA instruction stream.
 *
 * W: Q4_K matrix (format above).  X: fp16 [B][ldx] (ldx >= K, ldx % 8 == 0,
 * 16-byte aligned).  Y: fp32 [B][ldy] (ldy >= N).  residual: fp32 [B][ldr] or
 * NULL (then Y = product); it may alias Y.  1 <= B <= 16, N <= 2^20.
 * workspace: device memory of at least qkdec_gemm_q4k_workspace_size(N, K, B)
 * bytes, zeroed once with qkdec_workspace_init before its first use (holds a
 * fixed 64 KiB area of split-K arrival counters, then the partial sums; every
 * call leaves the counters zero again, so one workspace serves calls of any
 * shapes it is large enough for).  Calls that share a workspace must not
 * overlap.  The workspace contract is common to the GEMM entry points: each
 * 16-row output tile is computed in one work-group (K split over its waves,
 * partial sums added in LDS), except where K is split across work-groups as
 * well (by shape, e.g. K = 12288), whose partial sums and arrival counters
 * live in the workspace.
 * Partial sums are added in a fixed order: results are deterministic and
 * independent of scheduling.
 */
size_t qkdec_gemm_q4k_workspace_size(int64_t N, int64_t K, int32_t B);
qkdec_status qkdec_gemm_q4k(const void* W, int64_t N, int64_t K,
                            const uint16_t* X, int64_t ldx, int32_t B,
                            float* Y, int64_t ldy, const float* residual, int64_t ldr,
                            void* workspace, size_t ws_bytes, void* stream);

/* Which engine forms the products.  P1 "RDNA4 pads the batch dimension to 16
 * whether you fill it or not": a one-row GEMM is a matrix-vector product,
 * bandwidth-bound, which the pages run as a dequant-matvec below about four
 * sequences and on the matrix cores above.  QKDEC_GEMM_MATVEC runs the same
 * exact Q4_K decode and forms the products on the vector ALU (packed fp16 dot
 * products into fp32) for the live sequences only, B <= QKDEC_MATVEC_MAX_B;
 * QKDEC_GEMM_MFMA pads the batch to the 16-row tile; QKDEC_GEMM_AUTO takes the
 * matvec for B <= QKDEC_MATVEC_AUTO_MAX_B, the crossover measured on MI355X
 * (36-layer pass of the four projections: matvec 1.49 ms against MFMA 1.54 ms
 * at B = 1, 1.79 against 1.53 ms at B = 2; the decode step uses AUTO).  The choice applies where the multi-item
 * kernel serves the shape (K = 4096; K = 12288 without SwiGLU); elsewhere the
 * MFMA kernels run. */
enum { QKDEC_GEMM_AUTO = 0, QKDEC_GEMM_MFMA = 1, QKDEC_GEMM_MATVEC = 2 };
#define QKDEC_MATVEC_MAX_B 2
#define QKDEC_MATVEC_AUTO_MAX_B 1
/* As qkdec_gemm_q4k with the engine chosen (a QKDEC_GEMM_* value);
 * QKDEC_E_SHAPE for QKDEC_GEMM_MATVEC with B > QKDEC_MATVEC_MAX_B. */
qkdec_status qkdec_gemm_q4k_engine(const void* W, int64_t N, int64_t K,
                                   const uint16_t* X, int64_t ldx, int32_t B,
                                   float* Y, int64_t ldy, const float* residual, int64_t ldr,
                                   int32_t engine, void* workspace, size_t ws_bytes, void* stream);

/* As qkdec_gemm_q4k, with fp32 activations X (ldx % 4 == 0, 16-byte
 * aligned).  Each row's activations are rounded to fp16 in blocks of 256
 * consecutive values (one Q4_K super-block); a block whose largest magnitude
 * exceeds 65504 is first scaled by the smallest power of two 2^-s that brings
 * it into fp16's range, and the products are scaled back by 2^s exactly.  A
 * block already inside fp16's range is rounded exactly as plain fp16.  This
 * is the input of the down projection, whose activation can exceed fp16's
 * range on weights whose mean is not zero. */
qkdec_status qkdec_gemm_q4k_xf32(const void* W, int64_t N, int64_t K,
                                 const float* X, int64_t ldx, int32_t B,
                                 float* Y, int64_t ldy, const float* residual, int64_t ldr,
                                 void* workspace, size_t ws_bytes, void* stream);

/* A[b][n] = silu(G[b][n]) * U[b][n] (fp32) where [G;U] = X W^T, W having 2*F
 * rows (gate rows 0..F-1, up rows F..2F-1): the SwiGLU of the pages' small
 * kernels (P1 "The weight read is the only term that does not scale") fused
 * into the GEMM epilogue.  A: fp32 [B][lda] (lda >= F), the input of
 * qkdec_gemm_q4k_xf32.  F % 16 == 0.  workspace as for qkdec_gemm_q4k, sized
 * by qkdec_gemm_q4k_swiglu_workspace_size. */
size_t qkdec_gemm_q4k_swiglu_workspace_size(int64_t F, int64_t K, int32_t B);
qkdec_status qkdec_gemm_q4k_swiglu(const void* W, int64_t F, int64_t K,
                                   const uint16_t* X, int64_t ldx, int32_t B,
                                   float* A, int64_t lda, void* workspace, size_t ws_bytes,
                                   void* stream);

/* Test export: out[256*i + k] = RN_fp32(d*sc*q - dmin*m) of weight k of the
 * i-th stored block (blocks in storage order).  Bit-exact.  out: fp32. */
qkdec_status qkdec_dequant_q4k(const void* W, int64_t n_blocks, float* out, void* stream);

/* ------------------------------------------------------------- KV cache ---
 * One layer of a slot-arena cache: n_slots independent sequences of up to
 * `capacity` tokens (capacity % 32 == 0), n_kv heads of head_dim (64 or 128).
 *   QKDEC_KV_F16:  k  fp16 [n_slots][n_kv][capacity][head_dim]
 *                  v  fp16 [n_slots][n_kv][capacity/32][head_dim][32]
 *                     (transposed within blocks of 32 tokens: value d of
 *                     token t at [t/32][d][t%32], so a 32-token tile of one
 *                     head is one contiguous run)
 *                  k_scale = v_scale = NULL
 *   QKDEC_KV_Q8_0: k  int8 [n_slots][n_kv][capacity][head_dim]
 *                  v  int8 [n_slots][n_kv][capacity/32][head_dim][32]
 *                  k_scale, v_scale fp16 [n_slots][n_kv][capacity][head_dim/32]
 *   QKDEC_KV_Q8_0_K_F16_V: keys as in QKDEC_KV_Q8_0 (k, k_scale), values as in
 *                  QKDEC_KV_F16 (v), v_scale = NULL
 *   QKDEC_KV_F16_K_Q8_0_V: keys as in QKDEC_KV_F16 (k), k_scale = NULL, values
 *                  as in QKDEC_KV_Q8_0 (v, v_scale)
 *   QKDEC_KV_FP8_E4M3: k  uint8 [n_slots][n_kv][capacity][head_dim]
 *                  v  uint8 [n_slots][n_kv][capacity/32][head_dim][32]
 *                  one OCP FP8 E4M3 code per element, no scale (sign, 4-bit
 *                  exponent with bias 7, 3-bit mantissa, subnormals at
 *                  exponent field 0, no infinity, S.1111.111 = NaN, largest
 *                  finite 448); k_scale = v_scale = NULL
 * All pointers in use 16-byte aligned.  P3 "Why Q8 is close to free and where
 * the sharp edges are": one byte per element plus the per-block scale, read
 * by the attention kernel directly.  The same section and the FAQ "Does KV
 * cache quantization hurt output quality?": keys are more sensitive to
 * quantization than values, so the key and value formats are chosen
 * independently (Q8_0 keys with fp16 values, or the reverse).  P2 "What a
 * long-running swarm should actually tune" and P3 (same section): an 8-bit
 * float cache halves the fp16 bytes per token; the pages name no variant and
 * no scale, read here as unscaled E4M3. */
typedef struct {
  int32_t type;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  int32_t n_slots;
  void* k;
  void* v;
  void* k_scale;
  void* v_scale;
} qkdec_kv_layer;

/* Store one token per sequence: k[b], v[b] (fp32 [B][n_kv][head_dim], keys
 * already rotated) go to index pos[b] of slot slot[b].  fp16: round to
 * nearest even.  Q8_0, per block of 32 values, in fp64: d = RN_fp16(amax/127),
 * q = x/d rounded half away from zero, clamped to [-127, 127] (q = 0 when d is
 * 0).  FP8 E4M3: the fp32 value rounded to the nearest code (ties to even),
 * magnitudes above 448 stored as +-448, NaN as 0x7F with its sign.  slot, pos:
 * device int32 [B].  A pos[b] outside [0, capacity) or slot
 * outside [0, n_slots) stores nothing for b and sets *err (device int32, may
 * be NULL) to QKDEC_E_CAPACITY.  The type in kv must match the entry point. */
qkdec_status qkdec_kv_append_f16(const qkdec_kv_layer* kv, const int32_t* slot, const int32_t* pos,
                                 const float* k, const float* v, int32_t B, int32_t* err,
                                 void* stream);
qkdec_status qkdec_kv_append_q8_0(const qkdec_kv_layer* kv, const int32_t* slot, const int32_t* pos,
                                  const float* k, const float* v, int32_t B, int32_t* err,
                                  void* stream);
/* The same store for any cache type: each of k and v is stored in its own
 * format (fp16 rounding, the Q8_0 quantizer or the E4M3 rounding above) as
 * kv->type gives it. */
qkdec_status qkdec_kv_append(const qkdec_kv_layer* kv, const int32_t* slot, const int32_t* pos,
                             const float* k, const float* v, int32_t B, int32_t* err, void* stream);

/* ------------------------------------------------------------ attention ---
 * O[b][h] = sum_t softmax_t(scale * Q[b][h] . K[s][g][t]) V[s][g][t]
 *           over t < n_ctx[b], s = slot[b], g = h / (n_q_heads / n_kv_heads).
 *
 * P2 "The two halves of a decode-step memory bill": every sequence reads its
 * whole private cache each step, with query heads grouped onto KV heads.  P3
 * FAQ "Is KV cache quantization a kernel change or a storage change?": a
 * quantized cache is dequantized inside the fused attention kernel, never
 * expanded in memory first (E4M3 codes convert to fp16 exactly).  Split-K flash decoding: each work item covers a
 * run of tokens of one (sequence, KV head) and the partial results are merged
 * with their log-sum-exp weights.
 *
 * Q: fp16 [B][n_q_heads][head_dim].  O: fp32 [B][n_q_heads][head_dim] and/or
 * O16: fp16, same shape (either may be NULL, not both).  slot, n_ctx: device
 * int32 [B]; 1 <= n_ctx[b] <= capacity (n_ctx is clamped to capacity; a
 * sequence with n_ctx <= 0 gets O = 0).  n_q_heads % n_kv_heads == 0,
 * n_q_heads / n_kv_heads <= 16.  1 <= B <= 16.
 * workspace: device memory of at least qkdec_attn_workspace_size() bytes
 * (the partial results of the runs; calls that share it must not overlap);
 * the size functions return 0 for a shape the entry points reject. */
size_t qkdec_attn_workspace_size(int32_t B, int32_t n_q_heads, const qkdec_kv_layer* kv);
qkdec_status qkdec_attn_decode(const qkdec_kv_layer* kv, const int32_t* slot, const int32_t* n_ctx,
                               int32_t B, const uint16_t* Q, int32_t n_q_heads, float scale,
                               float* O, uint16_t* O16, void* workspace, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------ paged KV ---
 * P1 "Where it stops, and the argument I got wrong in May": sequences of very
 * different lengths share one pool of fixed-size pages (admitted and released
 * between steps).  A pool is a qkdec_kv_layer whose slots are pages:
 * n_slots = number of pages, capacity = tokens per page (a power of two,
 * >= 32), any cache type, the layouts above per page.  pages: device int32
 * [B][max_pages]; token t of sequence b is in page pages[b * max_pages +
 * t / capacity] at position t % capacity.  max_pages * capacity <= 2^30.
 * A page entry outside [0, n_slots) (e.g. -1 for a page not handed out) maps
 * nothing: attention leaves the tokens it would hold out of the softmax (a
 * sequence with no mapped token among its first n_ctx gets O = 0; nothing
 * outside the pool is read), and a store to it stores nothing and reports
 * QKDEC_E_CAPACITY.  Two sequences must not write the same page in one call.
 *
 * Attention: as qkdec_attn_decode, with n_ctx[b] clamped to max_pages *
 * capacity; workspace of at least qkdec_attn_paged_workspace_size() bytes. */
size_t qkdec_attn_paged_workspace_size(int32_t B, int32_t n_q_heads, const qkdec_kv_layer* kv, int32_t max_pages);
qkdec_status qkdec_attn_decode_paged(const qkdec_kv_layer* kv, const int32_t* pages, int32_t max_pages,
                                     const int32_t* n_ctx, int32_t B, const uint16_t* Q, int32_t n_q_heads,
                                     float scale, float* O, uint16_t* O16, void* workspace, size_t ws_bytes,
                                     void* stream);
/* Append: as qkdec_kv_append (each tensor in its format), token pos[b] of
 * sequence b into its page; a pos[b] outside [0, max_pages * capacity) or a
 * page entry outside the pool stores nothing for b and sets *err to
 * QKDEC_E_CAPACITY. */
qkdec_status qkdec_kv_append_paged(const qkdec_kv_layer* kv, const int32_t* pages, int32_t max_pages,
                                   const int32_t* pos, const float* k, const float* v, int32_t B, int32_t* err,
                                   void* stream);

/* -------------------------------------------------------------- LM head ---
 * logits[b][v] = sum_k Wlm[v][k] * X[b][k];  tok[b] = argmax_v logits[b][v]
 * (lowest v on ties).  P1 "The weight read is the only term that does not
 * scale": the output-embedding read is shared, the matmul and sampling are per
 * sequence.  Wlm fp16 [V][H] row-major, X fp16 [B][H]; H % 256 == 0,
 * V % 16 == 0.  logits fp32 [B][V] may be NULL; tok device int32 [B].
 * workspace: at least qkdec_lm_head_workspace_size() bytes. */
size_t qkdec_lm_head_workspace_size(int64_t V, int32_t B);
qkdec_status qkdec_lm_head_argmax(const uint16_t* Wlm, int64_t V, int64_t H, const uint16_t* X,
                                  int32_t B, float* logits, int32_t* tok, void* workspace,
                                  size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ full step ---
 * Model description.  All pointers are device pointers except `layers`, a
 * HOST array of n_layers descriptors.  Per layer: w_qkv Q4_K
 * [(n_q_heads + 2 n_kv_heads) head_dim x hidden] (rows: q heads, k heads, v
 * heads), w_o Q4_K [hidden x n_q_heads head_dim], w_gate_up Q4_K
 * [2 ffn x hidden] (rows: gate, up), w_down Q4_K [hidden x ffn], norm gains
 * fp32 [hidden].  embed, lm_head fp16 [vocab][hidden].  hidden % 256 == 0
 * and hidden <= 8192; ffn % 256 == 0; vocab % 16 == 0. */
typedef struct {
  const void* w_qkv;
  const void* w_o;
  const void* w_gate_up;
  const void* w_down;
  const float* norm_attn;
  const float* norm_ffn;
} qkdec_layer;

typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps, rope_base;
  const uint16_t* embed;
  const uint16_t* lm_head;
  const float* norm_final;
  const qkdec_layer* layers;
} qkdec_model;

/* Zero a workspace (any of this library's workspaces) on `stream`. */
qkdec_status qkdec_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/* One batched decode step (P1 FAQ "Why does adding sequences barely increase
 * the per-token time?"): reads tok[b] and pos[b] (device int32 [B]), runs
 * every layer of the pre-norm decoder
 *   h = f16(RMSNorm(x)); [q;k;v] = h W_qkv^T; rotate q, k at pos[b] (rotate-
 *   half RoPE, angle pos*base^(-2i/head_dim) formed in fp64); append k, v at
 *   pos[b]; x += f16(Attn(f16(q), n_ctx = pos[b]+1)) W_o^T;
 *   h2 = f16(RMSNorm(x)); x += f16b(silu(h2 W_g^T) * h2 W_u^T) W_d^T
 * then hf = f16(RMSNorm_final(x)), logits = hf W_lm^T, and writes
 * tok[b] = argmax, pos[b] += 1 on the device (so a captured step replays as
 * the next step).  x is fp32; f16b is the blocked fp16 rounding of
 * qkdec_gemm_q4k_xf32.  logits fp32 [B][vocab] written iff non-NULL.
 * kv: HOST array of n_layers cache descriptors (all of one type).  slot:
 * device int32 [B].  workspace: at least qkdec_step_workspace_size(m, B, kv)
 * bytes, zeroed once with qkdec_workspace_init before first use.  A pos[b]
 * that reaches capacity stores nothing and is reported by qkdec_step_status. */
size_t qkdec_step_workspace_size(const qkdec_model* m, int32_t B, const qkdec_kv_layer* kv);
qkdec_status qkdec_step(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* slot,
                        int32_t* pos, int32_t* tok, int32_t B, float* logits, void* workspace,
                        size_t ws_bytes, void* stream);
/* The decode step over paged pools: as qkdec_step, with every layer of kv a
 * pool of the same shape (pages of capacity tokens) and pages / max_pages
 * the page table shared by all layers (a sequence's token t sits in the same
 * page index of every layer); there is no slot argument.  The new token goes
 * to position pos[b] of sequence b, whose page must already be in the table
 * (the host grows a sequence before the step that crosses into a new page);
 * a position outside the table sets the step's error word (qkdec_step_status)
 * to QKDEC_E_CAPACITY.  Workspace: qkdec_step_paged_workspace_size(). */
size_t qkdec_step_paged_workspace_size(const qkdec_model* m, int32_t B_max, const qkdec_kv_layer* kv,
                                       int32_t max_pages);
qkdec_status qkdec_step_paged(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* pages,
                              int32_t max_pages, int32_t* pos, int32_t* tok, int32_t B, float* logits,
                              void* workspace, size_t ws_bytes, void* stream);
/* Prefill (P2 "This is the mirror image of the prefill story": a prompt is
 * many tokens of one sequence processed together, which batches the weight
 * read the way decode batches sequences): the n prompt tokens (device int32
 * [n]) of slot `slot` go through every layer at positions start .. start+n-1,
 * their keys and values are appended to the cache, and the final norm, LM
 * head and argmax run for the last token only: logits fp32 [vocab] (may be
 * NULL) and tok_out (device int32 [1]) = its argmax, the first generated
 * token.  Positions before start must already be cached.  The prompt is taken
 * in chunks of 2048 tokens, each chunk one pass of the layers with its
 * tokens as the rows: the projections are matrix-core products over 64-row
 * tiles (each weight read once per chunk and tile, RMSNorm and SwiGLU between
 * them in the decode step's rounding); the attention is a flash kernel for
 * an fp16 cache and the split-K decode attention with several prompt rows
 * per work item otherwise: token t attends over positions <= start+t, the
 * chunk's earlier tokens included (appended before the attention runs).
 * 0 <= slot < n_slots, n >= 1, start + n <= capacity (else QKDEC_E_CAPACITY,
 * nothing launched).  workspace: qkdec_prefill_workspace_size() bytes, zeroed
 * once with qkdec_workspace_init. */
size_t qkdec_prefill_workspace_size(const qkdec_model* m, const qkdec_kv_layer* kv);
qkdec_status qkdec_prefill(const qkdec_model* m, const qkdec_kv_layer* kv, int32_t slot, int32_t start,
                           const int32_t* tokens, int32_t n, float* logits, int32_t* tok_out, void* workspace,
                           size_t ws_bytes, void* stream);

/* Prefill into a paged pool (P1 "What I am building next": a sequence
 * admitted between steps brings its prompt; PagedAttention's pool holds it):
 * as qkdec_prefill for one sequence whose cache is every layer's paged pool
 * (kv[l].capacity = tokens per page, a power of two; kv[l].n_slots = pages in
 * the pool), its page table row pages (device int32 [max_pages]: logical
 * page j of the sequence is pool page pages[j]).  Positions before start
 * must already be in its pages.  A position whose table entry is outside the
 * pool (for instance -1) is not stored and raises QKDEC_E_CAPACITY in the
 * workspace's error word (qkdec_step_status); attention skips such pages.
 * Rejected with nothing launched: start + n > max_pages * capacity
 * (QKDEC_E_CAPACITY), a page size that is not a power of two, or query heads
 * per KV head that are not a power of two (QKDEC_E_SHAPE).  workspace:
 * qkdec_prefill_paged_workspace_size() bytes, zeroed once with
 * qkdec_workspace_init. */
size_t qkdec_prefill_paged_workspace_size(const qkdec_model* m, const qkdec_kv_layer* kv);
qkdec_status qkdec_prefill_paged(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* pages,
                                 int32_t max_pages, int32_t start, const int32_t* tokens, int32_t n, float* logits,
                                 int32_t* tok_out, void* workspace, size_t ws_bytes, void* stream);

/* The decode step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): as qkdec_step, with no workspace argument.  Its intermediates
 * live in a fixed device array of qkdec_step_noalloc_max_bytes() bytes
 * (32 MiB) inside the library, one per GPU it runs on, held until the
 * process ends; the call never allocates or frees.  A step whose workspace
 * (qkdec_step_workspace_size) exceeds that size returns QKDEC_E_WORKSPACE
 * (the Qwen-shaped 36-layer model fits at B <= 16 with caches of up to 64K
 * tokens).  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (different streams or host threads) race and must be ordered by
 * the caller.  err: device int32, set to QKDEC_E_CAPACITY when a position
 * reached the capacity (the caller clears it); this entry point keeps no
 * status for qkdec_step_status. */
size_t qkdec_step_noalloc_max_bytes(void);
qkdec_status qkdec_step_noalloc(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* slot, int32_t* pos,
                                int32_t* tok, int32_t B, float* logits, int32_t* err, void* stream);
/* Synchronizes `stream`, returns QKDEC_E_CAPACITY if any step since the last
 * call hit the capacity, else QKDEC_OK; the flag is cleared. */
qkdec_status qkdec_step_status(void* workspace, void* stream);

/* Where a step leaves its intermediates inside `workspace` (byte offsets),
 * for tests and debugging.  After qkdec_step they hold the LAST layer's
 * stages: x fp32 [B][hidden] (residual stream after that layer), h fp16
 * [B][hidden] (final RMSNorm output fed to the LM head), qkv fp32
 * [B][(n_q_heads + 2 n_kv_heads) head_dim] (projection before RoPE), q16 fp16
 * [B][n_q_heads head_dim] (rotated queries), o16 fp16 [B][n_q_heads head_dim]
 * (attention output), a fp32 [B][ffn] (SwiGLU activation before the f16b
 * rounding, which the down projection applies as it reads it).  Returns QKDEC_E_ARG/E_SHAPE on a model the step rejects. */
typedef struct {
  size_t x, h, qkv, q16, o16, a;
} qkdec_step_views;
qkdec_status qkdec_step_workspace_views(const qkdec_model* m, int32_t B, const qkdec_kv_layer* kv,
                                        qkdec_step_views* out);

/* ---------------------------------------------------------------- plans ---
 * P1 (opening section): reusing the recorded command stream takes the CPU
 * rebuild off the critical path.  qkdec_plan_create captures one qkdec_step
 * with these exact arguments into a HIP graph; qkdec_plan_launch replays it
 * (each replay is the next decode step, since pos and tok advance on the
 * device).  The plan owns the graph; destroy it before freeing its buffers. */
typedef struct qkdec_plan qkdec_plan;
qkdec_status qkdec_plan_create(qkdec_plan** plan, const qkdec_model* m, const qkdec_kv_layer* kv,
                               const int32_t* slot, int32_t* pos, int32_t* tok, int32_t B,
                               float* logits, void* workspace, size_t ws_bytes, void* stream);
qkdec_status qkdec_plan_launch(qkdec_plan* plan, void* stream);
void qkdec_plan_destroy(qkdec_plan* plan);

#ifdef __cplusplus
}
#endif
#endif /* QKDEC_H */
