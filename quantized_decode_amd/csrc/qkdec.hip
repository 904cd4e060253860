// The extern "C" entry points of libqkdec: argument validation, workspace
// carving, the kernel chain of one decode step, and HIP-graph plans.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "common.h"
#include "internal.h"

namespace {

using namespace qk;

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline qkdec_status hip_status(hipError_t e) { return e == hipSuccess ? QKDEC_OK : QKDEC_E_HIP; }
// HIP's last-error state is sticky per thread: clear whatever an earlier call
// (of this library or of the caller) left there, so that the check after our
// own launches reports only our launches.
inline void clear_stale_error() { (void)hipGetLastError(); }

// LDS a work-group may use on the current device (queried per call: cheap,
// and keeps the library free of mutable global state)
qkdec_status check_lds(size_t bytes) {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QKDEC_E_HIP;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return QKDEC_E_HIP;
  return bytes <= (size_t)v ? QKDEC_OK : QKDEC_E_UNSUPPORTED;
}

qkdec_status check_gemm(const void* W, int64_t N, int64_t K, const uint16_t* X, int64_t ldx, int32_t B) {
  if (!W || !X) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  if (N <= 0 || K <= 0 || N % 16 != 0 || K % 256 != 0) return QKDEC_E_SHAPE;
  if (N > kGemmMaxRows || K / 256 > (int64_t)1 << 20) return QKDEC_E_SHAPE;
  if (ldx < K) return QKDEC_E_SHAPE;
  if (!aligned(W, 16) || !aligned(X, 16) || ldx % 8 != 0) return QKDEC_E_ALIGN;
  return QKDEC_OK;
}

qkdec_status check_kv(const qkdec_kv_layer* kv) {
  if (!kv) return QKDEC_E_ARG;
  if (kv->type < QKDEC_KV_F16 || kv->type > QKDEC_KV_FP8_E4M3) return QKDEC_E_ARG;
  if (!kv->k || !kv->v) return QKDEC_E_ARG;
  if (kv->head_dim != 64 && kv->head_dim != 128) return QKDEC_E_SHAPE;
  if (kv->n_kv_heads < 1 || kv->n_slots < 1 || kv->capacity < 32 || kv->capacity % 32 != 0) return QKDEC_E_SHAPE;
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16)) return QKDEC_E_ALIGN;
  if (kv_k_q8(kv->type)) {
    if (!kv->k_scale) return QKDEC_E_ARG;
    if (!aligned(kv->k_scale, 16)) return QKDEC_E_ALIGN;
  }
  if (kv_v_q8(kv->type)) {
    if (!kv->v_scale) return QKDEC_E_ARG;
    if (!aligned(kv->v_scale, 16)) return QKDEC_E_ALIGN;
  }
  return QKDEC_OK;
}

bool same_kv_shape(const qkdec_kv_layer& a, const qkdec_kv_layer& b) {
  return a.type == b.type && a.n_kv_heads == b.n_kv_heads && a.head_dim == b.head_dim &&
         a.capacity == b.capacity && a.n_slots == b.n_slots;
}

qkdec_status check_model(const qkdec_model* m, const qkdec_kv_layer* kv) {
  if (!m || !kv) return QKDEC_E_ARG;
  if (m->n_layers < 1 || !m->layers || !m->embed || !m->lm_head || !m->norm_final) return QKDEC_E_ARG;
  if (m->hidden <= 0 || m->hidden % 256 != 0 || m->ffn <= 0 || m->ffn % 256 != 0 || m->vocab <= 0 ||
      m->vocab % 16 != 0)
    return QKDEC_E_SHAPE;
  if (m->n_q_heads < 1 || m->n_kv_heads < 1 || m->n_q_heads % m->n_kv_heads != 0 ||
      m->n_q_heads / m->n_kv_heads > 16)
    return QKDEC_E_SHAPE;
  if (m->head_dim != 64 && m->head_dim != 128) return QKDEC_E_SHAPE;
  if (((int64_t)m->n_q_heads * m->head_dim) % 256 != 0) return QKDEC_E_SHAPE;
  if (((int64_t)m->n_q_heads + 2 * (int64_t)m->n_kv_heads) * m->head_dim > kGemmMaxRows ||
      2 * (int64_t)m->ffn > kGemmMaxRows ||
      m->hidden > kSsMaxSlots * kSsCols)
    return QKDEC_E_SHAPE;
  if (!(m->rms_eps >= 0.f) || !(m->rope_base > 0.f)) return QKDEC_E_ARG;
  if (!aligned(m->embed, 16) || !aligned(m->lm_head, 16)) return QKDEC_E_ALIGN;
  for (int l = 0; l < m->n_layers; ++l) {
    const qkdec_layer& ly = m->layers[l];
    if (!ly.w_qkv || !ly.w_o || !ly.w_gate_up || !ly.w_down || !ly.norm_attn || !ly.norm_ffn) return QKDEC_E_ARG;
    if (!aligned(ly.w_qkv, 16) || !aligned(ly.w_o, 16) || !aligned(ly.w_gate_up, 16) || !aligned(ly.w_down, 16))
      return QKDEC_E_ALIGN;
    const qkdec_status s = check_kv(&kv[l]);
    if (s != QKDEC_OK) return s;
    if (!same_kv_shape(kv[l], kv[0])) return QKDEC_E_SHAPE;
  }
  if (kv[0].n_kv_heads != m->n_kv_heads || kv[0].head_dim != m->head_dim) return QKDEC_E_SHAPE;
  return QKDEC_OK;
}

// ---- step workspace layout (every region 256-byte aligned)
struct StepWs {
  int32_t* err;
  float* x;
  float* ss;
  uint16_t* h;
  float* qkv;
  uint16_t* q16;
  uint16_t* o16;
  float* a;
  float* attn_part;
  float2* rope;        // rotary (cos, sin) of each row's position, [B][head_dim/2]
  int32_t* page;       // paged step: page of each sequence's new token (-1: outside)
  int32_t* page_pos;   // and its position within the page
  float* kv_new;       // a cache with a Q8_0 part: the new token's rotated k, v [B][2][n_kv][head_dim]
  void* lm_part;
  void* gemm_ws;
  size_t bytes;
};

StepWs step_layout(const qkdec_model* m, int B, const qkdec_kv_layer* kv, char* base, int max_pages = 0) {
  StepWs w{};
  size_t off = 0;
  auto take = [&](size_t n) {
    char* p = base ? base + off : nullptr;
    off += round_up(n, 256);
    return p;
  };
  const int64_t hq = (int64_t)m->n_q_heads * m->head_dim;
  const int64_t nqkv = (int64_t)(m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim;
  w.err = reinterpret_cast<int32_t*>(take(256));
  w.x = reinterpret_cast<float*>(take((size_t)B * m->hidden * 4));
  w.ss = reinterpret_cast<float*>(take((size_t)kSsMaxSlots * 16 * 4));
  w.h = reinterpret_cast<uint16_t*>(take((size_t)B * m->hidden * 2));
  w.qkv = reinterpret_cast<float*>(take((size_t)B * nqkv * 4));
  w.q16 = reinterpret_cast<uint16_t*>(take((size_t)B * hq * 2));
  w.o16 = reinterpret_cast<uint16_t*>(take((size_t)B * hq * 2));
  w.a = reinterpret_cast<float*>(take((size_t)B * m->ffn * 4));
  w.attn_part = reinterpret_cast<float*>(
      take(attn_partials_bytes(B, m->n_q_heads, m->head_dim, attn_seq_cap(kv[0], max_pages), kv[0].n_kv_heads)));
  w.rope = reinterpret_cast<float2*>(take((size_t)B * (m->head_dim / 2) * sizeof(float2)));
  w.page = reinterpret_cast<int32_t*>(take((size_t)B * 4));
  w.page_pos = reinterpret_cast<int32_t*>(take((size_t)B * 4));
  w.kv_new = reinterpret_cast<float*>(take((size_t)B * 2 * m->n_kv_heads * m->head_dim * 4));
  w.lm_part = take(lm_head_partials_bytes(m->vocab, B));
  size_t g = gemm_workspace_bytes(nqkv, m->hidden, B, false);
  g = std::max(g, gemm_workspace_bytes(m->hidden, hq, B, false));
  g = std::max(g, gemm_workspace_bytes(2 * (int64_t)m->ffn, m->hidden, B, true));
  g = std::max(g, gemm_workspace_bytes(m->hidden, m->ffn, B, false));
  w.gemm_ws = take(g);
  w.bytes = off;
  return w;
}

// pages != nullptr: every layer of kv is a paged pool and sequence b's pages
// are pages[b * max_pages ...]; slot is unused
// err != nullptr: the capacity flag goes there instead of the workspace's
// error word
// The embedding and every layer of a step for B rows (row b: token tok[b] at
// position pos[b] of slot slot[b]), leaving the residual stream in w.x and its
// sum-of-squares slots in w.ss; w may be laid out for more rows than B.
qkdec_status run_layers(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* slot, const int32_t* pos,
                        const int32_t* tok, int B, const StepWs& w, hipStream_t st, const int32_t* pages,
                        int max_pages, int32_t* err) {
  int32_t* const err_word = err ? err : w.err;
  const int H = m->hidden, F = m->ffn, D = m->head_dim, Hq = m->n_q_heads;
  const int64_t hq = (int64_t)Hq * D;
  const int64_t nqkv = (int64_t)(Hq + 2 * m->n_kv_heads) * D;
  const float scale = 1.0f / sqrtf((float)D);
#define QK_TRY(expr)                                 \
  do {                                               \
    const hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return QKDEC_E_HIP;        \
  } while (0)
  // paged: every layer stores the new token of sequence b at the same page and
  // position within it, located once per step
  if (pages)
    QK_TRY(launch_page_locate(pages, max_pages, kv[0].capacity, kv[0].n_slots, pos, B, w.page, w.page_pos, st));
  QK_TRY(launch_rope_table(pos, B, D, m->rope_base, w.rope, st));
  QK_TRY(launch_embed(m->embed, H, m->vocab, tok, B, w.x, w.ss, st));
  for (int l = 0; l < m->n_layers; ++l) {
    const qkdec_layer& ly = m->layers[l];
    // RMSNorm is applied while each projection stages x (statistics in w.ss,
    // written by the kernel that last wrote x)
    GemmLaunch qkv{};
    qkv.W = ly.w_qkv; qkv.n_rows = nqkv; qkv.K = H; qkv.X = w.x; qkv.x_f32 = true; qkv.ldx = H; qkv.B = B;
    qkv.gamma = ly.norm_attn; qkv.ss_in = w.ss; qkv.eps = m->rms_eps;
    qkv.Y = w.qkv; qkv.ldy = nqkv; qkv.ws = w.gemm_ws;
    // ... finished per head: RoPE, q -> fp16, k and v appended to the cache
    RopeAppendArgs ra{};
    ra.slot = pages ? w.page : slot; ra.pos = pos; ra.spos = pages ? w.page_pos : pos;
    ra.k = reinterpret_cast<uint8_t*>(kv[l].k); ra.v = reinterpret_cast<uint8_t*>(kv[l].v);
    ra.ks = reinterpret_cast<uint16_t*>(kv[l].k_scale); ra.vs = reinterpret_cast<uint16_t*>(kv[l].v_scale);
    ra.n_kv = kv[l].n_kv_heads; ra.cap = kv[l].capacity; ra.n_slots = kv[l].n_slots; ra.Hq = Hq;
    ra.kf = kv_k_fmt(kv[l].type); ra.vf = kv_v_fmt(kv[l].type); ra.rope_base = m->rope_base; ra.rope = w.rope; ra.q16 = w.q16; ra.err = err_word;
    const bool q8 = ra.kf == kFmtQ8 || ra.vf == kFmtQ8;
    ra.kv_new = q8 ? w.kv_new : nullptr;
    // K = 4096: the resident multi-item projection, finishing each head slice
    // itself: fp16 and E4M3 parts appended, a Q8_0 part staged for the
    // attention kernel (its blocks span two work-groups), which quantizes and
    // appends it.  Otherwise the multi-item projection followed by RoPE and
    // the append as a small launch, or the split-K projection finishing each
    // head.
    const float* kv_new = nullptr;
    hipError_t eq = launch_gemm_wi_qkv(qkv, ra, D, st);
    if (eq == hipSuccess && q8) kv_new = w.kv_new;
    if (eq == hipErrorNotSupported) {
      eq = launch_gemm_wi(qkv, st);
      if (eq == hipErrorNotSupported) {
        QK_TRY(launch_gemm_qkv_rope(qkv, ra, D, st));
      } else {
        QK_TRY(eq);
        QK_TRY(launch_rope_append(kv[l], w.qkv, nqkv, Hq, B, ra.slot, pos, m->rope_base, w.q16, err_word, st,
                                  ra.spos, w.rope));
      }
    } else {
      QK_TRY(eq);
    }
    QK_TRY(launch_attn_decode(kv[l], slot, pos, B, w.q16, Hq, scale, nullptr, w.o16, w.attn_part, 1, st, pages,
                              max_pages, kv_new));
    // O projection: fp16 activations, K split over the waves of one work-group
    // per output tile (no split-K round trips); the fp32-activation projections
    // stage their activations once per work-group and split K across work-groups
    GemmLaunch o{};
    o.W = ly.w_o; o.n_rows = H; o.K = hq; o.X = w.o16; o.ldx = hq; o.B = B;
    o.Y = w.x; o.ldy = H; o.residual = w.x; o.ldr = H; o.ss_out = w.ss; o.ws = w.gemm_ws;
    QK_TRY(launch_gemm(o, st));
    GemmLaunch gu{};
    gu.W = ly.w_gate_up; gu.n_rows = F; gu.K = H; gu.X = w.x; gu.x_f32 = true; gu.ldx = H; gu.B = B;
    gu.gamma = ly.norm_ffn; gu.ss_in = w.ss; gu.eps = m->rms_eps;
    gu.swiglu = true; gu.A = w.a; gu.lda = F; gu.ws = w.gemm_ws;
    QK_TRY(launch_gemm(gu, st));
    GemmLaunch dn{};
    dn.W = ly.w_down; dn.n_rows = H; dn.K = F; dn.X = w.a; dn.x_f32 = true; dn.ldx = F; dn.B = B;
    dn.Y = w.x; dn.ldy = H; dn.residual = w.x; dn.ldr = H; dn.ss_out = w.ss; dn.ws = w.gemm_ws;
    QK_TRY(launch_gemm(dn, st));
  }
#undef QK_TRY
  return QKDEC_OK;
}

// err != nullptr: the capacity flag goes there instead of the workspace's
// error word
qkdec_status run_step(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* slot, int32_t* pos,
                      int32_t* tok, int B, float* logits, void* workspace, hipStream_t st,
                      const int32_t* pages = nullptr, int max_pages = 0, int32_t* err = nullptr) {
  const StepWs w = step_layout(m, B, kv, reinterpret_cast<char*>(workspace), max_pages);
  const qkdec_status s = run_layers(m, kv, slot, pos, tok, B, w, st, pages, max_pages, err);
  if (s != QKDEC_OK) return s;
  if (launch_rmsnorm_f16(w.x, m->norm_final, w.ss, m->hidden, B, m->rms_eps, w.h, st) != hipSuccess)
    return QKDEC_E_HIP;
  if (launch_lm_head_argmax(m->lm_head, m->vocab, m->hidden, w.h, B, logits, tok, w.lm_part, pos, st) != hipSuccess)
    return QKDEC_E_HIP;
  return QKDEC_OK;
}

// ---- prefill: the prompt in chunks of up to kPfChunk tokens of the one
// sequence (consecutive positions), each chunk one pass of the layers with its
// tokens as the rows: every projection a 64-row-tile MFMA GEMM over split K
// (gemm_pf) and the finish that adds the K ranges and stages the next input
// (pf_finish, pf_norm); RoPE, the KV append and the attention (kPfAttnRows
// rows per call) are the decode kernels.
struct PrefillWs {
  int32_t* err;
  float* x;        // residual stream [kPfChunk][H]
  float* ss;       // sum-of-squares slots the embedding writes (unused here)
  uint16_t* h;     // fp16 input of the next projection [kPfChunk][max(H, F)]
  void* xs;        // its sub-block sums [kPfChunk][max(H, F, Hq D) / 256][4] (half4)
  float* fd;       // and factors [kPfChunk][max(H, F, Hq D) / 256]
  float* ssq;      // block sums of squares of the residual stream [kPfChunk][H / 256]
  float* qkv;      // [kPfChunk][nqkv]
  uint16_t* q16;   // [kPfChunk][Hq D]
  uint16_t* o16;   // [kPfChunk][Hq D]
  float* part;     // K-range partial sums of the widest projection
  float* attn_part;
  float2* rope;
  void* lm_part;
  int32_t *rs, *rp, *rt;   // the chunk's slot (paged: page), position and token of each row
  int32_t* rsp;            // paged: each row's position within its page
  size_t bytes;
};

PrefillWs prefill_layout(const qkdec_model* m, const qkdec_kv_layer* kv, char* base) {
  PrefillWs w{};
  size_t off = 0;
  auto take = [&](size_t n) {
    char* p = base ? base + off : nullptr;
    off += round_up(n, 256);
    return p;
  };
  const int64_t R = kPfChunk, H = m->hidden, F = m->ffn;
  const int64_t hq = (int64_t)m->n_q_heads * m->head_dim;
  const int64_t nqkv = (int64_t)(m->n_q_heads + 2 * m->n_kv_heads) * m->head_dim;
  w.err = reinterpret_cast<int32_t*>(take(256));
  w.x = reinterpret_cast<float*>(take((size_t)(R * H) * 4));
  // the embedding kernel writes slot (c / 16) * 16 + row for column c: at most H + R floats
  w.ss = reinterpret_cast<float*>(take((size_t)(H + R) * 4));
  w.h = reinterpret_cast<uint16_t*>(take((size_t)(R * std::max(H, F)) * 2));
  const int64_t kbmax = std::max(std::max(H, F), hq) / 256;
  w.xs = take((size_t)(R * kbmax) * 4 * 8);
  w.fd = reinterpret_cast<float*>(take((size_t)(R * kbmax) * 4));
  w.ssq = reinterpret_cast<float*>(take((size_t)(R * (H / 256)) * 4));
  w.qkv = reinterpret_cast<float*>(take((size_t)(R * nqkv) * 4));
  w.q16 = reinterpret_cast<uint16_t*>(take((size_t)(R * hq) * 2));
  w.o16 = reinterpret_cast<uint16_t*>(take((size_t)(R * hq) * 2));
  // the partial sums of any chunk length (the K split grows as the rows shrink)
  size_t pb = 0;
  const int64_t shapes[4][2] = {{nqkv, H}, {H, hq}, {2 * F, H}, {H, F}};
  for (const auto& nk : shapes)
    for (int t = kPfRows; t <= kPfChunk; t += kPfRows)
      pb = std::max(pb, (size_t)pf_ksplit(nk[0], nk[1], t) * (size_t)(t * nk[0]) * 4);
  w.part = reinterpret_cast<float*>(take(pb));
  w.attn_part = reinterpret_cast<float*>(take(attn_prefill_partials_bytes(kPfAttnRows, m->n_q_heads, kv[0])));
  w.rope = reinterpret_cast<float2*>(take((size_t)R * (m->head_dim / 2) * sizeof(float2)));
  w.lm_part = take(lm_head_partials_bytes(m->vocab, 1));
  w.rs = reinterpret_cast<int32_t*>(take(R * 4));
  w.rp = reinterpret_cast<int32_t*>(take(R * 4));
  w.rt = reinterpret_cast<int32_t*>(take(R * 4));
  w.rsp = reinterpret_cast<int32_t*>(take(R * 4));
  w.bytes = off;
  return w;
}

size_t prefill_bytes(const qkdec_model* m, const qkdec_kv_layer* kv) { return prefill_layout(m, kv, nullptr).bytes; }

// pages != nullptr: every layer of kv is a paged pool and the sequence's page
// table row is pages[0 .. max_pages - 1]; slot is unused
qkdec_status run_prefill(const qkdec_model* m, const qkdec_kv_layer* kv, int slot, int start, const int32_t* tokens,
                         int n, float* logits, int32_t* tok_out, void* workspace, hipStream_t st,
                         const int32_t* pages = nullptr, int max_pages = 0) {
  const PrefillWs w = prefill_layout(m, kv, reinterpret_cast<char*>(workspace));
  const int H = m->hidden, F = m->ffn, D = m->head_dim, Hq = m->n_q_heads;
  const int64_t hq = (int64_t)Hq * D;
  const int nqkv = (Hq + 2 * m->n_kv_heads) * D;
  const float scale = 1.0f / sqrtf((float)D);
#define QK_TRY(expr)                                 \
  do {                                               \
    const hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return QKDEC_E_HIP;        \
  } while (0)
  int rows = 0;
  for (int off = 0; off < n; off += kPfChunk) {
    rows = n - off < kPfChunk ? n - off : kPfChunk;
    const int ks_qkv = pf_ksplit(nqkv, H, rows), ks_o = pf_ksplit(H, hq, rows),
              ks_gu = pf_ksplit(2 * (int64_t)F, H, rows), ks_dn = pf_ksplit(H, F, rows);
    if (pages)
      QK_TRY(launch_prefill_page_rows(pages, max_pages, kv[0].capacity, kv[0].n_slots, start + off, tokens + off, rows,
                                      w.rs, w.rp, w.rsp, w.rt, st));
    else
      QK_TRY(launch_prefill_rows(slot, start + off, tokens + off, rows, w.rs, w.rp, w.rt, st));
    QK_TRY(launch_rope_table(w.rp, rows, D, m->rope_base, w.rope, st));
    QK_TRY(launch_embed(m->embed, H, m->vocab, w.rt, rows, w.x, w.ss, st));
    // the first layer's input: RMSNorm of the embedding rows
    QK_TRY(launch_pf_finish(w.part, 0, rows, H, w.x, w.x, H, kPfNorm, w.ssq, nullptr, nullptr, nullptr, st));
    QK_TRY(launch_pf_norm(w.x, w.ssq, m->layers[0].norm_attn, m->rms_eps, H, rows, w.h, w.xs, w.fd, st));
    for (int l = 0; l < m->n_layers; ++l) {
      const qkdec_layer& ly = m->layers[l];
      QK_TRY(launch_gemm_pf(ly.w_qkv, nqkv, H, w.h, H, w.xs, nullptr, rows, w.part, ks_qkv, st));
      // one K range: the partial sums are the projection rows themselves
      const float* qkv = w.part;
      if (ks_qkv > 1) {
        QK_TRY(launch_pf_finish(w.part, ks_qkv, rows, nqkv, nullptr, w.qkv, nqkv, kPfOut, nullptr, nullptr, nullptr,
                                nullptr, st));
        qkv = w.qkv;
      }
      QK_TRY(launch_rope_append(kv[l], qkv, nqkv, Hq, rows, w.rs, w.rp, m->rope_base, w.q16, w.err, st,
                                pages ? w.rsp : w.rp, w.rope));
      QK_TRY(launch_attn_prefill(kv[l], w.rs, w.rp, rows, w.q16, Hq, scale, w.o16, w.attn_part, 1, st, pages,
                                 max_pages));
      QK_TRY(launch_pf_norm(nullptr, nullptr, nullptr, 0.f, (int)hq, rows, w.o16, w.xs, w.fd, st));
      QK_TRY(launch_gemm_pf(ly.w_o, H, hq, w.o16, hq, w.xs, nullptr, rows, w.part, ks_o, st));
      QK_TRY(launch_pf_finish(w.part, ks_o, rows, H, w.x, w.x, H, kPfNorm, w.ssq, nullptr, nullptr, nullptr, st));
      QK_TRY(launch_pf_norm(w.x, w.ssq, ly.norm_ffn, m->rms_eps, H, rows, w.h, w.xs, w.fd, st));
      QK_TRY(launch_gemm_pf(ly.w_gate_up, 2 * (int64_t)F, H, w.h, H, w.xs, nullptr, rows, w.part, ks_gu, st));
      QK_TRY(launch_pf_finish(w.part, ks_gu, rows, 2 * F, nullptr, nullptr, 0, kPfSwiglu, nullptr, w.h, w.xs, w.fd,
                              st));
      QK_TRY(launch_gemm_pf(ly.w_down, H, F, w.h, F, w.xs, w.fd, rows, w.part, ks_dn, st));
      QK_TRY(launch_pf_finish(w.part, ks_dn, rows, H, w.x, w.x, H, kPfNorm, w.ssq, nullptr, nullptr, nullptr, st));
      // the next layer's attention input, or after the last layer the final norm
      const float* gamma = l + 1 < m->n_layers ? m->layers[l + 1].norm_attn : m->norm_final;
      QK_TRY(launch_pf_norm(w.x, w.ssq, gamma, m->rms_eps, H, rows, w.h, w.xs, w.fd, st));
    }
  }
  // the LM head of the prompt's last token (row rows - 1 of the last chunk)
  QK_TRY(launch_lm_head_argmax(m->lm_head, m->vocab, H, w.h + (size_t)(rows - 1) * H, 1, logits, tok_out, w.lm_part,
                               nullptr, st));
#undef QK_TRY
  return QKDEC_OK;
}

// ---- the step's fixed device scratch (qkdec_step_noalloc): one array per
// GPU the library runs on, held until the process ends.  Host code never
// passes the array's name to a kernel or a copy: it is a host-side stand-in.
// Each device's address comes from hipGetSymbolAddress, taken once with that
// device current, and only that address is used.
constexpr size_t kStepScratchBytes = (size_t)32 << 20;
__device__ __align__(256) char scratch[kStepScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (nullptr on failure).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

struct qkdec_plan {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

extern "C" {

const char* qkdec_status_str(qkdec_status s) {
  switch (s) {
    case QKDEC_OK: return "QKDEC_OK";
    case QKDEC_E_ARG: return "QKDEC_E_ARG: invalid argument";
    case QKDEC_E_SHAPE: return "QKDEC_E_SHAPE: unsupported or inconsistent shape";
    case QKDEC_E_ALIGN: return "QKDEC_E_ALIGN: misaligned pointer or leading dimension";
    case QKDEC_E_WORKSPACE: return "QKDEC_E_WORKSPACE: workspace missing or too small";
    case QKDEC_E_CAPACITY: return "QKDEC_E_CAPACITY: position reached the cache capacity";
    case QKDEC_E_UNSUPPORTED: return "QKDEC_E_UNSUPPORTED: not supported by this build";
    case QKDEC_E_HIP: return "QKDEC_E_HIP: HIP runtime error";
    default: return "QKDEC: unknown status";
  }
}

int32_t qkdec_abi_version(void) { return QKDEC_ABI_VERSION; }

#ifndef QKDEC_BUILD_ID
#define QKDEC_BUILD_ID "unknown"
#endif
const char* qkdec_build_id(void) { return QKDEC_BUILD_ID; }

size_t qkdec_gemm_q4k_workspace_size(int64_t N, int64_t K, int32_t B) {
  if (N <= 0 || K <= 0 || N % 16 || K % 256 || B < 1 || B > 16) return 0;
  return gemm_workspace_bytes(N, K, B, false);
}

qkdec_status qkdec_gemm_q4k(const void* W, int64_t N, int64_t K, const uint16_t* X, int64_t ldx, int32_t B,
                            float* Y, int64_t ldy, const float* residual, int64_t ldr, void* workspace,
                            size_t ws_bytes, void* stream) {
  qkdec_status s = check_gemm(W, N, K, X, ldx, B);
  if (s != QKDEC_OK) return s;
  if (!Y) return QKDEC_E_ARG;
  if (ldy < N || (residual && ldr < N)) return QKDEC_E_SHAPE;
  if (!workspace || ws_bytes < gemm_workspace_bytes(N, K, B, false)) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 256)) return QKDEC_E_ALIGN;
  clear_stale_error();
  // the multi-item kernel where it serves the shape (K split over the waves
  // of a work-group; at K = 12288 also over four work-groups, through the
  // workspace), else K over the waves of one work-group per tile
  GemmLaunch L{};
  L.W = W; L.n_rows = N; L.K = K; L.X = X; L.ldx = ldx; L.B = B;
  L.Y = Y; L.ldy = ldy; L.residual = residual; L.ldr = ldr; L.ws = workspace;
  return hip_status(launch_gemm(L, as_stream(stream)));
}

qkdec_status qkdec_gemm_q4k_engine(const void* W, int64_t N, int64_t K, const uint16_t* X, int64_t ldx, int32_t B,
                                   float* Y, int64_t ldy, const float* residual, int64_t ldr, int32_t engine,
                                   void* workspace, size_t ws_bytes, void* stream) {
  if (engine < QKDEC_GEMM_AUTO || engine > QKDEC_GEMM_MATVEC) return QKDEC_E_ARG;
  if (engine == QKDEC_GEMM_MATVEC && B > QKDEC_MATVEC_MAX_B) return QKDEC_E_SHAPE;
  qkdec_status s = check_gemm(W, N, K, X, ldx, B);
  if (s != QKDEC_OK) return s;
  if (!Y) return QKDEC_E_ARG;
  if (ldy < N || (residual && ldr < N)) return QKDEC_E_SHAPE;
  if (!workspace || ws_bytes < gemm_workspace_bytes(N, K, B, false)) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 256)) return QKDEC_E_ALIGN;
  clear_stale_error();
  GemmLaunch L{};
  L.W = W; L.n_rows = N; L.K = K; L.X = X; L.ldx = ldx; L.B = B;
  L.Y = Y; L.ldy = ldy; L.residual = residual; L.ldr = ldr; L.ws = workspace; L.kernel = engine;
  return hip_status(launch_gemm(L, as_stream(stream)));
}

qkdec_status qkdec_gemm_q4k_xf32(const void* W, int64_t N, int64_t K, const float* X, int64_t ldx, int32_t B,
                                 float* Y, int64_t ldy, const float* residual, int64_t ldr, void* workspace,
                                 size_t ws_bytes, void* stream) {
  if (!W || !X) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  if (N <= 0 || K <= 0 || N % 16 != 0 || K % 256 != 0) return QKDEC_E_SHAPE;
  if (N > kGemmMaxRows || K / 256 > (int64_t)1 << 20) return QKDEC_E_SHAPE;
  if (ldx < K) return QKDEC_E_SHAPE;
  if (!aligned(W, 16) || !aligned(X, 16) || ldx % 4 != 0) return QKDEC_E_ALIGN;
  if (!Y) return QKDEC_E_ARG;
  if (ldy < N || (residual && ldr < N)) return QKDEC_E_SHAPE;
  if (!workspace || ws_bytes < gemm_workspace_bytes(N, K, B, false)) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 256)) return QKDEC_E_ALIGN;
  clear_stale_error();
  return hip_status(
      launch_gemm_q4k_xf32(W, N, K, X, ldx, B, Y, ldy, residual, ldr, workspace, as_stream(stream)));
}

size_t qkdec_gemm_q4k_swiglu_workspace_size(int64_t F, int64_t K, int32_t B) {
  if (F <= 0 || K <= 0 || F % 16 || K % 256 || B < 1 || B > 16) return 0;
  return gemm_workspace_bytes(2 * F, K, B, true);
}

qkdec_status qkdec_gemm_q4k_swiglu(const void* W, int64_t F, int64_t K, const uint16_t* X, int64_t ldx, int32_t B,
                                   float* A, int64_t lda, void* workspace, size_t ws_bytes, void* stream) {
  if (F <= 0 || F % 16 != 0) return QKDEC_E_SHAPE;
  qkdec_status s = check_gemm(W, 2 * F, K, X, ldx, B);
  if (s != QKDEC_OK) return s;
  if (!A) return QKDEC_E_ARG;
  if (lda < F) return QKDEC_E_SHAPE;
  if (!workspace || ws_bytes < gemm_workspace_bytes(2 * F, K, B, true)) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 256)) return QKDEC_E_ALIGN;
  clear_stale_error();
  return hip_status(launch_gemm_q4k_swiglu(W, F, K, X, ldx, B, A, lda, workspace, as_stream(stream)));
}

qkdec_status qkdec_dequant_q4k(const void* W, int64_t n_blocks, float* out, void* stream) {
  if (!W || !out) return QKDEC_E_ARG;
  if (n_blocks <= 0 || n_blocks > ((int64_t)1 << 31) - 1) return QKDEC_E_SHAPE;
  if (!aligned(W, 4)) return QKDEC_E_ALIGN;
  clear_stale_error();
  return hip_status(launch_dequant_q4k(W, n_blocks, out, as_stream(stream)));
}

static qkdec_status kv_append_common(const qkdec_kv_layer* kv, int type, const int32_t* slot, const int32_t* pos,
                                     const float* k, const float* v, int32_t B, int32_t* err, void* stream) {
  qkdec_status s = check_kv(kv);
  if (s != QKDEC_OK) return s;
  if (type >= 0 && kv->type != type) return QKDEC_E_ARG;
  if (!slot || !pos || !k || !v) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  clear_stale_error();
  return hip_status(launch_kv_append(*kv, slot, pos, k, v, B, err, as_stream(stream)));
}

qkdec_status qkdec_kv_append_f16(const qkdec_kv_layer* kv, const int32_t* slot, const int32_t* pos, const float* k,
                                 const float* v, int32_t B, int32_t* err, void* stream) {
  return kv_append_common(kv, QKDEC_KV_F16, slot, pos, k, v, B, err, stream);
}

qkdec_status qkdec_kv_append_q8_0(const qkdec_kv_layer* kv, const int32_t* slot, const int32_t* pos, const float* k,
                                  const float* v, int32_t B, int32_t* err, void* stream) {
  return kv_append_common(kv, QKDEC_KV_Q8_0, slot, pos, k, v, B, err, stream);
}

qkdec_status qkdec_kv_append(const qkdec_kv_layer* kv, const int32_t* slot, const int32_t* pos, const float* k,
                             const float* v, int32_t B, int32_t* err, void* stream) {
  return kv_append_common(kv, -1, slot, pos, k, v, B, err, stream);
}

// The shapes qkdec_attn_decode(_paged) accept (pointers aside): 0 otherwise.
static bool attn_shape_ok(int32_t B, int32_t n_q_heads, const qkdec_kv_layer* kv) {
  return kv && (kv->head_dim == 64 || kv->head_dim == 128) && kv->n_kv_heads >= 1 && kv->capacity >= 32 &&
         kv->capacity % 32 == 0 && B >= 1 && B <= 16 && n_q_heads >= 1 && n_q_heads % kv->n_kv_heads == 0 &&
         n_q_heads / kv->n_kv_heads <= 16;
}

size_t qkdec_attn_workspace_size(int32_t B, int32_t n_q_heads, const qkdec_kv_layer* kv) {
  if (!attn_shape_ok(B, n_q_heads, kv)) return 0;
  return attn_partials_bytes(B, n_q_heads, kv->head_dim, kv->capacity, kv->n_kv_heads);
}

qkdec_status qkdec_attn_decode(const qkdec_kv_layer* kv, const int32_t* slot, const int32_t* n_ctx, int32_t B,
                               const uint16_t* Q, int32_t n_q_heads, float scale, float* O, uint16_t* O16,
                               void* workspace, size_t ws_bytes, void* stream) {
  qkdec_status s = check_kv(kv);
  if (s != QKDEC_OK) return s;
  if (!slot || !n_ctx || !Q || (!O && !O16)) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  if (n_q_heads < 1 || n_q_heads % kv->n_kv_heads != 0 || n_q_heads / kv->n_kv_heads > 16) return QKDEC_E_SHAPE;
  if (!(scale == scale)) return QKDEC_E_ARG;
  if (!aligned(Q, 16) || (O && !aligned(O, 16))) return QKDEC_E_ALIGN;
  const size_t need = attn_partials_bytes(B, n_q_heads, kv->head_dim, kv->capacity, kv->n_kv_heads);
  if (!workspace || ws_bytes < need) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 16)) return QKDEC_E_ALIGN;
  clear_stale_error();
  return hip_status(launch_attn_decode(*kv, slot, n_ctx, B, Q, n_q_heads, scale, O, O16,
                                       reinterpret_cast<float*>(workspace), 0, as_stream(stream)));
}

// ---- paged pool: kv's slots are pages of kv->capacity tokens
static qkdec_status check_pages(const qkdec_kv_layer* kv, const int32_t* pages, int32_t max_pages) {
  if (!pages) return QKDEC_E_ARG;
  if (kv->capacity & (kv->capacity - 1)) return QKDEC_E_SHAPE;          // page size: a power of two
  if (max_pages < 1 || (int64_t)max_pages * kv->capacity > ((int64_t)1 << 30)) return QKDEC_E_SHAPE;
  if (!aligned(pages, 4)) return QKDEC_E_ALIGN;
  return QKDEC_OK;
}

size_t qkdec_attn_paged_workspace_size(int32_t B, int32_t n_q_heads, const qkdec_kv_layer* kv, int32_t max_pages) {
  if (!attn_shape_ok(B, n_q_heads, kv) || max_pages < 1 || (int64_t)max_pages * kv->capacity > ((int64_t)1 << 30))
    return 0;
  return attn_partials_bytes(B, n_q_heads, kv->head_dim, attn_seq_cap(*kv, max_pages), kv->n_kv_heads);
}

qkdec_status qkdec_attn_decode_paged(const qkdec_kv_layer* kv, const int32_t* pages, int32_t max_pages,
                                     const int32_t* n_ctx, int32_t B, const uint16_t* Q, int32_t n_q_heads,
                                     float scale, float* O, uint16_t* O16, void* workspace, size_t ws_bytes,
                                     void* stream) {
  qkdec_status s = check_kv(kv);
  if (s != QKDEC_OK) return s;
  s = check_pages(kv, pages, max_pages);
  if (s != QKDEC_OK) return s;
  if (!n_ctx || !Q || (!O && !O16)) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  if (n_q_heads < 1 || n_q_heads % kv->n_kv_heads != 0 || n_q_heads / kv->n_kv_heads > 16) return QKDEC_E_SHAPE;
  if (!(scale == scale)) return QKDEC_E_ARG;
  if (!aligned(Q, 16) || (O && !aligned(O, 16))) return QKDEC_E_ALIGN;
  const size_t need =
      attn_partials_bytes(B, n_q_heads, kv->head_dim, attn_seq_cap(*kv, max_pages), kv->n_kv_heads);
  if (!workspace || ws_bytes < need) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 16)) return QKDEC_E_ALIGN;
  clear_stale_error();
  return hip_status(launch_attn_decode(*kv, nullptr, n_ctx, B, Q, n_q_heads, scale, O, O16,
                                       reinterpret_cast<float*>(workspace), 0, as_stream(stream), pages, max_pages));
}

qkdec_status qkdec_kv_append_paged(const qkdec_kv_layer* kv, const int32_t* pages, int32_t max_pages,
                                   const int32_t* pos, const float* k, const float* v, int32_t B, int32_t* err,
                                   void* stream) {
  qkdec_status s = check_kv(kv);
  if (s != QKDEC_OK) return s;
  s = check_pages(kv, pages, max_pages);
  if (s != QKDEC_OK) return s;
  if (!pos || !k || !v) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  clear_stale_error();
  return hip_status(launch_kv_append(*kv, nullptr, pos, k, v, B, err, as_stream(stream), pages, max_pages));
}

size_t qkdec_lm_head_workspace_size(int64_t V, int32_t B) {
  if (V < 1 || B < 1) return 0;
  return lm_head_partials_bytes(V, B);
}

qkdec_status qkdec_lm_head_argmax(const uint16_t* Wlm, int64_t V, int64_t H, const uint16_t* X, int32_t B,
                                  float* logits, int32_t* tok, void* workspace, size_t ws_bytes, void* stream) {
  if (!Wlm || !X || !tok) return QKDEC_E_ARG;
  if (B < 1 || B > 16 || V < 16 || V % 16 != 0 || V > ((int64_t)1 << 30) || H < 256 || H % 256 != 0 ||
      H > ((int64_t)1 << 20))
    return QKDEC_E_SHAPE;
  if (!aligned(Wlm, 16) || !aligned(X, 16)) return QKDEC_E_ALIGN;
  if (!workspace || ws_bytes < lm_head_partials_bytes(V, B)) return QKDEC_E_WORKSPACE;
  qkdec_status s = check_lds(lm_head_lds_bytes(H, B));
  if (s != QKDEC_OK) return s;
  clear_stale_error();
  return hip_status(launch_lm_head_argmax(Wlm, V, H, X, B, logits, tok, workspace, nullptr, as_stream(stream)));
}

size_t qkdec_step_workspace_size(const qkdec_model* m, int32_t B, const qkdec_kv_layer* kv) {
  if (check_model(m, kv) != QKDEC_OK || B < 1 || B > 16) return 0;
  return step_layout(m, B, kv, nullptr).bytes;
}

qkdec_status qkdec_step_workspace_views(const qkdec_model* m, int32_t B, const qkdec_kv_layer* kv,
                                        qkdec_step_views* out) {
  if (!out) return QKDEC_E_ARG;
  const qkdec_status s = check_model(m, kv);
  if (s != QKDEC_OK) return s;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  char* const base = reinterpret_cast<char*>(256);  // any non-null base; offsets are relative to it
  const StepWs w = step_layout(m, B, kv, base);
  auto off = [&](const void* p) { return (size_t)(reinterpret_cast<const char*>(p) - base); };
  out->x = off(w.x);
  out->h = off(w.h);
  out->qkv = off(w.qkv);
  out->q16 = off(w.q16);
  out->o16 = off(w.o16);
  out->a = off(w.a);
  return QKDEC_OK;
}

qkdec_status qkdec_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || ws_bytes == 0) return QKDEC_E_ARG;
  if (!aligned(workspace, 4)) return QKDEC_E_ALIGN;
  clear_stale_error();
  return hip_status(launch_fill_zero(workspace, ws_bytes, as_stream(stream)));
}

qkdec_status qkdec_step(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* slot, int32_t* pos,
                        int32_t* tok, int32_t B, float* logits, void* workspace, size_t ws_bytes, void* stream) {
  qkdec_status s = check_model(m, kv);
  if (s != QKDEC_OK) return s;
  if (!slot || !pos || !tok) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  if (!workspace || ws_bytes < step_layout(m, B, kv, nullptr).bytes) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 256)) return QKDEC_E_ALIGN;
  s = check_lds(lm_head_lds_bytes(m->hidden, B));
  if (s != QKDEC_OK) return s;
  clear_stale_error();
  return run_step(m, kv, slot, pos, tok, B, logits, workspace, as_stream(stream));
}

size_t qkdec_step_paged_workspace_size(const qkdec_model* m, int32_t B, const qkdec_kv_layer* kv,
                                       int32_t max_pages) {
  if (check_model(m, kv) != QKDEC_OK || B < 1 || B > 16 || max_pages < 1 ||
      (int64_t)max_pages * kv[0].capacity > ((int64_t)1 << 30))
    return 0;
  return step_layout(m, B, kv, nullptr, max_pages).bytes;
}

qkdec_status qkdec_step_paged(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* pages,
                              int32_t max_pages, int32_t* pos, int32_t* tok, int32_t B, float* logits,
                              void* workspace, size_t ws_bytes, void* stream) {
  qkdec_status s = check_model(m, kv);
  if (s != QKDEC_OK) return s;
  for (int l = 0; l < m->n_layers; ++l) {
    s = check_pages(&kv[l], pages, max_pages);
    if (s != QKDEC_OK) return s;
  }
  if (!pos || !tok) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  if (!workspace || ws_bytes < step_layout(m, B, kv, nullptr, max_pages).bytes) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 256)) return QKDEC_E_ALIGN;
  s = check_lds(lm_head_lds_bytes(m->hidden, B));
  if (s != QKDEC_OK) return s;
  clear_stale_error();
  return run_step(m, kv, nullptr, pos, tok, B, logits, workspace, as_stream(stream), pages, max_pages);
}

size_t qkdec_step_noalloc_max_bytes(void) { return kStepScratchBytes; }

qkdec_status qkdec_step_noalloc(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* slot, int32_t* pos,
                                int32_t* tok, int32_t B, float* logits, int32_t* err, void* stream) {
  qkdec_status s = check_model(m, kv);
  if (s != QKDEC_OK) return s;
  if (!slot || !pos || !tok || !err) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  const size_t need = step_layout(m, B, kv, nullptr).bytes;
  if (need > kStepScratchBytes) return QKDEC_E_WORKSPACE;
  s = check_lds(lm_head_lds_bytes(m->hidden, B));
  if (s != QKDEC_OK) return s;
  clear_stale_error();
  void* base = device_scratch();
  if (!base) return QKDEC_E_HIP;
  hipStream_t st = as_stream(stream);
  // The split-K arrival counters must read zero at the first GEMM; where they
  // sit depends on this call's shapes, so the area is cleared every call (the
  // previous call on this device may have left other data there).
  const StepWs w = step_layout(m, B, kv, reinterpret_cast<char*>(base));
  const size_t ctr = gemm_workspace_bytes(16, 256, 1, false);   // the fixed counter area at the start
  if (launch_fill_zero(w.gemm_ws, ctr, st) != hipSuccess) return QKDEC_E_HIP;
  return run_step(m, kv, slot, pos, tok, B, logits, base, st, nullptr, 0, err);
}

size_t qkdec_prefill_workspace_size(const qkdec_model* m, const qkdec_kv_layer* kv) {
  if (check_model(m, kv) != QKDEC_OK) return 0;
  return prefill_bytes(m, kv);
}

qkdec_status qkdec_prefill(const qkdec_model* m, const qkdec_kv_layer* kv, int32_t slot, int32_t start,
                           const int32_t* tokens, int32_t n, float* logits, int32_t* tok_out, void* workspace,
                           size_t ws_bytes, void* stream) {
  qkdec_status s = check_model(m, kv);
  if (s != QKDEC_OK) return s;
  if (!tokens || !tok_out) return QKDEC_E_ARG;
  if (n < 1 || start < 0 || slot < 0 || slot >= kv[0].n_slots) return QKDEC_E_SHAPE;
  if ((int64_t)start + n > kv[0].capacity) return QKDEC_E_CAPACITY;
  if (!workspace || ws_bytes < prefill_bytes(m, kv)) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 256)) return QKDEC_E_ALIGN;
  s = check_lds(lm_head_lds_bytes(m->hidden, 1));
  if (s != QKDEC_OK) return s;
  clear_stale_error();
  return run_prefill(m, kv, slot, start, tokens, n, logits, tok_out, workspace, as_stream(stream));
}

size_t qkdec_prefill_paged_workspace_size(const qkdec_model* m, const qkdec_kv_layer* kv) {
  return qkdec_prefill_workspace_size(m, kv);
}

qkdec_status qkdec_prefill_paged(const qkdec_model* m, const qkdec_kv_layer* kv, const int32_t* pages,
                                 int32_t max_pages, int32_t start, const int32_t* tokens, int32_t n, float* logits,
                                 int32_t* tok_out, void* workspace, size_t ws_bytes, void* stream) {
  qkdec_status s = check_model(m, kv);
  if (s != QKDEC_OK) return s;
  for (int l = 0; l < m->n_layers; ++l) {
    s = check_pages(&kv[l], pages, max_pages);
    if (s != QKDEC_OK) return s;
  }
  const int G = m->n_q_heads / m->n_kv_heads;
  if (G & (G - 1)) return QKDEC_E_SHAPE;   // the paged prompt attention takes G a power of two
  if (!tokens || !tok_out) return QKDEC_E_ARG;
  if (n < 1 || start < 0) return QKDEC_E_SHAPE;
  if ((int64_t)start + n > (int64_t)max_pages * kv[0].capacity) return QKDEC_E_CAPACITY;
  if (!workspace || ws_bytes < prefill_bytes(m, kv)) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 256)) return QKDEC_E_ALIGN;
  s = check_lds(lm_head_lds_bytes(m->hidden, 1));
  if (s != QKDEC_OK) return s;
  clear_stale_error();
  return run_prefill(m, kv, 0, start, tokens, n, logits, tok_out, workspace, as_stream(stream), pages, max_pages);
}

qkdec_status qkdec_step_status(void* workspace, void* stream) {
  if (!workspace) return QKDEC_E_ARG;
  int32_t flag = 0;
  hipStream_t st = as_stream(stream);
  if (hipMemcpyAsync(&flag, workspace, sizeof(flag), hipMemcpyDeviceToHost, st) != hipSuccess) return QKDEC_E_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return QKDEC_E_HIP;
  if (flag == 0) return QKDEC_OK;
  const int32_t zero = 0;
  if (hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, st) != hipSuccess) return QKDEC_E_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return QKDEC_E_HIP;
  return QKDEC_E_CAPACITY;
}

qkdec_status qkdec_plan_create(qkdec_plan** plan, const qkdec_model* m, const qkdec_kv_layer* kv,
                               const int32_t* slot, int32_t* pos, int32_t* tok, int32_t B, float* logits,
                               void* workspace, size_t ws_bytes, void* stream) {
  if (!plan || !stream) return QKDEC_E_ARG;
  *plan = nullptr;
  qkdec_status s = check_model(m, kv);
  if (s != QKDEC_OK) return s;
  if (!slot || !pos || !tok) return QKDEC_E_ARG;
  if (B < 1 || B > 16) return QKDEC_E_SHAPE;
  if (!workspace || ws_bytes < step_layout(m, B, kv, nullptr).bytes) return QKDEC_E_WORKSPACE;
  if (!aligned(workspace, 256)) return QKDEC_E_ALIGN;
  s = check_lds(lm_head_lds_bytes(m->hidden, B));
  if (s != QKDEC_OK) return s;
  hipStream_t st = as_stream(stream);
  clear_stale_error();
  if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess) return QKDEC_E_HIP;
  const qkdec_status rs = run_step(m, kv, slot, pos, tok, B, logits, workspace, st);
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(st, &graph);
  if (rs != QKDEC_OK || ec != hipSuccess || !graph) {
    if (graph) (void)hipGraphDestroy(graph);
    return rs != QKDEC_OK ? rs : QKDEC_E_HIP;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return QKDEC_E_HIP;
  }
  qkdec_plan* p = new (std::nothrow) qkdec_plan{graph, exec};
  if (!p) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return QKDEC_E_ARG;
  }
  *plan = p;
  return QKDEC_OK;
}

qkdec_status qkdec_plan_launch(qkdec_plan* plan, void* stream) {
  if (!plan) return QKDEC_E_ARG;
  return hip_status(hipGraphLaunch(plan->exec, as_stream(stream)));
}

void qkdec_plan_destroy(qkdec_plan* plan) {
  if (!plan) return;
  (void)hipGraphExecDestroy(plan->exec);
  (void)hipGraphDestroy(plan->graph);
  delete plan;
}

}  // extern "C"
