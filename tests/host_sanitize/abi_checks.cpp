// Host-side checks of the C-ABI's validation and size arithmetic, for a build
// of the library's host code with AddressSanitizer and UndefinedBehavior-
// Sanitizer (test_host_sanitizers.py builds and runs it).  Every call here is
// rejected by the library's own checks before anything reaches the GPU, or is
// a pure host computation (sizes, workspace views, status strings); device
// pointers are fake aligned addresses that are never dereferenced.  The
// program refuses to run where a GPU is visible.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <limits>
#include <vector>

#include "../../include/qkdec.h"

static int g_failures = 0;
static int g_checks = 0;

#define EXPECT_EQ(call, want)                                                                             \
  do {                                                                                                   \
    const long long got_ = (long long)(call);                                                            \
    ++g_checks;                                                                                          \
    if (got_ != (long long)(want)) {                                                                     \
      std::printf("FAIL line %d: %s -> %lld (want %lld)\n", __LINE__, #call, got_, (long long)(want));  \
      ++g_failures;                                                                                      \
    }                                                                                                    \
  } while (0)
#define EXPECT_TRUE(cond)                                       \
  do {                                                          \
    ++g_checks;                                                 \
    if (!(cond)) {                                              \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);      \
      ++g_failures;                                             \
    }                                                           \
  } while (0)

template <typename T>
static T* fake(uintptr_t a) {
  return reinterpret_cast<T*>(a);
}

// A well-formed Qwen-shaped description over fake device addresses.
struct Model {
  std::vector<qkdec_layer> layers;
  std::vector<qkdec_kv_layer> kv;
  qkdec_model m{};
  explicit Model(int n_layers = 4, int32_t kv_type = QKDEC_KV_F16) {
    layers.resize(n_layers);
    kv.resize(n_layers);
    for (int l = 0; l < n_layers; ++l) {
      const uintptr_t base = 0x100000000ull + (uintptr_t)l * 0x10000000ull;
      layers[l] = qkdec_layer{fake<void>(base), fake<void>(base + 0x1000000), fake<void>(base + 0x2000000),
                              fake<void>(base + 0x3000000), fake<float>(base + 0x4000000),
                              fake<float>(base + 0x5000000)};
      kv[l] = qkdec_kv_layer{kv_type, 8, 128, 2432, 8, fake<void>(base + 0x6000000), fake<void>(base + 0x7000000),
                             fake<void>(base + 0x8000000), fake<void>(base + 0x9000000)};
    }
    m.n_layers = n_layers;
    m.hidden = 4096;
    m.n_q_heads = 32;
    m.n_kv_heads = 8;
    m.head_dim = 128;
    m.ffn = 12288;
    m.vocab = 151936;
    m.rms_eps = 1e-6f;
    m.rope_base = 1e6f;
    m.embed = fake<uint16_t>(0x10000000);
    m.lm_head = fake<uint16_t>(0x20000000);
    m.norm_final = fake<float>(0x30000000);
    m.layers = layers.data();
  }
};

static void status_strings() {
  for (int s = -10; s <= 2; ++s) EXPECT_TRUE(qkdec_status_str(s) != nullptr);
  EXPECT_TRUE(qkdec_abi_version() > 0);
  EXPECT_TRUE(qkdec_build_id() != nullptr);
}

static void size_functions() {
  const int64_t big = std::numeric_limits<int64_t>::max();
  const int64_t ns[] = {-4096, -1, 0, 16, 4096, 6144, 24576, (int64_t)1 << 40, big};
  const int32_t bs[] = {-1, 0, 1, 8, 16, 17, std::numeric_limits<int32_t>::max()};
  for (int64_t n : ns)
    for (int64_t k : ns)
      for (int32_t b : bs) {
        (void)qkdec_gemm_q4k_workspace_size(n, k, b);
        (void)qkdec_gemm_q4k_swiglu_workspace_size(n, k, b);
      }
  for (int64_t v : ns)
    for (int32_t b : bs) (void)qkdec_lm_head_workspace_size(v, b);
  EXPECT_TRUE(qkdec_gemm_q4k_workspace_size(4096, 12288, 8) > 0);
  EXPECT_EQ(qkdec_step_noalloc_max_bytes(), (size_t)32 << 20);
  // attention workspace over extreme cache shapes
  const int32_t caps[] = {-1, 0, 32, 2432, 1 << 20, std::numeric_limits<int32_t>::max()};
  for (int32_t cap : caps)
    for (int32_t hq : {-1, 0, 32, 1 << 20})
      for (int32_t b : bs) {
        qkdec_kv_layer kv{QKDEC_KV_F16, 8, 128, cap, 8, fake<void>(0x1000), fake<void>(0x2000), nullptr, nullptr};
        (void)qkdec_attn_workspace_size(b, hq, &kv);
        for (int32_t mp : {-1, 0, 1, 64, 1 << 20}) (void)qkdec_attn_paged_workspace_size(b, hq, &kv, mp);
      }
  EXPECT_EQ(qkdec_attn_workspace_size(8, 32, nullptr), 0);
}

static void model_shapes() {
  Model q;
  size_t ws = qkdec_step_workspace_size(&q.m, 8, q.kv.data());
  EXPECT_TRUE(ws > 0);
  qkdec_step_views v{};
  EXPECT_EQ(qkdec_step_workspace_views(&q.m, 8, q.kv.data(), &v), QKDEC_OK);
  EXPECT_TRUE(v.x < ws && v.h < ws && v.qkv < ws && v.q16 < ws && v.o16 < ws && v.a < ws);
  EXPECT_TRUE(qkdec_prefill_workspace_size(&q.m, q.kv.data()) > 0);
  EXPECT_TRUE(qkdec_step_paged_workspace_size(&q.m, 8, q.kv.data(), 16) > 0);
  // dimensions at and past every limit: rejected, with no overflow on the way
  const int32_t vals[] = {std::numeric_limits<int32_t>::min(), -256, -1, 0, 1, 16, 64, 96, 128, 255, 256, 4096,
                          12288, 1 << 24, 1 << 30, std::numeric_limits<int32_t>::max()};
  for (int field = 0; field < 7; ++field)
    for (int32_t val : vals) {
      Model t;
      int32_t* f[] = {&t.m.n_layers, &t.m.hidden, &t.m.n_q_heads, &t.m.n_kv_heads, &t.m.head_dim, &t.m.ffn,
                      &t.m.vocab};
      if (field == 0 && val > 4) continue;   // the layer arrays hold 4 entries
      *f[field] = val;
      (void)qkdec_step_workspace_size(&t.m, 8, t.kv.data());
      (void)qkdec_prefill_workspace_size(&t.m, t.kv.data());
      (void)qkdec_prefill_paged_workspace_size(&t.m, t.kv.data());
      (void)qkdec_step_paged_workspace_size(&t.m, 8, t.kv.data(), 16);
      qkdec_step_views tv{};
      (void)qkdec_step_workspace_views(&t.m, 8, t.kv.data(), &tv);
    }
  // both head counts at 2^30 (their sum overflows 32 bits)
  {
    Model t;
    t.m.n_q_heads = 1 << 30;
    t.m.n_kv_heads = 1 << 30;
    EXPECT_EQ(qkdec_step_workspace_size(&t.m, 8, t.kv.data()), 0);
  }
  // cache shapes at the limits
  const int32_t kvals[] = {std::numeric_limits<int32_t>::min(), -1, 0, 1, 31, 32, 2432, 1 << 30,
                           std::numeric_limits<int32_t>::max()};
  for (int field = 0; field < 5; ++field)
    for (int32_t val : kvals) {
      Model t;
      for (auto& kv : t.kv) {
        int32_t* f[] = {&kv.type, &kv.n_kv_heads, &kv.head_dim, &kv.capacity, &kv.n_slots};
        *f[field] = val;
      }
      (void)qkdec_step_workspace_size(&t.m, 8, t.kv.data());
      (void)qkdec_step_paged_workspace_size(&t.m, 8, t.kv.data(), 64);
      (void)qkdec_attn_workspace_size(8, 32, t.kv.data());
    }
  // non-finite or negative norm / rotary constants
  {
    Model t;
    t.m.rms_eps = -1.f;
    EXPECT_EQ(qkdec_step_workspace_size(&t.m, 8, t.kv.data()), 0);
    t.m.rms_eps = std::numeric_limits<float>::quiet_NaN();
    EXPECT_EQ(qkdec_step_workspace_size(&t.m, 8, t.kv.data()), 0);
    t.m.rms_eps = 1e-6f;
    t.m.rope_base = 0.f;
    EXPECT_EQ(qkdec_step_workspace_size(&t.m, 8, t.kv.data()), 0);
  }
  EXPECT_EQ(qkdec_step_workspace_size(nullptr, 8, q.kv.data()), 0);
  EXPECT_EQ(qkdec_step_workspace_size(&q.m, 8, nullptr), 0);
  EXPECT_EQ(qkdec_step_workspace_size(&q.m, 0, q.kv.data()), 0);
  EXPECT_EQ(qkdec_step_workspace_size(&q.m, 17, q.kv.data()), 0);
}

static void rejected_calls() {
  Model q;
  const qkdec_model* m = &q.m;
  const qkdec_kv_layer* kv = q.kv.data();
  int32_t* dev_i32 = fake<int32_t>(0x40000000);
  float* dev_f32 = fake<float>(0x50000000);
  uint16_t* dev_u16 = fake<uint16_t>(0x60000000);
  void* dev_ws = fake<void>(0x70000000);
  const size_t ws = qkdec_step_workspace_size(m, 8, kv);
  // the step: null arguments, batch size, workspace size and alignment
  EXPECT_EQ(qkdec_step(nullptr, kv, dev_i32, dev_i32, dev_i32, 8, dev_f32, dev_ws, ws, nullptr), QKDEC_E_ARG);
  EXPECT_EQ(qkdec_step(m, nullptr, dev_i32, dev_i32, dev_i32, 8, dev_f32, dev_ws, ws, nullptr), QKDEC_E_ARG);
  EXPECT_EQ(qkdec_step(m, kv, nullptr, dev_i32, dev_i32, 8, dev_f32, dev_ws, ws, nullptr), QKDEC_E_ARG);
  EXPECT_EQ(qkdec_step(m, kv, dev_i32, dev_i32, dev_i32, 0, dev_f32, dev_ws, ws, nullptr), QKDEC_E_SHAPE);
  EXPECT_EQ(qkdec_step(m, kv, dev_i32, dev_i32, dev_i32, 17, dev_f32, dev_ws, ws, nullptr), QKDEC_E_SHAPE);
  EXPECT_EQ(qkdec_step(m, kv, dev_i32, dev_i32, dev_i32, 8, dev_f32, nullptr, ws, nullptr), QKDEC_E_WORKSPACE);
  EXPECT_EQ(qkdec_step(m, kv, dev_i32, dev_i32, dev_i32, 8, dev_f32, dev_ws, ws - 1, nullptr), QKDEC_E_WORKSPACE);
  EXPECT_EQ(qkdec_step(m, kv, dev_i32, dev_i32, dev_i32, 8, dev_f32, fake<void>(0x70000010), ws, nullptr),
            QKDEC_E_ALIGN);
  {
    Model t;
    t.layers[2].w_down = fake<void>(0x123457);   // misaligned weights of one layer
    EXPECT_EQ(qkdec_step(&t.m, t.kv.data(), dev_i32, dev_i32, dev_i32, 8, dev_f32, dev_ws, ws, nullptr),
              QKDEC_E_ALIGN);
    t.layers[2].w_down = nullptr;
    EXPECT_EQ(qkdec_step(&t.m, t.kv.data(), dev_i32, dev_i32, dev_i32, 8, dev_f32, dev_ws, ws, nullptr),
              QKDEC_E_ARG);
  }
  {
    Model t;
    t.kv[3].capacity = 1024;   // layers' caches of different shapes
    EXPECT_EQ(qkdec_step(&t.m, t.kv.data(), dev_i32, dev_i32, dev_i32, 8, dev_f32, dev_ws, ws, nullptr),
              QKDEC_E_SHAPE);
  }
  // paged step
  const size_t pws = qkdec_step_paged_workspace_size(m, 8, kv, 16);
  EXPECT_EQ(qkdec_step_paged(m, kv, nullptr, 16, dev_i32, dev_i32, 8, dev_f32, dev_ws, pws, nullptr), QKDEC_E_ARG);
  EXPECT_TRUE(qkdec_step_paged(m, kv, dev_i32, 0, dev_i32, dev_i32, 8, dev_f32, dev_ws, pws, nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_step_paged(m, kv, dev_i32, 16, dev_i32, dev_i32, 8, dev_f32, dev_ws, pws - 1, nullptr) !=
              QKDEC_OK);
  // prefill
  const size_t fws = qkdec_prefill_workspace_size(m, kv);
  EXPECT_EQ(qkdec_prefill(m, kv, 0, 0, nullptr, 16, nullptr, dev_i32, dev_ws, fws, nullptr), QKDEC_E_ARG);
  EXPECT_EQ(qkdec_prefill(m, kv, 0, 0, dev_i32, 0, nullptr, dev_i32, dev_ws, fws, nullptr), QKDEC_E_SHAPE);
  EXPECT_EQ(qkdec_prefill(m, kv, -1, 0, dev_i32, 16, nullptr, dev_i32, dev_ws, fws, nullptr), QKDEC_E_SHAPE);
  EXPECT_EQ(qkdec_prefill(m, kv, 8, 0, dev_i32, 16, nullptr, dev_i32, dev_ws, fws, nullptr), QKDEC_E_SHAPE);
  EXPECT_EQ(qkdec_prefill(m, kv, 0, -5, dev_i32, 16, nullptr, dev_i32, dev_ws, fws, nullptr), QKDEC_E_SHAPE);
  EXPECT_EQ(qkdec_prefill(m, kv, 0, 2430, dev_i32, 16, nullptr, dev_i32, dev_ws, fws, nullptr), QKDEC_E_CAPACITY);
  EXPECT_EQ(qkdec_prefill(m, kv, 0, std::numeric_limits<int32_t>::max(), dev_i32, std::numeric_limits<int32_t>::max(),
                          nullptr, dev_i32, dev_ws, fws, nullptr),
            QKDEC_E_CAPACITY);
  EXPECT_EQ(qkdec_prefill(m, kv, 0, 0, dev_i32, 16, nullptr, dev_i32, dev_ws, fws - 1, nullptr), QKDEC_E_WORKSPACE);
  // prefill into a paged pool (this cache's 2432-token slots are not a page size)
  EXPECT_EQ(qkdec_prefill_paged(m, kv, nullptr, 16, 0, dev_i32, 16, nullptr, dev_i32, dev_ws, fws, nullptr),
            QKDEC_E_ARG);
  EXPECT_EQ(qkdec_prefill_paged(m, kv, dev_i32, 16, 0, dev_i32, 16, nullptr, dev_i32, dev_ws, fws, nullptr),
            QKDEC_E_SHAPE);
  EXPECT_EQ(qkdec_prefill_paged(m, kv, dev_i32, std::numeric_limits<int32_t>::max(), 0, dev_i32, 16, nullptr,
                                dev_i32, dev_ws, fws, nullptr),
            QKDEC_E_SHAPE);
  // the step on the library's fixed scratch
  EXPECT_EQ(qkdec_step_noalloc(m, kv, dev_i32, dev_i32, dev_i32, 8, dev_f32, nullptr, nullptr), QKDEC_E_ARG);
  EXPECT_EQ(qkdec_step_noalloc(m, kv, dev_i32, dev_i32, dev_i32, 17, dev_f32, dev_i32, nullptr), QKDEC_E_SHAPE);
  {
    Model t;
    for (auto& c : t.kv) c.capacity = 1 << 20;   // a workspace past the fixed scratch
    EXPECT_EQ(qkdec_step_noalloc(&t.m, t.kv.data(), dev_i32, dev_i32, dev_i32, 16, dev_f32, dev_i32, nullptr),
              QKDEC_E_WORKSPACE);
  }
  EXPECT_EQ(qkdec_step_status(nullptr, nullptr), QKDEC_E_ARG);
  EXPECT_EQ(qkdec_workspace_init(nullptr, 256, nullptr), QKDEC_E_ARG);
  EXPECT_EQ(qkdec_workspace_init(dev_ws, 0, nullptr), QKDEC_E_ARG);
  EXPECT_EQ(qkdec_workspace_init(fake<void>(0x70000001), 256, nullptr), QKDEC_E_ALIGN);
  // graph plans
  EXPECT_EQ(qkdec_plan_create(nullptr, m, kv, dev_i32, dev_i32, dev_i32, 8, dev_f32, dev_ws, ws, nullptr),
            QKDEC_E_ARG);
  qkdec_plan* plan = nullptr;
  EXPECT_TRUE(qkdec_plan_create(&plan, m, kv, dev_i32, dev_i32, dev_i32, 0, dev_f32, dev_ws, ws, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(plan == nullptr);
  EXPECT_EQ(qkdec_plan_launch(nullptr, nullptr), QKDEC_E_ARG);
  qkdec_plan_destroy(nullptr);
  // GEMM entry points
  const void* W = fake<void>(0x80000000);
  EXPECT_EQ(qkdec_gemm_q4k(nullptr, 4096, 4096, dev_u16, 4096, 8, dev_f32, 4096, nullptr, 0, nullptr, 0, nullptr),
            QKDEC_E_ARG);
  EXPECT_TRUE(qkdec_gemm_q4k(W, 4095, 4096, dev_u16, 4096, 8, dev_f32, 4096, nullptr, 0, nullptr, 0, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k(W, 4096, 4000, dev_u16, 4096, 8, dev_f32, 4096, nullptr, 0, nullptr, 0, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k(W, 4096, 4096, dev_u16, 4096, 0, dev_f32, 4096, nullptr, 0, nullptr, 0, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k(W, 4096, 4096, dev_u16, 4096, 17, dev_f32, 4096, nullptr, 0, nullptr, 0, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k(W, 4096, 4096, dev_u16, 100, 8, dev_f32, 4096, nullptr, 0, nullptr, 0, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k(W, std::numeric_limits<int64_t>::max(), 4096, dev_u16, 4096, 8, dev_f32, 4096, nullptr,
                             0, nullptr, 0, nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k(W, 4096, std::numeric_limits<int64_t>::max() - 255, dev_u16,
                             std::numeric_limits<int64_t>::max(), 8, dev_f32, 4096, nullptr, 0, nullptr, 0,
                             nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k_engine(W, 4096, 4096, dev_u16, 4096, 4, dev_f32, 4096, nullptr, 0, QKDEC_GEMM_MATVEC,
                                    nullptr, 0, nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k_engine(W, 4096, 4096, dev_u16, 4096, 1, dev_f32, 4096, nullptr, 0, 7, nullptr, 0,
                                    nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k_xf32(nullptr, 4096, 12288, dev_f32, 12288, 8, dev_f32, 4096, nullptr, 0, nullptr, 0,
                                  nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_gemm_q4k_swiglu(W, 12288, 4096, dev_u16, 4096, 8, nullptr, 12288, nullptr, 0, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(qkdec_dequant_q4k(nullptr, 16, dev_f32, nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_dequant_q4k(W, 0, dev_f32, nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_dequant_q4k(W, -1, dev_f32, nullptr) != QKDEC_OK);
  // KV appends and attention
  EXPECT_TRUE(qkdec_kv_append(nullptr, dev_i32, dev_i32, dev_f32, dev_f32, 8, nullptr, nullptr) != QKDEC_OK);
  {
    qkdec_kv_layer bad = kv[0];
    bad.type = 9;
    EXPECT_TRUE(qkdec_kv_append(&bad, dev_i32, dev_i32, dev_f32, dev_f32, 8, nullptr, nullptr) != QKDEC_OK);
    bad = kv[0];
    bad.head_dim = 96;
    EXPECT_TRUE(qkdec_kv_append(&bad, dev_i32, dev_i32, dev_f32, dev_f32, 8, nullptr, nullptr) != QKDEC_OK);
    bad = kv[0];
    EXPECT_TRUE(qkdec_kv_append_q8_0(&bad, dev_i32, dev_i32, dev_f32, dev_f32, 8, nullptr, nullptr) != QKDEC_OK);
  }
  EXPECT_TRUE(qkdec_kv_append(kv, dev_i32, dev_i32, dev_f32, dev_f32, 0, nullptr, nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_kv_append_paged(kv, nullptr, 16, dev_i32, dev_f32, dev_f32, 8, nullptr, nullptr) != QKDEC_OK);
  const size_t aws = qkdec_attn_workspace_size(8, 32, kv);
  EXPECT_TRUE(qkdec_attn_decode(kv, dev_i32, dev_i32, 8, nullptr, 32, 0.088f, nullptr, dev_u16, dev_ws, aws,
                                nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_attn_decode(kv, dev_i32, dev_i32, 8, dev_u16, 30, 0.088f, nullptr, dev_u16, dev_ws, aws,
                                nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_attn_decode(kv, dev_i32, dev_i32, 8, dev_u16, 32, 0.088f, nullptr, dev_u16, dev_ws, aws - 1,
                                nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_attn_decode(kv, dev_i32, dev_i32, 8, dev_u16, 32, 0.088f, nullptr, nullptr, dev_ws, aws,
                                nullptr) != QKDEC_OK);
  EXPECT_TRUE(qkdec_attn_decode_paged(kv, dev_i32, 0, dev_i32, 8, dev_u16, 32, 0.088f, nullptr, dev_u16, dev_ws,
                                      aws, nullptr) != QKDEC_OK);
  // LM head
  const size_t lws = qkdec_lm_head_workspace_size(151936, 8);
  EXPECT_TRUE(qkdec_lm_head_argmax(nullptr, 151936, 4096, dev_u16, 8, nullptr, dev_i32, dev_ws, lws, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(qkdec_lm_head_argmax(dev_u16, 151936, 4096, dev_u16, 17, nullptr, dev_i32, dev_ws, lws, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(qkdec_lm_head_argmax(dev_u16, 151936, 4096, dev_u16, 8, nullptr, nullptr, dev_ws, lws, nullptr) !=
              QKDEC_OK);
  EXPECT_TRUE(qkdec_lm_head_argmax(dev_u16, 151936, 4096, dev_u16, 8, nullptr, dev_i32, dev_ws, lws - 1, nullptr) !=
              QKDEC_OK);
}

int main() {
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) == hipSuccess && n_dev > 0) {
    std::printf("skipped: a GPU is visible (these checks pass fake device addresses)\n");
    return 0;
  }
  status_strings();
  size_functions();
  model_shapes();
  rejected_calls();
  std::printf("%d checks, %d failures\n", g_checks, g_failures);
  return g_failures ? 1 : 0;
}
