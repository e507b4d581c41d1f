// Host-side checks of the C ABI (include/moe_layer.h), built together with
// the library's sources compiled for the host only (no device code) under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Nothing here runs on a
// GPU: every call either returns before it touches the device (validation,
// workspace sizes and layouts, argument checks) or meets a HIP runtime with
// no device and must report MOE_ERR_HIP cleanly.  Out-of-bounds accesses,
// signed overflow in the size arithmetic and other undefined behaviour are
// reported by the sanitizers; the checks below fail on wrong results.
//
// Exit status 0 when every check passed.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "moe_layer.h"

static int g_fail = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

static moe_layer_desc_t desc(int T, int d, int E, int K, int I, int Ks, int Is, int dtype,
                             int groups = 1, int kg = 1, int score = MOE_SCORE_SOFTMAX,
                             int norm = 0) {
  moe_layer_desc_t x{};
  x.T = T; x.d = d; x.n_routed = E; x.top_k = K; x.inner = I;
  x.n_shared = Ks; x.shared_inner = Is; x.n_groups = groups; x.topk_groups = kg;
  x.score = score; x.norm_topk = norm; x.routed_scale = 1.0f; x.dtype = dtype;
  return x;
}

// The five workloads' shapes (tiny fp32, 2B, 16B, V3, skewed batch) plus the
// FP8 16B layer.
static std::vector<moe_layer_desc_t> workloads() {
  return {desc(64, 64, 16, 4, 32, 1, 32, MOE_F32),
          desc(8192, 1280, 63, 7, 1280, 1, 1280, MOE_BF16),
          desc(16384, 2048, 64, 6, 1408, 2, 1408, MOE_BF16),
          desc(4096, 7168, 256, 8, 2048, 1, 2048, MOE_BF16, 8, 4, MOE_SCORE_SIGMOID, 1),
          desc(128, 2048, 64, 6, 1408, 2, 1408, MOE_BF16),
          desc(16384, 2048, 64, 6, 1408, 2, 1408, MOE_FP8)};
}

// Every region of a layout is 256-byte aligned, inside the workspace and
// disjoint from the others.
static void check_layout(const moe_layer_desc_t& d) {
  size_t bytes = 0;
  CHECK(moe_layer_workspace_size(&d, &bytes) == MOE_OK);
  moe_workspace_layout_t L{};
  CHECK(moe_layer_workspace_layout(&d, &L) == MOE_OK);
  CHECK((size_t)L.total_bytes == bytes);
  const int64_t TK = (int64_t)d.T * d.top_k;
  const int64_t ksi = (int64_t)d.n_shared * d.shared_inner;
  const int64_t es = d.dtype == MOE_F32 ? 4 : 2;
  const int64_t hs = d.dtype == MOE_FP8 ? 1 : es;
  struct R { int64_t off, len; };
  std::vector<R> regions = {
      {L.topk_idx_i32, TK * 4}, {L.topk_w_f32, TK * 4}, {L.counts_i32, (int64_t)d.n_routed * 4},
      {L.offsets_i32, (int64_t)(d.n_routed + 1) * 4}, {L.slot_row_i32, TK * 4},
      {L.row_src_i32, TK * 4}, {L.h_routed, TK * d.inner * hs},
      {L.h_shared, (int64_t)d.T * ksi * hs},
      {L.y, TK * d.d * (d.dtype == MOE_F32 ? 4 : 2)},
      {L.y_scale_f32, d.dtype == MOE_F32 ? 0 : TK * (d.d / 64) * 4},
      {L.s_f32, (int64_t)d.T * d.d * 4}, {L.x_q, (int64_t)d.T * d.d},
      {L.x_scale, (int64_t)d.T * (d.d / 128)},
      {L.h_routed_scale, TK * (d.inner / 128)}, {L.h_shared_scale, (int64_t)d.T * (ksi / 128)}};
  for (size_t i = 0; i < regions.size(); ++i) {
    const R& a = regions[i];
    if (a.off < 0) continue;
    CHECK(a.off % 256 == 0);
    CHECK(a.off + a.len <= L.total_bytes);
    for (size_t j = i + 1; j < regions.size(); ++j) {
      const R& b = regions[j];
      if (b.off < 0 || a.len == 0 || b.len == 0) continue;
      CHECK(a.off + a.len <= b.off || b.off + b.len <= a.off);
    }
  }
  CHECK(L.xp == -1);
  CHECK((L.s_f32 >= 0) == (d.n_shared > 0));
  CHECK((L.x_q >= 0) == (d.dtype == MOE_FP8));
  size_t bwd = 0;
  const moe_status_t st = moe_layer_backward_workspace_size(&d, &bwd);
  if (d.dtype == MOE_BF16) {
    CHECK(st == MOE_OK);
    CHECK(bwd >= bytes);
  } else {
    CHECK(st == MOE_ERR_UNSUPPORTED);
  }
}

static void check_validation() {
  for (const auto& w : workloads()) {
    CHECK(moe_layer_validate(&w) == MOE_OK);
    check_layout(w);
  }
  CHECK(moe_layer_validate(nullptr) == MOE_ERR_INVALID_ARG);
  size_t b = 0;
  moe_layer_desc_t ok = workloads()[2];
  CHECK(moe_layer_workspace_size(&ok, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_layer_workspace_layout(&ok, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_layer_workspace_size(nullptr, &b) == MOE_ERR_INVALID_ARG);
  struct Case { void (*edit)(moe_layer_desc_t&); moe_status_t want; };
  const Case cases[] = {
      {[](moe_layer_desc_t& d) { d.T = -1; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.T = 0; }, MOE_OK},
      {[](moe_layer_desc_t& d) { d.d = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.n_routed = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.n_routed = 257; d.top_k = 6; }, MOE_ERR_UNSUPPORTED},
      {[](moe_layer_desc_t& d) { d.top_k = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.top_k = 65; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.top_k = 33; }, MOE_ERR_UNSUPPORTED},
      {[](moe_layer_desc_t& d) { d.inner = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.inner = 100; }, MOE_ERR_UNSUPPORTED},
      {[](moe_layer_desc_t& d) { d.n_shared = -1; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.shared_inner = 0; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.n_shared = 0; d.shared_inner = 0; }, MOE_OK},
      {[](moe_layer_desc_t& d) { d.n_groups = 3; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.n_groups = 8; d.topk_groups = 9; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.n_groups = 64; d.topk_groups = 1; d.top_k = 2; },
       MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.n_groups = 64; d.topk_groups = 6; }, MOE_OK},
      {[](moe_layer_desc_t& d) { d.score = 2; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.norm_topk = 2; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.routed_scale = 1.0f / 0.0f; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.dtype = 7; }, MOE_ERR_INVALID_ARG},
      {[](moe_layer_desc_t& d) { d.d = 2048 + 32; }, MOE_ERR_UNSUPPORTED},
      {[](moe_layer_desc_t& d) { d.dtype = MOE_F32; d.d = 2048 + 4; }, MOE_OK},
      {[](moe_layer_desc_t& d) { d.dtype = MOE_FP8; d.d = 2048 + 64; }, MOE_ERR_UNSUPPORTED},
      {[](moe_layer_desc_t& d) { d.dtype = MOE_FP8; d.d = 8192 + 128; },
       MOE_ERR_UNSUPPORTED},
      {[](moe_layer_desc_t& d) { d.T = 1 << 30; }, MOE_ERR_UNSUPPORTED},   // rows * d >= 2^31
      {[](moe_layer_desc_t& d) { d.T = 2147483647; d.top_k = 32; }, MOE_ERR_UNSUPPORTED},
  };
  for (const Case& c : cases) {
    moe_layer_desc_t d = workloads()[2];
    c.edit(d);
    const moe_status_t st = moe_layer_validate(&d);
    if (st != c.want) std::fprintf(stderr, "validate: got %d want %d\n", st, c.want);
    CHECK(st == c.want);
    size_t bytes = 0;
    CHECK(moe_layer_workspace_size(&d, &bytes) == c.want);
    if (st == MOE_OK) check_layout(d);
  }
}

// Random valid descriptors: layouts stay consistent, sizes never overflow.
static void check_random_layouts() {
  std::mt19937_64 rng(1234);
  auto pick = [&](int lo, int hi) { return lo + (int)(rng() % (uint64_t)(hi - lo + 1)); };
  int n_ok = 0;
  for (int i = 0; i < 4000; ++i) {
    const int dtype = pick(0, 2);
    const int q = dtype == MOE_FP8 ? 128 : dtype == MOE_BF16 ? 64 : 4;
    const int E = pick(1, 256);
    int groups = 1;
    for (int g : {64, 32, 16, 8, 4, 2})
      if (E % g == 0 && pick(0, 3) == 0) { groups = g; break; }
    const int kg = pick(1, groups);
    const int K = pick(1, std::min(std::min(E, 32), kg * (E / groups)));
    moe_layer_desc_t d = desc(pick(0, 1 << pick(0, 17)), q * pick(1, dtype == MOE_FP8 ? 64 : 80),
                              E, K, q * pick(1, dtype == MOE_FP8 ? 64 : 64), pick(0, 3),
                              q * pick(1, 16), dtype, groups, kg, pick(0, 1), pick(0, 1));
    if (moe_layer_validate(&d) != MOE_OK) continue;
    ++n_ok;
    check_layout(d);
  }
  CHECK(n_ok > 1000);
}

// The entry points' argument checks: each returns before the device is used.
static void check_argument_errors() {
  moe_layer_desc_t d = workloads()[2];
  d.T = 512;
  size_t bytes = 0;
  CHECK(moe_layer_workspace_size(&d, &bytes) == MOE_OK);
  std::vector<char> fake(4096);   // distinct, never dereferenced host addresses
  const void* x = fake.data();
  void* out = fake.data() + 1024;
  const float* wg = reinterpret_cast<const float*>(fake.data() + 2048);
  moe_ffn_weights_t r{fake.data(), fake.data(), fake.data(), nullptr, nullptr, nullptr};
  moe_ffn_weights_t s = r;
  alignas(256) static char ws_probe[512];
  void* ws = ws_probe;
  CHECK(moe_layer_forward(nullptr, x, wg, nullptr, nullptr, r, s, out, nullptr, nullptr,
                          nullptr, ws, bytes, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_layer_forward(&d, x, nullptr, nullptr, nullptr, r, s, out, nullptr, nullptr,
                          nullptr, ws, bytes, nullptr) == MOE_ERR_INVALID_ARG);
  moe_ffn_weights_t r0 = r;
  r0.w2 = nullptr;
  CHECK(moe_layer_forward(&d, x, wg, nullptr, nullptr, r0, s, out, nullptr, nullptr, nullptr,
                          ws, bytes, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_layer_forward(&d, x, wg, nullptr, nullptr, r, r0, out, nullptr, nullptr, nullptr,
                          ws, bytes, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_layer_forward(&d, nullptr, wg, nullptr, nullptr, r, s, out, nullptr, nullptr,
                          nullptr, ws, bytes, nullptr) == MOE_ERR_INVALID_ARG);
  // workspace: NULL, too small, misaligned
  CHECK(moe_layer_forward(&d, x, wg, nullptr, nullptr, r, s, out, nullptr, nullptr, nullptr,
                          nullptr, bytes, nullptr) == MOE_ERR_WORKSPACE);
  CHECK(moe_layer_forward(&d, x, wg, nullptr, nullptr, r, s, out, nullptr, nullptr, nullptr,
                          ws, bytes - 1, nullptr) == MOE_ERR_WORKSPACE);
  CHECK(moe_layer_forward(&d, x, wg, nullptr, nullptr, r, s, out, nullptr, nullptr, nullptr,
                          static_cast<char*>(ws) + 16, bytes, nullptr) == MOE_ERR_WORKSPACE);
  // out overlapping x
  CHECK(moe_layer_forward(&d, x, wg, nullptr, nullptr, r, s,
                          const_cast<char*>(static_cast<const char*>(x)) + 2, nullptr, nullptr,
                          nullptr, ws, bytes, nullptr) == MOE_ERR_ALIAS);
  // FP8 layers need every scale pointer
  moe_layer_desc_t d8 = d;
  d8.dtype = MOE_FP8;
  CHECK(moe_layer_forward(&d8, x, wg, nullptr, nullptr, r, s, out, nullptr, nullptr, nullptr,
                          ws, bytes, nullptr) == MOE_ERR_INVALID_ARG);
  // traced: too few or missing events
  void* ev[8] = {};
  CHECK(moe_layer_forward_traced(&d, x, wg, nullptr, nullptr, r, s, out, nullptr, nullptr,
                                 nullptr, ws, bytes, nullptr, ev, 2) == MOE_ERR_INVALID_ARG);
  CHECK(moe_layer_forward_traced(&d, x, wg, nullptr, nullptr, r, s, out, nullptr, nullptr,
                                 nullptr, ws, bytes, nullptr, ev, 8) == MOE_ERR_INVALID_ARG);
  CHECK(moe_layer_forward_traced(&d, x, wg, nullptr, nullptr, r, s, out, nullptr, nullptr,
                                 nullptr, ws, bytes, nullptr, nullptr, 8) ==
        MOE_ERR_INVALID_ARG);
  // no tokens and nothing to write: nothing is enqueued
  moe_layer_desc_t d0 = d;
  d0.T = 0;
  CHECK(moe_layer_forward(&d0, nullptr, wg, nullptr, nullptr, r, s, nullptr, nullptr, nullptr,
                          nullptr, nullptr, 0, nullptr) == MOE_OK);
  // no-allocation forward: a layer beyond the fixed buffer is refused first
  CHECK(moe_layer_forward_noalloc(&workloads()[2], x, wg, nullptr, nullptr, r, s, out, nullptr,
                                  nullptr, nullptr, nullptr) == MOE_ERR_SCRATCH);
  CHECK(moe_layer_forward_noalloc(nullptr, x, wg, nullptr, nullptr, r, s, out, nullptr,
                                  nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  // backward
  size_t bb = 0;
  CHECK(moe_layer_backward_workspace_size(&d, &bb) == MOE_OK);
  moe_ffn_grads_t g{reinterpret_cast<float*>(fake.data()), reinterpret_cast<float*>(fake.data()),
                    reinterpret_cast<float*>(fake.data())};
  float* dwg = reinterpret_cast<float*>(fake.data() + 3072);
  void* dx = fake.data() + 512;
  CHECK(moe_layer_backward(&d8, x, wg, nullptr, nullptr, r, s, x, dx, dwg, nullptr, g, g,
                           nullptr, ws, bb, nullptr) == MOE_ERR_UNSUPPORTED);
  CHECK(moe_layer_backward(&d, x, wg, nullptr, nullptr, r, s, x, dx, nullptr, nullptr, g, g,
                           nullptr, ws, bb, nullptr) == MOE_ERR_INVALID_ARG);
  moe_ffn_grads_t g0 = g;
  g0.dw3 = nullptr;
  CHECK(moe_layer_backward(&d, x, wg, nullptr, nullptr, r, s, x, dx, dwg, nullptr, g0, g,
                           nullptr, ws, bb, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_layer_backward(&d, x, wg, nullptr, nullptr, r, s, x, dx, dwg, nullptr, g, g,
                           nullptr, ws, bb - 1, nullptr) == MOE_ERR_WORKSPACE);
  CHECK(moe_layer_backward(&d, x, wg, nullptr, nullptr, r, s, out, static_cast<char*>(out) + 4,
                           dwg, nullptr, g, g, nullptr, ws, bb, nullptr) == MOE_ERR_ALIAS);
  // quantiser and bias update
  uint8_t* codes = reinterpret_cast<uint8_t*>(fake.data());
  CHECK(moe_quantize_fp8_blocks(x, MOE_BF16, 0, 128, 128, codes, codes, nullptr) == MOE_OK);
  CHECK(moe_quantize_fp8_blocks(x, MOE_BF16, 2, 100, 128, codes, codes, nullptr) ==
        MOE_ERR_UNSUPPORTED);
  CHECK(moe_quantize_fp8_blocks(x, MOE_FP8, 2, 128, 128, codes, codes, nullptr) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_quantize_fp8_blocks(nullptr, MOE_BF16, 2, 128, 128, codes, codes, nullptr) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_quantize_fp8_blocks(x, MOE_BF16, -1, 128, 128, codes, codes, nullptr) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_quantize_fp8_blocks(x, MOE_BF16, 1ll << 40, 1 << 14, 1 << 14, codes, codes,
                                nullptr) == MOE_ERR_UNSUPPORTED);
  const int32_t* cnt = reinterpret_cast<const int32_t*>(fake.data());
  CHECK(moe_bias_update(nullptr, 64, 1e-3f, nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_bias_update(cnt, 0, 1e-3f, nullptr, nullptr, nullptr) == MOE_ERR_INVALID_ARG);
  CHECK(moe_bias_update(cnt, 257, 1e-3f, nullptr, nullptr, nullptr) == MOE_ERR_UNSUPPORTED);
  CHECK(moe_bias_update(cnt, 64, 0.0f / 0.0f, nullptr, nullptr, nullptr) ==
        MOE_ERR_INVALID_ARG);
}

static void check_names() {
  for (int st = 0; st >= -6; --st) {
    const char* m = moe_strerror(static_cast<moe_status_t>(st));
    CHECK(m && std::strlen(m) > 0 && std::strcmp(m, "unknown status") != 0);
  }
  CHECK(std::strcmp(moe_strerror(static_cast<moe_status_t>(-99)), "unknown status") == 0);
  const int n = moe_layer_trace_stage_count();
  CHECK(n == 6);
  for (int i = 0; i < n; ++i) CHECK(moe_layer_trace_stage_name(i) != nullptr);
  CHECK(moe_layer_trace_stage_name(-1) == nullptr && moe_layer_trace_stage_name(n) == nullptr);
  const int nb = moe_layer_backward_stage_count();
  CHECK(nb > 0 && moe_layer_backward_stage_name(nb) == nullptr);
  for (int i = 0; i < nb; ++i) CHECK(moe_layer_backward_stage_name(i) != nullptr);
  CHECK(moe_side_stream_count() == 0);
}

int main() {
  check_validation();
  check_random_layouts();
  check_argument_errors();
  check_names();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
