// Host side of the C ABI (include/moe_layer.h): validation, workspace
// layout, and the kernel sequence of one layer forward pass, enqueued on the
// caller's stream with no host synchronisation and no device allocation.
// Each GEMM stage of the forward is one launch over the routed experts' tiles
// and the shared experts'.  The backward runs its shared experts' branch on a
// side stream (one per host thread and device, created on first use and
// destroyed when the thread exits), forked from and joined back into the
// caller's stream.
#include "moe_layer.h"

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "common.h"

using namespace moe;

namespace {

constexpr int kStages = 6;
const char* const kStageNames[kStages] = {"router",      "scan",      "permute",
                                          "gemm_gateup", "gemm_down", "combine"};

// Stages of the backward pass (moe_layer_backward_traced).
constexpr int kBwdStages = 13;
const char* const kBwdStageNames[kBwdStages] = {
    "route",          "dh_routed",      "dh_shared",   "gateup_bwd_routed",
    "gateup_bwd_shared", "router_bwd",  "dx_routed",   "dx_shared",
    "dx_combine",     "dw2_routed",     "dw13_routed", "dw2_shared",
    "dw13_shared"};

int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Every launch is checked with hipGetLastError, which also returns an error
// left pending on the calling thread by any earlier HIP call (another
// library's failed probe, a query that returned not-ready).  Entry points that
// launch work clear that state first, so that a status reports this call's
// own work only.  A device fault is sticky and still fails the next call.
void clear_pending_error() { (void)hipGetLastError(); }

// Bytes per element of x / out (bf16 for bf16 and FP8 layers) and of the
// SwiGLU activations H (one E4M3 byte for FP8 layers).
int elem_size(const moe_layer_desc_t& d) { return d.dtype == MOE_F32 ? 4 : 2; }
int h_elem_size(const moe_layer_desc_t& d) {
  return d.dtype == MOE_FP8 ? 1 : d.dtype == MOE_BF16 ? 2 : 4;
}

// Rows per routed M-tile: large tiles when experts receive many rows, smaller
// ones when the average expert group is short (weight-streaming regime).
int choose_bm(const moe_layer_desc_t& d) {
  if (d.dtype == MOE_F32) return 64;
  const int64_t avg = (int64_t)d.T * d.top_k / d.n_routed;
  if (avg >= 192) return 256;
  if (avg >= 96) return 128;
  return 64;
}

// The backward's side stream and its fork / join events, per host thread and
// device (so concurrent host threads never share them).  Default priority,
// non-blocking with respect to the legacy default stream.  They live as long
// as the host thread: its thread-exit destructor destroys them (HIP releases
// a stream or event that still has work queued once that work completes).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, join2 = nullptr;
};

std::atomic<int32_t> g_live_side_streams{0};   // across threads (introspection)

void destroy_side(SideStream& ss) {
  if (ss.join2) (void)hipEventDestroy(ss.join2);
  if (ss.join) (void)hipEventDestroy(ss.join);
  if (ss.fork) (void)hipEventDestroy(ss.fork);
  if (ss.s) {
    (void)hipStreamDestroy(ss.s);
    g_live_side_streams.fetch_sub(1, std::memory_order_relaxed);
  }
  ss = SideStream{};
}

struct SideStreamCache {
  std::unordered_map<int, SideStream> by_device;
  ~SideStreamCache() {
    int cur = -1;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (auto& kv : by_device) {
      (void)hipSetDevice(kv.first);
      destroy_side(kv.second);
    }
    if (have_cur) (void)hipSetDevice(cur);
  }
};

// The side stream of the caller's stream's device (the null stream: the
// current device); created with that device current.  nullptr on any
// failure, and the call then runs every stage in order on `s`.
SideStream* side_stream_or_null(hipStream_t s) {
  thread_local SideStreamCache cache;
  int dev = 0;
  if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return nullptr;
  auto it = cache.by_device.find(dev);
  if (it != cache.by_device.end()) return &it->second;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  SideStream ss;
  bool ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess;
  if (ok) g_live_side_streams.fetch_add(1, std::memory_order_relaxed);
  else ss.s = nullptr;
  ok = ok && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&ss.join2, hipEventDisableTiming) == hipSuccess;
  if (!ok) destroy_side(ss);
  if (cur != dev) (void)hipSetDevice(cur);
  if (!ok) return nullptr;
  return &cache.by_device.emplace(dev, ss).first->second;
}

// The same; a failure also clears the error it left pending, since the call
// then goes on in order and checks its launches.
SideStream* side_stream(hipStream_t s) {
  SideStream* r = side_stream_or_null(s);
  if (!r) clear_pending_error();
  return r;
}

moe_status_t validate(const moe_layer_desc_t* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->d < 1 || d->n_routed < 1 || d->inner < 1) return MOE_ERR_INVALID_ARG;
  if (d->top_k < 1 || d->top_k > d->n_routed) return MOE_ERR_INVALID_ARG;
  if (d->n_shared < 0 || (d->n_shared > 0 && d->shared_inner < 1)) return MOE_ERR_INVALID_ARG;
  if (d->n_groups < 1 || d->n_routed % d->n_groups != 0) return MOE_ERR_INVALID_ARG;
  if (d->topk_groups < 1 || d->topk_groups > d->n_groups) return MOE_ERR_INVALID_ARG;
  if ((int64_t)d->topk_groups * (d->n_routed / d->n_groups) < d->top_k)
    return MOE_ERR_INVALID_ARG;
  if (d->score != MOE_SCORE_SOFTMAX && d->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (d->norm_topk != 0 && d->norm_topk != 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(d->routed_scale)) return MOE_ERR_INVALID_ARG;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16 && d->dtype != MOE_FP8)
    return MOE_ERR_INVALID_ARG;
  if (d->n_routed > MAX_EXPERTS || d->top_k > MAX_TOPK || d->n_groups > MAX_GROUPS)
    return MOE_ERR_UNSUPPORTED;
  const int q = d->dtype == MOE_FP8 ? 128 : d->dtype == MOE_BF16 ? 64 : 4;
  if (d->d % q || d->inner % q || (d->n_shared > 0 && d->shared_inner % q))
    return MOE_ERR_UNSUPPORTED;
  if (d->dtype == MOE_FP8 &&   // scale bytes of a tile are staged in LDS
      (d->d > 8192 || d->inner > 8192 || (int64_t)d->n_shared * d->shared_inner > 8192))
    return MOE_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)d->T * d->top_k;
  const int64_t lim = int64_t(1) << 31;
  if (rows * d->d >= lim || rows * d->inner >= lim ||
      (int64_t)d->T * d->n_shared * d->shared_inner >= lim)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

Layout layout_of(const moe_layer_desc_t& d) {
  Layout L;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const int64_t esz = elem_size(d);
  const int64_t TK = (int64_t)d.T * d.top_k;
  const int rt = router_tokens_per_block(d.T, d.n_routed, d.d, d.dtype != MOE_F32 ? 1 : 0);
  L.nblk = (d.T + rt - 1) / rt;
  L.bm = choose_bm(d);
  L.max_mtiles = (int32_t)((TK + (int64_t)d.n_routed * (L.bm - 1)) / L.bm);
  L.topk_idx = take(TK * 4);
  L.topk_w = take(TK * 4);
  L.rank = take(TK * 4);
  L.block_counts = take((int64_t)L.nblk * d.n_routed * 4);
  L.block_base = take((int64_t)L.nblk * d.n_routed * 4);
  L.counts = take((int64_t)d.n_routed * 4);
  L.offsets = take((int64_t)(d.n_routed + 1) * 4);
  L.tiles = take((int64_t)L.max_mtiles * (int64_t)sizeof(MTile));
  L.n_tiles = take(4);
  L.slot_row = take(TK * 4);
  L.row_src = take(TK * 4);
  L.xp = -1;   // routed gate/up tiles gather token rows from x directly
  const int64_t hsz = h_elem_size(d);
  const bool fp8 = d.dtype == MOE_FP8;
  const int64_t ksi = (int64_t)d.n_shared * d.shared_inner;
  L.h_routed = take(TK * d.inner * hsz);
  L.h_shared = d.n_shared > 0 ? take((int64_t)d.T * ksi * hsz) : -1;
  L.h_routed_scale = fp8 ? take(TK * (d.inner / 128)) : -1;
  L.h_shared_scale = (fp8 && d.n_shared > 0) ? take((int64_t)d.T * (ksi / 128)) : -1;
  L.x_q = fp8 ? take((int64_t)d.T * d.d) : -1;
  L.x_scale = fp8 ? take((int64_t)d.T * (d.d / 128)) : -1;
  // Routed expert outputs: fp32 for fp32 layers; for bf16 layers fp16 with a
  // power-of-two inverse scale per 64 columns of a row.
  const bool bf16 = d.dtype != MOE_F32;   // bf16 activations (bf16, FP8)
  L.y = take(TK * d.d * (bf16 ? 2 : 4));
  L.y_scale = bf16 ? take(TK * (d.d / Y_GROUP) * 4) : -1;
  // S = x + shared experts (fp32), written by the shared down-projection and
  // read by the combine.
  L.s = d.n_shared > 0 ? take((int64_t)d.T * d.d * 4) : -1;
  L.ds = router_dsplit(d.T, d.n_routed, d.d, bf16 ? 1 : 0);
  L.ep = (d.n_routed + 3) & ~3;
  // router: the gate's bf16 parts (fused and split paths), partial logits
  // (split and small-batch paths)
  const bool small = router_small(d.T, d.n_routed, d.d, bf16 ? 1 : 0);
  const bool fused = router_fused(d.T, d.n_routed, d.top_k, d.n_groups, bf16 ? 1 : 0);
  L.planes = (bf16 && !small) ? take((int64_t)3 * d.n_routed * d.d * 2) : -1;
  const int64_t slices = small ? router_small_slices(d.d) : L.ds;
  L.plog = fused ? -1 : take(slices * d.T * L.ep * 4);

  L.total = off;
  return L;
}

bool overlaps(const void* a, const void* b, size_t n) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + n && pb < pa + n;
}

// The token rows in E4M3, per 1 x 128 of the hidden dimension (FP8 layers).
hipError_t quant_x_rows(const moe_layer_desc_t& d, const Layout& L, char* ws, const void* x,
                        hipStream_t s) {
  QuantArgs q{};
  q.src = x; q.src_f32 = 0; q.batch = 1; q.rows = d.T; q.cols = d.d;
  q.codes = reinterpret_cast<uint8_t*>(ws + L.x_q);
  q.scales = reinterpret_cast<uint8_t*>(ws + L.x_scale);
  return launch_quant_rows(q, s);
}

// Router, per-expert scan and tile schedule, and the row maps (steps 1-3
// of the forward; the backward re-runs them to recover the same expert
// choice).  mark(i) records trace event i before step i.
// (FP8 layers: also the token rows in E4M3.)
template <class Mark>
// logits (or NULL): where the fused and small-batch routers store the logits
// before the logit bias, [T][ep] (the split router leaves them in L.plog).
moe_status_t route_dispatch(const moe_layer_desc_t& d, const Layout& L, char* ws,
                            const void* x, const float* w_gate, const float* logit_bias,
                            const float* select_bias, int32_t* idx, float* gw,
                            int32_t* expert_counts, hipStream_t s, Mark mark,
                            float* logits = nullptr) {
  auto at = [&](int64_t off) -> void* { return off < 0 ? nullptr : ws + off; };
  const bool bf16 = d.dtype != MOE_F32;
  const bool fp8 = d.dtype == MOE_FP8;
  hipError_t err;
#define MOE_CHECK(call)                      \
  do {                                       \
    err = (call);                            \
    if (err != hipSuccess) return MOE_ERR_HIP; \
  } while (0)
  // 1. router
  if (!mark(0)) return MOE_ERR_HIP;
  {
    RouterArgs r{};
    r.x = x; r.dtype = bf16 ? 1 : 0;
    r.w_gate = w_gate; r.logit_bias = logit_bias; r.select_bias = select_bias;
    r.T = d.T; r.d = d.d; r.E = d.n_routed; r.K = d.top_k; r.score = d.score;
    r.n_groups = d.n_groups; r.topk_groups = d.topk_groups; r.norm_topk = d.norm_topk;
    r.routed_scale = d.routed_scale;
    r.ds = L.ds; r.ep = L.ep;
    r.planes = static_cast<bf16_t*>(at(L.planes));
    r.plog = static_cast<float*>(at(L.plog));
    r.logits = logits;
    r.topk_idx = idx; r.topk_w = gw;
    r.rank = static_cast<int32_t*>(at(L.rank));
    r.block_counts = static_cast<int32_t*>(at(L.block_counts));
    MOE_CHECK(launch_router(r, s));
    if (fp8) MOE_CHECK(quant_x_rows(d, L, ws, x, s));
  }
  // 2. scan + tile schedule; 3. permute (small batches: in the scan's launch)
  if (!mark(1)) return MOE_ERR_HIP;
  PermuteArgs p{};
  p.T = d.T; p.K = d.top_k; p.E = d.n_routed;
  p.rt = router_tokens_per_block(d.T, d.n_routed, d.d, bf16 ? 1 : 0);
  p.nblk = L.nblk;
  p.topk_idx = idx; p.rank = static_cast<const int32_t*>(at(L.rank));
  p.block_base = static_cast<const int32_t*>(at(L.block_base));
  p.offsets = static_cast<const int32_t*>(at(L.offsets));
  p.slot_row = static_cast<int32_t*>(at(L.slot_row));
  p.row_src = static_cast<int32_t*>(at(L.row_src));
  const bool fuse = (int64_t)d.T * d.top_k <= SCAN_PERMUTE_MAX_SLOTS;
  {
    ScanArgs c{};
    c.block_counts = static_cast<const int32_t*>(at(L.block_counts));
    c.block_base = static_cast<int32_t*>(at(L.block_base));
    c.counts = static_cast<int32_t*>(at(L.counts));
    c.user_counts = expert_counts;
    c.offsets = static_cast<int32_t*>(at(L.offsets));
    c.tiles = static_cast<MTile*>(at(L.tiles));
    c.n_tiles = static_cast<int32_t*>(at(L.n_tiles));
    c.nblk = L.nblk; c.E = d.n_routed; c.bm = L.bm;
    MOE_CHECK(launch_scan(c, s, fuse ? &p : nullptr));
  }
  if (!mark(2)) return MOE_ERR_HIP;
  if (!fuse) MOE_CHECK(launch_permute(p, s));
#undef MOE_CHECK
  return MOE_OK;
}

moe_status_t forward_impl(const moe_layer_desc_t* desc, const void* x,
                          const float* w_gate, const float* logit_bias,
                          const float* select_bias, moe_ffn_weights_t routed,
                          moe_ffn_weights_t shared, void* out,
                          int32_t* topk_idx, float* topk_w,
                          int32_t* expert_counts, void* workspace,
                          size_t workspace_bytes, void* stream_ptr,
                          void* const* events) {
  clear_pending_error();
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const moe_layer_desc_t& d = *desc;
  if (!w_gate || !routed.w1 || !routed.w3 || !routed.w2) return MOE_ERR_INVALID_ARG;
  if (d.n_shared > 0 && (!shared.w1 || !shared.w3 || !shared.w2)) return MOE_ERR_INVALID_ARG;
  if (d.dtype == MOE_FP8 && (!routed.s1 || !routed.s3 || !routed.s2 ||
                             (d.n_shared > 0 && (!shared.s1 || !shared.s3 || !shared.s2))))
    return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!x || !out)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream_ptr);
  auto mark = [&](int i) -> bool {
    return !events || hipEventRecord(static_cast<hipEvent_t>(events[i]), s) == hipSuccess;
  };
  if (d.T == 0) {   // nothing to compute; every expert's count is zero
    if (!mark(0)) return MOE_ERR_HIP;
    if (expert_counts && launch_zero_counts(expert_counts, d.n_routed, s) != hipSuccess)
      return MOE_ERR_HIP;
    for (int i = 1; i <= kStages; ++i)
      if (!mark(i)) return MOE_ERR_HIP;
    return MOE_OK;
  }
  const Layout L = layout_of(d);
  if (!workspace || workspace_bytes < (size_t)L.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return MOE_ERR_WORKSPACE;
  const size_t xbytes = (size_t)d.T * d.d * elem_size(d);
  if (overlaps(x, out, xbytes)) return MOE_ERR_ALIAS;

  char* ws = static_cast<char*>(workspace);
  auto at = [&](int64_t off) -> void* { return off < 0 ? nullptr : ws + off; };
  int32_t* idx = topk_idx ? topk_idx : static_cast<int32_t*>(at(L.topk_idx));
  float* gw = topk_w ? topk_w : static_cast<float*>(at(L.topk_w));
  const bool bf16 = d.dtype != MOE_F32;   // bf16 activations (bf16, FP8)
  const bool fp8 = d.dtype == MOE_FP8;
  hipError_t err;
#define MOE_CHECK(call)                      \
  do {                                       \
    err = (call);                            \
    if (err != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

  MTile* tiles = static_cast<MTile*>(at(L.tiles));
  int32_t* n_tiles = static_cast<int32_t*>(at(L.n_tiles));
  // One launch per GEMM stage holds the routed experts' tiles and, after
  // them, the shared experts' (bf16 and FP8 layers): the shared tiles fill
  // the GPU beside the routed ones (the routed experts' tile count is only
  // known on the device).  fp32 layers launch the two groups one after the
  // other.
  auto gemm = [&](const GemmArgs& g, const GemmArgs* sh) -> hipError_t {
    if (fp8) return launch_gemm_fp8(g, s, sh);
    if (bf16) return launch_gemm_bf16(g, s, sh);
    hipError_t e = launch_gemm_f32(g, s);
    if (e == hipSuccess && sh) e = launch_gemm_f32(*sh, s);
    return e;
  };
  const int64_t ksi = (int64_t)d.n_shared * d.shared_inner;
  GemmArgs base{};
  base.d = d.d; base.tiles = tiles; base.n_tiles = n_tiles;
  base.max_mtiles = L.max_mtiles; base.T = d.T; base.bm = L.bm; base.x = x;

  st = route_dispatch(d, L, ws, x, w_gate, logit_bias, select_bias, idx, gw, expert_counts,
                      s, mark);
  if (st != MOE_OK) return st;
  // 4. gate/up: H = silu(A W1^T) * (A W3^T), routed rows gathered from x
  if (!mark(3)) return MOE_ERR_HIP;
  {
    GemmArgs g = base;
    g.mode = 0; g.shared = false; g.a = x; g.lda = d.d;
    g.a_rows = static_cast<const int32_t*>(at(L.row_src));
    g.w1 = routed.w1; g.w3 = routed.w3; g.inner = d.inner; g.n_experts = d.n_routed;
    g.out = at(L.h_routed); g.ldo = d.inner;
    GemmArgs h = base;
    h.mode = 0; h.shared = true; h.a = x; h.lda = d.d;
    h.w1 = shared.w1; h.w3 = shared.w3; h.inner = d.shared_inner; h.n_experts = d.n_shared;
    h.out = at(L.h_shared); h.ldo = (int)ksi;
    if (fp8) {
      g.a = h.a = at(L.x_q);
      g.a_scale = h.a_scale = static_cast<const uint8_t*>(at(L.x_scale));
      g.lda_s = h.lda_s = d.d / 128;
      g.s1 = routed.s1; g.s3 = routed.s3;
      g.out_scale = static_cast<uint8_t*>(at(L.h_routed_scale)); g.ldo_s = d.inner / 128;
      h.s1 = shared.s1; h.s3 = shared.s3;
      h.out_scale = static_cast<uint8_t*>(at(L.h_shared_scale)); h.ldo_s = (int)(ksi / 128);
    }
    MOE_CHECK(gemm(g, d.n_shared > 0 ? &h : nullptr));
  }
  // 5. down: Y = H W2^T of the routed rows; S = x + sum of the shared experts
  if (!mark(4)) return MOE_ERR_HIP;
  {
    GemmArgs g = base;
    g.mode = 1; g.a = at(L.h_routed); g.lda = d.inner;
    g.w2 = routed.w2; g.inner = d.inner; g.n_experts = d.n_routed;
    g.out = at(L.y); g.ldo = d.d;
    g.yscale = bf16 ? static_cast<float*>(at(L.y_scale)) : nullptr;
    GemmArgs h = base;
    h.mode = 2; h.a = at(L.h_shared); h.lda = (int)ksi;
    h.w2 = shared.w2; h.inner = d.shared_inner; h.n_experts = d.n_shared;
    h.out = at(L.s); h.ldo = d.d;
    if (fp8) {
      g.a_scale = static_cast<const uint8_t*>(at(L.h_routed_scale)); g.lda_s = d.inner / 128;
      g.s2 = routed.s2;
      h.a_scale = static_cast<const uint8_t*>(at(L.h_shared_scale)); h.lda_s = (int)(ksi / 128);
      h.s2 = shared.s2;
    }
    MOE_CHECK(gemm(g, d.n_shared > 0 ? &h : nullptr));
  }
  // 6. combine: out = RNE(base + sum_k g_k Y[slot_row[t, k]]), base = S or x
  if (!mark(5)) return MOE_ERR_HIP;
  {
    CombineArgs c{};
    c.base = d.n_shared > 0 ? at(L.s) : x;
    c.base_f32 = d.n_shared > 0;
    c.y = at(L.y);
    c.yscale = bf16 ? static_cast<const float*>(at(L.y_scale)) : nullptr;
    c.topk_w = gw; c.slot_row = static_cast<const int32_t*>(at(L.slot_row));
    c.out = out; c.dtype = bf16 ? 1 : 0; c.T = d.T; c.d = d.d; c.K = d.top_k;
    MOE_CHECK(launch_combine(c, s));
  }
  if (!mark(6)) return MOE_ERR_HIP;
#undef MOE_CHECK
  return MOE_OK;
}

// Backward workspace: the forward's regions (routing, row maps; the H
// regions hold g h for the weight gradients), then the backward's own.
struct BwdLayout {
  Layout f;
  int64_t plog, g_r, g_s, da_r, da_s, dx_rows, dx_s, row_g, dg_part, dg, dl, dlp, dwg_part, zero,
      part, total;
  int32_t n_part, gg_splits, ldp;
  int32_t splits2, splits3;   // k splits of the shared dW2 and dW1/dW3 GEMMs
};

// Split the shared experts' weight gradients (k = all T tokens) along k
// until the grid holds about two tiles per CU, keeping >= 4 k-blocks per
// split.
int32_t shared_wgrad_splits(int64_t tiles, int64_t T) {
  int64_t s = (512 + tiles - 1) / std::max<int64_t>(tiles, 1);
  s = std::min<int64_t>(s, std::max<int64_t>(T / 256, 1));
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(s, 16));
}

// k splits of the gate gradient's GEMM (dl^T x, 2 inner_p x d per split):
// about one tile per CU, keeping >= 512 tokens per split.
int32_t gate_grad_splits(int64_t d, int64_t T) {
  const int64_t tiles = (d + 255) / 256;
  int64_t s = (256 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(T / 512, 1));
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(s, 64));
}

BwdLayout bwd_layout_of(const moe_layer_desc_t& d) {
  BwdLayout B;
  B.f = layout_of(d);
  int64_t off = B.f.total;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const int64_t TK = (int64_t)d.T * d.top_k;
  const int64_t ksi = (int64_t)d.n_shared * d.shared_inner;
  B.n_part = (d.inner + 127) / 128;
  B.gg_splits = gate_grad_splits(d.d, d.T);
  B.ldp = 2 * ((d.n_routed + 3) & ~3);
  // logits left by the fused and small-batch routers (the split router's
  // partial slices stay in the forward layout's plog)
  const int rdt = d.dtype != MOE_F32 ? 1 : 0;
  const bool one_slice = router_fused(d.T, d.n_routed, d.top_k, d.n_groups, rdt) ||
                         router_small(d.T, d.n_routed, d.d, rdt);
  B.plog = one_slice ? take((int64_t)d.T * B.f.ep * 4) : -1;
  B.g_r = take(TK * d.inner * 4);
  B.g_s = d.n_shared > 0 ? take((int64_t)d.T * ksi * 4) : -1;
  B.da_r = take(TK * 2 * d.inner * 2);
  B.da_s = d.n_shared > 0 ? take((int64_t)d.T * 2 * ksi * 2) : -1;
  B.dx_rows = take(TK * d.d * 2);
  B.dx_s = d.n_shared > 0 ? take((int64_t)d.T * d.d * 2) : -1;
  B.row_g = take(TK * 4);
  B.dg_part = take(TK * B.n_part * 4);
  B.dg = take(TK * 4);
  B.dl = take((int64_t)d.T * d.n_routed * 4);
  const int64_t colsum = (int64_t)((d.T + 255) / 256) * d.n_routed;
  B.dlp = take((int64_t)d.T * B.ldp * 2);
  B.dwg_part = take(std::max<int64_t>((int64_t)B.gg_splits * B.ldp * d.d, colsum) * 4);
  B.zero = take(1024);
  B.splits2 = B.splits3 = 1;
  if (d.n_shared > 0) {
    const int64_t Is = d.shared_inner, Ks = d.n_shared;
    const int64_t t2 = Ks * ((d.d + 255) / 256) * ((Is + 255) / 256);
    const int64_t t3 = Ks * ((2 * Is + 255) / 256) * ((d.d + 255) / 256);
    B.splits2 = shared_wgrad_splits(t2, d.T);
    B.splits3 = shared_wgrad_splits(t3, d.T);
  }
  const int64_t ps = std::max<int64_t>(B.splits2 > 1 ? B.splits2 : 0,
                                       B.splits3 > 1 ? B.splits3 : 0);
  B.part = ps > 0 ? take(ps * (int64_t)d.n_shared * 2 * d.shared_inner * d.d * 4) : -1;
  B.total = off;
  return B;
}

moe_status_t backward_impl(const moe_layer_desc_t* desc, const void* x, const float* w_gate,
                           const float* logit_bias, const float* select_bias,
                           moe_ffn_weights_t routed, moe_ffn_weights_t shared,
                           const void* dout, void* dx, float* dw_gate, float* dlogit_bias,
                           moe_ffn_grads_t d_routed, moe_ffn_grads_t d_shared,
                           int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                           void* stream_ptr, void* const* events) {
  clear_pending_error();
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const moe_layer_desc_t& d = *desc;
  if (d.dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!w_gate || !routed.w1 || !routed.w3 || !routed.w2 || !dw_gate) return MOE_ERR_INVALID_ARG;
  if (!d_routed.dw1 || !d_routed.dw3 || !d_routed.dw2) return MOE_ERR_INVALID_ARG;
  if (d.n_shared > 0 && (!shared.w1 || !shared.w3 || !shared.w2 || !d_shared.dw1 ||
                         !d_shared.dw3 || !d_shared.dw2))
    return MOE_ERR_INVALID_ARG;
  if (d.T > 0 && (!x || !dout || !dx)) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream_ptr);
  auto mark = [&](int i) -> bool {
    return !events || hipEventRecord(static_cast<hipEvent_t>(events[i]), s) == hipSuccess;
  };
  const int64_t I = d.inner, Is = d.shared_inner, Ks = d.n_shared, E = d.n_routed;
  if (d.T == 0) {   // no tokens: every parameter gradient is zero
    if (!mark(0)) return MOE_ERR_HIP;
    hipError_t e = launch_fill_zero(dw_gate, E * d.d, s);
    if (e == hipSuccess && dlogit_bias) e = launch_fill_zero(dlogit_bias, E, s);
    if (e == hipSuccess) e = launch_fill_zero(d_routed.dw1, E * I * d.d, s);
    if (e == hipSuccess) e = launch_fill_zero(d_routed.dw3, E * I * d.d, s);
    if (e == hipSuccess) e = launch_fill_zero(d_routed.dw2, E * I * d.d, s);
    if (e == hipSuccess && Ks > 0) e = launch_fill_zero(d_shared.dw1, Ks * Is * d.d, s);
    if (e == hipSuccess && Ks > 0) e = launch_fill_zero(d_shared.dw3, Ks * Is * d.d, s);
    if (e == hipSuccess && Ks > 0) e = launch_fill_zero(d_shared.dw2, Ks * Is * d.d, s);
    for (int i = 1; i <= kBwdStages && e == hipSuccess; ++i)
      if (!mark(i)) return MOE_ERR_HIP;
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  const BwdLayout B = bwd_layout_of(d);
  const Layout& L = B.f;
  if (!workspace || workspace_bytes < (size_t)B.total ||
      (reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return MOE_ERR_WORKSPACE;
  const size_t xbytes = (size_t)d.T * d.d * 2;
  if (overlaps(dx, dout, xbytes) || overlaps(dx, x, xbytes)) return MOE_ERR_ALIAS;

  char* ws = static_cast<char*>(workspace);
  auto at = [&](int64_t off) -> void* { return off < 0 ? nullptr : ws + off; };
  int32_t* idx = topk_idx ? topk_idx : static_cast<int32_t*>(at(L.topk_idx));
  float* gw = static_cast<float*>(at(L.topk_w));
  if (!mark(0)) return MOE_ERR_HIP;
  auto no_mark = [](int) { return true; };
  // The routing pass leaves the logits for the router backward: the fused
  // and small-batch routers store them (one slice) in B.plog, the split
  // router's partial slices are in L.plog.
  const int rdt = d.dtype != MOE_F32 ? 1 : 0;
  const bool one_slice = router_fused(d.T, d.n_routed, d.top_k, d.n_groups, rdt) ||
                         router_small(d.T, d.n_routed, d.d, rdt);
  st = route_dispatch(d, L, ws, x, w_gate, logit_bias, select_bias, idx, gw, nullptr, s,
                      no_mark, one_slice ? static_cast<float*>(at(B.plog)) : nullptr);
  if (st != MOE_OK) return st;
  hipError_t err;
#define MOE_CHECK(call)                      \
  do {                                       \
    err = (call);                            \
    if (err != hipSuccess) return MOE_ERR_HIP; \
  } while (0)
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bf16_t* dyb = static_cast<const bf16_t*>(dout);
  const int32_t* slot_row = static_cast<const int32_t*>(at(L.slot_row));
  const int32_t* row_src = static_cast<const int32_t*>(at(L.row_src));

  BwdAuxArgs aux{};
  aux.T = d.T; aux.d = d.d; aux.E = d.n_routed; aux.K = d.top_k; aux.score = d.score;
  aux.norm_topk = d.norm_topk; aux.routed_scale = d.routed_scale;
  aux.plog = static_cast<const float*>(at(one_slice ? B.plog : L.plog));
  aux.ds = one_slice ? 1 : L.ds; aux.ep = L.ep;
  aux.logit_bias = logit_bias; aux.w_gate = w_gate;
  aux.topk_idx = idx; aux.topk_w = gw; aux.slot_row = slot_row;
  aux.dg_part = static_cast<const float*>(at(B.dg_part)); aux.n_part = B.n_part;
  aux.row_g = static_cast<float*>(at(B.row_g));
  aux.dg = static_cast<float*>(at(B.dg));
  aux.dl = static_cast<float*>(at(B.dl));
  aux.dlogit_bias = dlogit_bias;
  aux.x = xb; aux.dy = dyb;
  aux.dlp = static_cast<bf16_t*>(at(B.dlp)); aux.ldp = B.ldp;
  aux.dwg_part = static_cast<float*>(at(B.dwg_part)); aux.gg_splits = B.gg_splits;
  aux.dw_gate = dw_gate;
  aux.dx_rows = static_cast<const bf16_t*>(at(B.dx_rows));
  aux.dx_shared = static_cast<const bf16_t*>(at(B.dx_s));
  aux.dx = static_cast<bf16_t*>(dx);
  aux.zero = static_cast<bf16_t*>(at(B.zero)); aux.n_zero = 512;
  MOE_CHECK(launch_bwd_prep(aux, s));

  BwdGemmArgs rb{};
  rb.T = d.T; rb.d = d.d; rb.inner = d.inner; rb.n_experts = d.n_routed; rb.shared = false;
  rb.tiles = static_cast<const MTile*>(at(L.tiles));
  rb.n_tiles = static_cast<const int32_t*>(at(L.n_tiles)); rb.max_mtiles = L.max_mtiles;
  rb.offsets = static_cast<const int32_t*>(at(L.offsets)); rb.row_src = row_src;
  rb.dy = dyb; rb.x = xb;
  rb.splits = 1; rb.part = nullptr;
  rb.w1 = static_cast<const bf16_t*>(routed.w1);
  rb.w3 = static_cast<const bf16_t*>(routed.w3);
  rb.w2 = static_cast<const bf16_t*>(routed.w2);
  rb.da = static_cast<const bf16_t*>(at(B.da_r)); rb.ldda = 2 * d.inner;
  rb.hg = static_cast<const bf16_t*>(at(L.h_routed)); rb.ldhg = d.inner;
  rb.zero = static_cast<const bf16_t*>(at(B.zero));
  rb.dw1 = d_routed.dw1; rb.dw3 = d_routed.dw3; rb.dw2 = d_routed.dw2;
  BwdGemmArgs sb = rb;
  if (Ks > 0) {
    sb.shared = true; sb.inner = d.shared_inner; sb.n_experts = d.n_shared;
    sb.w1 = static_cast<const bf16_t*>(shared.w1);
    sb.w3 = static_cast<const bf16_t*>(shared.w3);
    sb.w2 = static_cast<const bf16_t*>(shared.w2);
    sb.da = static_cast<const bf16_t*>(at(B.da_s)); sb.ldda = (int)(2 * Ks * Is);
    sb.hg = static_cast<const bf16_t*>(at(L.h_shared)); sb.ldhg = (int)(Ks * Is);
    sb.dw1 = d_shared.dw1; sb.dw3 = d_shared.dw3; sb.dw2 = d_shared.dw2;
  }

  // The shared experts' branch: G_s = dy W2_s; gate/up recomputed with the
  // SwiGLU backward (dA_s, g h); dx_s; dW2_s and dW1/dW3_s (split k, ordered
  // reductions).  It needs no routing.  Untraced calls run it on the side
  // stream (forked here, after the zero row is written): `join` after dx_s
  // (before the dx combine), `join2` at the end.  It writes only g_s,
  // h_shared, da_s, dx_s, the split partials and the shared gradients.
  SideStream* side = (!events && Ks > 0) ? side_stream(s) : nullptr;
  auto shared_dh = [&](hipStream_t st_) {
    BwdGemmArgs g = sb;
    g.kind = 0; g.c = static_cast<float*>(at(B.g_s)); g.ldc = (int)(Ks * Is);
    return launch_gemm_bwd(g, st_);
  };
  auto shared_gateup = [&](hipStream_t st_) {
    GemmArgs g{};
    g.mode = 3; g.d = d.d; g.tiles = static_cast<const MTile*>(at(L.tiles));
    g.n_tiles = static_cast<const int32_t*>(at(L.n_tiles)); g.max_mtiles = L.max_mtiles;
    g.T = d.T; g.bm = L.bm; g.x = x;
    g.shared = true; g.a = x; g.lda = d.d; g.a_rows = nullptr;
    g.w1 = shared.w1; g.w3 = shared.w3; g.inner = d.shared_inner; g.n_experts = d.n_shared;
    g.out = at(L.h_shared); g.ldo = (int)(Ks * Is);
    g.gin = static_cast<const float*>(at(B.g_s)); g.ldgin = (int)(Ks * Is);
    g.row_g = nullptr;
    g.da = static_cast<bf16_t*>(at(B.da_s)); g.ldda = (int)(2 * Ks * Is);
    g.dg_part = nullptr; g.n_part = 0;
    return launch_gemm_bf16(g, st_);
  };
  auto shared_dx = [&](hipStream_t st_) {
    BwdGemmArgs g = sb;
    g.kind = 1; g.cx = static_cast<bf16_t*>(at(B.dx_s)); g.ldc = d.d;
    return launch_gemm_bwd(g, st_);
  };
  auto shared_dw = [&](int kind, hipStream_t st_) {
    BwdGemmArgs g = sb;
    g.part = static_cast<float*>(at(B.part));
    g.kind = kind; g.splits = kind == 2 ? B.splits2 : B.splits3;
    return launch_gemm_bwd(g, st_);
  };
  if (side) {
    MOE_CHECK(hipEventRecord(side->fork, s));
    MOE_CHECK(hipStreamWaitEvent(side->s, side->fork, 0));
    MOE_CHECK(shared_dh(side->s));
    MOE_CHECK(shared_gateup(side->s));
    MOE_CHECK(shared_dx(side->s));
    MOE_CHECK(hipEventRecord(side->join, side->s));
    MOE_CHECK(shared_dw(2, side->s));
    MOE_CHECK(shared_dw(3, side->s));
    MOE_CHECK(hipEventRecord(side->join2, side->s));
  }
  const bool in_order = Ks > 0 && !side;

  // 1. G = dy W2 of every row (before the gate weight)
  {
    if (!mark(1)) return MOE_ERR_HIP;
    BwdGemmArgs g = rb;
    g.kind = 0; g.c = static_cast<float*>(at(B.g_r)); g.ldc = d.inner;
    MOE_CHECK(launch_gemm_bwd(g, s));
    if (!mark(2)) return MOE_ERR_HIP;
    if (in_order) MOE_CHECK(shared_dh(s));
  }
  // 2. gate/up recomputed with the SwiGLU backward: dA, g h, dg row sums
  {
    if (!mark(3)) return MOE_ERR_HIP;
    GemmArgs g{};
    g.mode = 3; g.d = d.d; g.tiles = static_cast<const MTile*>(at(L.tiles));
    g.n_tiles = static_cast<const int32_t*>(at(L.n_tiles)); g.max_mtiles = L.max_mtiles;
    g.T = d.T; g.bm = L.bm; g.x = x;
    g.shared = false; g.a = x; g.lda = d.d; g.a_rows = row_src;
    g.w1 = routed.w1; g.w3 = routed.w3; g.inner = d.inner; g.n_experts = d.n_routed;
    g.out = at(L.h_routed); g.ldo = d.inner;
    g.gin = static_cast<const float*>(at(B.g_r)); g.ldgin = d.inner;
    g.row_g = static_cast<const float*>(at(B.row_g));
    g.da = static_cast<bf16_t*>(at(B.da_r)); g.ldda = 2 * d.inner;
    g.dg_part = static_cast<float*>(at(B.dg_part)); g.n_part = B.n_part;
    MOE_CHECK(launch_gemm_bf16(g, s));
    if (!mark(4)) return MOE_ERR_HIP;
    if (in_order) MOE_CHECK(shared_gateup(s));
  }
  // 3. router: scores from the routing pass's logits, dg, dl, logit-bias and
  // gate gradients
  {
    if (!mark(5)) return MOE_ERR_HIP;
    MOE_CHECK(launch_router_bwd(aux, s));
    MOE_CHECK(launch_gate_grad(aux, s));
  }
  // 4. input gradient of every row and of the shared experts, then dx
  {
    if (!mark(6)) return MOE_ERR_HIP;
    BwdGemmArgs g = rb;
    g.kind = 1; g.cx = static_cast<bf16_t*>(at(B.dx_rows)); g.ldc = d.d;
    MOE_CHECK(launch_gemm_bwd(g, s));
    if (!mark(7)) return MOE_ERR_HIP;
    if (in_order) MOE_CHECK(shared_dx(s));
    if (side) MOE_CHECK(hipStreamWaitEvent(s, side->join, 0));
    if (!mark(8)) return MOE_ERR_HIP;
    MOE_CHECK(launch_dx_combine(aux, s));
  }
  // 5. weight gradients
  {
    if (!mark(9)) return MOE_ERR_HIP;
    BwdGemmArgs g = rb;
    g.kind = 2;
    MOE_CHECK(launch_gemm_bwd(g, s));
    if (!mark(10)) return MOE_ERR_HIP;
    g.kind = 3;
    MOE_CHECK(launch_gemm_bwd(g, s));
    if (!mark(11)) return MOE_ERR_HIP;
    if (in_order) MOE_CHECK(shared_dw(2, s));
    if (!mark(12)) return MOE_ERR_HIP;
    if (in_order) MOE_CHECK(shared_dw(3, s));
    if (side) MOE_CHECK(hipStreamWaitEvent(s, side->join2, 0));
  }
  if (!mark(13)) return MOE_ERR_HIP;
#undef MOE_CHECK
  return MOE_OK;
}

// The no-allocation forward's workspace: one fixed array per device, resolved
// to a device address once per device with that device current (the array's
// name is a host-side stand-in and is never passed to a kernel).  Every call
// on a device shares it; it keeps the last call's contents.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device of stream s (null stream: the
// current device); nullptr if it cannot be resolved.
void* scratch_ptr(hipStream_t s) {
  int dev = 0;
  if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return nullptr;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev] = p;
  return p;
}

}  // namespace

extern "C" {

moe_status_t moe_layer_validate(const moe_layer_desc_t* desc) { return validate(desc); }

moe_status_t moe_layer_workspace_size(const moe_layer_desc_t* desc, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  *bytes = (size_t)layout_of(*desc).total;
  return MOE_OK;
}

moe_status_t moe_layer_workspace_layout(const moe_layer_desc_t* desc,
                                        moe_workspace_layout_t* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const Layout L = layout_of(*desc);
  out->topk_idx_i32 = L.topk_idx;
  out->topk_w_f32 = L.topk_w;
  out->counts_i32 = L.counts;
  out->offsets_i32 = L.offsets;
  out->slot_row_i32 = L.slot_row;
  out->row_src_i32 = L.row_src;
  out->xp = L.xp;
  out->h_routed = L.h_routed;
  out->h_shared = L.h_shared;
  out->y = L.y;
  out->y_scale_f32 = L.y_scale;
  out->x_q = L.x_q;
  out->x_scale = L.x_scale;
  out->h_routed_scale = L.h_routed_scale;
  out->h_shared_scale = L.h_shared_scale;
  out->s_f32 = L.s;
  out->total_bytes = L.total;
  return MOE_OK;
}

moe_status_t moe_layer_forward(const moe_layer_desc_t* desc, const void* x,
                               const float* w_gate, const float* logit_bias,
                               const float* select_bias, moe_ffn_weights_t routed,
                               moe_ffn_weights_t shared, void* out, int32_t* topk_idx,
                               float* topk_w, int32_t* expert_counts, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return forward_impl(desc, x, w_gate, logit_bias, select_bias, routed, shared, out,
                      topk_idx, topk_w, expert_counts, workspace, workspace_bytes,
                      stream, nullptr);
}

moe_status_t moe_layer_forward_noalloc(const moe_layer_desc_t* desc, const void* x,
                                       const float* w_gate, const float* logit_bias,
                                       const float* select_bias, moe_ffn_weights_t routed,
                                       moe_ffn_weights_t shared, void* out,
                                       int32_t* topk_idx, float* topk_w,
                                       int32_t* expert_counts, void* stream) {
  const moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  const int64_t need = layout_of(*desc).total;
  if (need > (int64_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  if (desc->T > 0) {
    ws = scratch_ptr(static_cast<hipStream_t>(stream));
    if (!ws) return MOE_ERR_HIP;
  }
  return forward_impl(desc, x, w_gate, logit_bias, select_bias, routed, shared, out,
                      topk_idx, topk_w, expert_counts, ws, MOE_NOALLOC_SCRATCH_BYTES, stream,
                      nullptr);
}

int32_t moe_side_stream_count(void) {
  return g_live_side_streams.load(std::memory_order_relaxed);
}

int32_t moe_layer_trace_stage_count(void) { return kStages; }

const char* moe_layer_trace_stage_name(int32_t i) {
  return (i >= 0 && i < kStages) ? kStageNames[i] : nullptr;
}

moe_status_t moe_layer_forward_traced(
    const moe_layer_desc_t* desc, const void* x, const float* w_gate,
    const float* logit_bias, const float* select_bias, moe_ffn_weights_t routed,
    moe_ffn_weights_t shared, void* out, int32_t* topk_idx, float* topk_w,
    int32_t* expert_counts, void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int32_t n_events) {
  if (!events || n_events < kStages + 1) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i <= kStages; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  return forward_impl(desc, x, w_gate, logit_bias, select_bias, routed, shared, out,
                      topk_idx, topk_w, expert_counts, workspace, workspace_bytes,
                      stream, events);
}

moe_status_t moe_layer_backward_workspace_size(const moe_layer_desc_t* desc, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe_status_t st = validate(desc);
  if (st != MOE_OK) return st;
  if (desc->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  *bytes = (size_t)bwd_layout_of(*desc).total;
  return MOE_OK;
}

moe_status_t moe_layer_backward(const moe_layer_desc_t* desc, const void* x,
                                const float* w_gate, const float* logit_bias,
                                const float* select_bias, moe_ffn_weights_t routed,
                                moe_ffn_weights_t shared, const void* dout, void* dx,
                                float* dw_gate, float* dlogit_bias, moe_ffn_grads_t d_routed,
                                moe_ffn_grads_t d_shared, int32_t* topk_idx, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return backward_impl(desc, x, w_gate, logit_bias, select_bias, routed, shared, dout, dx,
                       dw_gate, dlogit_bias, d_routed, d_shared, topk_idx, workspace,
                       workspace_bytes, stream, nullptr);
}

int32_t moe_layer_backward_stage_count(void) { return kBwdStages; }

const char* moe_layer_backward_stage_name(int32_t i) {
  return (i >= 0 && i < kBwdStages) ? kBwdStageNames[i] : nullptr;
}

moe_status_t moe_layer_backward_traced(
    const moe_layer_desc_t* desc, const void* x, const float* w_gate,
    const float* logit_bias, const float* select_bias, moe_ffn_weights_t routed,
    moe_ffn_weights_t shared, const void* dout, void* dx, float* dw_gate,
    float* dlogit_bias, moe_ffn_grads_t d_routed, moe_ffn_grads_t d_shared, int32_t* topk_idx,
    void* workspace, size_t workspace_bytes, void* stream, void* const* events,
    int32_t n_events) {
  if (!events || n_events < kBwdStages + 1) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i <= kBwdStages; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARG;
  return backward_impl(desc, x, w_gate, logit_bias, select_bias, routed, shared, dout, dx,
                       dw_gate, dlogit_bias, d_routed, d_shared, topk_idx, workspace,
                       workspace_bytes, stream, events);
}

moe_status_t moe_quantize_fp8_blocks(const void* src, int32_t src_dtype, int64_t batch,
                                     int32_t rows, int32_t cols, uint8_t* codes,
                                     uint8_t* scales, void* stream) {
  if (batch < 0 || rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (src_dtype != MOE_F32 && src_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (rows % 128 || cols % 128) return MOE_ERR_UNSUPPORTED;
  if (batch == 0 || rows == 0 || cols == 0) return MOE_OK;
  if (!src || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if ((int64_t)rows * cols >= (int64_t(1) << 40) / batch) return MOE_ERR_UNSUPPORTED;
  clear_pending_error();
  QuantArgs q{};
  q.src = src; q.src_f32 = src_dtype == MOE_F32; q.batch = batch; q.rows = rows; q.cols = cols;
  q.codes = codes; q.scales = scales;
  if (launch_quant_blocks(q, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status_t moe_bias_update(const int32_t* counts, int32_t n_routed, float gamma,
                             float* select_bias, float* rel_load, void* stream) {
  if (!counts || n_routed < 1 || !std::isfinite(gamma)) return MOE_ERR_INVALID_ARG;
  if (n_routed > MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  clear_pending_error();
  BiasUpdateArgs a{};
  a.counts = counts; a.n = n_routed; a.gamma = gamma;
  a.bias = select_bias; a.rel_load = rel_load;
  if (launch_bias_update(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

const char* moe_strerror(moe_status_t status) {
  // A C caller may pass any int: read the bits as one, since an enum value
  // outside the enumerators' range may not be loaded as the enum in C++.
  int32_t v;
  static_assert(sizeof(v) == sizeof(status), "status is an int");
  std::memcpy(&v, &status, sizeof v);
  switch (v) {
    case MOE_OK: return "success";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_UNSUPPORTED: return "layer shape not supported by this build";
    case MOE_ERR_ALIAS: return "out overlaps x";
    case MOE_ERR_HIP: return "HIP runtime or kernel launch error";
    case MOE_ERR_SCRATCH:
      return "layer needs more workspace than the no-allocation forward's fixed buffer holds";
  }
  return "unknown status";
}

}  // extern "C"
