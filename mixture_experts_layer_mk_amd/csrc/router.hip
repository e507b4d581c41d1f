// Router: fp32 gate GEMM, score (softmax or sigmoid), optional group limit,
// top-K in registers, gate weights, and the per-block expert histogram with
// each kept slot's rank inside its block (the inputs of a stable dispatch).
//
// Method: DeepSeekMoE paper abstract (mK of mN fine-grained experts kept per
// token); DeepSeek-V3 Technical Report summary, "2. Architecture" (selection
// bias, limit on the number of nodes -- here groups -- a token may use).
#include "common.h"

namespace moe {

namespace {

constexpr int RK = 32;        // d-chunk per LDS stage
constexpr int NT = 256;       // threads per workgroup

struct Cand {
  float key;
  int idx;
  float s;
};

// Total order of the top-K: larger key first, then smaller expert index.
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float k2 = __shfl_xor(c.key, off, 64);
    int i2 = __shfl_xor(c.idx, off, 64);
    float s2 = __shfl_xor(c.s, off, 64);
    if (better(k2, i2, c.key, c.idx)) { c.key = k2; c.idx = i2; c.s = s2; }
  }
  return c;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// RT tokens per workgroup; TN experts per thread (16*TN >= E).
template <typename XT, int RT, int TN>
__global__ __launch_bounds__(NT) void router_kernel(RouterArgs a) {
  constexpr int TM = RT / 16;           // tokens per thread
  constexpr int EP = 16 * TN;           // padded expert count
  constexpr int V = (EP + 63) / 64;     // experts per lane in selection
  __shared__ float xs[RK][RT + 1];
  __shared__ float ws[RK][EP + 1];
  __shared__ float lg[RT][EP + 1];
  __shared__ int sel[RT * MAX_TOPK];
  __shared__ float keybuf[4][EP];

  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int t0 = blockIdx.x * RT;
  const int d = a.d, E = a.E, K = a.K;
  const XT* x = static_cast<const XT*>(a.x);

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

  for (int d0 = 0; d0 < d; d0 += RK) {
    // x chunk -> xs[k][t] (fp32)
    for (int li = tid; li < RT * RK; li += NT) {
      int t = li / RK, k = li % RK;
      float v = 0.f;
      if (t0 + t < a.T && d0 + k < d) v = ld_f32<XT>(x + (size_t)(t0 + t) * d + d0 + k);
      xs[k][t] = v;
    }
    // gate chunk -> ws[k][e]
    for (int li = tid; li < EP * RK; li += NT) {
      int e = li / RK, k = li % RK;
      float v = 0.f;
      if (e < E && d0 + k < d) v = a.w_gate[(size_t)e * d + d0 + k];
      ws[k][e] = v;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < RK; ++k) {
      float xv[TM], wv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) xv[i] = xs[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < TN; ++j) wv[j] = ws[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int e = tx + 16 * j;
      float v = acc[i][j];
      if (a.logit_bias && e < E) v += a.logit_bias[e];
      lg[ty + 16 * i][e] = v;
    }
  __syncthreads();

  // ---- selection: one wave per token ----
  const int lane = tid % 64, wave = tid / 64;
  const int ntok = min(RT, a.T - t0);
  for (int t = wave; t < ntok; t += 4) {
    float l[V], s[V], key[V];
    bool taken[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      int e = lane + 64 * v;
      l[v] = (e < E) ? lg[t][e] : -INFINITY;
      taken[v] = false;
    }
    if (a.score == 0) {
      float m = -INFINITY;
#pragma unroll
      for (int v = 0; v < V; ++v) m = fmaxf(m, l[v]);
      m = wave_max(m);
      float z = 0.f;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        s[v] = (lane + 64 * v < E) ? expf(l[v] - m) : 0.f;
        z += s[v];
      }
      z = wave_sum(z);
#pragma unroll
      for (int v = 0; v < V; ++v) s[v] = s[v] / z;
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) s[v] = 1.f / (1.f + expf(-l[v]));
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      int e = lane + 64 * v;
      key[v] = (e < E) ? s[v] + (a.select_bias ? a.select_bias[e] : 0.f) : -INFINITY;
      if (key[v] != key[v]) key[v] = -INFINITY;   // NaN never outranks a score
    }
    if (a.n_groups > 1) {
      const int gsz = E / a.n_groups;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        int e = lane + 64 * v;
        if (e < E) keybuf[wave][e] = key[v];
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      // lane g scores group g: sum of its two highest keys
      float gscore = -INFINITY;
      if (lane < a.n_groups) {
        float b1 = -INFINITY, b2 = -INFINITY;
        for (int q = 0; q < gsz; ++q) {
          float kv = keybuf[wave][lane * gsz + q];
          if (kv > b1) { b2 = b1; b1 = kv; } else if (kv > b2) { b2 = kv; }
        }
        gscore = (gsz > 1) ? b1 + b2 : b1;
      }
      uint64_t keep = 0;
      bool gtaken = false;
      for (int r = 0; r < a.topk_groups; ++r) {
        Cand c{(lane < a.n_groups && !gtaken) ? gscore : -INFINITY,
               (lane < a.n_groups && !gtaken) ? lane : 0x7fffffff, 0.f};
        c = wave_best(c);
        keep |= (uint64_t)1 << c.idx;
        if (lane == c.idx) gtaken = true;
      }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        int e = lane + 64 * v;
        if (e < E && !((keep >> (e / gsz)) & 1)) key[v] = -INFINITY;
      }
      __builtin_amdgcn_wave_barrier();
    }
    float gsum = 0.f, my_g = 0.f;
    int my_id = 0;
    for (int k = 0; k < K; ++k) {
      Cand c{-INFINITY, 0x7fffffff, 0.f};
#pragma unroll
      for (int v = 0; v < V; ++v) {
        int e = lane + 64 * v;
        if (e < E && !taken[v] && better(key[v], e, c.key, c.idx)) {
          c.key = key[v]; c.idx = e; c.s = s[v];
        }
      }
      c = wave_best(c);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (lane + 64 * v == c.idx) taken[v] = true;
      if (lane == k) { my_g = c.s; my_id = c.idx; }
      gsum += c.s;
    }
    if (lane < K) {
      float g = my_g;
      if (a.norm_topk) g = g / gsum;
      g *= a.routed_scale;
      size_t o = (size_t)(t0 + t) * K + lane;
      a.topk_idx[o] = my_id;
      a.topk_w[o] = g;
      sel[t * K + lane] = my_id;
    }
  }
  __syncthreads();

  // ---- block histogram and in-block ranks (token order) ----
  for (int e = tid; e < E; e += NT) {
    int c = 0;
    for (int q = 0; q < ntok * K; ++q) c += (sel[q] == e);
    a.block_counts[(size_t)blockIdx.x * E + e] = c;
  }
  for (int q = tid; q < ntok * K; q += NT) {
    const int t = q / K, e = sel[q];
    int r = 0;
    for (int p = 0; p < t * K; ++p) r += (sel[p] == e);
    a.rank[(size_t)t0 * K + q] = r;
  }
}

template <typename XT, int RT>
hipError_t launch_rt(const RouterArgs& a, hipStream_t s) {
  dim3 grid((a.T + RT - 1) / RT), block(NT);
  if (a.E <= 16) hipLaunchKernelGGL((router_kernel<XT, RT, 1>), grid, block, 0, s, a);
  else if (a.E <= 64) hipLaunchKernelGGL((router_kernel<XT, RT, 4>), grid, block, 0, s, a);
  else if (a.E <= 128) hipLaunchKernelGGL((router_kernel<XT, RT, 8>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((router_kernel<XT, RT, 16>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

int router_tokens_per_block(int T) {
  // 64-token workgroups when that still gives one per compute unit (256),
  // else 16-token ones so small batches spread over more of the chip.
  return (T >= 64 * 256) ? 64 : 16;
}

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  const int rt = router_tokens_per_block(a.T);
  if (a.dtype == 1)
    return rt == 64 ? launch_rt<bf16_t, 64>(a, s) : launch_rt<bf16_t, 16>(a, s);
  return rt == 64 ? launch_rt<float, 64>(a, s) : launch_rt<float, 16>(a, s);
}

}  // namespace moe
