// Router: gate logits, scores (softmax or sigmoid), optional group limit,
// top-K, gate weights, and per-block expert histograms with each kept slot's
// rank inside its block (the inputs of a stable dispatch).
//
// Method: DeepSeekMoE paper abstract (mK of mN fine-grained experts kept per
// token); DeepSeek-V3 Technical Report summary, "2. Architecture" (selection
// bias; limit on the nodes -- here expert groups -- a token may use).
//
// Three kernels:
//  1. split_gate: every fp32 gate weight w is split exactly into three bf16
//     parts, w = hi + mid + lo (each part holds the next 8 significant bits;
//     the residuals are exact in fp32).
//  2. logits (bf16 x): l = x.hi + x.mid + x.lo on the matrix cores, 32
//     experts x 32 tokens per wave.  x is bf16, so every product is exact in
//     fp32 and the fp32 accumulation makes l an fp32-accurate dot product.
//     The hidden dimension may be split over DS waves (more waves in flight);
//     the DS partial sums are added in a fixed order by the select kernel.
//     (fp32 x: a plain fp32 FMA GEMM instead.)
//  3. select: eight lanes per token, 64 tokens (= one histogram block) per
//     workgroup: scores in fp32, group limit, top-K ordered by (key
//     descending, index ascending) in K merge rounds, gate weights; per
//     expert a 64-bit mask of the block's tokens gives the block's count and
//     each slot's in-block rank.
// bf16 layers with at most 64 experts, K <= 8 and no group limit run 2 and 3
// fused in one kernel per 64-token block (4 below).
#include "common.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// 1. gate split
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void split_gate_kernel(const float* __restrict__ w,
                                                         bf16_t* __restrict__ planes,
                                                         int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float v = w[i];
  const bf16_t h = f32_to_bf16(v);
  const float r1 = v - bf16_to_f32(h);
  const bf16_t m = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(m);
  planes[i] = h;
  planes[n + i] = m;
  planes[2 * n + i] = f32_to_bf16(r2);
}

// ---------------------------------------------------------------------------
// 2a. logits on the matrix cores (bf16 x)
// ---------------------------------------------------------------------------
// One wave per (group of LG_TB token blocks, expert block, d-slice) tile; 4
// waves per workgroup, which take consecutive expert blocks of the same
// tokens (their x loads meet in the L1 cache).  Each weight fragment is read
// once per k-step and used for all LG_TB token blocks.  plog[ds][t][e] (row
// stride ep) receives the partial sum of the ds-th slice of the hidden
// dimension.
constexpr int LG_TB = 4;   // 32-token blocks per wave

__global__ __launch_bounds__(256) void logits_mfma_kernel(LogitsArgs a) {
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n_eb = (a.E + 31) / 32, n_tg = (a.T + 32 * LG_TB - 1) / (32 * LG_TB);
  if (tile >= n_eb * n_tg * a.ds) return;
  const int eb = tile % n_eb;
  const int tg = (tile / n_eb) % n_tg;
  const int ds = tile / (n_eb * n_tg);
  const int l32 = lane & 31, hi = lane >> 5;
  const int er = min(eb * 32 + l32, a.E - 1);
  const int kspan = a.d / a.ds;                      // multiple of 16
  const int k0 = ds * kspan;
  const size_t pn = (size_t)a.E * a.d;
  const bf16_t* xp[LG_TB];
#pragma unroll
  for (int b = 0; b < LG_TB; ++b) {
    const int tr = min((tg * LG_TB + b) * 32 + l32, a.T - 1);
    xp[b] = a.x + (size_t)tr * a.d + k0 + 8 * hi;
  }
  const bf16_t* wp = a.planes + (size_t)er * a.d + k0 + 8 * hi;

  f32x16 acc[LG_TB];
#pragma unroll
  for (int b = 0; b < LG_TB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
  constexpr int U = 2;   // k-steps of 16 per batch (loads of a batch in flight)
  auto step = [&](const bf16x8 (&xf)[LG_TB], bf16x8 wl, bf16x8 wm, bf16x8 wh) {
#pragma unroll
    for (int b = 0; b < LG_TB; ++b) {
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wl, xf[b], acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wm, xf[b], acc[b], 0, 0, 0);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh, xf[b], acc[b], 0, 0, 0);
    }
  };
  int k = 0;
  for (; k + 16 * U <= kspan; k += 16 * U) {
    bf16x8 xf[U][LG_TB], wh[U], wm[U], wl[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wh[u] = *reinterpret_cast<const bf16x8*>(wp + k + 16 * u);
      wm[u] = *reinterpret_cast<const bf16x8*>(wp + pn + k + 16 * u);
      wl[u] = *reinterpret_cast<const bf16x8*>(wp + 2 * pn + k + 16 * u);
#pragma unroll
      for (int b = 0; b < LG_TB; ++b)
        xf[u][b] = *reinterpret_cast<const bf16x8*>(xp[b] + k + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) step(xf[u], wl[u], wm[u], wh[u]);
  }
  for (; k < kspan; k += 16) {
    bf16x8 xf[LG_TB];
#pragma unroll
    for (int b = 0; b < LG_TB; ++b) xf[b] = *reinterpret_cast<const bf16x8*>(xp[b] + k);
    step(xf, *reinterpret_cast<const bf16x8*>(wp + 2 * pn + k),
         *reinterpret_cast<const bf16x8*>(wp + pn + k), *reinterpret_cast<const bf16x8*>(wp + k));
  }
  // acc[b][r] = D[e][t]: e = eb*32 + 8*(r/4) + 4*hi + r%4, t = token block b's row l32
#pragma unroll
  for (int b = 0; b < LG_TB; ++b) {
    const int t = (tg * LG_TB + b) * 32 + l32;
    if (t >= a.T) continue;
    float* row = a.plog + ((size_t)ds * a.T + t) * a.ep;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int e0 = eb * 32 + 8 * g + 4 * hi;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (e0 + q < a.E) row[e0 + q] = acc[b][4 * g + q];
    }
  }
}

// ---------------------------------------------------------------------------
// 2b. logits with fp32 FMA (fp32 x)
// ---------------------------------------------------------------------------
// 64 tokens x 64 experts per workgroup, 4 x 4 outputs per thread.
__global__ __launch_bounds__(256) void logits_f32_kernel(LogitsArgs a) {
  constexpr int RK = 32;
  __shared__ float xs[RK][64 + 1];
  __shared__ float ws[RK][64 + 1];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int n_eb = (a.E + 63) / 64;
  const int t0 = (blockIdx.x / n_eb) * 64, e0 = (blockIdx.x % n_eb) * 64;
  float acc[4][4] = {};
  for (int d0 = 0; d0 < a.d; d0 += RK) {
    for (int li = tid; li < 64 * RK; li += 256) {
      const int r = li / RK, k = li % RK;
      const bool kin = d0 + k < a.d;
      xs[k][r] = (kin && t0 + r < a.T) ? a.xf[(size_t)(t0 + r) * a.d + d0 + k] : 0.f;
      ws[k][r] = (kin && e0 + r < a.E) ? a.w_gate[(size_t)(e0 + r) * a.d + d0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < RK; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = fmaf(xs[k][ty + 16 * i], ws[k][tx + 16 * j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + ty + 16 * i, e = e0 + tx + 16 * j;
      if (t < a.T && e < a.E) a.plog[(size_t)t * a.ep + e] = acc[i][j];
    }
}

// ---------------------------------------------------------------------------
// 3. selection
// ---------------------------------------------------------------------------
// Total order of the top-K: larger key first, then smaller expert index.
__device__ __forceinline__ bool better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Eight waves per block of 64 tokens (one histogram block): all of them stage
// the block's logits (sum of the d-slice partials in slice order, plus the
// logit bias), then each token takes eight adjacent lanes, lane j over the
// j-th contiguous eighth of the experts:
//  a. scores in fp32, softmax (max and sum over the eight lanes) or
//     sigmoid, and the selection keys (score + selection bias), kept in the
//     lane's registers (at most 32 experts per lane);
//  b. group limit: each group's score is the sum of its two best keys (its
//     best key for groups of one expert), merged over the lanes, and the
//     topk_groups best groups are kept (ties to the lower group index);
//  c. top-K by K rounds: each lane offers its best expert still available
//     (in a kept group, not yet taken), the eight offers are merged, and the
//     round's winner (key descending, index ascending) is the next kept
//     expert -- the same total order as a sorted scan over all experts;
//  d. gate weights from the kept scores in selection order;
//  e. block histogram and in-block ranks: every kept (token, expert) ORs the
//     token's bit into the expert's 64-bit LDS mask (order-free, so
//     deterministic); counts and ranks are popcounts.
template <int KMAX>
__global__ __launch_bounds__(512) void select_kernel(SelectArgs a) {
  extern __shared__ float lg[];               // [64][E + 1]: logits, then scores
  __shared__ unsigned long long masks[MAX_EXPERTS];
  __shared__ float gsc[64][MAX_GROUPS + 1];
  __shared__ float sbias[MAX_EXPERTS];        // selection bias (0 without one)
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * 64;
  const int E = a.E, K = a.K, ld = E + 1;
  const int ntok = min(64, a.T - t0);

  const int q4 = a.ep / 4;
  const float4* p4 = reinterpret_cast<const float4*>(a.plog);
  const size_t slice4 = (size_t)a.T * q4;
  for (int e = tid; e < E; e += 512) {
    sbias[e] = a.select_bias ? a.select_bias[e] : 0.f;
    masks[e] = 0ull;
  }
  for (int i = tid; i < ntok * q4; i += 512) {
    const int r = i / q4, c = i % q4;
    const size_t o = (size_t)(t0 + r) * q4 + c;
    // all slices' loads in flight first, then the sum in slice order
    float4 w[16];
#pragma unroll
    for (int sl = 0; sl < 16; ++sl)
      if (sl < a.ds) w[sl] = p4[o + sl * slice4];
    float4 v = w[0];
#pragma unroll
    for (int sl = 1; sl < 16; ++sl)
      if (sl < a.ds) { v.x += w[sl].x; v.y += w[sl].y; v.z += w[sl].z; v.w += w[sl].w; }
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * c + j;
      if (e < E) lg[r * ld + e] = vv[j] + (a.logit_bias ? a.logit_bias[e] : 0.f);
    }
  }
  __syncthreads();

  const int j = tid & 7;                      // lane of the token's eight
  const int tl = tid >> 3;                    // token in the block
  const int t = t0 + tl;
  const bool live = tl < ntok;
  const float* my = lg + (live ? tl : 0) * ld;   // dead tokens shadow row 0
  constexpr int CM = MAX_EXPERTS / 8;         // experts per lane, at most
  const int C = (E + 7) / 8;
  const int e0 = min(E, j * C), e1 = min(E, e0 + C);
  auto xor8 = [](float v, int m) { return __shfl_xor(v, m, 8); };

  // a. scores and keys of the lane's experts, in registers
  float sv[CM], kv[CM];
#pragma unroll
  for (int i = 0; i < CM; ++i) sv[i] = (e0 + i < e1) ? my[e0 + i] : 0.f;
  if (a.score == 0) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < CM; ++i)
      if (e0 + i < e1) mx = fmaxf(mx, sv[i]);
    mx = fmaxf(mx, xor8(mx, 1));
    mx = fmaxf(mx, xor8(mx, 2));
    mx = fmaxf(mx, xor8(mx, 4));
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < CM; ++i)
      if (e0 + i < e1) {
        sv[i] = expf(sv[i] - mx);
        z += sv[i];
      }
    z += xor8(z, 1);
    z += xor8(z, 2);
    z += xor8(z, 4);
#pragma unroll
    for (int i = 0; i < CM; ++i) sv[i] = sv[i] / z;
  } else {
#pragma unroll
    for (int i = 0; i < CM; ++i) sv[i] = 1.f / (1.f + expf(-sv[i]));
  }
#pragma unroll
  for (int i = 0; i < CM; ++i) {
    const float k = sv[i] + ((e0 + i < e1) ? sbias[e0 + i] : 0.f);
    kv[i] = (k != k) ? -INFINITY : k;     // NaN never outranks a score
  }

  // b. group limit: bitmask of the kept groups, then the lane's kept experts
  uint64_t keep = ~0ull;
  int gsz = E;
  uint32_t avail = 0;                         // bit i: expert e0 + i may be kept
  if (a.n_groups > 1) {
    gsz = E / a.n_groups;
    const int g_lo = e0 / gsz, g_hi = (e1 > e0) ? (e1 - 1) / gsz : g_lo - 1;
    for (int g = 0; g < a.n_groups; ++g) {
      float b1 = -INFINITY, b2 = -INFINITY;
      if (g >= g_lo && g <= g_hi) {
        const int lo = g * gsz - e0, hi_i = (g + 1) * gsz - e0;
#pragma unroll
        for (int i = 0; i < CM; ++i) {
          if (i < lo || i >= hi_i || e0 + i >= e1) continue;
          const float k = kv[i];
          if (k > b1) { b2 = b1; b1 = k; } else if (k > b2) { b2 = k; }
        }
      }
#pragma unroll
      for (int m = 1; m < 8; m <<= 1) {   // top two of both lanes' top two
        const float c1 = xor8(b1, m), c2 = xor8(b2, m);
        const float n2 = fmaxf(fminf(b1, c1), fmaxf(b2, c2));
        b1 = fmaxf(b1, c1);
        b2 = n2;
      }
      if (j == 0) gsc[tl][g] = (gsz > 1) ? b1 + b2 : b1;
    }
    __builtin_amdgcn_wave_barrier();
    keep = 0;
    for (int r = 0; r < a.topk_groups; ++r) {
      float bk = -INFINITY;
      int bi = 0x7fffffff;
      for (int g = 0; g < a.n_groups; ++g) {
        if ((keep >> g) & 1) continue;
        const float v = gsc[tl][g];
        if (better(v, g, bk, bi)) { bk = v; bi = g; }
      }
      keep |= 1ull << bi;
    }
    for (int g = g_lo; g <= g_hi; ++g) {
      if (!((keep >> g) & 1)) continue;
      const int lo = max(0, g * gsz - e0), hi_i = min(e1 - e0, (g + 1) * gsz - e0);
      avail |= (uint32_t)((hi_i >= 32 ? ~0ull : ((1ull << hi_i) - 1)) & ~((1ull << lo) - 1));
    }
  } else {
    const int n = e1 - e0;
    avail = (n >= 32) ? ~0u : ((1u << n) - 1);
  }

  // c. top-K: K rounds of the best available expert over the eight lanes
  float ts[KMAX];
  int ti[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    ts[r] = 0.f;
    ti[r] = 0x7fffffff;
    if (r >= K) continue;
    // the lane's best: increasing index, so a tie keeps the lower index
    float bk = -INFINITY, bs = 0.f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < CM; ++i) {
      if (!((avail >> i) & 1)) continue;
      if (bi == 0x7fffffff || kv[i] > bk) { bk = kv[i]; bs = sv[i]; bi = e0 + i; }
    }
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
      const float ok = xor8(bk, m), os = xor8(bs, m);
      const int oi = __shfl_xor(bi, m, 8);
      if (better(ok, oi, bk, bi)) { bk = ok; bi = oi; bs = os; }
    }
    ts[r] = bs;
    ti[r] = bi;
    if (bi >= e0 && bi < e1) avail &= ~(1u << (bi - e0));
  }

  // d. gate weights; lane j writes the slots r = j mod 8
  float gsum = 0.f;
#pragma unroll
  for (int r = 0; r < KMAX; ++r)
    if (r < K) gsum += ts[r];
  if (live) {
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (r >= K || (r & 7) != j) continue;
      float g = ts[r];
      if (a.norm_topk) g = g / gsum;
      g *= a.routed_scale;
      a.topk_idx[(size_t)t * K + r] = ti[r];
      a.topk_w[(size_t)t * K + r] = g;
      atomicOr(&masks[ti[r]], 1ull << tl);
    }
  }
  __syncthreads();

  // e. block histogram and in-block ranks (token order)
  for (int e = tid; e < E; e += 512)   // layout [E][blocks]
    a.block_counts[(size_t)e * gridDim.x + blockIdx.x] = __popcll(masks[e]);
  if (live) {
    const uint64_t below = (tl == 0) ? 0ull : (~0ull >> (64 - tl));
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (r >= K || (r & 7) != j) continue;
      a.rank[(size_t)t * K + r] = __popcll(masks[ti[r]] & below);
    }
  }
}


// ---------------------------------------------------------------------------
// 4. fused logits + selection (bf16 x, at most 64 experts, K <= 8, no
//    group limit)
// ---------------------------------------------------------------------------
// One workgroup (4 waves) per block of 64 tokens (one histogram block):
//  a. logits: wave q takes the q-th quarter of the hidden dimension and
//     computes 64 tokens x 64 experts of it on the matrix cores (gate parts
//     lo, mid, hi as in 2a); the four quarter sums are added in order through
//     LDS, then the logit bias.
//  b. selection: four lanes per token, each over a quarter of the experts:
//     softmax (or sigmoid) with max and sum over the quad, a local top-K,
//     then K merge rounds; round j's winner (key descending, index
//     ascending) is the j-th kept expert.
//  c. block histogram and in-block ranks by ballots over the block's tokens.
constexpr int FR_TOK = 64;
constexpr int FR_KMAX = 8;   // largest K the fused path takes

// Exchange with the lane whose index differs in bit 0 / bit 1 (quad permutes).
__device__ __forceinline__ int quad_xor1i(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
}
__device__ __forceinline__ int quad_xor2i(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float quad_xor1(float v) { return __int_as_float(quad_xor1i(__float_as_int(v))); }
__device__ __forceinline__ float quad_xor2(float v) { return __int_as_float(quad_xor2i(__float_as_int(v))); }

__global__ __launch_bounds__(256) void router_fused_kernel(RouterArgs a) {
  __shared__ float red[4][FR_TOK][65];          // quarter sums, then logits in red[0]
  __shared__ int sel[FR_TOK][MAX_TOPK];
  __shared__ uint64_t masks[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int t0 = blockIdx.x * FR_TOK;
  const int E = a.E, K = a.K, T = a.T;

  // a. logits of the wave's quarter of the hidden dimension
  {
    const bf16_t* x = static_cast<const bf16_t*>(a.x);
    const int kq = a.d / 4;                      // multiple of 16
    const int k0 = wave * kq;
    const size_t pn = (size_t)E * a.d;
    const bf16_t* xp[2];
    const bf16_t* wp[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      xp[b] = x + (size_t)min(t0 + b * 32 + l32, T - 1) * a.d + k0 + 8 * hi;
      wp[b] = a.planes + (size_t)min(b * 32 + l32, E - 1) * a.d + k0 + 8 * hi;
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    constexpr int U = 2;   // k-steps of 16 per batch; two batches in flight
    int k = 0;
    auto step = [&](const bf16x8 (&xf)[2], const bf16x8 (&w)[2][3]) {
#pragma unroll
      for (int eb = 0; eb < 2; ++eb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          acc[eb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[eb][2], xf[tb], acc[eb][tb], 0, 0, 0);
          acc[eb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[eb][1], xf[tb], acc[eb][tb], 0, 0, 0);
          acc[eb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[eb][0], xf[tb], acc[eb][tb], 0, 0, 0);
        }
    };
    // software pipeline: the loads of batch i+1 are issued before the matrix
    // ops of batch i (each wave is alone on its SIMD: nothing else hides them)
    auto load_batch = [&](bf16x8 (&xf)[U][2], bf16x8 (&w)[U][2][3], int kb) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          xf[u][b] = *reinterpret_cast<const bf16x8*>(xp[b] + kb + 16 * u);
#pragma unroll
          for (int p = 0; p < 3; ++p)
            w[u][b][p] = *reinterpret_cast<const bf16x8*>(wp[b] + p * pn + kb + 16 * u);
        }
    };
    const int nb = kq / (16 * U);                // whole batches
    if (nb > 0) {
      bf16x8 xa[U][2], wa[U][2][3], xb[U][2], wb[U][2][3];
      load_batch(xa, wa, 0);
      int i = 0;
      for (; i + 2 <= nb; i += 2) {
        load_batch(xb, wb, (i + 1) * 16 * U);
#pragma unroll
        for (int u = 0; u < U; ++u) step(xa[u], wa[u]);
        if (i + 2 < nb) load_batch(xa, wa, (i + 2) * 16 * U);
#pragma unroll
        for (int u = 0; u < U; ++u) step(xb[u], wb[u]);
      }
      if (i < nb) {
#pragma unroll
        for (int u = 0; u < U; ++u) step(xa[u], wa[u]);
      }
      k = nb * 16 * U;
    }
    for (; k < kq; k += 16) {
      bf16x8 xf[2], w[2][3];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        xf[b] = *reinterpret_cast<const bf16x8*>(xp[b] + k);
#pragma unroll
        for (int p = 0; p < 3; ++p) w[b][p] = *reinterpret_cast<const bf16x8*>(wp[b] + p * pn + k);
      }
      step(xf, w);
    }
    // acc[eb][tb][r] = D[e][t]: e = eb*32 + 8*(r/4) + 4*hi + r%4, t = tb*32 + l32
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          red[wave][tb * 32 + l32][eb * 32 + 8 * (r / 4) + 4 * hi + (r % 4)] = acc[eb][tb][r];
  }
  __syncthreads();
  for (int i = tid; i < FR_TOK * 64; i += 256) {
    const int tt = i >> 6, e = i & 63;
    float v = ((red[0][tt][e] + red[1][tt][e]) + red[2][tt][e]) + red[3][tt][e];
    if (a.logit_bias && e < E) v += a.logit_bias[e];
    red[0][tt][e] = v;
  }
  __syncthreads();

  // b. selection: four lanes per token (16 tokens per wave); lane quarter q
  // scans experts 16q .. 16q + 15: softmax max and sum over the quad, a
  // local top-K in registers, then K rounds merging the four lists' heads
  // with quad permutes (no LDS traffic).
  {
    const int tt = wave * 16 + (lane >> 2), q = lane & 3;
    const int t = t0 + tt;
    float l[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = q * 16 + i;
      l[i] = e < E ? red[0][tt][e] : -INFINITY;
    }
    float s[16];
    if (a.score == 0) {
      float m = l[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) m = fmaxf(m, l[i]);
      m = fmaxf(m, quad_xor1(m));
      m = fmaxf(m, quad_xor2(m));
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = q * 16 + i < E ? expf(l[i] - m) : 0.f;
        z += s[i];
      }
      z += quad_xor1(z);
      z += quad_xor2(z);
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = s[i] / z;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = q * 16 + i < E ? 1.f / (1.f + expf(-l[i])) : 0.f;
    }
    // local top-K, sorted by (key descending, index ascending)
    float tk[FR_KMAX], ts[FR_KMAX];
    int ti[FR_KMAX];
#pragma unroll
    for (int j = 0; j < FR_KMAX; ++j) { tk[j] = -INFINITY; ti[j] = 0x7fffffff; ts[j] = 0.f; }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = q * 16 + i;
      if (e >= E) break;
      float ck = s[i] + (a.select_bias ? a.select_bias[e] : 0.f);
      if (ck != ck) ck = -INFINITY;             // NaN never outranks a score
      float cs = s[i];
      int ci = e;
#pragma unroll
      for (int j = 0; j < FR_KMAX; ++j) {
        if (j < K && better(ck, ci, tk[j], ti[j])) {   // carry the loser down
          const float k2 = tk[j], s2 = ts[j];
          const int i2 = ti[j];
          tk[j] = ck; ts[j] = cs; ti[j] = ci;
          ck = k2; cs = s2; ci = i2;
        }
      }
    }
    // merge: round j takes the best head of the quad's four lists
    float gsum = 0.f, os[FR_KMAX];
    int oi[FR_KMAX];
#pragma unroll
    for (int j = 0; j < FR_KMAX; ++j) {
      if (j >= K) break;
      float bk = tk[0], bs = ts[0];
      int bi = ti[0];
      {
        const float ok = quad_xor1(bk), os1 = quad_xor1(bs);
        const int oi1 = quad_xor1i(bi);
        if (better(ok, oi1, bk, bi)) { bk = ok; bi = oi1; bs = os1; }
      }
      {
        const float ok = quad_xor2(bk), os2 = quad_xor2(bs);
        const int oi2 = quad_xor2i(bi);
        if (better(ok, oi2, bk, bi)) { bk = ok; bi = oi2; bs = os2; }
      }
      oi[j] = bi; os[j] = bs;
      gsum += bs;
      if (ti[0] == bi) {                        // this lane's head was taken
#pragma unroll
        for (int u = 0; u + 1 < FR_KMAX; ++u) { tk[u] = tk[u + 1]; ts[u] = ts[u + 1]; ti[u] = ti[u + 1]; }
        tk[FR_KMAX - 1] = -INFINITY; ti[FR_KMAX - 1] = 0x7fffffff; ts[FR_KMAX - 1] = 0.f;
      }
    }
    if (q == 0 && t < T) {
#pragma unroll
      for (int j = 0; j < FR_KMAX; ++j) {
        if (j >= K) break;
        float g = os[j];
        if (a.norm_topk) g = g / gsum;
        g *= a.routed_scale;
        a.topk_idx[(size_t)t * K + j] = oi[j];
        a.topk_w[(size_t)t * K + j] = g;
        sel[tt][j] = oi[j];
      }
    }
  }
  __syncthreads();

  // c. block histogram and in-block ranks (token order = lane order)
  const int t = t0 + lane;
  const bool live = t < T;
  uint64_t mine = 0;
  if (live)
    for (int j = 0; j < K; ++j) mine |= 1ull << sel[lane][j];
  for (int ee = wave; ee < E; ee += 4) {
    const uint64_t m = __ballot(live && ((mine >> ee) & 1));
    if (lane == 0) masks[ee] = m;
  }
  __syncthreads();
  if (tid < E) a.block_counts[(size_t)tid * gridDim.x + blockIdx.x] = __popcll(masks[tid]);
  if (wave == 0 && live) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j = 0; j < K; ++j)
      a.rank[(size_t)t * K + j] = __popcll(masks[sel[lane][j]] & below);
  }
}

}  // namespace

int router_tokens_per_block(int) { return 64; }

// Waves of the logits kernel for one d-slice.
static int logits_tiles(int T, int E) {
  return ((T + 32 * LG_TB - 1) / (32 * LG_TB)) * ((E + 31) / 32);
}

int router_dsplit(int T, int E, int d, int dtype) {
  if (dtype != 1) return 1;
  const int tiles = logits_tiles(T, E);
  int ds = 1;
  // aim for ~1024 waves (one per SIMD); every slice a multiple of 64 columns
  while (tiles * ds * 2 <= 1024 && (d % (ds * 2 * 64)) == 0 && ds < 16) ds *= 2;
  return ds;
}

// The fused kernel takes one workgroup per 64 tokens; below 1024 tokens the
// split path (the logits over many more waves) is faster (128 tokens on the
// 16B shapes: 52 against 61 us), above it the fused one (16384: 67 against
// 75 us).
bool router_fused(int T, int E, int K, int n_groups, int dtype) {
  return dtype == 1 && T >= 1024 && E <= 64 && K <= FR_KMAX && n_groups == 1;
}

hipError_t launch_logits(const LogitsArgs& la, hipStream_t s) {
  if (la.T == 0) return hipSuccess;
  const int tiles = logits_tiles(la.T, la.E) * la.ds;
  hipLaunchKernelGGL(logits_mfma_kernel, dim3((tiles + 3) / 4), dim3(256), 0, s, la);
  return hipGetLastError();
}

hipError_t launch_router(const RouterArgs& r, hipStream_t s) {
  if (router_fused(r.T, r.E, r.K, r.n_groups, r.dtype)) {
    const int64_t n = (int64_t)r.E * r.d;
    hipLaunchKernelGGL(split_gate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       r.w_gate, r.planes, n);
    hipLaunchKernelGGL(router_fused_kernel, dim3((r.T + FR_TOK - 1) / FR_TOK), dim3(256), 0, s,
                       r);
    return hipGetLastError();
  }
  // 1 + 2: partial logits
  LogitsArgs la{};
  la.T = r.T; la.d = r.d; la.E = r.E; la.ep = r.ep; la.ds = r.ds;
  la.plog = r.plog;
  if (r.dtype == 1) {
    const int64_t n = (int64_t)r.E * r.d;
    hipLaunchKernelGGL(split_gate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       r.w_gate, r.planes, n);
    la.x = static_cast<const bf16_t*>(r.x);
    la.planes = r.planes;
    const int tiles = logits_tiles(r.T, r.E) * r.ds;
    hipLaunchKernelGGL(logits_mfma_kernel, dim3((tiles + 3) / 4), dim3(256), 0, s, la);
  } else {
    la.xf = static_cast<const float*>(r.x);
    la.w_gate = r.w_gate;
    la.ds = 1;
    const int nb = ((r.T + 63) / 64) * ((r.E + 63) / 64);
    hipLaunchKernelGGL(logits_f32_kernel, dim3(nb), dim3(256), 0, s, la);
  }
  // 3: selection
  SelectArgs sa{};
  sa.plog = r.plog; sa.ep = r.ep; sa.ds = r.dtype == 1 ? r.ds : 1;
  sa.logit_bias = r.logit_bias; sa.select_bias = r.select_bias;
  sa.T = r.T; sa.E = r.E; sa.K = r.K; sa.score = r.score;
  sa.n_groups = r.n_groups; sa.topk_groups = r.topk_groups; sa.norm_topk = r.norm_topk;
  sa.routed_scale = r.routed_scale;
  sa.topk_idx = r.topk_idx; sa.topk_w = r.topk_w; sa.rank = r.rank;
  sa.block_counts = r.block_counts;
  const dim3 grid((r.T + 63) / 64);
  const size_t lds = (size_t)64 * (r.E + 1) * sizeof(float);
  if (r.K <= 8) hipLaunchKernelGGL(select_kernel<8>, grid, dim3(512), lds, s, sa);
  else hipLaunchKernelGGL(select_kernel<MAX_TOPK>, grid, dim3(512), lds, s, sa);
  return hipGetLastError();
}

}  // namespace moe
