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
#include "gemm_common.h"

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
// Selection of one histogram block from its logits in LDS (lg, row stride
// ld): steps a-e above.  The first 8 TBK threads take the block's (at most
// TBK) tokens, eight lanes each, over at most EMAX experts; every thread of
// the workgroup reaches the barrier.  masks (per expert) start at zero;
// sbias holds the selection bias (or zeros); gsc has TBK rows.
template <int KMAX, int EMAX, int TBK>
__device__ __forceinline__ void select_block(const SelectArgs& a, const float* lg, int ld,
                                             int t0, int ntok,
                                             unsigned long long* masks,
                                             float (*gsc)[MAX_GROUPS + 1],
                                             const float* sbias) {
  const int tid = threadIdx.x;
  const int E = a.E, K = a.K;
  const bool act = tid < TBK * 8;             // whole waves: TBK * 8 is a multiple of 64
  const int j = tid & 7;                      // lane of the token's eight
  const int tl = tid >> 3;                    // token in the block
  const int t = t0 + tl;
  const bool live = tl < ntok;
  float ts[KMAX];                             // kept scores and experts, in order
  int ti[KMAX];
  if (act) {
    const float* my = lg + (live ? tl : 0) * ld;   // dead tokens shadow row 0
    constexpr int CM = EMAX / 8;                // experts per lane, at most
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
  }
  __syncthreads();

  // e. block histogram and in-block ranks (token order)
  for (int e = tid; e < E; e += (int)blockDim.x)   // layout [blocks][E]
    a.block_counts[(size_t)blockIdx.x * E + e] = __popcll(masks[e]);
  if (act && live) {
    const uint64_t below = (tl == 0) ? 0ull : (~0ull >> (64 - tl));
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (r >= K || (r & 7) != j) continue;
      a.rank[(size_t)t * K + r] = __popcll(masks[ti[r]] & below);
    }
  }
}

// TB tokens per block (64, or 16 for the small-batch path), 8 TB threads,
// at most EMAX experts (a lane holds EMAX / 8 of them in registers).
template <int KMAX, int TB, int EMAX>
__global__ __launch_bounds__(TB * 8) void select_kernel(SelectArgs a) {
  extern __shared__ float lg[];               // [TB][E + 1]: logits, then scores
  __shared__ unsigned long long masks[EMAX];
  __shared__ float gsc[TB][MAX_GROUPS + 1];
  __shared__ float sbias[EMAX];               // selection bias (0 without one)
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TB;
  const int E = a.E, K = a.K, ld = E + 1;
  const int ntok = min(TB, a.T - t0);

  const int q4 = a.ep / 4;
  const float4* p4 = reinterpret_cast<const float4*>(a.plog);
  const size_t slice4 = (size_t)a.T * q4;
  for (int e = tid; e < E; e += TB * 8) {
    sbias[e] = a.select_bias ? a.select_bias[e] : 0.f;
    masks[e] = 0ull;
  }
  for (int i = tid; i < ntok * q4; i += TB * 8) {
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
    if (a.logits)   // the logits before the bias, [T][ep]
      reinterpret_cast<float4*>(a.logits)[(size_t)(t0 + r) * q4 + c] = v;
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * c + j;
      if (e < E) lg[r * ld + e] = vv[j] + (a.logit_bias ? a.logit_bias[e] : 0.f);
    }
  }
  __syncthreads();
  select_block<KMAX, EMAX, TB>(a, lg, ld, t0, ntok, masks, gsc, sbias);
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

// Ring depths of the fused router's logits: token-row chunks (HBM) and gate
// plane chunks (L2-resident: every workgroup reads all of them).
constexpr int FR_NSX = 4, FR_NSW = 4;

template <int KT>
__global__ __launch_bounds__(256) void router_fused_kernel(RouterArgs a) {
  using gemm::u32x4;
  // LDS: token rows [NSX][64 rows][8 chunks of 16 B] (64 hidden columns per
  // chunk), gate planes [NSW][3][64 rows][8 chunks]; both XOR-swizzled by
  // chunk as in the expert GEMMs; then the 64 x 64 logits.
  // One LDS object per ring slot (eight in all: the compiler's wait
  // insertion tells apart that many direct-load destinations), selected
  // statically in an unrolled period of four chunks, so the direct loads
  // into one slot and the operand reads of another need no wait.
  __shared__ u32x4 xs0[FR_TOK * 8], xs1[FR_TOK * 8], xs2[FR_TOK * 8], xs3[FR_TOK * 8];
  __shared__ u32x4 ws0[3 * 64 * 8], ws1[3 * 64 * 8], ws2[3 * 64 * 8], ws3[3 * 64 * 8];
  __shared__ float lg[FR_TOK][65];
  __shared__ int sel[FR_TOK][FR_KMAX];
  __shared__ uint64_t masks[64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int t0 = blockIdx.x * FR_TOK;
  const int E = a.E, T = a.T;
  constexpr int K = KT;

  // a. logits, 64 tokens x 64 experts: wave w computes the 32 x 32 tile
  // (experts 32 (w & 1) .., tokens 32 (w >> 1) ..) over the whole hidden
  // dimension, l = x.hi + x.mid + x.lo on the matrix cores (bf16 x times the
  // bf16 parts of the fp32 gate: exact products, fp32 sums).  Chunks of 64
  // columns stream global -> LDS (direct loads: 8 rows of 128 B per wave
  // instruction); chunk kc + NSX - 1 of the rows and kc + NSW - 1 of the
  // planes are issued while chunk kc is multiplied.  Loads past the last
  // chunk re-read it (uniform op counts for the waits; never used).
  {
    const bf16_t* x = static_cast<const bf16_t*>(a.x);
    const size_t pn = (size_t)E * a.d;
    const int nch = a.d / 64;
    const int lr = lane >> 3;
    const int pos = lane & 7;
    // this lane's source rows: x blocks 2 wave + j (j < 2), plane blocks
    // 6 wave + j (j < 6; plane q / 8, row block q % 8)
    const bf16_t* xsrc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int blk = 2 * wave + j, row = blk * 8 + lr;
      const int cg = pos ^ gemm::swz_x(row);
      xsrc[j] = x + (size_t)min(t0 + row, T - 1) * a.d + cg * 8;
    }
    const bf16_t* wsrc[6];
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int q = 6 * wave + j, pl = q >> 3, row = (q & 7) * 8 + lr;
      const int cg = pos ^ gemm::swz_x(row);
      wsrc[j] = a.planes + pl * pn + (size_t)min(row, E - 1) * a.d + cg * 8;
    }
    auto issue_x = [&](u32x4* dst, int kc) {
      const size_t ko = (size_t)min(kc, nch - 1) * 64;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_global_load_lds((const gemm::glb_void*)(xsrc[j] + ko),
                                         (gemm::lds_void*)&dst[(2 * wave + j) * 64], 16, 0, 0);
    };
    auto issue_w = [&](u32x4* dst, int kc) {
      const size_t ko = (size_t)min(kc, nch - 1) * 64;
#pragma unroll
      for (int j = 0; j < 6; ++j)
        __builtin_amdgcn_global_load_lds((const gemm::glb_void*)(wsrc[j] + ko),
                                         (gemm::lds_void*)&dst[(6 * wave + j) * 64], 16, 0, 0);
    };
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const int er = (wave & 1) * 32 + l32;     // expert row of this lane's A fragments
    const int tr = (wave >> 1) * 32 + l32;    // token row of its B fragment
    auto mult = [&](const u32x4* xb, const u32x4* wb) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int c = 2 * kk + hi;
        const bf16x8 bx = __builtin_bit_cast(bf16x8, xb[tr * 8 + (c ^ gemm::swz_x(tr))]);
        bf16x8 w[3];
#pragma unroll
        for (int p = 0; p < 3; ++p)
          w[p] = __builtin_bit_cast(bf16x8, wb[(p * 64 + er) * 8 + (c ^ gemm::swz_x(er))]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[2], bx, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[1], bx, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w[0], bx, acc, 0, 0, 0);
      }
    };
    // one chunk: (after the first) wait for its loads and for every wave to
    // be done with the previous chunk, refill the previous chunk's slots
    // (rows NSX - 1 ahead, planes NSW - 1 ahead), multiply
    auto chunk = [&](int kc, const u32x4* xb, const u32x4* wb, u32x4* xf, u32x4* wf) {
      if (kc > 0) gemm::stage_sync<8>();
      issue_x(xf, kc + FR_NSX - 1);
      issue_w(wf, kc + FR_NSW - 1);
      mult(xb, wb);
    };
    // Chunk by chunk (rows, then planes), the order of every later refill:
    // the wait counts below count loads in issue order.
    issue_x(xs0, 0); issue_w(ws0, 0);
    issue_x(xs1, 1); issue_w(ws1, 1);
    issue_x(xs2, 2); issue_w(ws2, 2);
    // chunk 0: everything but chunks 1 and 2 (the last 16 ops) has landed
    gemm::stage_sync<16>();
    // The slots of chunk k0 + j are xs[j], ws[j].  The loop body is straight
    // line (a conditional chunk inside it made the compiler wait for every
    // outstanding load before the operand reads); the remainder follows it.
    int k0 = 0;
    for (; k0 + 4 <= nch; k0 += 4) {
      chunk(k0 + 0, xs0, ws0, xs3, ws3);
      chunk(k0 + 1, xs1, ws1, xs0, ws0);
      chunk(k0 + 2, xs2, ws2, xs1, ws1);
      chunk(k0 + 3, xs3, ws3, xs2, ws2);
    }
    if (k0 < nch) chunk(k0, xs0, ws0, xs3, ws3);
    if (k0 + 1 < nch) chunk(k0 + 1, xs1, ws1, xs0, ws0);
    if (k0 + 2 < nch) chunk(k0 + 2, xs2, ws2, xs1, ws1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the redundant tail loads
    // acc[r] = D[e][t]: e = 32 (w & 1) + 8 (r / 4) + 4 hi + r % 4, t = tr
    if (a.logits && t0 + tr < T) {   // before the bias; 4 consecutive experts per store
      float* row = a.logits + (size_t)(t0 + tr) * a.ep;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = (wave & 1) * 32 + 8 * g + 4 * hi;
        if (e < a.ep)
          *reinterpret_cast<float4*>(row + e) =
              make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = (wave & 1) * 32 + 8 * (r / 4) + 4 * hi + (r % 4);
      float v = acc[r];
      if (a.logit_bias && e < E) v += a.logit_bias[e];
      lg[tr][e] = v;
    }
  }
  __syncthreads();

  // b. selection: four lanes per token (16 tokens per wave); lane quarter q
  // scans experts 16q .. 16q + 15: softmax max and sum over the quad, a
  // local top-K in registers, then K rounds merging the four lists' heads
  // with quad permutes (no LDS traffic).  K is a compile-time constant and
  // every step selects with v_cndmask instead of branching.
  {
    const int tt = wave * 16 + (lane >> 2), q = lane & 3;
    const int t = t0 + tt;
    float l[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = q * 16 + i;
      l[i] = e < E ? lg[tt][e] : -INFINITY;
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
      const float rz = 1.f / z;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = s[i] * rz;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = q * 16 + i < E ? 1.f / (1.f + expf(-l[i])) : 0.f;
    }
    // local top-K, sorted by (key descending, index ascending).  The lane's
    // experts arrive in index order, so a new one goes below every kept one
    // of equal key: it lands at the first slot whose key is smaller.
    float tk[KT], ts[KT];
    int ti[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) { tk[j] = -INFINITY; ti[j] = 0x7fffffff; ts[j] = 0.f; }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = q * 16 + i;
      float ck = e < E ? s[i] + (a.select_bias ? a.select_bias[e] : 0.f) : -INFINITY;
      if (ck != ck) ck = -INFINITY;             // NaN never outranks a score
      const float cs = s[i];
      // bottom-up, so slot j - 1 is read before it is overwritten: slot j
      // keeps its entry, takes the new one (it lands exactly at j), or takes
      // slot j - 1's (it lands above j - 1)
#pragma unroll
      for (int j = KT - 1; j >= 0; --j) {
        const bool keep_j = tk[j] >= ck;
        const bool keep_prev = j == 0 ? true : (tk[j - 1] >= ck);
        if (j > 0) {
          const float nk = keep_j ? tk[j] : (keep_prev ? ck : tk[j - 1]);
          const float ns = keep_j ? ts[j] : (keep_prev ? cs : ts[j - 1]);
          const int ni = keep_j ? ti[j] : (keep_prev ? e : ti[j - 1]);
          tk[j] = nk; ts[j] = ns; ti[j] = ni;
        } else {
          tk[0] = keep_j ? tk[0] : ck;
          ts[0] = keep_j ? ts[0] : cs;
          ti[0] = keep_j ? ti[0] : e;
        }
      }
    }
    // merge: round j takes the best head of the quad's four lists
    float gsum = 0.f, os[KT];
    int oi[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float bk = tk[0], bs = ts[0];
      int bi = ti[0];
      {
        const float ok = quad_xor1(bk), os1 = quad_xor1(bs);
        const int oi1 = quad_xor1i(bi);
        const bool c = better(ok, oi1, bk, bi);
        bk = c ? ok : bk; bi = c ? oi1 : bi; bs = c ? os1 : bs;
      }
      {
        const float ok = quad_xor2(bk), os2 = quad_xor2(bs);
        const int oi2 = quad_xor2i(bi);
        const bool c = better(ok, oi2, bk, bi);
        bk = c ? ok : bk; bi = c ? oi2 : bi; bs = c ? os2 : bs;
      }
      oi[j] = bi; os[j] = bs;
      gsum += bs;
      const bool taken = ti[0] == bi;             // this lane's head was taken
#pragma unroll
      for (int u = 0; u < KT; ++u) {
        const float nk = u + 1 < KT ? tk[u + 1] : -INFINITY;
        const float ns = u + 1 < KT ? ts[u + 1] : 0.f;
        const int ni = u + 1 < KT ? ti[u + 1] : 0x7fffffff;
        tk[u] = taken ? nk : tk[u]; ts[u] = taken ? ns : ts[u]; ti[u] = taken ? ni : ti[u];
      }
    }
    if (q == 0 && t < T) {
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        float g = os[j];
        if (a.norm_topk) g = g / gsum;
        g *= a.routed_scale;
        a.topk_idx[(size_t)t * KT + j] = oi[j];
        a.topk_w[(size_t)t * KT + j] = g;
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
  if (tid < E) a.block_counts[(size_t)blockIdx.x * E + tid] = __popcll(masks[tid]);   // [blocks][E]
  if (wave == 0 && live) {
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j = 0; j < K; ++j)
      a.rank[(size_t)t * K + j] = __popcll(masks[sel[lane][j]] & below);
  }

}

// ---------------------------------------------------------------------------
// 5. small batches: logits over many workgroups, then the selection of 3
//    on 16-token blocks (bf16 x, at most 64 experts)
// ---------------------------------------------------------------------------
// Below a thousand tokens the router is latency-bound, and a workgroup that
// reads the whole gate for its tokens is bound by its CU's load path.  Here
// the hidden dimension is split over DS workgroups per 16-token histogram
// block (grid = blocks x DS): workgroup (b, s) computes the block's logits
// over the s-th slice, l = x.hi + x.mid + x.lo as in 2a with the fp32 gate
// split into its bf16 parts in registers, one quarter of the slice per wave,
// with every load of a wave in flight at once, and stores the slice's
// partial logits (its four waves added in order) as the split path's plog.
// select_kernel<K, 16, 64> then adds the slices in order and selects.  (A single
// kernel in which the last workgroup of a block went on to select, after a
// ticket between release and acquire fences, spent 15 us of 28 in the
// fences and the hand-off.)
constexpr int SR_TOK = 16;     // tokens per histogram block
constexpr int SR_WAVES = 4;    // waves per workgroup

__global__ __launch_bounds__(SR_WAVES * 64) void logits_small_kernel(RouterArgs r) {
  using gemm::u32x4;
  __shared__ float part[SR_WAVES][SR_TOK][65];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int slice = blockIdx.y, DS = gridDim.y;
  const int t0 = blockIdx.x * SR_TOK;
  const int E = r.E, d = r.d, T = r.T;
  const int ntok = min(SR_TOK, T - t0);

  // partial logits of the wave's quarter of the slice, 32 experts x 32
  // token columns per matrix op (columns past the block's tokens repeat its
  // last token and are dropped)
  const int kspan = d / (DS * SR_WAVES);     // a multiple of 16
  const int k0 = (slice * SR_WAVES + wave) * kspan;
  const bf16_t* xp =
      static_cast<const bf16_t*>(r.x) + (size_t)(t0 + min(l32, ntok - 1)) * d + k0 + 8 * hi;
  const int n_eb = (E + 31) / 32;            // expert blocks: 1 or 2
  const float* wp[2];
#pragma unroll
  for (int eb = 0; eb < 2; ++eb)
    wp[eb] = r.w_gate + (size_t)min(eb * 32 + l32, E - 1) * d + k0 + 8 * hi;
  f32x16 acc[2];
#pragma unroll
  for (int eb = 0; eb < 2; ++eb)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[eb][q] = 0.f;
  // split 8 fp32 gate weights into hi, mid, lo bf16 parts (as in 1)
  auto split8 = [](float4 a, float4 b, bf16x8& ph, bf16x8& pm, bf16x8& pl) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t hh[2], mm[2], ll[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float f = v[2 * i + q];
        const bf16_t bh = f32_to_bf16(f);
        const float r1 = f - bf16_to_f32(bh);
        const bf16_t bm = f32_to_bf16(r1);
        const float r2 = r1 - bf16_to_f32(bm);
        hh[q] = bh; mm[q] = bm; ll[q] = f32_to_bf16(r2);
      }
      h[i] = hh[0] | (hh[1] << 16); m[i] = mm[0] | (mm[1] << 16); l[i] = ll[0] | (ll[1] << 16);
    }
    ph = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
    pm = __builtin_bit_cast(bf16x8, (u32x4){m[0], m[1], m[2], m[3]});
    pl = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
  };
  constexpr int U = 4;   // k-steps of 16 whose loads are in flight together
  for (int k = 0; k < kspan; k += 16 * U) {
    bf16x8 xf[U];
    float4 wv[U][2][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = min(k + 16 * u, kspan - 16);   // past the end: re-read, unused
      xf[u] = *reinterpret_cast<const bf16x8*>(xp + kk);
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        if (eb >= n_eb) continue;
        wv[u][eb][0] = *reinterpret_cast<const float4*>(wp[eb] + kk);
        wv[u][eb][1] = *reinterpret_cast<const float4*>(wp[eb] + kk + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k + 16 * u >= kspan) continue;
#pragma unroll
      for (int eb = 0; eb < 2; ++eb) {
        if (eb >= n_eb) continue;
        bf16x8 ph, pm, pl;
        split8(wv[u][eb][0], wv[u][eb][1], ph, pm, pl);
        acc[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl, xf[u], acc[eb], 0, 0, 0);
        acc[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pm, xf[u], acc[eb], 0, 0, 0);
        acc[eb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph, xf[u], acc[eb], 0, 0, 0);
      }
    }
  }
  // acc[eb][q] = D[e][t]: e = 32 eb + 8 (q / 4) + 4 hi + q % 4, t = l32
  if (l32 < SR_TOK) {
#pragma unroll
    for (int eb = 0; eb < 2; ++eb)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int e = eb * 32 + 8 * (q / 4) + 4 * hi + (q % 4);
        if (eb < n_eb && e < E) part[wave][l32][e] = acc[eb][q];
      }
  }
  __syncthreads();
  // the slice's partial logits (its waves in order), [slice][T][ep]
  for (int i = tid; i < ntok * E; i += SR_WAVES * 64) {
    const int t = i / E, e = i % E;
    float v = part[0][t][e];
#pragma unroll
    for (int w = 1; w < SR_WAVES; ++w) v += part[w][t][e];
    r.plog[((size_t)slice * T + t0 + t) * r.ep + e] = v;
  }
}

}  // namespace

// Small batches (bf16 x, at most 64 experts, hidden dimension a multiple
// of 256): the fused 16-token kernel of 5.
bool router_small(int T, int E, int d, int dtype) {
  return dtype == 1 && T > 0 && T < 1024 && E <= 64 && d % 256 == 0;
}

// Hidden-dimension slices of the small-batch router (each wave's quarter of
// a slice a multiple of 16 columns).
int router_small_slices(int d) { return d % 512 == 0 ? 8 : 4; }

int router_tokens_per_block(int T, int E, int d, int dtype) {
  return router_small(T, E, d, dtype) ? SR_TOK : 64;
}

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

// The selection's arguments: partial logits in r.plog, ds slices.
static SelectArgs select_args(const RouterArgs& r, int ds) {
  SelectArgs sa{};
  sa.plog = r.plog; sa.ep = r.ep; sa.ds = ds;
  sa.logits = r.logits;
  sa.logit_bias = r.logit_bias; sa.select_bias = r.select_bias;
  sa.T = r.T; sa.E = r.E; sa.K = r.K; sa.score = r.score;
  sa.n_groups = r.n_groups; sa.topk_groups = r.topk_groups; sa.norm_topk = r.norm_topk;
  sa.routed_scale = r.routed_scale;
  sa.topk_idx = r.topk_idx; sa.topk_w = r.topk_w; sa.rank = r.rank;
  sa.block_counts = r.block_counts;
  return sa;
}

hipError_t launch_router(const RouterArgs& r, hipStream_t s) {
  if (router_small(r.T, r.E, r.d, r.dtype)) {
    const int nblk = (r.T + SR_TOK - 1) / SR_TOK;
    const int ds = router_small_slices(r.d);
    hipLaunchKernelGGL(logits_small_kernel, dim3(nblk, ds), dim3(SR_WAVES * 64), 0, s, r);
    SelectArgs sa = select_args(r, ds);
    const size_t lds = (size_t)SR_TOK * (r.E + 1) * sizeof(float);
    if (r.K <= 8)   // at most 64 experts on this path
      hipLaunchKernelGGL((select_kernel<8, SR_TOK, 64>), dim3(nblk), dim3(SR_TOK * 8), lds, s,
                         sa);
    else
      hipLaunchKernelGGL((select_kernel<MAX_TOPK, SR_TOK, 64>), dim3(nblk), dim3(SR_TOK * 8), lds,
                         s, sa);
    return hipGetLastError();
  }
  if (router_fused(r.T, r.E, r.K, r.n_groups, r.dtype)) {
    const int64_t n = (int64_t)r.E * r.d;
    hipLaunchKernelGGL(split_gate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       r.w_gate, r.planes, n);
    const dim3 grid((r.T + FR_TOK - 1) / FR_TOK), block(256);
    switch (r.K) {
      case 1: hipLaunchKernelGGL(router_fused_kernel<1>, grid, block, 0, s, r); break;
      case 2: hipLaunchKernelGGL(router_fused_kernel<2>, grid, block, 0, s, r); break;
      case 3: hipLaunchKernelGGL(router_fused_kernel<3>, grid, block, 0, s, r); break;
      case 4: hipLaunchKernelGGL(router_fused_kernel<4>, grid, block, 0, s, r); break;
      case 5: hipLaunchKernelGGL(router_fused_kernel<5>, grid, block, 0, s, r); break;
      case 6: hipLaunchKernelGGL(router_fused_kernel<6>, grid, block, 0, s, r); break;
      case 7: hipLaunchKernelGGL(router_fused_kernel<7>, grid, block, 0, s, r); break;
      default: hipLaunchKernelGGL(router_fused_kernel<8>, grid, block, 0, s, r); break;
    }
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
  // 3: selection (the split path's logits stay in plog: no logits output)
  SelectArgs sa = select_args(r, r.dtype == 1 ? r.ds : 1);
  sa.logits = nullptr;
  const dim3 grid((r.T + 63) / 64);
  const size_t lds = (size_t)64 * (r.E + 1) * sizeof(float);
  if (r.E <= 64) {
    if (r.K <= 8) hipLaunchKernelGGL((select_kernel<8, 64, 64>), grid, dim3(512), lds, s, sa);
    else hipLaunchKernelGGL((select_kernel<MAX_TOPK, 64, 64>), grid, dim3(512), lds, s, sa);
  } else if (r.K <= 8) {
    hipLaunchKernelGGL((select_kernel<8, 64, MAX_EXPERTS>), grid, dim3(512), lds, s, sa);
  } else {
    hipLaunchKernelGGL((select_kernel<MAX_TOPK, 64, MAX_EXPERTS>), grid, dim3(512), lds, s, sa);
  }
  return hipGetLastError();
}

}  // namespace moe
