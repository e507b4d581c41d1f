// Backward pass of the layer: the small kernels around the grouped GEMMs.
//
// The gradient is that of the forward function with the expert choice held
// fixed (the top-K choice is piecewise constant; the selection bias is set
// by the load rule, not by gradients -- DeepSeek-V3 Technical Report
// summary, "2. Architecture").  For L = sum(dy * y):
//   gate weights g_k = c s_k (c = routed_scale) or c s_k / S (renormalised,
//   S = sum_k s_k): ds_k = c dg_k, or c (dg_k - sum_j dg_j s_j / S) / S;
//   softmax scores: dl_e = s_e (ds_e - sum_k s_k ds_k); sigmoid:
//   dl_e = ds_e s_e (1 - s_e) (ds_e = 0 off the kept experts);
//   logits l = x Wg^T + b: dWg = dl^T x, db = sum_t dl_t, dx += dl Wg.
// Every sum runs in a fixed order, so results are bitwise reproducible.
#include "common.h"

namespace moe {

namespace {

// Gate weight of every expert-contiguous row, and the zero row the GEMMs
// read past the end of an expert.
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdAuxArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tk = (int64_t)a.T * a.K;
  if (i < tk) a.row_g[a.slot_row[i]] = a.topk_w[i];
  if (blockIdx.x == 0)
    for (int z = threadIdx.x; z < a.n_zero; z += 256) a.zero[z] = (bf16_t)0;
}

// One wave per token: scores from the partial logits, dg from the GEMM row
// sums, then ds and dl.
__global__ __launch_bounds__(256) void router_bwd_kernel(BwdAuxArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  constexpr int C = MAX_EXPERTS / 64;
  float l[C], sv[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = lane + 64 * c;
    float v = -INFINITY;
    if (e < a.E) {
      v = 0.f;
      for (int q = 0; q < a.ds; ++q) v += a.plog[((size_t)q * a.T + t) * a.ep + e];
      if (a.logit_bias) v += a.logit_bias[e];
    }
    l[c] = v;
  }
  if (a.score == 0) {      // softmax
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < C; ++c) mx = fmaxf(mx, l[c]);
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float z = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      sv[c] = (lane + 64 * c < a.E) ? expf(l[c] - mx) : 0.f;
      z += sv[c];
    }
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
#pragma unroll
    for (int c = 0; c < C; ++c) sv[c] = sv[c] / z;
  } else {                 // sigmoid
#pragma unroll
    for (int c = 0; c < C; ++c) sv[c] = (lane + 64 * c < a.E) ? 1.f / (1.f + expf(-l[c])) : 0.f;
  }

  // dg of kept expert k (lane k): the row's partial sums in tile order
  const int K = a.K;
  float dgk = 0.f;
  if (lane < K) {
    const int row = a.slot_row[(size_t)t * K + lane];
    const float* p = a.dg_part + (size_t)row * a.n_part;
    for (int q = 0; q < a.n_part; ++q) dgk += p[q];
    a.dg[(size_t)t * K + lane] = dgk;
  }
  // the kept experts' scores, their sum and the weighted dg sum
  float S = 0.f, dgw = 0.f;
  for (int k = 0; k < K; ++k) {
    const int e = a.topk_idx[(size_t)t * K + k];
    float se = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float v = __shfl(sv[c], e & 63);
      if ((e >> 6) == c) se = v;
    }
    S += se;
  }
  const float cs = a.routed_scale;
  // ds at each kept expert, and u = sum_k s_k ds_k (softmax)
  if (a.norm_topk) {
    for (int k = 0; k < K; ++k) {
      const int e = a.topk_idx[(size_t)t * K + k];
      float se = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float v = __shfl(sv[c], e & 63);
        if ((e >> 6) == c) se = v;
      }
      dgw += __shfl(dgk, k) * (se / S);
    }
  }
  float ds[C];
#pragma unroll
  for (int c = 0; c < C; ++c) ds[c] = 0.f;
  float u = 0.f;
  for (int k = 0; k < K; ++k) {
    const int e = a.topk_idx[(size_t)t * K + k];
    const float g = __shfl(dgk, k);
    const float dsk = a.norm_topk ? cs * (g - dgw) / S : cs * g;
    float se = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float v = __shfl(sv[c], e & 63);
      if ((e >> 6) == c) se = v;
      if ((e >> 6) == c && (e & 63) == lane) ds[c] = dsk;
    }
    u += se * dsk;
  }
  // dl in fp32, and as its bf16 hi and lo parts for the gate gradient's
  // matrix ops (dl - hi - lo is below 2^-16 |dl|); pad columns zero
  bf16_t* ph = a.dlp + (size_t)t * a.ldp;
  bf16_t* pl = ph + a.ldp / 2;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = lane + 64 * c;
    if (e >= a.ldp / 2) continue;
    if (e >= a.E) {
      ph[e] = pl[e] = (bf16_t)0;
      continue;
    }
    const float s = sv[c];
    const float dl = (a.score == 0) ? s * (ds[c] - u) : ds[c] * s * (1.f - s);
    a.dl[(size_t)t * a.E + e] = dl;
    const bf16_t h = f32_to_bf16(dl);
    ph[e] = h;
    pl[e] = f32_to_bf16(dl - bf16_to_f32(h));
  }
}

// Column sums of dl (the logit-bias gradient): partial sums over 256-token
// blocks, then the blocks in order.
__global__ __launch_bounds__(256) void dl_colsum_part_kernel(BwdAuxArgs a, float* part) {
  const int e = threadIdx.x;
  if (e >= a.E) return;
  const int t0 = blockIdx.x * 256, t1 = min(t0 + 256, a.T);
  float s = 0.f;
  for (int t = t0; t < t1; ++t) s += a.dl[(size_t)t * a.E + e];
  part[(size_t)blockIdx.x * a.E + e] = s;
}
__global__ __launch_bounds__(256) void dl_colsum_kernel(BwdAuxArgs a, const float* part,
                                                        int nb) {
  const int e = threadIdx.x;
  if (e >= a.E) return;
  float s = 0.f;
  for (int b = 0; b < nb; ++b) s += part[(size_t)b * a.E + e];
  a.dlogit_bias[e] = s;
}

// dWg = dl^T x on the matrix cores: the grouped backward GEMM's shared
// dW1/dW3 product (k = tokens, both operands mn-major) with dl's bf16 hi
// and lo parts as the "dA" operand, so the hi rows of the result are hi^T x
// and the lo rows lo^T x.  k is split into gg_splits ranges; the GEMM's own
// split reduction adds them in order into split 0's place (its dW1 / dW3
// outputs are pointed there), and the gate gradient is hi rows + lo rows.
__global__ __launch_bounds__(256) void gate_grad_sum_kernel(BwdAuxArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)a.E * a.d;
  if (i >= n) return;
  a.dw_gate[i] = a.dwg_part[i] + a.dwg_part[(size_t)(a.ldp / 2) * a.d + i];
}

// dx = RNE(dy + dx_shared + sum_k dx_rows[slot_row[t][k]] + dl Wg), one
// workgroup (4 waves) per 32 tokens x 256 columns:
//  a. the router term r = dl Wg on the matrix cores (32 x 32 x 16 bf16): wave
//     w takes the tile's columns 64 w .. 64 w + 63 for its 32 tokens, over the
//     experts in steps of 16.  dl enters as its bf16 hi and lo parts (written
//     by the router backward, |dl - hi - lo| < 2^-16 |dl|), Wg as its hi and
//     mid parts split here (|w - hi - mid| < 2^-16 |w|); the three products
//     hi hi, mid hi and hi lo carry r to about 2^-15 of its terms' size,
//     far below the bf16 rounding of dx.  r goes to LDS.
//  b. the row sums: dy, dx_shared, then the kept experts' rows in slot
//     order, 8 columns (16 bytes) per lane and four tokens per lane (their
//     loads of a slot in flight together), and one rounding of sum + r.
// The router term's Wg reads (64 KB per workgroup) are shared by 32 tokens.
// Measured on the 16B-shaped backward: 0.183 ms for the stage with the
// router term as fp32 FMAs (each workgroup reading all of Wg's columns for 8
// tokens), 0.164 with this layout at two tokens per lane, 0.156 at four;
// loading four slots' row indices and rows together was slower (0.182).
constexpr int DX_T = 32, DX_C = 256;

// Two floats to packed bf16, round to nearest even.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
// Non-temporal 16-byte load and store (the dx combine streams its rows once).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const void* p) {
  const u32x4_nt q = __builtin_nontemporal_load(static_cast<const u32x4_nt*>(p));
  return make_uint4(q.x, q.y, q.z, q.w);
}
__device__ __forceinline__ void add_bf16x8(float* v, uint4 p) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] += __uint_as_float(w[i] << 16);
    v[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
  }
}

__global__ __launch_bounds__(256) void dx_combine_kernel(BwdAuxArgs a) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  constexpr int RP = DX_C + 4;                  // LDS row pitch (floats)
  __shared__ float rt[DX_T * RP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int t0 = blockIdx.x * DX_T, c0 = blockIdx.y * DX_C;
  const int nt = min(DX_T, a.T - t0);
  const int half = a.ldp / 2;                   // dl parts' columns (E rounded up to 4, zero pad)

  // a. router term
  {
    f32x16_t acc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nb][r] = 0.f;
    const bf16_t* dh = a.dlp + (size_t)(t0 + min(l32, nt - 1)) * a.ldp;
    const int cw = c0 + wave * 64;
    for (int e0 = 0; e0 < a.E; e0 += 16) {
      const int ek = e0 + 8 * hi;               // this lane's 8 experts
      uint4 ph = make_uint4(0, 0, 0, 0), pl = ph;
      if (ek + 8 <= half) {
        ph = *reinterpret_cast<const uint4*>(dh + ek);
        pl = *reinterpret_cast<const uint4*>(dh + half + ek);
      } else if (ek + 4 <= half) {
        const uint2 h2 = *reinterpret_cast<const uint2*>(dh + ek);
        const uint2 l2 = *reinterpret_cast<const uint2*>(dh + half + ek);
        ph.x = h2.x; ph.y = h2.y; pl.x = l2.x; pl.y = l2.y;
      }
      const bf16x8_t fh = __builtin_bit_cast(bf16x8_t, ph);
      const bf16x8_t fl = __builtin_bit_cast(bf16x8_t, pl);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int c = min(cw + nb * 32 + l32, a.d - 1);
        float w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          w[i] = (ek + i < a.E) ? a.w_gate[(size_t)(ek + i) * a.d + c] : 0.f;
        uint32_t wh[4], wm[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wh[i] = bf16x2_rne(w[2 * i], w[2 * i + 1]);
          const float r0 = w[2 * i] - __uint_as_float(wh[i] << 16);
          const float r1 = w[2 * i + 1] - __uint_as_float(wh[i] & 0xffff0000u);
          wm[i] = bf16x2_rne(r0, r1);
        }
        const bf16x8_t gh = __builtin_bit_cast(bf16x8_t, make_uint4(wh[0], wh[1], wh[2], wh[3]));
        const bf16x8_t gm = __builtin_bit_cast(bf16x8_t, make_uint4(wm[0], wm[1], wm[2], wm[3]));
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gh, fh, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gm, fh, acc[nb], 0, 0, 0);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gh, fl, acc[nb], 0, 0, 0);
      }
    }
    // acc[nb][r] = r[token l32][column 64 wave + 32 nb + 8 (r / 4) + 4 hi + r % 4]
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(&rt[l32 * RP + wave * 64 + nb * 32 + 8 * g + 4 * hi]) =
            make_float4(acc[nb][4 * g], acc[nb][4 * g + 1], acc[nb][4 * g + 2],
                        acc[nb][4 * g + 3]);
  }
  __syncthreads();

  // b. row sums: lane group (tid & 31) takes columns 8 (tid & 31) .., row
  // group tid >> 5 the tokens tid / 32 + 8 i
  const int cl = (tid & 31) * 8, j = c0 + cl;
  if (j >= a.d) return;   // d is a multiple of 64
  const int tr = tid >> 5;
  constexpr int NQ = DX_T / 8;   // tokens per lane
#pragma unroll
  for (int i0 = 0; i0 < DX_T / 8; i0 += NQ) {
    float v[NQ][8];
    int tt[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      tt[q] = tr + 8 * (i0 + q);
      const size_t t = (size_t)(t0 + min(tt[q], nt - 1));
#pragma unroll
      for (int c = 0; c < 8; ++c) v[q][c] = 0.f;
      add_bf16x8(v[q], ld_nt(a.dy + t * a.d + j));
      if (a.dx_shared) add_bf16x8(v[q], ld_nt(a.dx_shared + t * a.d + j));
    }
    for (int k = 0; k < a.K; ++k) {
      uint4 p[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const size_t t = (size_t)(t0 + min(tt[q], nt - 1));
        const size_t row = (size_t)a.slot_row[t * a.K + k];
        p[q] = ld_nt(a.dx_rows + row * a.d + j);
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) add_bf16x8(v[q], p[q]);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (tt[q] >= nt) continue;
      const float* r = &rt[tt[q] * RP + cl];
      uint4 o;
      o.x = bf16x2_rne(v[q][0] + r[0], v[q][1] + r[1]);
      o.y = bf16x2_rne(v[q][2] + r[2], v[q][3] + r[3]);
      o.z = bf16x2_rne(v[q][4] + r[4], v[q][5] + r[5]);
      o.w = bf16x2_rne(v[q][6] + r[6], v[q][7] + r[7]);
      __builtin_nontemporal_store(u32x4_nt{o.x, o.y, o.z, o.w},
                                  reinterpret_cast<u32x4_nt*>(a.dx + (size_t)(t0 + tt[q]) * a.d + j));
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const BwdAuxArgs& a, hipStream_t s) {
  const int64_t tk = (int64_t)a.T * a.K;
  const unsigned grid = (unsigned)std::max<int64_t>(1, (tk + 255) / 256);
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const BwdAuxArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(router_bwd_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  if (a.dlogit_bias) {
    const int nb = (a.T + 255) / 256;
    float* part = a.dwg_part;     // scratch: nb x E floats (before the gate gradient)
    hipLaunchKernelGGL(dl_colsum_part_kernel, dim3(nb), dim3(256), 0, s, a, part);
    hipLaunchKernelGGL(dl_colsum_kernel, dim3(1), dim3(256), 0, s, a, (const float*)part, nb);
  }
  return hipGetLastError();
}

hipError_t launch_gate_grad(const BwdAuxArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.E * a.d;
  if (a.T > 0) {
    BwdGemmArgs g{};
    g.kind = 3; g.shared = true;
    g.T = a.T; g.d = a.d; g.inner = a.ldp / 2; g.n_experts = 1;
    g.x = a.x; g.da = a.dlp; g.ldda = a.ldp; g.zero = a.zero;
    // the product's hi rows, then its lo rows, in split 0's place
    g.dw1 = a.dwg_part; g.dw3 = a.dwg_part + (size_t)(a.ldp / 2) * a.d;
    g.splits = a.gg_splits; g.part = a.dwg_part;
    const hipError_t e = launch_gemm_bwd(g, s);
    if (e != hipSuccess) return e;
  } else {
    return launch_fill_zero(a.dw_gate, n, s);
  }
  hipLaunchKernelGGL(gate_grad_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_dx_combine(const BwdAuxArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.T + DX_T - 1) / DX_T, (a.d + DX_C - 1) / DX_C);
  hipLaunchKernelGGL(dx_combine_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
