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
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = lane + 64 * c;
    if (e >= a.E) continue;
    const float s = sv[c];
    const float dl = (a.score == 0) ? s * (ds[c] - u) : ds[c] * s * (1.f - s);
    a.dl[(size_t)t * a.E + e] = dl;
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

// dWg partials: thread = column j, 32 experts per workgroup, one chunk of
// tokens; dl of 64 tokens at a time staged in LDS.
constexpr int GG_E = 32, GG_T = 64;
__global__ __launch_bounds__(256) void gate_grad_part_kernel(BwdAuxArgs a) {
  __shared__ float sdl[GG_T][GG_E];
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int e0 = blockIdx.y * GG_E;
  const int chunk = blockIdx.z;
  const int per = (a.T + a.n_chunk - 1) / a.n_chunk;
  const int t0 = chunk * per, t1 = min(t0 + per, a.T);
  float acc[GG_E];
#pragma unroll
  for (int i = 0; i < GG_E; ++i) acc[i] = 0.f;
  for (int tb = t0; tb < t1; tb += GG_T) {
    __syncthreads();
    for (int i = threadIdx.x; i < GG_T * GG_E; i += 256) {
      const int tt = i / GG_E, ee = i % GG_E;
      const int t = tb + tt, e = e0 + ee;
      sdl[tt][ee] = (t < t1 && e < a.E) ? a.dl[(size_t)t * a.E + e] : 0.f;
    }
    __syncthreads();
    if (j < a.d) {
      const int n = min(GG_T, t1 - tb);
      for (int t8 = 0; t8 < n; t8 += 8) {
        float xv[8];      // eight token loads in flight (zeros past the chunk)
#pragma unroll
        for (int q = 0; q < 8; ++q)
          xv[q] = (t8 + q < n) ? bf16_to_f32(a.x[(size_t)(tb + t8 + q) * a.d + j]) : 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int i = 0; i < GG_E; ++i) acc[i] = fmaf(sdl[t8 + q][i], xv[q], acc[i]);
      }
    }
  }
  if (j >= a.d) return;
#pragma unroll
  for (int i = 0; i < GG_E; ++i) {
    const int e = e0 + i;
    if (e < a.E) a.dwg_part[((size_t)chunk * a.E + e) * a.d + j] = acc[i];
  }
}
__global__ __launch_bounds__(256) void gate_grad_sum_kernel(BwdAuxArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = (int64_t)a.E * a.d;
  if (i >= n) return;
  float s = 0.f;
  for (int c = 0; c < a.n_chunk; ++c) s += a.dwg_part[(size_t)c * n + i];
  a.dw_gate[i] = s;
}

// dx = RNE(dy + dx_shared + sum_k dx_rows[slot_row[t][k]] + dl Wg): thread =
// column j, DX_T tokens per workgroup.  The router term first (each Wg
// element read once per workgroup, the tokens' dl rows staged in LDS), then
// the row sums, four tokens' loads at a time.
constexpr int DX_T = 16;
__global__ __launch_bounds__(256) void dx_combine_kernel(BwdAuxArgs a) {
  __shared__ float sdl[DX_T][MAX_EXPERTS];
  const int t0 = blockIdx.x * DX_T;
  const int j = blockIdx.y * 256 + threadIdx.x;
  const int nt = min(DX_T, a.T - t0);
  for (int i = threadIdx.x; i < DX_T * a.E; i += 256) {
    const int tt = i / a.E, e = i % a.E;
    sdl[tt][e] = (tt < nt) ? a.dl[(size_t)(t0 + tt) * a.E + e] : 0.f;
  }
  __syncthreads();
  if (j >= a.d) return;
  float r[DX_T];
#pragma unroll
  for (int tt = 0; tt < DX_T; ++tt) r[tt] = 0.f;
  for (int e = 0; e < a.E; ++e) {
    const float w = a.w_gate[(size_t)e * a.d + j];
#pragma unroll
    for (int tt = 0; tt < DX_T; ++tt) r[tt] = fmaf(sdl[tt][e], w, r[tt]);
  }
#pragma unroll
  for (int t4 = 0; t4 < DX_T; t4 += 4) {
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = t0 + t4 + q;
      v[q] = 0.f;
      if (t4 + q >= nt) continue;
      v[q] = bf16_to_f32(a.dy[(size_t)t * a.d + j]);
      if (a.dx_shared) v[q] += a.dx_shared[(size_t)t * a.d + j];
    }
    for (int k = 0; k < a.K; ++k) {
      float w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + t4 + q;
        w[q] = (t4 + q < nt)
                   ? a.dx_rows[(size_t)a.slot_row[(size_t)t * a.K + k] * a.d + j] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] += w[q];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = t0 + t4 + q;
      if (t4 + q < nt) a.dx[(size_t)t * a.d + j] = f32_to_bf16(v[q] + r[t4 + q]);
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
  const dim3 grid((a.d + 255) / 256, (a.E + GG_E - 1) / GG_E, a.n_chunk);
  hipLaunchKernelGGL(gate_grad_part_kernel, grid, dim3(256), 0, s, a);
  const int64_t n = (int64_t)a.E * a.d;
  hipLaunchKernelGGL(gate_grad_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dx_combine(const BwdAuxArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.T + DX_T - 1) / DX_T, (a.d + 255) / 256);
  hipLaunchKernelGGL(dx_combine_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
