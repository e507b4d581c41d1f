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

// dx = RNE(dy + dx_shared + sum_k dx_rows[slot_row[t][k]] + dl Wg): thread =
// columns 4 j .. 4 j + 3, DX_T tokens per workgroup.  The router term first
// (each 4-column group of Wg read once per workgroup, the tokens' dl rows
// staged in LDS), then the row sums, in a fixed order.  Eight tokens per
// workgroup (measured on the 16B-shaped backward: 0.185 ms against 0.202
// with four, 0.224 with sixteen, 0.295 with 32: the router term's registers
// limit the waves in flight).
constexpr int DX_T = 8;
__device__ __forceinline__ void add_bf16x4(float* v, uint2 p) {
  v[0] += __uint_as_float(p.x << 16);
  v[1] += __uint_as_float(p.x & 0xffff0000u);
  v[2] += __uint_as_float(p.y << 16);
  v[3] += __uint_as_float(p.y & 0xffff0000u);
}
__global__ __launch_bounds__(256) void dx_combine_kernel(BwdAuxArgs a) {
  __shared__ float sdl[DX_T][MAX_EXPERTS];
  const int t0 = blockIdx.x * DX_T;
  const int j = (blockIdx.y * 256 + threadIdx.x) * 4;
  const int nt = min(DX_T, a.T - t0);
  for (int i = threadIdx.x; i < DX_T * a.E; i += 256) {
    const int tt = i / a.E, e = i % a.E;
    sdl[tt][e] = (tt < nt) ? a.dl[(size_t)(t0 + tt) * a.E + e] : 0.f;
  }
  __syncthreads();
  if (j >= a.d) return;   // d is a multiple of 4
  float r[DX_T][4];
#pragma unroll
  for (int tt = 0; tt < DX_T; ++tt)
#pragma unroll
    for (int q = 0; q < 4; ++q) r[tt][q] = 0.f;
  for (int e = 0; e < a.E; ++e) {
    const float4 w = *reinterpret_cast<const float4*>(a.w_gate + (size_t)e * a.d + j);
#pragma unroll
    for (int tt = 0; tt < DX_T; ++tt) {
      const float l = sdl[tt][e];
      r[tt][0] = fmaf(l, w.x, r[tt][0]);
      r[tt][1] = fmaf(l, w.y, r[tt][1]);
      r[tt][2] = fmaf(l, w.z, r[tt][2]);
      r[tt][3] = fmaf(l, w.w, r[tt][3]);
    }
  }
  // four tokens at a time, their rows' loads issued together
#pragma unroll
  for (int t4 = 0; t4 < DX_T; t4 += 4) {
    float v[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tt = t4 + q;
      const size_t t = (size_t)(t0 + min(tt, nt - 1));
      v[q][0] = v[q][1] = v[q][2] = v[q][3] = 0.f;
      add_bf16x4(v[q], *reinterpret_cast<const uint2*>(a.dy + t * a.d + j));
      if (a.dx_shared)
        add_bf16x4(v[q], *reinterpret_cast<const uint2*>(a.dx_shared + t * a.d + j));
    }
    for (int k = 0; k < a.K; ++k) {
      uint2 p[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const size_t t = (size_t)(t0 + min(t4 + q, nt - 1));
        const size_t row = (size_t)a.slot_row[t * a.K + k];
        p[q] = *reinterpret_cast<const uint2*>(a.dx_rows + row * a.d + j);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) add_bf16x4(v[q], p[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tt = t4 + q;
      if (tt >= nt) continue;
      uint2 o;
      o.x = (uint32_t)f32_to_bf16(v[q][0] + r[tt][0]) |
            ((uint32_t)f32_to_bf16(v[q][1] + r[tt][1]) << 16);
      o.y = (uint32_t)f32_to_bf16(v[q][2] + r[tt][2]) |
            ((uint32_t)f32_to_bf16(v[q][3] + r[tt][3]) << 16);
      *reinterpret_cast<uint2*>(a.dx + (size_t)(t0 + tt) * a.d + j) = o;
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
  const dim3 grid((a.T + DX_T - 1) / DX_T, (a.d + 1023) / 1024);
  hipLaunchKernelGGL(dx_combine_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
