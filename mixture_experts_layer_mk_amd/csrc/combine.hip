// Combine: out[t] = base[t] + sum_k g[t,k] * Y[slot_row[t,k]] (Y fp32), summed in slot
// order k = 0..K-1 in fp32 and rounded once to the output type.  base is
// x + (shared experts) in fp32, or x itself when there are no shared experts.
// Every output element has one owner thread: no atomics, deterministic.
//
// Method: DeepSeekMoE paper abstract and blog post "Shared Expert Isolation
// (Section 3.2)" -- shared experts always contribute with weight one; routed
// experts contribute with their gate weights; the residual is added back.
#include "common.h"

namespace moe {

namespace {

template <typename T, int VEC, bool BASE_F32>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int per_row = (a.d / VEC + 255) / 256;
  const int t = blockIdx.x / per_row;
  const int n0 = ((blockIdx.x % per_row) * 256 + threadIdx.x) * VEC;
  if (n0 >= a.d) return;
  float acc[VEC];
  if (BASE_F32) {
    const float* b = static_cast<const float*>(a.base) + (size_t)t * a.d + n0;
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = b[v];
  } else {
    const T* b = static_cast<const T*>(a.base) + (size_t)t * a.d + n0;
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = ld_f32<T>(b + v);
  }
  const float* y = a.y;
  for (int k = 0; k < a.K; ++k) {
    const int q = t * a.K + k;
    const float g = a.topk_w[q];
    const float4* yr = reinterpret_cast<const float4*>(y + (size_t)a.slot_row[q] * a.d + n0);
#pragma unroll
    for (int v = 0; v < VEC / 4; ++v) {
      const float4 yv = yr[v];
      acc[4 * v + 0] = fmaf(g, yv.x, acc[4 * v + 0]);
      acc[4 * v + 1] = fmaf(g, yv.y, acc[4 * v + 1]);
      acc[4 * v + 2] = fmaf(g, yv.z, acc[4 * v + 2]);
      acc[4 * v + 3] = fmaf(g, yv.w, acc[4 * v + 3]);
    }
  }
  T o[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) o[v] = from_f32<T>(acc[v]);
  *reinterpret_cast<uint4*>(static_cast<T*>(a.out) + (size_t)t * a.d + n0) =
      *reinterpret_cast<const uint4*>(o);
}

template <typename T, int VEC>
void launch_t(const CombineArgs& a, hipStream_t s) {
  dim3 grid(((a.d / VEC + 255) / 256) * a.T);
  if (a.base_f32) hipLaunchKernelGGL((combine_kernel<T, VEC, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((combine_kernel<T, VEC, false>), grid, dim3(256), 0, s, a);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.dtype == 1) launch_t<bf16_t, 8>(a, s);
  else launch_t<float, 4>(a, s);
  return hipGetLastError();
}

}  // namespace moe
