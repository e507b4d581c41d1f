// Combine: out[t] = base[t] + sum_k g[t,k] * Y[slot_row[t,k]], summed in slot
// order k = 0..K-1 in fp32 and rounded once to the output type.  base is
// x + (shared experts) in fp32, or x itself when there are no shared experts.
// Y is fp32 (fp32 layers) or fp16 times a power-of-two inverse scale per 64
// columns of a row (bf16 layers).  Every output element has one owner
// thread: no atomics, deterministic.
//
// Method: DeepSeekMoE paper abstract and blog post "Shared Expert Isolation
// (Section 3.2)" -- shared experts always contribute with weight one; routed
// experts contribute with their gate weights; the residual is added back.
#include "common.h"

namespace moe {

namespace {

constexpr int CB_K = 8;   // slots whose loads are all issued up front

// Every input element is read once and every output written once: the
// loads and the store are non-temporal, so the streams do not displace
// cached lines (measured on the 16B-shaped layer: 0.121 -> 0.094 ms, from
// 5.2 to 6.6 TB/s).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const void* p) {
  const u32x4_nt q = __builtin_nontemporal_load(static_cast<const u32x4_nt*>(p));
  return make_uint4(q.x, q.y, q.z, q.w);
}

template <typename T, int VEC, bool BASE_F32, bool Y16>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  static_assert(!Y16 || VEC == 8, "fp16 rows are read 8 columns at a time");
  const int per_row = (a.d / VEC + 255) / 256;
  const int t = blockIdx.x / per_row;
  const int n0 = ((blockIdx.x % per_row) * 256 + threadIdx.x) * VEC;
  if (n0 >= a.d) return;
  float acc[VEC];
  if (BASE_F32) {
    const f32x4_nt* b = reinterpret_cast<const f32x4_nt*>(static_cast<const float*>(a.base) +
                                                          (size_t)t * a.d + n0);
#pragma unroll
    for (int v = 0; v < VEC / 4; ++v) {
      const f32x4_nt w = __builtin_nontemporal_load(b + v);
      acc[4 * v] = w.x; acc[4 * v + 1] = w.y; acc[4 * v + 2] = w.z; acc[4 * v + 3] = w.w;
    }
  } else {
    const T* b = static_cast<const T*>(a.base) + (size_t)t * a.d + n0;
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = ld_f32<T>(b + v);
  }
  if (Y16 && a.K <= CB_K) {
    // All slots' row indices and weights, then all their rows and scales in
    // flight together, then the sums in slot order (as below).
    int rows[CB_K];
    float gk[CB_K], inv[CB_K];
    uint4 hv[CB_K];
#pragma unroll
    for (int k = 0; k < CB_K; ++k)
      if (k < a.K) {
        rows[k] = a.slot_row[t * a.K + k];
        gk[k] = a.topk_w[t * a.K + k];
      }
#pragma unroll
    for (int k = 0; k < CB_K; ++k)
      if (k < a.K) {
        hv[k] = ld_nt(static_cast<const uint16_t*>(a.y) + (size_t)rows[k] * a.d + n0);
        inv[k] = a.yscale[(size_t)rows[k] * (a.d / Y_GROUP) + n0 / Y_GROUP];
      }
#pragma unroll
    for (int k = 0; k < CB_K; ++k) {
      if (k >= a.K) break;
      const uint32_t w[4] = {hv[k].x, hv[k].y, hv[k].z, hv[k].w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[v] & 0xffffu));
        const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[v] >> 16));
        acc[2 * v + 0] = fmaf(gk[k], lo * inv[k], acc[2 * v + 0]);
        acc[2 * v + 1] = fmaf(gk[k], hi * inv[k], acc[2 * v + 1]);
      }
    }
  } else
  for (int k = 0; k < a.K; ++k) {
    const int q = t * a.K + k;
    const float g = a.topk_w[q];
    const size_t row = (size_t)a.slot_row[q];
    if (Y16) {
      const uint4 hv = ld_nt(static_cast<const uint16_t*>(a.y) + row * a.d + n0);
      const float inv = a.yscale[row * (a.d / Y_GROUP) + n0 / Y_GROUP];
      const uint32_t w[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[v] & 0xffffu));
        const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[v] >> 16));
        acc[2 * v + 0] = fmaf(g, lo * inv, acc[2 * v + 0]);
        acc[2 * v + 1] = fmaf(g, hi * inv, acc[2 * v + 1]);
      }
    } else {
      const float4* yr = reinterpret_cast<const float4*>(static_cast<const float*>(a.y) +
                                                         row * a.d + n0);
#pragma unroll
      for (int v = 0; v < VEC / 4; ++v) {
        const float4 yv = yr[v];
        acc[4 * v + 0] = fmaf(g, yv.x, acc[4 * v + 0]);
        acc[4 * v + 1] = fmaf(g, yv.y, acc[4 * v + 1]);
        acc[4 * v + 2] = fmaf(g, yv.z, acc[4 * v + 2]);
        acc[4 * v + 3] = fmaf(g, yv.w, acc[4 * v + 3]);
      }
    }
  }
  T o[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) o[v] = from_f32<T>(acc[v]);
  const uint4 ov = *reinterpret_cast<const uint4*>(o);
  __builtin_nontemporal_store(u32x4_nt{ov.x, ov.y, ov.z, ov.w},
                              reinterpret_cast<u32x4_nt*>(static_cast<T*>(a.out) +
                                                          (size_t)t * a.d + n0));
}

template <typename T, int VEC, bool Y16>
void launch_t(const CombineArgs& a, hipStream_t s) {
  dim3 grid(((a.d / VEC + 255) / 256) * a.T);
  if (a.base_f32) hipLaunchKernelGGL((combine_kernel<T, VEC, true, Y16>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((combine_kernel<T, VEC, false, Y16>), grid, dim3(256), 0, s, a);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.yscale) launch_t<bf16_t, 8, true>(a, s);
    else launch_t<bf16_t, 8, false>(a, s);
  } else {
    launch_t<float, 4, false>(a, s);
  }
  return hipGetLastError();
}

}  // namespace moe
