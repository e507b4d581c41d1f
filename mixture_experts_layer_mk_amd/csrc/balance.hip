// Auxiliary-loss-free load balancing: after a step, every routed expert's
// selection bias moves by a fixed step toward balance -- down when the expert
// was overloaded, up when it was underloaded (DeepSeek-V3 Technical Report
// summary, "2. Architecture", auxiliary-loss-free load balancing).
//
// An expert is overloaded when its token count exceeds the mean count
// total / n, underloaded when below it; the comparison count * n vs total is
// done in integers, so it is exact.  The relative load count * n / total is
// reported beside (1 = balanced).  One workgroup; the total is summed in a
// fixed order.
#include "common.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void bias_update_kernel(BiasUpdateArgs a) {
  __shared__ long long part[256];
  const int tid = threadIdx.x;
  long long s = 0;
  for (int e = tid; e < a.n; e += 256) s += a.counts[e];
  part[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  const long long total = part[0];
  for (int e = tid; e < a.n; e += 256) {
    const long long cn = (long long)a.counts[e] * a.n;
    if (a.bias) {
      if (cn > total) a.bias[e] = a.bias[e] - a.gamma;
      else if (cn < total) a.bias[e] = a.bias[e] + a.gamma;
    }
    if (a.rel_load) a.rel_load[e] = total > 0 ? (float)cn / (float)total : 0.f;
  }
}

}  // namespace

hipError_t launch_bias_update(const BiasUpdateArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
