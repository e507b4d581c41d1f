// E4M3 quantisation with power-of-two scales (DeepSeek-V3 Technical Report
// summary, "3.3 FP8 Training": fine-grained scaling, power-of-two scaling
// factors for activations; "B.2 Discussion About Block-Wise Quantization":
// activations grouped 1 x 128, unlike 128 x 128 blocks).
//
// Every group (128 consecutive values of a row, or a 128 x 128 block) gets
// the smallest power of two 2^E with max|v| <= 448 * 2^E (448 = the largest
// finite E4M3 value), stored as the byte E + 127; each value becomes the
// E4M3 code nearest to v * 2^-E (ties to even, the hardware conversion's
// rounding).  A group of zeros gets E = 0.  Scaling by a power of two is
// exact, so the codes depend only on the inputs.
#include "common.h"

namespace moe {

namespace {

// Smallest E with amax <= 448 * 2^E, clamped to [-127, 127]; 0 for zero.
// With amax = f 2^e, f in [0.5, 1): E = e - 9 when f <= 0.875, else e - 8.
__device__ __forceinline__ int e4m3_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(amax);
  const float f = __builtin_amdgcn_frexp_mantf(amax);
  const int E = e - 9 + (f > 0.875f ? 1 : 0);
  return min(max(E, -127), 127);
}

// 2^-E for E in [-127, 126] (a normal float).
__device__ __forceinline__ float pow2_neg(int E) { return __int_as_float((127 - E) << 23); }

// Eight values to eight E4M3 codes (round to nearest even), low byte first.
__device__ __forceinline__ uint2 e4m3_pack8(const float (&v)[8], float s) {
  uint2 r;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * s, v[1] * s, 0, false);
  r.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2] * s, v[3] * s, w, true);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * s, v[5] * s, 0, false);
  r.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[6] * s, v[7] * s, w, true);
  return r;
}

__device__ __forceinline__ void load8(const void* src, int f32, int64_t i, float (&v)[8]) {
  if (f32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + i);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(src) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_to_f32((bf16_t)(w[k] & 0xffff));
      v[2 * k + 1] = bf16_to_f32((bf16_t)(w[k] >> 16));
    }
  }
}

// 1 x 128 groups: 16 lanes per group, 8 values per lane.
__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs a) {
  const int G = a.cols / 128;
  const int64_t ngroups = (int64_t)a.rows * G;
  const int64_t gid = (int64_t)blockIdx.x * 16 + threadIdx.x / 16;
  const int l16 = threadIdx.x & 15;
  const bool live = gid < ngroups;
  const int64_t row = live ? gid / G : 0;
  const int g = live ? (int)(gid % G) : 0;
  const int64_t i = row * a.cols + g * 128 + l16 * 8;
  float v[8];
  if (live) load8(a.src, a.src_f32, i, v);
  else for (int k = 0; k < 8; ++k) v[k] = 0.f;
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const int E = e4m3_scale_exp(amax);
  if (!live) return;
  *reinterpret_cast<uint2*>(a.codes + i) = e4m3_pack8(v, pow2_neg(E));
  if (l16 == 0) a.scales[row * G + g] = (uint8_t)(E + 127);
}

// 128 x 128 blocks: one workgroup per block, thread t covers row t / 2,
// columns 64 (t % 2) .. + 63.
__global__ __launch_bounds__(256) void quant_blocks_kernel(QuantArgs a) {
  __shared__ float red[256];
  const int RB = a.rows / 128, CB = a.cols / 128;
  const int64_t blk = blockIdx.x;
  const int64_t b = blk / ((int64_t)RB * CB);
  const int rb = (int)((blk / CB) % RB), cb = (int)(blk % CB);
  const int t = threadIdx.x;
  const int64_t base = (b * a.rows + rb * 128 + t / 2) * a.cols + cb * 128 + (t % 2) * 64;
  float v[8][8];
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    load8(a.src, a.src_f32, base + c * 8, v[c]);
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[c][k]));
  }
  red[t] = amax;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  const int E = e4m3_scale_exp(red[0]);
  const float s = pow2_neg(E);
#pragma unroll
  for (int c = 0; c < 8; ++c)
    *reinterpret_cast<uint2*>(a.codes + base + c * 8) = e4m3_pack8(v[c], s);
  if (t == 0) a.scales[(b * RB + rb) * CB + cb] = (uint8_t)(E + 127);
}

}  // namespace

hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t s) {
  const int64_t ngroups = (int64_t)a.rows * (a.cols / 128);
  if (ngroups == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((ngroups + 15) / 16)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quant_blocks(const QuantArgs& a, hipStream_t s) {
  const int64_t nblk = a.batch * (a.rows / 128) * (a.cols / 128);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_blocks_kernel, dim3((unsigned)nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
