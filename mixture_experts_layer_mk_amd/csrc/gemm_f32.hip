// Grouped expert GEMMs for fp32 layers (LDS-tiled fp32 FMA, 64 x 64 tiles).
//
// Each expert is a SwiGLU FFN W2 (silu(W1 u) * (W3 u)) (expert form of the
// DeepSeekMoE layer; blog post "Fine-Grained Expert Segmentation (Section
// 3.1)").  Stages:
//   GATEUP      H = silu(A W1^T) * (A W3^T) for every routed M-tile (A = the
//               tile's token rows, gathered from x) or for all tokens through
//               each shared expert (A = x)
//   DOWN        Y = H W2^T for every routed M-tile
//   DOWN_SHARED S = x + sum_s H_s W2_s^T over the shared experts, fp32
#include "common.h"

namespace moe {

namespace {

constexpr int FB = 64;   // tile rows and columns
constexpr int FK = 16;   // k per LDS stage

__device__ __forceinline__ float silu_f(float v) { return v / (1.f + expf(-v)); }

template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  __shared__ float As[FK][FB + 1];
  __shared__ float B1s[FK][FB + 1];
  __shared__ float B3s[FK][FB + 1];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const bool routed = !(MODE == 2 || (MODE == 0 && a.shared));
  const int mdim = routed ? a.max_mtiles : (a.T + FB - 1) / FB;
  const int mt = blockIdx.x % mdim, nt = blockIdx.x / mdim;
  int row0, rows, e;
  if (routed) {
    if (mt >= *a.n_tiles) return;
    const MTile t = a.tiles[mt];
    row0 = t.row0; rows = t.rows; e = t.expert;
  } else {
    row0 = mt * FB; rows = min(FB, a.T - row0); e = 0;
  }

  float acc1[4][4], acc3[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) { acc1[i][j] = 0.f; acc3[i][j] = 0.f; }

  // acc1 (+= A B1^T), acc3 (+= A B3^T): A rows row0.., B rows n0.. of width
  // Kd; B rows >= nvalid and k >= Kd read as zero.
  auto kloop = [&](const float* A, int lda, const float* B1, const float* B3,
                   int ldb, int n0, int nvalid, int Kd) {
    for (int k0 = 0; k0 < Kd; k0 += FK) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int li = tid + 256 * q, r = li / FK, k = li % FK;
        const bool kin = k0 + k < Kd;
        const int rr = min(r, rows - 1);
        const int src = a.a_rows ? a.a_rows[row0 + rr] : row0 + rr;
        As[k][r] = kin ? A[(size_t)src * lda + k0 + k] : 0.f;
        const int nn = n0 + r;
        const bool nin = kin && nn < nvalid;
        B1s[k][r] = nin ? B1[(size_t)nn * ldb + k0 + k] : 0.f;
        if (MODE == 0) B3s[k][r] = nin ? B3[(size_t)nn * ldb + k0 + k] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < FK; ++k) {
        float av[4], bv[4], cv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = As[k][ty + 16 * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bv[j] = B1s[k][tx + 16 * j];
          if (MODE == 0) cv[j] = B3s[k][tx + 16 * j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc1[i][j] = fmaf(av[i], bv[j], acc1[i][j]);
            if (MODE == 0) acc3[i][j] = fmaf(av[i], cv[j], acc3[i][j]);
          }
      }
      __syncthreads();
    }
  };

  const float* A = static_cast<const float*>(a.a);
  float* out = static_cast<float*>(a.out);
  if (MODE == 0) {
    const int tiles_per = (a.inner + FB - 1) / FB;
    const int grp = routed ? e : nt / tiles_per;
    const int n0 = (routed ? nt : nt % tiles_per) * FB;
    const size_t wo = (size_t)grp * a.inner * a.d;
    kloop(A, a.lda, static_cast<const float*>(a.w1) + wo,
          static_cast<const float*>(a.w3) + wo, a.d, n0, a.inner, a.d);
    const int col_off = routed ? 0 : grp * a.inner;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = ty + 16 * i, n = n0 + tx + 16 * j;
        if (m < rows && n < a.inner)
          out[(size_t)(row0 + m) * a.ldo + col_off + n] =
              silu_f(acc1[i][j]) * acc3[i][j];
      }
  } else {
    const int n0 = nt * FB;
    if (MODE == 1) {
      kloop(A, a.lda, static_cast<const float*>(a.w2) + (size_t)e * a.d * a.inner,
            nullptr, a.inner, n0, a.d, a.inner);
    } else {
      for (int s = 0; s < a.n_experts; ++s)
        kloop(A + (size_t)s * a.inner, a.lda,
              static_cast<const float*>(a.w2) + (size_t)s * a.d * a.inner,
              nullptr, a.inner, n0, a.d, a.inner);
    }
    const float* x = static_cast<const float*>(a.x);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = ty + 16 * i, n = n0 + tx + 16 * j;
        if (m < rows && n < a.d) {
          const size_t o = (size_t)(row0 + m) * a.ldo + n;
          out[o] = (MODE == 2) ? x[(size_t)(row0 + m) * a.d + n] + acc1[i][j]
                               : acc1[i][j];
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s) {
  const bool routed = !(a.mode == 2 || (a.mode == 0 && a.shared));
  const int mdim = routed ? a.max_mtiles : (a.T + FB - 1) / FB;
  int ndim;
  if (a.mode == 0) ndim = ((a.inner + FB - 1) / FB) * (routed ? 1 : a.n_experts);
  else ndim = (a.d + FB - 1) / FB;
  dim3 grid(mdim * ndim), block(256);
  if (a.mode == 0) hipLaunchKernelGGL(gemm_f32_kernel<0>, grid, block, 0, s, a);
  else if (a.mode == 1) hipLaunchKernelGGL(gemm_f32_kernel<1>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(gemm_f32_kernel<2>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
