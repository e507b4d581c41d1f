// Grouped expert GEMMs for bf16 layers on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Each expert is a SwiGLU FFN W2 (silu(W1 u) * (W3 u)) (expert form of the
// DeepSeekMoE layer; blog post "Fine-Grained Expert Segmentation (Section
// 3.1)").  Stages (same as the fp32 path):
//   GATEUP      H = silu(A W1^T) * (A W3^T), gate and up fused in one tile
//   DOWN        Y = H W2^T (routed rows, bf16 out)
//   DOWN_SHARED S = x + sum_s H_s W2_s^T (all tokens, fp32 out)
//
// Tiling.  A workgroup (4 waves) owns BM token rows x 256 weight rows with a
// 64-wide k step.  Both operands are k-contiguous in memory (token rows and
// linear-layer weight rows), so every lane moves 16-byte chunks.  Tiles are
// double-buffered in LDS (2 x (BM + 256) x 128 B), with the 16-byte chunks
// of each 128-byte row XOR-swizzled so the matrix-core operand reads and the
// tile writes are free of bank conflicts.  The matrix instruction takes the
// weight fragment as its first operand, so each lane's accumulator holds 4
// consecutive output columns of one token row (8- or 16-byte stores).
// For GATEUP each wave's weight rows are 50% W1 and 50% W3 for the same
// inner columns, so silu(gate) * up is formed in registers.
// Blocks are remapped so that each XCD (blocks are dealt round-robin over the
// 8 XCDs) runs a contiguous range of tiles, with the M-tiles of one weight
// tile adjacent: the weight tile is then fetched into that XCD's L2 once.
#include "common.h"

namespace moe {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = 256;   // weight rows per workgroup
constexpr int BK = 64;    // k per stage (8 chunks of 16 B)

// Chunk position of 16-byte chunk c of LDS row `row` (8 chunks per row).
// Consecutive 8 rows, and 16 rows split by bank half, hit distinct banks.
__device__ __forceinline__ int swz(int row, int c) {
  return c ^ (row & 7) ^ ((row >> 3) & 1);
}

__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, j = b >> 3, q = n >> 3, r = n & 7;
  return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

__device__ __forceinline__ float silu_f(float v) { return v / (1.f + expf(-v)); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// MODE 0 GATEUP, 1 DOWN, 2 DOWN_SHARED.  WAVES_M x (4 / WAVES_M) waves.
template <int MODE, int BM, int WAVES_M>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int A_CH = BM / 32;     // A chunks per thread per stage
  constexpr int B_CH = BN / 32;     // B chunks per thread per stage
  static_assert(MB >= 1 && NB >= 2 && (NB % 2) == 0, "tile shape");

  __shared__ u32x4 As[2][BM * 8];
  __shared__ u32x4 Bs[2][BN * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const bool routed = !(MODE == 2 || (MODE == 0 && a.shared));
  const int mdim = routed ? a.max_mtiles : (a.T + BM - 1) / BM;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = L % mdim, nt = L / mdim;

  int row0, rows, e;
  if (routed) {
    if (mt >= *a.n_tiles) return;
    const MTile t = a.tiles[mt];
    row0 = t.row0; rows = t.rows; e = t.expert;
  } else {
    row0 = mt * BM; rows = min(BM, a.T - row0); e = 0;
  }

  const bf16_t* A = static_cast<const bf16_t*>(a.a);
  const int c8 = (tid & 7) * 8;          // element offset of this thread's chunk
  const int rbase = tid >> 3;            // first row this thread loads

  // A source rows (clamped into the tile's valid rows).
  const bf16_t* pa[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int r = min(i * 32 + rbase, rows - 1);
    pa[i] = A + (size_t)(row0 + r) * a.lda + c8;
  }

  // B source rows.
  const bf16_t* pb[B_CH];
  int kdim, n0 = 0, grp = 0, inner0 = 0;
  if (MODE == 0) {
    const int half = WN / 2;                       // inner columns per wave
    const int per_wg = WAVES_N * half;             // inner columns per tile
    const int tiles_per = (a.inner + per_wg - 1) / per_wg;
    grp = routed ? e : nt / tiles_per;
    inner0 = (routed ? nt : nt % tiles_per) * per_wg;
    const size_t wo = (size_t)grp * a.inner * a.d;
    const bf16_t* w1 = static_cast<const bf16_t*>(a.w1) + wo;
    const bf16_t* w3 = static_cast<const bf16_t*>(a.w3) + wo;
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int r = i * 32 + rbase;
      const int rw = r / WN, rr = r % WN;
      const int inner = min(inner0 + rw * half + (rr % half), a.inner - 1);
      pb[i] = ((rr < half) ? w1 : w3) + (size_t)inner * a.d + c8;
    }
    kdim = a.d;
  } else {
    n0 = nt * BN;
    const bf16_t* w2 = static_cast<const bf16_t*>(a.w2) +
                       (MODE == 1 ? (size_t)e * a.d * a.inner : 0);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int n = min(n0 + i * 32 + rbase, a.d - 1);
      pb[i] = w2 + (size_t)n * a.inner + c8;
    }
    kdim = (MODE == 1) ? a.inner : a.inner * a.n_experts;
  }
  const int nk = kdim / BK;

  // Element offset of k-block kb in the B rows (DOWN_SHARED walks the
  // shared experts one after the other along k).
  auto boff = [&](int kb) -> size_t {
    if (MODE != 2) return (size_t)kb * BK;
    const int k = kb * BK, s = k / a.inner;
    return (size_t)s * a.d * a.inner + (k - s * a.inner);
  };

  u32x4 ra[A_CH], rb[B_CH];
  auto gload = [&](int kb) {
    const size_t ka = (size_t)kb * BK, kbo = boff(kb);
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const u32x4*>(pa[i] + ka);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = *reinterpret_cast<const u32x4*>(pb[i] + kbo);
  };
  auto lstore = [&](int buf) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int r = i * 32 + rbase;
      As[buf][r * 8 + swz(r, c)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int r = i * 32 + rbase;
      Bs[buf][r * 8 + swz(r, c)] = rb[i];
    }
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();
  const int l32 = lane & 31, hi = lane >> 5;
  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nk) gload(kb + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = 2 * kk + hi;
      bf16x8 af[MB], bfr[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int r = wm * WM + mb * 32 + l32;
        af[mb] = __builtin_bit_cast(bf16x8, As[cur][r * 8 + swz(r, c)]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = wn * WN + nb * 32 + l32;
        bfr[nb] = __builtin_bit_cast(bf16x8, Bs[cur][r * 8 + swz(r, c)]);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[nb], af[mb],
                                                               acc[nb][mb], 0, 0, 0);
    }
    if (kb + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  // acc[nb][mb][r] = D[n][m] with n = nb*32 + 8*(r/4) + 4*hi + (r%4) and
  // m = mb*32 + l32 inside the wave's tile.
  if (MODE == 0) {
    constexpr int HALF_NB = NB / 2;
    const int col_off = routed ? 0 : grp * a.inner;
    bf16_t* out = static_cast<bf16_t*>(a.out);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = wm * WM + mb * 32 + l32;
      if (m >= rows) continue;
      bf16_t* orow = out + (size_t)(row0 + m) * a.ldo + col_off;
#pragma unroll
      for (int nb = 0; nb < HALF_NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int inner = inner0 + wn * (WN / 2) + nb * 32 + 8 * g + 4 * hi;
          if (inner >= a.inner) continue;
          float h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            h[q] = silu_f(acc[nb][mb][4 * g + q]) * acc[nb + HALF_NB][mb][4 * g + q];
          uint2 v;
          v.x = pack2(h[0], h[1]);
          v.y = pack2(h[2], h[3]);
          *reinterpret_cast<uint2*>(orow + inner) = v;
        }
    }
  } else if (MODE == 1) {
    bf16_t* out = static_cast<bf16_t*>(a.out);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = wm * WM + mb * 32 + l32;
      if (m >= rows) continue;
      bf16_t* orow = out + (size_t)(row0 + m) * a.ldo;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + nb * 32 + 8 * g + 4 * hi;
          if (n >= a.d) continue;
          uint2 v;
          v.x = pack2(acc[nb][mb][4 * g + 0], acc[nb][mb][4 * g + 1]);
          v.y = pack2(acc[nb][mb][4 * g + 2], acc[nb][mb][4 * g + 3]);
          *reinterpret_cast<uint2*>(orow + n) = v;
        }
    }
  } else {
    float* out = static_cast<float*>(a.out);
    const bf16_t* x = static_cast<const bf16_t*>(a.x);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = wm * WM + mb * 32 + l32;
      if (m >= rows) continue;
      float* orow = out + (size_t)(row0 + m) * a.ldo;
      const bf16_t* xrow = x + (size_t)(row0 + m) * a.d;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + nb * 32 + 8 * g + 4 * hi;
          if (n >= a.d) continue;
          const uint2 xv = *reinterpret_cast<const uint2*>(xrow + n);
          float4 o;
          o.x = bf16_to_f32((bf16_t)(xv.x & 0xffff)) + acc[nb][mb][4 * g + 0];
          o.y = bf16_to_f32((bf16_t)(xv.x >> 16)) + acc[nb][mb][4 * g + 1];
          o.z = bf16_to_f32((bf16_t)(xv.y & 0xffff)) + acc[nb][mb][4 * g + 2];
          o.w = bf16_to_f32((bf16_t)(xv.y >> 16)) + acc[nb][mb][4 * g + 3];
          *reinterpret_cast<float4*>(orow + n) = o;
        }
    }
  }
}

template <int MODE, int BM, int WAVES_M>
void launch_mode(const GemmArgs& a, hipStream_t s) {
  const bool routed = !(a.mode == 2 || (a.mode == 0 && a.shared));
  const int mdim = routed ? a.max_mtiles : (a.T + BM - 1) / BM;
  int ndim;
  if (MODE == 0) {
    const int per_wg = BN / 2;
    ndim = ((a.inner + per_wg - 1) / per_wg) * (routed ? 1 : a.n_experts);
  } else {
    ndim = (a.d + BN - 1) / BN;
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, BM, WAVES_M>), dim3(mdim * ndim),
                     dim3(256), 0, s, a);
}

template <int BM, int WAVES_M>
void launch_bm(const GemmArgs& a, hipStream_t s) {
  if (a.mode == 0) launch_mode<0, BM, WAVES_M>(a, s);
  else if (a.mode == 1) launch_mode<1, BM, WAVES_M>(a, s);
  else launch_mode<2, BM, WAVES_M>(a, s);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s) {
  switch (a.bm) {
    case 256: launch_bm<256, 2>(a, s); break;
    case 128: launch_bm<128, 1>(a, s); break;
    case 64: launch_bm<64, 1>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
