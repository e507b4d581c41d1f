// Dispatch: per-expert totals and prefix scan over the router's block
// histograms, the GEMM M-tile schedule, and the stable permutation of token
// rows into expert-contiguous order (expert ascending, token ascending).
//
// No token is dropped (DeepSeek-V3 Technical Report summary, "2. Architecture"):
// every (token, kept expert) pair gets exactly one row.
#include "common.h"

namespace moe {

namespace {

// One workgroup; thread e owns expert e (E <= 256).
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  __shared__ int tot[MAX_EXPERTS];
  __shared__ int off[MAX_EXPERTS + 1];
  __shared__ int tstart[MAX_EXPERTS + 1];
  const int e = threadIdx.x;
  if (e < a.E) {
    int run = 0;
#pragma unroll 8
    for (int b = 0; b < a.nblk; ++b) {
      const size_t o = (size_t)b * a.E + e;
      const int c = a.block_counts[o];
      a.block_base[o] = run;      // rows of earlier blocks for this expert
      run += c;
    }
    tot[e] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int o = 0, ts = 0;
    for (int q = 0; q < a.E; ++q) {
      off[q] = o;
      tstart[q] = ts;
      o += tot[q];
      ts += (tot[q] + a.bm - 1) / a.bm;
    }
    off[a.E] = o;
    tstart[a.E] = ts;
  }
  __syncthreads();
  if (e < a.E) {
    const int c = tot[e];
    a.counts[e] = c;
    if (a.user_counts) a.user_counts[e] = c;
    a.offsets[e] = off[e];
    const int nt = tstart[e + 1] - tstart[e];
    for (int i = 0; i < nt; ++i) {
      MTile t;
      t.expert = e;
      t.row0 = off[e] + i * a.bm;
      t.rows = min(a.bm, c - i * a.bm);
      t.pad = 0;
      a.tiles[tstart[e] + i] = t;
    }
  }
  if (threadIdx.x == 0) {
    a.offsets[a.E] = off[a.E];
    *a.n_tiles = tstart[a.E];
  }
}

// One wave per token: compute the K destination rows, record the maps, and
// copy the token's row into each of them (16-byte vectors).
__global__ __launch_bounds__(256) void permute_kernel(PermuteArgs a) {
  const int t = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (t >= a.T) return;
  const int b = t / a.rt;
  const int esz = a.dtype == 1 ? 2 : 4;
  const int nvec = a.d * esz / 16;
  const uint4* src = reinterpret_cast<const uint4*>(
      static_cast<const char*>(a.x) + (size_t)t * a.d * esz);
  for (int k = 0; k < a.K; ++k) {
    const int q = t * a.K + k;
    const int e = a.topk_idx[q];
    const int row = a.offsets[e] + a.block_base[(size_t)b * a.E + e] + a.rank[q];
    if (lane == 0) {
      a.slot_row[q] = row;
      a.row_src[row] = t;
    }
    if (a.xp) {
      uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(a.xp) +
                                            (size_t)row * a.d * esz);
      for (int v = lane; v < nvec; v += 64) dst[v] = src[v];
    }
  }
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
