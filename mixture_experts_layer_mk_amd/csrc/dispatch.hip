// Dispatch: per-expert totals and prefix scan over the router's block
// histograms, the GEMM M-tile schedule, and the stable permutation of token
// rows into expert-contiguous order (expert ascending, token ascending).
//
// No token is dropped (DeepSeek-V3 Technical Report summary, "2. Architecture"):
// every (token, kept expert) pair gets exactly one row.
#include "common.h"

namespace moe {

namespace {

// Scan over router blocks, one workgroup per expert: the block's rows for
// expert e start at block_base[e][b] (relative to the expert's first row);
// the expert's total goes to counts[e].  block_counts / block_base are
// [E][nblk] (each expert's blocks contiguous).
__global__ __launch_bounds__(256) void scan_blocks_kernel(ScanArgs a) {
  __shared__ int part[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int per = (a.nblk + 255) / 256;
  const int b0 = min(tid * per, a.nblk), b1 = min(b0 + per, a.nblk);
  const int32_t* bc = a.block_counts + (size_t)e * a.nblk;
  int32_t* bb = a.block_base + (size_t)e * a.nblk;
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += bc[b];
  part[tid] = sum;
  __syncthreads();
  // inclusive scan of the 256 partial sums (Hillis-Steele)
  for (int off = 1; off < 256; off <<= 1) {
    const int v = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;            // exclusive prefix of this thread's range
  for (int b = b0; b < b1; ++b) {
    bb[b] = run;
    run += bc[b];
  }
  if (tid == 255) a.counts[e] = part[255];
}

// Exclusive scan over experts, user counts, and the GEMM M-tile schedule
// (one workgroup; thread e owns expert e, E <= 256).
__global__ __launch_bounds__(256) void scan_experts_kernel(ScanArgs a) {
  __shared__ int tot[MAX_EXPERTS];
  __shared__ int off[MAX_EXPERTS + 1];
  __shared__ int tstart[MAX_EXPERTS + 1];
  const int e = threadIdx.x;
  if (e < a.E) tot[e] = a.counts[e];
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
    const int row = a.offsets[e] + a.block_base[(size_t)e * a.nblk + b] + a.rank[q];
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
  hipLaunchKernelGGL(scan_blocks_kernel, dim3(a.E), dim3(256), 0, s, a);
  hipLaunchKernelGGL(scan_experts_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
