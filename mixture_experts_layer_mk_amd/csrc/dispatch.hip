// Dispatch: per-expert totals and prefix scan over the router's block
// histograms, the GEMM M-tile schedule, and the stable permutation of token
// rows into expert-contiguous order (expert ascending, token ascending).
//
// No token is dropped (DeepSeek-V3 Technical Report summary, "2. Architecture"):
// every (token, kept expert) pair gets exactly one row.
#include "common.h"

namespace moe {

namespace {

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// The whole dispatch scan in one workgroup:
//  (a) per expert, the exclusive prefix of the router blocks' counts: the
//      block's rows for expert e start at block_base[b][e] (relative to the
//      expert's first row); the expert's total goes to counts[e].
//      block_counts / block_base are [nblk][E] (one router block's counts
//      contiguous), so thread (g, e) -- expert e, one of NT / EP groups of
//      consecutive blocks -- reads and writes with the lanes of a wave on
//      consecutive experts.  The groups' sums are scanned through LDS.
//  (b) wave 0: the exclusive scan over experts (offsets) and over their
//      M-tile counts ceil(count / bm) (where each expert's tiles start).
//  (c) the M-tile list, one tile per thread: expert found by binary search
//      over the tile starts.
template <int NT>
__device__ __forceinline__ void dispatch_scan(const ScanArgs& a) {
  __shared__ int tot[MAX_EXPERTS];
  __shared__ int off[MAX_EXPERTS + 1];
  __shared__ int tstart[MAX_EXPERTS + 1];
  __shared__ int part[NT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  int ep = 1;                                   // E rounded up to a power of two
  while (ep < E) ep <<= 1;
  const int ng = NT / ep;                       // block groups (E <= 256 <= NT)
  const int e = tid % ep, g = tid / ep;
  const int per = (a.nblk + ng - 1) / ng;
  const int b0 = min(g * per, a.nblk), b1 = min(b0 + per, a.nblk);
  const bool live = e < E && g < ng;
  const int32_t* __restrict__ bc = a.block_counts;
  int32_t* __restrict__ bb = a.block_base;
  // The first RR counts of the thread's range are loaded at once (one
  // latency) and kept in registers for the second pass; a longer range
  // (more than RR blocks per group) streams the rest.
  constexpr int RR = 16384 / NT;
  int v[RR];
  int sum = 0;
  if (live) {
#pragma unroll
    for (int q = 0; q < RR; ++q) v[q] = b0 + q < b1 ? bc[(size_t)(b0 + q) * E + e] : 0;
#pragma unroll
    for (int q = 0; q < RR; ++q) sum += v[q];
    for (int b = b0 + RR; b < b1; ++b) sum += bc[(size_t)b * E + e];
  }
  part[tid] = sum;
  __syncthreads();
  if (live) {
    int base = 0, total = 0;
    for (int h = 0; h < ng; ++h) {
      const int w = part[h * ep + e];
      base += h < g ? w : 0;
      total += w;
    }
    int run = base;
#pragma unroll
    for (int q = 0; q < RR; ++q) {
      if (b0 + q < b1) bb[(size_t)(b0 + q) * E + e] = run;
      run += v[q];
    }
    for (int b = b0 + RR; b < b1; ++b) {
      const int w = bc[(size_t)b * E + e];
      bb[(size_t)b * E + e] = run;
      run += w;
    }
    if (g == 0) {
      tot[e] = total;
      a.counts[e] = total;
      if (a.user_counts) a.user_counts[e] = total;
    }
  }
  __syncthreads();
  if (wave == 0) {
    int o = 0, ts = 0;
    for (int c = 0; c < a.E; c += 64) {
      const int e = c + lane;
      const int v = e < a.E ? tot[e] : 0;
      const int nt = (v + a.bm - 1) / a.bm;
      const int iv = wave_incl_scan(v), it = wave_incl_scan(nt);
      if (e < a.E) {
        off[e] = o + iv - v;
        tstart[e] = ts + it - nt;
        a.offsets[e] = o + iv - v;
      }
      o += __shfl(iv, 63, 64);
      ts += __shfl(it, 63, 64);
    }
    if (lane == 0) {
      off[a.E] = o;
      tstart[a.E] = ts;
      a.offsets[a.E] = o;
      *a.n_tiles = ts;
    }
  }
  __syncthreads();
  const int n = tstart[a.E];
  for (int i = tid; i < n; i += NT) {
    int lo = 0, hi = a.E - 1;   // last expert with tstart[e] <= i (it has >= 1 tile)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tstart[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int e = lo, j = i - tstart[e];
    MTile t;
    t.expert = e;
    t.row0 = off[e] + j * a.bm;
    t.rows = min(a.bm, tot[e] - j * a.bm);
    t.pad = 0;
    a.tiles[i] = t;
  }
}

constexpr int SCAN_THREADS = 1024;   // one workgroup, 16 waves

__global__ __launch_bounds__(SCAN_THREADS) void scan_kernel(ScanArgs a) {
  dispatch_scan<SCAN_THREADS>(a);
}

// Slot q = (token, slot): its row is the expert's first row, plus the rows
// of the expert in earlier router blocks, plus the slot's rank among the
// expert's slots in its own block (token order).  Writes the two row maps.
__device__ __forceinline__ void permute_slot(const PermuteArgs& a, int q) {
  const int t = q / a.K;
  const int b = t / a.rt;
  const int e = a.topk_idx[q];
  const int row = a.offsets[e] + a.block_base[(size_t)b * a.E + e] + a.rank[q];
  a.slot_row[q] = row;
  a.row_src[row] = t;
}

// One thread per slot.
__global__ __launch_bounds__(256) void permute_kernel(PermuteArgs a) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q < a.T * a.K) permute_slot(a, q);
}

// Small batches: the scan, then the permute by the same workgroup (one
// launch fewer on a latency-bound path).  The barrier makes the scan's
// offsets and block bases, written to global memory, visible to the
// workgroup's threads.
__global__ __launch_bounds__(SCAN_THREADS) void scan_permute_kernel(ScanArgs a, PermuteArgs p) {
  dispatch_scan<SCAN_THREADS>(a);
  __syncthreads();
  for (int q = threadIdx.x; q < p.T * p.K; q += SCAN_THREADS) permute_slot(p, q);
}

// counts[0 .. n) = 0 (a forward with no tokens still reports its counts).
__global__ __launch_bounds__(256) void zero_counts_kernel(int32_t* counts, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) counts[i] = 0;
}

}  // namespace

hipError_t launch_zero_counts(int32_t* counts, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_counts_kernel, dim3((n + 255) / 256), dim3(256), 0, s, counts, n);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s, const PermuteArgs* p) {
  if (p && (int64_t)p->T * p->K > SCAN_PERMUTE_MAX_SLOTS) return hipErrorInvalidValue;
  if (p) hipLaunchKernelGGL(scan_permute_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, a, *p);
  else hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.T * a.K;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
