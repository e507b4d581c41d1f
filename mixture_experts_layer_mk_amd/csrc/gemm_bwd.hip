// Grouped GEMMs of the layer's backward pass on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation, fp32 results).
//
// The backward needs products whose reduction runs along the strided
// dimension of an operand: the weights in the input gradients (dy W2, dA W1)
// and the token rows in the weight gradients (dy^T H, dA^T X).  Such an
// operand is "mn-major": a row in memory holds consecutive m (or n) for one
// k.  Its tiles go global -> LDS unchanged (64 k-rows of 256 values, 16-byte
// direct loads), and the matrix operand fragments come out of LDS through
// the transpose loads (ds_read_b64_tr_b16): in each group of 16 lanes,
// source lane 4j + q reads 4 consecutive m of k-row j, and lane i receives
// the 4 values of k-rows 0..3 at m = 4 (i / 4) + i % 4 -- one 16 (m) x 4 (k)
// block turned into the k-consecutive layout the matrix op wants.  Two such
// loads give a lane its 8 k-values.  k-major operands (rows hold consecutive
// k) use the same tiles as the forward GEMMs.
//
// Tile: 256 (M) x 256 (N) per workgroup of 4 waves (2 x 2, 128 x 128 each),
// k in steps of 64, LDS double-buffered (2 x 64 KB), operand fragments
// double-buffered in registers as in the forward kernels.
#include "gemm_common.h"

namespace moe {

namespace {

using namespace gemm;

constexpr int TM = 256;     // tile rows (M)
constexpr int TK = 64;      // k per stage

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Chunk swizzle of mn-major LDS rows (32 chunks of 16 B per k-row).  Half a
// wave's transpose load (32 lanes, 256 B) reads 4 consecutive k-rows
// (k = 0..3 mod 4) times 4 consecutive chunks (a 4-aligned group); XOR-ing
// the chunk with 4 (k mod 4) puts those 16 chunks on 16 different 16-byte
// bank groups (one full pass over the banks, no conflict).
__device__ __forceinline__ int swz_mn(int k) { return (k & 3) << 2; }

// A 32 (mn) x 16 (k) operand fragment for the matrix op from an mn-major
// LDS tile (64 k-rows x 32 chunks): lanes 0-31 hold mn = base + lane % 32 at
// k = 16 kk + 0..7, lanes 32-63 the same mn at k + 8.
__device__ __forceinline__ bf16x8 frag_mn(const u32x4* T, int base, int kk, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int mn = base + 16 * (g & 1) + 4 * (s & 3);
  const int chunk = mn >> 3, half = (mn >> 2) & 1;
  const int k0 = kk * 16 + 8 * (g >> 1) + (s >> 2);
  const char* t = reinterpret_cast<const char*>(T);
  const int o0 = k0 * 512 + ((chunk ^ swz_mn(k0)) << 4) + half * 8;
  const int k1 = k0 + 4;
  const int o1 = k1 * 512 + ((chunk ^ swz_mn(k1)) << 4) + half * 8;
  const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + o0));
  const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + o1));
  const v4s r[2] = {r0, r1};
  return __builtin_bit_cast(bf16x8, r);
}

// Where one tile's operands and results live.
struct TileDesc {
  int m0, n0;           // tile origin in the group's M x N
  int mval, nval;       // valid extent of M and N in the group (masks)
  int K;                // reduction length (k-rows for mn-major operands)
  int grp;              // expert (routed) or shared expert / 0
  int row0;             // KIND 0/1: first row of the tile (expert-contiguous)
  int koff;             // KIND 2/3 routed: first row of the expert
  int kbeg, split;      // KIND 2/3: first k-row of this split, split index
};

template <int KIND, bool SH>
__device__ __forceinline__ bool decode(const BwdGemmArgs& a, TileDesc& t) {
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  if (KIND == 0 || KIND == 1) {
    const int per = (KIND == 0) ? (a.inner + BN - 1) / BN : (a.d + BN - 1) / BN;
    const int ndim = (KIND == 0 && SH) ? per * a.n_experts : per;
    const int mt = L / ndim, nt = L % ndim;
    if (!SH) {
      if (mt >= *a.n_tiles) return false;
      const MTile m = a.tiles[mt];
      t.row0 = m.row0; t.mval = m.rows; t.grp = m.expert;
    } else {
      t.row0 = mt * TM; t.mval = min(TM, a.T - t.row0); t.grp = (KIND == 0) ? nt / per : 0;
    }
    t.m0 = 0;
    t.n0 = (nt % per) * BN;
    t.nval = (KIND == 0) ? a.inner : a.d;
    t.K = (KIND == 0) ? a.d : (SH ? 2 * a.inner * a.n_experts : 2 * a.inner);
    t.koff = 0; t.kbeg = 0; t.split = 0;
  } else {
    const int M = (KIND == 2) ? a.d : 2 * a.inner;
    const int N = (KIND == 2) ? a.inner : a.d;
    const int mdim = (M + TM - 1) / TM, ndim = (N + BN - 1) / BN;
    const int per_split = a.n_experts * mdim * ndim;
    t.split = L / per_split;
    const int L2 = L % per_split;
    t.grp = L2 / (mdim * ndim);
    const int rem = L2 % (mdim * ndim);
    t.m0 = (rem / ndim) * TM; t.n0 = (rem % ndim) * BN;
    t.mval = M; t.nval = N;
    int k_all;
    if (SH) { t.koff = 0; k_all = a.T; }
    else { t.koff = a.offsets[t.grp]; k_all = a.offsets[t.grp + 1] - t.koff; }
    // k-rows [kbeg, kbeg + K) of the group: split s of `splits` takes a
    // range of whole k-blocks
    const int kc = ((k_all + a.splits * TK - 1) / (a.splits * TK)) * TK;
    t.kbeg = min(t.split * kc, k_all);
    t.K = min(kc, k_all - t.kbeg);
    t.row0 = 0;
  }
  return true;
}

template <int KIND, bool SH>
__global__ __launch_bounds__(256, 1) void gemm_bwd_kernel(BwdGemmArgs a) {
  __shared__ u32x4 As0[2048], As1[2048];   // 32 KB each: 256 x 8 or 64 x 32 chunks
  __shared__ u32x4 Bs0[2048], Bs1[2048];

  TileDesc t;
  if (!decode<KIND, SH>(a, t)) return;

  constexpr bool AK = (KIND == 0 || KIND == 1);   // A k-major; B is always mn-major
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const int nk = (t.K + TK - 1) / TK;

  // ---- k-major A (KIND 0, 1): 256 rows x 8 chunks per stage ----
  // Lane slot: LDS row (wave * 8 + j) * 8 + lr, chunk (lane & 7) after the
  // row swizzle, as in the forward kernels.  Element offsets from the
  // operand's base (32 bits: validation bounds every operand below 2^32
  // elements); each stage adds k0.
  const int lr = lane >> 3;
  const int cg0 = (lane & 7) ^ lr, cg1 = cg0 ^ 1;
  const bf16_t* abase = nullptr;
  uint32_t aoff[8];
  if constexpr (AK) {
    int ld;
    if (KIND == 0) { abase = a.dy; ld = a.d; }
    else { abase = a.da; ld = a.ldda; }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = wave * 8 + j;
      const int r = min(blk * 8 + lr, t.mval - 1);
      // routed dy rows: the row's token (a gather resolved once per tile)
      const int row = (KIND == 0 && !SH) ? a.row_src[t.row0 + r] : t.row0 + r;
      aoff[j] = (uint32_t)row * (uint32_t)ld + ((blk & 1) ? cg1 : cg0) * 8;
    }
  }

  // ---- mn-major operands: 64 k-rows x 32 chunks per stage ----
  // Lane slot: k-row kr_j = 2 (wave * 8 + j) + (lane >> 5), chunk (lane & 31),
  // which holds global chunk (lane & 31) ^ swz_mn(kr_j) of that row (the
  // tile's first chunk past the operand's last column: never stored).  The
  // offset of the lane's chunk inside the stage's first k-row is fixed; a
  // stage adds its uniform row base, and k-rows past the end read zeros.
  const int ks = lane >> 5, cs = lane & 31;
  auto mn_off = [&](int j, int col0, int extent, int ld) -> uint32_t {
    const int kr = 2 * (wave * 8 + j) + ks;
    int c = cs ^ swz_mn(kr);
    if (col0 + c * 8 >= extent) c = 0;
    return (uint32_t)kr * (uint32_t)ld + (uint32_t)(col0 + c * 8);
  };
  uint32_t moff_a[8], moff_b[8];
  int lda_mn = 0, ldb_mn;
  if (KIND == 0) ldb_mn = a.inner;
  else if (KIND == 1) ldb_mn = a.d;
  else if (KIND == 2) { lda_mn = a.d; ldb_mn = a.ldhg; }
  else { lda_mn = a.ldda; ldb_mn = a.d; }
  // Routed weight gradients read one operand's k-rows from token rows (dy
  // for KIND 2's A, x for KIND 3's B): that operand's offsets hold only the
  // column part, and the tokens of the next stage's k-rows are loaded one
  // stage ahead (the wait before each stage's barrier covers them).
  constexpr bool gath = (KIND == 2 || KIND == 3) && !SH;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (!AK) moff_a[j] = mn_off(j, t.m0, t.mval, (KIND == 2 && gath) ? 0 : lda_mn);
    moff_b[j] = mn_off(j, t.n0, t.nval, (KIND == 3 && gath) ? 0 : ldb_mn);
  }
  int tok[8];
  auto load_tokens = [&](int kb) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = kb * TK + 2 * (wave * 8 + j) + ks;
      tok[j] = (k < t.K) ? a.row_src[t.koff + t.kbeg + k] : 0;
    }
  };
  if constexpr (gath) {
    if (nk > 0) load_tokens(0);
  }
  // uniform base of the stage's first k-row (k0 relative to the tile's k range)
  auto a_stage = [&](int k0) -> const bf16_t* {
    const size_t row = (size_t)t.koff + t.kbeg + k0;
    if (KIND == 2) return SH ? a.dy + row * a.d : a.dy;     // routed: gathered
    return a.da + row * a.ldda + (SH ? (size_t)t.grp * 2 * a.inner : 0);   // KIND 3
  };
  auto b_stage = [&](int k0) -> const bf16_t* {
    if (KIND == 0) return a.w2 + ((size_t)t.grp * a.d + k0) * a.inner;
    if (KIND == 1) {
      const int per = 2 * a.inner;
      const int e = SH ? k0 / per : t.grp;
      const int r = SH ? k0 % per : k0;
      const bf16_t* w = (r < a.inner) ? a.w1 : a.w3;
      return w + ((size_t)e * a.inner + (r % a.inner)) * a.d;
    }
    const size_t row = (size_t)t.koff + t.kbeg + k0;
    if (KIND == 2) return a.hg + row * a.ldhg + (SH ? (size_t)t.grp * a.inner : 0);
    return SH ? a.x + row * a.d : a.x;                      // KIND 3; routed: gathered
  };

  auto issue = [&](int kb, u32x4* Ab, u32x4* Bb) {
    const int k0 = kb * TK;
    const bf16_t* zr = a.zero + cs * 8;
    const bf16_t* as = nullptr;
    if constexpr (!AK) as = a_stage(k0);
    const bf16_t* bs = b_stage(k0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = wave * 8 + j;
      const bool live = k0 + 2 * blk + ks < t.K;   // k-major A: K is whole stages
      const uint32_t trow = (uint32_t)tok[j] * (uint32_t)a.d;
      const bf16_t* ga;
      if constexpr (AK) ga = abase + aoff[j] + k0;
      else ga = live ? as + moff_a[j] + ((KIND == 2 && gath) ? trow : 0u) : zr;
      __builtin_amdgcn_global_load_lds((const glb_void*)ga, (lds_void*)&Ab[blk * 64], 16, 0, 0);
      const bf16_t* gb = live ? bs + moff_b[j] + ((KIND == 3 && gath) ? trow : 0u) : zr;
      __builtin_amdgcn_global_load_lds((const glb_void*)gb, (lds_void*)&Bb[blk * 64], 16, 0, 0);
    }
    if constexpr (gath) load_tokens(min(kb + 1, nk - 1));    // the next stage issued
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
  auto load_frags = [&](bf16x8* fa, bf16x8* fb, const u32x4* Ab, const u32x4* Bb, int kk) {
    const int c = 2 * kk + hi;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if constexpr (AK) {
        const int r = wm * 128 + mb * 32 + l32;
        fa[mb] = __builtin_bit_cast(bf16x8, Ab[r * 8 + (c ^ swz_x(r))]);
      } else {
        fa[mb] = frag_mn(Ab, wm * 128 + mb * 32, kk, lane);
      }
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) fb[nb] = frag_mn(Bb, wn * 128 + nb * 32, kk, lane);
  };
  auto mma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nb], fa[mb], acc[nb][mb],
                                                             0, 0, 0);
  };
  constexpr int N_DS = (AK ? 4 : 8) + 8;
  auto sched_ds = [&]() { sched_groups<16, N_DS, 0>(); };
  auto sched_ds_vm = [&]() { sched_groups<16, N_DS, 16>(); };

  // Same pipeline as the forward kernels: block kb from (Ac, Bc) while kb+1
  // streams into (An, Bn); kb+2 is issued into (Ac, Bc) once every wave
  // holds its last fragments of kb.  Blocks past the end re-load the last.
  auto block = [&](int next2, u32x4* Ac, u32x4* Bc, const u32x4* An, const u32x4* Bn) {
    load_frags(fa1, fb1, Ac, Bc, 1);
    mma(fa0, fb0);
    sched_ds();
    load_frags(fa0, fb0, Ac, Bc, 2);
    mma(fa1, fb1);
    sched_ds();
    load_frags(fa1, fb1, Ac, Bc, 3);
    mma(fa0, fb0);
    sched_ds();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    issue(next2, Ac, Bc);
    load_frags(fa0, fb0, An, Bn, 0);
    mma(fa1, fb1);
    sched_ds_vm();
  };

  if (nk > 0) {
    issue(0, As0, Bs0);
    issue(min(1, nk - 1), As1, Bs1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<16>());
    __syncthreads();
    load_frags(fa0, fb0, As0, Bs0, 0);
    int kb = 0;
    for (; kb + 2 <= nk; kb += 2) {
      block(min(kb + 2, nk - 1), As0, Bs0, As1, Bs1);
      block(min(kb + 3, nk - 1), As1, Bs1, As0, Bs0);
    }
    if (kb < nk) block(nk - 1, As0, Bs0, As1, Bs1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load left in flight
  }

  // ---- epilogue: acc[nb][mb][r] = C[m][n], m = mb*32 + l32 and
  // n = nb*32 + 8*(r/4) + 4*hi + r%4 inside the wave's 128 x 128 ----
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = t.m0 + wm * 128 + mb * 32 + l32;
    if (m >= t.mval) continue;
    float* crow;
    if (KIND == 0) {
      const size_t col = SH ? (size_t)t.grp * a.inner : 0;
      crow = a.c + (size_t)(t.row0 + m) * a.ldc + col;
    } else if (KIND == 1) {
      crow = a.c + (size_t)(t.row0 + m) * a.ldc;
    } else if (a.splits > 1) {   // partial sums [split][group][M][N], reduced later
      crow = a.part + (((size_t)t.split * a.n_experts + t.grp) * t.mval + m) * t.nval;
    } else if (KIND == 2) {
      crow = a.dw2 + ((size_t)t.grp * a.d + m) * a.inner;
    } else {
      crow = (m < a.inner) ? a.dw1 + ((size_t)t.grp * a.inner + m) * a.d
                           : a.dw3 + ((size_t)t.grp * a.inner + (m - a.inner)) * a.d;
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = t.n0 + wn * 128 + nb * 32 + 8 * g + 4 * hi;
        if (n >= t.nval) continue;
        float4 v;
        v.x = acc[nb][mb][4 * g + 0];
        v.y = acc[nb][mb][4 * g + 1];
        v.z = acc[nb][mb][4 * g + 2];
        v.w = acc[nb][mb][4 * g + 3];
        *reinterpret_cast<float4*>(crow + n) = v;
      }
  }
}

// Sum of the split-k partials of a weight gradient, splits in order, into
// the gradient's own layout (4 consecutive elements per thread).
template <int KIND>
__global__ __launch_bounds__(256) void split_reduce_kernel(BwdGemmArgs a) {
  const int M = (KIND == 2) ? a.d : 2 * a.inner;
  const int N = (KIND == 2) ? a.inner : a.d;
  const int64_t per = (int64_t)M * N;
  const int64_t n = (int64_t)a.n_experts * per;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  float4 v = *reinterpret_cast<const float4*>(a.part + i);
  for (int sp = 1; sp < a.splits; ++sp) {
    const float4 w = *reinterpret_cast<const float4*>(a.part + (size_t)sp * n + i);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  const int64_t g = i / per, r = i % per;
  const int m = (int)(r / N), c = (int)(r % N);
  float* dst;
  if (KIND == 2) dst = a.dw2 + ((size_t)g * a.d + m) * a.inner + c;
  else dst = (m < a.inner) ? a.dw1 + ((size_t)g * a.inner + m) * a.d + c
                           : a.dw3 + ((size_t)g * a.inner + (m - a.inner)) * a.d + c;
  *reinterpret_cast<float4*>(dst) = v;
}

template <int KIND, bool SH>
void launch_kind(const BwdGemmArgs& a, hipStream_t s) {
  int grid;
  if (KIND == 0 || KIND == 1) {
    const int per = (KIND == 0) ? (a.inner + BN - 1) / BN : (a.d + BN - 1) / BN;
    const int ndim = (KIND == 0 && a.shared) ? per * a.n_experts : per;
    const int mdim = a.shared ? (a.T + TM - 1) / TM : a.max_mtiles;
    grid = mdim * ndim;
  } else {
    const int M = (KIND == 2) ? a.d : 2 * a.inner;
    const int N = (KIND == 2) ? a.inner : a.d;
    grid = a.splits * a.n_experts * ((M + TM - 1) / TM) * ((N + BN - 1) / BN);
  }
  if (grid <= 0) return;
  hipLaunchKernelGGL((gemm_bwd_kernel<KIND, SH>), dim3(grid), dim3(256), 0, s, a);
  if ((KIND == 2 || KIND == 3) && a.splits > 1) {
    const int M = (KIND == 2) ? a.d : 2 * a.inner;
    const int N = (KIND == 2) ? a.inner : a.d;
    const int64_t n = (int64_t)a.n_experts * M * N;
    hipLaunchKernelGGL(split_reduce_kernel<KIND>, dim3((unsigned)((n / 4 + 255) / 256)),
                       dim3(256), 0, s, a);
  }
}

}  // namespace

hipError_t launch_gemm_bwd(const BwdGemmArgs& a, hipStream_t s) {
  switch (a.kind * 2 + (a.shared ? 1 : 0)) {
    case 0: launch_kind<0, false>(a, s); break;
    case 1: launch_kind<0, true>(a, s); break;
    case 2: launch_kind<1, false>(a, s); break;
    case 3: launch_kind<1, true>(a, s); break;
    case 4: launch_kind<2, false>(a, s); break;
    case 5: launch_kind<2, true>(a, s); break;
    case 6: launch_kind<3, false>(a, s); break;
    case 7: launch_kind<3, true>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
