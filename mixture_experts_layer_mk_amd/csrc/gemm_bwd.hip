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
#include <type_traits>

#include "gemm_common.h"

namespace moe {

namespace {

using namespace gemm;

constexpr int TM = 256;     // tile rows (M)
constexpr int TK = 32;      // k per stage
constexpr int NS = 4;       // stages in the LDS ring: NS - 1 in flight while one is computed

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float fv4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Chunk swizzle of mn-major LDS rows (32 chunks of 16 B per k-row).  Half a
// wave's transpose load (32 lanes, 256 B) reads 4 consecutive k-rows
// (k = 0..3 mod 4) times 4 consecutive chunks (a 4-aligned group); XOR-ing
// the chunk with 4 (k mod 4) puts those 16 chunks on 16 different 16-byte
// bank groups (one full pass over the banks, no conflict).
__device__ __forceinline__ int swz_mn(int k) { return (k & 3) << 2; }

// A 32 (mn) x 16 (k) operand fragment for the matrix op from an mn-major
// LDS tile (32 k-rows x 32 chunks): lanes 0-31 hold mn = base + lane % 32 at
// k = 16 kk + 0..7, lanes 32-63 the same mn at k + 8.  With base = 128 w +
// 32 i, lane (g = lane / 16, s = lane % 16) reads 4 consecutive mn at k-rows
// k0 = 16 kk + 8 (g / 2) + s / 4 and k0 + 4, chunk 16 w + 4 i + 2 (g % 2) +
// (s % 4) / 2, half s % 2.  The chunk swizzle 4 (k0 mod 4) = 4 (s / 4) only
// flips bits 2-3, the bits of i, so the byte offset is a lane term for each
// i plus 8192 kk (+ 2048 for the second k-row): the lane terms are computed
// once per tile and the k-step parts are instruction immediates.
__device__ __forceinline__ uint32_t frag_mn_off(int w, int i, int lane) {
  const int g = lane >> 4, s = lane & 15, q = s >> 2;
  const int chunk = 16 * w + ((i ^ q) << 2) + 2 * (g & 1) + ((s & 3) >> 1);
  return (uint32_t)((8 * (g >> 1) + q) * 512 + (chunk << 4) + (s & 1) * 8);
}

template <int KK>
__device__ __forceinline__ bf16x8 frag_mn(const u32x4* T, uint32_t off) {
  const char* t = reinterpret_cast<const char*>(T) + off + KK * 8192;
  const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)t);
  const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(t + 2048));
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
  if (KIND == 0 || KIND == 1) {
    const int per = (KIND == 0) ? (a.inner + BN - 1) / BN : (a.d + BN - 1) / BN;
    const int ndim = (KIND == 0 && SH) ? per * a.n_experts : per;
    // Routed launches are sized for the most M-tiles any routing can make;
    // tiles are numbered over the ones it did make (the blocks past them
    // exit), so every XCD gets an equal share of real tiles.
    const int nreal = SH ? (int)gridDim.x : *a.n_tiles * ndim;
    if ((int)blockIdx.x >= nreal) return false;
    const int L = xcd_remap(blockIdx.x, nreal);
    const int mt = L / ndim, nt = L % ndim;
    if (!SH) {
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
    const int L = xcd_remap(blockIdx.x, gridDim.x);
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
  // The LDS ring: NS stages of A and B, 16 KB each (256 x 4 or 32 x 32
  // chunks).  Distinct objects, so that the compiler's waits for the direct
  // loads tell the stages apart.
  __shared__ u32x4 A0[1024], A1[1024], A2[NS > 2 ? 1024 : 1], A3[NS > 3 ? 1024 : 1], A4[NS > 4 ? 1024 : 1];
  __shared__ u32x4 B0[1024], B1[1024], B2[NS > 2 ? 1024 : 1], B3[NS > 3 ? 1024 : 1], B4[NS > 4 ? 1024 : 1];

  TileDesc t;
  if (!decode<KIND, SH>(a, t)) return;

  constexpr bool AK = (KIND == 0 || KIND == 1);   // A k-major; B is always mn-major
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform: the LDS destinations of the direct loads stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const int nk = (t.K + TK - 1) / TK;

  // ---- k-major A (KIND 0, 1): 256 rows x 4 chunks per stage ----
  // Direct load j of the wave fills LDS slots (4 wave + j) 64 + lane: row
  // (4 wave + j) 16 + lane / 4, slot chunk lane % 4, which holds global
  // chunk (lane % 4) ^ swz_k(row).  Element offsets from the operand's base
  // (validation keeps every activation below 2^31 elements); a stage adds k0.
  const bf16_t* abase = nullptr;
  uint32_t aoff[4];
  if constexpr (AK) {
    int ld;
    if (KIND == 0) { abase = a.dy; ld = a.d; }
    else { abase = a.da; ld = a.ldda; }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (wave * 4 + j) * 16 + (lane >> 2);
      const int rc = min(r, t.mval - 1);
      // routed dy rows: the row's token (a gather resolved once per tile)
      const int row = (KIND == 0 && !SH) ? a.row_src[t.row0 + rc] : t.row0 + rc;
      aoff[j] = (uint32_t)row * (uint32_t)ld + (uint32_t)(((lane & 3) ^ swz_k(r)) * 8);
    }
  }

  // ---- mn-major operands: 32 k-rows x 32 chunks per stage ----
  // Direct load j fills k-row kr_j = 2 (4 wave + j) + (lane >> 5), slot
  // chunk (lane & 31), which holds global chunk (lane & 31) ^ swz_mn(kr_j)
  // of that row (the tile's first chunk past the operand's last column: never
  // stored).  The lane's offset inside the stage's first k-row is fixed; a
  // stage adds its uniform row base, and k-rows past the end read zeros.
  const int ks = lane >> 5, cs = lane & 31;
  auto mn_off = [&](int j, int col0, int extent, int ld) -> uint32_t {
    const int kr = 2 * (wave * 4 + j) + ks;
    int c = cs ^ swz_mn(kr);
    if (col0 + c * 8 >= extent) c = 0;
    return (uint32_t)kr * (uint32_t)ld + (uint32_t)(col0 + c * 8);
  };
  uint32_t moff_a[4], moff_b[4];
  int lda_mn = 0, ldb_mn;
  if (KIND == 0) ldb_mn = a.inner;
  else if (KIND == 1) ldb_mn = a.d;
  else if (KIND == 2) { lda_mn = a.d; ldb_mn = a.ldhg; }
  else { lda_mn = a.ldda; ldb_mn = a.d; }
  // Routed weight gradients read one operand's k-rows from token rows (dy
  // for KIND 2's A, x for KIND 3's B): that operand's offsets hold only the
  // column part, and each stage adds its k-rows' tokens.
  constexpr bool gath = (KIND == 2 || KIND == 3) && !SH;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (!AK) moff_a[j] = mn_off(j, t.m0, t.mval, (KIND == 2 && gath) ? 0 : lda_mn);
    moff_b[j] = mn_off(j, t.n0, t.nval, (KIND == 3 && gath) ? 0 : ldb_mn);
  }
  // The tokens of a stage's k-rows: wave-uniform addresses, read through the
  // scalar cache, so that their wait is the LDS counter's, not the direct
  // loads'.  A block reads the tokens of the stage it issues at its start;
  // the wait before its barrier covers them.
  const __attribute__((address_space(4))) int32_t* rsrc = nullptr;
  if constexpr (gath)
    rsrc = (const __attribute__((address_space(4))) int32_t*)(a.row_src + t.koff + t.kbeg);
  struct Tok { int t0[4], t1[4]; };   // tokens of k-rows 2 (4 wave + j) and 2 (4 wave + j) + 1
  auto load_tok = [&](int kb) {
    Tok tk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tk.t0[j] = tk.t1[j] = 0;
      if constexpr (gath) {
        const int k = kb * TK + 2 * (wave * 4 + j);
        // k-rows past the end read the last token (never used: zero rows)
        tk.t0[j] = rsrc[min(k, t.K - 1)];
        tk.t1[j] = rsrc[min(k + 1, t.K - 1)];
      }
    }
    return tk;
  };
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

  // Direct loads of stage kb into (Ab, Bb): 4 + 4 per wave.  Stages past the
  // end load the zero row (their buffers are never read).
  auto issue = [&](int kb, u32x4* Ab, u32x4* Bb, const Tok& tk) {
    const int k0 = kb * TK;
    const bool stage_live = k0 < t.K;
    const int kc = stage_live ? k0 : 0;   // keeps the unused stage bases in range
    const bf16_t* zr = a.zero + cs * 8;
    const bf16_t* as = nullptr;
    if constexpr (!AK) as = a_stage(kc);
    const bf16_t* bs = b_stage(kc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int blk = wave * 4 + j;
      const bool live = k0 + 2 * blk + ks < t.K;
      uint32_t trow = 0;
      if constexpr (gath) trow = (uint32_t)(ks ? tk.t1[j] : tk.t0[j]) * (uint32_t)a.d;
      const bf16_t* ga;
      if constexpr (AK) ga = stage_live ? abase + aoff[j] + k0 : zr;   // K is whole stages
      else ga = live ? as + moff_a[j] + ((KIND == 2 && gath) ? trow : 0u) : zr;
      __builtin_amdgcn_global_load_lds((const glb_void*)ga, (lds_void*)&Ab[blk * 64], 16, 0, 0);
      const bf16_t* gb = live ? bs + moff_b[j] + ((KIND == 3 && gath) ? trow : 0u) : zr;
      __builtin_amdgcn_global_load_lds((const glb_void*)gb, (lds_void*)&Bb[blk * 64], 16, 0, 0);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Byte offsets of the lane's fragments inside an LDS buffer at k-step 0.
  // k-major A: row r = 128 wm + 32 mb + l32 holds k-step kk's chunk
  // (2 kk + hi) ^ swz_k(r) at byte 64 r + 16 chunk; swz_k(r) depends only on
  // l32, so one lane term per kk with 2048 mb as an immediate.
  uint32_t fo_a[4], fo_b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (AK) {
      const int r = wm * 128 + l32;
      fo_a[i] = (uint32_t)(r * 64 + ((((2 * i + hi) & 3) ^ swz_k(r)) << 4));
    } else {
      fo_a[i] = frag_mn_off(wm, i, lane);
    }
    fo_b[i] = frag_mn_off(wn, i, lane);
  }
  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
  auto load_frags = [&](bf16x8* fa, bf16x8* fb, const u32x4* Ab, const u32x4* Bb, auto kk_c) {
    constexpr int kk = decltype(kk_c)::value;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if constexpr (AK) {
        const char* p = reinterpret_cast<const char*>(Ab) + fo_a[kk] + mb * 2048;
        fa[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
      } else {
        fa[mb] = frag_mn<kk>(Ab, fo_a[mb]);
      }
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) fb[nb] = frag_mn<kk>(Bb, fo_b[nb]);
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  auto mma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nb], fa[mb], acc[nb][mb],
                                                             0, 0, 0);
  };
  constexpr int N_DS = (AK ? 4 : 8) + 8;
  constexpr int N_VM = 8;   // direct loads per stage and wave

  // Stage kb from (Ac, Bc); stage kb+1 is in (An, Bn) or streaming into it,
  // with the NS - 2 stages after it.  Half-way through (every wave holds its
  // last fragments of kb), the wait for stage kb+1 and the barrier; then
  // stage kb+NS streams into (Ac, Bc) while the second half runs.
  auto block = [&](int kb, u32x4* Ac, u32x4* Bc, const u32x4* An, const u32x4* Bn) {
    const Tok tk = load_tok(kb + NS);
    load_frags(fa1, fb1, Ac, Bc, K1{});
    mma(fa0, fb0);
    sched_groups<16, N_DS, 0>();
    stage_sync<(NS - 2) * N_VM>();
    issue(kb + NS, Ac, Bc, tk);
    load_frags(fa0, fb0, An, Bn, K0{});
    mma(fa1, fb1);
    sched_groups<16, N_DS, N_VM>();
  };

  if (nk > 0) {
    Tok tp[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) tp[i] = load_tok(i);
    issue(0, A0, B0, tp[0]);
    issue(1, A1, B1, tp[1]);
    if constexpr (NS > 2) issue(2, A2, B2, tp[2]);
    if constexpr (NS > 3) issue(3, A3, B3, tp[3]);
    if constexpr (NS > 4) issue(4, A4, B4, tp[4]);
    stage_sync<(NS - 1) * N_VM>();   // stage 0 landed
    load_frags(fa0, fb0, A0, B0, K0{});
    // NS blocks per iteration, each with its own static buffers.  Stages
    // past the tile's end (at most NS - 1, in the last iteration) hold zero
    // rows and add nothing; running them keeps the loop free of branches.
    for (int kb = 0; kb < nk; kb += NS) {
      block(kb, A0, B0, A1, B1);
      if constexpr (NS == 2) {
        block(kb + 1, A1, B1, A0, B0);
      } else {
        block(kb + 1, A1, B1, A2, B2);
        if constexpr (NS == 3) {
          block(kb + 2, A2, B2, A0, B0);
        } else {
          block(kb + 2, A2, B2, A3, B3);
          if constexpr (NS == 4) {
            block(kb + 3, A3, B3, A0, B0);
          } else {
            block(kb + 3, A3, B3, A4, B4);
            block(kb + 4, A4, B4, A0, B0);
          }
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load left in flight
  }

  // ---- epilogue: acc[nb][mb][r] = C[m][n], m = mb*32 + l32 and
  // n = nb*32 + 8*(r/4) + 4*hi + r%4 inside the wave's 128 x 128.  A lane
  // holds one row, so direct stores would write 32 bytes into each of 32
  // rows per instruction.  Each 32 x 64 half block (one mb, two nb) goes
  // through the wave's own LDS buffer instead (rows padded to 68 floats) and
  // leaves in whole row segments: the rows' input gradients (KIND 1) rounded
  // to bf16, 8 columns per lane; G and the weight gradients in fp32, 4
  // columns per lane.  The buffers are free once every wave has passed the
  // barrier (each wave's direct loads have completed above); a wave's LDS
  // operations run in order, so the buffers need no further barrier. ----
  __syncthreads();
  constexpr int SP = 68;
  float* stg = reinterpret_cast<float*>(wave == 0 ? A0 : wave == 1 ? A1 : wave == 2 ? A2 : A3);
  // read-back position: KIND 1 row rq + 8 i, columns cq..cq+7 of the half;
  // the others row rq + 4 i, columns cq..cq+3
  constexpr int CPL = (KIND == 1) ? 8 : 4, LPR = 64 / CPL, RPI = 64 / LPR;
  const int rq = lane / LPR, cq = (lane % LPR) * CPL;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nb = 2 * h + q;
          float4 v;
          v.x = acc[nb][mb][4 * g + 0];
          v.y = acc[nb][mb][4 * g + 1];
          v.z = acc[nb][mb][4 * g + 2];
          v.w = acc[nb][mb][4 * g + 3];
          *reinterpret_cast<float4*>(stg + l32 * SP + q * 32 + 8 * g + 4 * hi) = v;
        }
      const int n = t.n0 + wn * 128 + h * 64 + cq;
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int rr = rq + RPI * i;
        const int m = t.m0 + wm * 128 + mb * 32 + rr;
        const float4 v = *reinterpret_cast<const float4*>(stg + rr * SP + cq);
        if constexpr (KIND == 1) {
          const float4 w = *reinterpret_cast<const float4*>(stg + rr * SP + cq + 4);
          if (m >= t.mval || n >= t.nval) continue;
          bf16_t* crow = a.cx + (size_t)(t.row0 + m) * a.ldc;
          const u32x4 p = {pack2(v.x, v.y), pack2(v.z, v.w), pack2(w.x, w.y), pack2(w.z, w.w)};
          *reinterpret_cast<u32x4*>(crow + n) = p;
        } else {
          if (m >= t.mval || n >= t.nval) continue;
          float* crow;
          if (KIND == 0) {
            const size_t col = SH ? (size_t)t.grp * a.inner : 0;
            crow = a.c + (size_t)(t.row0 + m) * a.ldc + col;
          } else if (a.splits > 1) {   // partial sums [split][group][M][N], reduced later
            crow = a.part + (((size_t)t.split * a.n_experts + t.grp) * t.mval + m) * t.nval;
          } else if (KIND == 2) {
            crow = a.dw2 + ((size_t)t.grp * a.d + m) * a.inner;
          } else {
            crow = (m < a.inner) ? a.dw1 + ((size_t)t.grp * a.inner + m) * a.d
                                 : a.dw3 + ((size_t)t.grp * a.inner + (m - a.inner)) * a.d;
          }
          // non-temporal: not read again by this kernel
          __builtin_nontemporal_store(fv4{v.x, v.y, v.z, v.w}, reinterpret_cast<fv4*>(crow + n));
        }
      }
    }
  }
}

// Sum of the split-k partials of a weight gradient, splits in order, into
// the gradient's own layout (4 consecutive elements per thread).  The
// outputs may alias split 0's partials (the gate gradient points them
// there): a thread reads its elements of every split before it writes them.
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
