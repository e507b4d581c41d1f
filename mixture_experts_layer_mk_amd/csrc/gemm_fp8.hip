// Grouped expert GEMMs on FP8 operands for FP8 layers (gfx950 block-scaled
// matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 inputs, fp32
// accumulation).
//
// FP8 recipe (DeepSeek-V3 Technical Report summary, "3.3 FP8 Training": most
// GEMMs in FP8 with fine-grained scaling and high-precision accumulation;
// "B.2 Discussion About Block-Wise Quantization": activations grouped 1 x 128
// along the reduction dimension, weights in 128 x 128 blocks).  Every scale is
// a power of two, so the matrix instruction applies it: each lane passes the
// 8-bit exponent of its own row's 128-wide k-group (token rows: one per row;
// weight rows: one per 128 x 128 block) and the products come out scaled.
//
// Stages as in the bf16 kernels:
//   GATEUP      H = silu(A W1^T) * (A W3^T); H is written in E4M3 with one
//               power-of-two scale per 128 inner columns of a row (the max
//               over the group is exchanged between the waves that hold it)
//   DOWN        Y = H W2^T (fp16 with a power-of-two scale per 64 columns)
//   DOWN_SHARED S = x + sum_s H_s W2_s^T (fp32)
//
// Tiling is the bf16 kernel's with the k step doubled: a 128-wide k-block is
// one 128-byte LDS row per operand row and one scale group; it feeds two
// 64-deep matrix steps.  The scale bytes of the tile's token rows and weight
// blocks are staged in LDS at the start of the tile.
#include "gemm_common.h"

namespace moe {

namespace {

using namespace gemm;

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int BK8 = 128;       // k per stage: one 128-byte row, one scale group
constexpr int MAX_NK = 64;     // k-blocks per tile (k up to 8192)

// Scale exponent of a group with largest magnitude amax: the smallest E with
// amax <= 448 * 2^E (448 = largest finite E4M3), in [-127, 127]; 0 for zero.
__device__ __forceinline__ int e4m3_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(amax);
  const float f = __builtin_amdgcn_frexp_mantf(amax);
  const int E = e - 9 + (f > 0.875f ? 1 : 0);
  return min(max(E, -127), 127);
}

// Four floats (already scaled) to four E4M3 codes, low byte first.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// One tile: rows [row0, row0 + rows) (at most BM) of the M dimension (expert
// e for routed tiles) times N-tile nt.  LDS: operand buffers As0/As1 (at least
// BM x 128 B) and Bs0/Bs1, the tile's scale bytes sA [BM][MAX_NK] and
// sB [2][MAX_NK], and gmax [4][BM] for the GATEUP epilogue.
template <int MODE, int BM, int WAVES_M, int NS>
__device__ __forceinline__ void gemm8_tile(const GemmArgs& a, int row0, int rows, int e,
                                           int nt, u32x4* As0, u32x4* As1, u32x4* As2,
                                           u32x4* Bs0, u32x4* Bs1, u32x4* Bs2, uint8_t* sA,
                                           uint8_t* sB, float* gmax) {
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int A_LD = BM / 32;     // 1 KB direct loads per wave per stage (A)
  constexpr int B_LD = BN / 32;     // (B)
  static_assert(MB >= 1 && NB >= 2 && (NB % 2) == 0, "tile shape");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool routed = !(MODE == 2 || (MODE == 0 && a.shared));

  const int lr = lane >> 3;
  const int cg0 = (lane & 7) ^ lr;         // rows with (row >> 3) even
  const int cg1 = cg0 ^ 1;                 // rows with (row >> 3) odd

  // A: tile row r = (wave * A_LD + j) * 8 + lr, clamped into the valid rows;
  // byte offsets (one byte per element).
  const uint8_t* A = static_cast<const uint8_t*>(a.a);
  uint32_t aoff[A_LD];
#pragma unroll
  for (int j = 0; j < A_LD; ++j) {
    const int blk = wave * A_LD + j;
    const int r = min(blk * 8 + lr, rows - 1);
    const int src = a.a_rows ? a.a_rows[row0 + r] : row0 + r;
    aoff[j] = (uint32_t)src * a.lda + ((blk & 1) ? cg1 : cg0) * 16;
  }

  // B: tile row r = (wave * B_LD + j) * 8 + lr.
  const uint8_t* B1;
  const uint8_t* B3 = nullptr;
  uint32_t boff[B_LD];
  int kdim, n0 = 0, grp = 0, inner0 = 0;
  if (MODE == 0) {
    const int half = WN / 2;                       // inner columns per wave
    const int per_wg = WAVES_N * half;             // inner columns per tile (128)
    const int tiles_per = (a.inner + per_wg - 1) / per_wg;
    grp = routed ? e : nt / tiles_per;
    inner0 = (routed ? nt : nt % tiles_per) * per_wg;
    const size_t wo = (size_t)grp * a.inner * a.d;
    B1 = static_cast<const uint8_t*>(a.w1) + wo;
    B3 = static_cast<const uint8_t*>(a.w3) + wo;
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
      const int blk = wave * B_LD + j;
      const int r = blk * 8 + lr;
      const int rw = r / WN, rr = r % WN;
      const int inner = min(inner0 + rw * half + (rr % half), a.inner - 1);
      boff[j] = (uint32_t)inner * a.d + ((blk & 1) ? cg1 : cg0) * 16;
    }
    kdim = a.d;
  } else {
    n0 = nt * BN;
    B1 = static_cast<const uint8_t*>(a.w2) + (MODE == 1 ? (size_t)e * a.d * a.inner : 0);
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
      const int blk = wave * B_LD + j;
      const int n = min(n0 + blk * 8 + lr, a.d - 1);
      boff[j] = (uint32_t)n * a.inner + ((blk & 1) ? cg1 : cg0) * 16;
    }
    kdim = (MODE == 1) ? a.inner : a.inner * a.n_experts;
  }
  const int nk = kdim / BK8;

  // Scale bytes of the tile: token rows (sA[kb][r]: a wave's 32 rows of one
  // k-block are 32 consecutive bytes, read without bank conflicts) and the
  // weight blocks (sB[h][kb]: GATEUP h = 0 / 1 for W1 / W3 of the tile's 128
  // inner rows; DOWN h = the 128-row halves of the 256 output columns).
  // Each row's gather index is read once, by the 256 / BM threads that share
  // the row (each takes every (256 / BM)-th k-block), and the row's scale bytes
  // go out back to back (measured: one index and one byte load per element
  // cost about 5% of the 16B-shaped FP8 layer).
  {
    static_assert(256 % BM == 0, "rows divide the workgroup");
    constexpr int TPR = 256 / BM;                      // threads per row
    const int r = tid / TPR, part = tid % TPR;
    const int rr = min(r, rows - 1);
    const int src = a.a_rows ? a.a_rows[row0 + rr] : row0 + rr;
    const uint8_t* srow = a.a_scale + (size_t)src * a.lda_s;
#pragma unroll 8
    for (int kb = part; kb < nk; kb += TPR) sA[kb * BM + r] = srow[kb];
  }
  for (int i = tid; i < 2 * nk; i += 256) {
    const int h = i / nk, kb = i % nk;
    uint8_t v;
    if (MODE == 0) {
      const int ib = inner0 / 128, dB = a.d / 128, iB = a.inner / 128;
      const uint8_t* s = h ? a.s3 : a.s1;
      v = s[((size_t)grp * iB + ib) * dB + kb];
    } else {
      const int dB = a.d / 128, iB = a.inner / 128;
      const int nb = min(n0 / 128 + h, dB - 1);
      const int ex = (MODE == 1) ? e : kb / iB;           // shared experts along k
      const int kk = (MODE == 1) ? kb : kb % iB;
      v = a.s2[((size_t)ex * dB + nb) * iB + kk];
    }
    sB[h * MAX_NK + kb] = v;
  }

  // Issue the direct loads of k-block kb into the LDS buffers (Ab, Bb).
  auto issue = [&](int kb, u32x4* Ab, u32x4* Bb) {
    const size_t ka = (size_t)kb * BK8;
    size_t kbo = ka;
    if (MODE == 2) {   // shared experts follow one another along k
      const int k = kb * BK8, s = k / a.inner;
      kbo = (size_t)s * a.d * a.inner + (k - s * a.inner);
    }
#pragma unroll
    for (int j = 0; j < A_LD; ++j)
      __builtin_amdgcn_global_load_lds((const glb_void*)(A + aoff[j] + ka),
                                       (lds_void*)&Ab[(wave * A_LD + j) * 64], 16, 0, 0);
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
      const uint8_t* base = B1;
      if (MODE == 0) {
        const int r = (wave * B_LD + j) * 8;        // uniform: W1 or W3 half
        if ((r % WN) >= WN / 2) base = B3;
      }
      __builtin_amdgcn_global_load_lds((const glb_void*)(base + boff[j] + kbo),
                                       (lds_void*)&Bb[(wave * B_LD + j) * 64], 16, 0, 0);
    }
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Fragments: 32 bytes of one row per lane (k 32 hi .. 32 hi + 31 of the
  // 64-deep step kk), two 16-byte LDS chunks.
  i32x8 fa0[MB], fb0[NB], fa1[MB], fb1[NB];
  auto frag = [&](const u32x4* Xb, int r, int kk) -> i32x8 {
    const int c = 4 * kk + 2 * hi, s = swz_x(r);
    const u32x4 p = Xb[r * 8 + (c ^ s)], q = Xb[r * 8 + ((c + 1) ^ s)];
    i32x8 v;
    v[0] = (int)p.x; v[1] = (int)p.y; v[2] = (int)p.z; v[3] = (int)p.w;
    v[4] = (int)q.x; v[5] = (int)q.y; v[6] = (int)q.z; v[7] = (int)q.w;
    return v;
  };
  auto load_frags = [&](i32x8* fa, i32x8* fb, const u32x4* Ab, const u32x4* Bb, int kk) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) fa[mb] = frag(Ab, wm * WM + mb * 32 + l32, kk);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) fb[nb] = frag(Bb, wn * WN + nb * 32 + l32, kk);
  };
  // Scales of k-block kb: token rows per lane, weight blocks per wave.
  int sa[MB], sb[2];
  auto load_scales = [&](int kb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) sa[mb] = sA[kb * BM + wm * WM + mb * 32 + l32];
    if (MODE == 0) {
      sb[0] = sB[kb];
      sb[1] = sB[MAX_NK + kb];
    } else {
      sb[0] = sB[((wn * WN) / 128) * MAX_NK + kb];
      sb[1] = sb[0];
    }
  };
  auto mma = [&](const i32x8* fa, const i32x8* fb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fb[nb], fa[mb], acc[nb][mb], 0, 0, 0, sb[nb < NB / 2 ? 0 : 1], 0, sa[mb]);
  };
  constexpr int N_MMA = NB * MB, N_DS = 2 * (NB + MB), N_VM = A_LD + B_LD;
  auto sched_ds = [&]() { sched_groups<N_MMA, N_DS, 0>(); };
  auto sched_ds_vm = [&]() { sched_groups<N_MMA, N_DS, N_VM>(); };

  // One k-block (two 64-deep steps) from (Ac, Bc); the next block is already
  // streaming into (An, Bn).  After the first step every wave holds its last
  // fragments of this block (barrier): (Ac, Bc) are free and block `next2`
  // starts streaming into them.  Blocks past the end re-load the last block
  // (never read).
  // With three stages the block after next may still be in flight at the
  // barrier: the wait leaves the most recent stage's N_VM loads outstanding.
  auto block = [&](int kb, int next2, u32x4* Ac, u32x4* Bc, const u32x4* An,
                   const u32x4* Bn) {
    load_scales(kb);
    load_frags(fa1, fb1, Ac, Bc, 1);
    mma(fa0, fb0);
    sched_ds();
    // Block kb+1 landed: the count wait the compiler sees, then the barrier
    // (with the wait hidden in asm, or a fence, the compiler also waited for
    // the loads issued just after it before the next fragment reads;
    // measured: V3-shaped FP8 layer -8.5%, 16B-shaped -1.8%).
    stage_sync<NS == 3 ? N_VM : 0>();
    issue(next2, Ac, Bc);
    load_frags(fa0, fb0, An, Bn, 0);
    mma(fa1, fb1);
    sched_ds_vm();
  };

  if constexpr (NS == 3) {
    // Three-stage ring (tiles of at most 128 rows, which stream their
    // weights): two blocks in flight while one is computed.
    issue(0, As0, Bs0);
    issue(min(1, nk - 1), As1, Bs1);
    issue(min(2, nk - 1), As2, Bs2);
    stage_sync<2 * N_VM>();                              // block 0 and the scales
    load_frags(fa0, fb0, As0, Bs0, 0);
    int kb = 0;
    for (; kb + 3 <= nk; kb += 3) {
      block(kb, min(kb + 3, nk - 1), As0, Bs0, As1, Bs1);
      block(kb + 1, min(kb + 4, nk - 1), As1, Bs1, As2, Bs2);
      block(kb + 2, min(kb + 5, nk - 1), As2, Bs2, As0, Bs0);
    }
    if (kb < nk) block(kb, nk - 1, As0, Bs0, As1, Bs1);
    if (kb + 1 < nk) block(kb + 1, nk - 1, As1, Bs1, As2, Bs2);
  } else {
    issue(0, As0, Bs0);
    issue(min(1, nk - 1), As1, Bs1);
    stage_sync<N_VM>();   // block 0 and the scales (block 1 may still fly)
    load_frags(fa0, fb0, As0, Bs0, 0);
    int kb = 0;
    for (; kb + 2 <= nk; kb += 2) {
      block(kb, min(kb + 2, nk - 1), As0, Bs0, As1, Bs1);
      block(kb + 1, min(kb + 3, nk - 1), As1, Bs1, As0, Bs0);
    }
    if (kb < nk) block(kb, nk - 1, As0, Bs0, As1, Bs1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // no load left in flight

  // ---- epilogue ----
  // acc[nb][mb][r] = D[n][m] with n = nb*32 + 8*(r/4) + 4*hi + (r%4) and
  // m = mb*32 + l32 inside the wave's tile.
  if (MODE == 0) {
    // H = silu(gate) * up; the 128 inner columns of a tile row are spread
    // over the WAVES_N waves with the same rows (WN / 2 each): each wave's
    // row maximum goes through LDS, then every wave scales its part by the
    // group's power of two and writes E4M3 codes; wave 0 of the row writes
    // the scale byte.
    constexpr int HALF_NB = NB / 2;
    float h[MB][HALF_NB][4][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float amax = 0.f;
#pragma unroll
      for (int nb = 0; nb < HALF_NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float v = silu_f(acc[nb][mb][4 * g + q]) * acc[nb + HALF_NB][mb][4 * g + q];
            h[mb][nb][g][q] = v;
            amax = fmaxf(amax, fabsf(v));
          }
      amax = max_halves(amax);
      if (hi == 0) gmax[wn * BM + wm * WM + mb * 32 + l32] = amax;
    }
    __syncthreads();
    const int col_off = routed ? 0 : grp * a.inner;
    uint8_t* out = static_cast<uint8_t*>(a.out);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = wm * WM + mb * 32 + l32;
      float ga = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES_N; ++w) ga = fmaxf(ga, gmax[w * BM + m]);
      const int E = e4m3_scale_exp(ga);
      const float s = __int_as_float((127 - E) << 23);    // 2^-E
      if (m >= rows) continue;
      uint8_t* orow = out + (size_t)(row0 + m) * a.ldo + col_off;
#pragma unroll
      for (int nb = 0; nb < HALF_NB; ++nb) {
        // inner is a multiple of 128: a 32-column block is all in or all out.
        const int ib = inner0 + wn * (WN / 2) + nb * 32;
        if (ib >= a.inner) continue;
        uint32_t p[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          p[g] = e4m3_pack4(h[mb][nb][g][0] * s, h[mb][nb][g][1] * s, h[mb][nb][g][2] * s,
                            h[mb][nb][g][3] * s);
        swap_halves_bytes(p);
        *reinterpret_cast<uint4*>(orow + ib + 16 * hi) = make_uint4(p[0], p[1], p[2], p[3]);
      }
      if (wn == 0 && hi == 0)
        a.out_scale[(size_t)(row0 + m) * a.ldo_s + (col_off + inner0) / 128] = (uint8_t)(E + 127);
    }
  } else if (MODE == 1) {
    // Y rows in fp16, each 64-column group of a row scaled so that its
    // largest magnitude lands just below 2^15 (as in the bf16 layer).
    uint16_t* out = static_cast<uint16_t*>(a.out);
    const int gpr = a.d / Y_GROUP;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      __builtin_amdgcn_sched_barrier(0);
      const int m = wm * WM + mb * 32 + l32;
#pragma unroll
      for (int gi = 0; gi < NB / 2; ++gi) {
        float amax = 0.f;
#pragma unroll
        for (int nb = 2 * gi; nb < 2 * gi + 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(acc[nb][mb][r]));
        amax = max_halves(amax);
        float sc, inv;
        y_scale_of(amax, sc, inv);
        if (m >= rows) continue;
        uint16_t* orow = out + (size_t)(row0 + m) * a.ldo;
#pragma unroll
        for (int nb = 2 * gi; nb < 2 * gi + 2; ++nb) {
          // d is a multiple of 128: a 32-column block is all in or all out.
          const int n = n0 + wn * WN + nb * 32;
          if (n >= a.d) continue;
          uint32_t p[4][2];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            p[g][0] = pack_h2(acc[nb][mb][4 * g + 0] * sc, acc[nb][mb][4 * g + 1] * sc);
            p[g][1] = pack_h2(acc[nb][mb][4 * g + 2] * sc, acc[nb][mb][4 * g + 3] * sc);
          }
          swap_halves(p);
          store_block(orow + n + 8 * hi, p);
        }
        const int ng = n0 + wn * WN + gi * Y_GROUP;
        if (hi == 0 && ng < a.d) a.yscale[(size_t)(row0 + m) * gpr + ng / Y_GROUP] = inv;
      }
    }
  } else {
    // Shared experts' down-projection: S = x + sum_s H_s W2_s^T in fp32 (as
    // in the bf16 layer; the combine adds the kept experts).  The rows of x
    // are read in 16-byte chunks swapped into the accumulator layout (a block
    // past d reads the row's last block; its values are never stored).
    const bf16_t* x = static_cast<const bf16_t*>(a.x);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      __builtin_amdgcn_sched_barrier(0);
      const int m = wm * WM + mb * 32 + l32;
      if (m >= rows) continue;
      const int t = row0 + m;
      const bf16_t* xrow = x + (size_t)t * a.d;
      float* srow = static_cast<float*>(a.out) + (size_t)t * a.ldo;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int cblk = min(n0 + wn * WN + nb * 32, a.d - 32) + 8 * hi;
        uint32_t p[4][2];
        load_block(xrow + cblk, p);
        swap_halves(p);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + nb * 32 + 8 * g + 4 * hi;
          if (n >= a.d) continue;
          *reinterpret_cast<float4*>(srow + n) = make_float4(
              bf16_to_f32((bf16_t)(p[g][0] & 0xffff)) + acc[nb][mb][4 * g + 0],
              bf16_to_f32((bf16_t)(p[g][0] >> 16)) + acc[nb][mb][4 * g + 1],
              bf16_to_f32((bf16_t)(p[g][1] & 0xffff)) + acc[nb][mb][4 * g + 2],
              bf16_to_f32((bf16_t)(p[g][1] >> 16)) + acc[nb][mb][4 * g + 3]);
        }
      }
    }
  }
}

// One part of a grouped FP8 GEMM launch (block `blk` of `nblk`): an expert's
// last routed tile runs the 64-row layout for at most 64 rows in the 256-row
// launches, and the half-height layout for at most BM / 2 rows.
template <int MODE, int BM, int WAVES_M, int NS>
__device__ __forceinline__ void gemm8_part(const GemmArgs& a, int blk, int nblk, u32x4* As0,
                                           u32x4* As1, u32x4* As2, u32x4* Bs0, u32x4* Bs1,
                                           u32x4* Bs2, uint8_t* sA, uint8_t* sB, float* gmax) {
  const bool routed = !(MODE == 2 || (MODE == 0 && a.shared));
  // Tiles numbered over the M-tiles the routing made (blocks past them exit),
  // so every XCD gets an equal share of real tiles.
  const int mdim = routed ? *a.n_tiles : (a.T + BM - 1) / BM;
  const int ndim = n_tiles_of<MODE, BM>(a);
  const int ntl = mdim * ndim;
  const int L = !routed ? xcd_remap(blk, nblk) : (blk < ntl ? xcd_remap(blk, ntl) : ntl);
  if (L >= ntl) return;                      // padding
  int mt, nt;
  constexpr int NGRP = ngrp_for<BM>();
  {
    const int full = ndim / NGRP;
    const int ntg = L / (mdim * NGRP);
    const int g = (ntg < full) ? NGRP : ndim - full * NGRP;
    const int rem = L - ntg * mdim * NGRP;
    mt = rem / g;
    nt = ntg * NGRP + rem % g;
  }
  if (routed) {
    const MTile t = a.tiles[mt];
    if constexpr (BM == 256) {
      // an expert's last rows: 64-row layout for at most 64 of them
      if (t.rows <= 64) {
        gemm8_tile<MODE, 64, 1, NS>(a, t.row0, t.rows, t.expert, nt, As0, As1, As2, Bs0, Bs1,
                                    Bs2, sA, sB, gmax);
        return;
      }
    }
    if constexpr (BM >= 128) {
      if (t.rows <= BM / 2) {
        gemm8_tile<MODE, BM / 2, 1, NS>(a, t.row0, t.rows, t.expert, nt, As0, As1, As2, Bs0,
                                        Bs1, Bs2, sA, sB, gmax);
        return;
      }
    }
    gemm8_tile<MODE, BM, WAVES_M, NS>(a, t.row0, t.rows, t.expert, nt, As0, As1, As2, Bs0, Bs1,
                                      Bs2, sA, sB, gmax);
  } else {
    const int row0 = mt * BM;
    gemm8_tile<MODE, BM, WAVES_M, NS>(a, row0, min(BM, a.T - row0), 0, nt, As0, As1, As2, Bs0,
                                      Bs1, Bs2, sA, sB, gmax);
  }
}

// The grouped FP8 GEMM: one workgroup per tile; blocks [0, a_blocks) run
// stage MODE on `a` (routed experts), the rest stage MODE_B on `b` (shared
// experts), a_blocks a multiple of 8 (XCD-aware orders in both parts).
template <int MODE, int MODE_B, int BM, int WAVES_M>
__global__ __launch_bounds__(256, 1) void gemm_fp8_kernel(GemmArgs a, GemmArgs b,
                                                          int a_blocks) {
  // Tiles of at most 128 rows keep a third stage (3 x (BM + 256) x 128 B
  // <= 144 KB of LDS).
  constexpr int NS = (BM <= 128) ? 3 : 2;
  __shared__ u32x4 As0[BM * 8], As1[BM * 8], As2[NS == 3 ? BM * 8 : 1];
  __shared__ u32x4 Bs0[BN * 8], Bs1[BN * 8], Bs2[NS == 3 ? BN * 8 : 1];
  __shared__ uint8_t sA[BM * MAX_NK];
  __shared__ uint8_t sB[2 * MAX_NK];
  __shared__ float gmax[4 * BM];
  // Each part reads its own argument struct (a run-time choice of struct
  // made the compiler copy both to scratch memory).
  const int blk = blockIdx.x;
  if (blk >= a_blocks)
    gemm8_part<MODE_B, BM, WAVES_M, NS>(b, blk - a_blocks, (int)gridDim.x - a_blocks, As0, As1,
                                        As2, Bs0, Bs1, Bs2, sA, sB, gmax);
  else
    gemm8_part<MODE, BM, WAVES_M, NS>(a, blk, a_blocks, As0, As1, As2, Bs0, Bs1, Bs2, sA, sB,
                                      gmax);
}

template <int MODE, int BM>
int part_blocks8(const GemmArgs& g) {
  const bool routed = !(MODE == 2 || (MODE == 0 && g.shared));
  const int mdim = routed ? g.max_mtiles : (g.T + BM - 1) / BM;
  return mdim * n_tiles_of<MODE, BM>(g);
}

template <int MODE, int MODE_B, int BM, int WAVES_M>
void launch_pair8(const GemmArgs& a, const GemmArgs* b, hipStream_t s) {
  if (!b) {
    hipLaunchKernelGGL((gemm_fp8_kernel<MODE, MODE, BM, WAVES_M>),
                       dim3(part_blocks8<MODE, BM>(a)), dim3(256), 0, s, a, a,
                       part_blocks8<MODE, BM>(a));
    return;
  }
  const int na = (part_blocks8<MODE, BM>(a) + 7) & ~7;
  const int nb = part_blocks8<MODE_B, BM>(*b);
  hipLaunchKernelGGL((gemm_fp8_kernel<MODE, MODE_B, BM, WAVES_M>), dim3(na + nb), dim3(256), 0,
                     s, a, *b, na);
}

template <int BM, int WAVES_M>
void launch_bm8(const GemmArgs& a, const GemmArgs* b, hipStream_t s) {
  if (a.mode == 0) launch_pair8<0, 0, BM, WAVES_M>(a, b, s);
  else launch_pair8<1, 2, BM, WAVES_M>(a, b, s);
}

}  // namespace

hipError_t launch_gemm_fp8(const GemmArgs& a, hipStream_t s, const GemmArgs* b) {
  // DOWN_SHARED runs only as the second part of a DOWN launch.
  if (a.mode == 2 || (b && (b->bm != a.bm || (a.mode == 1 ? b->mode != 2 : b->mode != a.mode))))
    return hipErrorInvalidValue;
  switch (a.bm) {
    case 256: launch_bm8<256, 2>(a, b, s); break;
    case 128: launch_bm8<128, 1>(a, b, s); break;
    case 64: launch_bm8<64, 1>(a, b, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
