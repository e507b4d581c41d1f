// Grouped expert GEMMs for bf16 layers on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Each expert is a SwiGLU FFN W2 (silu(W1 u) * (W3 u)) (expert form of the
// DeepSeekMoE layer; blog post "Fine-Grained Expert Segmentation (Section
// 3.1)").  Stages (same as the fp32 path):
//   GATEUP      H = silu(A W1^T) * (A W3^T), gate and up fused in one tile;
//               routed tiles gather their token rows straight from x
//   DOWN        Y = H W2^T (routed rows; fp16 scaled by a power of two per
//               64 columns of a row, inverse scales beside)
//   DOWN_SHARED S = x + sum_s H_s W2_s^T (fp32; the shared experts, which
//               the combine then adds the kept experts to)
//   GATEUP_BWD  the gate/up tile recomputed for the backward pass, with the
//               SwiGLU backward in the epilogue (see GemmArgs)
//
// Tiling.  A workgroup (4 or 8 waves) owns BM token rows x 256 weight rows
// with a 64-wide k step.  Both operands are k-contiguous in memory (token rows and
// linear-layer weight rows), so tiles move as 16-byte chunks, global -> LDS
// directly (global_load_lds_dwordx4: no staging registers, no LDS write
// instructions), double-buffered (2 x (BM + 256) x 128 B of LDS).  The 16-byte
// chunks of each 128-byte LDS row are XOR-swizzled so the matrix-operand
// reads are free of bank conflicts; a direct load writes 1 KB of consecutive
// LDS per wave, so each lane fetches the global chunk that the swizzle puts
// in its slot.  Operand fragments are double-buffered in registers: the LDS
// reads of k-step kk+1 are in flight while the 16 matrix ops of kk run.
// The matrix instruction takes the weight fragment as its first operand, so
// each lane's accumulator holds 4 consecutive output columns of one token
// row.  For GATEUP each wave's weight rows are half W1, half W3 for the same
// inner columns, so silu(gate) * up is formed in registers.
// Blocks are remapped so that each XCD (blocks are dealt round-robin over the
// 8 XCDs) runs a contiguous range of tiles, with the M-tiles of one weight
// tile adjacent: the weight tile is then fetched into that XCD's L2 once.
// One launch holds the routed experts' tiles of a stage and, after them, the
// shared experts' (one grouped GEMM over all experts of the layer).
#include "gemm_common.h"

namespace moe {

namespace {

using namespace gemm;

constexpr int BK = 64;    // k per stage (8 chunks of 16 B)

// Epilogue of the down-projection tiles (DOWN, DOWN_SHARED) from the
// accumulators of a wave's WM x WN sub-tile: acc[nb][mb][r] = D[n][m] with
// n = nb*32 + 8*(r/4) + 4*hi + (r%4) and m = mb*32 + l32 inside it.
template <int MODE, int MB, int NB, int WM, int WN>
__device__ __forceinline__ void down_epilogue(const GemmArgs& a, const f32x16 (&acc)[NB][MB],
                                              int row0, int rows, int n0, int wm, int wn,
                                              int l32, int hi) {
  if constexpr (MODE == 1) {
    // Y rows in fp16, each 64-column group of a row scaled so that its
    // largest magnitude lands just below 2^15; the inverse scales go to
    // yscale[row][col / 64].  The group's columns are column blocks
    // nb = 2 gi, 2 gi + 1 of this lane and of lane ^ 32 (same row).
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
          // d is a multiple of 64: a 32-column block is all in or all out.
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
    // Shared experts' down-projection: S = x + sum_s H_s W2_s^T in fp32
    // (the residual and the shared experts; the combine adds the kept
    // experts).  The rows of x are read in 16-byte chunks, 8 consecutive
    // columns per lane, then swapped into the accumulator layout (a block
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

// One tile: rows [row0, row0 + rows) (at most BM) of the M dimension (expert
// e for routed tiles) times N-tile nt, through the LDS buffers As0/As1 (at
// least BM x 128 B each) and Bs0/Bs1.  MODE 0 GATEUP, 1 DOWN, 2 DOWN_SHARED,
// 3 GATEUP_BWD; WAVES_M x (NW / WAVES_M) waves.  `red` (4 x BM floats of LDS)
// carries GATEUP_BWD's row sums across the waves of a tile.
template <int MODE, int BM, int WAVES_M, int NS, int NW>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, int row0, int rows, int e,
                                          int nt, u32x4* As0, u32x4* As1, u32x4* As2,
                                          u32x4* Bs0, u32x4* Bs1, u32x4* Bs2, float* red) {
  constexpr int WAVES_N = NW / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int A_LD = BM / (8 * NW);     // 1 KB direct loads per wave per stage (A)
  constexpr int B_LD = BN / (8 * NW);     // (B)
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the waves");
  static_assert(MB >= 1 && NB >= 2 && (NB % 2) == 0, "tile shape");

  // The wave index is uniform: kept in a scalar register, so the per-wave
  // LDS bases of the direct loads (M0) and the fragment rows need no
  // per-load vector-to-scalar moves.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  constexpr bool GU = is_gateup<MODE>();
  const bool routed = !(MODE == 2 || (GU && a.shared));

  // This lane's slot in a wave's 1 KB load block: LDS row lr (of 8) and the
  // global chunk that belongs in slot (lane & 7) of that row.
  const int lr = lane >> 3;
  const int cg0 = (lane & 7) ^ lr;         // rows with (row >> 3) even
  const int cg1 = cg0 ^ 1;                 // rows with (row >> 3) odd

  // A: tile row r = (wave * A_LD + j) * 8 + lr, clamped into the valid rows.
  const bf16_t* A = static_cast<const bf16_t*>(a.a);
  uint32_t aoff[A_LD];
#pragma unroll
  for (int j = 0; j < A_LD; ++j) {
    const int blk = wave * A_LD + j;
    const int r = min(blk * 8 + lr, rows - 1);
    const int src = a.a_rows ? a.a_rows[row0 + r] : row0 + r;
    aoff[j] = (uint32_t)src * a.lda + ((blk & 1) ? cg1 : cg0) * 8;
  }

  // B: tile row r = (wave * B_LD + j) * 8 + lr.
  const bf16_t* B1;
  const bf16_t* B3 = nullptr;
  uint32_t boff[B_LD];
  int kdim, n0 = 0, grp = 0, inner0 = 0;
  if (GU) {
    const int half = WN / 2;                       // inner columns per wave
    const int per_wg = WAVES_N * half;             // inner columns per tile
    const int tiles_per = (a.inner + per_wg - 1) / per_wg;
    grp = routed ? e : nt / tiles_per;
    inner0 = (routed ? nt : nt % tiles_per) * per_wg;
    const size_t wo = (size_t)grp * a.inner * a.d;
    B1 = static_cast<const bf16_t*>(a.w1) + wo;
    B3 = static_cast<const bf16_t*>(a.w3) + wo;
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
      const int blk = wave * B_LD + j;
      const int r = blk * 8 + lr;
      const int rw = r / WN, rr = r % WN;
      const int inner = min(inner0 + rw * half + (rr % half), a.inner - 1);
      boff[j] = (uint32_t)inner * a.d + ((blk & 1) ? cg1 : cg0) * 8;
    }
    kdim = a.d;
  } else {
    n0 = nt * BN;
    B1 = static_cast<const bf16_t*>(a.w2) + (MODE == 1 ? (size_t)e * a.d * a.inner : 0);
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
      const int blk = wave * B_LD + j;
      const int n = min(n0 + blk * 8 + lr, a.d - 1);
      boff[j] = (uint32_t)n * a.inner + ((blk & 1) ? cg1 : cg0) * 8;
    }
    kdim = (MODE == 1) ? a.inner : a.inner * a.n_experts;
  }
  const int nk = kdim / BK;

  // Issue the direct loads of k-block kb into the LDS buffers (Ab, Bb).
  // The direct loads of k-block kb into the LDS buffers (Ab, Bb): A_LD + B_LD
  // per wave, numbered q (A first).  They are issued in NPART parts -- part p
  // takes q in [p N / NPART, (p + 1) N / NPART) -- spread over successive
  // k-steps rather than all beside the matrix ops of one step (measured: two
  // parts for the two-stage 256-row tiles, four for the three-stage ring).
  constexpr int N_VM = A_LD + B_LD;
  constexpr int NPART = (NS == 3) ? 4 : 2;
  auto issue = [&](int kb, u32x4* Ab, u32x4* Bb, int part) {
    const int lo = part * N_VM / NPART, hi_q = (part + 1) * N_VM / NPART;
    const size_t ka = (size_t)kb * BK;
    size_t kbo = ka;
    if (MODE == 2) {   // shared experts follow one another along k
      const int k = kb * BK, s = k / a.inner;
      kbo = (size_t)s * a.d * a.inner + (k - s * a.inner);
    }
#pragma unroll
    for (int j = 0; j < A_LD; ++j)
      if (j >= lo && j < hi_q)
        __builtin_amdgcn_global_load_lds((const glb_void*)(A + aoff[j] + ka),
                                         (lds_void*)&Ab[(wave * A_LD + j) * 64], 16, 0, 0);
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
      if (A_LD + j < lo || A_LD + j >= hi_q) continue;
      const bf16_t* base = B1;
      if (GU) {
        const int r = (wave * B_LD + j) * 8;        // uniform: W1 or W3 half
        if ((r % WN) >= WN / 2) base = B3;
      }
      __builtin_amdgcn_global_load_lds((const glb_void*)(base + boff[j] + kbo),
                                       (lds_void*)&Bb[(wave * B_LD + j) * 64], 16, 0, 0);
    }
  };
  auto issue_all = [&](int kb, u32x4* Ab, u32x4* Bb) {
#pragma unroll
    for (int p = 0; p < NPART; ++p) issue(kb, Ab, Bb, p);
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int l32 = lane & 31, hi = lane >> 5;
  // Fragment registers, two sets: one feeds the matrix ops while the other
  // is being read from LDS.
  bf16x8 fa0[MB], fb0[NB], fa1[MB], fb1[NB];
  auto load_frags = [&](bf16x8* fa, bf16x8* fb, const u32x4* Ab, const u32x4* Bb,
                        int kk) {
    const int c = 2 * kk + hi;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = wm * WM + mb * 32 + l32;
      fa[mb] = __builtin_bit_cast(bf16x8, Ab[r * 8 + (c ^ swz_x(r))]);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int r = wn * WN + nb * 32 + l32;
      fb[nb] = __builtin_bit_cast(bf16x8, Bb[r * 8 + (c ^ swz_x(r))]);
    }
  };
  auto mma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nb], fa[mb],
                                                             acc[nb][mb], 0, 0, 0);
  };
  // Scheduling: spread the LDS reads (and the direct loads) of a k-step
  // between its matrix ops so the matrix pipe never waits on LDS latency.
  constexpr int N_MMA = NB * MB, N_DS = NB + MB;
  constexpr int P0 = N_VM / NPART;                       // loads in part 0
  constexpr int P1 = 2 * N_VM / NPART - P0, P2 = 3 * N_VM / NPART - 2 * N_VM / NPART;
  constexpr int P3 = 4 * N_VM / NPART - 3 * N_VM / NPART;

  // One k-block from buffers (Ac, Bc); block kb+1 is already in (An, Bn)
  // or streaming into them (and with three stages kb+2 into the third
  // pair).  Parts 1.. of block `pend` (issued last) stream into (Ap, Bp)
  // during the first k-steps.  Once every wave has its last fragments of
  // this block in registers (barrier), (Ac, Bc) are free and part 0 of the
  // block NS steps ahead starts streaming into them.  Blocks past the end
  // re-load the last block (no branch; never read).
  auto block = [&](int pend, u32x4* Ap, u32x4* Bp, int next, u32x4* Ac, u32x4* Bc,
                   const u32x4* An, const u32x4* Bn) {
    load_frags(fa1, fb1, Ac, Bc, 1);
    if (NPART > 1) issue(pend, Ap, Bp, 1);
    mma(fa0, fb0);
    sched_groups<N_MMA, N_DS, (NPART > 1 ? P1 : 0)>();
    load_frags(fa0, fb0, Ac, Bc, 2);
    if (NPART > 2) issue(pend, Ap, Bp, 2);
    mma(fa1, fb1);
    sched_groups<N_MMA, N_DS, (NPART > 2 ? P2 : 0)>();
    load_frags(fa1, fb1, Ac, Bc, 3);
    if (NPART > 3) issue(pend, Ap, Bp, 3);
    mma(fa0, fb0);
    sched_groups<N_MMA, N_DS, (NPART > 3 ? P3 : 0)>();
    stage_sync<NS == 3 ? N_VM : 0>();   // block kb+1 landed (with NS = 3 kb+2 may fly)
    issue(next, Ac, Bc, 0);
    load_frags(fa0, fb0, An, Bn, 0);
    mma(fa1, fb1);
    sched_groups<N_MMA, N_DS, P0>();
  };

  if constexpr (NS == 3) {
    // Three-stage ring (tiles of at most 128 rows, which stream their
    // weights: two blocks in flight while one is computed).
    issue_all(0, As0, Bs0);
    issue_all(min(1, nk - 1), As1, Bs1);
    issue(min(2, nk - 1), As2, Bs2, 0);
    stage_sync<N_VM + P0>();   // block 0 landed
    load_frags(fa0, fb0, As0, Bs0, 0);
    int kb = 0;
    for (; kb + 3 <= nk; kb += 3) {
      block(min(kb + 2, nk - 1), As2, Bs2, min(kb + 3, nk - 1), As0, Bs0, As1, Bs1);
      block(min(kb + 3, nk - 1), As0, Bs0, min(kb + 4, nk - 1), As1, Bs1, As2, Bs2);
      block(min(kb + 4, nk - 1), As1, Bs1, min(kb + 5, nk - 1), As2, Bs2, As0, Bs0);
    }
    if (kb < nk) block(nk - 1, As2, Bs2, nk - 1, As0, Bs0, As1, Bs1);
    if (kb + 1 < nk) block(nk - 1, As0, Bs0, nk - 1, As1, Bs1, As2, Bs2);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    issue_all(0, As0, Bs0);
    issue(min(1, nk - 1), As1, Bs1, 0);
    stage_sync<P0>();   // block 0 landed
    load_frags(fa0, fb0, As0, Bs0, 0);
    int kb = 0;
    for (; kb + 2 <= nk; kb += 2) {
      block(min(kb + 1, nk - 1), As1, Bs1, min(kb + 2, nk - 1), As0, Bs0, As1, Bs1);
      block(min(kb + 2, nk - 1), As0, Bs0, min(kb + 3, nk - 1), As1, Bs1, As0, Bs0);
    }
    if (kb < nk) block(nk - 1, As1, Bs1, nk - 1, As0, Bs0, As1, Bs1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
      __builtin_amdgcn_sched_barrier(0);
      const int m = wm * WM + mb * 32 + l32;
      if (m >= rows) continue;
      bf16_t* orow = out + (size_t)(row0 + m) * a.ldo + col_off;
#pragma unroll
      for (int nb = 0; nb < HALF_NB; ++nb) {
        // inner is a multiple of 64: a 32-column block is all in or all out.
        const int inner = inner0 + wn * (WN / 2) + nb * 32;
        if (inner >= a.inner) continue;
        uint32_t p[4][2];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            h[q] = silu_f(acc[nb][mb][4 * g + q]) * acc[nb + HALF_NB][mb][4 * g + q];
          p[g][0] = pack2(h[0], h[1]);
          p[g][1] = pack2(h[2], h[3]);
        }
        swap_halves(p);
        store_block(orow + inner + 8 * hi, p);
      }
    }
  } else if (MODE == 3) {
    // SwiGLU backward on the recomputed pre-activations a1 (W1 half) and a3:
    //   h = silu(a1) a3, dh = g gin,
    //   da1 = dh a3 sig(a1) (1 + a1 (1 - sig(a1))), da3 = dh silu(a1),
    // and the row's share of dg = sum gin h over this tile's inner columns,
    // summed over the lane's columns, the two lane halves and the tile's
    // waves in a fixed order.
    constexpr int HALF_NB = NB / 2;
    const int col_off = routed ? 0 : grp * a.inner;          // H and gin columns
    const int da_off = routed ? 0 : grp * 2 * a.inner;       // dA columns
    bf16_t* out = static_cast<bf16_t*>(a.out);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      __builtin_amdgcn_sched_barrier(0);
      const int m = wm * WM + mb * 32 + l32;
      const bool live = m < rows;
      const int row = row0 + min(m, rows - 1);
      const float g = (routed && a.row_g) ? a.row_g[row] : 1.f;
      const float* grow = a.gin + (size_t)row * a.ldgin + col_off;
      bf16_t* orow = out + (size_t)row * a.ldo + col_off;
      bf16_t* darow = a.da + (size_t)row * a.ldda + da_off;
      float part = 0.f;
#pragma unroll
      for (int nb = 0; nb < HALF_NB; ++nb) {
        // inner is a multiple of 64: a 32-column block is all in or all out.
        const int ib = inner0 + wn * (WN / 2) + nb * 32;
        if (ib >= a.inner) continue;
        uint32_t ph[4][2], p1[4][2], p3[4][2];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int inner = ib + 8 * q4 + 4 * hi;
          const float4 gv = *reinterpret_cast<const float4*>(grow + inner);
          const float gi[4] = {gv.x, gv.y, gv.z, gv.w};
          float hv[4], d1[4], d3[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float a1 = acc[nb][mb][4 * q4 + q];
            const float a3 = acc[nb + HALF_NB][mb][4 * q4 + q];
            const float sg = __builtin_amdgcn_rcpf(
                1.f + __builtin_amdgcn_exp2f(a1 * -1.4426950408889634f));
            const float sl = a1 * sg;
            hv[q] = sl * a3;
            part = fmaf(gi[q], hv[q], part);
            const float dh = g * gi[q];
            d1[q] = dh * a3 * (sg * (1.f + a1 * (1.f - sg)));
            d3[q] = dh * sl;
          }
          ph[q4][0] = pack2(g * hv[0], g * hv[1]);
          ph[q4][1] = pack2(g * hv[2], g * hv[3]);
          p1[q4][0] = pack2(d1[0], d1[1]);
          p1[q4][1] = pack2(d1[2], d1[3]);
          p3[q4][0] = pack2(d3[0], d3[1]);
          p3[q4][1] = pack2(d3[2], d3[3]);
        }
        swap_halves(ph);
        swap_halves(p1);
        swap_halves(p3);
        if (!live) continue;
        store_block(orow + ib + 8 * hi, ph);
        store_block(darow + ib + 8 * hi, p1);
        store_block(darow + a.inner + ib + 8 * hi, p3);
      }
      if (routed && a.dg_part) {
        part = sum_halves(part);
        if (hi == 0) red[wn * BM + m] = part;
      }
    }
    if (routed && a.dg_part) {
      __syncthreads();
      for (int m = threadIdx.x; m < rows; m += NW * 64) {
        float sum = 0.f;
        for (int w = 0; w < WAVES_N; ++w) sum += red[w * BM + m];
        a.dg_part[(size_t)(row0 + m) * a.n_part + nt] = sum;
      }
    }
  } else {
    down_epilogue<MODE, MB, NB, WM, WN>(a, acc, row0, rows, n0, wm, wn, l32, hi);
  }
}

// Tile `blk` of `nblk` of a stage-MODE part: M-tile mt, N-tile nt; false
// for the padding blocks.  Routed launches are sized for the most M-tiles any
// routing can make; the tiles are numbered over the M-tiles the routing did
// make, so the blocks past them (which exit at once) are the last ones and
// every XCD gets an equal share of real tiles.
// Tile order: N-tiles in groups of NGRP; inside a group the NGRP N-tiles of
// one M-tile are adjacent, then the next M-tile (same expert, same weight
// tiles).  A run of adjacent tiles (one XCD's resident set) then shares both
// its token-row tiles and its weight tiles in L2.
template <int MODE, int BM>
__device__ __forceinline__ bool tile_of(const GemmArgs& a, int blk, int nblk, int& mt,
                                        int& nt) {
  const bool routed = !(MODE == 2 || (is_gateup<MODE>() && a.shared));
  const int mdim = routed ? *a.n_tiles : (a.T + BM - 1) / BM;
  const int ndim = n_tiles_of<MODE, BM>(a);
  const int ntl = mdim * ndim;
  const int L = !routed ? xcd_remap(blk, nblk) : (blk < ntl ? xcd_remap(blk, ntl) : ntl);
  if (L >= ntl) return false;                // padding
  constexpr int NGRP = ngrp_for<BM>();
  const int full = ndim / NGRP;
  const int ntg = L / (mdim * NGRP);
  const int g = (ntg < full) ? NGRP : ndim - full * NGRP;
  const int rem = L - ntg * mdim * NGRP;
  mt = rem / g;
  nt = ntg * NGRP + rem % g;
  return true;
}

// One part of a grouped GEMM launch: block `blk` of `nblk` runs one tile of
// stage MODE.  An expert's last routed tile (its remaining rows) runs the
// smallest layout that holds them: 64, 128 or 192 rows in the 256-row
// launches, half height in the others, with matrix work in proportion.
template <int MODE, int BM, int WAVES_M, int NW, int NS>
__device__ __forceinline__ void gemm_part(const GemmArgs& a, int blk, int nblk, u32x4* As0,
                                          u32x4* As1, u32x4* As2, u32x4* Bs0, u32x4* Bs1,
                                          u32x4* Bs2, float* red) {
  const bool routed = !(MODE == 2 || (is_gateup<MODE>() && a.shared));
  int mt, nt;
  if (!tile_of<MODE, BM>(a, blk, nblk, mt, nt)) return;
  if (routed) {
    const MTile t = a.tiles[mt];
    if constexpr (BM == 256) {
      // An expert's last tile at 64-row granularity: 64, 128 or 192 rows.
      if (t.rows <= 64) {
        gemm_tile<MODE, 64, NW / 4, NS, NW>(a, t.row0, t.rows, t.expert, nt, As0, As1, As2,
                                            Bs0, Bs1, Bs2, red);
        return;
      }
      if (t.rows <= 128) {
        gemm_tile<MODE, 128, NW / 4, NS, NW>(a, t.row0, t.rows, t.expert, nt, As0, As1, As2,
                                             Bs0, Bs1, Bs2, red);
        return;
      }
      if (t.rows <= 192) {
        gemm_tile<MODE, 192, 2, NS, NW>(a, t.row0, t.rows, t.expert, nt, As0, As1, As2, Bs0,
                                        Bs1, Bs2, red);
        return;
      }
    } else if constexpr (BM >= 128) {
      if (t.rows <= BM / 2) {
        gemm_tile<MODE, BM / 2, NW / 4, NS, NW>(a, t.row0, t.rows, t.expert, nt, As0, As1,
                                                As2, Bs0, Bs1, Bs2, red);
        return;
      }
    }
    gemm_tile<MODE, BM, WAVES_M, NS, NW>(a, t.row0, t.rows, t.expert, nt, As0, As1, As2, Bs0,
                                         Bs1, Bs2, red);
  } else {
    const int row0 = mt * BM;
    gemm_tile<MODE, BM, WAVES_M, NS, NW>(a, row0, min(BM, a.T - row0), 0, nt, As0, As1, As2,
                                         Bs0, Bs1, Bs2, red);
  }
}

// The grouped GEMM: one workgroup per tile.  A launch holds up to two parts:
// blocks [0, a_blocks) run stage MODE on `a` (the routed experts), the rest
// stage MODE_B on `b` (the shared experts), so the shared tiles fill the GPU
// beside the routed ones.  a_blocks is a multiple of 8: blocks are dealt
// round-robin over the 8 XCDs, so both parts' tile orders stay XCD-aware.
template <int MODE, int MODE_B, int BM, int WAVES_M, int NW>
__global__ __launch_bounds__(NW * 64, 1) void gemm_bf16_kernel(GemmArgs a, GemmArgs b,
                                                               int a_blocks) {
  // Two LDS buffers per operand as distinct objects: accesses name their
  // buffer statically, so the compiler can tell the direct loads into one
  // buffer from the operand reads of the other and need not wait between.
  // Tiles of at most 128 rows stream their weights and keep three stages
  // in flight-or-compute (3 x (BM + 256) x 128 B <= 144 KB of LDS).
  constexpr int NS = (BM <= 128) ? 3 : 2;
  const int blk = blockIdx.x;
  __shared__ u32x4 As0[BM * 8], As1[BM * 8], As2[NS == 3 ? BM * 8 : 1];
  __shared__ u32x4 Bs0[BN * 8], Bs1[BN * 8], Bs2[NS == 3 ? BN * 8 : 1];
  // Row sums of GATEUP_BWD (the A buffers are free by the epilogue, but a
  // separate array keeps the buffers' accesses static).
  __shared__ float red[MODE == 3 ? 4 * BM : 1];
  // Each part reads its own argument struct (a run-time choice of struct
  // made the compiler copy both to scratch memory).
  if (blk >= a_blocks)
    gemm_part<MODE_B, BM, WAVES_M, NW, NS>(b, blk - a_blocks, (int)gridDim.x - a_blocks, As0,
                                           As1, As2, Bs0, Bs1, Bs2, red);
  else
    gemm_part<MODE, BM, WAVES_M, NW, NS>(a, blk, a_blocks, As0, As1, As2, Bs0, Bs1, Bs2, red);
}

// Blocks of one part: the routed M-tile bound (or the shared experts' row
// tiles) times the part's N-tiles.
template <int MODE, int BM>
int part_blocks(const GemmArgs& g) {
  const bool routed = !(MODE == 2 || (is_gateup<MODE>() && g.shared));
  const int mdim = routed ? g.max_mtiles : (g.T + BM - 1) / BM;
  return mdim * n_tiles_of<MODE, BM>(g);
}

template <int MODE, int MODE_B, int BM, int WAVES_M, int NW>
void launch_pair(const GemmArgs& a, const GemmArgs* b, hipStream_t s) {
  if (!b) {
    hipLaunchKernelGGL((gemm_bf16_kernel<MODE, MODE, BM, WAVES_M, NW>),
                       dim3(part_blocks<MODE, BM>(a)), dim3(NW * 64), 0, s, a, a,
                       part_blocks<MODE, BM>(a));
    return;
  }
  const int na = (part_blocks<MODE, BM>(a) + 7) & ~7;
  const int nb = part_blocks<MODE_B, BM>(*b);
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, MODE_B, BM, WAVES_M, NW>), dim3(na + nb),
                     dim3(NW * 64), 0, s, a, *b, na);
}

// Waves per workgroup: the 256-row gate/up tiles (forward and backward) run
// eight waves, two per SIMD, each with a 128 x 64 sub-tile (measured: shared
// gate/up -3%, backward gate/up -6%, routed gate/up even); the
// down-projections keep four waves of 128 x 128 (eight measured even).
// Tiles of at most 128 rows keep four waves.
template <int BM, int WAVES_M>
void launch_bm(const GemmArgs& a, const GemmArgs* b, hipStream_t s) {
  constexpr int NWG = (BM == 256) ? 8 : 4;
  if (a.mode == 0) launch_pair<0, 0, BM, WAVES_M, NWG>(a, b, s);
  else if (a.mode == 1) launch_pair<1, 2, BM, WAVES_M, 4>(a, b, s);
  else launch_pair<3, 3, BM, WAVES_M, NWG>(a, b, s);
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s, const GemmArgs* b) {
  // DOWN_SHARED runs only as the second part of a DOWN launch.
  if (a.mode == 2 || (b && (b->bm != a.bm || (a.mode == 1 ? b->mode != 2 : b->mode != a.mode))))
    return hipErrorInvalidValue;
  switch (a.bm) {
    case 256: launch_bm<256, 2>(a, b, s); break;
    case 128: launch_bm<128, 1>(a, b, s); break;
    case 64: launch_bm<64, 1>(a, b, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
