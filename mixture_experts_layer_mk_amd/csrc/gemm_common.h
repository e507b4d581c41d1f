// Device helpers shared by the grouped expert GEMMs (bf16 and FP8): LDS
// swizzle, XCD-aware tile order, SwiGLU, output packing, the fp16 routed-output
// scales, instruction-scheduling groups and wait-count encodings.
#pragma once

#include "common.h"

namespace moe {
namespace gemm {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int BN = 256;   // weight rows per workgroup

// XOR applied to the chunk index of LDS row `row` (8 chunks per row):
// 8 consecutive rows, and 16 rows split by bank half, hit distinct banks.
__device__ __forceinline__ int swz_x(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Chunk swizzle of k-major LDS rows (32 k = 4 chunks of 16 B per row).  A
// fragment load reads the same chunk of consecutive rows; 8 consecutive
// rows span 512 B and 16 span 1 KB, and in either group the rows sharing a
// 128-byte (respectively 256-byte) bank window get 4 different chunks from
// f(r) = 2 r2 + (r1 ^ r3) (r_i: bit i of the row), so a pass over 8 or 16
// lanes hits each 16-byte bank group once.
__device__ __forceinline__ int swz_k(int r) {
  return (((r >> 2) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1);
}

__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, j = b >> 3, q = n >> 3, r = n & 7;
  return (x < r) ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}

// silu(v) = v * sigmoid(v) = v / (1 + e^-v), evaluated as v * rcp(1 + 2^(-v log2 e))
// with the hardware base-2 exponential and reciprocal (about 1 ulp each; the
// result is rounded to bf16 right after).  Large |v| saturates correctly:
// 2^+big = inf gives rcp = 0, 2^-big = 0 gives rcp(1) = 1.
__device__ __forceinline__ float silu_f(float v) {
  const float e = __builtin_amdgcn_exp2f(v * -1.4426950408889634f);
  return v * __builtin_amdgcn_rcpf(1.f + e);
}

// Two floats to packed bf16 (round to nearest even) in one conversion.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Two floats to packed fp16 (round to nearest even) and back.
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
// Max and sum over lanes l and l ^ 32, with one swap of the wave's halves (a
// VALU op) instead of a cross-lane read through LDS.  Both lanes combine the
// same two values, and max and + are commutative, so both get the same bits.
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lanes l and l + 32 of a wave hold the same output row of a 32-column block:
// lane half h (0 or 1) has columns 8 g + 4 h + {0, 1} in p[g][0] and {2, 3} in
// p[g][1], g = 0..3.  Two swaps between the halves (the low half's g = 1 and 3
// words for the high half's g = 0 and 2 words) leave each lane 8 consecutive
// columns per pair of g: the low half 0-7 and 16-23, the high half 8-15 and
// 24-31, as {p[0], p[1]} and {p[2], p[3]}, so the row is written with 16-byte
// stores.
__device__ __forceinline__ void swap_halves(uint32_t (&p)[4][2]) {
#pragma unroll
  for (int g = 0; g < 4; g += 2)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto r = __builtin_amdgcn_permlane32_swap(p[g][j], p[g + 1][j], false, false);
      p[g][j] = r[0];
      p[g + 1][j] = r[1];
    }
}
// The same for one-byte elements: p[g] holds columns 8 g + 4 h .. + 3.  The
// first round leaves the low half 0-7 and 16-23 (p[0], p[1] and p[2], p[3]),
// the high half 8-15 and 24-31; the second swaps the low half's 16-23 with the
// high half's 8-15, so the low half holds columns 0-15 and the high half
// 16-31, in p[0..3] order.
__device__ __forceinline__ void swap_halves_bytes(uint32_t (&p)[4]) {
#pragma unroll
  for (int g = 0; g < 4; g += 2) {
    const auto r = __builtin_amdgcn_permlane32_swap(p[g], p[g + 1], false, false);
    p[g] = r[0];
    p[g + 1] = r[1];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(p[j], p[j + 2], false, false);
    p[j] = r[0];
    p[j + 2] = r[1];
  }
}
__device__ __forceinline__ void store_block(void* row_at_8h, const uint32_t (&p)[4][2]) {
  uint4* q = static_cast<uint4*>(row_at_8h);
  q[0] = make_uint4(p[0][0], p[0][1], p[1][0], p[1][1]);   // columns 8 h .. 8 h + 7
  q[2] = make_uint4(p[2][0], p[2][1], p[3][0], p[3][1]);   // 16 + 8 h .. 16 + 8 h + 7
}

// The inverse: a lane's two 16-byte chunks of a row (at columns 8 h and
// 16 + 8 h of a 32-column block) as p[0..3], before swap_halves puts them in
// the accumulator layout.
__device__ __forceinline__ void load_block(const void* row_at_8h, uint32_t (&p)[4][2]) {
  const uint4* q = static_cast<const uint4*>(row_at_8h);
  const uint4 u = q[0], v = q[2];
  p[0][0] = u.x; p[0][1] = u.y; p[1][0] = u.z; p[1][1] = u.w;
  p[2][0] = v.x; p[2][1] = v.y; p[3][0] = v.z; p[3][1] = v.w;
}

__device__ __forceinline__ float h_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float h_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Scale of one 64-column group of a routed output row whose largest
// magnitude is amax: s = 2^(15 - E) with amax = f 2^E, f in [0.5, 1), so
// every scaled value is below 2^15 (inside fp16's range), and inv = 1 / s.
// Both are exact powers of two (E clamped so that both stay normal).
__device__ __forceinline__ void y_scale_of(float amax, float& s, float& inv) {
  int E = __builtin_amdgcn_frexp_expf(amax);
  E = min(max(E, -111), 141);
  s = __int_as_float((142 - E) << 23);
  inv = __int_as_float((112 + E) << 23);
}

// Instruction-scheduling groups for one k-step: N_MMA matrix ops with the
// N_DS LDS reads (of the next k-step) spread over the first half, so they
// land well before use, and N_VM global->LDS loads spread over all of them.
template <int N_MMA, int N_DS, int N_VM, int I = 0>
__device__ __forceinline__ void sched_groups() {
  if constexpr (I < N_MMA) {
    constexpr int S = (N_MMA / 2 > 0) ? N_MMA / 2 : 1;
    constexpr int ds = (I < S) ? (I + 1) * N_DS / S - I * N_DS / S : 0;
    constexpr int vm = (I + 1) * N_VM / N_MMA - I * N_VM / N_MMA;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // matrix op
    if constexpr (ds > 0) __builtin_amdgcn_sched_group_barrier(0x100, ds, 0);  // LDS read
    if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);  // VMEM
    sched_groups<N_MMA, N_DS, N_VM, I + 1>();
  }
}

// N-tiles per tile-order group, by tile height: BM / 64.  Measured on the
// layers each height is chosen for: 256-row tiles (16B-shaped) 4, with 2 and 8
// slower; 128-row tiles (V3-shaped) 2 against 4 -5.6% bf16 and -8% FP8, with 1
// slower; 64-row tiles (a skewed 128-token batch) 1 against 4 -6%.
template <int BM> constexpr int ngrp_for() { return BM >= 128 ? BM / 64 : 1; }

// s_waitcnt immediate that waits until at most N vector-memory operations
// are outstanding (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[5:4] in bits [15:14]; the other counters left at their maximum).
template <int N>
constexpr int vmcnt_imm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  return (N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14);
}

// Work-group barrier between pipeline stages: wait until at most N of this
// wave's vector-memory loads are outstanding (the direct-to-LDS loads of the
// stage about to be read have landed) and its LDS reads are done, then every
// wave meets.  Unlike __syncthreads(), whose work-group fence makes the
// compiler drain every outstanding vector-memory load here, this keeps the
// later stages' loads in flight.  The count wait is the builtin, which the
// compiler's wait insertion sees (so it adds no wait of its own for these
// loads after the barrier) and which no memory access is moved across; the
// barrier's memory clobber keeps LDS reads and loads on their side of it.
template <int N>
__device__ __forceinline__ void stage_sync() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<N>());
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Stages whose tiles are gate/up tiles (GATEUP and its backward).
template <int MODE>
constexpr bool is_gateup() { return MODE == 0 || MODE == 3; }

// N-tiles of one GEMM stage (GATEUP: 128 inner columns per tile, for each
// expert of the shared group; DOWN: 256 output columns per tile).
template <int MODE, int BM>
__host__ __device__ __forceinline__ int n_tiles_of(const GemmArgs& a) {
  const bool routed = !(MODE == 2 || (is_gateup<MODE>() && a.shared));
  if (is_gateup<MODE>()) return ((a.inner + BN / 2 - 1) / (BN / 2)) * (routed ? 1 : a.n_experts);
  return (a.d + BN - 1) / BN;
}

}  // namespace gemm
}  // namespace moe
