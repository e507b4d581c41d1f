// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------------------
// Element helpers
// ---------------------------------------------------------------------------
typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays a quiet NaN).
// fp32 -> bf16, round to nearest even (NaN stays NaN): the hardware
// conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Load one element as fp32 / store fp32 as the element type.
template <typename T> __device__ __forceinline__ float ld_f32(const T* p);
template <> __device__ __forceinline__ float ld_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld_f32<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(*p);
}
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  return f32_to_bf16(v);
}

// ---------------------------------------------------------------------------
// Workspace layout (byte offsets; -1 = absent)
// ---------------------------------------------------------------------------
struct Layout {
  int64_t topk_idx, topk_w, rank, block_counts, block_base, counts, offsets,
      tiles, n_tiles, slot_row, row_src, xp, h_routed, h_shared, y, y_scale, s,
      planes, plog, x_q, x_scale, h_routed_scale, h_shared_scale, total;
  int32_t ds, ep;     // router: d-slices, logit row stride
  int32_t nblk;       // router workgroups (histogram blocks)
  int32_t bm;         // rows per GEMM M-tile
  int32_t max_mtiles; // upper bound on routed M-tiles
};

// Tile of the routed grouped GEMMs: rows [row0, row0 + rows) of expert e.
struct MTile {
  int32_t expert, row0, rows, pad;
};

constexpr int MAX_EXPERTS = 256;
constexpr int MAX_TOPK = 32;
constexpr int MAX_GROUPS = 64;

// ---------------------------------------------------------------------------
// Launchers (each in the .hip file that holds its kernel)
// ---------------------------------------------------------------------------
struct ScanArgs {
  const int32_t* block_counts; int32_t* block_base; int32_t* counts;
  int32_t* user_counts; int32_t* offsets; MTile* tiles; int32_t* n_tiles;
  int nblk, E, bm;
};

struct RouterArgs {
  const void* x; int dtype;   // 0 = f32, 1 = bf16
  const float* w_gate; const float* logit_bias; const float* select_bias;
  int T, d, E, K, score, n_groups, topk_groups, norm_topk;
  float routed_scale;
  int ds, ep;                 // d-slices of the logits GEMM; logit row stride
  bf16_t* planes;             // [3][E][d] gate split into bf16 parts (bf16 x)
  float* plog;                // [ds][T][ep] partial logits
  float* logits;              // or NULL: [T][ep] logits before the logit bias (fused and
                              // small-batch paths; the split path leaves them in plog)
  int32_t* topk_idx; float* topk_w; int32_t* rank; int32_t* block_counts;
};
struct LogitsArgs {
  const bf16_t* x; const float* xf; const bf16_t* planes; const float* w_gate;
  int T, d, E, ep, ds;
  float* plog;
};
struct SelectArgs {
  const float* plog; int ep, ds;
  float* logits;              // or NULL: the summed logits before the bias, [T][ep]
  const float* logit_bias; const float* select_bias;
  int T, E, K, score, n_groups, topk_groups, norm_topk;
  float routed_scale;
  int32_t* topk_idx; float* topk_w; int32_t* rank; int32_t* block_counts;
};
hipError_t launch_router(const RouterArgs& a, hipStream_t s);
// Tokens per histogram block (dtype: 0 = f32, 1 = bf16 x).
int router_tokens_per_block(int T, int E, int d, int dtype);
int router_dsplit(int T, int E, int d, int dtype);   // d-slices of the logits GEMM
// True when logits and selection run fused (no partial-logit buffer).
bool router_fused(int T, int E, int K, int n_groups, int dtype);
// True when small batches route with the fused 16-token kernel, and its
// hidden-dimension slices (partial logits [slices][T][ep] in plog).
bool router_small(int T, int E, int d, int dtype);
int router_small_slices(int d);

hipError_t launch_zero_counts(int32_t* counts, int n, hipStream_t s);

struct PermuteArgs {
  int T, K, E, rt, nblk;   // rt: tokens per router block
  const int32_t* topk_idx; const int32_t* rank; const int32_t* block_base;
  const int32_t* offsets; int32_t* slot_row; int32_t* row_src;
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// The dispatch scan; with `p`, also the permute in the same launch (at most
// SCAN_PERMUTE_MAX_SLOTS slots T K).
constexpr int64_t SCAN_PERMUTE_MAX_SLOTS = 8192;
hipError_t launch_scan(const ScanArgs& a, hipStream_t s, const PermuteArgs* p = nullptr);

// Grouped GEMM stages.
//  GATEUP : H[r][c] = silu(A W1^T) * (A W3^T)   A = xp rows (routed) or x (shared)
//  DOWN   : Y[r][n] = H W2^T                     routed rows (fp32 out)
//  DOWN_SHARED : S[t][n] = x[t][n] + sum_s H_s W2_s^T   (fp32)
struct GemmArgs {
  int mode;           // 0 GATEUP, 1 DOWN, 2 DOWN_SHARED, 3 GATEUP_BWD
  bool shared;        // GATEUP: the shared-expert group (rows = tokens)
  const void* a; int lda;        // activation rows
  const int32_t* a_rows;         // optional: source row of each tile row
                                 // (gathers token rows of x; NULL = contiguous)
  const void* w1; const void* w3; const void* w2;
  int d, inner, n_experts;       // inner of the group; n_experts in group
  void* out; int ldo;            // H (dtype) / Y / S (f32)
  // bf16 layers: routed Y is stored as fp16 scaled by a power of two per 64
  // columns of a row; yscale[row][d / 64] holds the inverse scales (written
  // by DOWN, read by the combine).  fp32 layers: Y is fp32.
  float* yscale;
  const void* x;                 // DOWN_SHARED residual
  const MTile* tiles; const int32_t* n_tiles; int max_mtiles;
  int T;                          // rows for shared group
  int bm;
  // FP8 layers (E4M3 operands, power-of-two scales stored as bytes b, value
  // 2^(b - 127)): a_scale[row][k / 128] of the activation rows (rows of x for
  // gathered tiles), weight scales per 128 x 128 block (s1, s3
  // [E][inner / 128][d / 128], s2 [E][d / 128][inner / 128]), and GATEUP's
  // output scales out_scale[row][col / 128].
  const uint8_t* a_scale; int lda_s;
  const uint8_t* s1; const uint8_t* s3; const uint8_t* s2;
  uint8_t* out_scale; int ldo_s;
  // GATEUP_BWD (bf16): the gate/up pre-activations a1, a3 are recomputed
  // and the SwiGLU backward applied in the epilogue, from gin[row][col]
  // (fp32, = dy W2 of the row, before the gate weight) and the row's gate
  // weight row_g[row] (NULL: 1, the shared experts):
  //   out[row][col] = g h  (bf16),  da[row][col] = g gin a3 silu'(a1),
  //   da[row][col + inner] = g gin silu(a1)  (bf16, per expert of the group
  //   at 2 inner columns per expert), dg_part[row][tile] = sum gin h over
  //   the tile's inner columns (fp32, routed rows only).
  const float* gin; int ldgin;
  const float* row_g;
  bf16_t* da; int ldda;
  float* dg_part; int n_part;
};
// One launch of stage a.mode on `a`, plus, when `b` is given, the shared
// experts' tiles of the same stage in the same launch (b->mode == a.mode for
// GATEUP / GATEUP_BWD; DOWN takes a DOWN_SHARED part writing S).
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s, const GemmArgs* b = nullptr);

// Grouped GEMMs of the backward pass (bf16 operands, fp32 results), C = A B
// with either operand k-major (rows of the operand hold consecutive k) or
// mn-major (rows hold consecutive m or n; read through LDS transpose loads).
//   KIND 0  G  = dy W2          M = rows of an expert, N = inner, K = d
//   KIND 1  dX = dA [W1; W3]    M = rows,  N = d,  K = 2 inner (per expert)
//   KIND 2  dW2 = dy^T Hg       M = d,     N = inner, K = rows of the expert
//   KIND 3  [dW1; dW3] = dA^T X M = 2 inner, N = d, K = rows of the expert
// Routed groups are the experts (rows from the tile list / offsets, token
// rows through row_src); the shared group has all T tokens in order and
// n_experts experts side by side (KIND 0, 2, 3: one expert per group index;
// KIND 1: all shared experts along k).
struct BwdGemmArgs {
  int kind;
  bool shared;
  int T, d, inner, n_experts;       // inner of the group's experts
  const MTile* tiles; const int32_t* n_tiles; int max_mtiles;   // routed KIND 0/1
  const int32_t* offsets;           // routed KIND 2/3: rows of expert e
  const int32_t* row_src;           // routed: token of each row
  const bf16_t* dy;                 // [T][d]
  const bf16_t* x;                  // [T][d]
  const bf16_t* w1; const bf16_t* w3; const bf16_t* w2;   // the group's weights
  const bf16_t* da; int ldda;       // [rows][2 inner] (shared: per expert blocks)
  const bf16_t* hg; int ldhg;       // [rows][inner] g h (shared: per expert blocks)
  const bf16_t* zero;               // >= 512 zero bytes (k rows past the end)
  float* c; bf16_t* cx; int ldc;    // KIND 0: G [rows][ldc] (fp32); KIND 1: dX [rows][d] (bf16)
  float* dw1; float* dw3; float* dw2;   // KIND 2/3 outputs [experts][..][..]
  int splits;                       // KIND 2/3: k split into this many ranges (>= 1)
  float* part;                      // splits > 1: [splits][experts][M][N] partial sums
};
hipError_t launch_gemm_bwd(const BwdGemmArgs& a, hipStream_t s);

// Backward helpers (backward.hip).
struct BwdAuxArgs {
  int T, d, E, K, score, norm_topk;
  float routed_scale;
  const float* plog; int ds, ep;    // partial logits [ds][T][ep]
  const float* logit_bias;
  const float* w_gate;              // [E][d]
  const int32_t* topk_idx; const float* topk_w; const int32_t* slot_row;
  const float* dg_part; int n_part; // [rows][n_part]
  float* row_g;                     // [T K] gate weight of each row
  float* dg;                        // [T][K]
  float* dl;                        // [T][E] logit gradient
  float* dlogit_bias;               // [E] or NULL
  const bf16_t* x; const bf16_t* dy;
  bf16_t* dlp; int ldp;             // dl as bf16 hi and lo parts: [T][ldp], lo at ldp / 2
  float* dwg_part; int gg_splits;   // [gg_splits][ldp][d] partial gate gradients (hi rows, lo rows)
  float* dw_gate;                   // [E][d]
  const bf16_t* dx_rows;            // [T K][d]
  const bf16_t* dx_shared;          // [T][d] or NULL
  bf16_t* dx;                       // [T][d]
  bf16_t* zero; int n_zero;         // zero-filled at the start
};
hipError_t launch_bwd_prep(const BwdAuxArgs& a, hipStream_t s);      // row_g, zero
hipError_t launch_router_bwd(const BwdAuxArgs& a, hipStream_t s);    // dg, dl, dlogit_bias
hipError_t launch_gate_grad(const BwdAuxArgs& a, hipStream_t s);     // dw_gate
hipError_t launch_dx_combine(const BwdAuxArgs& a, hipStream_t s);    // dx
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
hipError_t launch_gemm_fp8(const GemmArgs& a, hipStream_t s, const GemmArgs* b = nullptr);

// E4M3 quantisation with power-of-two scales: rows of `src` [R][C] (bf16 or
// f32) per 1 x 128 (quant_rows), or [batch][R][C] per 128 x 128 block.
struct QuantArgs {
  const void* src; int src_f32;
  int64_t batch; int rows, cols;
  uint8_t* codes; uint8_t* scales;
};
hipError_t launch_quant_rows(const QuantArgs& a, hipStream_t s);
hipError_t launch_quant_blocks(const QuantArgs& a, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s);

struct CombineArgs {
  const void* base; bool base_f32;   // S (f32) or x (dtype) when no shared
  const void* y;                     // fp32 rows, or fp16 rows when yscale != NULL
  const float* yscale;               // [rows][d / 64] inverse scales of fp16 Y
  const float* topk_w; const int32_t* slot_row;
  void* out; int dtype; int T, d, K;
};

struct BiasUpdateArgs {
  const int32_t* counts; int n; float gamma;
  float* bias; float* rel_load;       // either may be NULL
};
hipError_t launch_bias_update(const BiasUpdateArgs& a, hipStream_t s);

// Columns sharing one scale in the fp16 routed-output rows of bf16 layers.
constexpr int Y_GROUP = 64;
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace moe
