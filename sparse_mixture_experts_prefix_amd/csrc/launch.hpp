// Kernel launchers (host functions defined next to their kernels).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace moe {

// Records a HIP error as the text moe_strerror(MOE_ERR_HIP) returns on this
// thread and returns MOE_ERR_HIP.
int record_hip_error(hipError_t e);

// moe_forward's host checks of every argument but the workspace: an error
// code, or MOE_OK (also for T == 0, where the call does nothing).
int check_forward_args(const moe_shape* shape, const moe_weights* w, const float* y,
                       const int32_t* topk_ids, const float* topk_w);

// Router: logits = x W_g^T (+ bias) in fp32, top-k, softmax over the chosen.
// sel (or NULL): selection-only bias, added to the keys of the top-k only.
hipError_t launch_router(const uint16_t* x, const uint16_t* w_g, const float* bias, const float* sel,
                         int T, int D, int E, int k, int32_t* ids, float* wts, hipStream_t s);

// Few tokens: the router's work per 16 tokens is split over router_parts(D)
// workgroups, which write partial logits [P][T][E] (fp32).
hipError_t launch_router_partial(const uint16_t* x, const uint16_t* w_g, int T, int D, int E,
                                 float* partial, hipStream_t s);
// ... and one wave per token adds them (part order) and the bias, and picks
// the top-k and the softmax over the chosen: the same ids and weights as
// launch_router, bitwise, for E <= kSmallRouteE.
hipError_t launch_route_finish(const float* partial, int P, int T, int E, int k, const float* bias,
                               const float* sel, int32_t* ids, float* wts, hipStream_t s);

// Expert grouping of the assignments (see moe_align in moe.h).
// E groups hold experts id_base .. id_base+E-1 (ids outside get no row).
hipError_t launch_align(const int32_t* ids, int T, int k, int E, int id_base, int BM, int shared_rows,
                        int32_t* counts, int32_t* offsets, int32_t* padded, int32_t* sorted_assign,
                        int32_t* row_of, int32_t* row_token, int32_t* tile_group, int32_t* n_tiles,
                        hipStream_t s);

// out[0..n) = v (a kernel, not a memset, so it is safe in a captured graph).
hipError_t launch_fill_i32(int32_t* out, int64_t n, int32_t v, hipStream_t s);

struct GroupedGemm {
  const uint16_t* A;          // gate/up: x [T, D] (rows gathered by row_token); down: H
  const int32_t* row_token;   // gate/up only
  int64_t lda;                // elements
  const void* B_routed;       // w_gate_up [E, 2F, D] or w_down [E, D, F]
  const void* B_shared;       // ws_gate_up [2Fs, D] or ws_down [D, Fs]; NULL without shared
  int fp8;                    // B holds E4M3 bytes with one fp32 scale per row (else bf16)
  const float* S_routed;      // fp8: row scales [E, 2F] or [E, D]
  const float* S_shared;      // fp8: row scales [2Fs] or [D]
  int E;
  int N_routed, N_shared;     // output columns (gate/up: F, Fs; down: D, D)
  int K_routed, K_shared;     // reduction length (gate/up: D, D; down: F, Fs)
  const int32_t* tile_group;  // group of each BM-row tile
  const int32_t* n_tiles;     // device count of valid tiles
  int64_t max_tiles;          // host upper bound of n_tiles
  int64_t min_tiles;          // host lower bound of n_tiles when every id is valid
  int64_t busy_tiles;         // host estimate of row tiles that hold rows (sizes decode column tiles)
  void* C;                    // gate/up: H bf16; down: Yp fp32
  int64_t ldc;                // elements
  int BM;
  const int32_t* group_count;   // rows of each group
  const int32_t* group_padded;  // first padded row of each group
  int64_t a_bytes;              // bytes addressable through A (gate/up: all of x)
  int stream_b;                 // prefill gate/up: weight loads non-temporal (groups of ~1 m-tile)
  int64_t n_tiles_n;            // set by the launcher
  // Prefill only: workgroups that run at once (0: never split a tile over K)
  // and room for that many fp32 partial tiles of BM x BN (row-major)
  int ctas;
  float* partial;
  // Gate/up only: when set, g and u of every valid row are also stored, bf16,
  // row r at gu_out + r * ld_gu as [g (N) | u (N)] (kept for the backward pass)
  uint16_t* gu_out;
  int64_t ld_gu;
  // Down (rows x weight) kernels, bf16 only: B_routed / B_shared are stored
  // K-major, [K][N] per group (row k holds the N weights that multiply
  // column k of A), instead of [N][K]
  int b_kmajor;
};

// 256 x 256 x 64 tiles for BM = 256 (prefill-sized groups); each launches
// the GEMM and, when ctas > 0, the kernel that finishes split tiles.
hipError_t launch_gemm_gate_up_prefill(const GroupedGemm& g, hipStream_t s);
hipError_t launch_gemm_down_prefill(const GroupedGemm& g, hipStream_t s);
// Weight-streaming tiles for BM = 16 or 32 (decode-sized groups).
hipError_t launch_gemm_gate_up_decode(const GroupedGemm& g, hipStream_t s);
hipError_t launch_gemm_down_decode(const GroupedGemm& g, hipStream_t s);

// Weight gradients of the grouped GEMMs: for each group g (E routed, then
// the shared one when G > E), C_g[m][n] = sum over the group's rows r in
// [padded[g], padded[g] + counts[g]) of A[m][r] * B[n][r].  A: rows_a rows,
// B: rows_b rows, both bf16 with row stride ld; the group's padding rows hold
// zeros (the K loop reads whole 8-element chunks).
// Weight gradients: per group C[m][n] = sum over its rows r of A[r][m] B[r][n]
// (A, B: bf16 row buffers of the layer's padded rows, row strides lda, ldb).
struct WgradGemm {
  const uint16_t* A;
  const uint16_t* B;
  int64_t lda, ldb;
  int M_routed, N_routed, M_shared, N_shared;
  int E, G;
  const int32_t* padded;  // first row of each group
  const int32_t* counts;  // rows of each group
  float* C_routed;  // [E][M_routed][N_routed]
  float* C_shared;  // [M_shared][N_shared]
  int64_t tiles_m, tiles_n;  // 256 x 256 tiles per group (max over both kinds)
  // > 0 only when every group has at most 64 rows: that many workgroups walk
  // the tiles, each issuing the next tile's loads before storing the current one
  int one_stage_ctas;
};
hipError_t launch_gemm_wgrad(const WgradGemm& g, hipStream_t s);

// ---- backward pass (backward.hip)
// The rows of one backward call: align outputs and per-row buffers.
struct BwdRows {
  int64_t cap;                 // allocated rows
  const int32_t* total;        // padded[G] on the device: rows in use
  const int32_t* row_token;
  const int32_t* row_assign;
  const int32_t* padded;
  const int32_t* tile_group;
  const float* topk_w;         // [T k]
  const float* dy;             // [T][D]
  int E, BM, D, F, Fs, ldh;
  const float* gu;             // [cap][2 ldh] (recomputed), or NULL when gu16 is set
  const uint16_t* gu16;        // [cap][2 ldh] bf16, kept by a training forward
  uint16_t* dgu_w;             // [cap][2 ldh], written by the SwiGLU backward
};
hipError_t launch_gather_rows(const void* src, bool src_f32, const int32_t* row_token,
                              const int32_t* total, int64_t cap, int D, uint16_t* dst, hipStream_t s);
hipError_t launch_row_assign(const int32_t* row_of, int A, int64_t cap, int32_t* row_assign,
                             hipStream_t s);
hipError_t launch_fill_f32(float* out, int64_t n, hipStream_t s);
// dst[r][c] (bf16, row stride ld) of rows r in use, c < C (C % 8 == 0);
// kind 0: p_r dy[t_r], 1: bf16(SiLU(g) u)
hipError_t launch_rows(const BwdRows& b, int kind, int C, uint16_t* dst, int64_t ld, hipStream_t s);
hipError_t launch_swiglu_bwd(const BwdRows& b, const float* dhp, float* dp, hipStream_t s);
hipError_t launch_router_bwd(const float* topk_w, const float* dp, int T, int k, float* dl,
                             hipStream_t s);
hipError_t launch_router_wgrad(const float* dl, const uint16_t* x, const int32_t* offsets,
                               const int32_t* sorted_assign, int E, int k, int D, int bias_grad,
                               float* dwg, float* dbias, hipStream_t s);
hipError_t launch_combine_bwd(const float* dxr, const int32_t* row_of, const int32_t* ids,
                              const float* dl, const uint16_t* w_g, const int32_t* padded, int T, int D,
                              int k, int E, int has_shared, float* dx, hipStream_t s);

// y[t] = sum_j w[t,j] * Yp[row_of[t*k+j]] (+ Yp[shared_base + t]) in fixed order.
hipError_t launch_combine(const float* Yp, const int32_t* row_of, const float* wts,
                          const int32_t* padded, int T, int D, int k, int E, int has_shared,
                          float* y, hipStream_t s);

}  // namespace moe
