// Host-side argument checks and workspace layout of the MoE layer call.
// No HIP calls: this unit is plain C++ so its logic can be exercised on a
// machine without a GPU.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Few tokens (T <= kSmallRouteT, E <= kSmallRouteE): the router's 16 waves per
// 16 tokens are split over kRouterGroups workgroups of four waves, each
// writing its partial logits, and a per-token kernel finishes the routing.
constexpr int kSmallRouteT = 64;
constexpr int kSmallRouteE = 64;
constexpr int kRouterGroups = 4;
inline int router_parts(int64_t /*D*/) { return kRouterGroups; }

// Workgroups the prefill GEMMs balance their last round over (one per CU,
// at most this many), and so the number of partial tiles the workspace holds.
constexpr int kSplitCtas = 256;
// A partial tile: up to 256 + 32 rows (a 256-row tile with the next m-tile's
// few rows folded in) x 256 columns.
constexpr int64_t kPartialTileFloats = (256 + 32) * 256;

// Row-tile height of the grouped GEMMs and the per-call workspace layout.
struct Plan {
  int64_t T, D, E, F, k, Fs;
  int64_t e0, E_loc;  // experts held by this call: e0 .. e0+E_loc-1 (all E unless sharded)
  int G;              // groups: E_loc routed (+1 shared)
  int BM;             // row-tile height; every group is padded to a multiple of it
  int64_t A;          // assignments T*k
  int64_t cap_rows;   // upper bound of padded rows over all groups
  int64_t max_tiles;  // upper bound of BM-row tiles
  int64_t ldh;        // row stride (elements) of the hidden activations H: max(F, Fs)
  int fp8;            // expert weights are E4M3 codes with per-row scales
  // byte offsets inside the workspace
  size_t off_ids, off_w, off_counts, off_offsets, off_padded, off_ntiles, off_sorted, off_rowof,
      off_rowtoken, off_tilegroup, off_h, off_yp, off_partial, off_rpart, total;
  // training forward: the same layout, then g | u of every row (bf16 [cap][2 ldh])
  size_t off_gusave, total_train;
};

// Backward-pass workspace: the forward's layout (align outputs, split
// partials; Yp holds the per-row dx) followed by the backward's buffers.
// cap = P.cap_rows.
struct BwdPlan {
  Plan P;
  size_t off_rowa;          // int32 [cap]: assignment of each row, -1 elsewhere
  size_t off_xr, off_dyr;   // bf16 [cap][D]: x and dy rows in expert order
  size_t off_gu;            // fp32 [cap][2 ldh]: g | u recomputed
  size_t off_dhp;           // fp32 [cap][ldh]: W_down^T dy
  size_t off_dgu;           // bf16 [cap][2 ldh]: dg | du
  size_t off_dp, off_dl;    // fp32 [T k]
  size_t off_pdy, off_hr;   // bf16 [cap][D]: p dy rows; [cap][ldh]: h rows (recomputed g | u)
  size_t total;
};
int make_backward_plan(const moe_shape* s, BwdPlan* b);

// Shape checks shared by every entry point (MOE_OK or an error code).
int check_shape(const moe_shape* s);

// Tile height for a shape (assumes check_shape passed).
int choose_block_m(const moe_shape* s);

// Fill `p` for a valid shape; returns check_shape's code.
int make_plan(const moe_shape* s, Plan* p);

// Pointer checks of moe_forward / moe_forward_routed (routed: ids/w given).
int check_weights(const moe_shape* s, const moe_weights* w, bool need_router);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace moe
