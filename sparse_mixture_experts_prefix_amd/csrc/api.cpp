// extern "C" entry points of libmoe (declared and documented in moe.h).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>

#include "launch.hpp"
#include "moe.h"
#include "plan.hpp"

namespace {

thread_local char g_hip_msg[256] = "no HIP error recorded";

int hip_fail(hipError_t e) {
  std::snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return MOE_ERR_HIP;
}

}  // namespace

int moe::record_hip_error(hipError_t e) { return hip_fail(e); }

namespace {

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// Compute units of the current device, capped at the split workspace size:
// the prefill GEMMs balance their last round of tiles over this many
// workgroups (one resident per CU).
hipError_t split_ctas(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::atomic<int> cached[64];  // zero-initialised; every writer stores the same value
  if (dev >= 0 && dev < 64 && cached[dev].load(std::memory_order_relaxed) > 0) {
    *out = cached[dev].load(std::memory_order_relaxed);
    return hipSuccess;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int n = cus < moe::kSplitCtas ? cus : moe::kSplitCtas;
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

// Records events[i] on the stream when timing is requested.
struct Marks {
  void* const* ev;
  hipError_t mark(int i, hipStream_t s) const {
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), s) : hipSuccess;
  }
};

// Row tiles that hold rows, as the host can bound them: each assignment sits
// in at most one tile and each routed group's rows in ceil(rows / BM) tiles,
// so at most min(T k, E) tiles for groups of at most BM rows (decode), plus
// the shared expert's.
int64_t busy_tiles(const moe::Plan& P) {
  const int64_t routed = P.A < P.E_loc ? P.A : P.E_loc;
  const int64_t est = routed > (P.A + P.BM - 1) / P.BM ? routed : (P.A + P.BM - 1) / P.BM;
  return est + (P.Fs > 0 ? (P.T + P.BM - 1) / P.BM : 0);
}

// Everything after routing: align -> gate/up -> down -> combine.
// gu_save (or NULL): keep g | u of every row, bf16 [cap][2 ldh] (training forward)
int run_experts(const moe::Plan& P, const moe_weights* w, const int32_t* ids, const float* wts,
                float* y, void* ws, hipStream_t s, Marks mk = Marks{nullptr},
                uint16_t* gu_save = nullptr) {
  using namespace moe;
  int32_t* counts = at<int32_t>(ws, P.off_counts);
  int32_t* offsets = at<int32_t>(ws, P.off_offsets);
  int32_t* padded = at<int32_t>(ws, P.off_padded);
  int32_t* n_tiles = at<int32_t>(ws, P.off_ntiles);
  int32_t* sorted = at<int32_t>(ws, P.off_sorted);
  int32_t* row_of = at<int32_t>(ws, P.off_rowof);
  int32_t* row_token = at<int32_t>(ws, P.off_rowtoken);
  int32_t* tile_group = at<int32_t>(ws, P.off_tilegroup);
  uint16_t* H = at<uint16_t>(ws, P.off_h);
  float* Yp = at<float>(ws, P.off_yp);
  const int shared_rows = P.Fs > 0 ? (int)P.T : 0;
  const bool prefill = P.BM == 256;
  int ctas = 0;
  if (prefill) {
    hipError_t e0 = split_ctas(&ctas);
    if (e0 != hipSuccess) return hip_fail(e0);
  }

  hipError_t e = launch_align(ids, (int)P.T, (int)P.k, (int)P.E_loc, (int)P.e0, P.BM, shared_rows, counts, offsets,
                              padded, sorted, row_of, row_token, tile_group, n_tiles, s);
  if (e == hipSuccess) e = mk.mark(2, s);
  if (e != hipSuccess) return hip_fail(e);

  GroupedGemm gu{};
  gu.A = static_cast<const uint16_t*>(w->x);
  gu.row_token = row_token;
  gu.lda = P.D;
  gu.B_routed = w->w_gate_up;
  gu.B_shared = w->ws_gate_up;
  gu.fp8 = P.fp8;
  gu.S_routed = P.fp8 ? w->w_gate_up_scale : nullptr;
  gu.S_shared = P.fp8 ? w->ws_gate_up_scale : nullptr;
  gu.E = (int)P.E_loc;
  gu.N_routed = (int)P.F;
  gu.N_shared = (int)P.Fs;
  gu.K_routed = (int)P.D;
  gu.K_shared = (int)P.D;
  gu.tile_group = tile_group;
  gu.n_tiles = n_tiles;
  gu.max_tiles = P.max_tiles;
  gu.min_tiles = (P.A + P.BM - 1) / P.BM + (P.Fs > 0 ? (P.T + P.BM - 1) / P.BM : 0);
  gu.busy_tiles = busy_tiles(P);
  gu.C = H;
  gu.ldc = P.ldh;
  gu.BM = P.BM;
  gu.group_count = counts;
  gu.group_padded = padded;
  gu.a_bytes = P.T * P.D * 2;
  // expert groups of at most one m-tile and its folded rows on average: each
  // weight tile is read by one workgroup (measured on the DeepSeek shape:
  // gate/up 3.96 -> 3.82 ms; with four m-tiles per group, Mixtral shape,
  // the plain policy is 2.5% faster, and the down GEMM is too)
  gu.stream_b = P.A <= (int64_t)(P.BM + 32) * P.E;
  gu.ctas = ctas;
  gu.partial = prefill ? at<float>(ws, P.off_partial) : nullptr;
  gu.gu_out = gu_save;
  gu.ld_gu = 2 * P.ldh;
  e = P.BM == 256 ? launch_gemm_gate_up_prefill(gu, s) : launch_gemm_gate_up_decode(gu, s);
  if (e == hipSuccess) e = mk.mark(3, s);
  if (e != hipSuccess) return hip_fail(e);

  GroupedGemm dn = gu;
  dn.gu_out = nullptr;
  dn.stream_b = 0;
  dn.A = H;
  dn.row_token = nullptr;
  dn.lda = P.ldh;
  dn.B_routed = w->w_down;
  dn.B_shared = w->ws_down;
  dn.S_routed = P.fp8 ? w->w_down_scale : nullptr;
  dn.S_shared = P.fp8 ? w->ws_down_scale : nullptr;
  dn.N_routed = (int)P.D;
  dn.N_shared = (int)P.D;
  dn.K_routed = (int)P.F;
  dn.K_shared = (int)P.Fs;
  dn.C = Yp;
  dn.ldc = P.D;
  dn.a_bytes = P.cap_rows * P.ldh * 2;
  e = P.BM == 256 ? launch_gemm_down_prefill(dn, s) : launch_gemm_down_decode(dn, s);
  if (e == hipSuccess) e = mk.mark(4, s);
  if (e != hipSuccess) return hip_fail(e);

  e = launch_combine(Yp, row_of, wts, padded, (int)P.T, (int)P.D, (int)P.k, (int)P.E_loc,
                     P.Fs > 0 ? 1 : 0, y, s);
  if (e == hipSuccess) e = mk.mark(5, s);
  if (e != hipSuccess) return hip_fail(e);
  return MOE_OK;
}

// Backward pass for a given routing (see moe_backward in moe.h).
// saved (or NULL): the workspace of a training forward call with the same
// shape and routing: its grouping, g | u and h rows are used instead of
// redoing them (it is only read).
int run_backward(const moe::BwdPlan& B, const moe_shape* shape, const moe_weights* w,
                 const int32_t* ids, const float* wts, const float* dy, const moe_grads* gr,
                 void* ws, hipStream_t s, const void* saved = nullptr) {
  using namespace moe;
  const Plan& P = B.P;
  // the grouping: the saved forward's (read only) or this call's own
  void* grp = saved ? const_cast<void*>(saved) : ws;
  int32_t* counts = at<int32_t>(grp, P.off_counts);
  int32_t* offsets = at<int32_t>(grp, P.off_offsets);
  int32_t* padded = at<int32_t>(grp, P.off_padded);
  int32_t* n_tiles = at<int32_t>(grp, P.off_ntiles);
  int32_t* sorted = at<int32_t>(grp, P.off_sorted);
  int32_t* row_of = at<int32_t>(grp, P.off_rowof);
  int32_t* row_token = at<int32_t>(grp, P.off_rowtoken);
  int32_t* tile_group = at<int32_t>(grp, P.off_tilegroup);
  int32_t* row_assign = at<int32_t>(ws, B.off_rowa);
  uint16_t* xr = at<uint16_t>(ws, B.off_xr);
  uint16_t* dyr = at<uint16_t>(ws, B.off_dyr);
  float* gu = at<float>(ws, B.off_gu);
  float* dhp = at<float>(ws, B.off_dhp);
  uint16_t* dgu = at<uint16_t>(ws, B.off_dgu);
  float* dxr = at<float>(ws, P.off_yp);
  float* dp = at<float>(ws, B.off_dp);
  float* dl = at<float>(ws, B.off_dl);
  const int E = (int)P.E_loc, D = (int)P.D, F = (int)P.F, Fs = (int)P.Fs, T = (int)P.T,
            k = (int)P.k, ldh = (int)P.ldh;
  const int64_t cap = P.cap_rows;
  const int G = P.G;
  const bool prefill = P.BM == 256;
  int ctas = 0;
  if (prefill) {
    hipError_t e0 = split_ctas(&ctas);
    if (e0 != hipSuccess) return hip_fail(e0);
  }
  hipError_t e = hipSuccess;
  if (!saved)
    e = launch_align(ids, T, k, E, 0, P.BM, Fs > 0 ? T : 0, counts, offsets, padded, sorted, row_of,
                     row_token, tile_group, n_tiles, s);
  if (e == hipSuccess) e = launch_row_assign(row_of, (int)P.A, cap, row_assign, s);
  const int32_t* total = padded + G;  // rows in use
  if (e == hipSuccess) e = launch_gather_rows(w->x, false, row_token, total, cap, D, xr, s);
  if (e == hipSuccess) e = launch_gather_rows(dy, true, row_token, total, cap, D, dyr, s);
  if (e != hipSuccess) return hip_fail(e);

  // row-space products on the forward's grouped GEMM (rows x weight^T)
  GroupedGemm g{};
  g.E = E;
  g.tile_group = tile_group;
  g.n_tiles = n_tiles;
  g.max_tiles = P.max_tiles;
  g.min_tiles = (P.A + P.BM - 1) / P.BM + (Fs > 0 ? (P.T + P.BM - 1) / P.BM : 0);
  g.busy_tiles = busy_tiles(P);
  g.BM = P.BM;
  g.group_count = counts;
  g.group_padded = padded;
  g.ctas = ctas;
  g.partial = prefill ? at<float>(ws, P.off_partial) : nullptr;
  auto gemm = [&](const uint16_t* A, int64_t lda, const void* Br, const void* Bs, int Nr, int Ns,
                  int Kr, int Ks, float* C, int64_t ldc, bool bk = false) {
    GroupedGemm q = g;
    q.b_kmajor = bk ? 1 : 0;
    q.A = A;
    q.lda = lda;
    q.a_bytes = cap * lda * 2;
    q.B_routed = Br;
    q.B_shared = Fs > 0 ? Bs : nullptr;
    q.N_routed = Nr;
    q.N_shared = Ns;
    q.K_routed = Kr;
    q.K_shared = Ks;
    q.C = C;
    q.ldc = ldc;
    return prefill ? launch_gemm_down_prefill(q, s) : launch_gemm_down_decode(q, s);
  };
  // g | u (kept by the training forward, or computed again), then dh' = W_down^T dy
  const uint16_t* gu16 = saved ? at<const uint16_t>(grp, P.off_gusave) : nullptr;
  if (!saved) e = gemm(xr, D, w->w_gate_up, w->ws_gate_up, 2 * F, 2 * Fs, D, D, gu, 2 * ldh);
  // (both GEMM families read W_down and W_gate_up K-major, as stored)
  if (e == hipSuccess) e = gemm(dyr, D, w->w_down, w->ws_down, F, Fs, D, D, dhp, ldh, true);
  BwdRows rows{cap, total, row_token, row_assign, padded, tile_group, wts, dy, E, P.BM, D, F, Fs,
               ldh, saved ? nullptr : gu, gu16, dgu};
  if (e == hipSuccess) e = launch_swiglu_bwd(rows, dhp, dp, s);
  if (e == hipSuccess) e = launch_router_bwd(wts, dp, T, k, dl, s);
  // per-row dx = [dg du] W_gate_up, then dx
  if (e == hipSuccess)
    e = gemm(dgu, 2 * ldh, w->w_gate_up, w->ws_gate_up, D, D, 2 * F, 2 * Fs, dxr, D, true);
  if (e == hipSuccess)
    e = launch_combine_bwd(dxr, row_of, ids, dl, static_cast<const uint16_t*>(w->w_g), padded, T, D, k,
                           E, Fs > 0 ? 1 : 0, gr->dx, s);
  if (e == hipSuccess)
    e = launch_router_wgrad(dl, static_cast<const uint16_t*>(w->x), offsets, sorted, E, k, D,
                            shape->has_router_bias == MOE_ROUTER_BIAS_LOGITS ? 1 : 0, gr->dw_g,
                            gr->d_bias, s);
  if (e != hipSuccess) return hip_fail(e);

  // weight gradients over the per-row buffers (the rows are the reduction):
  // dW_down = sum (p dy) h^T, dW_gate_up = sum [dg du] x^T
  uint16_t* pdy = at<uint16_t>(ws, B.off_pdy);
  e = launch_rows(rows, 0, D, pdy, D, s);
  const uint16_t* hr = saved ? at<const uint16_t>(grp, P.off_h)  // the training forward's h rows
                             : at<const uint16_t>(ws, B.off_hr);
  if (!saved && e == hipSuccess) e = launch_rows(rows, 1, ldh, at<uint16_t>(ws, B.off_hr), ldh, s);
  auto tiles = [](int64_t n) { return (n + 255) / 256; };
  // a token picks an expert at most once, so with T <= 64 every group has at
  // most 64 rows: one K stage per tile, run by one workgroup per CU
  int one_stage = 0;
  if (e == hipSuccess && T <= 64) e = split_ctas(&one_stage);
  WgradGemm wd{pdy, hr, D, ldh, D, F, D, Fs, E, G, padded, counts, gr->dw_down, gr->dws_down,
               tiles(D), tiles(F > Fs ? F : Fs), one_stage};
  if (e == hipSuccess) e = launch_gemm_wgrad(wd, s);
  WgradGemm wu{dgu, xr, 2 * ldh, D, 2 * F, D, 2 * Fs, D, E, G, padded, counts, gr->dw_gate_up,
               gr->dws_gate_up, tiles(2 * ldh), tiles(D), one_stage};
  if (e == hipSuccess) e = launch_gemm_wgrad(wu, s);
  if (e != hipSuccess) return hip_fail(e);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_workspace_size(const moe_shape* shape, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe::Plan P;
  int rc = moe::make_plan(shape, &P);
  if (rc) return rc;
  *bytes = P.total;
  return MOE_OK;
}

int moe_block_m(const moe_shape* shape) {
  int rc = moe::check_shape(shape);
  if (rc) return rc;
  return moe::choose_block_m(shape);
}

}  // extern "C"

// moe_forward's checks of everything but the workspace (MOE_OK: T == 0 or valid)
int moe::check_forward_args(const moe_shape* shape, const moe_weights* w, const float* y,
                            const int32_t* topk_ids, const float* topk_w) {
  moe::Plan P;
  int rc = moe::make_plan(shape, &P);
  if (rc) return rc;
  rc = moe::check_weights(shape, w, true);
  if (rc) return rc;
  if (P.T == 0) return MOE_OK;
  if (!y) return MOE_ERR_INVALID_ARG;
  if (!moe::aligned16(y)) return MOE_ERR_ALIGNMENT;
  if ((topk_ids && !moe::aligned16(topk_ids)) || (topk_w && !moe::aligned16(topk_w)))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

extern "C" {

static int forward_impl(const moe_shape* shape, const moe_weights* w, float* y, int32_t* topk_ids,
                        float* topk_w, void* workspace, size_t ws_bytes, void* stream,
                        void* const* events, bool train = false) {
  int rc = moe::check_forward_args(shape, w, y, topk_ids, topk_w);
  if (rc) return rc;
  moe::Plan P;
  moe::make_plan(shape, &P);
  if (P.T == 0) return MOE_OK;
  if (!workspace) return MOE_ERR_INVALID_ARG;
  if (!moe::aligned16(workspace)) return MOE_ERR_ALIGNMENT;
  if (ws_bytes < (train ? P.total_train : P.total)) return MOE_ERR_WORKSPACE;
  uint16_t* gu_save = train ? at<uint16_t>(workspace, P.off_gusave) : nullptr;
  if (events)
    for (int i = 0; i < 6; ++i)
      if (!events[i]) return MOE_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Marks mk{events};
  int32_t* ids = topk_ids ? topk_ids : at<int32_t>(workspace, P.off_ids);
  float* wts = topk_w ? topk_w : at<float>(workspace, P.off_w);
  const float* bias = shape->has_router_bias == MOE_ROUTER_BIAS_LOGITS ? w->router_bias : nullptr;
  const float* sel = shape->has_router_bias == MOE_ROUTER_BIAS_SELECT ? w->router_bias : nullptr;
  hipError_t e = mk.mark(0, s);
  if (P.T <= moe::kSmallRouteT && P.E <= moe::kSmallRouteE) {
    // few tokens: partial logits over many workgroups, then one wave per token
    float* rpart = at<float>(workspace, P.off_rpart);
    if (e == hipSuccess)
      e = moe::launch_router_partial(static_cast<const uint16_t*>(w->x),
                                     static_cast<const uint16_t*>(w->w_g), (int)P.T, (int)P.D,
                                     (int)P.E, rpart, s);
    if (e == hipSuccess)
      e = moe::launch_route_finish(rpart, moe::router_parts(P.D), (int)P.T, (int)P.E, (int)P.k, bias,
                                   sel, ids, wts, s);
    if (e == hipSuccess) e = mk.mark(1, s);
    if (e != hipSuccess) return hip_fail(e);
    return run_experts(P, w, ids, wts, y, workspace, s, mk, gu_save);
  }
  if (e == hipSuccess)
    e = moe::launch_router(static_cast<const uint16_t*>(w->x), static_cast<const uint16_t*>(w->w_g),
                           bias, sel, (int)P.T, (int)P.D, (int)P.E, (int)P.k, ids, wts, s);
  if (e == hipSuccess) e = mk.mark(1, s);
  if (e != hipSuccess) return hip_fail(e);
  return run_experts(P, w, ids, wts, y, workspace, s, mk, gu_save);
}

int moe_forward(const moe_shape* shape, const moe_weights* w, float* y, int32_t* topk_ids,
                float* topk_w, void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(shape, w, y, topk_ids, topk_w, workspace, ws_bytes, stream, nullptr);
}

int moe_forward_timed(const moe_shape* shape, const moe_weights* w, float* y, int32_t* topk_ids,
                      float* topk_w, void* workspace, size_t ws_bytes, void* stream,
                      void* const* events) {
  if (!events) return MOE_ERR_INVALID_ARG;
  return forward_impl(shape, w, y, topk_ids, topk_w, workspace, ws_bytes, stream, events);
}

int moe_route(const moe_shape* shape, const moe_weights* w, int32_t* topk_ids, float* topk_w,
              void* stream) {
  int rc = moe::check_shape(shape);
  if (rc) return rc;
  if (!w) return MOE_ERR_INVALID_ARG;
  if (shape->T == 0) return MOE_OK;
  if (!w->x || !w->w_g || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (shape->has_router_bias && !w->router_bias) return MOE_ERR_INVALID_ARG;
  if (!moe::aligned16(w->x) || !moe::aligned16(w->w_g) || !moe::aligned16(topk_ids) ||
      !moe::aligned16(topk_w))
    return MOE_ERR_ALIGNMENT;
  const int mode = shape->has_router_bias;
  hipError_t e = moe::launch_router(
      static_cast<const uint16_t*>(w->x), static_cast<const uint16_t*>(w->w_g),
      mode == MOE_ROUTER_BIAS_LOGITS ? w->router_bias : nullptr,
      mode == MOE_ROUTER_BIAS_SELECT ? w->router_bias : nullptr, shape->T, shape->D, shape->E,
      shape->k, topk_ids, topk_w, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return MOE_OK;
}

int moe_align(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t block_m,
              int32_t shared_rows, int32_t* counts, int32_t* offsets, int32_t* padded_offsets,
              int32_t* sorted_assign, int32_t* row_of, int32_t* row_token, int32_t* tile_group,
              int32_t* n_tiles, void* stream) {
  if (T < 0 || k <= 0 || E <= 0 || block_m <= 0 || block_m > 1024 || shared_rows < 0)
    return MOE_ERR_INVALID_ARG;
  if (E > 256 || k > 8) return MOE_ERR_UNSUPPORTED;
  const int64_t G = E + (shared_rows > 0 ? 1 : 0);
  if ((int64_t)T * k + G * block_m + shared_rows >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets || !padded_offsets || !row_token || !tile_group || !n_tiles)
    return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !sorted_assign || !row_of)) return MOE_ERR_INVALID_ARG;
  hipError_t e = moe::launch_align(topk_ids, T, k, E, 0, block_m, shared_rows, counts, offsets,
                                   padded_offsets, sorted_assign, row_of, row_token, tile_group,
                                   n_tiles, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  return MOE_OK;
}

int moe_forward_routed(const moe_shape* shape, const moe_weights* w, const int32_t* topk_ids,
                       const float* topk_w, float* y, void* workspace, size_t ws_bytes,
                       void* stream) {
  moe::Plan P;
  int rc = moe::make_plan(shape, &P);
  if (rc) return rc;
  rc = moe::check_weights(shape, w, false);
  if (rc) return rc;
  if (P.T == 0) return MOE_OK;
  if (!y || !workspace || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!moe::aligned16(y) || !moe::aligned16(workspace) || !moe::aligned16(topk_ids) ||
      !moe::aligned16(topk_w))
    return MOE_ERR_ALIGNMENT;
  if (ws_bytes < P.total) return MOE_ERR_WORKSPACE;
  return run_experts(P, w, topk_ids, topk_w, y, workspace, static_cast<hipStream_t>(stream));
}

int moe_expert_load(const moe_shape* shape, const void* workspace, size_t ws_bytes,
                    int32_t* counts, void* stream) {
  moe::Plan P;
  int rc = moe::make_plan(shape, &P);
  if (rc) return rc;
  if (!counts || (P.T > 0 && !workspace)) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(counts) & 3u) return MOE_ERR_ALIGNMENT;
  if (P.T > 0 && ws_bytes < P.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (P.T == 0) {
    e = moe::launch_fill_i32(counts, P.G, 0, s);
  } else {
    const int32_t* src = reinterpret_cast<const int32_t*>(static_cast<const char*>(workspace) +
                                                          P.off_counts);
    e = hipMemcpyAsync(counts, src, sizeof(int32_t) * (size_t)P.G, hipMemcpyDeviceToDevice, s);
  }
  return e == hipSuccess ? MOE_OK : hip_fail(e);
}

int moe_backward_workspace_size(const moe_shape* shape, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe::BwdPlan B;
  int rc = moe::make_backward_plan(shape, &B);
  if (rc) return rc;
  *bytes = B.total;
  return MOE_OK;
}

int moe_train_workspace_size(const moe_shape* shape, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe::BwdPlan B;  // a training forward is only useful where the backward pass runs
  int rc = moe::make_backward_plan(shape, &B);
  if (rc) return rc;
  *bytes = B.P.total_train;
  return MOE_OK;
}

int moe_forward_train(const moe_shape* shape, const moe_weights* w, float* y, int32_t* topk_ids,
                      float* topk_w, void* workspace, size_t ws_bytes, void* stream) {
  moe::BwdPlan B;
  int rc = moe::make_backward_plan(shape, &B);
  if (rc) return rc;
  if (shape->T > 0 && (!topk_ids || !topk_w)) return MOE_ERR_INVALID_ARG;
  return forward_impl(shape, w, y, topk_ids, topk_w, workspace, ws_bytes, stream, nullptr, true);
}

static int backward_impl(const moe_shape* shape, const moe_weights* w, const int32_t* topk_ids,
                         const float* topk_w, const float* dy, const moe_grads* grads,
                         const void* saved, size_t saved_bytes, void* workspace, size_t ws_bytes,
                         void* stream) {
  moe::BwdPlan B;
  int rc = moe::make_backward_plan(shape, &B);
  if (rc) return rc;
  rc = moe::check_weights(shape, w, true);
  if (rc) return rc;
  const moe::Plan& P = B.P;
  if (!grads || !grads->dw_g || !grads->dw_gate_up || !grads->dw_down) return MOE_ERR_INVALID_ARG;
  if (P.Fs > 0 && (!grads->dws_gate_up || !grads->dws_down)) return MOE_ERR_INVALID_ARG;
  const void* outs[] = {grads->dx, grads->dw_g, grads->d_bias, grads->dw_gate_up, grads->dw_down,
                        grads->dws_gate_up, grads->dws_down};
  for (const void* q : outs)
    if (q && !moe::aligned16(q)) return MOE_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (P.T == 0) {  // no tokens: every weight gradient is zero
    const int64_t E = P.E_loc, D = P.D, F = P.F, Fs = P.Fs;
    hipError_t e = moe::launch_fill_f32(grads->dw_g, E * D, s);
    if (e == hipSuccess && grads->d_bias) e = moe::launch_fill_f32(grads->d_bias, E, s);
    if (e == hipSuccess) e = moe::launch_fill_f32(grads->dw_gate_up, E * 2 * F * D, s);
    if (e == hipSuccess) e = moe::launch_fill_f32(grads->dw_down, E * D * F, s);
    if (e == hipSuccess && Fs > 0) e = moe::launch_fill_f32(grads->dws_gate_up, 2 * Fs * D, s);
    if (e == hipSuccess && Fs > 0) e = moe::launch_fill_f32(grads->dws_down, D * Fs, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e);
  }
  if (!topk_ids || !topk_w || !dy || !grads->dx || !workspace) return MOE_ERR_INVALID_ARG;
  if (!moe::aligned16(topk_ids) || !moe::aligned16(topk_w) || !moe::aligned16(dy) ||
      !moe::aligned16(workspace))
    return MOE_ERR_ALIGNMENT;
  if (ws_bytes < B.total) return MOE_ERR_WORKSPACE;
  if (saved) {
    if (!moe::aligned16(saved)) return MOE_ERR_ALIGNMENT;
    if (saved_bytes < P.total_train) return MOE_ERR_WORKSPACE;
  }
  return run_backward(B, shape, w, topk_ids, topk_w, dy, grads, workspace, s, saved);
}

int moe_backward(const moe_shape* shape, const moe_weights* w, const int32_t* topk_ids,
                 const float* topk_w, const float* dy, const moe_grads* grads, void* workspace,
                 size_t ws_bytes, void* stream) {
  return backward_impl(shape, w, topk_ids, topk_w, dy, grads, nullptr, 0, workspace, ws_bytes,
                       stream);
}

int moe_backward_saved(const moe_shape* shape, const moe_weights* w, const int32_t* topk_ids,
                       const float* topk_w, const float* dy, const moe_grads* grads,
                       const void* train_workspace, size_t train_ws_bytes, void* workspace,
                       size_t ws_bytes, void* stream) {
  if (!train_workspace && shape && shape->T > 0) return MOE_ERR_INVALID_ARG;
  return backward_impl(shape, w, topk_ids, topk_w, dy, grads, train_workspace, train_ws_bytes,
                       workspace, ws_bytes, stream);
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, size out of range, k > E, or D/F not a multiple of 8)";
    case MOE_ERR_UNSUPPORTED: return "unsupported size (E > 256, k > 8, or row indices beyond 32 bits)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size()";
    case MOE_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case MOE_ERR_HIP: return g_hip_msg;
    case MOE_ERR_SCRATCH:
      return "moe_forward_noalloc: the shape's workspace exceeds MOE_STATIC_SCRATCH_BYTES (64 MiB); "
             "call moe_forward with a workspace";
    default: return "unknown error code";
  }
}

}  // extern "C"
