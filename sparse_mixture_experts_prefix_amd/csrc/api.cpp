// extern "C" entry points of libmoe (declared and documented in moe.h).
#include <hip/hip_runtime.h>

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
  static int cached[64] = {0};
  if (dev >= 0 && dev < 64 && cached[dev] > 0) {
    *out = cached[dev];
    return hipSuccess;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int n = cus < moe::kSplitCtas ? cus : moe::kSplitCtas;
  if (dev >= 0 && dev < 64) cached[dev] = n;
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

// Everything after routing: align -> gate/up -> down -> combine.
int run_experts(const moe::Plan& P, const moe_weights* w, const int32_t* ids, const float* wts,
                float* y, void* ws, hipStream_t s, Marks mk = Marks{nullptr},
                const moe::RouteFinish* fin = nullptr) {
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
                              padded, sorted, row_of, row_token, tile_group, n_tiles, fin, s);
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
  gu.C = H;
  gu.ldc = P.ldh;
  gu.BM = P.BM;
  gu.group_count = counts;
  gu.group_padded = padded;
  gu.a_bytes = P.T * P.D * 2;
  gu.ctas = ctas;
  gu.partial = prefill ? at<float>(ws, P.off_partial) : nullptr;
  e = P.BM == 256 ? launch_gemm_gate_up_prefill(gu, s) : launch_gemm_gate_up_decode(gu, s);
  if (e == hipSuccess) e = mk.mark(3, s);
  if (e != hipSuccess) return hip_fail(e);

  GroupedGemm dn = gu;
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

static int forward_impl(const moe_shape* shape, const moe_weights* w, float* y, int32_t* topk_ids,
                        float* topk_w, void* workspace, size_t ws_bytes, void* stream,
                        void* const* events) {
  moe::Plan P;
  int rc = moe::make_plan(shape, &P);
  if (rc) return rc;
  rc = moe::check_weights(shape, w, true);
  if (rc) return rc;
  if (P.T == 0) return MOE_OK;
  if (!y || !workspace) return MOE_ERR_INVALID_ARG;
  if (!moe::aligned16(y) || !moe::aligned16(workspace)) return MOE_ERR_ALIGNMENT;
  if ((topk_ids && !moe::aligned16(topk_ids)) || (topk_w && !moe::aligned16(topk_w)))
    return MOE_ERR_ALIGNMENT;
  if (ws_bytes < P.total) return MOE_ERR_WORKSPACE;
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
    // few tokens: partial logits over many workgroups, routing finished in align
    float* rpart = at<float>(workspace, P.off_rpart);
    if (e == hipSuccess)
      e = moe::launch_router_partial(static_cast<const uint16_t*>(w->x),
                                     static_cast<const uint16_t*>(w->w_g), (int)P.T, (int)P.D,
                                     (int)P.E, rpart, s);
    if (e == hipSuccess) e = mk.mark(1, s);
    if (e != hipSuccess) return hip_fail(e);
    const moe::RouteFinish fin{rpart, moe::router_parts(P.D), (int)P.E, bias, sel, ids, wts};
    return run_experts(P, w, ids, wts, y, workspace, s, mk, &fin);
  }
  if (e == hipSuccess)
    e = moe::launch_router(static_cast<const uint16_t*>(w->x), static_cast<const uint16_t*>(w->w_g),
                           bias, sel, (int)P.T, (int)P.D, (int)P.E, (int)P.k, ids, wts, s);
  if (e == hipSuccess) e = mk.mark(1, s);
  if (e != hipSuccess) return hip_fail(e);
  return run_experts(P, w, ids, wts, y, workspace, s, mk);
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
                                   n_tiles, nullptr, static_cast<hipStream_t>(stream));
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

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, size out of range, k > E, or D/F not a multiple of 8)";
    case MOE_ERR_UNSUPPORTED: return "unsupported size (E > 256, k > 8, or row indices beyond 32 bits)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size()";
    case MOE_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case MOE_ERR_HIP: return g_hip_msg;
    default: return "unknown error code";
  }
}

}  // extern "C"
