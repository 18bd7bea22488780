// Host-side argument checks and workspace layout (no HIP calls).
#include "plan.hpp"

namespace moe {

namespace {
constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
}  // namespace

int check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->T < 0 || s->D <= 0 || s->E <= 0 || s->F <= 0 || s->k <= 0 || s->F_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (s->k > s->E) return MOE_ERR_INVALID_ARG;
  if (s->has_router_bias != MOE_ROUTER_BIAS_NONE && s->has_router_bias != MOE_ROUTER_BIAS_LOGITS &&
      s->has_router_bias != MOE_ROUTER_BIAS_SELECT)
    return MOE_ERR_INVALID_ARG;
  if (s->weight_format != MOE_WEIGHTS_BF16 && s->weight_format != MOE_WEIGHTS_FP8_E4M3)
    return MOE_ERR_INVALID_ARG;
  if (s->expert_begin < 0 || s->num_local_experts < 0 ||
      (int64_t)s->expert_begin + s->num_local_experts > s->E ||
      (s->num_local_experts == 0 && s->expert_begin != 0))
    return MOE_ERR_INVALID_ARG;
  if (s->D % 8 || s->F % 8 || s->F_shared % 8) return MOE_ERR_INVALID_ARG;
  if (s->E > 256 || s->k > 8) return MOE_ERR_UNSUPPORTED;
  // every padded row index and every x/y element offset per row must fit 32 bits
  const int64_t bm = 256;  // largest tile height any plan uses
  const int64_t rows = (int64_t)s->T * s->k + (int64_t)(s->E + 1) * bm + s->T;
  if (rows >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  // operands are addressed through 32-bit buffer offsets below 2^31 bytes
  const int64_t lim = int64_t(1) << 31;
  if ((int64_t)s->T * s->D * 2 >= lim) return MOE_ERR_UNSUPPORTED;
  const int64_t fmax = s->F > s->F_shared ? s->F : s->F_shared;
  if ((int64_t)fmax * s->D * 4 >= lim) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Rows per expert decide the kernel family: a few rows per expert stream the
// weights (16- or 32-row tiles), many rows per expert are MFMA-bound
// (256-row tiles).
int choose_block_m(const moe_shape* s) {
  const int64_t rows = (int64_t)s->T * s->k;
  if (rows <= (int64_t)20 * s->E) return 16;
  if (rows <= (int64_t)48 * s->E) return 32;
  // The 256-row tiles move E4M3 weights in 16-code chunks, which must not
  // straddle the end of a row; other widths keep the 32-row tiles, whose
  // loads check K in 8-element steps.
  if (s->weight_format == MOE_WEIGHTS_FP8_E4M3 &&
      (s->D % 16 || s->F % 16 || s->F_shared % 16))
    return 32;
  return 256;
}

int make_plan(const moe_shape* s, Plan* p) {
  int rc = check_shape(s);
  if (rc) return rc;
  p->T = s->T;
  p->D = s->D;
  p->E = s->E;
  p->F = s->F;
  p->k = s->k;
  p->Fs = s->F_shared;
  p->e0 = s->expert_begin;
  p->E_loc = s->num_local_experts > 0 ? s->num_local_experts : s->E;
  p->G = (int)p->E_loc + (s->F_shared > 0 ? 1 : 0);
  p->BM = choose_block_m(s);
  p->A = p->T * p->k;
  p->cap_rows = p->A + (int64_t)p->G * (p->BM - 1) + (p->Fs > 0 ? p->T : 0);
  p->max_tiles = p->cap_rows / p->BM + 1;
  p->ldh = p->F > p->Fs ? p->F : p->Fs;
  p->fp8 = s->weight_format == MOE_WEIGHTS_FP8_E4M3;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = round_up(o + bytes);
    return at;
  };
  p->off_ids = take(sizeof(int32_t) * p->A);
  p->off_w = take(sizeof(float) * p->A);
  p->off_counts = take(sizeof(int32_t) * (p->G + 1));
  p->off_offsets = take(sizeof(int32_t) * (p->G + 1));
  p->off_padded = take(sizeof(int32_t) * (p->G + 1));
  p->off_ntiles = take(sizeof(int32_t));
  p->off_sorted = take(sizeof(int32_t) * p->A);
  p->off_rowof = take(sizeof(int32_t) * p->A);
  p->off_rowtoken = take(sizeof(int32_t) * p->cap_rows);
  p->off_tilegroup = take(sizeof(int32_t) * p->max_tiles);
  p->off_h = take(sizeof(uint16_t) * (size_t)p->cap_rows * p->ldh);
  p->off_yp = take(sizeof(float) * (size_t)p->cap_rows * p->D);
  const bool split = p->BM == 256;  // only the 256-row kernels split tiles over K
  p->off_partial = take(split ? sizeof(float) * kSplitCtas * kPartialTileFloats : 0);
  // partial router logits of the few-token path
  p->off_rpart = take(p->T <= kSmallRouteT && p->E <= kSmallRouteE
                          ? sizeof(float) * router_parts(p->D) * p->T * p->E
                          : 0);
  p->total = o;
  p->off_gusave = take(sizeof(uint16_t) * (size_t)p->cap_rows * 2 * p->ldh);
  p->total_train = o;
  return MOE_OK;
}

int make_backward_plan(const moe_shape* s, BwdPlan* b) {
  int rc = make_plan(s, &b->P);
  if (rc) return rc;
  const Plan& P = b->P;
  if (P.fp8) return MOE_ERR_UNSUPPORTED;                       // bf16 expert weights only
  if (s->num_local_experts > 0 && s->num_local_experts != s->E) return MOE_ERR_UNSUPPORTED;
  // the row buffers the weight-gradient GEMMs read are addressed through
  // 32-bit buffer offsets
  const int64_t widest = P.D > 2 * P.ldh ? P.D : 2 * P.ldh;
  if (P.cap_rows * widest * 2 >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  size_t o = P.total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += (bytes + 255) / 256 * 256;
    return at;
  };
  const size_t cap = (size_t)P.cap_rows;
  b->off_rowa = take(sizeof(int32_t) * cap);
  b->off_xr = take(2 * cap * P.D);
  b->off_dyr = take(2 * cap * P.D);
  b->off_gu = take(4 * cap * 2 * P.ldh);
  b->off_dhp = take(4 * cap * P.ldh);
  b->off_dgu = take(2 * cap * 2 * P.ldh);
  b->off_dp = take(4 * (size_t)P.A);
  b->off_dl = take(4 * (size_t)P.A);
  b->off_pdy = take(2 * cap * P.D);
  b->off_hr = take(2 * cap * P.ldh);
  b->total = o;
  return MOE_OK;
}

int check_weights(const moe_shape* s, const moe_weights* w, bool need_router) {
  if (!w) return MOE_ERR_INVALID_ARG;
  if (s->T > 0 && !w->x) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate_up || !w->w_down) return MOE_ERR_INVALID_ARG;
  if (need_router) {
    if (!w->w_g) return MOE_ERR_INVALID_ARG;
    if (s->has_router_bias && !w->router_bias) return MOE_ERR_INVALID_ARG;
  }
  if (s->F_shared > 0 && (!w->ws_gate_up || !w->ws_down)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {w->x, w->w_gate_up, w->w_down, w->ws_gate_up, w->ws_down,
                        need_router ? w->w_g : nullptr};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MOE_ERR_ALIGNMENT;
  if (s->weight_format == MOE_WEIGHTS_FP8_E4M3) {
    if (!w->w_gate_up_scale || !w->w_down_scale) return MOE_ERR_INVALID_ARG;
    if (s->F_shared > 0 && (!w->ws_gate_up_scale || !w->ws_down_scale)) return MOE_ERR_INVALID_ARG;
    const float* sc[] = {w->w_gate_up_scale, w->w_down_scale, w->ws_gate_up_scale,
                         w->ws_down_scale};
    for (const float* q : sc)
      if (q && (reinterpret_cast<uintptr_t>(q) & 3u)) return MOE_ERR_ALIGNMENT;
  }
  if (need_router && s->has_router_bias && (reinterpret_cast<uintptr_t>(w->router_bias) & 3u))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

}  // namespace moe
