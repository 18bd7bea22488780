// moe_router: router GEMM with fused top-k and softmax over the chosen logits.
//
// Definition: "Mixture of experts: por qué un modelo enorme apenas usa sus
// parámetros", section "El router: la pieza que de verdad decide" (a linear
// projection scores every expert, the k best are kept, their scores are
// normalised by a softmax among themselves); glossary "MoE (Mixture of
// Experts - Mezcla de Expertos)", section 2 diagram row 2, p = Softmax(TopK(W_g x)).
//
// One workgroup of 16 wavefronts (8 when E > 128) owns 16 tokens.  Logits are an MFMA
// 16x16x32 bf16 contraction with fp32 accumulation: wave w takes the 64-wide
// slices w, w+16, w+32, ... of D (w, w+8, ... with 8 waves), and the partial
// sums are added in LDS in groups of four waves, the groups in order.  So a
// token's logits are bitwise the same for any T (one configuration for every
// batch size), and with E <= 64 also on the few-token path, whose workgroups
// each run one group of four waves.  Each wave then
// ranks tokens in (value desc, index asc) order: with E <= 64 every lane
// counts the logits that beat its own; with more experts, 4 logits per lane
// and k rounds of a wave-wide arg-max pick them.
#include "device.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace moe {
namespace {

constexpr int kTok = 16;  // tokens per workgroup
// The few-token router splits the full router's 16 waves over workgroups of
// kPartWaves waves (see moe_router_partial_kernel).
constexpr int kPartWaves = 4;
static_assert(kRouterGroups * kPartWaves == 16, "one partial workgroup per group of four waves");

// Waves per workgroup: 16, or 8 when E > 128 (64 accumulators per lane leave
// no room for 16 waves' worth of registers).  Fixed per E, so logits do not
// depend on T.
template <int NCT>
constexpr int waves_for() { return NCT > 8 ? 8 : 16; }
// 16-token tiles per workgroup: 2 when E > 128, where every workgroup streams
// all of W_g (E x D) for very little MFMA work; each W_g chunk a wave loads
// then serves both tiles.  A token's arithmetic is the same either way.
template <int NCT>
constexpr int tiles_for() { return NCT > 8 ? 2 : 1; }

template <int NCT>  // 16-expert column tiles; E <= 16 * NCT
__global__ __launch_bounds__(waves_for<NCT>() * 64) void moe_router_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wg,
                                                          const float* __restrict__ bias,
                                                          const float* __restrict__ sel, int T,
                                                          int D, int E, int k,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ wts) {
  constexpr int EP = 16 * NCT;
  constexpr int kWaves = waves_for<NCT>();
  constexpr int TT = tiles_for<NCT>();
  // 64-wide K chunks whose loads are in flight together (the same chunk order
  // per wave for every UNR, so the sums do not depend on it)
  constexpr int UNR = NCT <= 2 ? 3 : (NCT <= 4 ? 2 : 1);
  extern __shared__ float part[];        // [kWaves][kTok][EP + 1]: partials, then logits
  auto slot = [&](int s, int row, int col) -> float& {
    return part[(s * kTok + row) * (EP + 1) + col];
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tb = blockIdx.x * kTok * TT;  // first token of the workgroup

  // ---- this wave's share of the reduction over D
  f32x4 acc[TT][NCT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[tt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Inside a 64-wide chunk, x and W_g use the same K permutation: lane
  // (r16, kb) holds bytes [32kb, 32kb+32) of its row for two MFMAs, so the
  // four lanes of a row read one whole 128-byte line.
  const int r16 = lane & 15, kb = lane >> 4;
  const bf16_t* xr[TT];
  bool tin[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int tok = tb + tt * kTok + r16;
    tin[tt] = tok < T;
    xr[tt] = x + (int64_t)(tin[tt] ? tok : 0) * D;
  }
  const int nchunks = (D + 63) / 64;
  // column tiles whose weights are loaded together (fewer with two token
  // tiles, for their accumulators' registers)
  constexpr int CG = TT > 1 ? 4 : (NCT < 8 ? NCT : 8);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  if constexpr (TT > 1) {
    // E > 128: a chunk's x fragments are loaded once and its W_g column tiles
    // in groups of GP, each group's loads issued before the MFMAs of the one
    // before (the next chunk's first group before the last group's MFMAs, its
    // x right after them), so loads are in flight while the MFMAs run.  Every
    // accumulator still takes its MFMAs in chunk order.
    static_assert(UNR == 1, "one chunk at a time");
    constexpr int GP = 2;  // column tiles per group (registers: 128 accumulators beside them)
    constexpr int NG = NCT / GP;
    u32x4 xa[TT][2], wb[2][GP][2];
    auto load_x = [&](int ch) {
      const int kk = ch * 64 + kb * 16;
      const bool in0 = ch < nchunks && kk < D, in1 = in0 && kk + 8 < D;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        xa[tt][0] = (tin[tt] && in0) ? ld16(xr[tt] + kk) : zero;
        xa[tt][1] = (tin[tt] && in1) ? ld16(xr[tt] + kk + 8) : zero;
      }
    };
    auto load_w = [&](int ch, int grp, int wbuf) {
      const int kk = ch * 64 + kb * 16;
      const bool in0 = ch < nchunks && kk < D, in1 = in0 && kk + 8 < D;
#pragma unroll
      for (int c = 0; c < GP; ++c) {
        const int e = (grp * GP + c) * 16 + r16;
        const bf16_t* wr = wg + (int64_t)(e < E ? e : 0) * D + kk;
        wb[wbuf][c][0] = (e < E && in0) ? ld16(wr) : zero;
        wb[wbuf][c][1] = (e < E && in1) ? ld16(wr + 8) : zero;
      }
    };
    if (wave < nchunks) {
      load_x(wave);
      load_w(wave, 0, 0);
    }
    for (int ch = wave; ch < nchunks; ch += kWaves) {
#pragma unroll
      for (int grp = 0; grp < NG; ++grp) {
        const int wbuf = grp & 1;  // NG is even: group 0 of every chunk is buffer 0
        if (grp + 1 < NG)
          load_w(ch, grp + 1, wbuf ^ 1);
        else if (ch + kWaves < nchunks)
          load_w(ch + kWaves, 0, wbuf ^ 1);
        __builtin_amdgcn_sched_barrier(0);  // the next loads before these MFMAs
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < GP; ++c)
              acc[tt][grp * GP + c] = mfma16(as_bf16x8(xa[tt][h]), as_bf16x8(wb[wbuf][c][h]),
                                             acc[tt][grp * GP + c]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ch + kWaves < nchunks) load_x(ch + kWaves);
    }
  } else {
    for (int ch0 = wave; ch0 < nchunks; ch0 += UNR * kWaves) {
#pragma unroll
      for (int c0 = 0; c0 < NCT; c0 += CG) {
        u32x4 av[TT][UNR][2], bv[UNR][CG][2];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int kk = (ch0 + u * kWaves) * 64 + kb * 16;  // D % 8 == 0: 8-runs are all in or out
          const bool in0 = ch0 + u * kWaves < nchunks && kk < D, in1 = in0 && kk + 8 < D;
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            av[tt][u][0] = (tin[tt] && in0) ? ld16(xr[tt] + kk) : zero;
            av[tt][u][1] = (tin[tt] && in1) ? ld16(xr[tt] + kk + 8) : zero;
          }
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            const int e = (c0 + c) * 16 + r16;
            const bf16_t* wr = wg + (int64_t)(e < E ? e : 0) * D + kk;
            bv[u][c][0] = (e < E && in0) ? ld16(wr) : zero;
            bv[u][c][1] = (e < E && in1) ? ld16(wr + 8) : zero;
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // all loads of the trip before the MFMAs
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            if (ch0 + u * kWaves >= nchunks) break;  // past the end: nothing to add
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int c = 0; c < CG; ++c)
                acc[tt][c0 + c] =
                    mfma16(as_bf16x8(av[tt][u][h]), as_bf16x8(bv[u][c][h]), acc[tt][c0 + c]);
          }
      }
    }
  }

#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int t0 = tb + tt * kTok;
    if (tt > 0) __syncthreads();  // the previous tile's logits are no longer read
    // ---- partial sums of all waves into LDS; each logit is then the sum over
    // the waves in wave order (one barrier instead of a tree of them)
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) slot(wave, 4 * kb + r, c * 16 + r16) = acc[tt][c][r];
    __syncthreads();
    for (int idx = tid; idx < kTok * EP; idx += kWaves * 64) {
      const int row = idx / EP, col = idx - row * EP;
      // waves in groups of four, ((w0 + w1) + w2) + w3, then the groups in
      // order: the association the few-token router (one workgroup per group
      // of four waves) reproduces
      float sum = 0.f;
#pragma unroll
      for (int g4 = 0; g4 < kWaves; g4 += kPartWaves) {
        float gs = slot(g4, row, col);
#pragma unroll
        for (int w = 1; w < kPartWaves; ++w) gs += slot(g4 + w, row, col);
        sum = g4 == 0 ? gs : sum + gs;
      }
      if (bias && col < E) sum += bias[col];
      slot(0, row, col) = sum;  // only this thread reads or writes this element
    }
    __syncthreads();

    // ---- top-k + softmax: wave w ranks tokens w, w + kWaves, ...
    for (int r = wave; r < kTok; r += kWaves) {
      const int t = t0 + r;
      if (t >= T) break;
      topk_softmax(&slot(0, r, 0), sel, E, k, lane, [&](int q, int e, float w) {
        ids[(int64_t)t * k + q] = e;
        wts[(int64_t)t * k + q] = w;
      });
    }
  }
}

template <int NCT>
hipError_t launch_nct(const uint16_t* x, const uint16_t* w_g, const float* bias, const float* sel,
                      int T, int D, int E, int k, int32_t* ids, float* wts, hipStream_t s) {
  constexpr int kWaves = waves_for<NCT>();
  const size_t lds = sizeof(float) * kWaves * kTok * (16 * NCT + 1);
  // set once per process (a function-local static is initialised thread-safely)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)moe_router_kernel<NCT>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const int per_block = kTok * tiles_for<NCT>();
  const int blocks = (T + per_block - 1) / per_block;
  hipLaunchKernelGGL(moe_router_kernel<NCT>, dim3(blocks), dim3(kWaves * 64), lds, s, x, w_g, bias,
                     sel, T, D, E, k, ids, wts);
  return hipGetLastError();
}


// Partial logits for few tokens (E <= 64, where the full router runs 16
// waves): workgroup (token tile, p) runs the full router's waves 4p .. 4p + 3,
// wave s walking the 64-wide K chunks 4p + s, 4p + s + 16, ... in ascending
// order with the same MFMA sequence, adds its four waves in wave order and
// stores the sum as partial[p][t][e].  moe_route_finish_kernel adds the four parts in
// part order, which is the full router's grouped sum: a token's logits are
// bitwise the same on either path and for every T.
template <int NCT>
__global__ __launch_bounds__(kPartWaves * 64) void moe_router_partial_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, int T, int D, int E,
    float* __restrict__ partial) {
  constexpr int EP = 16 * NCT;
  constexpr int CG = NCT < 8 ? NCT : 8;
  extern __shared__ float part[];  // [kPartWaves][kTok][EP + 1]
  auto slot = [&](int s, int row, int col) -> float& {
    return part[(s * kTok + row) * (EP + 1) + col];
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * kTok, p = blockIdx.y;
  constexpr int kFullWaves = kRouterGroups * kPartWaves;  // the full router's waves
  const int fw = p * kPartWaves + wave;                   // this wave's index there
  f32x4 acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r16 = lane & 15, kb = lane >> 4;
  const int tok = t0 + r16;
  const bf16_t* xr = x + (int64_t)(tok < T ? tok : 0) * D;
  const int nchunks = (D + 63) / 64;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  constexpr int UNR = 4;  // chunks whose loads are in flight together
  for (int ch0 = fw; ch0 < nchunks; ch0 += UNR * kFullWaves) {
#pragma unroll
    for (int c0 = 0; c0 < NCT; c0 += CG) {
      u32x4 av[UNR][2], bv[UNR][CG][2];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int ch = ch0 + u * kFullWaves;
        const int kk = ch * 64 + kb * 16;  // same K permutation as the full router
        const bool in0 = ch < nchunks && kk < D, in1 = in0 && kk + 8 < D;
        av[u][0] = (tok < T && in0) ? ld16(xr + kk) : zero;
        av[u][1] = (tok < T && in1) ? ld16(xr + kk + 8) : zero;
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          const int e = (c0 + c) * 16 + r16;
          const bf16_t* wr = wg + (int64_t)(e < E ? e : 0) * D + kk;
          bv[u][c][0] = (e < E && in0) ? ld16(wr) : zero;
          bv[u][c][1] = (e < E && in1) ? ld16(wr + 8) : zero;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // chunks past the end are not multiplied (as in the full router)
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (ch0 + u * kFullWaves >= nchunks) break;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int c = 0; c < CG; ++c)
            acc[c0 + c] = mfma16(as_bf16x8(av[u][h]), as_bf16x8(bv[u][c][h]), acc[c0 + c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < NCT; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) slot(wave, 4 * kb + r, c * 16 + r16) = acc[c][r];
  __syncthreads();
  for (int idx = tid; idx < kTok * E; idx += kPartWaves * 64) {
    const int row = idx / E, col = idx - row * E;
    if (t0 + row >= T) continue;
    float sum = slot(0, row, col);
#pragma unroll
    for (int w = 1; w < kPartWaves; ++w) sum += slot(w, row, col);
    partial[((int64_t)p * T + t0 + row) * E + col] = sum;
  }
}

template <int NCT>
hipError_t launch_partial_nct(const uint16_t* x, const uint16_t* w_g, int T, int D, int E,
                              float* partial, hipStream_t s) {
  const size_t lds = sizeof(float) * kPartWaves * kTok * (16 * NCT + 1);
  // set once per process (a function-local static is initialised thread-safely)
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)moe_router_partial_kernel<NCT>, hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)lds);
  if (attr != hipSuccess) return attr;
  const dim3 grid((T + kTok - 1) / kTok, kRouterGroups);
  hipLaunchKernelGGL(moe_router_partial_kernel<NCT>, grid, dim3(kPartWaves * 64), lds, s, x, w_g, T,
                     D, E, partial);
  return hipGetLastError();
}

// One wave per token: lane e < E adds the token's partial logits of the
// router_parts groups in group order, then the bias, and the wave picks the
// top-k and the softmax over the chosen (topk_softmax), as the full router
// does with its grouped sum.
__global__ __launch_bounds__(64) void moe_route_finish_kernel(const float* __restrict__ partial,
                                                              int P, int T, int E, int k,
                                                              const float* __restrict__ bias,
                                                              const float* __restrict__ sel,
                                                              int32_t* __restrict__ ids,
                                                              float* __restrict__ wts) {
  __shared__ float lg[64];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x;
  if (lane < E) {
    float pv[kRouterGroups];
#pragma unroll
    for (int q = 0; q < kRouterGroups; ++q)
      pv[q] = q < P ? partial[((int64_t)q * T + t) * E + lane] : 0.f;
    float v = pv[0];
#pragma unroll
    for (int q = 1; q < kRouterGroups; ++q)
      if (q < P) v += pv[q];
    if (bias) v += bias[lane];
    lg[lane] = v;
  }
  __syncthreads();
  topk_softmax(lg, sel, E, k, lane, [&](int q, int e, float p) {
    ids[t * k + q] = e;
    wts[t * k + q] = p;
  });
}

}  // namespace

hipError_t launch_route_finish(const float* partial, int P, int T, int E, int k, const float* bias,
                               const float* sel, int32_t* ids, float* wts, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (E > 64 || P > kRouterGroups || k > 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_route_finish_kernel, dim3(T), dim3(64), 0, s, partial, P, T, E, k, bias, sel,
                     ids, wts);
  return hipGetLastError();
}

hipError_t launch_router_partial(const uint16_t* x, const uint16_t* w_g, int T, int D, int E,
                                 float* partial, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nct = (E + 15) / 16;
  if (nct <= 1) return launch_partial_nct<1>(x, w_g, T, D, E, partial, s);
  if (nct <= 2) return launch_partial_nct<2>(x, w_g, T, D, E, partial, s);
  if (nct <= 4) return launch_partial_nct<4>(x, w_g, T, D, E, partial, s);
  if (nct <= 8) return launch_partial_nct<8>(x, w_g, T, D, E, partial, s);
  return launch_partial_nct<16>(x, w_g, T, D, E, partial, s);
}

hipError_t launch_router(const uint16_t* x, const uint16_t* w_g, const float* bias, const float* sel,
                         int T, int D, int E, int k, int32_t* ids, float* wts, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nct = (E + 15) / 16;
  if (nct <= 1) return launch_nct<1>(x, w_g, bias, sel, T, D, E, k, ids, wts, s);
  if (nct <= 2) return launch_nct<2>(x, w_g, bias, sel, T, D, E, k, ids, wts, s);
  if (nct <= 4) return launch_nct<4>(x, w_g, bias, sel, T, D, E, k, ids, wts, s);
  if (nct <= 8) return launch_nct<8>(x, w_g, bias, sel, T, D, E, k, ids, wts, s);
  return launch_nct<16>(x, w_g, bias, sel, T, D, E, k, ids, wts, s);
}

}  // namespace moe
