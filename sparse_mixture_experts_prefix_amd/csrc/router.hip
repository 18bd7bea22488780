// moe_router: router GEMM with fused top-k and softmax over the chosen logits.
//
// Definition: "Mixture of experts: por qué un modelo enorme apenas usa sus
// parámetros", section "El router: la pieza que de verdad decide" (a linear
// projection scores every expert, the k best are kept, their scores are
// normalised by a softmax among themselves); glossary "MoE (Mixture of
// Experts - Mezcla de Expertos)", section 2 diagram row 2, p = Softmax(TopK(W_g x)).
//
// One workgroup of 16 wavefronts (8 when E > 128) owns 16 tokens.  Logits are an MFMA
// 16x16x32 bf16 contraction with fp32 accumulation: wave w takes the 32-wide
// slices w, w+16, w+32, ... of D (w, w+8, ... with 8 waves), and the partial
// sums are added by a fixed tree in LDS, so a token's logits are bitwise the same for any
// T (one configuration for every batch size; 16 waves keep enough loads in
// flight when T is a handful of tokens).  Each wave then ranks tokens: the
// E <= 256 logits sit 4 per lane, and k rounds of a wave-wide
// (value desc, index asc) arg-max pick the experts.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kTok = 16;  // tokens per workgroup

// Waves per workgroup: 16, or 8 when E > 128 (64 accumulators per lane leave
// no room for 16 waves' worth of registers).  Fixed per E, so logits do not
// depend on T.
template <int NCT>
constexpr int waves_for() { return NCT > 8 ? 8 : 16; }

// (v, i) beats (w, j) when v > w, or v == w and i < j.
__device__ __forceinline__ bool better(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

template <int NCT>  // 16-expert column tiles; E <= 16 * NCT
__global__ __launch_bounds__(waves_for<NCT>() * 64) void moe_router_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wg,
                                                          const float* __restrict__ bias, int T,
                                                          int D, int E, int k,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ wts) {
  constexpr int EP = 16 * NCT;
  constexpr int kWaves = waves_for<NCT>();
  constexpr int kLevels = kWaves == 16 ? 4 : 3;
  // chunks whose loads are in flight together (the same chunk order per wave
  // for every UNR, so the sums do not depend on it)
  constexpr int UNR = NCT <= 2 ? 6 : (NCT <= 4 ? 3 : 1);
  extern __shared__ float part[];        // [kWaves/2][kTok][EP + 1]: partials, then logits
  auto slot = [&](int s, int row, int col) -> float& {
    return part[(s * kTok + row) * (EP + 1) + col];
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * kTok;

  // ---- this wave's share of the reduction over D
  f32x4 acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r16 = lane & 15, kb = lane >> 4;
  const int tok = t0 + r16;
  const bf16_t* xr = x + (int64_t)(tok < T ? tok : 0) * D;
  const int nchunks = (D + 31) / 32;
  constexpr int CG = NCT < 8 ? NCT : 8;  // column tiles whose weights are loaded together
  for (int ch0 = wave; ch0 < nchunks; ch0 += UNR * kWaves) {
#pragma unroll
    for (int c0 = 0; c0 < NCT; c0 += CG) {
      u32x4 av[UNR], bv[UNR][CG];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int kk = (ch0 + u * kWaves) * 32 + kb * 8;  // D % 8 == 0: 8-runs are all in or out
        const bool kin = ch0 + u * kWaves < nchunks && kk < D;
        av[u] = (tok < T && kin) ? ld16(xr + kk) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          const int e = (c0 + c) * 16 + r16;
          bv[u][c] = (e < E && kin) ? ld16(wg + (int64_t)e * D + kk) : u32x4{0u, 0u, 0u, 0u};
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // all loads of the trip before the MFMAs
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int c = 0; c < CG; ++c)
          acc[c0 + c] = mfma16(as_bf16x8(av[u]), as_bf16x8(bv[u][c]), acc[c0 + c]);
    }
  }

  // ---- fixed tree over the partial sums: level h adds wave w + 2^h into wave w
#pragma unroll
  for (int h = kLevels - 1; h >= 0; --h) {
    const int half = 1 << h;
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) slot(wave - half, 4 * kb + r, c * 16 + r16) = acc[c][r];
    }
    __syncthreads();
    if (wave < half) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[c][r] += slot(wave, 4 * kb + r, c * 16 + r16);
    }
    __syncthreads();
  }
  if (wave == 0) {
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = c * 16 + r16;
        float s = acc[c][r];
        if (bias && col < E) s += bias[col];
        slot(0, 4 * kb + r, col) = s;
      }
  }
  __syncthreads();

  // ---- top-k + softmax: wave w ranks tokens w, w + kWaves, ...
  for (int r = wave; r < kTok; r += kWaves) {
    const int t = t0 + r;
    if (t >= T) break;
    float v[4];
    bool live[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      live[q] = e < E;
      v[q] = live[q] ? slot(0, r, e) : 0.f;
    }
    float my_v = 0.f, vmax = 0.f;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
      float bv = 0.f;
      int bi = 0x7fffffff;
      bool have = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        if (live[q] && (!have || better(v[q], e, bv, bi))) {
          bv = v[q];
          bi = e;
          have = true;
        }
      }
      // lanes with nothing left carry index INT_MAX and lose every comparison
      if (!have) bv = -__builtin_inff();
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q == bi) live[q] = false;
      if (j == 0) vmax = bv;
      if (lane == j) {
        my_v = bv;
        my_i = bi;
      }
    }
    float s = lane < k ? expf(my_v - vmax) : 0.f;
    float tot = s;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
    if (lane < k) {
      ids[(int64_t)t * k + lane] = my_i;
      wts[(int64_t)t * k + lane] = s / tot;
    }
  }
}

template <int NCT>
hipError_t launch_nct(const uint16_t* x, const uint16_t* w_g, const float* bias, int T, int D,
                      int E, int k, int32_t* ids, float* wts, hipStream_t s) {
  constexpr int kWaves = waves_for<NCT>();
  const size_t lds = sizeof(float) * (kWaves / 2) * kTok * (16 * NCT + 1);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)moe_router_kernel<NCT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int blocks = (T + kTok - 1) / kTok;
  hipLaunchKernelGGL(moe_router_kernel<NCT>, dim3(blocks), dim3(kWaves * 64), lds, s, x, w_g, bias,
                     T, D, E, k, ids, wts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* w_g, const float* bias, int T, int D,
                         int E, int k, int32_t* ids, float* wts, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nct = (E + 15) / 16;
  if (nct <= 1) return launch_nct<1>(x, w_g, bias, T, D, E, k, ids, wts, s);
  if (nct <= 2) return launch_nct<2>(x, w_g, bias, T, D, E, k, ids, wts, s);
  if (nct <= 4) return launch_nct<4>(x, w_g, bias, T, D, E, k, ids, wts, s);
  if (nct <= 8) return launch_nct<8>(x, w_g, bias, T, D, E, k, ids, wts, s);
  return launch_nct<16>(x, w_g, bias, T, D, E, k, ids, wts, s);
}

}  // namespace moe
