// moe_router: router GEMM with fused top-k and softmax over the chosen logits.
//
// Definition: "Mixture of experts: por qué un modelo enorme apenas usa sus
// parámetros", section "El router: la pieza que de verdad decide" (a linear
// projection scores every expert, the k best are kept, their scores are
// normalised by a softmax among themselves); glossary "MoE (Mixture of
// Experts - Mezcla de Expertos)", section 2 diagram row 2, p = Softmax(TopK(W_g x)).
//
// One workgroup of 4 wavefronts owns 16 tokens.  Logits are an MFMA
// 16x16x32 bf16 contraction with fp32 accumulation; the four waves take
// interleaved 32-wide slices of D and their partial sums are added in LDS in
// a fixed order (deterministic).  Each wave then ranks 4 tokens: the E <= 256
// logits of a token sit 4 per lane, and k rounds of a wave-wide
// (value desc, index asc) arg-max pick the experts.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kTok = 16;  // tokens per workgroup

// (v, i) beats (w, j) when v > w, or v == w and i < j.
__device__ __forceinline__ bool better(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

template <int NCT>  // 16-expert column tiles; E <= 16 * NCT
__global__ __launch_bounds__(256) void moe_router_kernel(const bf16_t* __restrict__ x,
                                                     const bf16_t* __restrict__ wg,
                                                     const float* __restrict__ bias, int T, int D,
                                                     int E, int k, int32_t* __restrict__ ids,
                                                     float* __restrict__ wts) {
  constexpr int EP = 16 * NCT;
  __shared__ float part[3][kTok][EP + 1];  // partial sums of waves 1..3; then the logits
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kTok;

  // ---- logits: this wave's share of the reduction over D
  f32x4 acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r16 = lane & 15, kb = lane >> 4;
  const int tok = t0 + r16;
  const bf16_t* xr = x + (int64_t)(tok < T ? tok : 0) * D;
  const int nchunks = (D + 31) / 32;
  for (int ch = wave; ch < nchunks; ch += 4) {
    const int kk = ch * 32 + kb * 8;  // D % 8 == 0: an 8-run is all in or all out
    u32x4 av = {0u, 0u, 0u, 0u};
    if (tok < T && kk < D) av = ld16(xr + kk);
    const bf16x8 a = as_bf16x8(av);
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int e = c * 16 + r16;
      u32x4 bv = {0u, 0u, 0u, 0u};
      if (e < E && kk < D) bv = ld16(wg + (int64_t)e * D + kk);
      acc[c] = mfma16(a, as_bf16x8(bv), acc[c]);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave - 1][4 * kb + r][c * 16 + r16] = acc[c][r];
  }
  __syncthreads();
  if (wave == 0) {  // fixed order: ((w0 + w1) + w2) + w3, then the bias
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * kb + r, col = c * 16 + r16;
        float s = ((acc[c][r] + part[0][row][col]) + part[1][row][col]) + part[2][row][col];
        if (bias && col < E) s += bias[col];
        part[0][row][col] = s;
      }
  }
  __syncthreads();

  // ---- top-k + softmax: wave w ranks tokens 4w .. 4w+3
  for (int rr = 0; rr < 4; ++rr) {
    const int r = wave * 4 + rr;
    const int t = t0 + r;
    if (t >= T) break;  // uniform across the wave
    float v[4];
    bool live[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      live[q] = e < E;
      v[q] = live[q] ? part[0][r][e] : 0.f;
    }
    float my_v = 0.f;
    int my_i = 0;
    float vmax = 0.f;
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
  const int blocks = (T + kTok - 1) / kTok;
  hipLaunchKernelGGL(moe_router_kernel<NCT>, dim3(blocks), dim3(256), 0, s, x, w_g, bias, T, D, E, k,
                     ids, wts);
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
