// Backward pass of the layer: the kernels around the grouped GEMMs.
//
// Gradients of sum_t <dy[t], y[t]> for a given routing, by the chain rule of
// the forward pass (the pages' training sections name grouped-GEMM kernels
// but no formulas: "Mixture of Experts optimiza Transformers y LLMs", section
// on training; "Transformers v5 El Secreto Detrás de los Modelos MoE Más
// Rápidos", section "Entrenamiento MoE").  The row-space products (g and u
// again, dh' = W_down^T dy, dx rows = [dg du] W_gate_up) run on the forward's
// grouped GEMM families, reading the weights K-major as stored; the weight
// gradients on a variable-K grouped GEMM over per-row buffers.  This file
// holds the rest, all bandwidth-bound:
//  - gathering x and dy rows in expert order (bf16, padding rows zero),
//  - per-row bf16 operand rows (p dy, h) of the weight gradients,
//  - the SwiGLU backward per row, which also forms dp = <dy, O_row>,
//  - the router's softmax backward dl = p (dp - sum p dp), dW_g and the bias
//    gradient (sums over an expert's assignments in ascending order),
//  - dx = sum of the slots' dx rows + the shared row + sum_j dl_j W_g[e_j].
// Every sum runs in a fixed order: the gradients are bitwise reproducible.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ float load_f(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float load_f(const float* p, int64_t i) { return p[i]; }

// dst[r][d] = src[row_token[r]][d] as bf16 (0 where row_token[r] < 0), rows < padded[G]
template <class Src>
__global__ __launch_bounds__(256) void moe_gather_rows_kernel(const Src* __restrict__ src,
                                                              const int32_t* __restrict__ row_token,
                                                              const int32_t* __restrict__ total,
                                                              int D, bf16_t* __restrict__ dst) {
  const int64_t r = blockIdx.x;
  if (r >= total[0]) return;
  const int t = row_token[r];
  for (int d = threadIdx.x; d < D; d += blockDim.x)
    dst[r * D + d] = t >= 0 ? f32_to_bf16(load_f(src, (int64_t)t * D + d)) : (bf16_t)0;
}

__global__ void moe_fill_f32_kernel(float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = 0.f;
}

// row_assign[row_of[a]] = a
__global__ void moe_row_assign_kernel(const int32_t* __restrict__ row_of, int A,
                                      int32_t* __restrict__ row_assign) {
  const int a = blockIdx.x * blockDim.x + threadIdx.x;
  if (a < A) row_assign[row_of[a]] = a;
}

__device__ __forceinline__ u32x4 pack8(const bf16_t (&e)[8]) {
  u32x4 v;
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = (uint32_t)e[2 * u] | ((uint32_t)e[2 * u + 1] << 16);
  return v;
}

// Row-space operands of the weight gradients that no kernel stores as bf16
// rows: dst[r][c] (row stride ld) for rows r < padded[G] of the layer and
// columns c < C.
struct RowSource {
  int kind;  // 0: p_r * dy[t_r] (dO), 1: bf16(SiLU(g) u) (h)
  const float* dy;            // [T][D]
  const float* topk_w;        // [T*k]
  const int32_t* row_token;   // [rows]
  const int32_t* row_assign;  // [rows], -1 off routed rows
  const int32_t* padded;      // group offsets; padded[E] is the first shared row
  const int32_t* tile_group;
  int E, BM, D, F, Fs, ldh;
  const float* gu;            // [rows][2 ldh], fp32 ...
  const bf16_t* gu16;         // ... or bf16 (kept by a training forward)
};

// eight consecutive values of a g | u row, fp32 or bf16
__device__ __forceinline__ void load8(const float* f32, const bf16_t* b16, int64_t i, float (&v)[8]) {
  if (b16) {
    const u32x4 w = ld16(b16 + i);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[2 * u] = bf16_to_f32((bf16_t)(w[u] & 0xffff));
      v[2 * u + 1] = bf16_to_f32((bf16_t)(w[u] >> 16));
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(f32 + i);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// columns c .. c + 7 (c % 8 == 0) of row r, as bf16
__device__ __forceinline__ u32x4 row_values8(const RowSource& q, int64_t r, int c) {
  const int t = q.row_token[r];
  if (t < 0) return u32x4{0, 0, 0, 0};
  bf16_t e[8];
  switch (q.kind) {
    case 0: {
      const int a = q.row_assign[r];
      const float p = a >= 0 ? q.topk_w[a] : 1.f;  // the shared expert's rows: weight 1
      const float4* src = reinterpret_cast<const float4*>(q.dy + (int64_t)t * q.D + c);
      const float4 v0 = src[0], v1 = src[1];
      const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) e[u] = f32_to_bf16(p * f[u]);
      return pack8(e);
    }
    default: {  // 1
      const int Fg = q.tile_group[r / q.BM] >= q.E ? q.Fs : q.F;
      if (c >= Fg) return u32x4{0, 0, 0, 0};  // Fg % 8 == 0: a chunk is all in or all out
      float g[8], u[8];
      load8(q.gu, q.gu16, r * 2 * q.ldh + c, g);
      load8(q.gu, q.gu16, r * 2 * q.ldh + Fg + c, u);
#pragma unroll
      for (int w = 0; w < 8; ++w) e[w] = f32_to_bf16(silu(g[w]) * u[w]);
      return pack8(e);
    }
  }
}

__global__ __launch_bounds__(256) void moe_rows_kernel(RowSource q, const int32_t* total, int C,
                                                      int64_t ld, bf16_t* __restrict__ dst) {
  const int per_row = C / 8;  // C % 8 == 0
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = i / per_row;
  if (r >= total[0]) return;
  const int c = (int)(i - r * per_row) * 8;
  st16(dst + r * ld + c, row_values8(q, r, c));
}

// One wave per row: SwiGLU backward.  dh' = W_down^T dy (fp32 rows), p the
// row's routing weight (1 on shared rows):
//   dp = sum_f dh'_f h_f (h rounded to bf16, as the forward stores it),
//   dh = p dh',  dg = dh u SiLU'(g),  du = dh SiLU(g);
// dGU[r] = [dg | du] (bf16; zeros past 2 Fg and on padding rows), dp per
// assignment.  Each lane sums its columns in order, then the wave's lanes are
// added by a fixed shuffle tree.
__global__ __launch_bounds__(256) void moe_swiglu_bwd_kernel(
    const float* __restrict__ gu, const bf16_t* __restrict__ gu16, const float* __restrict__ dhp,
    const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ row_assign, const int32_t* __restrict__ tile_group,
    const float* __restrict__ topk_w, const int32_t* __restrict__ total, int E, int BM, int F, int Fs,
    int ldh, bf16_t* __restrict__ dgu, float* __restrict__ dp) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= total[0]) return;
  const bool shared = tile_group[r / BM] >= E;
  const int Fg = shared ? Fs : F;
  const int a = row_assign[r];
  const bool valid = row_token[r] >= 0;
  const float p = shared ? 1.f : (a >= 0 ? topk_w[a] : 0.f);
  const int64_t gbase = r * 2 * ldh;  // g at gbase + f, u at gbase + Fg + f
  const float* hr = dhp + r * ldh;
  bf16_t* out = dgu + r * 2 * ldh;
  float acc = 0.f;
  // eight consecutive columns per lane and step (F, Fs and ldh are multiples
  // of 8, so a chunk is all inside or all outside [0, Fg))
  for (int f = 8 * lane; f < ldh; f += 8 * 64) {
    bf16_t eg[8], eu[8];
    if (f < Fg) {
      if (valid) {
        float g[8], u[8];
        load8(gu, gu16, gbase + f, g);
        load8(gu, gu16, gbase + Fg + f, u);
        const float4 d0 = *reinterpret_cast<const float4*>(hr + f);
        const float4 d4 = *reinterpret_cast<const float4*>(hr + f + 4);
        const float d1[8] = {d0.x, d0.y, d0.z, d0.w, d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const float s = 1.f / (1.f + __builtin_amdgcn_exp2f(-g[w] * 1.4426950408889634f));
          const float sl = g[w] * s;
          const float h = bf16_to_f32(f32_to_bf16(sl * u[w]));
          acc += d1[w] * h;
          const float dh = p * d1[w];
          eg[w] = f32_to_bf16(dh * u[w] * s * (1.f + g[w] * (1.f - s)));
          eu[w] = f32_to_bf16(dh * sl);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 8; ++w) eg[w] = eu[w] = 0;
      }
      st16(out + f, pack8(eg));
      st16(out + Fg + f, pack8(eu));
    } else {  // columns 2 Fg .. 2 ldh - 1 (reached when Fg < ldh)
      st16(out + Fg + f, u32x4{0, 0, 0, 0});
      st16(out + f + ldh, u32x4{0, 0, 0, 0});
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0 && !shared && a >= 0) dp[a] = acc;
}

// Per token: dl_j = p_j (dp_j - sum_i p_i dp_i), the sum in slot order.
__global__ void moe_router_bwd_kernel(const float* __restrict__ topk_w, const float* __restrict__ dp,
                                      int T, int k, float* __restrict__ dl) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += topk_w[t * k + j] * dp[t * k + j];
  for (int j = 0; j < k; ++j) dl[t * k + j] = topk_w[t * k + j] * (dp[t * k + j] - s);
}

// dW_g[e][d] = sum over expert e's assignments of dl_a x[t_a][d]: workgroup
// (64 columns, e); wave w adds assignments i = i0 + w, i0 + w + 4, ... (in
// order) and the four partial sums are added in wave order.  dbias[e] = the
// same sum of dl_a (bias inside the logits) or 0.
__global__ __launch_bounds__(256) void moe_router_wgrad_kernel(
    const float* __restrict__ dl, const bf16_t* __restrict__ x, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_assign, int k, int D, int bias_grad, float* __restrict__ dwg,
    float* __restrict__ dbias) {
  __shared__ float part[4][64];
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d = blockIdx.x * 64 + lane;
  const int i0 = offsets[e], i1 = offsets[e + 1];
  float acc = 0.f;
  if (d < D)
    for (int i = i0 + wave; i < i1; i += 4) {
      const int a = sorted_assign[i];
      acc += dl[a] * bf16_to_f32(x[(int64_t)(a / k) * D + d]);
    }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && d < D)
    dwg[(int64_t)e * D + d] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
  if (dbias && blockIdx.x == 0 && threadIdx.x == 0) {
    float sb = 0.f;
    if (bias_grad)
      for (int i = i0; i < i1; ++i) sb += dl[sorted_assign[i]];
    dbias[e] = sb;
  }
}

// dx[t] = sum_j dX[row_of[t k + j]] + dX[shared_row(t)] + sum_j dl_j W_g[e_j]
__global__ __launch_bounds__(256) void moe_combine_bwd_kernel(
    const float* __restrict__ dxr, const int32_t* __restrict__ row_of, const int32_t* __restrict__ ids,
    const float* __restrict__ dl, const bf16_t* __restrict__ w_g, const int32_t* __restrict__ padded,
    int T, int D, int k, int E, int has_shared, float* __restrict__ dx) {
  const int t = blockIdx.x;  // tokens on x: their count is the large one
  const int d = blockIdx.y * blockDim.x + threadIdx.x;
  if (t >= T || d >= D) return;
  float v = 0.f;
  for (int j = 0; j < k; ++j) v += dxr[(int64_t)row_of[t * k + j] * D + d];
  if (has_shared) v += dxr[(int64_t)(padded[E] + t) * D + d];
  for (int j = 0; j < k; ++j)
    v += dl[t * k + j] * bf16_to_f32(w_g[(int64_t)ids[t * k + j] * D + d]);
  dx[(int64_t)t * D + d] = v;
}

}  // namespace

hipError_t launch_gather_rows(const void* src, bool src_f32, const int32_t* row_token,
                              const int32_t* total, int64_t cap, int D, uint16_t* dst, hipStream_t s) {
  if (cap <= 0) return hipSuccess;
  if (src_f32)
    hipLaunchKernelGGL(moe_gather_rows_kernel<float>, dim3((unsigned)cap), dim3(256), 0, s,
                       static_cast<const float*>(src), row_token, total, D, dst);
  else
    hipLaunchKernelGGL(moe_gather_rows_kernel<bf16_t>, dim3((unsigned)cap), dim3(256), 0, s,
                       static_cast<const bf16_t*>(src), row_token, total, D, dst);
  return hipGetLastError();
}

hipError_t launch_row_assign(const int32_t* row_of, int A, int64_t cap, int32_t* row_assign,
                             hipStream_t s) {
  hipError_t e = launch_fill_i32(row_assign, cap, -1, s);
  if (e != hipSuccess) return e;
  if (A > 0)
    hipLaunchKernelGGL(moe_row_assign_kernel, dim3((A + 255) / 256), dim3(256), 0, s, row_of, A,
                       row_assign);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, out, n);
  return hipGetLastError();
}

hipError_t launch_rows(const BwdRows& b, int kind, int C, uint16_t* dst, int64_t ld, hipStream_t s) {
  if (b.cap <= 0 || C <= 0) return hipSuccess;
  RowSource q{kind, b.dy, b.topk_w, b.row_token, b.row_assign, b.padded, b.tile_group, b.E, b.BM,
              b.D, b.F, b.Fs, b.ldh, b.gu, b.gu16};
  const int64_t n = b.cap * (C / 8);
  hipLaunchKernelGGL(moe_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, q, b.total,
                     C, ld, dst);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const BwdRows& b, const float* dhp, float* dp, hipStream_t s) {
  if (b.cap <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_swiglu_bwd_kernel, dim3((unsigned)((b.cap + 3) / 4)), dim3(256), 0, s, b.gu,
                     b.gu16, dhp, b.row_token, b.row_assign, b.tile_group, b.topk_w, b.total, b.E, b.BM, b.F,
                     b.Fs, b.ldh, b.dgu_w, dp);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* topk_w, const float* dp, int T, int k, float* dl,
                             hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_router_bwd_kernel, dim3((T + 255) / 256), dim3(256), 0, s, topk_w, dp, T, k,
                     dl);
  return hipGetLastError();
}

hipError_t launch_router_wgrad(const float* dl, const uint16_t* x, const int32_t* offsets,
                               const int32_t* sorted_assign, int E, int k, int D, int bias_grad,
                               float* dwg, float* dbias, hipStream_t s) {
  hipLaunchKernelGGL(moe_router_wgrad_kernel, dim3((D + 63) / 64, E), dim3(256), 0, s, dl, x, offsets,
                     sorted_assign, k, D, bias_grad, dwg, dbias);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const float* dxr, const int32_t* row_of, const int32_t* ids,
                              const float* dl, const uint16_t* w_g, const int32_t* padded, int T, int D,
                              int k, int E, int has_shared, float* dx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_combine_bwd_kernel, dim3(T, (D + 255) / 256), dim3(256), 0, s, dxr, row_of, ids,
                     dl, w_g, padded, T, D, k, E, has_shared, dx);
  return hipGetLastError();
}

}  // namespace moe
