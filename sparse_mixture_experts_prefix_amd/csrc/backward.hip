// Backward pass of the layer: the kernels around the grouped GEMMs.
//
// Gradients of sum_t <dy[t], y[t]> for a given routing, by the chain rule of
// the forward pass (the pages' training sections name grouped-GEMM kernels
// but no formulas: "Mixture of Experts optimiza Transformers y LLMs", section
// on training; "Transformers v5 El Secreto Detrás de los Modelos MoE Más
// Rápidos", section "Entrenamiento MoE").  The row-space products (g and u
// again, dh' = W_down^T dy, dx rows = [dg du] W_gate_up) run on the forward's
// grouped GEMM over transposed weight copies; the weight gradients on the
// variable-K grouped GEMM over transposed row buffers.  This file holds the
// rest, all bandwidth-bound:
//  - gathering x and dy rows in expert order (bf16, padding rows zero),
//  - a batched tiled transpose with a per-element source function,
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

__global__ void moe_fill_i32_rows_kernel(int32_t* __restrict__ out, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = v;
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

// Batched transpose: dst[b][c][r] = src[b][r][c], bf16, 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void moe_transpose_kernel(const bf16_t* __restrict__ src,
                                                            bf16_t* __restrict__ dst, int R, int C) {
  __shared__ bf16_t tile[64][66];
  const int64_t b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const bf16_t* s = src + b * (int64_t)R * C;
  bf16_t* d = dst + b * (int64_t)R * C;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < C) tile[i][tx] = s[(int64_t)r * C + c];
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < R && c < C) d[(int64_t)c * R + r] = tile[tx][i];
  }
}

// The row-space operands of the weight gradients, transposed: dst[c][r]
// (row stride ld) for rows r < padded[G] of the layer and columns c < C.
struct RowSource {
  int kind;  // 0: p_r * dy[t_r] (dO), 1: bf16(SiLU(g) u) (h), 2: dGU rows, 3: x rows
  const float* dy;            // [T][D]
  const float* topk_w;        // [T*k]
  const int32_t* row_token;   // [rows]
  const int32_t* row_assign;  // [rows], -1 off routed rows
  const int32_t* padded;      // group offsets; padded[E] is the first shared row
  const int32_t* tile_group;
  int E, BM, D, F, Fs, ldh;
  const float* gu;            // [rows][2 ldh]
  const bf16_t* rows16;       // [rows][cols] (kind 2: stride 2 ldh; kind 3: stride D)
};

__device__ __forceinline__ float row_value(const RowSource& q, int64_t r, int c) {
  const int t = q.row_token[r];
  if (t < 0) return 0.f;
  switch (q.kind) {
    case 0: {
      const int a = q.row_assign[r];
      const float p = a >= 0 ? q.topk_w[a] : 1.f;  // the shared expert's rows: weight 1
      return p * q.dy[(int64_t)t * q.D + c];
    }
    case 1: {
      const int Fg = q.tile_group[r / q.BM] >= q.E ? q.Fs : q.F;
      if (c >= Fg) return 0.f;
      const float g = q.gu[r * 2 * q.ldh + c], u = q.gu[r * 2 * q.ldh + Fg + c];
      return bf16_to_f32(f32_to_bf16(silu(g) * u));
    }
    case 2: return bf16_to_f32(q.rows16[r * 2 * q.ldh + c]);
    default: return bf16_to_f32(q.rows16[r * q.D + c]);
  }
}

__global__ __launch_bounds__(256) void moe_rows_transpose_kernel(RowSource q, const int32_t* total,
                                                                 int C, int64_t ld,
                                                                 bf16_t* __restrict__ dst) {
  __shared__ bf16_t tile[64][66];
  const int64_t r0 = (int64_t)blockIdx.x * 64;  // rows on x: their count is the large one
  const int c0 = blockIdx.y * 64;
  const int64_t R = total[0];
  if (r0 >= R) return;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i;
    const int c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? f32_to_bf16(row_value(q, r, c)) : (bf16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i;
    const int64_t r = r0 + tx;
    if (r < R && c < C) dst[(int64_t)c * ld + r] = tile[tx][i];
  }
}

// One wave per row: SwiGLU backward.  dh' = W_down^T dy (fp32 rows), p the
// row's routing weight (1 on shared rows):
//   dp = sum_f dh'_f h_f (h rounded to bf16, as the forward stores it),
//   dh = p dh',  dg = dh u SiLU'(g),  du = dh SiLU(g);
// dGU[r] = [dg | du] (bf16; zeros past 2 Fg and on padding rows), dp per
// assignment.  The wave's sum over f is a fixed shuffle tree.
__global__ __launch_bounds__(256) void moe_swiglu_bwd_kernel(
    const float* __restrict__ gu, const float* __restrict__ dhp, const int32_t* __restrict__ row_token,
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
  const float* gr = gu + r * 2 * ldh;
  const float* hr = dhp + r * ldh;
  bf16_t* out = dgu + r * 2 * ldh;
  float acc = 0.f;
  for (int f = lane; f < ldh; f += 64) {
    float dg = 0.f, du = 0.f;
    if (valid && f < Fg) {
      const float g = gr[f], u = gr[Fg + f];
      const float s = 1.f / (1.f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
      const float sl = g * s;
      const float h = bf16_to_f32(f32_to_bf16(sl * u));
      const float d1 = hr[f];
      acc += d1 * h;
      const float dh = p * d1;
      dg = dh * u * s * (1.f + g * (1.f - s));
      du = dh * sl;
    }
    if (f < Fg) {
      out[f] = f32_to_bf16(dg);
      out[Fg + f] = f32_to_bf16(du);
    } else {
      out[Fg + f] = (bf16_t)0;  // columns 2 Fg .. 2 ldh - 1 (reached when Fg < ldh)
      out[f + ldh] = (bf16_t)0;
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

// dW_g[e][d] = sum over expert e's assignments (ascending a) of dl_a x[t_a][d];
// dbias[e] = the same sum of dl_a (bias inside the logits) or 0.
__global__ __launch_bounds__(256) void moe_router_wgrad_kernel(
    const float* __restrict__ dl, const bf16_t* __restrict__ x, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_assign, int k, int D, int bias_grad, float* __restrict__ dwg,
    float* __restrict__ dbias) {
  const int e = blockIdx.y;
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  const int i0 = offsets[e], i1 = offsets[e + 1];
  if (d < D) {
    float acc = 0.f;
    for (int i = i0; i < i1; ++i) {
      const int a = sorted_assign[i];
      acc += dl[a] * bf16_to_f32(x[(int64_t)(a / k) * D + d]);
    }
    dwg[(int64_t)e * D + d] = acc;
  }
  if (dbias && blockIdx.x == 0 && threadIdx.x == 0) {
    float s = 0.f;
    if (bias_grad)
      for (int i = i0; i < i1; ++i) s += dl[sorted_assign[i]];
    dbias[e] = s;
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
  if (cap > 0)
    hipLaunchKernelGGL(moe_fill_i32_rows_kernel, dim3((unsigned)((cap + 255) / 256)), dim3(256), 0, s,
                       row_assign, cap, -1);
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

hipError_t launch_transpose(const uint16_t* src, uint16_t* dst, int B, int R, int C, hipStream_t s) {
  if (B <= 0 || R <= 0 || C <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_transpose_kernel, dim3((C + 63) / 64, (R + 63) / 64, B), dim3(256), 0, s, src,
                     dst, R, C);
  return hipGetLastError();
}

hipError_t launch_rows_transpose(const BwdRows& b, int kind, int C, uint16_t* dst, hipStream_t s) {
  if (b.cap <= 0 || C <= 0) return hipSuccess;
  RowSource q{kind, b.dy, b.topk_w, b.row_token, b.row_assign, b.padded, b.tile_group, b.E, b.BM,
              b.D, b.F, b.Fs, b.ldh, b.gu, kind == 2 ? b.dgu : b.xr};
  hipLaunchKernelGGL(moe_rows_transpose_kernel, dim3((unsigned)((b.cap + 63) / 64), (C + 63) / 64),
                     dim3(256), 0, s, q, b.total, C, b.cap, dst);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const BwdRows& b, const float* dhp, float* dp, hipStream_t s) {
  if (b.cap <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_swiglu_bwd_kernel, dim3((unsigned)((b.cap + 3) / 4)), dim3(256), 0, s, b.gu,
                     dhp, b.row_token, b.row_assign, b.tile_group, b.topk_w, b.total, b.E, b.BM, b.F,
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
  hipLaunchKernelGGL(moe_router_wgrad_kernel, dim3((D + 255) / 256, E), dim3(256), 0, s, dl, x, offsets,
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
