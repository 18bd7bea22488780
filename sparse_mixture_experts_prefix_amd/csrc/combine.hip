// moe_combine: weighted return of the expert outputs to token order.
//
// Glossary "MoE (Mixture of Experts - Mezcla de Expertos)", section 3 step 4
// and diagram row 4: y = sum_i p_i * Expert_i(x); "Mixture of Experts optimiza
// Transformers y LLMs", section "Ejecución eficiente: backends de expertos":
// the routing weights are applied and the results regrouped in the original
// order.  The shared expert (glossary section 2, item 3) is added last with
// weight 1.
//
// One workgroup per token gathers its k expert rows of Yp (fp32) and sums them
// in slot order with float4 loads; no atomics, so the result is bitwise
// reproducible.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kMaxK = 8;

__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ Yp,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ wts,
                                                      const int32_t* __restrict__ padded, int T,
                                                      int D, int k, int E, int has_shared,
                                                      float* __restrict__ y) {
  const int t = blockIdx.x;
  int64_t rows[kMaxK];
  float w[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const int r = (j < k) ? row_of[(int64_t)t * k + j] : -1;
    rows[j] = r;
    w[j] = (r >= 0) ? wts[(int64_t)t * k + j] : 0.f;
  }
  const int64_t srow = has_shared ? (int64_t)padded[E] + t : -1;
  const int D4 = D / 4;
  for (int d = threadIdx.x; d < D4; d += blockDim.x) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (rows[j] >= 0) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(Yp + rows[j] * D + 4 * d);
        s += w[j] * v;
      }
    }
    if (srow >= 0) s += *reinterpret_cast<const f32x4*>(Yp + srow * D + 4 * d);
    *reinterpret_cast<f32x4*>(y + (int64_t)t * D + 4 * d) = s;
  }
}

}  // namespace

hipError_t launch_combine(const float* Yp, const int32_t* row_of, const float* wts,
                          const int32_t* padded, int T, int D, int k, int E, int has_shared,
                          float* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(T), dim3(256), 0, s, Yp, row_of, wts, padded, T, D, k, E,
                     has_shared, y);
  return hipGetLastError();
}

}  // namespace moe
