// moe_align: group the T*k token-to-expert assignments by expert.
//
// Dispatch step of "Mixture of Experts optimiza Transformers y LLMs", section
// "Ejecución eficiente: backends de expertos" (tokens sorted by expert id
// before the grouped products) and of the glossary "MoE (Mixture of Experts -
// Mezcla de Expertos)", section 3 step 3 (a token's vector is duplicated to
// each chosen expert).
//
// One workgroup per group g (E routed experts, plus the shared-expert group).
// Every workgroup builds the full expert histogram in LDS (integer counts, so
// the atomics' order does not matter) and derives offsets and padded offsets;
// workgroup g then walks the assignments in ascending order and compacts the
// ones routed to g with a ballot/popcount rank, so the output is the stable
// order by assignment index and bitwise reproducible.
#include "device.hpp"
#include "launch.hpp"
#include "topk.hpp"  // ranks_before

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__global__ __launch_bounds__(kThreads) void moe_align_kernel(
    const int32_t* __restrict__ ids, int A, int k, int E, int id_base, int BM, int shared_rows,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ padded,
    int32_t* __restrict__ sorted_assign, int32_t* __restrict__ row_of,
    int32_t* __restrict__ row_token, int32_t* __restrict__ tile_group,
    int32_t* __restrict__ n_tiles, RouteFinish fin) {
  __shared__ int hist[258];
  __shared__ int s_ids[kSmallRouteT * 8];
  __shared__ int s_off[258];
  __shared__ int s_pad[258];
  __shared__ int wave_tot[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = E + (shared_rows > 0 ? 1 : 0);
  const int g = blockIdx.x;

  if (fin.partial) {
    // Few tokens: finish the routing here.  Every workgroup adds the partial
    // logits of all T <= kSmallRouteT tokens (part order, then the bias),
    // picks each token's top-k (E <= kSmallRouteE) and keeps the ids in LDS;
    // workgroup 0 also stores ids and weights.
    // [T][EL + 1] logits, then (selection-only bias) [T][EL + 1] top-k keys
    extern __shared__ float lg[];
    const int T = A / k, EL = fin.E;
    float* const key = fin.sel ? lg + T * (EL + 1) : lg;
    for (int idx = tid; idx < T * EL; idx += kThreads) {
      const int t = idx / EL, e = idx - t * EL;
      const float* src = fin.partial + (int64_t)t * EL + e;
      const int64_t stride = (int64_t)T * EL;
      float v = 0.f;
      for (int q0 = 0; q0 < fin.P; q0 += 16) {
        float pv[16];  // every load of the group in flight before the in-order sum
#pragma unroll
        for (int q = 0; q < 16; ++q) pv[q] = q0 + q < fin.P ? src[(q0 + q) * stride] : 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q)
          if (q0 + q < fin.P) v = (q0 + q == 0) ? pv[q] : v + pv[q];
      }
      if (fin.bias) v += fin.bias[e];
      lg[t * (EL + 1) + e] = v;
      if (fin.sel) key[t * (EL + 1) + e] = v + fin.sel[e];
    }
    __syncthreads();
    // slot of every (token, expert): the number of the token's keys that
    // rank before its own (value descending, ties to the lower index); one
    // thread per pair, so all tokens are ranked at once
    for (int idx = tid; idx < T * EL; idx += kThreads) {
      const int t = idx / EL, e = idx - t * EL;
      const float* row = key + t * (EL + 1);
      const float v = row[e];
      int rank = 0;
      for (int j = 0; j < EL; ++j) rank += ranks_before(row[j], j, v, e) ? 1 : 0;
      if (rank < k) s_ids[t * k + rank] = e;
    }
    __syncthreads();
    if (g == 0) {  // softmax over the chosen logits, adding exp(l - l_max) in slot order
      for (int idx = tid; idx < T * k; idx += kThreads) {
        const int t = idx / k, q = idx - t * k;
        const float* row = lg + t * (EL + 1);
        float vmax = row[s_ids[t * k]];
        for (int j = 1; j < k; ++j) vmax = fmaxf(vmax, row[s_ids[t * k + j]]);
        float tot = 0.f, mine = 0.f;
        for (int j = 0; j < k; ++j) {
          const float ex = expf(row[s_ids[t * k + j]] - vmax);
          tot += ex;
          if (j == q) mine = ex;
        }
        fin.ids[idx] = s_ids[idx];
        fin.wts[idx] = mine / tot;
      }
    }
  }
  // group of assignment a (ids are global; this call holds experts id_base ..)
  auto id_of = [&](int a) { return (fin.partial ? s_ids[a] : ids[a]) - id_base; };

  for (int i = tid; i < G; i += kThreads) hist[i] = (i == E) ? shared_rows : 0;
  __syncthreads();
  for (int a = tid; a < A; a += kThreads) {
    const int e = id_of(a);
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int o = 0, p = 0;
    for (int i = 0; i < G; ++i) {
      s_off[i] = o;
      s_pad[i] = p;
      o += hist[i];
      p += (hist[i] + BM - 1) / BM * BM;
    }
    s_off[G] = o;
    s_pad[G] = p;
  }
  __syncthreads();
  if (g == 0) {
    for (int i = tid; i < G; i += kThreads) counts[i] = hist[i];
    for (int i = tid; i <= G; i += kThreads) {
      offsets[i] = s_off[i];
      padded[i] = s_pad[i];
    }
    if (tid == 0) n_tiles[0] = s_pad[G] / BM;
    // assignments with an id outside [0, E) get no row
    for (int a = tid; a < A; a += kThreads) {
      const int e = id_of(a);
      if (e < 0 || e >= E) row_of[a] = -1;
    }
  }
  const int cnt = hist[g], pbeg = s_pad[g], pend = s_pad[g + 1], obeg = s_off[g];

  if (g < E) {
    int running = 0;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < A; base += kThreads) {
      const int a = base + tid;
      const bool pred = a < A && id_of(a) == g;
      const uint64_t m = __ballot(pred);
      const int rank = __popcll(m & below);
      if (lane == 0) wave_tot[wave] = __popcll(m);
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int c = wave_tot[w];
        before += (w < wave) ? c : 0;
        total += c;
      }
      if (pred) {
        const int pos = running + before + rank;
        sorted_assign[obeg + pos] = a;
        row_of[a] = pbeg + pos;
        row_token[pbeg + pos] = a / k;
      }
      running += total;
      __syncthreads();  // wave_tot is rewritten by the next chunk
    }
  } else {
    for (int t = tid; t < shared_rows; t += kThreads) row_token[pbeg + t] = t;
  }
  for (int r = pbeg + cnt + tid; r < pend; r += kThreads) row_token[r] = -1;
  for (int i = pbeg / BM + tid; i < pend / BM; i += kThreads) tile_group[i] = g;
}

}  // namespace

hipError_t launch_align(const int32_t* ids, int T, int k, int E, int id_base, int BM, int shared_rows,
                        int32_t* counts, int32_t* offsets, int32_t* padded, int32_t* sorted_assign,
                        int32_t* row_of, int32_t* row_token, int32_t* tile_group, int32_t* n_tiles,
                        const RouteFinish* fin, hipStream_t s) {
  const int G = E + (shared_rows > 0 ? 1 : 0);
  RouteFinish f{};
  size_t lds = 0;
  if (fin) {
    if (T > kSmallRouteT || k > 8 || fin->E > kSmallRouteE) return hipErrorInvalidValue;
    f = *fin;
    lds = sizeof(float) * (size_t)T * (fin->E + 1) * (fin->sel ? 2 : 1);
    // set once per process (a function-local static is initialised thread-safely)
    static const hipError_t attr = hipFuncSetAttribute(
        (const void*)moe_align_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)(sizeof(float) * 2 * kSmallRouteT * (kSmallRouteE + 1)));
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL(moe_align_kernel, dim3(G), dim3(kThreads), lds, s, ids, T * k, k, E, id_base, BM,
                     shared_rows, counts, offsets, padded, sorted_assign, row_of, row_token,
                     tile_group, n_tiles, f);
  return hipGetLastError();
}

__global__ void moe_fill_i32_kernel(int32_t* __restrict__ out, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = v;
}

hipError_t launch_fill_i32(int32_t* out, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, out, n,
                     v);
  return hipGetLastError();
}

}  // namespace moe
