// moe_align: group the T*k token-to-expert assignments by expert.
//
// Dispatch step of "Mixture of Experts optimiza Transformers y LLMs", section
// "Ejecución eficiente: backends de expertos" (tokens sorted by expert id
// before the grouped products) and of the glossary "MoE (Mixture of Experts -
// Mezcla de Expertos)", section 3 step 3 (a token's vector is duplicated to
// each chosen expert).
//
// Output order: the assignments of group g in ascending assignment index
// (stable), so the result is bitwise reproducible; no atomic decides a
// position.  Two kernels compute it:
//  - few assignments (A <= kSmallA, the decode sizes): one workgroup holds
//    every id in LDS.  Each wave ranks its 64 lanes among the lanes of the
//    same expert (one ballot per distinct expert), per-wave counts give each
//    wave's base inside a group, and a wave-wide scan gives the offsets.
//  - many assignments: one workgroup per group; each builds the full
//    histogram in LDS (integer counts, so the atomics' order does not
//    matter), scans it, and compacts the assignments of its own group with a
//    ballot/popcount rank while walking them in ascending order.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxG = 257;        // 256 routed experts + the shared one
constexpr int kSmallA = kThreads; // one assignment per thread of the one-workgroup path
constexpr int kScanPer = 5;       // groups per lane of the wave-wide scan (64 * 5 >= kMaxG)

// Exclusive prefix sums of v[0..n) (n <= 64 * kScanPer), each value first
// rounded up to a multiple of bm (bm = 1: plain counts), into out[0..n];
// out[n] is the total.  Called by all 64 lanes of one wave.
__device__ __forceinline__ void wave_scan(const int* v, int n, int bm, int* out, int lane) {
  int loc[kScanPer];
  int s = 0;
#pragma unroll
  for (int q = 0; q < kScanPer; ++q) {
    const int i = lane * kScanPer + q;
    const int c = i < n ? (v[i] + bm - 1) / bm * bm : 0;
    loc[q] = s;
    s += c;
  }
  int inc = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  const int excl = inc - s;
#pragma unroll
  for (int q = 0; q < kScanPer; ++q) {
    const int i = lane * kScanPer + q;
    if (i < n) out[i] = excl + loc[q];
  }
  if (lane == 63) out[n] = inc;
}

// Rows that no assignment fills: padding rows read as token -1, the shared
// expert's rows hold tokens 0 .. T-1 in order; and the group of every tile.
// Row r belongs to the last group g with pad[g] <= r (empty groups have
// pad[g] == pad[g + 1], so the search skips them).
__device__ __forceinline__ void fill_rows(const int* hist, const int* pad, int G, int E, int BM,
                                          int32_t* row_token, int32_t* tile_group, int tid) {
  const int rows = pad[G];
  for (int r = tid; r < rows; r += kThreads) {
    int lo = 0, hi = G - 1;  // pad[lo] <= r < pad[hi + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pad[mid] <= r) lo = mid; else hi = mid - 1;
    }
    const int j = r - pad[lo];
    if (j >= hist[lo]) row_token[r] = -1;
    else if (lo == E) row_token[r] = j;
    if (j % BM == 0) tile_group[r / BM] = lo;
  }
}

__global__ __launch_bounds__(kThreads) void moe_align_small_kernel(
    const int32_t* __restrict__ ids, int A, int k, int E, int id_base, int BM, int shared_rows,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ padded,
    int32_t* __restrict__ sorted_assign, int32_t* __restrict__ row_of,
    int32_t* __restrict__ row_token, int32_t* __restrict__ tile_group,
    int32_t* __restrict__ n_tiles) {
  __shared__ int s_ids[kSmallA];
  __shared__ int wcnt[kWaves][kMaxG];  // per-wave counts, then each wave's base in a group
  __shared__ int hist[kMaxG];
  __shared__ int s_off[kMaxG + 1];
  __shared__ int s_pad[kMaxG + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = E + (shared_rows > 0 ? 1 : 0);
  for (int i = tid; i < kWaves * kMaxG; i += kThreads) (&wcnt[0][0])[i] = 0;

  for (int a = tid; a < A; a += kThreads) s_ids[a] = ids[a];
  __syncthreads();

  // rank of assignment a = tid among the lanes of its wave routed to the same
  // group (ascending lane order), and the wave's count of each group
  const int a = tid;
  const int e = a < A ? s_ids[a] - id_base : -1;
  const bool valid = a < A && e >= 0 && e < E;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
  uint64_t pending = __ballot(valid);
  while (pending) {
    const int leader = (int)__builtin_ctzll(pending);
    const int el = __builtin_amdgcn_readlane(e, leader);
    const bool mine = valid && e == el;
    const uint64_t m = __ballot(mine);
    if (mine) rank = __popcll(m & below);
    if (lane == 0) wcnt[wave][el] = __popcll(m);
    pending &= ~m;
  }
  __syncthreads();
  // group totals; wcnt becomes each wave's exclusive base inside the group
  for (int i = tid; i < G; i += kThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = wcnt[w][i];
      wcnt[w][i] = run;
      run += c;
    }
    hist[i] = (i == E) ? shared_rows : run;
  }
  __syncthreads();
  if (wave == 0) {
    wave_scan(hist, G, 1, s_off, lane);
    wave_scan(hist, G, BM, s_pad, lane);
  }
  __syncthreads();

  if (valid) {
    const int r = wcnt[wave][e] + rank;
    sorted_assign[s_off[e] + r] = a;
    row_of[a] = s_pad[e] + r;
    row_token[s_pad[e] + r] = a / k;
  } else if (a < A) {
    row_of[a] = -1;  // an id outside the held experts gets no row
  }
  for (int i = tid; i < G; i += kThreads) counts[i] = hist[i];
  for (int i = tid; i <= G; i += kThreads) {
    offsets[i] = s_off[i];
    padded[i] = s_pad[i];
  }
  if (tid == 0) n_tiles[0] = s_pad[G] / BM;
  fill_rows(hist, s_pad, G, E, BM, row_token, tile_group, tid);
}

__global__ __launch_bounds__(kThreads) void moe_align_kernel(
    const int32_t* __restrict__ ids, int A, int k, int E, int id_base, int BM, int shared_rows,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ padded,
    int32_t* __restrict__ sorted_assign, int32_t* __restrict__ row_of,
    int32_t* __restrict__ row_token, int32_t* __restrict__ tile_group,
    int32_t* __restrict__ n_tiles) {
  __shared__ int hist[kMaxG];
  __shared__ int s_off[kMaxG + 1];
  __shared__ int s_pad[kMaxG + 1];
  __shared__ int wave_tot[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = E + (shared_rows > 0 ? 1 : 0);
  const int g = blockIdx.x;
  // group of assignment a (ids are global; this call holds experts id_base ..)
  auto id_of = [&](int a) { return ids[a] - id_base; };

  for (int i = tid; i < G; i += kThreads) hist[i] = (i == E) ? shared_rows : 0;
  __syncthreads();
  for (int a = tid; a < A; a += kThreads) {
    const int e = id_of(a);
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (wave == 0) {
    wave_scan(hist, G, 1, s_off, lane);
    wave_scan(hist, G, BM, s_pad, lane);
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
                        hipStream_t s) {
  const int G = E + (shared_rows > 0 ? 1 : 0);
  if (G > kMaxG) return hipErrorInvalidValue;
  const int64_t A = (int64_t)T * k;
  if (A <= kSmallA)
    hipLaunchKernelGGL(moe_align_small_kernel, dim3(1), dim3(kThreads), 0, s, ids, (int)A, k, E,
                       id_base, BM, shared_rows, counts, offsets, padded, sorted_assign, row_of,
                       row_token, tile_group, n_tiles);
  else
    hipLaunchKernelGGL(moe_align_kernel, dim3(G), dim3(kThreads), 0, s, ids, (int)A, k, E, id_base,
                       BM, shared_rows, counts, offsets, padded, sorted_assign, row_of, row_token,
                       tile_group, n_tiles);
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
