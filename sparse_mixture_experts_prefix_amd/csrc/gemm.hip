// moe_gemm_gate_up / moe_gemm_down: grouped bf16 MFMA GEMMs over the
// expert-contiguous rows produced by moe_align.
//
// The expert FFN is the SwiGLU of the glossary "MoE (Mixture of Experts -
// Mezcla de Expertos)", section 3 step 3: h = SiLU(W_a x) * (W_b x), then
// W_down h.  The packed [E, 2F, D] gate/up tensor follows "Transformers v5 El
// Secreto Detrás de los Modelos MoE Más Rápidos", section "La Solución:
// WeightConverter" (experts on dim 0, the two projections concatenated on
// dim 1); rows 0..F-1 of an expert are the activated half.
//
// Tile (BM x BN x 64) per workgroup of 4 wavefronts in a 2 x 2 layout; each
// wave owns (BM/2) x (BN/2) of the output as 32x32 MFMA tiles.  For gate/up
// the BN rows of the B tile are BN/2 gate rows followed by the BN/2 matching
// up rows, and every wave holds the gate and up accumulators of the same
// columns, so SiLU(g)*u is formed in registers and H is stored once in bf16.
// A rows of gate/up are gathered from x through row_token (-1 = padding row,
// read as zeros).  Both operands are K-contiguous; one 16-byte load per lane
// feeds one MFMA operand.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kBK = 64;
constexpr int kLds = kBK + 8;  // padded LDS row (bf16): 144 B keeps 16-lane b128 reads conflict-free

template <bool GATE_UP, int BM, int BN>
__device__ __forceinline__ void grouped_gemm_tile(const GroupedGemm& p) {
  constexpr int WM = BM / 2;            // rows per wave
  constexpr int MT = WM / 32;           // 32-row MFMA tiles per wave
  constexpr int NT = BN / 64;           // 32-col MFMA tiles per wave (gate/up: half gate, half up)
  constexpr int A_CH = BM * (kBK / 8) / 256;  // 16-byte chunks per thread
  constexpr int B_CH = BN * (kBK / 8) / 256;
  static_assert(MT >= 1 && NT >= 1 && A_CH >= 1 && B_CH >= 1, "tile too small");
  static_assert(!GATE_UP || NT % 2 == 0, "gate/up needs paired tiles");

  __shared__ __attribute__((aligned(16))) bf16_t sA[BM * kLds];
  __shared__ __attribute__((aligned(16))) bf16_t sB[BN * kLds];

  const int64_t bid = blockIdx.x;
  const int64_t m_tile = bid % p.max_tiles;
  const int64_t n_tile = bid / p.max_tiles;
  if (m_tile >= p.n_tiles[0]) return;
  const int g = p.tile_group[m_tile];
  const bool shared = g >= p.E;
  const int N = shared ? p.N_shared : p.N_routed;
  const int K = shared ? p.K_shared : p.K_routed;
  constexpr int NB = GATE_UP ? BN / 2 : BN;  // output columns per tile
  const int n0 = (int)n_tile * NB;
  if (n0 >= N) return;
  const bf16_t* Bg = shared ? p.B_shared
                            : p.B_routed + (int64_t)g * (GATE_UP ? 2 : 1) * (int64_t)N * K;
  const int64_t row0 = m_tile * BM;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global source of every 16-byte chunk this thread stages
  const bf16_t* a_src[A_CH];
  bool a_ok[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
    if (GATE_UP) {
      const int t = p.row_token[row0 + r];
      a_ok[i] = t >= 0;
      a_src[i] = p.A + (int64_t)(t >= 0 ? t : 0) * p.lda + kc;
    } else {
      a_ok[i] = true;
      a_src[i] = p.A + (row0 + r) * p.lda + kc;
    }
  }
  const bf16_t* b_src[B_CH];
  bool b_ok[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * 256, r = c >> 3, kc = (c & 7) * 8;
    int brow;
    if (GATE_UP) {
      const int half = r / (BN / 2), f = n0 + r % (BN / 2);
      b_ok[i] = f < N;
      brow = half * N + (f < N ? f : 0);
    } else {
      const int n = n0 + r;
      b_ok[i] = n < N;
      brow = n < N ? n : 0;
    }
    b_src[i] = Bg + (int64_t)brow * K + kc;
  }

  u32x4 ra[A_CH], rb[B_CH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int kk = k0 + ((tid + i * 256) & 7) * 8;
      ra[i] = (a_ok[i] && kk < K) ? ld16(a_src[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int kk = k0 + ((tid + i * 256) & 7) * 8;
      rb[i] = (b_ok[i] && kk < K) ? ld16(b_src[i] + k0) : u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS row of this wave's j-th B tile
  auto b_row = [&](int j) {
    if (GATE_UP) {
      constexpr int H = NT / 2;
      return (j < H) ? wn * (BN / 4) + j * 32 : BN / 2 + wn * (BN / 4) + (j - H) * 32;
    }
    return wn * (BN / 2) + j * 32;
  };

  gload(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * 256;
      st16(&sA[(c >> 3) * kLds + (c & 7) * 8], ra[i]);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * 256;
      st16(&sB[(c >> 3) * kLds + (c & 7) * 8], rb[i]);
    }
    __syncthreads();
    if (k0 + kBK < K) gload(k0 + kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int kofs = ks * 16 + (lane >> 5) * 8;
      bf16x8 af[MT], bfr[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        af[i] = as_bf16x8(ld16(&sA[(wm * WM + i * 32 + (lane & 31)) * kLds + kofs]));
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bfr[j] = as_bf16x8(ld16(&sB[(b_row(j) + (lane & 31)) * kLds + kofs]));
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  }

  // ---- epilogue
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int64_t grow = row0 + row;
      if (GATE_UP) {
        bf16_t* H = reinterpret_cast<bf16_t*>(p.C);
#pragma unroll
        for (int j = 0; j < NT / 2; ++j) {
          const int f = n0 + wn * (BN / 4) + j * 32 + (lane & 31);
          if (f < N) {
            const float gv = acc[i][j][r], uv = acc[i][j + NT / 2][r];
            H[grow * p.ldc + f] = f32_to_bf16(silu(gv) * uv);
          }
        }
      } else {
        float* Y = reinterpret_cast<float*>(p.C);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int n = n0 + wn * (BN / 2) + j * 32 + (lane & 31);
          if (n < N) Y[grow * p.ldc + n] = acc[i][j][r];
        }
      }
    }
  }
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void moe_gemm_gate_up_kernel(GroupedGemm p) {
  grouped_gemm_tile<true, BM, BN>(p);
}

template <int BM, int BN>
__global__ __launch_bounds__(256) void moe_gemm_down_kernel(GroupedGemm p) {
  grouped_gemm_tile<false, BM, BN>(p);
}

template <bool GATE_UP, int BM, int BN>
hipError_t launch_tiles(const GroupedGemm& g, hipStream_t s) {
  const int nmax = GATE_UP ? (g.N_routed > g.N_shared ? g.N_routed : g.N_shared)
                           : (g.N_routed > g.N_shared ? g.N_routed : g.N_shared);
  constexpr int NB = GATE_UP ? BN / 2 : BN;
  const int64_t n_tiles_n = (nmax + NB - 1) / NB;
  const int64_t blocks = g.max_tiles * n_tiles_n;
  if (blocks == 0) return hipSuccess;
  if (GATE_UP)
    hipLaunchKernelGGL((moe_gemm_gate_up_kernel<BM, BN>), dim3((unsigned)blocks), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((moe_gemm_down_kernel<BM, BN>), dim3((unsigned)blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gate_up(const GroupedGemm& g, hipStream_t s) {
  if (g.BM != 128) return hipErrorInvalidValue;
  return launch_tiles<true, 128, 128>(g, s);
}

hipError_t launch_gemm_down(const GroupedGemm& g, hipStream_t s) {
  if (g.BM != 128) return hipErrorInvalidValue;
  return launch_tiles<false, 128, 128>(g, s);
}

}  // namespace moe
