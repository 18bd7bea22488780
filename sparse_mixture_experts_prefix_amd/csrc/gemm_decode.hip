// Decode-sized grouped GEMMs (a few rows per expert): weight streaming.
//
// Same operation as the prefill kernels (SwiGLU expert FFN of the glossary
// "MoE (Mixture of Experts - Mezcla de Expertos)", section 3 step 3; packed
// [E, 2F, D] gate/up tensor of "Transformers v5 El Secreto Detrás de los
// Modelos MoE Más Rápidos", section "La Solución: WeightConverter").  With
// 16-32 rows per expert every weight byte feeds only 16-32 MACs, so the time
// is the time to stream the touched experts' weights from HBM (the pages'
// "decode time follows active bytes over bandwidth", "Mixture of Experts
// optimiza Transformers y LLMs", section "¿Por qué MoEs importan ...").
//  - A workgroup owns one m-tile (16*MT rows of one expert) and 16*NG weight
//    rows (gate/up: NG/2 groups of gate rows with the matching up rows);
//    its 4 waves split K and their partial sums are added in LDS in a fixed
//    order (deterministic).  All loads of a trip are issued before its
//    MFMAs (a scheduling barrier), so each wave keeps two chunks in flight.
//  - MFMA 16x16x32 bf16.  The K order inside a 64-wide chunk is permuted the
//    same way for A and B: lane (col c, group g) holds bytes [32g, 32g+32) of
//    its row for two consecutive MFMAs, so the four lanes of a row read one
//    full 128-byte line.  Weights go straight from HBM to registers (each
//    byte is used once); loads of two chunks are in flight per wave.
//  - Out-of-range buffer offsets read as zero: padding rows, rows past the
//    group's count and K tails need no branches.  Weight rows of tiles that
//    lie wholly in bounds are read with plain global loads instead (faster).
//  - E4M3 weights (one fp32 scale per weight row): a lane's 16 weights of a
//    chunk are one 16-byte load, widened to bf16 exactly in registers
//    (v_cvt_scalef32_pk_bf16_fp8 with scale 1; every E4M3 value is a bf16
//    value), and each output column's sum is multiplied by its row's scale
//    after the reduction: sum_k x_k (q_k s) = s sum_k x_k q_k.  Half the
//    weight bytes of bf16, for the same MFMAs.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0));
}

// Eight E4M3 codes (bytes 0..7 of two dwords, element i in byte i) widened to bf16.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <bool GATE_UP, int MT, int NG, int kWaves, int kUnroll, bool FP8>
__device__ __forceinline__ void decode_tile(const GroupedGemm& p) {
  constexpr int BMD = 16 * MT;
  constexpr int NOUT = GATE_UP ? NG / 2 * 16 : NG * 16;  // output columns per tile
  __shared__ f32x4 red[kWaves > 1 ? kWaves - 1 : 1][MT][NG][64];

  const int64_t bid = blockIdx.x;
  const int64_t n_tile = bid % p.n_tiles_n;
  const int64_t m_tile = bid / p.n_tiles_n;
  if (m_tile >= p.n_tiles[0]) return;
  const int g = p.tile_group[m_tile];
  const bool shared = g >= p.E;
  const int N = shared ? p.N_shared : p.N_routed;
  const int K = shared ? p.K_shared : p.K_routed;
  const int n0 = (int)n_tile * NOUT;
  if (n0 >= N) return;
  const int64_t row0 = m_tile * BMD;
  const int valid_rows = min(BMD, (int)(p.group_count[g] - (row0 - p.group_padded[g])));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, gq = lane >> 4;  // row/column within 16, 32-byte quarter of a line

  // ---- operand row offsets (bytes, chunk 0)
  const __amdgpu_buffer_rsrc_t rsA =
      GATE_UP ? make_rsrc(p.A, (uint32_t)p.a_bytes)
              : make_rsrc(p.A + row0 * p.lda, (uint32_t)(BMD * p.lda * 2));
  // weight bytes per element, and the lane's bytes within a 64-wide K chunk
  constexpr int EB = FP8 ? 1 : 2;
  const int64_t brows = (int64_t)(GATE_UP ? 2 : 1) * N;  // weight rows of this group
  const char* Bbytes = shared ? static_cast<const char*>(p.B_shared)
                              : static_cast<const char*>(p.B_routed) + (int64_t)g * brows * K * EB;
  const float* Sg = !FP8 ? nullptr : shared ? p.S_shared : p.S_routed + (int64_t)g * brows;
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(Bbytes, (uint32_t)(brows * K * EB));
  uint32_t offA[MT], offB[NG];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int r = i * 16 + c;
    if (GATE_UP) {
      const int t = r < valid_rows ? p.row_token[row0 + r] : -1;
      offA[i] = t >= 0 ? (uint32_t)t * (uint32_t)(p.lda * 2) + gq * 32 : kOob;
    } else {
      offA[i] = r < valid_rows ? (uint32_t)r * (uint32_t)(p.lda * 2) + gq * 32 : kOob;
    }
  }
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    int brow;
    bool ok;
    if (GATE_UP) {
      const int half = j / (NG / 2), f = n0 + (j % (NG / 2)) * 16 + c;
      ok = f < N;
      brow = half * N + f;
    } else {
      const int n = n0 + j * 16 + c;
      ok = n < N;
      brow = n;
    }
    offB[j] = ok ? (uint32_t)brow * (uint32_t)(K * EB) + gq * 16 * EB : kOob;
  }

  f32x4 acc[MT][NG];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- K loop: 64-wide chunks q = wave, wave + kWaves, ...; kUnroll chunks per trip.
  // A tile whose weight rows and K range are all in bounds (the usual case)
  // reads the weights with plain global loads, which stream faster than
  // bounds-checked buffer loads; a ragged tile uses the buffer loads, whose
  // out-of-range offsets read as zero.
  const int nq = (K + 63) / 64;
  constexpr int BV = FP8 ? 1 : 2;  // 16-byte registers per weight row and chunk
  auto run = [&](auto exact_tag) {
    constexpr bool kExact = decltype(exact_tag)::value;
    auto load_chunk = [&](int q, u32x4 (&a)[MT][2], u32x4 (&b)[NG][BV]) {
      const int k0 = q * 64;
      // K tail (K % 64 != 0): a lane's 32 bytes are all in or all out when K % 16 == 0;
      // otherwise its two 16-byte halves are checked separately
      const int kk = k0 + gq * 16;
      const bool in0 = kk < K, in1 = kk + 8 < K;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        a[i][0] = bload(rsA, in0 ? offA[i] : kOob, k0 * 2);
        a[i][1] = bload(rsA, in1 ? offA[i] + 16 : kOob, k0 * 2);
      }
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        if constexpr (FP8) {
          if constexpr (kExact) {
            b[j][0] = *reinterpret_cast<const u32x4*>(Bbytes + offB[j] + k0);
          } else {  // each 8-byte half checked against K like A's halves
            const u32x2 lo = bload8(rsB, in0 ? offB[j] : kOob, k0);
            const u32x2 hi = bload8(rsB, in1 ? offB[j] + 8 : kOob, k0);
            b[j][0] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
        } else if constexpr (kExact) {
          const char* pb = Bbytes + offB[j] + k0 * 2;
          b[j][0] = *reinterpret_cast<const u32x4*>(pb);
          b[j][1] = *reinterpret_cast<const u32x4*>(pb + 16);
        } else {
          b[j][0] = bload(rsB, in0 ? offB[j] : kOob, k0 * 2);
          b[j][1] = bload(rsB, in1 ? offB[j] + 16 : kOob, k0 * 2);
        }
      }
    };
    auto mma_chunk = [&](const u32x4 (&a)[MT][2], const u32x4 (&b)[NG][BV]) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          bf16x8 bv;
          if constexpr (FP8)
            bv = e4m3x8_to_bf16(b[j][0][2 * h], b[j][0][2 * h + 1]);
          else
            bv = as_bf16x8(b[j][h]);
#pragma unroll
          for (int i = 0; i < MT; ++i) acc[i][j] = mfma16(as_bf16x8(a[i][h]), bv, acc[i][j]);
        }
    };
    int q = wave;
    for (; q + (kUnroll - 1) * kWaves < nq; q += kUnroll * kWaves) {
      u32x4 a[kUnroll][MT][2], b[kUnroll][NG][BV];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load_chunk(q + u * kWaves, a[u], b[u]);
      // every load of the trip goes out before the first MFMA; left alone,
      // the compiler sinks loads to their uses and keeps only ~6 in flight
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) mma_chunk(a[u], b[u]);
    }
    for (; q < nq; q += kWaves) {
      u32x4 a0[MT][2], b0[NG][BV];
      load_chunk(q, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma_chunk(a0, b0);
    }
  };
  if (K % 64 == 0 && n0 + NOUT <= N)
    run(std::true_type{});
  else
    run(std::false_type{});

  // ---- fixed-order reduction over the waves: (((w0 + w1) + w2) + ...)
  if (kWaves > 1) {
    if (wave > 0) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j) red[wave - 1][i][j][lane] = acc[i][j];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w)
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j) acc[i][j] += red[w][i][j][lane];
  }

  // ---- per-row weight scales (E4M3 weights): column c of group j is weight row
  // half * N + f (gate/up) or n (down)
  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      int brow;
      bool ok;
      if (GATE_UP) {
        const int half = j / (NG / 2), f = n0 + (j % (NG / 2)) * 16 + c;
        ok = f < N;
        brow = half * N + f;
      } else {
        brow = n0 + j * 16 + c;
        ok = brow < N;
      }
      const float sc = ok ? Sg[brow] : 0.f;
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i][j] *= sc;
    }
  }

  // ---- epilogue: lane (c, gq) holds rows 4*gq + r, column c of each 16x16 tile
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t grow = row0 + i * 16 + 4 * gq + r;
      if (GATE_UP) {
        bf16_t* H = reinterpret_cast<bf16_t*>(p.C);
#pragma unroll
        for (int j = 0; j < NG / 2; ++j) {
          const int f = n0 + j * 16 + c;
          if (f < N) H[grow * p.ldc + f] = f32_to_bf16(silu(acc[i][j][r]) * acc[i][j + NG / 2][r]);
        }
      } else {
        float* Y = reinterpret_cast<float*>(p.C);
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          const int n = n0 + j * 16 + c;
          if (n < N) Y[grow * p.ldc + n] = acc[i][j][r];
        }
      }
    }
  }
}

// 16-row column groups per tile (gate/up: half gate, half up), waves splitting
// K, and 64-wide K-chunks whose loads are in flight together per wave.
// Measured on the gpt-oss-shaped decode layer: 32-64 output columns, 4 waves.
constexpr int kNgGateUp = 4, kNgDown = 4, kKw = 4, kUnr = 2;

template <int MT, bool FP8>
__global__ __launch_bounds__(kKw * 64) void moe_gemm_gate_up_decode_kernel(GroupedGemm p) {
  decode_tile<true, MT, kNgGateUp, kKw, kUnr, FP8>(p);
}

template <int MT, bool FP8>
__global__ __launch_bounds__(kKw * 64) void moe_gemm_down_decode_kernel(GroupedGemm p) {
  decode_tile<false, MT, kNgDown, kKw, kUnr, FP8>(p);
}

template <int MT, bool FP8>
hipError_t launch_mt(bool gate_up, GroupedGemm g, hipStream_t s) {
  const int nmax = g.N_routed > g.N_shared ? g.N_routed : g.N_shared;
  const int nout = gate_up ? kNgGateUp / 2 * 16 : kNgDown * 16;
  g.n_tiles_n = (nmax + nout - 1) / nout;
  const int64_t blocks = g.max_tiles * g.n_tiles_n;
  if (blocks == 0) return hipSuccess;
  if (gate_up)
    hipLaunchKernelGGL((moe_gemm_gate_up_decode_kernel<MT, FP8>), dim3((unsigned)blocks),
                       dim3(kKw * 64), 0, s, g);
  else
    hipLaunchKernelGGL((moe_gemm_down_decode_kernel<MT, FP8>), dim3((unsigned)blocks),
                       dim3(kKw * 64), 0, s, g);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_fmt(bool gate_up, const GroupedGemm& g, hipStream_t s) {
  return g.fp8 ? launch_mt<MT, true>(gate_up, g, s) : launch_mt<MT, false>(gate_up, g, s);
}

}  // namespace

hipError_t launch_gemm_gate_up_decode(const GroupedGemm& g, hipStream_t s) {
  if (g.BM == 16) return launch_fmt<1>(true, g, s);
  if (g.BM == 32) return launch_fmt<2>(true, g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_down_decode(const GroupedGemm& g, hipStream_t s) {
  if (g.BM == 16) return launch_fmt<1>(false, g, s);
  if (g.BM == 32) return launch_fmt<2>(false, g, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
