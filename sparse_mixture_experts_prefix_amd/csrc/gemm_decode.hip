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
//  - MFMA 16x16x32 bf16.  The K order inside a chunk is permuted the same
//    way for A and B: lane (col c, group g) holds 128 / 4 bytes of weights of
//    its row (16 bf16 or 32 E4M3 values) for two or four consecutive MFMAs,
//    so the four lanes of a row read one full 128-byte line.  Weights go
//    straight from HBM to registers (each byte is used once); the loads of
//    several chunks are in flight per wave.
//  - Out-of-range buffer offsets read as zero: padding rows, rows past the
//    group's count and K tails need no branches.  Weight rows of tiles that
//    lie wholly in bounds are read with plain global loads instead (faster).
//  - E4M3 weights (one fp32 scale per weight row): a lane's 32 weights of a
//    chunk are two 16-byte loads, widened to bf16 exactly in registers
//    (v_cvt_scalef32_pk_bf16_fp8 with scale 1; every E4M3 value is a bf16
//    value), and each output column's sum is multiplied by its row's scale
//    after the reduction: sum_k x_k (q_k s) = s sum_k x_k q_k.  Half the
//    weight bytes of bf16, for the same MFMAs.
//  - bf16 weights with the wide column tiles, and the backward pass's
//    products with the weights as stored (contracting over their row index),
//    stage the weights through LDS instead; see the staged tile below.
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

// Epilogue of a decode tile: lane (c, gq) holds rows 4 gq + r, column c of
// each 16x16 tile.  Gate/up: column groups j < NG/2 are gate, j + NG/2 the
// matching up columns; H = bf16(SiLU(g) u), and g | u of the valid rows when
// kept for the backward pass.  Down: fp32 rows.
template <bool GATE_UP, int MT, int NG>
__device__ __forceinline__ void store_tile(const GroupedGemm& p, const f32x4 (&acc)[MT][NG], int64_t row0,
                                           int n0, int N, int valid_rows, int c, int gq) {
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
        if (p.gu_out && i * 16 + 4 * gq + r < valid_rows) {  // g and u kept for the backward pass
          bf16_t* gr = reinterpret_cast<bf16_t*>(p.gu_out) + grow * p.ld_gu;
#pragma unroll
          for (int j = 0; j < NG / 2; ++j) {
            const int f = n0 + j * 16 + c;
            if (f < N) {
              gr[f] = f32_to_bf16(acc[i][j][r]);
              gr[N + f] = f32_to_bf16(acc[i][j + NG / 2][r]);
            }
          }
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
  // elements of K per lane and chunk (a chunk is CW = 4 * KE), MFMA steps per chunk
  constexpr int KE = FP8 ? 32 : 16, CW = 4 * KE, NH = KE / 8;
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
      offA[i] = t >= 0 ? (uint32_t)t * (uint32_t)(p.lda * 2) + gq * KE * 2 : kOob;
    } else {
      offA[i] = r < valid_rows ? (uint32_t)r * (uint32_t)(p.lda * 2) + gq * KE * 2 : kOob;
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
    offB[j] = ok ? (uint32_t)brow * (uint32_t)(K * EB) + gq * KE * EB : kOob;
  }

  f32x4 acc[MT][NG];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- K loop: chunks q = wave, wave + kWaves, ...; kUnroll chunks per trip.
  // A chunk is CW = 4 * KE elements of K: lane (c, gq) takes elements
  // [KE*gq, KE*gq + KE) of it, 8 per MFMA step, so the four lanes of a row
  // read 128 contiguous weight bytes (a full line) either way: KE = 16 bf16
  // or KE = 32 E4M3 weights.
  // Whole chunks of a tile whose weight rows are all in bounds (the usual
  // case) read the weights with plain global loads, which stream faster than
  // bounds-checked buffer loads; the ragged last chunk of K and tiles past
  // the last weight row use the buffer loads, whose out-of-range offsets read
  // as zero.  Each wave still takes its chunks in ascending order.
  constexpr int BV = 2;  // 16-byte weight registers per row and chunk
  const int nfull = K / CW, nq = (K + CW - 1) / CW;
  // chunks q_begin <= q < q_end of this wave
  auto run = [&](auto exact_tag, int q_begin, int q_end) {
    constexpr bool kExact = decltype(exact_tag)::value;
    auto load_chunk = [&](int q, u32x4 (&a)[MT][NH], u32x4 (&b)[NG][BV]) {
      const int k0 = q * CW;
      // K tail (K % CW != 0): each 8-element group of a lane is checked on its own
      bool in[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h) in[h] = k0 + gq * KE + 8 * h < K;
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int h = 0; h < NH; ++h) a[i][h] = bload(rsA, in[h] ? offA[i] + 16 * h : kOob, k0 * 2);
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        if constexpr (kExact) {
          const char* pb = Bbytes + offB[j] + k0 * EB;
          b[j][0] = *reinterpret_cast<const u32x4*>(pb);
          b[j][1] = *reinterpret_cast<const u32x4*>(pb + 16);
        } else if constexpr (FP8) {  // 8-byte pieces, checked like A's groups
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const u32x2 lo = bload8(rsB, in[2 * v] ? offB[j] + 16 * v : kOob, k0);
            const u32x2 hi = bload8(rsB, in[2 * v + 1] ? offB[j] + 16 * v + 8 : kOob, k0);
            b[j][v] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
        } else {
          b[j][0] = bload(rsB, in[0] ? offB[j] : kOob, k0 * 2);
          b[j][1] = bload(rsB, in[1] ? offB[j] + 16 : kOob, k0 * 2);
        }
      }
    };
    auto mma_chunk = [&](const u32x4 (&a)[MT][NH], const u32x4 (&b)[NG][BV]) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          bf16x8 bv;
          if constexpr (FP8)
            bv = e4m3x8_to_bf16(b[j][h / 2][2 * (h % 2)], b[j][h / 2][2 * (h % 2) + 1]);
          else
            bv = as_bf16x8(b[j][h]);
#pragma unroll
          for (int i = 0; i < MT; ++i) acc[i][j] = mfma16(as_bf16x8(a[i][h]), bv, acc[i][j]);
        }
    };
    int q = q_begin + (wave - q_begin % kWaves + kWaves) % kWaves;
    for (; q + (kUnroll - 1) * kWaves < q_end; q += kUnroll * kWaves) {
      u32x4 a[kUnroll][MT][NH], b[kUnroll][NG][BV];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load_chunk(q + u * kWaves, a[u], b[u]);
      // every load of the trip goes out before the first MFMA; left alone,
      // the compiler sinks loads to their uses and keeps only ~6 in flight
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) mma_chunk(a[u], b[u]);
    }
    for (; q < q_end; q += kWaves) {
      u32x4 a0[MT][NH], b0[NG][BV];
      load_chunk(q, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma_chunk(a0, b0);
    }
  };
  if (n0 + NOUT <= N) {
    run(std::true_type{}, 0, nfull);
    if (nq > nfull) run(std::false_type{}, nfull, nq);
  } else {
    run(std::false_type{}, 0, nq);
  }

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

  store_tile<GATE_UP, MT, NG>(p, acc, row0, n0, N, valid_rows, c, gq);
}

// 16-row column groups per tile (gate/up: half gate, half up), waves splitting
// K, and 64-wide K-chunks whose loads are in flight together per wave.
// Measured on the gpt-oss-shaped decode layer: 32-64 output columns, 4 waves.
constexpr int kNgGateUp = 4, kNgDown = 4, kKw = 4, kUnr = 2;
// E4M3 weights: a chunk is half the bytes, so more chunks go out per trip
constexpr int kNgGateUpFp8 = 4, kNgDownFp8 = 4, kUnrFp8 = 4;

// Few occupied row tiles (a handful of tokens): narrow column tiles (2 and 1
// column groups) so the grid still fills the chip; measured on the gpt-oss
// shape at T = 1: layer 59 -> 53 us.  Narrow is chosen when the wide tiles
// would give fewer than kFillBlocks workgroups (two per CU of the MI355X).
constexpr int kNgGateUpNarrow = 2, kNgDownNarrow = 1;
constexpr int64_t kFillBlocks = 512;

template <bool FP8, bool NARROW> constexpr int ng_gate_up() {
  return NARROW ? kNgGateUpNarrow : FP8 ? kNgGateUpFp8 : kNgGateUp;
}
template <bool FP8, bool NARROW> constexpr int ng_down() {
  return NARROW ? kNgDownNarrow : FP8 ? kNgDownFp8 : kNgDown;
}
template <bool FP8> constexpr int unroll() { return FP8 ? kUnrFp8 : kUnr; }

// ------------------------------------------------------- weights through LDS
// The backward pass's row products with W_down and W_gate_up as they are
// stored: C[r][n] = sum_k A[r][k] B[k][n], B being the group's [K][N] slab
// (k-row k holds the N weights that multiply column k of A).  An MFMA operand
// takes eight consecutive k of one column per lane, so each wave stages 64
// k-rows x 64 columns of B, with its 16 MT rows x 64 k of A, through LDS
// (16-byte LDS-direct loads) and reads B back with the transposing read.
// A wave owns a ring of stages, so the K loop has no workgroup barrier:
// the later chunks stream in while one is multiplied.  The waves
// split K by chunks as above, and their sums are added in the same order.
// The forward's bf16 products (row-major weights) use the same staging; see
// decode_tile_staged.
constexpr int kKmBBytes = 64 * 128;  // a stage's B: 64 k-rows x 64 columns, bf16
template <int MT> constexpr int km_a_bytes() { return 16 * MT * 128; }
// NG column groups of 16 weight rows (row-major weights; K-major stages are
// always 64 columns): a stage's B is NG * 2 KB
template <int MT, int NG = 4> constexpr int km_stage_bytes() { return km_a_bytes<MT>() + NG * 2048; }
// stages per wave: 16-row tiles take two, so two workgroups share a CU (80 KB
// each) and one's start and end overlap the other's streaming; 32-row tiles
// take three (144 KB, one workgroup per CU)
template <int MT> constexpr int km_stages() { return MT == 1 ? 2 : 3; }
template <int MT, int NG = 4> constexpr int km_lds_bytes() {
  return kKw * km_stages<MT>() * km_stage_bytes<MT, NG>();
}

// 16-byte chunk c (columns 8c .. 8c + 7) of k-row r of a B stage sits at
// chunk position c ^ km_b_swz(r) of the row's 128 bytes.  A 32-lane half of a
// transposing read covers k-rows R .. R + 3 and R + 8 .. R + 11 (R a multiple
// of 4 with bit 3 clear), two chunks each: row parity picks the 128-byte half
// of the 64 banks and the swizzle spreads the four rows of each parity over
// distinct chunk pairs, so every bank is hit once.  Row r of an A stage keeps
// chunk c (k 8c .. 8c + 7) at c ^ ((r >> 1) & 7): 16 rows' same chunk land in
// 16 distinct 16-byte bank groups.
__device__ __forceinline__ int km_b_swz(int r) { return 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1); }
__device__ __forceinline__ int km_a_swz(int r) { return (r >> 1) & 7; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// KMAJ = false: the forward's products with row-major weights ([N][K] per
// group; gate/up: 8 NG gate rows and the matching 8 NG up rows), staged the
// same way: a stage's B is 16 NG weight rows x 64 k, laid out like A, read
// with plain 16-byte LDS reads.  NG = 4 (64 weight rows) for most shapes; 2
// (gate/up) and 1 (down) when a handful of tokens occupy few row tiles, so
// the grid still fills the chip.
template <int MT, bool KMAJ, bool GATE_UP, int NG = 4>
__device__ __forceinline__ void decode_tile_staged(const GroupedGemm& p, char* lds) {
  static_assert(!(KMAJ && GATE_UP), "K-major weights: rows x weight products only");
  static_assert(!KMAJ || NG == 4, "K-major stages hold 64 columns");
  static_assert(!GATE_UP || NG % 2 == 0, "gate/up tiles pair gate and up groups");
  constexpr int BMD = 16 * MT, NOUT = GATE_UP ? 16 * NG / 2 : 16 * NG;
  constexpr int SB = km_stage_bytes<MT, NG>(), AB = km_a_bytes<MT>(), S = km_stages<MT>();
  constexpr int NA = AB / 1024, NB = NG * 2, V = NA + NB;  // 1-KB loads per chunk
  constexpr int HR = 8 * NG;  // gate/up: weight rows of each half of the tile

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
  const int c = lane & 15, gq = lane >> 4;

  const __amdgpu_buffer_rsrc_t rsA = GATE_UP ? make_rsrc(p.A, (uint32_t)p.a_bytes)
                                             : make_rsrc(p.A + row0 * p.lda, (uint32_t)(BMD * p.lda * 2));
  const int64_t slab = (int64_t)(GATE_UP ? 2 : 1) * K * N * 2;  // the group's weight bytes
  const char* Bbytes = shared ? static_cast<const char*>(p.B_shared)
                              : static_cast<const char*>(p.B_routed) + (int64_t)g * slab;
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(Bbytes, (uint32_t)slab);
  // LDS-direct load b of a stage: lane i writes 16 bytes at 16 i of its 1-KB
  // block, i.e. row (A) or k-row (B) 8 b + i / 8, chunk position i % 8.
  // Offsets at k = 0; out-of-range ones (rows past the group, columns past N)
  // stay out of range when k0's bytes are added.
  const int ir = lane >> 3, ip = lane & 7;
  uint32_t aoff[NA], boff[NB];
  int akc[NA], bkc[NB];  // first k of the chunk, inside the 64-wide K chunk (row-major operands)
#pragma unroll
  for (int b = 0; b < NA; ++b) {
    const int r = 8 * b + ir, ch = ip ^ km_a_swz(r);
    akc[b] = 8 * ch;
    if (GATE_UP) {  // gathered x rows
      const int t = r < valid_rows ? p.row_token[row0 + r] : -1;
      aoff[b] = t >= 0 ? (uint32_t)t * (uint32_t)(p.lda * 2) + ch * 16 : kOob;
    } else {
      aoff[b] = r < valid_rows ? (uint32_t)r * (uint32_t)(p.lda * 2) + ch * 16 : kOob;
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int r = 8 * b + ir;
    if (KMAJ) {
      const int n = n0 + 8 * (ip ^ km_b_swz(r));
      bkc[b] = 0;
      boff[b] = n < N ? (uint32_t)r * (uint32_t)(N * 2) + n * 2 : kOob;
    } else {  // weight row r of the tile: gate/up rows 0 .. HR - 1 gate, HR .. 2 HR - 1 up
      const int ch = ip ^ km_a_swz(r);
      const int f = GATE_UP ? n0 + r % HR : n0 + r;
      const int brow = GATE_UP ? (r / HR) * N + f : f;
      bkc[b] = 8 * ch;
      boff[b] = f < N ? (uint32_t)brow * (uint32_t)(K * 2) + ch * 16 : kOob;
    }
  }
  // Reads.  MFMA step h of a chunk takes k = 32 h + 8 gq + (0 .. 7) in lane
  // (c, gq).  A: row 16 i + c, chunk 4 h + gq.  B: a transposing read gives
  // lane i of each 16-lane group element i % 4 of the words of group lanes
  // i / 4, + 4, + 8, + 12, so lane c points at k-row 8 gq + c / 4 (+ 4 for the
  // upper four k, + 32 h) and columns 16 j + 4 (c % 4) .. + 3: lane c then gets
  // column 16 j + c at four consecutive k.  The swizzle of those k-rows does
  // not depend on h or the + 4.
  int rdA[MT][2], rdB[NG];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 16 * i + c;
      rdA[i][h] = r * 128 + 16 * ((4 * h + gq) ^ km_a_swz(r));
    }
  {
    const int rb = 8 * gq + (c >> 2);
#pragma unroll
    for (int j = 0; j < NG; ++j)
      rdB[j] = AB + rb * 128 + 16 * ((2 * j + ((c & 3) >> 1)) ^ km_b_swz(rb)) + 8 * (c & 1);
  }

  f32x4 acc[MT][NG];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NG; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's chunks: q = wave + kKw m, m = 0 .. nm - 1
  const int nq = (K + 63) / 64;
  const int nm = wave < nq ? (nq - 1 - wave) / kKw + 1 : 0;
  char* ring = lds + wave * (S * SB);
  auto issue = [&](int m, int slot) {
    const int k0 = (wave + kKw * m) * 64;
    char* st = ring + slot * SB;
#pragma unroll
    for (int b = 0; b < NA; ++b)
      lds_dma16(rsA, st + b * 1024, k0 + akc[b] < K ? aoff[b] + 2 * k0 : kOob, 0);
    // the weights are read once per call: non-temporal loads
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (KMAJ)
        lds_dma16<true>(rsB, st + AB + b * 1024,
                        k0 + 8 * b + ir < K ? boff[b] + (uint32_t)k0 * (uint32_t)(N * 2) : kOob, 0);
      else
        lds_dma16<true>(rsB, st + AB + b * 1024, k0 + bkc[b] < K ? boff[b] + 2 * k0 : kOob, 0);
    }
  };
  auto read_tr = [](const char* q) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_v4;
    typedef __attribute__((address_space(3))) char lds_char;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)((lds_char*)q));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)((lds_char*)(q + 4 * 128)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // all S stages start filling; chunk m + S refills chunk m's stage once its
  // MFMAs have taken their operands
#pragma unroll
  for (int m = 0; m < S; ++m)
    if (m < nm) issue(m, m);
  int slot = 0;
  for (int m = 0; m < nm; ++m) {
    // chunk m has landed once at most the loads of the later chunks issued so
    // far (min(nm - 1 - m, S - 1) chunks) are in flight
    const int later = min(nm - 1 - m, S - 1);
    if (S > 2 && later >= 2)
      wait_vmcnt<(S > 2 ? 2 : 1) * V>();
    else if (later >= 1)
      wait_vmcnt<V>();
    else
      wait_vmcnt<0>();
    const char* st = ring + slot * SB;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 a[MT], b[NG];
#pragma unroll
      for (int i = 0; i < MT; ++i) a[i] = *reinterpret_cast<const bf16x8*>(st + rdA[i][h]);
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        if (KMAJ) {
          b[j] = read_tr(st + rdB[j] + h * 32 * 128);
        } else {  // weight row 16 j + c, chunk 4 h + gq
          const int r = 16 * j + c;
          b[j] = *reinterpret_cast<const bf16x8*>(st + AB + r * 128 + 16 * ((4 * h + gq) ^ km_a_swz(r)));
        }
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NG; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
    if (m + S < nm) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this stage's reads are done
      issue(m + S, slot);
    }
    slot = slot == S - 1 ? 0 : slot + 1;
  }

  // ---- fixed-order sum over the waves, (((w0 + w1) + w2) + w3), in the
  // stage memory (every wave's loads have landed: its last wait was vmcnt(0))
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // [kKw - 1][MT][NG][64]
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NG; ++j) red[(((wave - 1) * MT + i) * NG + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kKw - 1; ++w)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NG; ++j) acc[i][j] += red[((w * MT + i) * NG + j) * 64 + lane];

  store_tile<GATE_UP, MT, NG>(p, acc, row0, n0, N, valid_rows, c, gq);
}

template <int MT, bool FP8, bool NARROW>
__global__ __launch_bounds__(kKw * 64) void moe_gemm_gate_up_decode_kernel(GroupedGemm p) {
  decode_tile<true, MT, ng_gate_up<FP8, NARROW>(), kKw, unroll<FP8>(), FP8>(p);
}

template <int MT, bool FP8, bool NARROW>
__global__ __launch_bounds__(kKw * 64) void moe_gemm_down_decode_kernel(GroupedGemm p) {
  decode_tile<false, MT, ng_down<FP8, NARROW>(), kKw, unroll<FP8>(), FP8>(p);
}

template <bool FP8, bool NARROW>
int column_tile(bool gate_up) {
  return gate_up ? ng_gate_up<FP8, NARROW>() / 2 * 16 : ng_down<FP8, NARROW>() * 16;
}

template <int MT, bool FP8, bool NARROW>
hipError_t launch_mt(bool gate_up, GroupedGemm g, hipStream_t s) {
  const int nmax = g.N_routed > g.N_shared ? g.N_routed : g.N_shared;
  const int nout = column_tile<FP8, NARROW>(gate_up);
  g.n_tiles_n = (nmax + nout - 1) / nout;
  const int64_t blocks = g.max_tiles * g.n_tiles_n;
  if (blocks == 0) return hipSuccess;
  if (gate_up)
    hipLaunchKernelGGL((moe_gemm_gate_up_decode_kernel<MT, FP8, NARROW>), dim3((unsigned)blocks),
                       dim3(kKw * 64), 0, s, g);
  else
    hipLaunchKernelGGL((moe_gemm_down_decode_kernel<MT, FP8, NARROW>), dim3((unsigned)blocks),
                       dim3(kKw * 64), 0, s, g);
  return hipGetLastError();
}

template <int MT, bool GATE_UP, int NG>
hipError_t launch_staged(const GroupedGemm& g0, hipStream_t s);

template <int MT, bool FP8>
hipError_t launch_width(bool gate_up, const GroupedGemm& g, hipStream_t s) {
  const int nmax = g.N_routed > g.N_shared ? g.N_routed : g.N_shared;
  const int nout = column_tile<FP8, false>(gate_up);
  const bool narrow = g.busy_tiles * ((nmax + nout - 1) / nout) < kFillBlocks;
  // bf16 weights stream through LDS (narrow tiles: the register path's
  // column groups), E4M3 codes into registers
  if constexpr (!FP8) {
    if (narrow)
      return gate_up ? launch_staged<MT, true, kNgGateUpNarrow>(g, s)
                     : launch_staged<MT, false, kNgDownNarrow>(g, s);
    return gate_up ? launch_staged<MT, true, 4>(g, s) : launch_staged<MT, false, 4>(g, s);
  } else {
    if (narrow) return launch_mt<MT, FP8, true>(gate_up, g, s);
    return launch_mt<MT, FP8, false>(gate_up, g, s);
  }
}

template <int MT>
__global__ __launch_bounds__(kKw * 64) void moe_gemm_rows_kmajor_decode_kernel(GroupedGemm p) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  decode_tile_staged<MT, true, false>(p, lds);
}

template <int MT, bool GATE_UP, int NG>
__global__ __launch_bounds__(kKw * 64) void moe_gemm_staged_decode_kernel(GroupedGemm p) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  decode_tile_staged<MT, false, GATE_UP, NG>(p, lds);
}

// bf16 weights: the weights stream through LDS, NG column groups per tile
template <int MT, bool GATE_UP, int NG>
hipError_t launch_staged(const GroupedGemm& g0, hipStream_t s) {
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)moe_gemm_staged_decode_kernel<MT, GATE_UP, NG>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, km_lds_bytes<MT, NG>());
  if (attr != hipSuccess) return attr;
  const int64_t brows = GATE_UP ? 2 : 1;
  if (brows * g0.K_routed * g0.N_routed * 2 >= (int64_t(1) << 31) ||
      brows * g0.K_shared * g0.N_shared * 2 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  GroupedGemm g = g0;
  const int nmax = g.N_routed > g.N_shared ? g.N_routed : g.N_shared;
  const int nout = GATE_UP ? 8 * NG : 16 * NG;
  g.n_tiles_n = (nmax + nout - 1) / nout;
  const int64_t blocks = g.max_tiles * g.n_tiles_n;
  if (blocks == 0) return hipSuccess;
  constexpr int lds = km_lds_bytes<MT, NG>();
  hipLaunchKernelGGL((moe_gemm_staged_decode_kernel<MT, GATE_UP, NG>), dim3((unsigned)blocks),
                     dim3(kKw * 64), lds, s, g);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_kmajor(const GroupedGemm& g0, hipStream_t s) {
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)moe_gemm_rows_kmajor_decode_kernel<MT>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, km_lds_bytes<MT>());
  if (attr != hipSuccess) return attr;
  // a group's slab is addressed with 32-bit offsets
  if ((int64_t)g0.K_routed * g0.N_routed * 2 >= (int64_t(1) << 31) ||
      (int64_t)g0.K_shared * g0.N_shared * 2 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  GroupedGemm g = g0;
  const int nmax = g.N_routed > g.N_shared ? g.N_routed : g.N_shared;
  g.n_tiles_n = (nmax + 63) / 64;
  const int64_t blocks = g.max_tiles * g.n_tiles_n;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((moe_gemm_rows_kmajor_decode_kernel<MT>), dim3((unsigned)blocks), dim3(kKw * 64),
                     km_lds_bytes<MT>(), s, g);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_fmt(bool gate_up, const GroupedGemm& g, hipStream_t s) {
  return g.fp8 ? launch_width<MT, true>(gate_up, g, s) : launch_width<MT, false>(gate_up, g, s);
}

}  // namespace

hipError_t launch_gemm_gate_up_decode(const GroupedGemm& g, hipStream_t s) {
  if (g.b_kmajor) return hipErrorInvalidValue;
  if (g.BM == 16) return launch_fmt<1>(true, g, s);
  if (g.BM == 32) return launch_fmt<2>(true, g, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_down_decode(const GroupedGemm& g, hipStream_t s) {
  if (g.b_kmajor) {
    if (g.fp8) return hipErrorInvalidValue;  // K-major weights: bf16 only
    if (g.BM == 16) return launch_kmajor<1>(g, s);
    if (g.BM == 32) return launch_kmajor<2>(g, s);
    return hipErrorInvalidValue;
  }
  if (g.BM == 16) return launch_fmt<1>(false, g, s);
  if (g.BM == 32) return launch_fmt<2>(false, g, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
