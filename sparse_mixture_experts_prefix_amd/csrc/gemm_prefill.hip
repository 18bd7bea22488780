// Prefill-sized grouped GEMMs (many rows per expert): 256 x 256 x 64 tiles.
//
// Same operation as the decode kernels in gemm_decode.hip (SwiGLU expert FFN of the
// glossary "MoE (Mixture of Experts - Mezcla de Expertos)", section 3 step 3;
// packed [E, 2F, D] gate/up tensor of "Transformers v5 El Secreto Detrás de
// los Modelos MoE Más Rápidos", section "La Solución: WeightConverter"), laid
// out for CDNA4:
//  - 4 wavefronts, each owning a 128 x 128 output block as 4 x 4 MFMA
//    32x32x16 tiles (256 fp32 accumulators per lane), so every 16-byte LDS
//    read feeds four MFMAs.
//  - Operands go HBM/L2 -> LDS with buffer_load ... lds (no registers, no
//    ds_write), double-buffered, and a wave's loads of a stage are spread
//    over three MFMA substeps (see k_loop).  Out-of-range buffer offsets read as zero, which handles
//    padding rows, gathered rows of -1 and N/K tails with no branches.
//  - LDS rows are 128 B (64 bf16 of K); the eight 16-byte chunks of row r are
//    stored XOR-swizzled by (r & 7) ^ ((r >> 3) & 1), which keeps both 8- and
//    16-lane phases of the b128 operand reads on distinct banks.
//  - The valid tiles are split into 8 equal runs, one per XCD (the hardware
//    deals workgroups to the 8 XCDs round-robin), each walked in blocks of
//    4 m-tiles x 8 n-tiles, so the workgroups an XCD runs together share
//    their A and B tiles in its L2 and no XCD gets more tiles than another.
//  - MFMA work of 32-row sub-tiles that hold only padding rows is skipped.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kStageBytes = (BM + BN) * BK * 2;  // 64 KB: A then B
constexpr int kLdsBytes = 2 * kStageBytes;       // double buffer
constexpr int MS = 4, NS = 8;                    // super-tile: MS m-tiles x NS n-tiles
constexpr uint32_t kOob = 0x80000000u;           // buffer offset that reads as zero

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword3 0x00020000: raw (untyped) 32-bit data, the gfx9 default for buffer ops
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// First LDS row of B sub-tile j of wave column wn.
template <bool GATE_UP>
__device__ __forceinline__ int b_row_of(int wn, int j) {
  if (GATE_UP) return (j < 2) ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32;
  return wn * 128 + j * 32;
}

// Main loop over K.  LDS holds two stages; registers hold two sets of operand
// fragments (the reads of k-substep ks+1 fly while the 16 MFMAs of ks run).
// The address unit is the scarce resource (one 1-KB load every ~20 cycles per
// CU), so the 16 loads a wave issues per stage are spread over three
// substeps instead of one burst: loads of stage s+1 go out in three groups,
// right after barrier s-1 (during substep 3 of stage s-1) and during substeps
// 0 and 1 of stage s; the barrier before substep 3 of stage s needs them all.
// The weight rows go out in the first groups: their misses travel to HBM and
// need the longest time in flight.
// ACT = active 32-row A sub-tiles of this wave.
template <bool GATE_UP, int ACT, class Issue>
__device__ __forceinline__ void k_loop(const char* lds, int K, int wm, int wn, int lane,
                                       Issue& issue, f32x16 (&acc)[4][4]) {
  const int lr = lane & 31, kh = lane >> 5;
  int rd[4];  // LDS byte offset of this lane's chunk inside a 32-row block, per k-substep
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) rd[ks] = (lr * 8 + ((2 * ks + kh) ^ swz(lr))) * 16;
  const int nk = (K + BK - 1) / BK;

  bf16x8 fa[2][4], fb[2][4];
  auto read = [&](int stage, int ks, int slot) {
    const char* sa = lds + (stage & 1) * kStageBytes;
    const char* sb = sa + BM * BK * 2;
#pragma unroll
    for (int i = 0; i < ACT; ++i)
      fa[slot][i] = *reinterpret_cast<const bf16x8*>(sa + (wm * 128 + i * 32) * 128 + rd[ks]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[slot][j] = *reinterpret_cast<const bf16x8*>(sb + b_row_of<GATE_UP>(wn, j) * 128 + rd[ks]);
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int i = 0; i < ACT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[slot][i], fb[slot][j], acc[i][j]);
  };

  issue(0, 0, 0, 16);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (nk > 1) issue(1, 1, 0, 6);
  read(0, 0, 0);
  // Instruction order of one substep: the fragment reads of the next substep
  // first, then one load per two MFMAs, so no wave stalls on a full address
  // FIFO while its MFMA pipe idles.
  auto pattern = [&](int nvmem) {
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the 8 fragment reads first
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      if (q < nvmem) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one load
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);     // the rest
  };
  for (int s = 0; s + 1 < nk; ++s) {
    const int nxt = s + 2 < nk ? s + 2 : nk - 1;  // past the end: a harmless reload
    read(s, 1, 1);
    issue(s + 1, (s + 1) & 1, 6, 12);
    mma(0);
    pattern(6);
    read(s, 2, 0);
    issue(s + 1, (s + 1) & 1, 12, 16);
    mma(1);
    pattern(4);
    read(s, 3, 1);
    mma(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): stage s+1 landed (this wave)
    __syncthreads();                     // all waves: s+1 landed, stage s fully read
    read(s + 1, 0, 0);
    issue(nxt, s & 1, 0, 6);
    mma(1);
    pattern(6);
  }
  // last stage: no loads, no barrier
  read(nk - 1, 1, 1);
  mma(0);
  read(nk - 1, 2, 0);
  mma(1);
  read(nk - 1, 3, 1);
  mma(0);
  mma(1);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no load may still be writing LDS at exit
}

template <bool GATE_UP>
__device__ __forceinline__ void prefill_tile(const GroupedGemm& p, char* lds) {
  // ---------------------------------------------------------------- schedule
  // The V = m_tiles x n_tiles valid tiles (m_tiles is known on the device
  // only) are cut into 8 equal runs, one per XCD: the hardware deals
  // workgroup b to XCD b % 8, so XCD x executes run x in order.  Inside a run,
  // tiles go in columns of NS n-tiles, and in each column in blocks of MS
  // m-tiles x NS n-tiles, so the workgroups an XCD runs together share A and
  // B tiles in its L2.
  const int64_t nt_n = p.n_tiles_n;
  const int64_t mt = p.n_tiles[0];
  const int64_t V = mt * nt_n;
  const int64_t run = (V + 7) / 8;
  const int64_t jb = blockIdx.x / 8;
  if (jb >= run) return;
  const int64_t L = (blockIdx.x % 8) * run + jb;
  if (L >= V) return;
  const int64_t colsz = mt * NS;
  const int64_t sn = L / colsz;
  const int64_t cw = min((int64_t)NS, nt_n - sn * NS);  // n-tiles in this column
  const int64_t rem = L - sn * colsz;
  const int64_t mb = rem / (MS * cw);
  const int64_t mh = min((int64_t)MS, mt - mb * MS);      // m-tiles in this block
  const int64_t inner = rem - mb * MS * cw;
  const int64_t m_tile = mb * MS + inner % mh;
  const int64_t n_tile = sn * NS + inner / mh;
  const int g = p.tile_group[m_tile];
  const bool shared = g >= p.E;
  const int N = shared ? p.N_shared : p.N_routed;
  const int K = shared ? p.K_shared : p.K_routed;
  constexpr int NB = GATE_UP ? BN / 2 : BN;
  const int n0 = (int)n_tile * NB;
  if (n0 >= N) return;
  const int64_t row0 = m_tile * BM;
  const int valid_rows = min(BM, (int)(p.group_count[g] - (row0 - p.group_padded[g])));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ------------------------------------------------------ operand sources
  // Wave `wave`, load j (0..7) writes LDS rows (wave*8 + j)*8 .. +7 of a
  // region; lane i of it carries row +i/8 and K-chunk (i%8) ^ swz(row).
  const __amdgpu_buffer_rsrc_t rsA =
      GATE_UP ? make_rsrc(p.A, (uint32_t)p.a_bytes)
              : make_rsrc(p.A + row0 * p.lda, (uint32_t)(BM * p.lda * 2));
  const bf16_t* Bg = shared ? p.B_shared
                            : p.B_routed + (int64_t)g * (GATE_UP ? 2 : 1) * (int64_t)N * K;
  const __amdgpu_buffer_rsrc_t rsB =
      make_rsrc(Bg, (uint32_t)((int64_t)(GATE_UP ? 2 : 1) * N * K * 2));
  uint32_t offA[8], offB[8];
  const int sub = lane >> 3;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (wave * 8 + j) * 8 + sub;  // 0..255
    const int kc = (lane & 7) ^ swz(r);
    const uint32_t kb = kc * 16;
    if (GATE_UP) {
      const int t = r < valid_rows ? p.row_token[row0 + r] : -1;
      offA[j] = t >= 0 ? (uint32_t)t * (uint32_t)(p.lda * 2) + kb : kOob;
      const int half = r >> 7, f = n0 + (r & 127);
      offB[j] = f < N ? (uint32_t)(half * N + f) * (uint32_t)(K * 2) + kb : kOob;
    } else {
      offA[j] = r < valid_rows ? (uint32_t)r * (uint32_t)(p.lda * 2) + kb : kOob;
      const int n = n0 + r;
      offB[j] = n < N ? (uint32_t)n * (uint32_t)(K * 2) + kb : kOob;
    }
  }
  const int kcl = (lane & 7);  // chunk position within the 8 of a row, before the swizzle

  // loads q in [q0, q1) of K-stage `stage` into LDS buffer `buf`: q 0..7 are
  // B rows (expert weights, mostly HBM misses, so they go out first), q 8..15
  // A rows (activations, mostly cache hits).  Chunks at or past K (only in the
  // last stage when K % 64 != 0) read as zero.
  auto issue = [&](int stage, int buf, int q0, int q1) {
    const int k0 = stage * BK;
    char* base = lds + buf * kStageBytes;
    const bool tail = k0 + BK > K;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < q0 || q >= q1) continue;
      const bool isB = q < 8;
      const int j = q & 7;
      uint32_t o = isB ? offB[j] : offA[j];
      if (tail) {
        const int r = (wave * 8 + j) * 8 + sub;
        const int kc = kcl ^ swz(r);
        if (k0 + kc * 8 >= K) o = kOob;
      }
      char* dst = base + (isB ? BM * BK * 2 : 0) + (wave * 8 + j) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isB ? rsB : rsA, (lds_void*)dst, 16, o, k0 * 2, 0, 0);
    }
  };

  // active 32-row sub-tiles of this wave (uniform): the K loop is compiled
  // once per count so no MFMA sits under a branch
  const int act = min(4, max(0, (valid_rows - wm * 128 + 31) / 32));
  const int lr = lane & 31, kh = lane >> 5;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  switch (act) {
    case 4: k_loop<GATE_UP, 4>(lds, K, wm, wn, lane, issue, acc); break;
    case 3: k_loop<GATE_UP, 3>(lds, K, wm, wn, lane, issue, acc); break;
    case 2: k_loop<GATE_UP, 2>(lds, K, wm, wn, lane, issue, acc); break;
    case 1: k_loop<GATE_UP, 1>(lds, K, wm, wn, lane, issue, acc); break;
    default: k_loop<GATE_UP, 0>(lds, K, wm, wn, lane, issue, acc); break;
  }
  auto a_row = [&](int i) { return wm * 128 + i * 32; };

  // -------------------------------------------------------------- epilogue
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= act) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = a_row(i) + 8 * (r >> 2) + 4 * kh + (r & 3);
      const int64_t grow = row0 + row;
      if (GATE_UP) {
        bf16_t* H = reinterpret_cast<bf16_t*>(p.C);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int f = n0 + wn * 64 + j * 32 + lr;
          if (f < N) H[grow * p.ldc + f] = f32_to_bf16(silu(acc[i][j][r]) * acc[i][j + 2][r]);
        }
      } else {
        float* Y = reinterpret_cast<float*>(p.C);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 128 + j * 32 + lr;
          if (n < N) Y[grow * p.ldc + n] = acc[i][j][r];
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void moe_gemm_gate_up_prefill_kernel(GroupedGemm p) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  prefill_tile<true>(p, lds);
}

__global__ __launch_bounds__(256) void moe_gemm_down_prefill_kernel(GroupedGemm p) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  prefill_tile<false>(p, lds);
}

hipError_t launch(bool gate_up, GroupedGemm g, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)moe_gemm_gate_up_prefill_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)moe_gemm_down_prefill_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nmax = g.N_routed > g.N_shared ? g.N_routed : g.N_shared;
  const int NB = gate_up ? BN / 2 : BN;
  g.n_tiles_n = (nmax + NB - 1) / NB;
  // enough workgroups for every XCD's run (see prefill_tile)
  const int64_t blocks = (g.max_tiles * g.n_tiles_n + 7) / 8 * 8;
  if (blocks == 0) return hipSuccess;
  if (gate_up)
    hipLaunchKernelGGL(moe_gemm_gate_up_prefill_kernel, dim3((unsigned)blocks), dim3(256), kLdsBytes,
                       s, g);
  else
    hipLaunchKernelGGL(moe_gemm_down_prefill_kernel, dim3((unsigned)blocks), dim3(256), kLdsBytes, s,
                       g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gate_up_prefill(const GroupedGemm& g, hipStream_t s) {
  return launch(true, g, s);
}

hipError_t launch_gemm_down_prefill(const GroupedGemm& g, hipStream_t s) {
  return launch(false, g, s);
}

}  // namespace moe
