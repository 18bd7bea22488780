// Prefill-sized grouped GEMMs (many rows per expert): 256 x 256 x 64 tiles.
//
// Same operation as the decode kernels in gemm_decode.hip (SwiGLU expert FFN of the
// glossary "MoE (Mixture of Experts - Mezcla de Expertos)", section 3 step 3;
// packed [E, 2F, D] gate/up tensor of "Transformers v5 El Secreto Detrás de
// los Modelos MoE Más Rápidos", section "La Solución: WeightConverter"), laid
// out for CDNA4:
//  - 4 wavefronts, each owning 128 x 128 outputs as 4 x 4 MFMA 32x32x16
//    tiles (256 fp32 accumulators per lane; in a partly filled tile its 4 row
//    blocks of 32 alternate with the other wave row's), so every 16-byte LDS
//    read feeds four MFMAs.
//  - Operands go HBM/L2 -> LDS with buffer_load ... lds (no registers, no
//    ds_write); A is double- and B triple-buffered, and a wave's loads of a
//    stage are spread evenly over the MFMA substeps (see k_loop).
//    Out-of-range buffer offsets read as zero, which handles padding rows,
//    gathered rows of -1 and N/K tails with no branches.
//  - LDS rows are 128 B (64 bf16 of K); the eight 16-byte chunks of row r are
//    stored XOR-swizzled by (r & 7) ^ ((r >> 3) & 1), which keeps both 8- and
//    16-lane phases of the b128 operand reads on distinct banks.
//  - The valid tiles are split into 8 equal runs, one per XCD (the hardware
//    deals workgroups to the 8 XCDs round-robin), each walked in blocks of
//    up to 4 m-tiles of one expert x 8 n-tiles, so the workgroups an XCD runs
//    together share their A and B tiles in its L2 and no XCD gets more tiles
//    than another.
//  - MFMA work of 32-row sub-tiles that hold only padding rows is skipped.
//  - A short, partial last round of tiles is cut along K (see split_of).
//  - A group's last m-tile of at most 32 rows is not a tile of its own: the
//    m-tile before it computes those rows too, with their A fragments loaded
//    straight into registers (see tile_rows and k_loop's XR).
//  - E4M3 weights (one fp32 scale per weight row): a B stage holds the codes,
//    64-byte rows of four 16-byte chunks swizzled by (r >> 1) & 3; a lane's
//    16-byte read carries its weights of two k-substeps (K is permuted the
//    same way for A), widened to bf16 exactly in registers, and each output
//    column is multiplied by its row's scale before the epilogue.  Half the
//    weight bytes and half the B loads of bf16, for the same MFMAs.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kABytes = BM * BK * 2;             // 32 KB: one K-stage of A
constexpr int kBBytes = BN * BK * 2;             // 32 KB: one K-stage of B
constexpr int kLdsBytes = 2 * kABytes + 3 * kBBytes;  // A double-, B triple-buffered: 160 KB
constexpr int kB8Bytes = BN * BK;                // 16 KB: one K-stage of E4M3 B
template <bool FP8> constexpr int b_stage_bytes() { return FP8 ? kB8Bytes : kBBytes; }
static_assert(2 * kABytes + 3 * kB8Bytes <= kLdsBytes, "E4M3 K stages must fit");
template <bool FP8> constexpr int lds_bytes() { return kLdsBytes; }
constexpr int MS = 4, NS = 8;                    // tile blocks: up to MS m-tiles x NS n-tiles
constexpr int kExtraRows = 32;                   // rows a full m-tile takes on from the next
constexpr int kTileRows = BM + kExtraRows;        // rows of the largest tile
static_assert(kTileRows * BN == kPartialTileFloats, "a partial tile holds the largest tile");
constexpr int kMaxSplit = 8;                     // pieces per tile of the last round
constexpr int kMinPieceStages = 4;               // K-stages per piece, at least
constexpr int kSplitRounds = 4;                  // cut only when V < kSplitRounds * ctas
constexpr uint32_t kOob = 0x80000000u;           // buffer offset that reads as zero

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword3 0x00020000: raw (untyped) 32-bit data, the gfx9 default for buffer ops
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// 16-byte chunk swizzle of the 64-byte rows of an E4M3 B stage
__device__ __forceinline__ int swz4(int r) { return (r >> 1) & 3; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight E4M3 codes (bytes 0..7 of two dwords, element i in byte i) widened to bf16.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// K-major B stage: 64 k-rows of 512 B (256 columns).  16-byte chunk c of
// k-row k is stored at chunk position c ^ (4 (k % 4)): the transposing reads of
// a 32-lane half (4 k-rows x 4 chunks) then hit 16 distinct chunk positions
// mod 16, i.e. all 64 banks once.
__device__ __forceinline__ int kmaj_chunk(int k, int c) { return c ^ (4 * (k & 3)); }
typedef short i16x4 __attribute__((ext_vector_type(4)));

// First row of A sub-tile i of wave row wm.  A full tile gives each wave row
// a contiguous half; in a partly filled tile (il) the 8 sub-tiles of 32 rows
// alternate between the two wave rows, so its MFMA work is split over both
// (the busier wave row sets a workgroup's pace).
__device__ __forceinline__ int a_row_of(int wm, int i, bool il) {
  return il ? 32 * (2 * i + wm) : 128 * wm + 32 * i;
}

// First LDS row of B sub-tile j of wave column wn.
template <bool GATE_UP>
__device__ __forceinline__ int b_row_of(int wn, int j) {
  if (GATE_UP) return (j < 2) ? wn * 64 + j * 32 : 128 + wn * 64 + (j - 2) * 32;
  return wn * 128 + j * 32;
}

// Main loop over K.  LDS holds two K-stages of A and three of B (all 160 KB);
// registers hold two sets of operand fragments (the reads of k-substep ks+1
// fly while the 16 MFMAs of ks run).  Per stage a wave issues 16 loads, four
// in each substep, since the CU's address unit (about one 1-KB load per ~20
// cycles) stalls the in-order issue when loads come in bursts:
//  - after barrier i (stage i fully read) and in substep 0 of stage i+1: the
//    A rows of stage i+2 (activations, mostly cache hits), into the A buffer
//    stage i used;
//  - in substeps 1 and 2 of stage i+1: the B rows of stage i+3 (expert
//    weights, whose misses go to HBM), into the B buffer stage i used, a
//    whole stage ahead of their use.
// The barrier before substep 3 of stage i+1 waits for A(i+2) and B(i+2)
// only (vmcnt(8): the eight B(i+3) loads issued after them may still fly).
// Stages s0 .. s0+n-1 (n >= 1); ACT = active 32-row A sub-tiles of this wave;
// NA = A loads per wave and stage (8; fewer when the tile has few rows: the
// rows a load slot j of any wave carries start at 32 j, so 2 tier slots cover
// the first 64 tier rows).
// E4M3 B: four loads per wave and stage instead of eight, so B(i+3) takes
// two per substep and the barrier waits with vmcnt(4).
// KMAJ: B is K-major (see kmaj_chunk); KA: A is too.
// XR: the tile also computes its folded rows (see tile_rows).  Their A
// fragments come from memory straight into registers, one 16-byte load per
// lane and k-substep (every wave loads the same 32 rows), issued a stage
// ahead together with the A rows of that stage, so that B's loads keep their
// lead; each wave takes two 32 x 32 output blocks of them with the B
// fragments it already holds: gate/up the gate and up blocks of column block
// wm of its half, down column blocks 2 wm and 2 wm + 1 of its half.
struct ExtraRows {
  __amdgpu_buffer_rsrc_t rs;  // A's buffer
  uint32_t off;               // this lane's row (lane % 32) at k = 0 (kOob past the rows)
  int K;
  f32x16 acc[2];
};
// column block (j of b_row_of) of folded-row output block h of wave row w
template <bool GATE_UP>
__device__ __forceinline__ constexpr int xblock(int w, int h) {
  return GATE_UP ? w + 2 * h : 2 * w + h;
}
// The folded rows' two MFMAs with their accumulators in VGPRs: the tile's
// 256 accumulators fill the AGPRs, and the compiler would put these in AGPRs
// too (and spill).  Written out, so the hazards the compiler handles for its
// own MFMAs are handled here: two wait states before (an E4M3 B fragment is
// written by VALU just before), and xr_settle after the K loop, before any
// other instruction reads the accumulators.
__device__ __forceinline__ void mfma32_x2(f32x16& c0, f32x16& c1, const bf16x8& a, const bf16x8& b0,
                                          const bf16x8& b1) {
  asm("s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %2, %4, %1"
      : "+v"(c0), "+v"(c1)
      : "v"(__builtin_bit_cast(u32x4, a)), "v"(__builtin_bit_cast(u32x4, b0)),
        "v"(__builtin_bit_cast(u32x4, b1)));
}
// wait states after the last of them (a 32x32x16 MFMA's result is read by
// VALU or memory instructions only 18 or more wait states later); the
// accumulators pass through, so nothing that reads them can move above it
__device__ __forceinline__ void xr_settle(f32x16& c0, f32x16& c1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1));
}

template <bool GATE_UP, int ACT, bool FP8, class IssueA, class IssueB, bool KMAJ = false,
          bool KA = false, bool PRE = false, int NA = 8, bool XR = false, int XW = 0>
__device__ __forceinline__ void k_loop(const char* lds, int s0, int n, int wm, int wn, bool il,
                                       int lane, IssueA& issue_a, IssueB& issue_b,
                                       f32x16 (&acc)[4][4], ExtraRows* xr = nullptr) {
  static_assert(!KMAJ || (!GATE_UP && !FP8), "K-major B: bf16 rows x weight products only");
  static_assert(!KA || KMAJ, "K-major A comes with K-major B");
  static_assert(!XR || (ACT == 4 && NA == 8 && !KMAJ), "folded rows: full tiles of the forward kernels");
  constexpr int NBL = FP8 ? 4 : 8;  // B loads per wave and stage
  const int lr = lane & 31, kh = lane >> 5;
  // LDS byte offset of this lane's A chunk inside a 32-row block, per k-substep.
  // bf16: substep ks takes K chunk 2ks + kh.  E4M3: substeps 2m, 2m+1 take
  // chunks 4m + 2kh and 4m + 2kh + 1, so a lane's B bytes of both are one
  // 16-byte chunk (2m + kh) of its 64-byte B row.
  int rd[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = FP8 ? 4 * (ks >> 1) + 2 * kh + (ks & 1) : 2 * ks + kh;
    rd[ks] = (lr * 8 + (c ^ swz(lr))) * 16;
  }
  int rd8[2];  // E4M3 B: byte offset of chunk 2m + kh inside a 32-row block
#pragma unroll
  for (int m = 0; m < 2; ++m) rd8[m] = lr * 64 + ((2 * m + kh) ^ swz4(lr)) * 16;
  // K-major B (a stage is 64 k-rows of 512 B; see kmaj_chunk): a transposing
  // 8-byte read gives lane i of each 16-lane group element (i % 4) of the
  // word that lane (i / 4) + 4 j of the group points at, as its element j.
  // So group lane q points at k-row 4 t + q / 4 (t: which half of the lane's
  // eight k) and columns 4 (q % 4) .. + 3 of its 16; the four words of a
  // lane's column then arrive as k, k + 1, k + 2, k + 3.
  // (A operand alike: lane l needs A[m = l % 32][8 consecutive k], the same shape)
  int rdk[4], rdka[4];
  {
    const int q = lane & 15, g16 = (lane >> 4) & 1;
    const int k = 8 * kh + (q >> 2);                     // k-row of this lane's word
    const int col = 16 * g16 + 4 * (q & 3);               // first column, inside a 32-wide sub-tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = b_row_of<false>(wn, j) + col;         // column in the 256-wide tile
      rdk[j] = k * 512 + kmaj_chunk(k, c >> 3) * 16 + (c & 7) * 2;
      const int ca = a_row_of(wm, j, il) + col;
      rdka[j] = k * 512 + kmaj_chunk(k, ca >> 3) * 16 + (ca & 7) * 2;
    }
  }
  // the fragment (8 consecutive k of one column) of a K-major stage, from two
  // transposing reads at byte offset `off` and 4 k-rows further
  auto read_tr = [](const char* base, int off) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    typedef __attribute__((address_space(3))) char lds_char;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_char*)(base + off)));
    const i16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_char*)(base + off + 4 * 512)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  bf16x8 fa[2][4], fb[2][4];
  u32x4 fq[4];  // E4M3 B: the codes of two substeps
  // fragments of k-substep ks of local stage ls (B buffer bb) into register set `slot`
  auto read = [&](int ls, int bb, int ks, int slot) {
    const char* sa = lds + (ls & 1) * kABytes;
    const char* sb = lds + 2 * kABytes + bb * b_stage_bytes<FP8>();
#pragma unroll
    for (int i = 0; i < ACT; ++i) {
      if constexpr (KA)
        fa[slot][i] = read_tr(sa, rdka[i] + ks * 16 * 512);
      else
        fa[slot][i] = *reinterpret_cast<const bf16x8*>(sa + a_row_of(wm, i, il) * 128 + rd[ks]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (FP8) {
        if ((ks & 1) == 0)
          fq[j] = *reinterpret_cast<const u32x4*>(sb + b_row_of<GATE_UP>(wn, j) * 64 + rd8[ks >> 1]);
        fb[slot][j] = e4m3x8_to_bf16(fq[j][2 * (ks & 1)], fq[j][2 * (ks & 1) + 1]);
      } else if constexpr (KMAJ) {
        // k-rows 16 ks + 4 t + ... of this lane's word; kmaj_chunk depends on
        // k % 4 only, which the 16 ks + 4 t step keeps
        fb[slot][j] = read_tr(sb, rdk[j] + ks * 16 * 512);
      } else {
        fb[slot][j] = *reinterpret_cast<const bf16x8*>(sb + b_row_of<GATE_UP>(wn, j) * 128 + rd[ks]);
      }
    }
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int i = 0; i < ACT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[slot][i], fb[slot][j], acc[i][j]);
  };
  // folded rows: fragments of the current and the next stage
  u32x4 xcur[4], xnext[4];
  auto issue_x = [&](int stage, u32x4(&dst)[4]) {
    if constexpr (XR) {
      const int k0 = stage * BK;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c = FP8 ? 4 * (ks >> 1) + 2 * kh + (ks & 1) : 2 * ks + kh;  // as rd[ks]
        const uint32_t o = k0 + 8 * c < xr->K ? xr->off + 16 * c : kOob;
        dst[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr->rs, o, 2 * k0, 0));
      }
    }
  };
  auto mma_x = [&](int slot, int ks) {
    if constexpr (XR) {
      // XW = wm, a compile-time copy of the loop per wave row
      const bf16x8 a = __builtin_bit_cast(bf16x8, xcur[ks]);
      mfma32_x2(xr->acc[0], xr->acc[1], a, fb[slot][xblock<GATE_UP>(XW, 0)],
                fb[slot][xblock<GATE_UP>(XW, 1)]);
    }
  };
  // instruction order of one substep (16 MFMAs): one MFMA, then the 8
  // fragment reads of the next substep each behind one MFMA (a burst of reads
  // queues behind the other waves' reads and the loads' LDS writes), then the
  // four loads, one per two MFMAs.  Measured 3-4% faster than reads first.
  // (K-major B: 12 reads, each B fragment being two transposing reads, and
  // one MFMA between the loads)
  // (both K-major: 16 reads, one per MFMA, with the loads among the last)
  auto pattern = [&]() {
    if constexpr (KA) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
      for (int q = 0; q < 12; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      return;
    }
    constexpr int RD = KMAJ ? 12 : 8, GAP = KMAJ ? 1 : 2;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int q = 0; q < RD; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one fragment read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    }
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // one load
    __builtin_amdgcn_sched_group_barrier(0x008, GAP, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, GAP, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, GAP, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    if constexpr (15 - RD - 3 * GAP > 0) __builtin_amdgcn_sched_group_barrier(0x008, 15 - RD - 3 * GAP, 0);
  };
  // XR: nl (4, or 8 with the folded rows' loads) loads spread over the 16
  // MFMAs after the reads (the folded rows' two MFMAs are written out, which
  // the scheduler does not count)
  auto pattern_x = [&](auto nl) {
    constexpr int NL = decltype(nl)::value, GAP = NL > 4 ? 1 : 2, REST = 16 - 9 - GAP * (NL - 1);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (q + 1 < NL) __builtin_amdgcn_sched_group_barrier(0x008, GAP, 0);
    }
    if constexpr (REST > 0) __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);
  };
  auto block_pattern = [&](auto nl) {
    if constexpr (XR)
      pattern_x(nl);
    else
      pattern();
  };
  using L4 = std::integral_constant<int, 4>;
  using L8 = std::integral_constant<int, 8>;

  if constexpr (!PRE) {  // PRE: the caller has issued stage s0's loads
    issue_b(s0, 0, 0, NBL);
    issue_a(s0, 0, 0, NA);
  }
  issue_x(s0, xcur);
  if (n > 1) issue_b(s0 + 1, 1, 0, NBL);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (n > 1) issue_a(s0 + 1, 1, 0, NA / 2);
  read(0, 0, 0, 0);
  int bcur = 0, b2 = 2;  // B buffers of stages i and i+2
  for (int i = 0; i + 1 < n; ++i) {
    const int a2 = i + 2 < n ? i + 2 : n - 1;  // past the end: harmless reloads
    read(i, bcur, 1, 1);
    issue_a(s0 + i + 1, (i + 1) & 1, NA / 2, NA);
    issue_x(s0 + i + 1, xnext);  // before B(i+2), whose loads may still fly at the barrier
    mma(0);
    mma_x(0, 0);
    block_pattern(L8{});
    read(i, bcur, 2, 0);
    issue_b(s0 + a2, b2, 0, NBL / 2);
    mma(1);
    mma_x(1, 1);
    block_pattern(L4{});
    read(i, bcur, 3, 1);
    issue_b(s0 + a2, b2, NBL / 2, NBL);
    mma(0);
    mma_x(0, 2);
    block_pattern(L4{});
    // vmcnt(NBL): A(i+1) and B(i+1) landed, B(i+2) may still fly; lgkmcnt(0):
    // this wave's reads of stage i are done.  A plain s_barrier, since the
    // fence of __syncthreads would wait for every load.
    if constexpr (FP8)
      __builtin_amdgcn_s_waitcnt(0x0074);
    else
      __builtin_amdgcn_s_waitcnt(0x0078);
    __builtin_amdgcn_s_barrier();
    bcur = bcur == 2 ? 0 : bcur + 1;
    b2 = b2 == 2 ? 0 : b2 + 1;
    read(i + 1, bcur, 0, 0);
    issue_a(s0 + a2, i & 1, 0, NA / 2);
    mma(1);
    mma_x(1, 3);
    block_pattern(L4{});
    if constexpr (XR) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) xcur[ks] = xnext[ks];
    }
  }
  // last stage: no loads, no barrier
  read(n - 1, bcur, 1, 1);
  mma(0);
  mma_x(0, 0);
  read(n - 1, bcur, 2, 0);
  mma(1);
  mma_x(1, 1);
  read(n - 1, bcur, 3, 1);
  mma(0);
  mma_x(0, 2);
  mma(1);
  mma_x(1, 3);
  if constexpr (XR) xr_settle(xr->acc[0], xr->acc[1]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no load may still be writing LDS at exit
}

// ------------------------------------------------------------------ schedule
// V = m_tiles x n_tiles valid tiles (m_tiles is known on the device only).
// When V is not a multiple of the `ctas` workgroups that run at once, the
// last, partial round is balanced: its R tiles are each cut into S pieces
// along K (R*S <= ctas).  Each piece stores its fp32 partial tile, and a
// second kernel adds the S partials in K order and runs the epilogue.  Only
// for a few rounds of tiles: with many rounds the hardware's dispatch of
// tiles to CUs as they free up already evens out the end, and the partial
// tiles would cost more than they save.
struct Split {
  int64_t V, R, n_dp;  // valid tiles, tiles cut in pieces (the last R), tiles run whole
  int S;               // pieces per cut tile (1: no cut)
};

__device__ __forceinline__ Split split_of(const GroupedGemm& p, int64_t mt) {
  Split sp;
  sp.V = mt * p.n_tiles_n;
  sp.R = 0;
  sp.S = 1;
  if (p.ctas > 0 && sp.V % p.ctas && sp.V < (int64_t)kSplitRounds * p.ctas) {
    const int64_t R = sp.V % p.ctas;
    const int kmin = p.B_shared && p.K_shared < p.K_routed ? p.K_shared : p.K_routed;
    const int64_t by_k = ((kmin + BK - 1) / BK) / kMinPieceStages;
    const int64_t S = min(min((int64_t)kMaxSplit, p.ctas / R), by_k);
    if (S >= 2) {
      sp.R = R;
      sp.S = (int)S;
    }
  }
  sp.n_dp = sp.V - sp.R;
  return sp;
}

// Rows of a group's m-tiles.  A group of two m-tiles (a few hundred rows:
// many experts, few rows each) shares its rows out evenly, q = ceil(count / 2)
// rounded up to whole 32-row sub-tiles: otherwise its second m-tile holds a
// few rows, runs ahead of the first (it is load-bound, with almost no MFMA
// work) and reads the expert's weights from HBM a second time instead of from
// L2 together with the first.  Larger groups keep full 256-row m-tiles (q =
// 256): there the light last m-tile costs a smaller share of the weight
// traffic, and evening out would make every m-tile as slow as a full one (the
// busier half of a workgroup's waves sets its pace).  Rows stay contiguous:
// m-tile j covers the group's rows j q .. j q + valid - 1, stored from padded
// row row0 = group_padded[g] + j q (its 256-row window may reach into the next
// m-tile's rows, which it neither reads nor writes).
// In the forward kernels (not K-major B) a group of two or more m-tiles whose
// last one would hold at most kExtraRows rows folds those rows into the m-tile
// before it, which then has valid = 256 rows through LDS plus `extra` rows
// 256 .. 256 + extra - 1; the last m-tile does not run.  It would stream the
// expert's whole weight tile for a few rows, at over half a full tile's time
// (and a group of 257-288 rows would be two half-empty tiles).  m-tiles of a
// group of c rows that run:
__device__ __forceinline__ int run_mtiles(int c) {
  const int mg = (c + BM - 1) / BM;
  return mg - (mg >= 2 && c - (mg - 1) * BM <= kExtraRows ? 1 : 0);
}

// A group's m-tiles as the kernel numbers them: the group, its row count, its
// first m-tile and its m-tiles.  FOLD: the m-tiles that run, numbered group by
// group in row order; else every BM-row m-tile of the padded layout (the
// align kernel's tile_group and n_tiles).
struct RunGroup {
  int g, cnt, mg;
  int64_t first;
};

// FOLD numbering: every wave derives it from the group counts, five groups per
// lane (one round of loads and a wave-wide prefix sum), so no workgroup is
// launched for a folded m-tile.  (Such workgroups, returning at once, left CUs
// idle behind longer tiles: the hardware hands workgroups out to the XCDs in
// order.  The same numbering read from tables the align kernel wrote measured
// slower: the down GEMM on the Mixtral shape took 0.96 ms instead of 0.82.)
constexpr int kGroupsPerLane = 5;  // 64 x 5 >= 257 groups
struct GroupScan {
  int cnt[kGroupsPerLane];  // counts of this lane's groups 5 l .. 5 l + 4 (0 past the last)
  int excl;                 // m-tiles that run in the groups before them
  int64_t mt;               // m-tiles that run in all groups
};

__device__ __forceinline__ GroupScan scan_groups(const GroupedGemm& p) {
  const int lane = threadIdx.x & 63;
  const int G = p.E + (p.B_shared ? 1 : 0);
  GroupScan sc;
  int tot = 0;
#pragma unroll
  for (int q = 0; q < kGroupsPerLane; ++q) {
    const int g = lane * kGroupsPerLane + q;
    sc.cnt[q] = g < G ? p.group_count[g] : 0;
    tot += run_mtiles(sc.cnt[q]);
  }
  int incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  sc.excl = incl - tot;
  sc.mt = __builtin_amdgcn_readlane(incl, 63);
  return sc;
}

template <bool FOLD>
__device__ __forceinline__ int64_t mtiles_of(const GroupedGemm& p) {
  if constexpr (FOLD) return scan_groups(p).mt;
  return p.n_tiles[0];
}

// the group of m-tile m (< mtiles_of), as wave-uniform (scalar) values
template <bool FOLD>
__device__ __forceinline__ RunGroup group_of_mtile(const GroupedGemm& p, int64_t m) {
  RunGroup rg;
  if constexpr (FOLD) {
    const GroupScan sc = scan_groups(p);
    const int lane = threadIdx.x & 63;
    int run = sc.excl, hit = -1, hfirst = 0, hmg = 0;
#pragma unroll
    for (int q = 0; q < kGroupsPerLane; ++q) {
      const int mm = run_mtiles(sc.cnt[q]);
      if (m >= run && m < run + mm) {
        hit = lane * kGroupsPerLane + q;
        hfirst = run;
        hmg = mm;
      }
      run += mm;
    }
    const int src = (int)__builtin_ctzll(__ballot(hit >= 0));  // the one lane that holds it
    rg.g = __builtin_amdgcn_readlane(hit, src);
    rg.first = __builtin_amdgcn_readlane(hfirst, src);
    rg.mg = __builtin_amdgcn_readlane(hmg, src);
  } else {
    rg.g = p.tile_group[m];
    rg.first = p.group_padded[rg.g] / p.BM;
    rg.mg = (int)(p.group_padded[rg.g + 1] / p.BM - rg.first);
  }
  rg.cnt = p.group_count[rg.g];
  return rg;
}

// Logical tile L -> (m-tile, n_tile) and its group: columns of NS n-tiles;
// inside a column the groups in order, each cut into blocks of up to MS of its
// m-tiles x the column's n-tiles, m-tile fastest.  Consecutive tiles (the
// workgroups an XCD runs together) then share their A and B tiles, and a
// block never straddles two experts' weights.
// A block that holds its group's folded m-tile (see tile_rows), whose tiles
// take longer than the others, lists that m-tile's tiles first (n fastest):
// workgroups are handed out in order to the CUs that free up first, so the
// heavy tiles of the next block go to CUs that just ran light ones.  In the
// m-tile order the CUs that finished a heavy tile last also took the next
// block's heavy tiles, and with two rounds of tiles (the down GEMM at the
// Mixtral shape) those CUs set the kernel's end.
template <bool FOLD>
__device__ __forceinline__ void tile_coords(const GroupedGemm& p, int64_t mt, int64_t L,
                                            int64_t& m_tile, int64_t& n_tile, RunGroup& rg) {
  const int64_t colsz = mt * NS;
  const int64_t sn = L / colsz;
  const int64_t cw = min((int64_t)NS, p.n_tiles_n - sn * NS);  // n-tiles in this column
  const int64_t u = L - sn * colsz;                               // < mt * cw
  rg = group_of_mtile<FOLD>(p, u / cw);
  const int64_t v = u - rg.first * cw;                            // < mg * cw
  const int64_t mb = v / (MS * cw);                               // block of the group
  const int64_t mh = min((int64_t)MS, rg.mg - mb * MS);           // its m-tiles
  const int64_t inner = v - mb * MS * cw;
  if (FOLD && mh > 1 && mb * MS + mh == rg.mg && rg.mg < (rg.cnt + BM - 1) / BM) {
    // the block's last m-tile holds the folded rows
    if (inner < cw) {
      m_tile = rg.first + mb * MS + mh - 1;
      n_tile = sn * NS + inner;
    } else {
      const int64_t j = inner - cw;
      m_tile = rg.first + mb * MS + j % (mh - 1);
      n_tile = sn * NS + j / (mh - 1);
    }
    return;
  }
  m_tile = rg.first + mb * MS + inner % mh;
  n_tile = sn * NS + inner / mh;
}

// Rows of the group's j-th m-tile (in row order; see above).
template <bool FOLD>
__device__ __forceinline__ void tile_rows(const GroupedGemm& p, const RunGroup& rg, int64_t j,
                                          int64_t& row0, int& valid, int& extra) {
  const int cnt = rg.cnt;
  const int64_t pad0 = p.group_padded[rg.g];
  const int mg = (cnt + BM - 1) / BM;  // m-tiles of the padded layout
  extra = 0;
  if (FOLD && rg.mg < mg) {  // the last m-tile's rows fold into m-tile mg - 2
    row0 = pad0 + j * BM;
    valid = BM;
    if (j == rg.mg - 1) extra = cnt - (int)(j + 1) * BM;
    return;
  }
  const int q = mg == 2 ? ((cnt + 1) / 2 + 31) / 32 * 32 : BM;
  row0 = pad0 + j * q;
  valid = max(0, min(q, cnt - (int)(j * q)));
}

// KT: K may end inside a K-stage (K % 64 != 0), so loads of the last stage
// mask the chunks past K; with KT false the K loop carries no such selects.
// FOLD (see tile_rows): bf16 row-major weights only; the E4M3 kernels keep
// their registers for widening the codes (the folded rows' fragments and
// accumulators made them spill in the K loop).
// NTB: the weight loads take the non-temporal cache policy, for launches
// whose expert groups are about one m-tile each (every weight tile is then
// read by one workgroup, and keeping it in L2 only evicts the shared rows).
template <bool GATE_UP, bool FP8, bool KMAJ = false, bool KT = true, bool NTB = false>
__device__ __forceinline__ void prefill_tile(const GroupedGemm& p, char* lds) {
  constexpr bool FOLD = !KMAJ && !FP8;
  // The V - R whole tiles are cut into 8 equal runs, one per XCD: the
  // hardware deals workgroup b to XCD b % 8, so XCD x executes run x in
  // order and the workgroups an XCD runs together share A and B tiles in its
  // L2.  The R*S pieces come after all of them.
  const int64_t mt = mtiles_of<FOLD>(p);
  const Split sp = split_of(p, mt);
  const int64_t run = (sp.n_dp + 7) / 8;
  const int64_t b = blockIdx.x;
  int64_t L;
  int part = 0, piece_tile = 0;
  if (b < 8 * run) {
    L = (b % 8) * run + b / 8;
    if (L >= sp.n_dp) return;
  } else {
    const int64_t q = b - 8 * run;
    if (q >= sp.R * sp.S) return;
    piece_tile = (int)(q % sp.R);
    part = (int)(q / sp.R);
    L = sp.n_dp + piece_tile;
  }
  const bool piece = L >= sp.n_dp;
  const int S = sp.S;
  int64_t m_tile, n_tile;
  RunGroup rg;
  tile_coords<FOLD>(p, mt, L, m_tile, n_tile, rg);
  const int g = rg.g;
  const bool shared = g >= p.E;
  const int N = shared ? p.N_shared : p.N_routed;
  const int K = shared ? p.K_shared : p.K_routed;
  constexpr int NB = GATE_UP ? BN / 2 : BN;
  const int n0 = (int)n_tile * NB;
  if (n0 >= N) return;
  int64_t row0;
  int valid_rows;
  int extra;  // folded rows 256 .. 256 + extra - 1 (see tile_rows)
  tile_rows<FOLD>(p, rg, m_tile - rg.first, row0, valid_rows, extra);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ------------------------------------------------------ operand sources
  // B: wave `wave`, load j (0..7) writes LDS rows (wave*8 + j)*8 .. +7 of a
  // stage; A: load j of wave w writes rows (4 j + w)*8 .. +7, so a tile with
  // few rows needs only the first loads of each wave (see k_loop's NA).  Lane
  // i of a load carries row +i/8 and K-chunk (i%8) ^ swz(row).
  const __amdgpu_buffer_rsrc_t rsA =
      GATE_UP ? make_rsrc(p.A, (uint32_t)p.a_bytes)
              : make_rsrc(p.A + row0 * p.lda, (uint32_t)((BM + extra) * p.lda * 2));
  constexpr int EB = FP8 ? 1 : 2;  // bytes per weight
  const int64_t brows = (int64_t)(GATE_UP ? 2 : 1) * N;  // weight rows of this group
  const char* Bg = shared ? static_cast<const char*>(p.B_shared)
                          : static_cast<const char*>(p.B_routed) + (int64_t)g * brows * K * EB;
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(Bg, (uint32_t)(brows * K * EB));
  // weight row of B-tile row r (0..255), or -1 past the matrix
  auto b_weight_row = [&](int r) {
    if (GATE_UP) {
      const int half = r >> 7, f = n0 + (r & 127);
      return f < N ? half * N + f : -1;
    }
    return n0 + r < N ? n0 + r : -1;
  };
  uint32_t offA[8], offB[8];
  const int sub = lane >> 3;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (wave * 8 + j) * 8 + sub;  // 0..255 (B rows)
    const int kc = (lane & 7) ^ swz(r);
    const uint32_t kb = kc * 16;
    {
      // A: slot j of wave w loads 8-row block 4 j + w, so a tile with few
      // rows needs only its first slots in every wave
      const int ra = (j * 4 + wave) * 8 + sub;
      const uint32_t kba = ((lane & 7) ^ swz(ra)) * 16;
      if (GATE_UP) {
        const int t = ra < valid_rows ? p.row_token[row0 + ra] : -1;
        offA[j] = t >= 0 ? (uint32_t)t * (uint32_t)(p.lda * 2) + kba : kOob;
      } else {
        offA[j] = ra < valid_rows ? (uint32_t)ra * (uint32_t)(p.lda * 2) + kba : kOob;
      }
    }
    if constexpr (KMAJ) {
      // K-major B: load j writes k-rows 2 (wave*8 + j) and + 1 of a stage;
      // lane i carries k-row +i/32, chunk position i % 32 (see kmaj_chunk)
      const int kr = 2 * (wave * 8 + j) + (lane >> 5);
      const int n = n0 + 8 * kmaj_chunk(kr, lane & 31);
      offB[j] = n < N ? (uint32_t)kr * (uint32_t)(N * 2) + (uint32_t)n * 2 : kOob;
    } else if constexpr (!FP8) {
      const int wr = b_weight_row(r);
      offB[j] = wr >= 0 ? (uint32_t)wr * (uint32_t)(K * 2) + kb : kOob;
    } else if (j < 4) {
      // E4M3: load j writes 16 rows of 64 bytes; lane i carries row +i/4 and
      // 16-byte K chunk (i%4) ^ swz4(row)
      const int r8 = (wave * 4 + j) * 16 + (lane >> 2);
      const int wr = b_weight_row(r8);
      const uint32_t kb8 = ((lane & 3) ^ swz4(r8)) * 16;
      offB[j] = wr >= 0 ? (uint32_t)wr * (uint32_t)K + kb8 : kOob;
    }
  }
  const int kcl = (lane & 7);  // chunk position within the 8 of a row, before the swizzle

  // loads j in [j0, j1) of the A (or B) rows of K-stage `stage` into A (or B)
  // buffer `buf`; chunks at or past K (only in the last stage when
  // K % 64 != 0) read as zero.  An E4M3 chunk of 16 codes that straddles K
  // (K % 16 == 8) brings 8 codes past K, which meet zero A.
  auto issue = [&](bool isB, int stage, int buf, int j0, int j1) {
    const int k0 = stage * BK;
    const bool b8 = FP8 && isB;
    char* base = isB ? lds + 2 * kABytes + buf * b_stage_bytes<FP8>() : lds + buf * kABytes;
    const bool tail = KT && k0 + BK > K;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < j0 || j >= j1) continue;
      uint32_t o = isB ? offB[j] : offA[j];
      if (tail) {
        if (KMAJ && isB) {
          if (k0 + 2 * (wave * 8 + j) + (lane >> 5) >= K) o = kOob;
        } else if (b8) {
          const int r8 = (wave * 4 + j) * 16 + (lane >> 2);
          if (k0 + ((lane & 3) ^ swz4(r8)) * 16 >= K) o = kOob;
        } else {
          const int r = isB ? (wave * 8 + j) * 8 + sub : (j * 4 + wave) * 8 + sub;
          const int kc = kcl ^ swz(r);
          if (k0 + kc * 8 >= K) o = kOob;
        }
      }
      const int blk = b8 ? wave * 4 + j : isB ? wave * 8 + j : j * 4 + wave;  // 1-KB block of the stage
      // stage offset: k0 elements along each row, or (K-major B) k0 rows of N
      const uint32_t soff = isB ? (KMAJ ? (uint32_t)k0 * (uint32_t)(N * 2) : (uint32_t)(k0 * EB))
                                : (uint32_t)(k0 * 2);
      if constexpr (KMAJ)
        lds_dma16(isB ? rsB : rsA, base + blk * 1024, o, soff);
      else if (NTB && isB)  // cache policy 2: non-temporal
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void*)(base + blk * 1024), 16, o,
                                                 (int)soff, 0, 2);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isB ? rsB : rsA, (lds_void*)(base + blk * 1024), 16,
                                                 o, (int)soff, 0, 0);
    }
  };
  auto issue_a = [&](int stage, int buf, int j0, int j1) { issue(false, stage, buf, j0, j1); };
  auto issue_b = [&](int stage, int buf, int j0, int j1) { issue(true, stage, buf, j0, j1); };

  // active 32-row sub-tiles of this wave (uniform): the K loop is compiled
  // once per count so no MFMA sits under a branch
  const bool il = valid_rows < BM;
  const int act = il ? min(4, max(0, ((valid_rows + 31) / 32 - wm + 1) / 2))
                     : min(4, max(0, (valid_rows - wm * 128 + 31) / 32));
  const int lr = lane & 31, kh = lane >> 5;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  const int s0 = piece ? (int)((int64_t)part * nk / S) : 0;
  const int s1 = piece ? (int)((int64_t)(part + 1) * nk / S) : nk;
  // row tier of the tile (64-row steps): its A loads per wave per stage are
  // 2 tier, and a wave's active sub-tiles are tier or tier - 1
  const int tier = min(4, max(1, (valid_rows + 63) / 64));
  auto a_row = [&](int i) { return a_row_of(wm, i, il); };

  // ---------------------------------------------------------- after K loop
  // XRT: the tile holds folded rows (xr); the other tiles' code does not
  // carry them, so their registers and schedule stay as they were.
  auto finish = [&](auto xrt, ExtraRows* xr) {
    constexpr bool XRT = decltype(xrt)::value;
    // E4M3: every output column times the scale of its weight row
    if constexpr (FP8) {
      const float* Sg = shared ? p.S_shared : p.S_routed + (int64_t)g * brows;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int wr = b_weight_row(b_row_of<GATE_UP>(wn, j) + lr);
        const float sc = wr >= 0 ? Sg[wr] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i >= act) continue;
          acc[i][j] *= sc;
        }
      }
      if constexpr (XRT) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int wr = b_weight_row(b_row_of<GATE_UP>(wn, xblock<GATE_UP>(wm, h)) + lr);
          xr->acc[h] *= wr >= 0 ? Sg[wr] : 0.f;
        }
      }
    }

    // ---------------------------------------------- pieces of a split tile
    if (piece) {  // row-major fp32 partial tile, columns in LDS B-row order
      // one per-lane base offset; every store adds a compile-time byte offset,
      // so the 256 stores need no address registers
      const __amdgpu_buffer_rsrc_t rsP = make_rsrc(
          p.partial + (int64_t)(piece_tile * S + part) * (kTileRows * BN), kTileRows * BN * 4);
      const uint32_t vbase = (uint32_t)(((a_row(0) + 4 * kh) * BN + b_row_of<GATE_UP>(wn, 0) + lr) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= act) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int off = ((a_row(i) - a_row(0) + 8 * (r >> 2) + (r & 3)) * BN +
                             (b_row_of<GATE_UP>(0, j) - b_row_of<GATE_UP>(0, 0))) * 4;
            const float v = acc[i][j][r];  // a scalar first: bit_cast of a vector element
                                           // reinterprets the vector's first lane
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsP, vbase, off, 0);
          }
      }
      if constexpr (XRT) {  // folded rows: partial rows 256 .. 287
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t vx =
              (uint32_t)(((BM + 4 * kh) * BN + b_row_of<GATE_UP>(wn, xblock<GATE_UP>(wm, h)) + lr) * 4);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float v = xr->acc[h][r];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsP, vx,
                                                  (8 * (r >> 2) + (r & 3)) * BN * 4, 0);
          }
        }
      }
      return;
    }

    // ------------------------------------------------------------ epilogue
    if (GATE_UP && p.gu_out) {  // keep g and u (bf16) of the valid rows for the backward pass
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= act) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = a_row(i) + 8 * (r >> 2) + 4 * kh + (r & 3);
          if (row >= valid_rows) continue;
          bf16_t* gr = reinterpret_cast<bf16_t*>(p.gu_out) + (row0 + row) * p.ld_gu;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int f = n0 + wn * 64 + j * 32 + lr;
            if (f < N) {
              gr[f] = f32_to_bf16(acc[i][j][r]);
              gr[N + f] = f32_to_bf16(acc[i][j + 2][r]);
            }
          }
        }
      }
      if constexpr (XRT) {  // folded rows: gate and up of column block wm of this wave's half
        const int f = n0 + wn * 64 + wm * 32 + lr;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = BM + 8 * (r >> 2) + 4 * kh + (r & 3);
          if (row >= BM + extra || f >= N) continue;
          bf16_t* gr = reinterpret_cast<bf16_t*>(p.gu_out) + (row0 + row) * p.ld_gu;
          gr[f] = f32_to_bf16(xr->acc[0][r]);
          gr[N + f] = f32_to_bf16(xr->acc[1][r]);
        }
      }
    }
    if (GATE_UP) {
      // SwiGLU in registers, h stored from registers as bf16 pairs (measured
      // 1.5-2% faster for the whole gate/up kernel than staging the fp32 tile
      // through LDS for 16-byte stores).  Register r of lane l holds row
      // 8 (r / 4) + 4 kh + r % 4, column l % 32 of its 32 x 32 block; for the
      // register pair (2q, 2q + 1) (rows R, R + 1) the even lane stores row R,
      // columns c, c + 1 and the odd lane row R + 1, columns c - 1, c, after
      // swapping one value (DPP quad permutation 1 0 3 2).  Rows past the
      // tile's count (padding, or the next m-tile's) are not stored; the
      // folded rows (gate and up of column block wm of the wave's half) alike.
      const int rows = XRT ? BM + extra : valid_rows;
      const __amdgpu_buffer_rsrc_t rsH = make_rsrc(reinterpret_cast<bf16_t*>(p.C) + row0 * p.ldc,
                                                  (uint32_t)((XRT ? BM + extra : BM) * p.ldc * 2));
      const bool odd = lane & 1;
      auto store_pair = [&](float g0, float u0, float g1, float u1, int row, int col) {
        const float h0 = silu(g0) * u0;
        const float h1 = silu(g1) * u1;
        const float send = odd ? h0 : h1;
        const float got = __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xB1, 0xF, 0xF, false));
        const float lo = odd ? got : h0, hi = odd ? h1 : got;
        const uint32_t v = (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
        const uint32_t off = (row < rows && col < N) ? (uint32_t)((row * p.ldc + col) * 2) : kOob;
        __builtin_amdgcn_raw_buffer_store_b32(v, rsH, off, 0, 0);
      };
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= act) continue;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = 2 * q + (odd ? 1 : 0);
          const int row = a_row(i) + 8 * (r >> 2) + 4 * kh + (r & 3);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            store_pair(acc[i][j][2 * q], acc[i][j + 2][2 * q], acc[i][j][2 * q + 1],
                       acc[i][j + 2][2 * q + 1], row, n0 + wn * 64 + j * 32 + (lr & ~1));
        }
      }
      if constexpr (XRT) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int r = 2 * q + (odd ? 1 : 0);
          store_pair(xr->acc[0][2 * q], xr->acc[1][2 * q], xr->acc[0][2 * q + 1], xr->acc[1][2 * q + 1],
                     BM + 8 * (r >> 2) + 4 * kh + (r & 3), n0 + wn * 64 + wm * 32 + (lr & ~1));
        }
      }
      return;
    }
    // fp32 rows of the tile through buffer stores: the row of register r is
    // wave-uniform and goes in the scalar offset, the lane's column (and its
    // 4-row half) in the vector offset, so no store needs a 64-bit address.
    // The scalar offset is outside the hardware's range check, so a tile with
    // rows past its count (the group's last) drops those rows through the
    // vector offset; full tiles take the same loop with the check folded away.
    {
      const __amdgpu_buffer_rsrc_t rsY =
          make_rsrc(reinterpret_cast<float*>(p.C) + row0 * p.ldc,
                    (uint32_t)((int64_t)(XRT ? valid_rows + extra : valid_rows) * p.ldc * 4));
      uint32_t voff[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 128 + j * 32 + lr;
        voff[j] = n < N ? (uint32_t)((4 * kh * p.ldc + n) * 4) : kOob;
      }
      auto store_rows = [&](const bool check) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i >= act) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rb = a_row(i) + 8 * (r >> 2) + (r & 3);
            const uint32_t soff = (uint32_t)(rb * p.ldc * 4);
            const bool ok = !check || rb + 4 * kh < valid_rows;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float v = acc[i][j][r];  // a scalar first (see the pieces' stores)
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsY,
                                                    ok ? voff[j] : kOob, soff, 0);
            }
          }
        }
      };
      if (valid_rows >= BM)
        store_rows(false);
      else
        store_rows(true);
      if constexpr (XRT) {  // folded rows: column blocks 2 wm, 2 wm + 1 of this wave's half
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t vo = wm ? voff[xblock<GATE_UP>(1, h)] : voff[xblock<GATE_UP>(0, h)];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rb = BM + 8 * (r >> 2) + (r & 3);
            const float v = xr->acc[h][r];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsY,
                                                  rb + 4 * kh < BM + extra ? vo : kOob,
                                                  (uint32_t)(rb * p.ldc * 4), 0);
          }
        }
      }
    }
  };
  if constexpr (FOLD) {
    if (extra > 0) {  // a full tile with folded rows (see tile_rows); this lane's is row 256 + lane % 32
      ExtraRows xr;
      xr.rs = rsA;
      xr.K = K;
      if (GATE_UP) {
        const int t = lr < extra ? p.row_token[row0 + BM + lr] : -1;
        xr.off = t >= 0 ? (uint32_t)t * (uint32_t)(p.lda * 2) : kOob;
      } else {
        xr.off = lr < extra ? (uint32_t)(BM + lr) * (uint32_t)(p.lda * 2) : kOob;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) xr.acc[h][r] = 0.f;
      // one copy of the loop per wave row (a wave-uniform branch)
      if (wm == 0)
        k_loop<GATE_UP, 4, FP8, decltype(issue_a), decltype(issue_b), false, false, false, 8, true, 0>(
            lds, s0, s1 - s0, wm, wn, il, lane, issue_a, issue_b, acc, &xr);
      else
        k_loop<GATE_UP, 4, FP8, decltype(issue_a), decltype(issue_b), false, false, false, 8, true, 1>(
            lds, s0, s1 - s0, wm, wn, il, lane, issue_a, issue_b, acc, &xr);
      finish(std::true_type{}, &xr);
      return;
    }
  }
#define MOE_KL(A_, N_)                                                                            \
  k_loop<GATE_UP, A_, FP8, decltype(issue_a), decltype(issue_b), KMAJ, false, false, N_>(         \
      lds, s0, s1 - s0, wm, wn, il, lane, issue_a, issue_b, acc)
  switch (tier * 8 + act) {
    case 4 * 8 + 4: MOE_KL(4, 8); break;
    case 4 * 8 + 3: MOE_KL(3, 8); break;
    case 3 * 8 + 3: MOE_KL(3, 6); break;
    case 3 * 8 + 2: MOE_KL(2, 6); break;
    case 2 * 8 + 2: MOE_KL(2, 4); break;
    case 2 * 8 + 1: MOE_KL(1, 4); break;
    case 1 * 8 + 1: MOE_KL(1, 2); break;
    default: MOE_KL(0, 2); break;
  }
#undef MOE_KL
  finish(std::false_type{}, nullptr);
}

template <bool FP8, bool KT, bool NTB>
__global__ __launch_bounds__(256) void moe_gemm_gate_up_prefill_kernel(GroupedGemm p) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  prefill_tile<true, FP8, false, KT, NTB>(p, lds);
}

template <bool FP8, bool KT>
__global__ __launch_bounds__(256) void moe_gemm_down_prefill_kernel(GroupedGemm p) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  prefill_tile<false, FP8, false, KT>(p, lds);
}

// rows x weight with the weight stored K-major ([K][N] per group): the
// backward pass's products with W_down and W_gate_up read in their own layout
__global__ __launch_bounds__(256) void moe_gemm_rows_kmajor_prefill_kernel(GroupedGemm p) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  prefill_tile<false, false, true>(p, lds);
}

// Finishes the cut tiles of the last round: block b owns rows
// 16*(b % 16) .. +15 of cut tile b / 16, adds the S partials of each output
// in K order (piece 0 first) and runs the GEMM's epilogue on the valid rows
// (gate/up: SwiGLU into H; down: rows of Yp).  All S loads of an output are
// issued before the sum, so the kernel streams instead of waiting on each.
constexpr int kFixRows = 16;
constexpr int kFixBlocksPerTile = kTileRows / kFixRows;

template <bool GATE_UP, bool FOLD>
__device__ __forceinline__ void fixup_tiles(const GroupedGemm& p) {
  const int64_t mt = mtiles_of<FOLD>(p);
  const Split sp = split_of(p, mt);
  const int64_t t = blockIdx.x / kFixBlocksPerTile;
  if (t >= sp.R) return;
  int64_t m_tile, n_tile;
  RunGroup rg;
  tile_coords<FOLD>(p, mt, sp.n_dp + t, m_tile, n_tile, rg);
  const int g = rg.g;
  const int N = g >= p.E ? p.N_shared : p.N_routed;
  constexpr int NB = GATE_UP ? BN / 2 : BN;  // output columns of a tile
  const int n0 = (int)n_tile * NB;
  if (n0 >= N) return;
  int64_t row0;
  int valid_rows, extra;
  tile_rows<FOLD>(p, rg, m_tile - rg.first, row0, valid_rows, extra);
  const int r0 = (blockIdx.x % kFixBlocksPerTile) * kFixRows;
  const int r1 = min(r0 + kFixRows, valid_rows + extra);  // folded rows included
  const float* P = p.partial + t * sp.S * (kTileRows * BN);
  constexpr int Q = NB / 4;  // float4 outputs per row
  // sum of the S partials of the float4 at (row, col), in piece order
  auto sum4 = [&](int row, int col) {
    float4 v[kMaxSplit];
#pragma unroll
    for (int q = 0; q < kMaxSplit; ++q)
      if (q < sp.S)
        v[q] = *reinterpret_cast<const float4*>(P + (int64_t)q * (kTileRows * BN) + row * BN + col);
    float4 a = v[0];
#pragma unroll
    for (int q = 1; q < kMaxSplit; ++q)
      if (q < sp.S) {
        a.x += v[q].x;
        a.y += v[q].y;
        a.z += v[q].z;
        a.w += v[q].w;
      }
    return a;
  };
  for (int e = threadIdx.x; e < (r1 - r0) * Q; e += blockDim.x) {
    const int row = r0 + e / Q, c = (e % Q) * 4;
    if (GATE_UP) {
      // LDS B-row order of a gate/up tile: gate columns 0..127, up columns 128..255
      const float4 gt = sum4(row, c), up = sum4(row, BN / 2 + c);
      const float h[4] = {silu(gt.x) * up.x, silu(gt.y) * up.y, silu(gt.z) * up.z, silu(gt.w) * up.w};
      bf16_t* H = reinterpret_cast<bf16_t*>(p.C) + (row0 + row) * p.ldc + n0 + c;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (n0 + c + u < N) H[u] = f32_to_bf16(h[u]);
      if (p.gu_out) {  // g and u kept for the backward pass
        const float g4[4] = {gt.x, gt.y, gt.z, gt.w}, u4[4] = {up.x, up.y, up.z, up.w};
        bf16_t* gr = reinterpret_cast<bf16_t*>(p.gu_out) + (row0 + row) * p.ld_gu;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (n0 + c + u < N) {
            gr[n0 + c + u] = f32_to_bf16(g4[u]);
            gr[N + n0 + c + u] = f32_to_bf16(u4[u]);
          }
      }
    } else {
      const float4 v = sum4(row, c);
      float* Y = reinterpret_cast<float*>(p.C) + (row0 + row) * p.ldc + n0 + c;
      const float y[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (n0 + c + u < N) Y[u] = y[u];
    }
  }
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) void moe_gemm_split_fixup_kernel(GroupedGemm p) {
  if (p.b_kmajor || p.fp8)
    fixup_tiles<GATE_UP, false>(p);  // the K-major and E4M3 kernels' m-tiles do not fold
  else
    fixup_tiles<GATE_UP, true>(p);
}

template <bool FP8, bool KT>
hipError_t launch_fmt(bool gate_up, GroupedGemm g, hipStream_t s) {
  constexpr int lds = lds_bytes<FP8>();
  // set once per process (a function-local static is initialised thread-safely)
  static const hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute((const void*)moe_gemm_gate_up_prefill_kernel<FP8, KT, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)moe_gemm_gate_up_prefill_kernel<FP8, KT, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)moe_gemm_down_prefill_kernel<FP8, KT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess && !FP8)
      e = hipFuncSetAttribute((const void*)moe_gemm_rows_kmajor_prefill_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  const int nmax = g.N_routed > g.N_shared ? g.N_routed : g.N_shared;
  const int NB = gate_up ? BN / 2 : BN;
  g.n_tiles_n = (nmax + NB - 1) / NB;
  // No split (and no second kernel) when the device could never choose one:
  // too many tiles for any routing, or K too short to cut.  With ids outside
  // [0, E) the bound may overstate the tiles; that only forgoes the split.
  {
    const int kmin = g.B_shared && g.K_shared < g.K_routed ? g.K_shared : g.K_routed;
    const bool short_k = ((kmin + BK - 1) / BK) / kMinPieceStages < 2;
    if (short_k || g.min_tiles * g.n_tiles_n >= (int64_t)kSplitRounds * g.ctas) g.ctas = 0;
  }
  // enough workgroups for every XCD's run plus the pieces of a split last
  // round (at most ctas of them; see prefill_tile)
  const int64_t blocks = (g.max_tiles * g.n_tiles_n + 7) / 8 * 8 + (g.ctas > 0 ? g.ctas : 0);
  if (blocks == 0) return hipSuccess;
  if (gate_up && g.stream_b)
    hipLaunchKernelGGL((moe_gemm_gate_up_prefill_kernel<FP8, KT, true>), dim3((unsigned)blocks),
                       dim3(256), lds, s, g);
  else if (gate_up)
    hipLaunchKernelGGL((moe_gemm_gate_up_prefill_kernel<FP8, KT, false>), dim3((unsigned)blocks),
                       dim3(256), lds, s, g);
  else if (g.b_kmajor)
    hipLaunchKernelGGL(moe_gemm_rows_kmajor_prefill_kernel, dim3((unsigned)blocks), dim3(256), lds,
                       s, g);
  else
    hipLaunchKernelGGL((moe_gemm_down_prefill_kernel<FP8, KT>), dim3((unsigned)blocks), dim3(256), lds,
                       s, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.ctas <= 0) return e;
  const unsigned fix_blocks = (unsigned)g.ctas * kFixBlocksPerTile;
  if (gate_up)
    hipLaunchKernelGGL(moe_gemm_split_fixup_kernel<true>, dim3(fix_blocks), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(moe_gemm_split_fixup_kernel<false>, dim3(fix_blocks), dim3(256), 0, s, g);
  return hipGetLastError();
}

hipError_t launch(bool gate_up, const GroupedGemm& g, hipStream_t s) {
  if (g.b_kmajor && (gate_up || g.fp8)) return hipErrorInvalidValue;  // no such variant
  // a K of some group that ends inside a 64-wide K-stage needs the masked loads
  const bool kt = g.K_routed % BK != 0 || (g.B_shared && g.K_shared % BK != 0);
  if (g.fp8)
    return kt ? launch_fmt<true, true>(gate_up, g, s) : launch_fmt<true, false>(gate_up, g, s);
  return kt ? launch_fmt<false, true>(gate_up, g, s) : launch_fmt<false, false>(gate_up, g, s);
}

// One tile of a weight gradient: its group, corner and row count.
struct WgradTile {
  int g, M, N, m0, n0, K;
  int64_t k0g;  // the group's first row
  float* C;
  bool valid;   // the tile's corner lies inside its group's matrix
};

__device__ __forceinline__ WgradTile wgrad_tile(const WgradGemm& p, int64_t t) {
  const int64_t per_group = p.tiles_m * p.tiles_n;
  WgradTile w;
  w.g = (int)(t / per_group);
  const int64_t rem = t - (int64_t)w.g * per_group;
  const int mt = (int)(rem / p.tiles_n), nt = (int)(rem % p.tiles_n);
  const bool shared = w.g >= p.E;
  w.M = shared ? p.M_shared : p.M_routed;
  w.N = shared ? p.N_shared : p.N_routed;
  w.m0 = mt * BM;
  w.n0 = nt * BN;
  w.valid = w.m0 < w.M && w.n0 < w.N;
  w.C = shared ? p.C_shared : p.C_routed + (int64_t)w.g * w.M * w.N;
  // uniform across the workgroup: they feed the loads' scalar descriptors
  w.k0g = __builtin_amdgcn_readfirstlane(p.padded[w.g]);
  w.K = __builtin_amdgcn_readfirstlane(p.counts[w.g]);
  return w;
}

// Issues K stage `stage` of tile w into LDS buffer `buf` (A at buf * kABytes,
// B at 2 kABytes + buf * kBBytes), the part of load slots j0 .. j1 - 1 of
// each wave: load j of a wave writes k-rows 2 (wave*8 + j) and + 1 of a
// stage; lane i carries k-row +i/32 and chunk position i % 32 (see
// kmaj_chunk).  Only the group's rows are addressable, so reads past them
// (the K tail) return zeros.
__device__ __forceinline__ void wgrad_issue(const WgradGemm& p, const WgradTile& w, char* lds, bool isB,
                                            int stage, int buf, int j0, int j1, int wave, int lane) {
  const int64_t ld = isB ? p.ldb : p.lda;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc((isB ? p.B : p.A) + w.k0g * ld, (uint32_t)((int64_t)w.K * ld * 2));
  const int lim = isB ? w.N : w.M, c0 = isB ? w.n0 : w.m0;
  const int k0 = stage * BK;
  char* base = isB ? lds + 2 * kABytes + buf * kBBytes : lds + buf * kABytes;
  const uint32_t soff = (uint32_t)k0 * (uint32_t)(ld * 2);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < j0 || j >= j1) continue;
    const int kr = 2 * (wave * 8 + j) + (lane >> 5);
    const int c8 = 8 * kmaj_chunk(kr, lane & 31);
    const uint32_t off = c0 + c8 < lim ? (uint32_t)kr * (uint32_t)(ld * 2) + (uint32_t)(c0 + c8) * 2 : kOob;
    lds_dma16(rs, base + (wave * 8 + j) * 1024, off, soff);
  }
}

// The tile's fp32 rows through buffer stores, as the down GEMM's epilogue:
// the wave-uniform row offset in the scalar offset, the lane's column (and
// 4-row half) in the vector offset, and rows past the matrix dropped through
// an out-of-range vector offset (the scalar offset is not range-checked).
__device__ __forceinline__ void wgrad_store(const WgradTile& w, int wm, int wn, int lane,
                                            const f32x16 (&acc)[4][4]) {
  const int lr = lane & 31, kh = lane >> 5;
  const int rows = w.M - w.m0 < BM ? w.M - w.m0 : BM;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(w.C + (int64_t)w.m0 * w.N, (uint32_t)((int64_t)rows * w.N * 4));
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = w.n0 + b_row_of<false>(wn, j) + lr;
    voff[j] = n < w.N ? (uint32_t)((4 * kh * w.N + n) * 4) : kOob;
  }
  auto store_rows = [&](const bool check) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rb = a_row_of(wm, i, false) + 8 * (r >> 2) + (r & 3);
        const uint32_t soff = (uint32_t)(rb * w.N * 4);
        const bool ok = !check || rb + 4 * kh < rows;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = acc[i][j][r];  // a scalar first (see the pieces' stores)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs,
                                                ok ? voff[j] : kOob, soff, 0);
        }
      }
  };
  if (rows >= BM)
    store_rows(false);
  else
    store_rows(true);
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// ------------------------------------------------------------ weight gradients
// Group g: C_g[m][n] = sum_r A[r][m] * B[r][n] over the group's rows
// r = padded[g] .. padded[g] + counts[g] - 1 (read on the device), with the
// same 256 x 256 x 64 tiles and K loop as the forward.  A and B are per-row
// buffers as the layer stores them (row r: its M, resp. N, values), read
// K-major (the rows are the reduction): both operands through the
// transposing LDS reads, the loads written out (see lds_dma16).  A group with
// no rows stores zeros.
__global__ __launch_bounds__(256) void moe_gemm_wgrad_kernel(WgradGemm p) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const WgradTile w = wgrad_tile(p, blockIdx.x);
  if (!w.valid) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[4][4];
  zero_acc(acc);
  if (w.K > 0) {
    // the group's rows only: reads past them (the K tail) return zeros
    const __amdgpu_buffer_rsrc_t rsA =
        make_rsrc(p.A + w.k0g * p.lda, (uint32_t)((int64_t)w.K * p.lda * 2));
    const __amdgpu_buffer_rsrc_t rsB =
        make_rsrc(p.B + w.k0g * p.ldb, (uint32_t)((int64_t)w.K * p.ldb * 2));
    // load slots as in wgrad_issue, their offsets computed once
    uint32_t offA[8], offB[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kr = 2 * (wave * 8 + j) + (lane >> 5);
      const int c8 = 8 * kmaj_chunk(kr, lane & 31);
      offA[j] = w.m0 + c8 < w.M ? (uint32_t)kr * (uint32_t)(p.lda * 2) + (uint32_t)(w.m0 + c8) * 2 : kOob;
      offB[j] = w.n0 + c8 < w.N ? (uint32_t)kr * (uint32_t)(p.ldb * 2) + (uint32_t)(w.n0 + c8) * 2 : kOob;
    }
    auto issue = [&](bool isB, int stage, int buf, int j0, int j1) {
      const int k0 = stage * BK;
      char* base = isB ? lds + 2 * kABytes + buf * kBBytes : lds + buf * kABytes;
      const uint32_t soff = (uint32_t)k0 * (uint32_t)((isB ? p.ldb : p.lda) * 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < j0 || j >= j1) continue;
        lds_dma16(isB ? rsB : rsA, base + (wave * 8 + j) * 1024, isB ? offB[j] : offA[j], soff);
      }
    };
    auto issue_a = [&](int stage, int buf, int j0, int j1) { issue(false, stage, buf, j0, j1); };
    auto issue_b = [&](int stage, int buf, int j0, int j1) { issue(true, stage, buf, j0, j1); };
    k_loop<false, 4, false, decltype(issue_a), decltype(issue_b), true, true>(
        lds, 0, (w.K + BK - 1) / BK, wm, wn, false, lane, issue_a, issue_b, acc);
  }
  wgrad_store(w, wm, wn, lane, acc);
}

// The same products when every group has at most 64 rows (a token picks an
// expert once, so T <= 64 guarantees it): one K stage per tile.  With 256
// accumulators per lane a CU runs one workgroup, which would wait for each
// tile's loads with nothing else to do; here a workgroup walks tiles
// blockIdx.x, + gridDim.x, ... and issues the next tile's stage into the other
// LDS buffer before storing the current tile, so the loads fly under the
// stores.
__global__ __launch_bounds__(256) void moe_gemm_wgrad_one_stage_kernel(WgradGemm p) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  const int64_t total = (int64_t)p.G * p.tiles_m * p.tiles_n;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  auto no_issue = [](int, int, int, int) {};
  f32x16 acc[4][4];
  int64_t t = blockIdx.x;
  int buf = 0;
  if (t < total) {
    const WgradTile w = wgrad_tile(p, t);
    if (w.valid && w.K > 0) {
      wgrad_issue(p, w, lds, false, 0, 0, 0, 8, wave, lane);
      wgrad_issue(p, w, lds, true, 0, 0, 0, 8, wave, lane);
    }
  }
  for (; t < total; t += gridDim.x) {
    const WgradTile w = wgrad_tile(p, t);
    zero_acc(acc);
    if (w.valid && w.K > 0)  // its stage is in buffer buf (issued one tile earlier)
      k_loop<false, 4, false, decltype(no_issue), decltype(no_issue), true, true, true>(
          lds + buf * kABytes, 0, 1, wm, wn, false, lane, no_issue, no_issue, acc);
    // every wave is done reading this tile's stage (and the one before, in
    // the other buffer) before the next tile's loads go there
    __syncthreads();
    const int64_t tn = t + gridDim.x;
    if (tn < total) {
      const WgradTile wn_ = wgrad_tile(p, tn);
      if (wn_.valid && wn_.K > 0) {
        wgrad_issue(p, wn_, lds, false, 0, buf ^ 1, 0, 8, wave, lane);
        wgrad_issue(p, wn_, lds, true, 0, buf ^ 1, 0, 8, wave, lane);
      }
    }
    if (w.valid) wgrad_store(w, wm, wn, lane, acc);
    buf ^= 1;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no load may still be writing LDS at exit
}

}  // namespace

hipError_t launch_gemm_wgrad(const WgradGemm& g, hipStream_t s) {
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)moe_gemm_wgrad_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (attr != hipSuccess) return attr;
  static const hipError_t attr1 =
      hipFuncSetAttribute((const void*)moe_gemm_wgrad_one_stage_kernel,
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (attr1 != hipSuccess) return attr1;
  const int64_t blocks = (int64_t)g.G * g.tiles_m * g.tiles_n;
  if (blocks == 0) return hipSuccess;
  if (g.one_stage_ctas > 0) {
    const int64_t grid = blocks < g.one_stage_ctas ? blocks : g.one_stage_ctas;
    hipLaunchKernelGGL(moe_gemm_wgrad_one_stage_kernel, dim3((unsigned)grid), dim3(256), kLdsBytes, s,
                       g);
  } else {
    hipLaunchKernelGGL(moe_gemm_wgrad_kernel, dim3((unsigned)blocks), dim3(256), kLdsBytes, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up_prefill(const GroupedGemm& g, hipStream_t s) {
  return launch(true, g, s);
}

hipError_t launch_gemm_down_prefill(const GroupedGemm& g, hipStream_t s) {
  return launch(false, g, s);
}

}  // namespace moe
