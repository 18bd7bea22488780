// Device-side types and helpers for the gfx950 (CDNA4) kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).  Lane l supplies row l%32
// of A and column l%32 of B, eight consecutive k each (k block l/32).  The
// result: register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32) * B(32x16).  Lane l supplies row l%16 of A and
// column l%16 of B, eight consecutive k each (k block l/16).  Register r of
// lane l is row 4*(l/16) + r, column l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);  // round to nearest even
}

// SiLU(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (each about
// 1 ulp in fp32); the result is rounded to bf16 right after, 2^16 times coarser.
__device__ __forceinline__ float silu(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// One 16-byte-per-lane buffer load into LDS (lane i writes bytes 16 i ..
// 16 i + 15 of the 1-KB block at `dst`), written out for the kernels that
// read B with the transposing LDS read: the compiler makes such a read wait
// for every LDS load it knows to be in flight (vmcnt(0), which would drain
// the prefetch of the coming stages), while the K loop's own waits and
// barriers already order these loads before the reads of their stage.
// NT: the non-temporal cache policy, for data read once (streamed expert
// weights): the same read-only stream measured 6.2 TB/s with plain loads and
// 7.0 TB/s with non-temporal ones on MI355X.
template <bool NT = false>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, const char* dst, uint32_t voff,
                                          uint32_t soff) {
  // M0 (the LDS base of the load) is saved and restored around it
  const uint32_t lds_addr = (uint32_t)(uintptr_t)dst;  // low bits of the generic pointer
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
        : "memory");
}

}  // namespace moe
