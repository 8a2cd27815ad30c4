// Shared device helpers for the MI355X (gfx950) kernels: bf16 bit handling,
// MFMA operand types, sortable float keys and the internal launcher API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte copy unit

// bf16 is carried as its 16-bit pattern in memory.
__device__ __forceinline__ float bf16_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float -> bf16 with the hardware conversion (v_cvt_pk_bf16_f32: round to
// nearest even, NaN stays NaN), two at a time.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Order-preserving map of a float to uint32 (larger float -> larger key).
// -0.0 is folded into +0.0 first.
__device__ __forceinline__ uint32_t sortable_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float sigmoidf_(float z) {
  return 1.0f / (1.0f + expf(-z));
}

// Wavefront-wide shuffle of 64-bit values (wave64).
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, mask, 64);
  hi = __shfl_xor(hi, mask, 64);
  return ((uint64_t)hi << 32) | lo;
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// ---- LDS operand slabs shared by the MFMA kernels -------------------------
// A slab row is 64 bf16 (128 bytes = 8 chunks of 16 B); chunk c of row r is
// stored at chunk c ^ (r & 7), so 16 rows read at one logical chunk (the
// operand of one v_mfma_f32_16x16x32_bf16) fall in distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) {  // bf16 element offset
  return row * 64 + ((chunk ^ (row & 7)) << 3);
}

#define MOE_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Workgroup barrier that orders LDS accesses in the compiler but does not wait
// for outstanding global loads; callers wait for exactly what they need first.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0], expcnt[6:4] = 7
// i.e. no wait, lgkmcnt[11:8], vmcnt high bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) only (vmcnt 63 = no wait on vector memory).
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
}

// One direct-to-LDS load of 8 whole slab rows (1 KB): lane l writes LDS bytes
// 16*l (row l/8, stored chunk l%8), so it must fetch logical chunk
// (l%8) ^ (l/8) of its row; 8 lanes cover one full 128-byte line.
__device__ __forceinline__ int dma_row(int lane) { return lane >> 3; }
__device__ __forceinline__ int dma_chunk(int lane) { return (lane & 7) ^ (lane >> 3); }
__device__ __forceinline__ void dma_rows(const uint16_t* src, uint16_t* lds_group) {
  __builtin_amdgcn_global_load_lds((const void*)src, MOE_LDS_PTR(lds_group), 16, 0, 0);
}

}  // namespace moe
