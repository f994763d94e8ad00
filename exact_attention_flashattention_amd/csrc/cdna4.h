// Small CDNA4 (gfx950) building blocks shared by the attention kernels:
// vector types, the bf16 32x32x16 MFMA, bf16 packing, lane-half reductions,
// the LDS chunk swizzle, HBM -> LDS copies and explicit vmcnt waits.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {
namespace cdna4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2_t));
}

// lo + hi + acc for a packed pair of bf16 values (exact products with 1.0)
__device__ __forceinline__ float add_bf16x2(unsigned pk, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk),
                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}

// Reductions across the two lane halves (lane l with lane l ^ 32):
// v_permlane32_swap(x, x) returns (x of lanes 0-31 in both halves,
// x of lanes 32-63 in both halves).
__device__ __forceinline__ float halves_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Physical 16-byte chunk position of logical chunk c in row r is c ^ swz(r).
// For 16 chunks per row swz is a bijection on every 16 consecutive rows (K
// reads: 16 lanes, 16 rows, one chunk) and maps 4 consecutive rows to values
// differing in bits 2-3 (transposed V reads: 4 rows x 2 adjacent chunks).
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 16)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return ((r & 3) << 1) | ((r >> 2) & 1);
}

// cache-policy bit of a non-temporal access (the SLC position on CDNA3/4)
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void load_to_lds(const void* g, unsigned char* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
// the same copy with the non-temporal cache policy, for data read once
__device__ __forceinline__ void load_to_lds_stream(const void* g, unsigned char* l) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, kCachePolicyNT);
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding)
template <int NCNT>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(NCNT >= 0 && NCNT < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((NCNT & 15) | ((NCNT >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(n) with the other counters left alone
template <int NCNT>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(NCNT >= 0 && NCNT < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (NCNT << 8));
}

// Work-group barrier without the release/acquire fences of __syncthreads():
// those fences make the compiler wait for every HBM -> LDS copy in flight
// (vmcnt(0)) at each barrier, which would drain a ring of prefetched tiles.
// The caller waits explicitly for what must be complete (its own copies of
// the tiles about to be read, its own LDS reads of buffers about to be
// overwritten). The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// Work-group id -> work item such that each of the 8 XCDs (which receive
// consecutive ids round-robin) gets one contiguous range of items.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  return xcd * q8 + min(xcd, r8) + slot;
}

}  // namespace cdna4
}  // namespace attn
