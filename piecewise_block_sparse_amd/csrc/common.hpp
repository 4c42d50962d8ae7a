// Device helpers shared by the gfx950 kernels of libpisa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace pisa {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// D[32x32] += A[32x16] * B[16x32], bf16 operands, fp32 accumulate.
// Lane l holds A[l % 32][8 (l / 32) + e] and B[8 (l / 32) + e][l % 32], e = 0..7;
// result register r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ void st8(void* p, const u32x2& v) {
  *reinterpret_cast<u32x2*>(p) = v;
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// two fp32 -> packed bf16 pair (round to nearest even), lo in bits 0..15
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  bf16x2 v = {(bf16)lo, (bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

// Workgroups are dealt round-robin over the 8 XCDs (id % 8).  Map them so that
// every XCD walks one contiguous range of logical ids; neighbouring query
// blocks of a head then share that XCD's L2.  Bijective for any grid size.
__device__ __forceinline__ int xcd_remap(int wg, int grid) {
  const int x = wg & 7, slot = wg >> 3, q = grid >> 3, r = grid & 7;
  return x * q + (x < r ? x : r) + slot;
}

// Orders one wave's own LDS accesses among its lanes (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Valid length of the sequence of (batch * heads) row bh: lens[bh / heads]
// clamped to [0, L], or L when no lengths are given.
__device__ __forceinline__ int valid_len(const int32_t* lens, int bh, int heads, int L) {
  if (!lens) return L;
  const int v = lens[bh / heads];
  return v < 0 ? 0 : (v > L ? L : v);
}

// tokens of block j that lie inside a sequence of Lv valid tokens
__device__ __forceinline__ int block_count(int Lv, int j, int BLK) {
  const int n = Lv - j * BLK;
  return n < 0 ? 0 : (n > BLK ? BLK : n);
}

}  // namespace pisa
