// Streaming row-major bf16 chunks through LDS on gfx950, shared by the
// attention and block-statistics kernels.
//
// A chunk is CK rows (tokens) of D bf16 values; a ring stage holds a K chunk
// (bytes [0, SUBB)) followed by a V chunk ([SUBB, 2 SUBB)).  Chunks are copied
// global -> LDS by global_load_lds_dwordx4 (no registers, no staging ALU),
// row-major, with the 16-byte slots of row r XOR-swizzled by swz(r) so that
// row reads (16 rows, one column each) and transposing reads
// (ds_read_b64_tr_b16) are both free of bank conflicts.
//
// The helpers take a configuration type C with the fields
//   D     row length (bf16 values)       RB   bytes per row (2 D)
//   CPR   16-byte slots per row (D / 8)  SUBB bytes of one K (or V) chunk
//   DPW   1 KB copies per wave and stage RPD  rows per 1 KB copy
#pragma once

#include "common.hpp"

namespace pisa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lvoid;
typedef __attribute__((address_space(3))) s16x4 ls16x4;

// 16-byte slot of logical column chunk c in row r is c ^ swz(r).
template <int D>
__device__ __forceinline__ int swz(int r) {
  return (D == 128) ? (4 * (r & 3) + ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
}

// Copies global -> LDS with global_load_lds_dwordx4: lane l copies 16 bytes
// from gbase + voff(l) + imm into LDS at m0 + imm + 16 l (the immediate offset
// moves both addresses).  Issued from asm so the compiler does not track the
// copies: it neither orders later LDS reads of another ring stage behind them
// nor waits on them; every use of a stage is preceded by a wait for its copies
// and a workgroup barrier instead.  The instructions have no register result.
//
// Each chunk is split in 1 KB pieces of RPD rows.  Wave w copies pieces
// w H .. w H + H - 1 of each half (H = DPW / 2), so one scalar base and one M0
// serve a half and the pieces follow as immediates 0, 1024, ...  Lane l writes
// slot l % CPR of row RPD n + l / CPR of piece n; that slot holds logical
// column chunk (l % CPR) ^ swz(row), so the lane's global offset within the
// wave's piece u is fixed for the whole kernel (H registers per lane).
template <class C>
struct DmaOff {
  unsigned v[C::DPW / 2];
};

template <class C>
__device__ __forceinline__ DmaOff<C> dma_lane_offsets(int w, int lane) {
  DmaOff<C> o;
#pragma unroll
  for (int u = 0; u < C::DPW / 2; ++u) {
    const int r = (w * (C::DPW / 2) + u) * C::RPD + lane / C::CPR;
    o.v[u] = 2u * ((lane / C::CPR) * C::D + 8 * ((lane % C::CPR) ^ swz<C::D>(r)));
  }
  return o;
}

// H consecutive 1 KB pieces: global gbase + 1024 u, LDS m0v + 1024 u
template <class C>
__device__ __forceinline__ void dma_half(const void* gbase, unsigned m0v, const DmaOff<C>& o) {
  if constexpr (C::DPW / 2 == 4) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
        "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
        "global_load_lds_dwordx4 %4, %5 offset:3072"
        :
        : "s"(m0v), "v"(o.v[0]), "v"(o.v[1]), "v"(o.v[2]), "v"(o.v[3]), "s"(gbase)
        : "memory", "m0");
  } else if constexpr (C::DPW / 2 == 2) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "global_load_lds_dwordx4 %2, %3 offset:1024"
        :
        : "s"(m0v), "v"(o.v[0]), "v"(o.v[1]), "s"(gbase)
        : "memory", "m0");
  } else {
    static_assert(C::DPW / 2 == 1, "1, 2 or 4 pieces per wave and half");
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(m0v), "v"(o.v[0]), "s"(gbase)
        : "memory", "m0");
  }
}

// gK, gV: first byte of the K and V chunk; stage_m0: LDS address of the stage
template <class C>
__device__ __forceinline__ void dma_stage(const char* gK, const char* gV, unsigned stage_m0,
                                          int w, const DmaOff<C>& loff) {
  const unsigned wo = (unsigned)w * (C::DPW / 2) * 1024u;
  dma_half<C>(gK + wo, stage_m0 + wo, loff);
  dma_half<C>(gV + wo, stage_m0 + C::SUBB + wo, loff);
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most `groups` (0, 1 or 2) stages' copies of this wave can
// still be in flight.  Vector memory operations retire in order, so once at
// most `groups` * DPW are outstanding, every stage issued before the last
// `groups` ones has landed (other memory operations issued in between only
// make the wait longer).
template <class C>
__device__ __forceinline__ void wait_groups(int groups) {
  static_assert(2 * C::DPW < 16, "two stages' copies fit the vmcnt field");
  if (groups <= 0) wait_vm0();
  else if (groups == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | C::DPW);
  else __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * C::DPW));
}

// Transposing fragment reads.  For 16-row slab sl and 32-column tile mt of a
// chunk, lane l receives the 8 values X[16 sl + 8 (e / 4) + 4 (l / 32) + e % 4]
// [32 mt + l % 32], e = 0 .. 7: an MFMA 32x32x16 operand whose k index runs
// over the slab's rows (as the A operand of X^T, or the B operand of X).  The
// row order within the slab is the same for every lane, so two operands read
// this way contract row with row.
// Byte offset (within a slab) of lane `lane`'s half h (rows 8 h ..) of tile mt.
template <class C>
__device__ __forceinline__ int tr_lane_offset(int lane, int mt, int h) {
  const int hh = lane >> 5, j = lane & 15, g = lane >> 4;
  const int row = 4 * hh + 8 * h + (j >> 2);
  const int chunk = (32 * mt + 16 * (g & 1)) / 8 + ((j & 3) >> 1);
  return row * C::RB + ((chunk ^ swz<C::D>(row)) << 4) + 8 * (j & 1);
}

// The fragment of slab sl whose two halves sit at byte offsets o0, o1.
template <class C>
__device__ __forceinline__ u32x4 tr_read(const char* base, int sl, int o0, int o1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4*)(base + sl * 16 * C::RB + o0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ls16x4*)(base + sl * 16 * C::RB + o1));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

}  // namespace pisa
