// Device-side helpers shared by the producer kernels.
#pragma once

#include "pgg_internal.h"

namespace pgg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct TBf16 { using elem = uint16_t; static constexpr int kPerChunk = 8; };
struct TF16 { using elem = uint16_t; static constexpr int kPerChunk = 8; };
struct TF32 { using elem = float; static constexpr int kPerChunk = 4; };


// Accumulate one chunk pair: lane half h holds chunk 2q+h of its row for both
// operands, so the MFMA's reduction slots pair equal reduction indices.
template <class T>
__device__ __forceinline__ void mma(f32x16_t& acc, u32x4_t a, u32x4_t b);

template <>
__device__ __forceinline__ void mma<TBf16>(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma<TF16>(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                               __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma<TF32>(f32x16_t& acc, u32x4_t a, u32x4_t b) {
  const f32x4_t fa = __builtin_bit_cast(f32x4_t, a);
  const f32x4_t fb = __builtin_bit_cast(f32x4_t, b);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
}

// Workgroup -> (m-tile slot, column tile) for the MFMA-bound tiles.
// Workgroups go to the 8 XCDs round-robin (id mod 8) and each XCD has its own
// L2.  Tiles are numbered in super-blocks of SM slots x SN column tiles (slot
// fastest, bands of SM slots), and super-block b runs on XCD b mod 8, so the
// 32 workgroups an XCD runs together share SM d_y slabs and SN weight slabs
// in its L2, and every XCD gets an equal share of the super-blocks (idle
// slots at the end of a chunk spread over all XCDs).  The grid is rounded up
// to a multiple of 8*SM*SN; returns false for the surplus.  Any mapping is
// correct; this one only serves locality and balance.
template <int SM, int SN>
__device__ __forceinline__ bool raster(int bid, int n_slots, int n_ct, int& slot, int& ct) {
  constexpr int SB = SM * SN;
  const int x = bid & 7, l = bid >> 3;
  const int t = ((l / SB) * 8 + x) * SB + (l % SB);
  if (t >= n_slots * n_ct) return false;
  const int band = t / (SM * n_ct);
  const int h = min(SM, n_slots - band * SM);
  const int r = t - band * SM * n_ct;
  const int grp = r / (h * SN);
  const int p = r - grp * h * SN;
  slot = band * SM + p % h;
  ct = grp * SN + p / h;
  return true;
}


// LDS byte offset of a __shared__ object (for M0 of direct-to-LDS loads).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

}  // namespace pgg
