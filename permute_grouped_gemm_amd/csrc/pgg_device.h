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


// Load one 16-byte chunk of a row (elements [n, n + kPerChunk)), zero outside
// the row or past N.  NT: aligned chunks are loaded with the non-temporal
// hint (data read once, such as a weight stream).
template <class T, bool ALIGNED, bool NT = false>
__device__ __forceinline__ u32x4_t load_chunk(const typename T::elem* __restrict__ row, bool row_ok,
                                              int64_t n, int64_t N) {
  using E = typename T::elem;
  constexpr int EPC = T::kPerChunk;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (!row_ok || n >= N) return v;
  if constexpr (ALIGNED && NT) {
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + n));
  } else if constexpr (ALIGNED) {
    v = *reinterpret_cast<const u32x4_t*>(row + n);
  } else {
    E e[EPC];
#pragma unroll
    for (int t = 0; t < EPC; ++t) e[t] = (n + t < N) ? row[n + t] : E(0);
    __builtin_memcpy(&v, e, sizeof(v));
  }
  return v;
}

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

// 16 zero bytes in global memory: the source of masked-off direct-to-LDS
// loads (every lane of such a load reads something; masked lanes read zeros).
__device__ const u32x4_t kZero16 = {0u, 0u, 0u, 0u};

// Direct global -> LDS load of 16 bytes per lane: lane i's bytes land at LDS
// byte offset m0 + 16 i.  Issued by inline assembly, so the compiler neither
// tracks nor waits for it: the waits on the vector-memory counter are explicit
// (vector memory operations complete in issue order, and these loads write no
// register).  An LDS load reads M0 one wait state after a scalar write of it
// (a hazard the compiler cannot see inside the asm), hence the s_nop.
__device__ __forceinline__ void dma16(const void* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0), "v"(src) : "memory", "m0");
}

// The same load with the non-temporal hint: for data read exactly once (a
// weight stream), so its lines do not displace operands that are reused.
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :: "s"(m0), "v"(src) : "memory", "m0");
}

// A byte offset past every buffer the buffer loads below read (each spans
// less than 2^31 bytes).
constexpr uint32_t kOutside = 0x80000000u;

// Direct buffer -> LDS load of 16 bytes per lane: lane i's bytes (at byte
// offset voff of the buffer; zeros, with no memory access, when voff is past
// its range) land at LDS byte offset m0 + 16 i.  The whole offset is in the
// vector offset, which the range check covers.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voff), "s"(r) : "memory", "m0");
}

// The same with the non-temporal hint (a weight stream read once).
__device__ __forceinline__ void dma16_buf_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(m0), "v"(voff), "s"(r) : "memory", "m0");
}

// Wait until at most N of this wave's vector memory operations are
// outstanding and its LDS reads are done, then barrier the workgroup.  The
// wait is the builtin (so the compiler knows the LDS reads are done); the
// empty asm statements keep memory accesses from moving across.
template <int N>
__device__ __forceinline__ void wait_then_barrier() {
  // s_waitcnt immediate: vmcnt[3:0] in bits 3:0, expcnt 6:4 (7 = no wait),
  // lgkmcnt 11:8 (0), vmcnt[5:4] in bits 15:14
  constexpr int kImm = (N & 15) | (7 << 4) | ((N >> 4) << 14);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kImm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// Wave-uniform loads through the scalar data cache (reads only).  The value
// lands in scalar registers and is waited for on the scalar/LDS counter, so
// direct-to-LDS loads in flight on the vector-memory counter are not drained
// for it (a vector load here would be: that counter completes in order).
// Kernels that also issue direct-to-LDS loads clobber memory in every asm
// statement, which stops the compiler from choosing scalar loads itself.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t scalar_load_i64(const int64_t* p) {
  i32x2_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(v[1])) << 32) |
                              static_cast<uint32_t>(v[0]));
}

__device__ __forceinline__ MTile scalar_load_tile(const MTile* p) {
  i32x4_t v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  MTile t;
  t.g = v[0];
  t.row0 = v[1];
  t.rows = v[2];
  t.pad = v[3];
  return t;
}

// Wait for this wave's LDS operations only, then barrier the workgroup (for
// data exchanged through LDS while direct-to-LDS loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
  constexpr int kImm = 15 | (7 << 4) | (3 << 14);   // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kImm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace pgg
