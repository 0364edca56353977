// device_common.h -- small device helpers shared by the attention kernels
// (gfx950 only): vector types, lane-pair reductions, barriers and waits, and
// the global -> LDS tile load.  Included by each kernel source; everything
// here has internal linkage.
#ifndef ATTN_DEVICE_COMMON_H
#define ATTN_DEVICE_COMMON_H

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#define LDS_AS __attribute__((address_space(3)))

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// max / sum of x over lanes l and l ^ 32
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroup barrier that does not wait for outstanding memory operations
// (the caller waits for exactly the loads the next tile needs); the signal
// fences keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void tile_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt with only a vector-memory count (expcnt and lgkmcnt at maximum)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) alone: every LDS read of this wave has returned
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Global -> LDS loads ("buffer_load ... lds": each lane's bytes at its
// voffset land at the wave's LDS destination in M0 plus the lane's slot).
//
// They are issued from inline assembly.  The compiler does not track them,
// so it adds no wait of its own for them; in particular it cannot treat
// every later LDS transpose read as a possible reader of the bytes in
// flight and wait for all outstanding loads before it, which would cut the
// prefetch distance of a load ring to nothing.  Every caller instead waits
// with an explicit s_waitcnt vmcnt for exactly the loads the next tile
// needs, then crosses a barrier (or, for wave-private LDS, only waits),
// before reading that tile, and waits for all of them before the wave ends.

// Buffer resource words over `bytes` bytes from `base` (both wave-uniform;
// the count is read into an SGPR so the whole resource stays scalar), raw
// 32-bit format, stride 0: loads at offsets past the end return zeros (the
// hardware range check).
__device__ __forceinline__ u32x4 buffer_words(const void* base, int bytes) {
  const unsigned long long addr = reinterpret_cast<unsigned long long>(base);
  u32x4 w;
  w[0] = (unsigned)addr;
  w[1] = (unsigned)(addr >> 32) & 0xffffu;
  w[2] = (unsigned)__builtin_amdgcn_readfirstlane(bytes);
  w[3] = 0x00020000u;
  return w;
}

// 16 bytes per lane at voffset, to LDS byte lds + 16 * lane
__device__ __forceinline__ void lds_load_b128(const u32x4& rsrc, int voffset, unsigned lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// 4 bytes per lane at voffset, to LDS byte lds + 4 * lane
__device__ __forceinline__ void lds_load_b32(const u32x4& rsrc, int voffset, unsigned lds) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds)
               : "memory");
}

// LDS byte address of a __shared__ pointer
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)reinterpret_cast<uintptr_t>((LDS_AS const unsigned char*)p);
}

// One wave's share of a K or V tile load, global -> LDS: `loads` loads of
// 1 KB, lane i of load s bringing the 16 bytes at source offset src[s]
// (relative to row j0 of rows of `row_bytes`) to LDS byte dst + 1 KB s + 16 i.
// A tile at or past row L reads as zeros and touches no memory.  The range
// covers at most one tile of tile_rows rows, so it fits the 32-bit record
// count at any L.
__device__ __forceinline__ void dma_tile(const void* base, const int* src, int loads,
                                         int row_bytes, int j0, int L, int tile_rows,
                                         unsigned char* dst_shared) {
  const u32x4 rsrc = buffer_words((const unsigned char*)base + (size_t)j0 * row_bytes,
                                  min(max(L - j0, 0), tile_rows) * row_bytes);
  const unsigned dst = lds_addr(dst_shared);
#pragma unroll
  for (int s = 0; s < loads; ++s) lds_load_b128(rsrc, src[s], dst + s * 1024);
}

// Host: do [a, a + an) and [b, b + bn) overlap?
inline bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

}  // namespace

#endif  // ATTN_DEVICE_COMMON_H
