// device_common.h -- small device helpers shared by the attention kernels
// (gfx950 only): vector types, lane-pair reductions, barriers and waits, the
// global -> LDS tile load and the forward kernels' work list.  Included by
// each kernel source; everything here has internal linkage except the host
// schedule planner declared at the end (defined with the bf16 launch).
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

// ---- the forward kernels' work list.  A work item is (batch, kv-head, head
// group, q-block); the list numbers the items and a persistent grid of G
// workgroups (at most one per CU) computes them in rounds.  `stream` below
// is b * n_kv + kv-head, whose K/V rows the item reads.
//
// * Default: heavy q-blocks first, neighbouring numbers on different head
//   groups and streams; round r is items r G .. r G + G - 1, taken forwards
//   when r is even and backwards when it is odd (in blocks of 8 when G is a
//   multiple of 8, so that a workgroup only sees items congruent to w mod
//   8), a zigzag that evens out the workgroups' causal work.  Workgroups are
//   dealt to the eight XCDs in turn (workgroup w runs on XCD w mod 8).
// * Stream blocks (sg > 0): the list is cut into super-groups of sg
//   q-blocks, heaviest first; inside one, every stream in turn lists its sg
//   q-blocks (heavy first) with their head groups.  Workgroup w = 8 s + x
//   (XCD x, slot s) takes position (G / 8) x + s of each round, backwards in
//   odd rounds, so an XCD works on a run of G / 8 consecutive entries:
//   adjacent q-blocks of one or two streams, which read the same K/V prefix
//   side by side, so the XCD's L2 fetches each tile once for all of them.
// * Balanced pairs (pair_t > 0, causal): q-blocks pair_t .. n_qblk - 1 form
//   the pairs (n_qblk - 1 - i, pair_t + i), whose causal lengths sum to the
//   same total for every i.  The pairs are listed in stream blocks of sg
//   values of i; pair round k (rounds 2k and 2k + 1) gives workgroup w the
//   pair at position k G + (G / 8) x + s, its heavy member in round 2k and
//   its light member in round 2k + 1.  Every workgroup of an XCD then starts
//   each even round at the same moment (no drift builds up between rounds),
//   so the run of adjacent q-blocks on the XCD stays in step and keeps
//   sharing its L2.  The host makes the pairs fill whole rounds; the items of
//   q-blocks 0 .. pair_t - 1 follow in the list, heavy first (the dynamic
//   tail's share; without the tail they run as zigzag rounds).
struct ItemList {
  int n_qblk, ipq, ngroups;   // q-blocks; items per q-block (streams x head groups); head groups
  int sg, pair_t, pair_rounds;
};

// The list entry workgroup w computes in round r of the static schedule.
// (Host and device: the host's schedule diagnostic runs the same code.)
__host__ __device__ __forceinline__ int list_item_at(const ItemList& s, int r, int w, int G) {
  if (s.sg > 0) {
    const int pos = (G >> 3) * (w & 7) + (w >> 3);
    if (s.pair_t > 0 && r < s.pair_rounds) return r * G + pos;
    const int rr = s.pair_t > 0 ? r - s.pair_rounds : r;
    return r * G + ((rr & 1) ? G - 1 - pos : pos);
  }
  if (!(r & 1)) return r * G + w;
  if ((G & 7) == 0) return r * G + (G - 8 - (w & ~7)) + (w & 7);
  return r * G + G - 1 - w;
}

// List entry -> (q-block, head group, stream).
__host__ __device__ __forceinline__ void list_decode(const ItemList& s, int item, int G, int& qb,
                                                     int& hg, int& stream) {
  if (s.pair_t > 0 && item < s.pair_rounds * G) {
    const int r = item / G;
    const int p = (r >> 1) * G + (item - r * G);   // pair index
    const int half = (s.n_qblk - s.pair_t) >> 1;
    const int span = s.sg * s.ipq;
    const int k_sg = p / span;
    const int in_sg = p - k_sg * span;
    const int left = half - k_sg * s.sg;   // values of i in this super-group
    const int per = (s.sg < left ? s.sg : left) * s.ngroups;
    stream = in_sg / per;
    const int in_st = in_sg - stream * per;
    const int i = k_sg * s.sg + in_st / s.ngroups;
    hg = in_st % s.ngroups;
    qb = (r & 1) ? s.pair_t + i : s.n_qblk - 1 - i;
  } else if (s.pair_t > 0) {
    const int u = item - s.pair_rounds * G;
    qb = s.pair_t - 1 - u / s.ipq;
    const int rest = u % s.ipq;
    hg = rest % s.ngroups;
    stream = rest / s.ngroups;
  } else if (s.sg > 0) {
    const int span = s.sg * s.ipq;
    const int k_sg = item / span;
    const int in_sg = item - k_sg * span;
    const int left = s.n_qblk - k_sg * s.sg;   // q-blocks in this super-group
    const int per = (s.sg < left ? s.sg : left) * s.ngroups;
    stream = in_sg / per;
    const int in_st = in_sg - stream * per;
    qb = s.n_qblk - 1 - (k_sg * s.sg + in_st / s.ngroups);
    hg = in_st % s.ngroups;
  } else {
    qb = s.n_qblk - 1 - item / s.ipq;
    const int rest = item % s.ipq;
    hg = rest % s.ngroups;
    stream = rest / s.ngroups;
  }
}

// Host: do [a, a + an) and [b, b + bn) overlap?
inline bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

}  // namespace

// Host: the list form and schedule of a persistent forward launch (defined
// with the bf16 kernel's launch, shared with the FP8 one): sg and pair_t as
// ItemList describes them, r_static rounds of the static schedule, then the
// dynamic tail through the counter pair dyn, or (dyn == nullptr) every round
// static.
struct ItemPlan {
  int sg, pair_t;
  long long r_static;
  unsigned* dyn;
};
__attribute__((visibility("hidden"))) ItemPlan attn_item_plan(long long n_items, long long ipq,
                                                              long long n_qblk, long long ngroups,
                                                              long long grid, int causal,
                                                              hipStream_t stream);

#endif  // ATTN_DEVICE_COMMON_H
