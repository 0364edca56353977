// attn_fp8.hip -- FP8 (OCP e4m3) variant of the causal GQA prefill attention
// forward pass for gfx950.
//
// Method: FP8 attention on the most compute-dense part of prefill, which
// buys matrix-core throughput and doubles the ridge ("flops /
// prefill-attention", section "Workarounds", FP8 attention).  Q, K and V
// arrive as e4m3 codes with one fp32 descale factor each (true value = code
// value x descale).  Q K^T and P V run on v_mfma_f32_32x32x64_f8f6f4 with
// fp32 accumulation; P is rounded to e4m3 (nearest even) before P V; O is
// written in bf16 and LSE in fp32.  Tiling, the online softmax, causal tile
// skipping, the chunk offset and the work items follow the bf16 kernel in
// attn_prefill.hip ("Why Attention Scaling Breaks", section "Flash
// Attention: the tiling insight"; "Long-Context Attention Explained",
// sections "Tiling" and "Online softmax").
//
// CDNA4 mapping (d_h = 128):
//  * A workgroup covers 256 query columns (HWG heads of one group x 256/HWG
//    rows) with 8 waves, one 32-column block each, as the bf16 kernel.
//  * K and V tiles of 128 keys x 128 bytes (16 KB, the bytes of a bf16 tile)
//    stream into 4-tile LDS rings by buffer loads with the LDS destination
//    bit, requested three tiles ahead, one barrier per tile.  As in the bf16
//    kernel the grid is persistent (one workgroup per CU, a zigzag over the
//    heavy-first items) and the ring runs on across items.
//  * The unit of compute is 64 keys: S^T = K Q^T for two 32-key blocks (two
//    64-deep k-steps each), the softmax of both, then O^T += V^T P^T as one
//    64-deep contraction per 32 rows of O^T.  A lane holds 16 scores of each
//    block; together they are the 32 bytes of its P^T operand, byte
//    16 b + r holding key 32 b + 8 (r / 4) + 4 (lane / 32) + r % 4.  The
//    matrix cores pair byte e of a lane half of one operand with byte e of
//    the same lane half of the other (verified on an MI355X), so any byte order
//    works as long as V^T uses the same one.
//  * V^T in that key order comes from the row-major V tile through
//    ds_read_b64_tr_b8 (verified on an MI355X: in each group of 16 lanes, lane
//    2 e + q supplies 8 bytes, and lane i receives byte i % 8 of the piece of
//    lane 2 e + i / 8 as its byte e).  Four reads give a lane its 32 keys.
//  * P = 2^(c s - m) never exceeds 2^8 (the reference max moves when a tile
//    max passes it by more than 2^8), inside e4m3's range (448); weights
//    below 2^-10 of the reference round to zero.  The row sum adds the fp32
//    weights before rounding.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "attn_prefill.h"
#include "device_common.h"

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kF8Cols = 256;     // query columns per workgroup
constexpr int kF8Waves = 8;      // one 32-column block per wave
constexpr int kF8D = 128;        // head size (bytes per K or V row)
constexpr int kF8Tile = 128;     // keys per K/V tile
constexpr int kF8Unit = 64;      // keys per unit of compute
constexpr float kF8Slack = 8.0f; // rescale only past 2^8 growth

// 16-byte chunk swizzles (row = key inside the tile, 128-byte rows).  K: 16
// lanes of a 16-byte read take 16 consecutive rows at one chunk; two rows
// share a 256-byte bank window, so XORing the chunk with (row >> 1) & 7
// spreads them over the 16 slots.  V: the 32 lanes of a transpose read take
// rows {0,1,2,3,8,9,10,11} (+4, +16 t) at one 32-byte column pair; XORing
// the chunk with 2 (bit 1 | bit 3 << 1) of the row puts them on the 8
// distinct 32-byte slots of the window.
__device__ __forceinline__ int f8_k_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int f8_v_swz(int row) {
  return 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1));
}

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // unscaled e4m3 x e4m3 (format selectors 0, scale operands 0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int HWG>
__global__ __launch_bounds__(64 * kF8Waves) void attn_fwd_fp8_kernel(
    const unsigned char* __restrict__ q, const unsigned char* __restrict__ k,
    const unsigned char* __restrict__ v, unsigned short* __restrict__ out,
    float* __restrict__ lse, int Lq, int Lk, int q_off, int n_q, int n_kv, int n_qblk,
    int items_per_qblk, int n_items, float c2, float v_mul, int causal, int sg, int pair_t,
    unsigned* __restrict__ dyn, int r_static) {
  constexpr int D = kF8D;
  constexpr int BR = kF8Cols / HWG;            // query rows per workgroup
  constexpr int KSTEPS = D / 64;               // 64-deep k-steps of Q K^T
  constexpr int TBLK = D / 32;                 // 32-row blocks of O^T
  constexpr int ROWB = D;                      // bytes per K or V row
  constexpr int TILE = kF8Tile * ROWB;         // bytes per K or V tile
  constexpr int LOADS = TILE / (kF8Waves * 1024);
  static_assert(LOADS * kF8Waves * 1024 == TILE, "tile must split into 1 KB loads");
  constexpr int RING = 4;
  constexpr int VRING = 0;
  constexpr int KRING = RING * TILE;

  // output staging: one wave's 32 bf16 output rows (8 KB); waves 0..3 use
  // ring slot 3 (idle once an item's last tile is done), waves 4..7 an area
  // after the rings
  constexpr int OROWB = 2 * D;                 // bytes per bf16 output row
  constexpr int OT = 32 * OROWB;               // bytes of one wave's output tile
  constexpr int STAGE = 2 * RING * TILE;
  static_assert(4 * OT == 2 * TILE && kF8Waves == 8, "half the output tiles fill one ring slot");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGE + 4 * OT];
  LDS_AS unsigned char* const smem_l = (LDS_AS unsigned char*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hi = lane >> 5;
  const int col = lane & 31;

  // ---- work items as the bf16 kernel: (b, kv-head, head group, q-block) in
  // the list order of ItemList (heavy-first zigzag, stream blocks or
  // balanced pairs, chosen by the host), then the dynamic tail
  const int g = n_q / n_kv;
  const int ngroups = g / HWG;
  const int c0 = 32 * wave;
  const size_t Lq64 = (size_t)Lq;
  ItemList lst;
  lst.n_qblk = n_qblk;
  lst.ipq = items_per_qblk;
  lst.ngroups = ngroups;
  lst.sg = sg;
  lst.pair_t = pair_t;
  lst.pair_rounds =
      pair_t > 0 ? 2 * ((((n_qblk - pair_t) >> 1) * items_per_qblk) / (int)gridDim.x) : 0;
  auto item_at = [&] __device__ (int r) __attribute__((always_inline)) {
    return list_item_at(lst, r, blockIdx.x, gridDim.x);
  };
  struct Geo {
    int b, hh, q0, n_tiles;       // batch, this wave's head and first row, tiles streamed
    const unsigned char* kb;
    const unsigned char* vb;
  };
  auto geo = [&] __device__ (int item) __attribute__((always_inline)) {
    Geo e;
    int qb, hg, rest;   // rest: the (batch, kv-head) stream
    list_decode(lst, item, gridDim.x, qb, hg, rest);
    const int kvh = rest % n_kv;
    e.b = rest / n_kv;
    e.hh = kvh * g + hg * HWG + c0 / BR;
    e.q0 = qb * BR + c0 % BR;
    const int wg_end = min(qb * BR + BR, Lq);
    e.n_tiles = causal ? (wg_end + q_off + kF8Tile - 1) / kF8Tile : (Lk + kF8Tile - 1) / kF8Tile;
    e.kb = k + ((size_t)e.b * n_kv + kvh) * (size_t)Lk * D;
    e.vb = v + ((size_t)e.b * n_kv + kvh) * (size_t)Lk * D;
    return e;
  };

  // ---- Q fragments (B operand of S^T = K Q^T): bytes 64 kk + 32 hi .. +32 of row q0 + col
  i32x8 qf[KSTEPS];
  auto load_q = [&] __device__ (const Geo& e) __attribute__((always_inline)) {
    const int qi = e.q0 + col;
    const unsigned char* qrow = q + (((size_t)e.b * n_q + e.hh) * Lq64 + (size_t)qi) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 lo = {0u, 0u, 0u, 0u}, up = {0u, 0u, 0u, 0u};
      if (qi < Lq) {
        lo = *reinterpret_cast<const u32x4*>(qrow + 64 * kk + 32 * hi);
        up = *reinterpret_cast<const u32x4*>(qrow + 64 * kk + 32 * hi + 16);
      }
      qf[kk] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
    }
  };

  // per-item state the pipeline reads
  int q0 = 0, n_tiles = 0, wave_units = 0;
  const unsigned char* kbase = k;
  const unsigned char* vbase = v;
  const unsigned char* nkbase = k;
  const unsigned char* nvbase = v;
  bool has_next = false;

  // ---- tile loads: load s of this wave fills LDS bytes [1 KB (wave * LOADS
  // + s), +1 KB) of a tile with the chunks the rows' swizzles put there
  int k_src[LOADS], v_src[LOADS];
#pragma unroll
  for (int s = 0; s < LOADS; ++s) {
    const int byte = (wave * LOADS + s) * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int pos = (byte % ROWB) >> 4;
    k_src[s] = row * ROWB + ((pos ^ f8_k_swz(row)) << 4);
    v_src[s] = row * ROWB + ((pos ^ f8_v_swz(row)) << 4);
  }
  auto load_tile = [&] __device__ (const unsigned char* base, const int (&src)[LOADS], int tile,
                       int lds_off) __attribute__((always_inline)) {
    dma_tile(base, src, LOADS, ROWB, tile * kF8Tile, Lk, kF8Tile,
             smem + lds_off + wave * LOADS * 1024);
  };

  // ---- per-lane LDS read offsets (ring slot 0, unit 0, block 0)
  // K: row col, logical chunks 4 kk + 2 hi + h
  int k_rd[KSTEPS][2];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      k_rd[kk][h] = KRING + col * ROWB + (((4 * kk + 2 * hi + h) ^ f8_k_swz(col)) << 4);
  // V^T: lane 16 G + j supplies, for transpose read t, the 8 bytes of row
  // 16 t + 8 ((j / 2) / 4) + 4 hi + (j / 2) % 4 at column 32 tb + 16 (G % 2) + 8 (j % 2)
  int v_rd[TBLK];
  {
    const int j = lane & 15;
    const int cg = (lane >> 4) & 1;
    const int row0 = 8 * ((j >> 1) >> 2) + 4 * hi + ((j >> 1) & 3);
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb)
      v_rd[tb] = VRING + row0 * ROWB + (((2 * tb + cg) ^ f8_v_swz(row0)) << 4) + 8 * (j & 1);
  }

  f32x16 acc[TBLK];
  float m_run = -INFINITY;   // reference max, log2 domain
  float l_run = 0.0f;        // this lane's part of the row sum
  const bool fast_scale = c2 > 0.0f;

  // K fragments of unit u (0..7 across the ring: slot u / 2, half u % 2)
  auto load_kfrags = [&] __device__ (i32x8 (&kf)[2][KSTEPS], int slot, int uu)
      __attribute__((always_inline)) {
#pragma unroll
    for (int bl = 0; bl < 2; ++bl)
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int off = slot * TILE + (uu * kF8Unit + bl * 32) * ROWB;
        const u32x4 lo = *reinterpret_cast<const LDS_AS u32x4*>(smem_l + k_rd[kk][0] + off);
        const u32x4 up = *reinterpret_cast<const LDS_AS u32x4*>(smem_l + k_rd[kk][1] + off);
        kf[bl][kk] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
      }
  };
  // V^T fragments of a unit: four transpose reads per 32 rows of O^T
  auto load_vfrags = [&] __device__ (i32x8 (&vf)[TBLK], int slot, int uu)
      __attribute__((always_inline)) {
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb) {
      i32x2 r[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        r[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (LDS_AS i32x2*)(smem_l + v_rd[tb] + slot * TILE + (uu * kF8Unit + 16 * t) * ROWB));
      vf[tb] = (i32x8){r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    }
  };
  auto qk = [&] __device__ (f32x16 (&S)[2], const i32x8 (&kf)[2][KSTEPS])
      __attribute__((always_inline)) {
#pragma unroll
    for (int bl = 0; bl < 2; ++bl) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[bl][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) S[bl] = mfma_f8(kf[bl][kk], qf[kk], S[bl]);
    }
  };

  // softmax of one unit (keys j0 .. j0 + 63): mask and pre-scale where the
  // unit straddles the diagonal or the end of the keys (or the scale is not
  // positive), move the reference max only past 2^8 growth, then
  // p = 2^(c s - m) rounded to e4m3 as the P^T operand
  auto softmax_unit = [&] __device__ (f32x16 (&S)[2], int j0, i32x8& pk)
      __attribute__((always_inline)) {
    const int qi = q0 + col;
    const bool need_mask = (causal && j0 + kF8Unit - 1 > q0 + q_off) || (j0 + kF8Unit > Lk);
    float c = c2;
    float mx;
    if (need_mask || !fast_scale) {
      mx = -INFINITY;
#pragma unroll
      for (int bl = 0; bl < 2; ++bl)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * bl + (r >> 2) * 8 + hi * 4 + (r & 3);
          const bool dead = (causal && j > qi + q_off) || j >= Lk;
          S[bl][r] = dead ? -INFINITY : S[bl][r] * c2;
          mx = fmaxf(mx, S[bl][r]);
        }
      c = 1.0f;
    } else {
      // (a running max taking two scores per step: one v_max3 each)
      mx = fmaxf(S[0][0], S[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, S[0][r]), S[1][r]);
    }
    const float m_cand = pair_max(mx) * c;
    if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kF8Slack) != 0) {
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tb][r] *= alpha;
    }
    const float mneg = -m_run;
#pragma unroll
    for (int bl = 0; bl < 2; ++bl)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(S[bl][4 * w + 0], c, mneg));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(S[bl][4 * w + 1], c, mneg));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(S[bl][4 * w + 2], c, mneg));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(S[bl][4 * w + 3], c, mneg));
        l_run += (p0 + p1) + (p2 + p3);
        // the first conversion fills the low half of the word and keeps the
        // high half, which the second one then writes: the word's previous
        // bits are never used, so it starts as p0's own (a register that dies
        // here) instead of a zeroed one
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, __builtin_bit_cast(int, p0), false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
        pk[4 * bl + w] = word;
      }
  };

  auto pv = [&] __device__ (const i32x8 (&vf)[TBLK], const i32x8& pk)
      __attribute__((always_inline)) {
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb) acc[tb] = mfma_f8(vf[tb], pk, acc[tb]);
  };

  // Pipeline over units U = 2 t + uu.  Entering region U: the raw scores of
  // U are in cur, the K fragments of U + 1 in kf.  The region puts the Q K^T
  // of U + 1 on the matrix pipe, reads the V^T fragments of U and the K
  // fragments of U + 2, runs the softmax of U next to those products, then
  // P V of U.  Past the wave's last unit it computes on stale LDS data whose
  // results are never used.
  f32x16 SA[2], SB[2];
  i32x8 kf[2][KSTEPS];
  i32x8 vf[TBLK];

  // Tile t of an item sits in ring slot t % 4; the ring runs on across
  // items.  During tile t the workgroup requests stream position t + 3 into
  // the slot tile t - 1 has freed: tile t + 3 of this item, or, past its last
  // tile, tile j of the next item when the slot is j < 3.  Every tile step
  // issues the same number of loads (otherwise a tile of this item past its
  // end: rows never used, or zeros), which keeps the vmcnt counts exact.
  auto issue_tile_loads = [&] __device__ (int TS, int t) __attribute__((always_inline)) {
    const int p = t + 3;
    const int slot = (TS + 3) & (RING - 1);
    const bool own = p < n_tiles || !has_next || slot == RING - 1;
    const int tile = own ? p : slot;
    load_tile(own ? vbase : nvbase, v_src, tile, VRING + slot * TILE);
    load_tile(own ? kbase : nkbase, k_src, tile, KRING + slot * TILE);
  };
  auto region = [&] __device__ (int t, int ts, int uu, f32x16 (&cur)[2], f32x16 (&nxt)[2])
      __attribute__((always_inline)) {
    // keep the scheduler from pulling this region's softmax up next to the
    // previous region's last MFMAs
    __builtin_amdgcn_sched_barrier(0);
    qk(nxt, kf);
    if (uu == 0) issue_tile_loads(ts, t);
    load_vfrags(vf, ts, uu);
    // K of unit U + 2: same half of the next tile
    load_kfrags(kf, (ts + 1) & (RING - 1), uu);
    i32x8 pk;
    softmax_unit(cur, t * kF8Tile + uu * kF8Unit, pk);
    pv(vf, pk);
  };

  auto tile_step = [&] __device__ (int TS, int t) __attribute__((always_inline)) {
    if (2 * t < wave_units) {
      region(t, TS, 0, SA, SB);   // issues the loads of stream position t + 3
      if (2 * t + 1 < wave_units) region(t, TS, 1, SB, SA);
    } else {
      issue_tile_loads(TS, t);
    }
    wait_vmcnt<2 * LOADS>();
    tile_barrier();
  };

  int r = 0;
  int item = item_at(0);           // the grid never exceeds the item count
  Geo cur = geo(item);
  load_q(cur);
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    load_tile(cur.kb, k_src, i, KRING + i * TILE);
    load_tile(cur.vb, v_src, i, VRING + i * TILE);
  }
  // the word through which wave 0 passes a dynamic-tail item to the others
  // (as in the bf16 kernel: the first bytes of its own output staging area)
  LDS_AS int* const dyn_word = (LDS_AS int*)(smem_l + VRING + 3 * TILE);
  const int n_dyn = n_items - r_static * (int)gridDim.x;
  for (;;) {
    // ---- item setup; the next item from the static schedule or, in the
    // dynamic tail, from the call's counter (as in the bf16 kernel)
    const bool dyn_next = dyn != nullptr && r + 1 >= r_static;
    int nxt_item = n_items;
    if (!dyn_next) {
      nxt_item = item_at(r + 1);
    } else if (wave == 0) {
      if (lane == 0) {
        const unsigned j = __hip_atomic_fetch_add(dyn, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_SYSTEM);
        *dyn_word = j < (unsigned)n_dyn ? r_static * (int)gridDim.x + (int)j : n_items;
      }
      wait_lgkm0();
    }
    kbase = cur.kb;
    vbase = cur.vb;
    n_tiles = cur.n_tiles;
    q0 = cur.q0;
    const int last_row = q0 < Lq ? min(q0 + 31, Lq - 1) : -1;
    wave_units = last_row < 0 ? 0 : (causal ? (last_row + q_off) / kF8Unit + 1 : 2 * n_tiles);
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tb][e] = 0.0f;
    m_run = -INFINITY;
    l_run = 0.0f;

    // ---- prologue: the item's tiles 0..2 and its Q have landed (and the
    // previous item's stores are done); scores of unit 0, K fragments of unit 1
    wait_vmcnt<0>();
    tile_barrier();
    if (dyn_next) {
      nxt_item = __builtin_amdgcn_readfirstlane(*dyn_word);
      wait_lgkm0();
      tile_barrier();
    }
    has_next = nxt_item < n_items;
    const Geo nx = geo(has_next ? nxt_item : item);
    nkbase = nx.kb;
    nvbase = nx.vb;
    if (wave_units > 0) {
      load_kfrags(kf, 0, 0);
      qk(SA, kf);
      load_kfrags(kf, 0, 1);
    }
    for (int t = 0; t < n_tiles; t += RING) {
      tile_step(0, t);
      if (t + 1 < n_tiles) tile_step(1, t + 1);
      if (t + 2 < n_tiles) tile_step(2, t + 2);
      if (t + 3 < n_tiles) tile_step(3, t + 3);
    }
    // No wave's tile load may still write ring slot 3, which the output
    // staging uses.  Its last load was issued by tile step (n_tiles - 1) & ~3;
    // a step ends (at its barrier) with only its own loads in flight, so
    // unless that step is the last one they have all landed.  If it is, every
    // wave must see every other wave's loads land: the barrier after the wait.
    wait_vmcnt<0>();
    if (n_tiles <= 0 || ((n_tiles - 1) & (RING - 1)) == 0) tile_barrier();
    if (has_next) {
      // the next item's tiles 0..2 the last tile steps could not request,
      // then its Q, landing while this item's output is written
      int req = 0;
      for (int t = max(0, n_tiles - 3); t < n_tiles; ++t) req |= 1 << ((t + 3) & (RING - 1));
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (!((req >> j) & 1)) {
          load_tile(nkbase, k_src, j, KRING + j * TILE);
          load_tile(nvbase, v_src, j, VRING + j * TILE);
        }
      load_q(nx);
    }

    // ---- epilogue: O = v_mul acc / l in bf16 through LDS (whole-row
    // stores), LSE = ln 2 (m + log2 l).  (The lane id is re-derived, opaque
    // to the compiler, so the staging addresses are computed here instead of
    // being kept across the tile loop.)
    int elane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(elane));
    const int ecol = elane & 31;
    const int ehi = elane >> 5;
    const float l_tot = pair_sum(l_run);
    const float inv = v_mul / l_tot;
    LDS_AS unsigned char* ot =
        smem_l + (wave < 2 ? VRING + 3 * TILE + wave * OT
                           : wave < 4 ? KRING + 3 * TILE + (wave - 2) * OT : STAGE + (wave - 4) * OT);
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[tb][grp * 4 + e] * inv);
        const int chunk = tb * 4 + grp;
        *reinterpret_cast<LDS_AS u32x2*>(ot + ecol * OROWB + ((chunk ^ (ecol & 15)) << 4) +
                                         ehi * 8) = __builtin_bit_cast(u32x2, o4);
      }
    if (hi == 0 && q0 + col < Lq && wave_units > 0)
      lse[((size_t)cur.b * n_q + cur.hh) * Lq64 + (size_t)(q0 + col)] =
          (m_run + __log2f(l_tot)) * kLn2;
    unsigned short* obase = out + (((size_t)cur.b * n_q + cur.hh) * Lq64 + (size_t)q0) * D;
#pragma unroll
    for (int st = 0; st < OT / 1024; ++st) {
      const int byte = st * 1024 + elane * 16;
      const int row = byte / OROWB;
      const int chunk = (byte % OROWB) >> 4;
      const u32x4 v4 =
          *reinterpret_cast<const LDS_AS u32x4*>(ot + row * OROWB + ((chunk ^ (row & 15)) << 4));
      if (q0 + row < Lq && wave_units > 0)
        // (non-temporal, as in the bf16 kernel)
        __builtin_nontemporal_store(v4, reinterpret_cast<u32x4*>(obase + (size_t)row * D + chunk * 8));
    }
    if (!has_next) break;
    cur = nx;
    item = nxt_item;
    ++r;
  }
  wait_vmcnt<0>();   // no tile load may still be writing LDS when the wave ends
  // the last workgroup out sets the call's counters back to zero
  if (dyn != nullptr && wave == 0 && lane == 0 &&
      __hip_atomic_fetch_add(dyn + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
          gridDim.x - 1) {
    __hip_atomic_store(dyn, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(dyn + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

int f8_pick_hwg(int g) {
  if (g % 8 == 0) return 8;
  if (g % 4 == 0) return 4;
  if (g % 2 == 0) return 2;
  return 1;
}

template <int HWG>
int f8_launch(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Lq,
              int Lk, int q_off, int n_q, int n_kv, float c2, float v_mul, int causal,
              hipStream_t stream) {
  constexpr int BR = kF8Cols / HWG;
  const int n_qblk = (Lq + BR - 1) / BR;
  const long long items_per_qblk = (long long)B * n_kv * ((n_q / n_kv) / HWG);
  const long long n_items = items_per_qblk * n_qblk;
  // (round r of the persistent schedule computes r G + w, which must not wrap)
  if (items_per_qblk > INT_MAX || n_items > INT_MAX / 2) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  // persistent grid: one workgroup per CU, never more than there are items
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu < 1)
    return ATTN_PREFILL_ERR_LAUNCH;
  const long long grid = n_items < n_cu ? n_items : n_cu;
  // the list form and the dynamic tail, chosen as for the bf16 kernel
  const ItemPlan plan =
      attn_item_plan(n_items, items_per_qblk, n_qblk, (n_q / n_kv) / HWG, grid, causal, stream);
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<HWG>), dim3((unsigned)grid), dim3(64 * kF8Waves), 0,
                     stream, static_cast<const unsigned char*>(q),
                     static_cast<const unsigned char*>(k), static_cast<const unsigned char*>(v),
                     static_cast<unsigned short*>(out), lse, Lq, Lk, q_off, n_q, n_kv, n_qblk,
                     (int)items_per_qblk, (int)n_items, c2, v_mul, causal, plan.sg, plan.pair_t,
                     plan.dyn, (int)plan.r_static);
  return hipGetLastError() == hipSuccess ? ATTN_PREFILL_OK : ATTN_PREFILL_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_prefill_fwd_fp8(const void* q, const void* k, const void* v, void* out,
                                    float* lse, int B, int Lq, int Lk, int q_offset, int n_q,
                                    int n_kv, int d_h, float scale, float descale_q,
                                    float descale_k, float descale_v, int causal,
                                    hipStream_t stream) {
  if (!q || !k || !v || !out || !lse) return ATTN_PREFILL_ERR_NULL_PTR;
  if (B < 1 || Lq < 1 || Lk < 1 || n_q < 1 || n_kv < 1) return ATTN_PREFILL_ERR_BAD_SHAPE;
  if (n_q % n_kv != 0) return ATTN_PREFILL_ERR_BAD_GQA;
  if (d_h != kF8D) return ATTN_PREFILL_ERR_BAD_HEADDIM;
  if (!std::isfinite(scale) || !std::isfinite(descale_q) || !std::isfinite(descale_k) ||
      !std::isfinite(descale_v))
    return ATTN_PREFILL_ERR_BAD_SCALE;
  if (causal != 0 && causal != 1) return ATTN_PREFILL_ERR_BAD_CAUSAL;
  if (q_offset < 0 || (causal && (long long)q_offset + Lq > Lk)) return ATTN_PREFILL_ERR_BAD_OFFSET;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if ((align & 15) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3) != 0)
    return ATTN_PREFILL_ERR_MISALIGNED;
  size_t rows, q_elems, kv_elems;
  if (__builtin_mul_overflow((size_t)B, (size_t)n_q, &rows) ||
      __builtin_mul_overflow(rows, (size_t)Lq, &rows) ||
      __builtin_mul_overflow(rows, (size_t)d_h, &q_elems) ||
      __builtin_mul_overflow((size_t)B, (size_t)n_kv, &kv_elems) ||
      __builtin_mul_overflow(kv_elems, (size_t)Lk, &kv_elems) ||
      __builtin_mul_overflow(kv_elems, (size_t)d_h, &kv_elems) ||
      q_elems > ((size_t)1 << 61) || kv_elems > ((size_t)1 << 61))
    return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  // the scaled scores must stay finite in fp32
  const double c2d = (double)scale * descale_q * descale_k * 1.4426950408889634;
  if (!std::isfinite((float)c2d)) return ATTN_PREFILL_ERR_BAD_SCALE;
  const size_t qb = q_elems, kvb = kv_elems, ob = q_elems * 2, lb = rows * 4;
  if (overlaps(out, ob, q, qb) || overlaps(out, ob, k, kvb) || overlaps(out, ob, v, kvb) ||
      overlaps(out, ob, lse, lb) || overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kvb) ||
      overlaps(lse, lb, v, kvb))
    return ATTN_PREFILL_ERR_ALIASING;
  const float c2 = (float)c2d;
  switch (f8_pick_hwg(n_q / n_kv)) {
    case 8: return f8_launch<8>(q, k, v, out, lse, B, Lq, Lk, q_offset, n_q, n_kv, c2, descale_v, causal, stream);
    case 4: return f8_launch<4>(q, k, v, out, lse, B, Lq, Lk, q_offset, n_q, n_kv, c2, descale_v, causal, stream);
    case 2: return f8_launch<2>(q, k, v, out, lse, B, Lq, Lk, q_offset, n_q, n_kv, c2, descale_v, causal, stream);
    default: return f8_launch<1>(q, k, v, out, lse, B, Lq, Lk, q_offset, n_q, n_kv, c2, descale_v, causal, stream);
  }
}
