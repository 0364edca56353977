// attn_prefill.hip -- causal GQA prefill attention forward pass for gfx950.
//
// Method (prior art, restated for CDNA4):
//  * Tiled exact attention with an online softmax: for each block of queries,
//    stream tiles of keys and values, keep a running max m, a running sum l
//    and a running weighted sum acc per query row, rescale l and acc by
//    exp(m_old - m_new) when the max grows, divide once at the end ("Why
//    Attention Scaling Breaks", section "Flash Attention: the tiling
//    insight"; "Long-Context Attention Explained", sections "Tiling" and
//    "Online softmax", steps 1-5).
//  * Queries in the outer loop, one block of queries per workgroup, so the
//    work spreads over query blocks as well as heads ("Long-Context Attention
//    Explained", FlashAttention-2 paragraph; "Why Attention Scaling Breaks",
//    section "Flash Attention 2 and 3").
//  * Tiles whose keys all come after all queries of the block are never
//    visited; only tiles that straddle the diagonal are masked ("flops /
//    prefill-attention", section "Workarounds"; "Long-Context Attention
//    Explained", causal block skipping).
//  * Grouped-query heads: the query heads of one key/value head read the
//    same K/V tile from LDS, so K and V bytes are amortised over the group
//    ("flops / prefill-attention", section "Arithmetic intensity").
//  * Chunked prefill: the queries may be a chunk sitting at an offset into a
//    longer K/V (query row i at key position q_off + i, causal mask anchored
//    there), and two partial results over disjoint key sets merge by their
//    LSEs ("flops / prefill-attention", section "Workarounds"; "Long-Context
//    Attention Explained", section "Online softmax").
//
// CDNA4 mapping:
//  * A workgroup covers 256 query columns: HWG heads of one group times
//    BR = 256 / HWG rows.  By default it is 8 wave64s, two per SIMD, each
//    owning one block of 32 columns: the two waves of a SIMD cover each
//    other's latencies, and at d_h = 128 one wave's softmax work nearly fills
//    the issue slots next to its own MFMAs, so a lone wave per SIMD stalls.
//    Each K or V^T fragment read from LDS feeds one MFMA per block; the LDS
//    (measured ~250 B/clk/CU for 16-byte reads) has room for that.  The
//    kernel is also written for two blocks per wave (4 waves, one per SIMD,
//    each fragment feeding two MFMAs), selectable at build time.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand, Q (held in
//    VGPRs for the whole loop) the B operand.  In the 32x32 result lane l
//    holds 16 keys of query column l % 32, so the row max and row sum are
//    lane-local except for one exchange between lanes l and l ^ 32
//    (v_permlane32_swap).
//  * The output is accumulated transposed, O^T += V^T P^T, with V^T as the A
//    operand and P^T as the B operand.  The score result's register layout
//    is used directly as the B operand (the 16 keys a lane holds are the
//    contraction slots of two k-steps, in a permuted key order), so P never
//    leaves the registers.  V^T fragments in that key order come from the
//    row-major V tile through the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16: in each group of 16 lanes, lane 4r+q supplies four
//    consecutive 16-bit values of row r and lane i receives column i of the
//    four rows).
//  * K and V tiles of 64 keys go from global memory straight into LDS
//    (buffer loads with the LDS destination bit): a 4-tile ring each for K
//    and V, tiles requested three ahead, one barrier per tile.  The compute
//    runs in 32-key halves: the scores of the next half are formed on the
//    MFMA pipe while the softmax of the current half is on the VALU.
//  * The grid is persistent, one workgroup per CU walking a zigzag over the
//    heavy-first list of work items, and the ring runs on across items: the
//    next item's first tiles are requested into the slots the current
//    item's last tiles free, and its Q is loaded while the current output is
//    written, so an item no longer starts by waiting on HBM.
//  * LDS rows are XOR-swizzled in 16-byte chunks so the MFMA operand reads
//    do not collide on banks (see k_swz / v_swz).
//  * exp is exp2 with scale*log2(e) folded into one FMA; l and acc are only
//    rescaled when the running max grows by more than 2^8 (the result is
//    unchanged up to rounding: numerator and denominator share the stale
//    reference, and no weight exceeds 2^8); the row sum adds the fp32
//    weights before they are rounded to bf16 for P V; LSE is converted back
//    to the natural log at the end.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn_prefill.h"
#include "device_common.h"

namespace {

#ifndef ATTN_BLOCKS_PER_WAVE
#define ATTN_BLOCKS_PER_WAVE 1
#endif
// 32-column blocks per wave: 2 (4 waves, one per SIMD) or 1 (8 waves, two
// per SIMD); a workgroup always covers kCols query columns
constexpr int kBlocksPerWave = ATTN_BLOCKS_PER_WAVE;
constexpr int kCols = 256;            // query columns (head, row) per workgroup
constexpr int kBC = 64;               // keys per K/V tile
constexpr float kSlack = 8.0f;        // rescale only past 2^8 growth

// 16-byte chunk swizzles of the K and V tiles (row = key inside the tile).
// gfx950's LDS has 64 four-byte banks and serves 16 lanes of a 16-byte read
// or 32 lanes of an 8-byte read per cycle (measured: conflict counters are
// zero for contiguous reads).  K: the 16 lanes of a 16-byte read take 16
// consecutive rows at one chunk, so the chunk is XORed with the row's low
// bits to land on 16 distinct 16-byte slots of a 256-byte bank window.  V:
// the 32 lanes of a transpose read take 4 rows x 2 chunk pairs; XORing the
// chunk with 4 (row & 3) (d_h = 128) puts the 8 32-byte pieces on distinct
// slots.  For d_h = 64 two rows share a 256-byte window, hence the shifts.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

template <int D, int HWG, int NB>
__global__ __launch_bounds__(kCols / NB * 2) void attn_fwd_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, unsigned short* __restrict__ out,
    float* __restrict__ lse, int Lq, int Lk, int q_off, int n_q, int n_kv, int n_qblk,
    int items_per_qblk, int n_items, float scale, int causal) {
  constexpr int NW = kCols / (32 * NB);        // waves per workgroup
  constexpr int BR = kCols / HWG;              // query rows per workgroup
  constexpr int KSTEPS = D / 16;               // k-steps of Q K^T
  constexpr int TBLK = D / 32;                 // 32-row blocks of O^T
  constexpr int ROWB = 2 * D;                  // bytes per K or V row
  constexpr int TILE = kBC * ROWB;             // bytes per K or V tile
  constexpr int LOADS = TILE / (NW * 1024);    // 1 KB loads per wave per tile
  static_assert(LOADS * NW * 1024 == TILE, "tile must split into 1 KB loads");
  constexpr int RING = 4;                      // tiles per ring
  constexpr int VRING = 0;                     // V ring at [0, 4 TILE)
  constexpr int KRING = RING * TILE;           // K ring at [4 TILE, 8 TILE)

  // output staging: one 32-row output tile per (wave, block); half of them
  // in the last ring slot, the other half in an area after the rings
  constexpr int OT = 32 * ROWB;                // bytes of one block's output tile
  constexpr int STAGE = 2 * RING * TILE;       // staging area offset
  static_assert(4 * OT == 2 * TILE && NW * NB == 8, "half the output tiles fill one ring slot");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGE + 4 * OT];
  LDS_AS unsigned char* const smem_l = (LDS_AS unsigned char*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hi = lane >> 5;     // which half of the wave
  const int col = lane & 31;    // query column inside a 32-column block

  // ---- work items: (b, kv-head, head group, q-block), numbered heavy
  // q-blocks first with neighbouring numbers on different heads.  The grid
  // is persistent (at most one workgroup per CU) and round r covers items
  // r G .. r G + G - 1: workgroup w takes item r G + w when r is even and
  // the round's items backwards when r is odd, a zigzag over the
  // heavy-first list that evens out the causal work of the workgroups.
  // When G is a multiple of 8 the backward rounds are taken in blocks of 8
  // (w = 8 a + x takes r G + 8 (G / 8 - 1 - a) + x), so a workgroup only
  // sees items congruent to w mod 8: workgroups are dealt to the eight XCDs
  // in turn, so each XCD keeps working on the same (batch, kv-head) streams
  // when their count is a multiple of 8, and its L2 keeps serving their K/V.
  const int g = n_q / n_kv;
  const int ngroups = g / HWG;
  const size_t Lq64 = (size_t)Lq;
  auto item_at = [&] __device__ (int r) __attribute__((always_inline)) {
    const int G = gridDim.x;
    const int w = blockIdx.x;
    if (!(r & 1)) return r * G + w;
    if ((G & 7) == 0) return r * G + (G - 8 - (w & ~7)) + (w & 7);
    return r * G + G - 1 - w;
  };
  struct Geo {
    int qb, hg, kvh, b, n_tiles;  // n_tiles: K/V tiles the workgroup streams
    const unsigned short* kb;     // K and V rows of the item's kv-head
    const unsigned short* vb;
  };
  auto geo = [&] __device__ (int item) __attribute__((always_inline)) {
    Geo e;
    e.qb = n_qblk - 1 - item / items_per_qblk;
    int rest = item % items_per_qblk;
    e.hg = rest % ngroups;
    rest /= ngroups;
    e.kvh = rest % n_kv;
    e.b = rest / n_kv;
    // query row i sits at key position q_off + i; K and V hold Lk rows
    const int wg_end = min(e.qb * BR + BR, Lq);
    e.n_tiles = causal ? (wg_end + q_off + kBC - 1) / kBC : (Lk + kBC - 1) / kBC;
    e.kb = k + ((size_t)e.b * n_kv + e.kvh) * (size_t)Lk * D;
    e.vb = v + ((size_t)e.b * n_kv + e.kvh) * (size_t)Lk * D;
    return e;
  };
  // the wave's NB 32-column blocks: columns 32 (wave + NW ib) of the
  // workgroup, column c being head c / BR, row c % BR of the q-block
  auto blk_head = [&] __device__ (const Geo& e, int ib) __attribute__((always_inline)) {
    return e.kvh * g + e.hg * HWG + 32 * (wave + NW * ib) / BR;
  };
  auto blk_q0 = [&] __device__ (const Geo& e, int ib) __attribute__((always_inline)) {
    return e.qb * BR + 32 * (wave + NW * ib) % BR;
  };

  // ---- Q fragments (B operand of S^T = K Q^T): Q[row][16 kk + 8 hi + 0..7]
  bf16x8 qf[NB][KSTEPS];
  auto load_q = [&] __device__ (const Geo& e) __attribute__((always_inline)) {
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      const int qi = blk_q0(e, ib) + col;
      const unsigned short* qrow =
          q + (((size_t)e.b * n_q + blk_head(e, ib)) * Lq64 + (size_t)qi) * D;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qi < Lq) raw = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hi * 8);
        qf[ib][kk] = __builtin_bit_cast(bf16x8, raw);
      }
    }
  };

  // per-item state the pipeline reads: the wave's block heads and first
  // rows, the tiles the workgroup streams and the tiles this wave computes,
  // the K/V rows of this item and of the next one
  int hb[NB], q0b[NB];
  int n_tiles = 0, wave_tiles = 0;
  const unsigned short* kbase = k;
  const unsigned short* vbase = v;
  const unsigned short* nkbase = k;
  const unsigned short* nvbase = v;
  bool has_next = false;

  // ---- tile loads, global -> LDS.  Load s of this wave fills LDS bytes
  // [1 KB (wave * LOADS + s), +1 KB) of a tile; lane i fills 16 bytes at 16 i
  // with the chunk the row's swizzle puts there.  These source offsets do not
  // change from tile to tile.
  int k_src[LOADS], v_src[LOADS];
#pragma unroll
  for (int s = 0; s < LOADS; ++s) {
    const int byte = (wave * LOADS + s) * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int pos = (byte % ROWB) >> 4;
    k_src[s] = row * ROWB + ((pos ^ k_swz<D>(row)) << 4);
    v_src[s] = row * ROWB + ((pos ^ v_swz<D>(row)) << 4);
  }
  auto load_tile = [&] __device__ (const unsigned short* base, const int (&src)[LOADS], int tile,
                       int lds_off) __attribute__((always_inline)) {
    dma_tile(base, src, LOADS, ROWB, tile * kBC, Lk, kBC, smem + lds_off + wave * LOADS * 1024);
  };

  // ---- per-lane LDS read offsets
  // K rows col (+32 jb), the A operand of S^T = K Q^T, k-step kk
  int k_rd[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
    k_rd[kk] = KRING + col * ROWB + (((2 * kk + hi) ^ k_swz<D>(col)) << 4);
  // V^T through ds_read_b64_tr_b16: lane 16G + 4r + qq reads V[key][t .. t+3],
  // key = 16 ks + 8 u + 4 (G / 2) + r, t = 32 tb + 16 (G % 2) + 4 qq, and
  // receives V^T[32 tb + lane % 32][keys]
  int v_rd[TBLK];
  {
    const int tr_r = (lane >> 2) & 3;
    const int tr_q = lane & 3;
    const int tr_g = (lane >> 4) & 1;
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb) {
      const int t = 32 * tb + 16 * tr_g + 4 * tr_q;
      const int key = 4 * hi + tr_r;  // plus 16 ks + 8 u, which keep the swizzle
      v_rd[tb] = VRING + key * ROWB + (((t >> 3) ^ v_swz<D>(key)) << 4) + ((t >> 2) & 1) * 8;
    }
  }

  // ---- running state per block: reference max m (log2 domain), lane
  // partial row sum l, accumulator O^T
  f32x16 acc[NB][TBLK];
  float m_run[NB], l_run[NB];
  const float c2 = scale * kLog2e;
  const bool fast_scale = c2 > 0.0f;

  // K fragments of ring slot `slot`, keys 32 jb .. 32 jb + 31
  auto load_kfrags = [&] __device__ (bf16x8 (&kf)[KSTEPS], int slot, int jb) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      kf[kk] = *reinterpret_cast<const LDS_AS bf16x8*>(smem_l + k_rd[kk] + slot * TILE +
                                                       jb * 32 * ROWB);
  };
  // V^T fragments of ring slot `slot`, k-steps 2 jb and 2 jb + 1
  auto load_vfrags = [&] __device__ (bf16x8 (&vf)[TBLK][2], int slot, int jb) __attribute__((always_inline)) {
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const LDS_AS unsigned char* base =
            smem_l + v_rd[tb] + slot * TILE + (2 * jb + h) * 16 * ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(base));
        const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(base + 8 * ROWB));
        vf[tb][h] = __builtin_bit_cast(
            bf16x8, (u32x4){__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                            __builtin_bit_cast(u32x2, up)[0], __builtin_bit_cast(u32x2, up)[1]});
      }
  };

  // S^T = K Q^T for the wave's blocks, k-steps [k0, k1); each K fragment
  // feeds NB MFMAs.  k0 = 0 starts from zero.
  auto qk_mfma = [&] __device__ (f32x16 (&S)[NB], const bf16x8 (&kf)[KSTEPS], int k0, int k1)
      __attribute__((always_inline)) {
    if (k0 == 0) {
#pragma unroll
      for (int ib = 0; ib < NB; ++ib)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[ib][r] = 0.0f;
    }
#pragma unroll
    for (int kk = k0; kk < k1; ++kk)
#pragma unroll
      for (int ib = 0; ib < NB; ++ib)
        S[ib] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[ib][kk], S[ib], 0, 0, 0);
  };

  // O^T += V^T P^T for one block (the TBLK accumulators interleave, so no
  // MFMA waits on the one just issued)
  auto pv_mfma = [&] __device__ (const bf16x8 (&vf)[TBLK][2], const bf16x8 (&pk)[2], int ib) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb)
        acc[ib][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[tb][h], pk[h], acc[ib][tb], 0, 0, 0);
  };

  // row max of one block's 32 scores per lane pair (branch-free)
  auto row_max = [&] __device__ (const f32x16& s) __attribute__((always_inline)) {
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
    return pair_max(mx);
  };

  // softmax, first part, for the scores of keys j0 .. j0+31 (may branch):
  // where the half straddles the diagonal (query q0 + i sees keys up to
  // q_off + q0 + i) or the end of the keys, or the
  // scale is not positive, mask and pre-scale the scores and retake the row
  // max; then move the reference max (rescaling l and acc) only when the
  // tile max exceeds it by more than 2^8.  Returns the multiplier and -m.
  auto prepare = [&] __device__ (f32x16& s, float mx, int ib, int j0, float& c_out,
                                 float& mneg_out) __attribute__((always_inline)) {
    const int q0 = q0b[ib];
    const int qi = q0 + col;
    const bool need_mask = (causal && j0 + 31 > q0 + q_off) || (j0 + 32 > Lk);
    float c = c2;
    if (need_mask || !fast_scale) {
      // score r of this lane is key j0 + 4 hi + o_r, o_r = 8 (r / 4) + r % 4,
      // visible to query qi (at key position qi + q_off) iff o_r <= lim.  A
      // scale <= 0 is applied before masking, so that a masked score stays
      // -inf; a positive one later, in the exponential.
      const int lim = (causal ? min(qi + q_off, Lk - 1) : Lk - 1) - j0 - 4 * hi;
      const float cm = fast_scale ? 1.0f : c2;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = (r >> 2) * 8 + (r & 3) > lim ? -INFINITY : s[r] * cm;
      c = fast_scale ? c2 : 1.0f;
      mx = row_max(s);
    }
    const float m_cand = mx * c;
    if (__builtin_amdgcn_ballot_w64(m_cand > m_run[ib] + kSlack) != 0) {
      const float m_new = fmaxf(m_run[ib], m_cand);
      const float alpha = __builtin_amdgcn_exp2f(m_run[ib] - m_new);
      m_run[ib] = m_new;
      l_run[ib] *= alpha;
#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ib][tb][r] *= alpha;
    }
    c_out = c;
    mneg_out = -m_run[ib];
  };

  // softmax, second part (branch-free): p = 2^(c s - m), the fp32 row sum,
  // and P^T rounded to bf16 as two B-operand fragments
  auto expo = [&] __device__ (const f32x16& s, int ib, float c, float mneg, bf16x8 (&pk)[2])
      __attribute__((always_inline)) {
    float psum = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 frag;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[half * 8 + e], c, mneg));
        psum += p;
        frag[e] = (__bf16)p;
      }
      pk[half] = frag;
    }
    l_run[ib] += psum;
  };

  // Software pipeline over 32-key half-steps h = 2 t + jb.  Entering the
  // region of half h: the raw scores of h are in registers, as are the K
  // fragments of half h+1 and the V^T fragments of half h.  The region first
  // puts a few QK^T MFMAs of h+1 on the pipe (they need nothing from the
  // softmax) and, in the first half of a tile, issues the tile loads; while
  // those run it takes the row max and the first softmax part of h (mask and
  // rescale decisions, rarely taken branches).  Then, branch-free: the rest
  // of the scores of h+1 next to the exponentials of h, block by block, each
  // followed by its P V, with the K fragments of h+2 and the V^T fragments
  // of h+1 read from LDS meanwhile.  Past the wave's last half the region
  // computes on stale LDS data whose results are never used.
  struct Half {
    f32x16 s[NB];
    bf16x8 kf[KSTEPS];
    bf16x8 vf[TBLK][2];
  };
  Half hA, hB;
  constexpr int KA = NB == 2 ? 3 : 2;  // k-steps of h+1 issued ahead of the branches

  // Tile t of an item sits in ring slot t % 4; the ring runs on across
  // items.  During tile t the workgroup requests stream position t + 3 into
  // the slot tile t - 1 has freed: tile t + 3 of this item, or, past its last
  // tile, tile j of the next item when the slot is j < 3 (so most of the
  // next item's first tiles arrive while this one finishes).  Every tile
  // step issues the same number of loads (otherwise a tile of this item past
  // its end: rows that are never used, or zeros), which keeps the vmcnt
  // counts exact and the step free of branches.
  auto issue_tile_loads = [&] __device__ (int TS, int t) __attribute__((always_inline)) {
    const int p = t + 3;
    const int slot = (TS + 3) & (RING - 1);
    const bool own = p < n_tiles || !has_next || slot == RING - 1;
    const int tile = own ? p : slot;
    load_tile(own ? vbase : nvbase, v_src, tile, VRING + slot * TILE);
    load_tile(own ? kbase : nkbase, k_src, tile, KRING + slot * TILE);
  };

  auto region = [&] __device__ (int t, int ts, int jb, Half& cur, Half& nxt)
      __attribute__((always_inline)) {
    // ring slots and key halves of h+1 and h+2
    const int slot1 = jb == 0 ? ts : (ts + 1) & (RING - 1);
    const int jb1 = jb ^ 1;
    const int slot2 = (ts + 1) & (RING - 1);
    const int jb2 = jb;
    // keep the scheduler from pulling this region's row max up next to the
    // previous region's last MFMAs (whose results it would then stall on)
    __builtin_amdgcn_sched_barrier(0);
    qk_mfma(nxt.s, cur.kf, 0, KA);
    if (jb == 0) issue_tile_loads(ts, t);
    float cc[NB], mn[NB];
    const int j0 = t * kBC + jb * 32;
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) prepare(cur.s[ib], row_max(cur.s[ib]), ib, j0, cc[ib], mn[ib]);
    load_kfrags(nxt.kf, slot2, jb2);
    load_vfrags(nxt.vf, slot1, jb1);
    qk_mfma(nxt.s, cur.kf, KA, KSTEPS);
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      bf16x8 pk[2];
      expo(cur.s[ib], ib, cc[ib], mn[ib], pk);
      pv_mfma(cur.vf, pk, ib);
    }
  };

  // one tile t in ring slot TS (a constant once inlined): the loads of
  // stream position t + 3 fly during this tile and the next two; at its end
  // the loads issued during the previous tile (the tile the next step reads
  // ahead) must have landed
  auto tile_step = [&] __device__ (int TS, int t) __attribute__((always_inline)) {
    if (t < wave_tiles) {
      region(t, TS, 0, hA, hB);
      region(t, TS, 1, hB, hA);
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
  for (int j = 0; j < 3; ++j) {
    load_tile(cur.kb, k_src, j, KRING + j * TILE);
    load_tile(cur.vb, v_src, j, VRING + j * TILE);
  }
  for (;;) {
    // ---- item setup
    const int nxt_item = item_at(r + 1);
    has_next = nxt_item < n_items;
    const Geo nx = geo(has_next ? nxt_item : item);
    kbase = cur.kb;
    vbase = cur.vb;
    nkbase = nx.kb;
    nvbase = nx.vb;
    n_tiles = cur.n_tiles;
    int last_row = -1;
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      hb[ib] = blk_head(cur, ib);
      q0b[ib] = blk_q0(cur, ib);
      if (q0b[ib] < Lq) last_row = max(last_row, min(q0b[ib] + 31, Lq - 1));
    }
    wave_tiles = last_row < 0 ? 0 : (causal ? (last_row + q_off) / kBC + 1 : n_tiles);
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[ib][tb][e] = 0.0f;
      m_run[ib] = -INFINITY;
      l_run[ib] = 0.0f;
    }

    // ---- prologue: the item's tiles 0..2 and its Q have landed (and the
    // previous item's stores are done); then the raw scores of half 0, the K
    // fragments of half 1 and the V^T fragments of half 0 in registers
    wait_vmcnt<0>();
    tile_barrier();
    if (wave_tiles > 0) {
      load_kfrags(hB.kf, 0, 0);
      qk_mfma(hA.s, hB.kf, 0, KSTEPS);
      load_kfrags(hA.kf, 0, 1);
      load_vfrags(hA.vf, 0, 0);
    }

    // ---- the item's tiles
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
      // the next item's tiles 0..2 that the last tile steps could not
      // request (the one whose slot held this item's last tile, and those
      // of a short item), now that every slot is free; then its Q, all
      // landing while this item's output is written
      int req = 0;   // slots the tile steps filled with the next item's tiles
      for (int t = max(0, n_tiles - 3); t < n_tiles; ++t) req |= 1 << ((t + 3) & (RING - 1));
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (!((req >> j) & 1)) {
          load_tile(nkbase, k_src, j, KRING + j * TILE);
          load_tile(nvbase, v_src, j, VRING + j * TILE);
        }
      load_q(nx);
    }

    // ---- epilogue: O = acc / l in bf16, LSE = ln 2 * (m + log2 l).  Each
    // block's 32 x d_h output tile goes through LDS (ring slot 3, or the
    // staging area) so that the global stores are whole rows: 1 KB
    // per store instruction instead of 8-byte pieces of 32 different rows.
    // (The lane id is re-derived here, opaque to the compiler, so that the
    // staging addresses are computed in place instead of being kept, or
    // spilled, across the tile loop.)
    int elane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(elane));
    const int ecol = elane & 31;
    const int ehi = elane >> 5;
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      const float l_tot = pair_sum(l_run[ib]);
      const float inv = 1.0f / l_tot;
      const int q0 = q0b[ib];
      if (hi == 0 && q0 + col < Lq && wave_tiles > 0)
        lse[((size_t)cur.b * n_q + hb[ib]) * Lq64 + (size_t)(q0 + col)] =
            (m_run[ib] + __log2f(l_tot)) * kLn2;
      const int idx = wave * NB + ib;
      LDS_AS unsigned char* ot =
          smem_l + (idx < 2 ? VRING + 3 * TILE + idx * OT
                            : idx < 4 ? KRING + 3 * TILE + (idx - 2) * OT : STAGE + (idx - 4) * OT);
      // lane (col, hi) holds row col, columns 32 tb + 8 grp + 4 hi + 0..3
#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[ib][tb][grp * 4 + e] * inv);
          const int chunk = tb * 4 + grp;                  // 16-byte chunk of the row
          *reinterpret_cast<LDS_AS u32x2*>(ot + ecol * ROWB + ((chunk ^ k_swz<D>(ecol)) << 4) +
                                           ehi * 8) = __builtin_bit_cast(u32x2, o4);
        }
      // read back whole rows: store st covers rows 1024 st / ROWB onwards
      unsigned short* obase = out + (((size_t)cur.b * n_q + hb[ib]) * Lq64 + (size_t)q0) * D;
#pragma unroll
      for (int st = 0; st < OT / 1024; ++st) {
        const int byte = st * 1024 + elane * 16;
        const int row = byte / ROWB;
        const int chunk = (byte % ROWB) >> 4;
        const u32x4 v4 =
            *reinterpret_cast<const LDS_AS u32x4*>(ot + row * ROWB + ((chunk ^ k_swz<D>(row)) << 4));
        if (q0 + row < Lq && wave_tiles > 0)
          *reinterpret_cast<u32x4*>(obase + (size_t)row * D + chunk * 8) = v4;
      }
    }
    if (!has_next) break;
    cur = nx;
    item = nxt_item;
    ++r;
  }
  wait_vmcnt<0>();   // no tile load may still be writing LDS when the wave ends
}

// Heads per workgroup: the largest of 8, 4, 2, 1 that divides g.
int pick_hwg(int g) {
  if (g % 8 == 0) return 8;
  if (g % 4 == 0) return 4;
  if (g % 2 == 0) return 2;
  return 1;
}

// Sizes of one call; Lq = Lk and q_off = 0 for a whole-sequence prefill.
struct Shape {
  int B, Lq, Lk, q_off, n_q, n_kv, d_h;
};

template <int D, int HWG>
int launch(const void* q, const void* k, const void* v, void* out, float* lse, const Shape& sh,
           float scale, int causal, hipStream_t stream) {
  constexpr int NB = kBlocksPerWave;
  constexpr int BR = kCols / HWG;
  const int n_qblk = (sh.Lq + BR - 1) / BR;
  const long long items_per_qblk = (long long)sh.B * sh.n_kv * ((sh.n_q / sh.n_kv) / HWG);
  const long long n_items = items_per_qblk * n_qblk;
  // (round r of the persistent schedule computes r G + w, which must not wrap)
  if (items_per_qblk > INT_MAX || n_items > INT_MAX / 2) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  // persistent grid: one workgroup per CU (a workgroup's LDS rings fill most
  // of a CU's LDS), never more than there are items
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu < 1)
    return ATTN_PREFILL_ERR_LAUNCH;
  const long long grid = n_items < n_cu ? n_items : n_cu;
  hipLaunchKernelGGL((attn_fwd_kernel<D, HWG, NB>), dim3((unsigned)grid), dim3(kCols / NB * 2), 0,
                     stream,
                     static_cast<const unsigned short*>(q), static_cast<const unsigned short*>(k),
                     static_cast<const unsigned short*>(v), static_cast<unsigned short*>(out), lse,
                     sh.Lq, sh.Lk, sh.q_off, sh.n_q, sh.n_kv, n_qblk, (int)items_per_qblk,
                     (int)n_items, scale, causal);
  return hipGetLastError() == hipSuccess ? ATTN_PREFILL_OK : ATTN_PREFILL_ERR_LAUNCH;
}

template <int D>
int launch_d(const void* q, const void* k, const void* v, void* out, float* lse, const Shape& sh,
             float scale, int causal, hipStream_t stream) {
  switch (pick_hwg(sh.n_q / sh.n_kv)) {
    case 8: return launch<D, 8>(q, k, v, out, lse, sh, scale, causal, stream);
    case 4: return launch<D, 4>(q, k, v, out, lse, sh, scale, causal, stream);
    case 2: return launch<D, 2>(q, k, v, out, lse, sh, scale, causal, stream);
    default: return launch<D, 1>(q, k, v, out, lse, sh, scale, causal, stream);
  }
}

// Argument checks shared by the entry points, then the launch.
int check_and_launch(const void* q, const void* k, const void* v, void* out, float* lse,
                     const Shape& sh, float scale, int causal, hipStream_t stream) {
  if (!q || !k || !v || !out || !lse) return ATTN_PREFILL_ERR_NULL_PTR;
  if (sh.B < 1 || sh.Lq < 1 || sh.Lk < 1 || sh.n_q < 1 || sh.n_kv < 1)
    return ATTN_PREFILL_ERR_BAD_SHAPE;
  if (sh.n_q % sh.n_kv != 0) return ATTN_PREFILL_ERR_BAD_GQA;
  if (sh.d_h != 64 && sh.d_h != 128) return ATTN_PREFILL_ERR_BAD_HEADDIM;
  if (!std::isfinite(scale)) return ATTN_PREFILL_ERR_BAD_SCALE;
  if (causal != 0 && causal != 1) return ATTN_PREFILL_ERR_BAD_CAUSAL;
  if (sh.q_off < 0 || (causal && (long long)sh.q_off + sh.Lq > sh.Lk))
    return ATTN_PREFILL_ERR_BAD_OFFSET;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if ((align & 15) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3) != 0)
    return ATTN_PREFILL_ERR_MISALIGNED;

  // element counts, checked for 64-bit overflow (bytes must fit in 2^62)
  size_t lse_elems, q_elems, kv_rows, kv_elems;
  if (__builtin_mul_overflow((size_t)sh.B, (size_t)sh.n_q, &lse_elems) ||
      __builtin_mul_overflow(lse_elems, (size_t)sh.Lq, &lse_elems) ||
      __builtin_mul_overflow(lse_elems, (size_t)sh.d_h, &q_elems) ||
      __builtin_mul_overflow((size_t)sh.B, (size_t)sh.n_kv, &kv_rows) ||
      __builtin_mul_overflow(kv_rows, (size_t)sh.Lk, &kv_rows) ||
      __builtin_mul_overflow(kv_rows, (size_t)sh.d_h, &kv_elems) ||
      q_elems > ((size_t)1 << 61) || kv_elems > ((size_t)1 << 61))
    return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  const size_t q_bytes = q_elems * 2, kv_bytes = kv_elems * 2, lse_bytes = lse_elems * 4;
  if (overlaps(out, q_bytes, q, q_bytes) || overlaps(out, q_bytes, k, kv_bytes) ||
      overlaps(out, q_bytes, v, kv_bytes) || overlaps(out, q_bytes, lse, lse_bytes) ||
      overlaps(lse, lse_bytes, q, q_bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
      overlaps(lse, lse_bytes, v, kv_bytes))
    return ATTN_PREFILL_ERR_ALIASING;

  if (sh.d_h == 128) return launch_d<128>(q, k, v, out, lse, sh, scale, causal, stream);
  return launch_d<64>(q, k, v, out, lse, sh, scale, causal, stream);
}

// ---- merge of two partial results over disjoint key sets ("Long-Context
// Attention Explained", section "Online softmax": the running max and sum of
// two parts combine by rescaling each to the larger max).  One thread per 8
// elements of a row; d_h / 8 threads per row.
__global__ __launch_bounds__(256) void merge_kernel(
    const unsigned short* __restrict__ oa, const float* __restrict__ la,
    const unsigned short* __restrict__ ob, const float* __restrict__ lb,
    unsigned short* __restrict__ out, float* __restrict__ lo, long long rows, int d_h) {
  const int per_row = d_h / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = gid / per_row;
  if (row >= rows) return;
  const int c8 = (int)(gid % per_row) * 8;
  const float a = la[row], bb = lb[row];
  const float m = fmaxf(a, bb);
  // a side with lse = -inf (no visible key) gets weight 0; both: O = 0, lse -inf
  const float wa = a == -INFINITY ? 0.0f : __expf(a - m);
  const float wb = bb == -INFINITY ? 0.0f : __expf(bb - m);
  const float sum = wa + wb;
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
  // a weight-0 side adds nothing, even if its o holds NaN or garbage: its
  // bits are masked to zero (integer arithmetic, which no floating-point
  // assumption of the compiler can fold away)
  const unsigned keep_a = wa > 0.0f ? 0xffffffffu : 0u;
  const unsigned keep_b = wb > 0.0f ? 0xffffffffu : 0u;
  const u32x4 va = *reinterpret_cast<const u32x4*>(oa + row * d_h + c8);
  const u32x4 vb = *reinterpret_cast<const u32x4*>(ob + row * d_h + c8);
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 xa = __builtin_bit_cast(bf16x2, va[e] & keep_a);
    const bf16x2 xb = __builtin_bit_cast(bf16x2, vb[e] & keep_b);
    bf16x2 y;
    y[0] = (__bf16)(((float)xa[0] * wa + (float)xb[0] * wb) * inv);
    y[1] = (__bf16)(((float)xa[1] * wa + (float)xb[1] * wb) * inv);
    r[e] = __builtin_bit_cast(unsigned, y);
  }
  *reinterpret_cast<u32x4*>(out + row * d_h + c8) = r;
  if (c8 == 0) lo[row] = sum > 0.0f ? m + __logf(sum) : -INFINITY;
}

// ---- decode: one new query per sequence against its whole K/V cache.  The
// query is a single vector, so attention is a matrix-vector product against
// the cache and its time is the cache bytes over the memory bandwidth
// ("Memory-bound vs compute-bound", sections "Prefill against decode" and
// "Attention itself"; "Long-Context Attention Explained", the paragraphs on
// prefill against decode).
//
// decode_split_kernel: work item = (b, kv-head, key range).  Four waves per
// workgroup and two workgroups per CU (65 KB of LDS each), two waves per SIMD
// so that one computes while the other waits for memory; wave w streams the
// 32-key tiles w, w + 4, ... of the range through its own LDS (K tile, V tile) with the same DMA loads, swizzles and fragment
// reads as the prefill kernel, and forms the g query heads of the group as
// the 32 columns of S^T = K Q^T (columns >= g hold zero queries and are
// never stored).  The waves' running states merge in LDS at the end, and the
// workgroup writes one fp32 partial per query head: O normalised by the
// range's own row sum, and the range's LSE.
// decode_combine_kernel then merges the partials of each row by their LSEs
// (the online-softmax combination, "Long-Context Attention Explained",
// section "Online softmax").
constexpr int kDecWaves = 4;
constexpr int kDecTile = 32;          // keys per wave tile
constexpr int kDecSlots = 512;        // workgroups resident at once (two per CU)
constexpr int kDecMaxSplits = 4096;   // partials per row the combine stages in LDS

template <int D>
__global__ __launch_bounds__(64 * kDecWaves) void decode_split_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    int Lk, long long kv_cap, int n_q, int n_kv, int n_split, int split_keys, float scale) {
  constexpr int KSTEPS = D / 16;
  constexpr int TBLK = D / 32;
  constexpr int ROWB = 2 * D;
  constexpr int TILE = kDecTile * ROWB;      // bytes of one 32-key K or V tile
  constexpr int LOADS = TILE / 1024;         // 1 KB loads per tile, one wave
  constexpr int WAVE_LDS = 2 * TILE;         // a wave's K tile then its V tile
  static_assert(32 * D * 4 <= WAVE_LDS, "a wave's accumulators must fit its LDS");

  __shared__ __attribute__((aligned(1024))) unsigned char smem[kDecWaves * WAVE_LDS];
  __shared__ float st_ml[kDecWaves][64];     // each wave's m[32] and l[32]
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hi = lane >> 5;
  const int col = lane & 31;
  unsigned char* const wbuf = smem + wave * WAVE_LDS;
  LDS_AS unsigned char* const wl = (LDS_AS unsigned char*)wbuf;

  const int item = blockIdx.x;
  const int split = item % n_split;
  const int rest = item / n_split;
  const int kvh = rest % n_kv;
  const int b = rest / n_kv;
  const int g = n_q / n_kv;
  const int j_begin = split * split_keys;
  const int j_end = min(Lk, j_begin + split_keys);
  const unsigned short* kbase = k + ((size_t)b * n_kv + kvh) * (size_t)kv_cap * D;
  const unsigned short* vbase = v + ((size_t)b * n_kv + kvh) * (size_t)kv_cap * D;

  // Q^T as the B operand: column col is query head kvh * g + col
  bf16x8 qf[KSTEPS];
  {
    const unsigned short* qrow = q + ((size_t)b * n_q + (size_t)kvh * g + col) * D;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (col < g) raw = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hi * 8);
      qf[kk] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // tile-load source offsets (the wave moves a whole tile: LOADS loads of
  // 1 KB) and fragment read offsets, as in the prefill kernel
  int k_src[LOADS], v_src[LOADS];
#pragma unroll
  for (int s = 0; s < LOADS; ++s) {
    const int byte = s * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int pos = (byte % ROWB) >> 4;
    k_src[s] = row * ROWB + ((pos ^ k_swz<D>(row)) << 4);
    v_src[s] = row * ROWB + ((pos ^ v_swz<D>(row)) << 4);
  }
  int k_rd[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
    k_rd[kk] = col * ROWB + (((2 * kk + hi) ^ k_swz<D>(col)) << 4);
  int v_rd[TBLK];
  {
    const int tr_r = (lane >> 2) & 3;
    const int tr_q = lane & 3;
    const int tr_g = (lane >> 4) & 1;
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb) {
      const int t = 32 * tb + 16 * tr_g + 4 * tr_q;
      const int key = 4 * hi + tr_r;
      v_rd[tb] = TILE + key * ROWB + (((t >> 3) ^ v_swz<D>(key)) << 4) + ((t >> 2) & 1) * 8;
    }
  }

  f32x16 acc[TBLK];
#pragma unroll
  for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tb][r] = 0.0f;
  float m_run = -INFINITY;   // log2 domain
  float l_run = 0.0f;        // this lane's part of the row sum
  const float c2 = scale * kLog2e;

  for (int t0 = j_begin + wave * kDecTile; t0 < j_end; t0 += kDecWaves * kDecTile) {
    wait_lgkm0();   // the previous tile's LDS reads are done before it is overwritten
    dma_tile(kbase, k_src, LOADS, ROWB, t0, j_end, kDecTile, wbuf);
    dma_tile(vbase, v_src, LOADS, ROWB, t0, j_end, kDecTile, wbuf + TILE);
    wait_vmcnt<0>();
    {
      constexpr int jb = 0;
      const int j0 = t0;
      bf16x8 kf[KSTEPS];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        kf[kk] = *reinterpret_cast<const LDS_AS bf16x8*>(wl + k_rd[kk] + jb * 32 * ROWB);
      f32x16 sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], sc, 0, 0, 0);
      // keys past the range are masked; j0 itself is always a key, so every
      // column's max is finite
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + (r >> 2) * 8 + hi * 4 + (r & 3);
        sc[r] = j < j_end ? sc[r] * c2 : -INFINITY;
        mx = fmaxf(mx, sc[r]);
      }
      const float m_new = fmaxf(m_run, pair_max(mx));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      bf16x8 pk[2];
      float psum = 0.0f;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sc[half * 8 + e] - m_new);
          psum += p;
          pk[half][e] = (__bf16)p;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tb][r] *= alpha;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int tb = 0; tb < TBLK; ++tb) {
          const LDS_AS unsigned char* base = wl + v_rd[tb] + (2 * jb + h) * 16 * ROWB;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(base));
          const s16x4 up =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(base + 8 * ROWB));
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, (u32x4){__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                              __builtin_bit_cast(u32x2, up)[0], __builtin_bit_cast(u32x2, up)[1]});
          acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk[h], acc[tb], 0, 0, 0);
        }
    }
  }

  // ---- merge the waves' states in LDS: wave w leaves m[32], l[32] in
  // st_ml[w] and its unnormalised O as [32 columns][D] fp32 in its own LDS
  const float l_tot = pair_sum(l_run);
  __syncthreads();   // every wave is past its last LDS read and tile load
  {
    float* acc_out = reinterpret_cast<float*>(wbuf);
    if (hi == 0) {
      st_ml[wave][col] = m_run;
      st_ml[wave][32 + col] = l_tot;
    }
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        float4 o4;
        o4.x = acc[tb][grp * 4 + 0];
        o4.y = acc[tb][grp * 4 + 1];
        o4.z = acc[tb][grp * 4 + 2];
        o4.w = acc[tb][grp * 4 + 3];
        *reinterpret_cast<float4*>(acc_out + col * D + 32 * tb + 8 * grp + 4 * hi) = o4;
      }
  }
  __syncthreads();
  // thread e of the workgroup takes elements e, e + 256, ... of [g][D]
  for (int e = tid; e < g * D; e += 64 * kDecWaves) {
    const int c = e / D;
    const int d = e % D;
    float mw[kDecWaves];
    float m_all = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      mw[w] = st_ml[w][c];
      m_all = fmaxf(m_all, mw[w]);
    }
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float* acc_w = reinterpret_cast<const float*>(smem + w * WAVE_LDS);
      // a wave without a tile has m = -inf, l = 0 and O = 0: weight 0
      const float f = __builtin_amdgcn_exp2f(mw[w] - m_all);
      den += f * st_ml[w][32 + c];
      num += f * acc_w[c * D + d];
    }
    const size_t prow = ((size_t)b * n_q + (size_t)kvh * g + c) * n_split + split;
    ws_o[prow * D + d] = num / den;
    if (d == 0) ws_lse[prow] = (m_all + __log2f(den)) * kLn2;
  }
}

// decode_combine_kernel: one workgroup of 256 threads per query row merges
// the row's n_split fp32 partials by their LSEs: M = max lse, w_s =
// exp(lse_s - M), O = sum w_s o_s / sum w_s (rounded once to bf16),
// LSE = M + ln sum w_s.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    unsigned short* __restrict__ out, float* __restrict__ lse, int n_split) {
  constexpr int C4 = D / 4;            // float4 columns of a row
  constexpr int SG = 256 / C4;         // split groups
  __shared__ float w_s[kDecMaxSplits];
  __shared__ float red[8];
  __shared__ float4 part[SG][C4];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const float* lrow = ws_lse + row * n_split;
  const float* orow = ws_o + row * n_split * D;

  // M: strided max, then across the wave (butterfly) and the four waves
  float m = -INFINITY;
  for (int s = tid; s < n_split; s += 256) {
    const float x = lrow[s];
    w_s[s] = x;
    m = fmaxf(m, x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // weights and their sum
  float wsum = 0.0f;
  for (int s = tid; s < n_split; s += 256) {
    const float w = __expf(w_s[s] - m);
    w_s[s] = w;
    wsum += w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wsum += __shfl_xor(wsum, o);
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = wsum;
  __syncthreads();
  wsum = (red[4] + red[5]) + (red[6] + red[7]);
  // weighted sum of the partial outputs: thread (sg, c4) takes splits sg, sg + SG, ...
  const int c4 = tid % C4;
  const int sg = tid / C4;
  float4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int s = sg; s < n_split; s += SG) {
    const float w = w_s[s];
    const float4 o = *reinterpret_cast<const float4*>(orow + (size_t)s * D + 4 * c4);
    a.x += w * o.x;
    a.y += w * o.y;
    a.z += w * o.z;
    a.w += w * o.w;
  }
  part[sg][c4] = a;
  __syncthreads();
  if (tid < C4) {
    float4 t = part[0][tid];
    for (int g2 = 1; g2 < SG; ++g2) {
      const float4 u = part[g2][tid];
      t.x += u.x;
      t.y += u.y;
      t.z += u.z;
      t.w += u.w;
    }
    const float inv = 1.0f / wsum;
    bf16x4 y;
    y[0] = (__bf16)(t.x * inv);
    y[1] = (__bf16)(t.y * inv);
    y[2] = (__bf16)(t.z * inv);
    y[3] = (__bf16)(t.w * inv);
    *reinterpret_cast<u32x2*>(out + row * D + 4 * tid) = __builtin_bit_cast(u32x2, y);
    if (tid == 0) lse[row] = m + __logf(wsum);
  }
}

// Key ranges of a decode call.  Two workgroups fill a CU (their LDS), so the
// workgroups run in rounds of 512 and a call takes about (rounds) x (keys per
// range + a fixed cost per workgroup).  Ranges are multiples of 256 keys (each of the four waves gets
// whole 32-key tiles); the count per row is chosen to minimise that product,
// preferring fewer ranges (less to combine), and never exceeds
// kDecMaxSplits.
struct DecodeSplit {
  int n_split, split_keys;
};
DecodeSplit decode_split(int B, int Lk, int n_kv) {
  const long long pairs = (long long)B * n_kv;
  const long long chunks = ((long long)Lk + 255) / 256;   // 256-key pieces
  const long long max_n = chunks < kDecMaxSplits ? chunks : kDecMaxSplits;
  long long best_n = 1, best_per = chunks * 256, best_cost = -1;
  // visit each distinct range length once: q = ceil(chunks / n) 256-key pieces
  for (long long n = 1; n <= max_n;) {
    const long long q = (chunks + n - 1) / n;
    const long long per = q * 256;                                // keys per range
    const long long n_act = ((long long)Lk + per - 1) / per;      // ranges actually used
    const long long rounds = (pairs * n_act + kDecSlots - 1) / kDecSlots;
    // keys x rounds, with each workgroup's start and merge costing about
    // 256 keys' worth of streaming; then fewer ranges
    const long long cost = rounds * (per + 256) * 64 + n_act;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_n = n_act;
      best_per = per;
    }
    if (q == 1) break;
    n = (chunks + q - 2) / (q - 1);   // the first n with fewer pieces per range
  }
  return DecodeSplit{(int)best_n, (int)best_per};
}

}  // namespace

extern "C" int attn_prefill_fwd(const void* q, const void* k, const void* v, void* out,
                                float* lse, int B, int L, int n_q, int n_kv, int d_h,
                                float scale, int causal, hipStream_t stream) {
  return check_and_launch(q, k, v, out, lse, Shape{B, L, L, 0, n_q, n_kv, d_h}, scale, causal,
                          stream);
}

extern "C" int attn_prefill_fwd_chunk(const void* q, const void* k, const void* v, void* out,
                                      float* lse, int B, int Lq, int Lk, int q_offset, int n_q,
                                      int n_kv, int d_h, float scale, int causal,
                                      hipStream_t stream) {
  return check_and_launch(q, k, v, out, lse, Shape{B, Lq, Lk, q_offset, n_q, n_kv, d_h}, scale,
                          causal, stream);
}

extern "C" int attn_merge_partials(const void* o_a, const float* lse_a, const void* o_b,
                                   const float* lse_b, void* out, float* lse_out, long long rows,
                                   int d_h, hipStream_t stream) {
  if (!o_a || !lse_a || !o_b || !lse_b || !out || !lse_out) return ATTN_PREFILL_ERR_NULL_PTR;
  if (rows < 1) return ATTN_PREFILL_ERR_BAD_SHAPE;
  if (d_h != 64 && d_h != 128) return ATTN_PREFILL_ERR_BAD_HEADDIM;
  const uintptr_t align = reinterpret_cast<uintptr_t>(o_a) | reinterpret_cast<uintptr_t>(o_b) |
                          reinterpret_cast<uintptr_t>(out);
  const uintptr_t align4 = reinterpret_cast<uintptr_t>(lse_a) |
                           reinterpret_cast<uintptr_t>(lse_b) |
                           reinterpret_cast<uintptr_t>(lse_out);
  if ((align & 15) != 0 || (align4 & 3) != 0) return ATTN_PREFILL_ERR_MISALIGNED;
  size_t elems;
  if (__builtin_mul_overflow((size_t)rows, (size_t)d_h, &elems) || elems > ((size_t)1 << 61))
    return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  const size_t ob = elems * 2, lb = (size_t)rows * 4;
  // out may not overlap anything; inputs may overlap each other (read only)
  if (overlaps(out, ob, o_a, ob) || overlaps(out, ob, o_b, ob) || overlaps(out, ob, lse_a, lb) ||
      overlaps(out, ob, lse_b, lb) || overlaps(out, ob, lse_out, lb) ||
      overlaps(lse_out, lb, o_a, ob) || overlaps(lse_out, lb, o_b, ob) ||
      overlaps(lse_out, lb, lse_a, lb) || overlaps(lse_out, lb, lse_b, lb))
    return ATTN_PREFILL_ERR_ALIASING;
  const long long threads = (long long)rows * (d_h / 8);
  const long long blocks = (threads + 255) / 256;
  if (blocks > INT_MAX) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const unsigned short*>(o_a), lse_a,
                     static_cast<const unsigned short*>(o_b), lse_b,
                     static_cast<unsigned short*>(out), lse_out, rows, d_h);
  return hipGetLastError() == hipSuccess ? ATTN_PREFILL_OK : ATTN_PREFILL_ERR_LAUNCH;
}

extern "C" size_t attn_decode_workspace_bytes(int B, int Lk, int n_q, int n_kv, int d_h) {
  if (B < 1 || Lk < 1 || n_q < 1 || n_kv < 1 || n_q % n_kv != 0) return 0;
  if (n_q / n_kv > 32 || Lk > INT_MAX - 4096) return 0;
  if (d_h != 64 && d_h != 128) return 0;
  const DecodeSplit sp = decode_split(B, Lk, n_kv);
  size_t rows;
  if (__builtin_mul_overflow((size_t)B, (size_t)n_q, &rows) ||
      __builtin_mul_overflow(rows, (size_t)sp.n_split, &rows))
    return 0;
  // fp32 partial outputs [rows][d_h], then fp32 partial LSEs [rows]
  size_t bytes;
  if (__builtin_mul_overflow(rows, (size_t)(d_h + 1) * 4, &bytes)) return 0;
  return bytes;
}

namespace {

// Checks of a decode call's arguments other than the workspace; fills the
// byte sizes of q/out, k/v and lse.
int decode_check(const void* q, const void* k, const void* v, const void* out, const float* lse,
                 int B, int Lk, long long kv_capacity, int n_q, int n_kv, int d_h, float scale,
                 size_t& qb, size_t& kvb, size_t& lb) {
  if (!q || !k || !v || !out || !lse) return ATTN_PREFILL_ERR_NULL_PTR;
  if (B < 1 || Lk < 1 || n_q < 1 || n_kv < 1) return ATTN_PREFILL_ERR_BAD_SHAPE;
  if (kv_capacity < Lk) return ATTN_PREFILL_ERR_BAD_OFFSET;
  if (Lk > INT_MAX - 4096) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;  // key indices stay in int
  if (n_q % n_kv != 0) return ATTN_PREFILL_ERR_BAD_GQA;
  if (n_q / n_kv > 32) return ATTN_PREFILL_ERR_UNSUPPORTED;
  if (d_h != 64 && d_h != 128) return ATTN_PREFILL_ERR_BAD_HEADDIM;
  if (!std::isfinite(scale)) return ATTN_PREFILL_ERR_BAD_SCALE;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if ((align & 15) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3) != 0)
    return ATTN_PREFILL_ERR_MISALIGNED;
  size_t q_elems, kv_elems;
  if (__builtin_mul_overflow((size_t)B, (size_t)n_q, &q_elems) ||
      __builtin_mul_overflow(q_elems, (size_t)d_h, &q_elems) ||
      __builtin_mul_overflow((size_t)B, (size_t)n_kv, &kv_elems) ||
      __builtin_mul_overflow(kv_elems, (size_t)kv_capacity, &kv_elems) ||
      __builtin_mul_overflow(kv_elems, (size_t)d_h, &kv_elems) ||
      q_elems > ((size_t)1 << 61) || kv_elems > ((size_t)1 << 61))
    return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  const DecodeSplit sp = decode_split(B, Lk, n_kv);
  if ((long long)B * n_kv * sp.n_split > INT_MAX || (long long)B * n_q > INT_MAX)
    return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  qb = q_elems * 2;
  kvb = kv_elems * 2;
  lb = (size_t)B * n_q * 4;
  if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kvb) || overlaps(out, qb, v, kvb) ||
      overlaps(out, qb, lse, lb) || overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kvb) ||
      overlaps(lse, lb, v, kvb))
    return ATTN_PREFILL_ERR_ALIASING;
  return ATTN_PREFILL_OK;
}

// The two decode kernels of a checked call on a workspace of at least
// attn_decode_workspace_bytes() bytes.
int decode_launch(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                  int Lk, long long kv_capacity, int n_q, int n_kv, int d_h, float scale,
                  void* workspace, hipStream_t stream) {
  const DecodeSplit sp = decode_split(B, Lk, n_kv);
  const long long grid = (long long)B * n_kv * sp.n_split;
  const long long rows = (long long)B * n_q;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o + (size_t)rows * sp.n_split * d_h;
  const unsigned short* qs = static_cast<const unsigned short*>(q);
  const unsigned short* ks = static_cast<const unsigned short*>(k);
  const unsigned short* vs = static_cast<const unsigned short*>(v);
  unsigned short* os = static_cast<unsigned short*>(out);
  if (d_h == 128) {
    hipLaunchKernelGGL(decode_split_kernel<128>, dim3((unsigned)grid), dim3(64 * kDecWaves), 0,
                       stream, qs, ks, vs, ws_o, ws_lse, Lk, kv_capacity, n_q, n_kv, sp.n_split,
                       sp.split_keys, scale);
    if (hipGetLastError() != hipSuccess) return ATTN_PREFILL_ERR_LAUNCH;
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)rows), dim3(256), 0, stream,
                       ws_o, ws_lse, os, lse, sp.n_split);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<64>, dim3((unsigned)grid), dim3(64 * kDecWaves), 0,
                       stream, qs, ks, vs, ws_o, ws_lse, Lk, kv_capacity, n_q, n_kv, sp.n_split,
                       sp.split_keys, scale);
    if (hipGetLastError() != hipSuccess) return ATTN_PREFILL_ERR_LAUNCH;
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((unsigned)rows), dim3(256), 0, stream,
                       ws_o, ws_lse, os, lse, sp.n_split);
  }
  return hipGetLastError() == hipSuccess ? ATTN_PREFILL_OK : ATTN_PREFILL_ERR_LAUNCH;
}

// Decode scratch for callers that cannot allocate: a static device array,
// one copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address (on the host it names a stand-in, not device
// memory): the device address of each GPU's copy is looked up once with
// hipGetSymbolAddress, with that GPU current, and kept per device.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch, or nullptr on failure.
void* current_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" int attn_decode_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                               int B, int Lk, long long kv_capacity, int n_q, int n_kv, int d_h,
                               float scale, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (!workspace) return ATTN_PREFILL_ERR_NULL_PTR;
  size_t qb = 0, kvb = 0, lb = 0;
  const int st = decode_check(q, k, v, out, lse, B, Lk, kv_capacity, n_q, n_kv, d_h, scale, qb,
                              kvb, lb);
  if (st != ATTN_PREFILL_OK) return st;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15) != 0) return ATTN_PREFILL_ERR_MISALIGNED;
  const size_t need = attn_decode_workspace_bytes(B, Lk, n_q, n_kv, d_h);
  if (need == 0) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  if (workspace_bytes < need) return ATTN_PREFILL_ERR_WORKSPACE;
  if (overlaps(out, qb, workspace, need) || overlaps(lse, lb, workspace, need) ||
      overlaps(workspace, need, q, qb) || overlaps(workspace, need, k, kvb) ||
      overlaps(workspace, need, v, kvb))
    return ATTN_PREFILL_ERR_ALIASING;
  return decode_launch(q, k, v, out, lse, B, Lk, kv_capacity, n_q, n_kv, d_h, scale, workspace,
                       stream);
}

extern "C" size_t attn_decode_scratch_bytes(void) { return kDecodeScratchBytes; }

extern "C" int attn_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                       float* lse, int B, int Lk, long long kv_capacity, int n_q,
                                       int n_kv, int d_h, float scale, hipStream_t stream) {
  size_t qb = 0, kvb = 0, lb = 0;
  const int st = decode_check(q, k, v, out, lse, B, Lk, kv_capacity, n_q, n_kv, d_h, scale, qb,
                              kvb, lb);
  if (st != ATTN_PREFILL_OK) return st;
  const size_t need = attn_decode_workspace_bytes(B, Lk, n_q, n_kv, d_h);
  if (need == 0) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  if (need > kDecodeScratchBytes) return ATTN_PREFILL_ERR_SCRATCH;
  void* ws = current_scratch();
  if (ws == nullptr) return ATTN_PREFILL_ERR_LAUNCH;
  return decode_launch(q, k, v, out, lse, B, Lk, kv_capacity, n_q, n_kv, d_h, scale, ws, stream);
}

extern "C" const char* attn_prefill_strerror(int status) {
  switch (status) {
    case ATTN_PREFILL_OK: return "success";
    case ATTN_PREFILL_ERR_NULL_PTR: return "a buffer pointer is NULL";
    case ATTN_PREFILL_ERR_BAD_SHAPE: return "B, L (Lq, Lk, rows), n_q and n_kv must be >= 1";
    case ATTN_PREFILL_ERR_BAD_GQA: return "n_q must be a multiple of n_kv";
    case ATTN_PREFILL_ERR_BAD_HEADDIM: return "d_h must be 64 or 128";
    case ATTN_PREFILL_ERR_BAD_SCALE: return "scale must be finite";
    case ATTN_PREFILL_ERR_BAD_CAUSAL: return "causal must be 0 or 1";
    case ATTN_PREFILL_ERR_MISALIGNED:
      return "q, k, v and out must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_PREFILL_ERR_SIZE_OVERFLOW: return "sizes overflow the supported range";
    case ATTN_PREFILL_ERR_ALIASING: return "out or lse overlaps another buffer";
    case ATTN_PREFILL_ERR_LAUNCH: return "HIP kernel launch failed";
    case ATTN_PREFILL_ERR_BAD_OFFSET:
      return "q_offset must be >= 0, q_offset + Lq <= Lk when causal, and kv_capacity >= Lk";
    case ATTN_PREFILL_ERR_UNSUPPORTED:
      return "decode supports at most 32 query heads per key/value head";
    case ATTN_PREFILL_ERR_WORKSPACE:
      return "workspace_bytes is smaller than attn_decode_workspace_bytes() for these sizes";
    case ATTN_PREFILL_ERR_SCRATCH:
      return "these sizes need more decode workspace than the static scratch holds "
             "(attn_decode_scratch_bytes())";
    default: return "unknown status";
  }
}

extern "C" int attn_prefill_version(void) { return 300; }
