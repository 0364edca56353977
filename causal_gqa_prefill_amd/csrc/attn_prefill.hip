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
//    BR = 256 / HWG rows, as 8 wave64s, two per SIMD, each owning a block of
//    32 columns: the two waves of a SIMD cover each other's latencies, and at
//    d_h = 128 one wave's softmax work nearly fills the issue slots next to
//    its own MFMAs, so a lone wave per SIMD stalls.  Each K or V^T fragment
//    read from LDS feeds one MFMA (32x32) or two (16x16); the LDS (measured
//    ~250 B/clk/CU for 16-byte reads) has room for that.
//  * Scores are computed transposed, S^T = K Q^T: K (from LDS) is the A
//    operand, Q (held in VGPRs for the whole loop) the B operand.  Two MFMA
//    shapes are built.  v_mfma_f32_32x32x16_bf16 (the default): lane l holds
//    16 keys of query column l % 32 per 32-key half.  v_mfma_f32_16x16x32_bf16
//    (ATTN_PREFILL_MFMA=16): lane l holds 8 keys of each of columns l % 16
//    and 16 + l % 16.  Either way the row max and row sum are lane-local
//    until the lanes of a column combine theirs (v_permlane32_swap, and
//    v_permlane16_swap for 16x16), which only happens when the reference max
//    moves and at the end.
//  * The output is accumulated transposed, O^T += V^T P^T, with V^T as the A
//    operand and P^T as the B operand.  The score result's register layout
//    is used directly as the B operand (32x32: the 16 keys a lane holds are
//    the contraction slots of two k-steps; 16x16: the 8 keys of each of its
//    columns those of one k-step; both in a permuted key order), so P never
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
//    written, so an item no longer starts by waiting on HBM.  Where the
//    numbers fit, each XCD takes runs of adjacent q-blocks of one (batch,
//    kv-head) stream (stream blocks; for long causal sequences as balanced
//    pairs of q-blocks, which keep the run's workgroups in step from round
//    to round; see ItemList), so its L2 fetches a K/V tile once for all the
//    workgroups that read it.  A schedule of 16 or more rounds ends in a
//    dynamic tail: the items of its last, lightest rounds go to whichever
//    workgroup is free next (a counter per call), so the XCDs, which do not
//    run equally fast, finish together.
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
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <mutex>

#include "attn_prefill.h"
#include "device_common.h"

namespace {

constexpr int kCols = 256;            // query columns (head, row) per workgroup
constexpr int kWaves = kCols / 32;    // wave64s per workgroup, 32 query columns each
constexpr int kBC = 64;               // keys per K/V tile
constexpr float kSlack = 8.0f;        // rescale only past 2^8 growth

// 16-byte chunk swizzles of the K and V tiles (row = key inside the tile).
// gfx950's LDS has 64 four-byte banks and serves 16 lanes of a 16-byte read
// or 32 lanes of an 8-byte read per cycle (measured: conflict counters are
// zero for contiguous reads).  K: the 16 lanes of a 16-byte read take 16
// consecutive rows at one chunk, so the chunk is XORed with the row's low
// bits to land on 16 distinct 16-byte slots of a 256-byte bank window.  V:
// with the 32x32 shape the 32 lanes of a transpose read take 4 rows x 2 chunk
// pairs, and XORing the chunk with 4 (row & 3) (d_h = 128) puts the 8 32-byte
// pieces on distinct slots.  The 16x16 shape's transpose reads take 8
// consecutive rows x 1 chunk pair: XORing the chunk with 2 (row & 7) puts
// them on 8 distinct slots (and keeps each 32-byte pair together).  That
// swizzle moves the odd fragments' pair by +-32 bytes depending on the row,
// so their read offset is the even fragment's XOR 32, formed at each read
// (the pipeline has no registers for four more offsets).  For d_h = 64 two
// rows share a 256-byte window, hence the shifts.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D, int MS>
__device__ __forceinline__ int v_swz(int row) {
  if (MS == 16) return D == 128 ? ((row & 7) << 1) : (((row >> 1) & 3) << 1);
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// Per-lane score and accumulator registers of the two MFMA shapes.
//   32x32x16: the lane holds one query column (l % 32) and, per 32-key half,
//     16 of its scores, keys 4 (l / 32) + 8 (e / 4) + e % 4 for e = 0..15;
//     O^T in D / 32 tiles of 32 x 32.
//   16x16x32: the lane holds two query columns (l % 16 and 16 + l % 16) and,
//     per half, 8 scores of each, keys 4 (l / 16) + 16 (e / 4) + e % 4 for
//     e = 0..7 (two 16-key blocks, S^T block kb = e / 4 in register e % 4);
//     O^T in D / 16 x 2 tiles of 16 x 16.
// In both, score e of a column is the contraction slot e (of k-step e / 8
// for 32x32) of the P^T operand the lane supplies, so P never moves.
template <int D, int MS>
struct Mfma;
template <int D>
struct Mfma<D, 32> {
  struct Scores { f32x16 v; };
  struct Acc { f32x16 t[D / 32]; };
  static constexpr int kCol = 1;              // query columns per lane
  static constexpr int kSpc = 16;             // scores per column per half
  static constexpr int kQks = D / 16;         // k-steps of Q K^T
  static constexpr int kKw = 16;              // contraction depth of a k-step
  __device__ static constexpr int off(int e) { return 8 * (e >> 2) + (e & 3); }
  __device__ static float get(const Scores& s, int, int e) { return s.v[e]; }
  __device__ static void set(Scores& s, int, int e, float x) { s.v[e] = x; }
  __device__ static float aget(const Acc& a, int, int i) { return a.t[i >> 4][i & 15]; }
  __device__ static void aset(Acc& a, int, int i, float x) { a.t[i >> 4][i & 15] = x; }
};
template <int D>
struct Mfma<D, 16> {
  struct Scores { f32x4 v[4]; };               // [kb * 2 + cb]
  struct Acc { f32x4 t[D / 16][2]; };          // [db][cb]
  static constexpr int kCol = 2;
  static constexpr int kSpc = 8;
  static constexpr int kQks = D / 32;
  static constexpr int kKw = 32;
  __device__ static constexpr int off(int e) { return 16 * (e >> 2) + (e & 3); }
  __device__ static float get(const Scores& s, int c, int e) { return s.v[(e >> 2) * 2 + c][e & 3]; }
  __device__ static void set(Scores& s, int c, int e, float x) { s.v[(e >> 2) * 2 + c][e & 3] = x; }
  __device__ static float aget(const Acc& a, int c, int i) { return a.t[i >> 2][c][i & 3]; }
  __device__ static void aset(Acc& a, int c, int i, float x) { a.t[i >> 2][c][i & 3] = x; }
};

template <int D, int HWG, int MS>
__global__ __launch_bounds__(kWaves * 64) void attn_fwd_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, unsigned short* __restrict__ out,
    float* __restrict__ lse, int Lq, int Lk, int q_off, int n_q, int n_kv, int n_qblk,
    int items_per_qblk, int n_items, float scale, int causal, int sg, int pair_t,
    unsigned* __restrict__ dyn, int r_static) {
  using SH = Mfma<D, MS>;
  using Scores = typename SH::Scores;
  using Acc = typename SH::Acc;
  constexpr int NW = kWaves;                   // waves per workgroup
  constexpr int BR = kCols / HWG;              // query rows per workgroup
  constexpr int NF = D / 16;                   // K, V^T and Q fragments per wave and half
  constexpr int NCOL = SH::kCol;               // query columns per lane
  constexpr int SPC = SH::kSpc;                // scores per column and half
  constexpr int QKS = SH::kQks;                // k-steps of Q K^T
  constexpr int NACC = D / 2 / NCOL;           // accumulator values per column
  constexpr int ROWB = 2 * D;                  // bytes per K or V row
  constexpr int TILE = kBC * ROWB;             // bytes per K or V tile
  constexpr int LOADS = TILE / (NW * 1024);    // 1 KB loads per wave per tile
  static_assert(LOADS * NW * 1024 == TILE, "tile must split into 1 KB loads");
  constexpr int RING = 4;                      // tiles per ring
  constexpr int VRING = 0;                     // V ring at [0, 4 TILE)
  constexpr int KRING = RING * TILE;           // K ring at [4 TILE, 8 TILE)

  // output staging: one 32-row output tile per wave; two of them in the last
  // slot of each ring, the other four in an area after the rings
  constexpr int OT = 32 * ROWB;                // bytes of one wave's output tile
  constexpr int STAGE = 2 * RING * TILE;       // staging area offset
  static_assert(4 * OT == 2 * TILE && NW == 8, "half the output tiles fill one ring slot");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[STAGE + 4 * OT];
  LDS_AS unsigned char* const smem_l = (LDS_AS unsigned char*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // the lane's column inside its block of MS columns and its key group
  const int lcol = lane & (MS - 1);
  const int lgrp = lane / MS;
  // query row offset (inside the wave's 32) of the lane's column c
  auto col_off = [&] __device__ (int c) __attribute__((always_inline)) { return 16 * c + lcol; };

  // ---- work items: (b, kv-head, head group, q-block) in the list order of
  // ItemList (heavy-first zigzag, stream blocks or balanced pairs, chosen by
  // the host).  Dynamic tail (dyn != nullptr, chosen by the host): only
  // rounds 0 .. r_static - 1 follow the static schedule; the entries from
  // r_static G on go out in list order, one per draw from the call's
  // counter, to the workgroups as they become free.
  const int g = n_q / n_kv;
  const int ngroups = g / HWG;
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
    int qb, hg, kvh, b, n_tiles;  // n_tiles: K/V tiles the workgroup streams
    const unsigned short* kb;     // K and V rows of the item's kv-head
    const unsigned short* vb;
  };
  auto geo = [&] __device__ (int item) __attribute__((always_inline)) {
    Geo e;
    int rest;   // the (batch, kv-head) stream
    list_decode(lst, item, gridDim.x, e.qb, e.hg, rest);
    e.kvh = rest % n_kv;
    e.b = rest / n_kv;
    // query row i sits at key position q_off + i; K and V hold Lk rows
    const int wg_end = min(e.qb * BR + BR, Lq);
    e.n_tiles = causal ? (wg_end + q_off + kBC - 1) / kBC : (Lk + kBC - 1) / kBC;
    e.kb = k + ((size_t)e.b * n_kv + e.kvh) * (size_t)Lk * D;
    e.vb = v + ((size_t)e.b * n_kv + e.kvh) * (size_t)Lk * D;
    return e;
  };
  // the wave's 32 columns: columns 32 wave .. 32 wave + 31 of the workgroup,
  // column c being head c / BR, row c % BR of the q-block
  auto blk_head = [&] __device__ (const Geo& e) __attribute__((always_inline)) {
    return e.kvh * g + e.hg * HWG + 32 * wave / BR;
  };
  auto blk_q0 = [&] __device__ (const Geo& e) __attribute__((always_inline)) {
    return e.qb * BR + 32 * wave % BR;
  };

  // ---- Q fragments (B operand of S^T = K Q^T), fragment f = c QKS + kk:
  // Q[row of column c][kKw kk + 8 lgrp + 0..7] (kKw: 16 or 32 per k-step)
  bf16x8 qf[NF];
  auto load_q = [&] __device__ (const Geo& e) __attribute__((always_inline)) {
    const int q0 = blk_q0(e);
    const unsigned short* qhead = q + ((size_t)e.b * n_q + blk_head(e)) * Lq64 * D;
#pragma unroll
    for (int c = 0; c < NCOL; ++c) {
      const int qi = q0 + col_off(c);
      const unsigned short* qrow = qhead + (size_t)qi * D;
#pragma unroll
      for (int kk = 0; kk < QKS; ++kk) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qi < Lq) raw = *reinterpret_cast<const u32x4*>(qrow + kk * SH::kKw + lgrp * 8);
        qf[c * QKS + kk] = __builtin_bit_cast(bf16x8, raw);
      }
    }
  };

  // per-item state the pipeline reads: the wave's head and first row, the
  // tiles the workgroup streams and the tiles this wave computes, the K/V
  // rows of this item and of the next one
  int hb = 0, q0b = 0;
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
    v_src[s] = row * ROWB + ((pos ^ v_swz<D, MS>(row)) << 4);
  }
  auto load_tile = [&] __device__ (const unsigned short* base, const int (&src)[LOADS], int tile,
                       int lds_off) __attribute__((always_inline)) {
    dma_tile(base, src, LOADS, ROWB, tile * kBC, Lk, kBC, smem + lds_off + wave * LOADS * 1024);
  };

  // ---- per-lane LDS read offsets (half 0 of ring slot 0; half jb adds 32 rows)
  // K fragment f, the A operand of S^T = K Q^T.  32x32: key lcol, k-step f,
  // chunk 2 f + lgrp.  16x16: f = kb QKS + kk, key 16 kb + lcol, chunk
  // 4 kk + lgrp.
  // (16x16: key block 1 sits 16 rows after block 0 under the same swizzle,
  // so only the QKS k-steps need offsets of their own)
  int k_rd[QKS];
#pragma unroll
  for (int kk = 0; kk < QKS; ++kk) {
    const int chunk = MS == 32 ? 2 * kk + lgrp : 4 * kk + lgrp;
    k_rd[kk] = KRING + lcol * ROWB + ((chunk ^ k_swz<D>(lcol)) << 4);
  }
  // V^T fragment f through ds_read_b64_tr_b16 (in each group of 16 lanes,
  // lane 4r+qq supplies four consecutive 16-bit values of row r and lane i
  // receives column i of the four rows), two reads per fragment.
  //   32x32: f = 2 tb + h; lane 16G + 4r + qq reads V[key][t .. t+3] with
  //     key = 16 (2 jb + h) + 8 u + 4 (G / 2) + r, t = 32 tb + 16 (G % 2) + 4 qq,
  //     u = 0, 1 the two reads (8 rows apart), and receives V^T[32 tb + l % 32]
  //     at the keys of its P^T slots.
  //   16x16: f = db; lane 16G + 4r + qq reads V[key][t .. t+3] with
  //     key = 32 jb + 16 u + 4 G + r, t = 16 db + 4 qq, u = 0, 1 (16 rows
  //     apart), and receives V^T[16 db + l % 16] at keys 16 u + 4 G + 0..3.
  // (32x32: the k-step h of fragment 2 tb + h moves the rows by 16, which
  // keeps the swizzle, so only the D / 32 column blocks need offsets)
  constexpr int NVRD = D / 32;
  int v_rd[NVRD];
  {
    const int tr_r = (lane >> 2) & 3;
    const int tr_q = lane & 3;
    const int tr_g = lane >> 4;
#pragma unroll
    for (int f = 0; f < NVRD; ++f) {
      int key, t;
      if constexpr (MS == 32) {
        key = 4 * (tr_g >> 1) + tr_r;                  // plus 32 jb + 16 h + 8 u
        t = 32 * f + 16 * (tr_g & 1) + 4 * tr_q;
      } else {
        key = 4 * tr_g + tr_r;                         // plus 32 jb + 16 u
        t = 32 * f + 4 * tr_q;                         // odd fragments: offset ^ 32
      }
      v_rd[f] = VRING + key * ROWB + (((t >> 3) ^ v_swz<D, MS>(key)) << 4) + ((t >> 2) & 1) * 8;
    }
  }
  constexpr int V_U = (MS == 32 ? 8 : 16) * ROWB;    // bytes between the two reads

  // ---- running state per column: reference max m (log2 domain), lane
  // partial row sum l, accumulator O^T
  Acc acc;
  float m_run[NCOL], l_run[NCOL];
  const float c2 = scale * kLog2e;
  const bool fast_scale = c2 > 0.0f;

  // K fragments of ring slot `slot`, keys 32 jb .. 32 jb + 31
  // (k-steps [kk0, kk1) only, for both key blocks of the 16x16 shape)
  auto load_kfrags = [&] __device__ (bf16x8 (&kf)[NF], int slot, int jb, int kk0 = 0,
                                     int kk1 = SH::kQks) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
      if (f % QKS >= kk0 && f % QKS < kk1)
        kf[f] = *reinterpret_cast<const LDS_AS bf16x8*>(smem_l + k_rd[f % QKS] + slot * TILE +
                                                        (jb * 32 + 16 * (f / QKS)) * ROWB);
  };
  // a ^ 32, computed where it is used (an opaque instruction the compiler
  // cannot hoist out of the tile loop into registers of its own)
  auto xor32 = [] __device__ (int a) __attribute__((always_inline)) {
    int r;
    asm volatile("v_xor_b32 %0, 32, %1" : "=v"(r) : "v"(a));
    return r;
  };
  // V^T fragments of ring slot `slot`, keys 32 jb .. 32 jb + 31
  auto load_vfrags = [&] __device__ (bf16x8 (&vf)[NF], int slot, int jb) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const LDS_AS unsigned char* base =
          smem_l + (MS == 32 ? v_rd[f >> 1] + (f & 1) * 16 * ROWB
                             : ((f & 1) ? xor32(v_rd[f >> 1]) : v_rd[f >> 1])) + slot * TILE +
          jb * 32 * ROWB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(base));
      const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(base + V_U));
      vf[f] = __builtin_bit_cast(
          bf16x8, (u32x4){__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, up)[0], __builtin_bit_cast(u32x2, up)[1]});
    }
  };

  // S^T = K Q^T, k-steps [k0, k1); k0 = 0 starts from zero.  The 16x16
  // shape runs four independent chains (two key blocks x two columns).
  auto qk_mfma = [&] __device__ (Scores& S, const bf16x8 (&kf)[NF], int k0, int k1)
      __attribute__((always_inline)) {
    if constexpr (MS == 32) {
      if (k0 == 0)
#pragma unroll
        for (int r = 0; r < 16; ++r) S.v[r] = 0.0f;
#pragma unroll
      for (int kk = k0; kk < k1; ++kk)
        S.v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], S.v, 0, 0, 0);
    } else {
      if (k0 == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) S.v[i][r] = 0.0f;
#pragma unroll
      for (int kk = k0; kk < k1; ++kk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c)
            S.v[kb * 2 + c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                kf[kb * QKS + kk], qf[c * QKS + kk], S.v[kb * 2 + c], 0, 0, 0);
    }
  };

  // O^T += V^T P^T (consecutive MFMAs write different accumulators).  pk:
  // 32x32: the two 16-key k-steps of the one column; 16x16: the one 32-key
  // k-step of each of the two columns.
  auto pv_mfma = [&] __device__ (const bf16x8 (&vf)[NF], const bf16x8 (&pk)[2]) __attribute__((always_inline)) {
    if constexpr (MS == 32) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int tb = 0; tb < D / 32; ++tb)
          acc.t[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * tb + h], pk[h], acc.t[tb],
                                                              0, 0, 0);
    } else {
#pragma unroll
      for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc.t[db][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pk[c], acc.t[db][c],
                                                                 0, 0, 0);
    }
  };

  // the lane's own maximum of column c's scores (branch-free; the lanes of a
  // column combine theirs only when the reference moves)
  auto lane_max = [&] __device__ (const Scores& s, int c) __attribute__((always_inline)) {
    float mx = fmaxf(SH::get(s, c, 0), SH::get(s, c, 1));
#pragma unroll
    for (int e = 2; e < SPC; ++e) mx = fmaxf(mx, SH::get(s, c, e));
    return mx;
  };
  // maximum / sum over the lanes that hold one column
  auto col_max = [&] __device__ (float x) __attribute__((always_inline)) {
    if constexpr (MS == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
      x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return pair_max(x);
  };
  auto col_sum = [&] __device__ (float x) __attribute__((always_inline)) {
    if constexpr (MS == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
      x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return pair_sum(x);
  };

  // softmax, first part, for the scores of keys j0 .. j0+31 (may branch):
  // where the half straddles the diagonal (query q0 + i sees keys up to
  // q_off + q0 + i) or the end of the keys, or the scale is not positive,
  // mask and pre-scale the scores.  Then move the reference max (rescaling l
  // and acc) only when some lane's own maximum exceeds it by more than 2^8:
  // no column's maximum can exceed it then, since a column's maximum is one
  // of its lanes' maxima.  When it moves, every column takes the maximum of
  // its lanes.  Returns the multiplier and -m per column.
  auto prepare = [&] __device__ (Scores& s, int j0, float& c_out, float (&mneg)[NCOL])
      __attribute__((always_inline)) {
    // the lane maxima first (the common case needs them as they are), so
    // their chain starts before the mask decision resolves
    float mx[NCOL];
#pragma unroll
    for (int cc = 0; cc < NCOL; ++cc) mx[cc] = lane_max(s, cc);
    const bool need_mask = (causal && j0 + 31 > q0b + q_off) || (j0 + 32 > Lk);
    float c = c2;
    if (need_mask || !fast_scale) {
      // score e of column c is key j0 + 4 lgrp + off(e), visible to query
      // qi (at key position qi + q_off) iff off(e) <= lim.  A scale <= 0 is
      // applied before masking, so that a masked score stays -inf; a
      // positive one later, in the exponential.
      const float cm = fast_scale ? 1.0f : c2;
      // (the lane id is re-derived here, opaque to the compiler, so that the
      // per-lane limits are computed in this rarely taken branch instead of
      // being kept, or spilled, across the tile loop)
      int mlane;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(mlane));
#pragma unroll
      for (int cc = 0; cc < NCOL; ++cc) {
        const int qi = q0b + 16 * cc + (mlane & (MS - 1));
        const int lim = (causal ? min(qi + q_off, Lk - 1) : Lk - 1) - j0 - 4 * (mlane / MS);
#pragma unroll
        for (int e = 0; e < SPC; ++e)
          SH::set(s, cc, e, SH::off(e) > lim ? -INFINITY : SH::get(s, cc, e) * cm);
        mx[cc] = lane_max(s, cc);
      }
      c = fast_scale ? c2 : 1.0f;
    }
    float m_cand[NCOL];
    bool grow = false;
#pragma unroll
    for (int cc = 0; cc < NCOL; ++cc) {
      m_cand[cc] = mx[cc] * c;
      grow = grow || (m_cand[cc] > m_run[cc] + kSlack);
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int cc = 0; cc < NCOL; ++cc) {
        const float m_new = fmaxf(m_run[cc], col_max(m_cand[cc]));
        const float alpha = __builtin_amdgcn_exp2f(m_run[cc] - m_new);
        m_run[cc] = m_new;
        l_run[cc] *= alpha;
#pragma unroll
        for (int i = 0; i < NACC; ++i) SH::aset(acc, cc, i, SH::aget(acc, cc, i) * alpha);
      }
    }
    c_out = c;
#pragma unroll
    for (int cc = 0; cc < NCOL; ++cc) mneg[cc] = -m_run[cc];
  };

  // softmax, second part (branch-free): p = 2^(c s - m) added to the lane's
  // fp32 row sum, and P^T rounded to bf16 as two B-operand fragments (32x32: the column's
  // two k-steps; 16x16: one k-step per column)
  auto expo = [&] __device__ (const Scores& s, float cm, const float (&mneg)[NCOL],
                              bf16x8 (&pk)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int cc = 0; cc < NCOL; ++cc) {
#pragma unroll
      for (int half = 0; half < SPC / 8; ++half) {
        bf16x8 frag;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(SH::get(s, cc, half * 8 + e), cm, mneg[cc]));
          l_run[cc] += p;
          frag[e] = (__bf16)p;
        }
        pk[cc + half] = frag;
      }
    }
  };

  // Software pipeline over 32-key half-steps h = 2 t + jb.  Entering the
  // region of half h: the raw scores of h are in registers, as are the K
  // fragments of half h+1 and the V^T fragments of half h.  The region first
  // puts a few QK^T MFMAs of h+1 on the pipe (they need nothing from the
  // softmax) and, in the first half of a tile, issues the tile loads; while
  // those run it takes the lane maxima and the first softmax part of h (mask
  // and rescale decisions, rarely taken branches).  Then, branch-free: the
  // rest of the scores of h+1 next to the exponentials of h, followed by its
  // P V, with the K fragments of h+2 and the V^T fragments of h+1 read from
  // LDS meanwhile.  Past the wave's last half the region computes on stale
  // LDS data whose results are never used.
  struct Half {
    Scores s;
    bf16x8 kf[NF];
    bf16x8 vf[NF];
  };
  Half hA, hB;
  constexpr int KA = 2;                 // k-steps of h+1 issued ahead of the branches

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
    // keep the scheduler from pulling this region's softmax up next to the
    // previous region's last MFMAs (whose results it would then stall on)
    __builtin_amdgcn_sched_barrier(0);
    qk_mfma(nxt.s, cur.kf, 0, KA);
    if (jb == 0) issue_tile_loads(ts, t);
    float cm, mn[NCOL];
    prepare(cur.s, t * kBC + jb * 32, cm, mn);
    if constexpr (MS == 32) {
      load_kfrags(nxt.kf, slot2, jb2);
      load_vfrags(nxt.vf, slot1, jb1);
      qk_mfma(nxt.s, cur.kf, KA, QKS);
    } else {
      // (16x16 needs more registers for its per-column state: it holds only
      // the first half of the next half-step's K fragments across a region,
      // reads the second half here, once the first half is consumed, and the
      // V^T fragments of h+1 once those of h are, so that one set of each is
      // live instead of two)
      load_kfrags(cur.kf, slot1, jb1, KA, QKS);
      qk_mfma(nxt.s, cur.kf, KA, QKS);
    }
    bf16x8 pk[2];
    expo(cur.s, cm, mn, pk);
    pv_mfma(cur.vf, pk);
    if constexpr (MS == 16) {
      load_vfrags(nxt.vf, slot1, jb1);
      load_kfrags(nxt.kf, slot2, jb2, 0, KA);
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
  // the word through which wave 0 passes a dynamic-tail item to the others:
  // the first bytes of its own output staging area, which no other wave
  // touches and no tile load writes between an item's epilogue and its
  // successor's first tile step
  LDS_AS int* const dyn_word = (LDS_AS int*)(smem_l + VRING + 3 * TILE);
  const int n_dyn = n_items - r_static * (int)gridDim.x;
  for (;;) {
    // ---- item setup.  The next item: round r + 1 of the static schedule,
    // or, in the dynamic tail, the next entry of the call's counter (taken
    // by one lane while the prologue's loads land)
    const bool dyn_next = dyn != nullptr && r + 1 >= r_static;
    int nxt_item = n_items;
    if (!dyn_next) {
      nxt_item = item_at(r + 1);
    } else if (wave == 0) {
      if (lane == 0) {
        // (system scope: performed past every XCD's L2, so that the
        // workgroups of all XCDs count on one copy)
        const unsigned j = __hip_atomic_fetch_add(dyn, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_SYSTEM);
        *dyn_word = j < (unsigned)n_dyn ? r_static * (int)gridDim.x + (int)j : n_items;
      }
      wait_lgkm0();
    }
    kbase = cur.kb;
    vbase = cur.vb;
    n_tiles = cur.n_tiles;
    hb = blk_head(cur);
    q0b = blk_q0(cur);
    const int last_row = q0b < Lq ? min(q0b + 31, Lq - 1) : -1;
    wave_tiles = last_row < 0 ? 0 : (causal ? (last_row + q_off) / kBC + 1 : n_tiles);
#pragma unroll
    for (int cc = 0; cc < NCOL; ++cc) {
#pragma unroll
      for (int i = 0; i < NACC; ++i) SH::aset(acc, cc, i, 0.0f);
      m_run[cc] = -INFINITY;
      l_run[cc] = 0.0f;
    }

    // ---- prologue: the item's tiles 0..2 and its Q have landed (and the
    // previous item's stores are done); then the raw scores of half 0, the K
    // fragments of half 1 and the V^T fragments of half 0 in registers
    wait_vmcnt<0>();
    tile_barrier();
    if (dyn_next) {
      // every wave reads the word before the barrier after which tile step
      // 0 may overwrite it
      nxt_item = __builtin_amdgcn_readfirstlane(*dyn_word);
      wait_lgkm0();
      tile_barrier();
    }
    has_next = nxt_item < n_items;
    const Geo nx = geo(has_next ? nxt_item : item);
    nkbase = nx.kb;
    nvbase = nx.vb;
    if (wave_tiles > 0) {
      load_kfrags(hB.kf, 0, 0);
      qk_mfma(hA.s, hB.kf, 0, QKS);
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
    // wave's 32 x d_h output tile goes through LDS (ring slot 3, or the
    // staging area) so that the global stores are whole rows: 1 KB
    // per store instruction instead of 8-byte pieces of 32 different rows.
    // (The lane id is re-derived here, opaque to the compiler, so that the
    // staging addresses are computed in place instead of being kept, or
    // spilled, across the tile loop.)
    int elane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(elane));
    const int ecol = elane & (MS - 1);
    const int egrp = elane / MS;
    const int q0 = q0b;
    LDS_AS unsigned char* ot =
        smem_l + (wave < 2 ? VRING + 3 * TILE + wave * OT
                           : wave < 4 ? KRING + 3 * TILE + (wave - 2) * OT : STAGE + (wave - 4) * OT);
#pragma unroll
    for (int cc = 0; cc < NCOL; ++cc) {
      const float l_tot = col_sum(l_run[cc]);
      const float inv = 1.0f / l_tot;
      const int row = 16 * cc * (MS == 16) + ecol;       // output row inside the wave's 32
      if (egrp == 0 && q0 + row < Lq && wave_tiles > 0)
        lse[((size_t)cur.b * n_q + hb) * Lq64 + (size_t)(q0 + row)] =
            (m_run[cc] + __log2f(l_tot)) * kLn2;
      // 32x32: lane (ecol, egrp) holds row ecol, columns 32 tb + 8 grp +
      // 4 egrp + 0..3 (accumulator values 16 tb + 4 grp + 0..3).
      // 16x16: lane (ecol, egrp) holds row 16 c + ecol, columns 16 db +
      // 4 egrp + 0..3 (values 4 db + 0..3).
#pragma unroll
      for (int grp = 0; grp < NACC / 4; ++grp) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(SH::aget(acc, cc, grp * 4 + e) * inv);
        const int col = MS == 32 ? 8 * grp + 4 * egrp : 16 * grp + 4 * egrp;
        *reinterpret_cast<LDS_AS u32x2*>(ot + row * ROWB + (((col >> 3) ^ k_swz<D>(row)) << 4) +
                                         ((col >> 2) & 1) * 8) = __builtin_bit_cast(u32x2, o4);
      }
    }
    // read back whole rows: store st covers rows 1024 st / ROWB onwards
    // (non-temporal stores: the output is not read again here, and the L2
    // keeps its room for the K/V tiles the XCD's other workgroups still read;
    // config-2 traffic 1.39 -> 1.25 times the compulsory bytes.  The same
    // hint on the Q loads made the next item's prologue wait longer, 5%
    // slower, and saved nothing.)
    unsigned short* obase = out + (((size_t)cur.b * n_q + hb) * Lq64 + (size_t)q0) * D;
#pragma unroll
    for (int st = 0; st < OT / 1024; ++st) {
      const int byte = st * 1024 + elane * 16;
      const int row = byte / ROWB;
      const int chunk = (byte % ROWB) >> 4;
      const u32x4 v4 =
          *reinterpret_cast<const LDS_AS u32x4*>(ot + row * ROWB + ((chunk ^ k_swz<D>(row)) << 4));
      if (q0 + row < Lq && wave_tiles > 0)
        __builtin_nontemporal_store(v4, reinterpret_cast<u32x4*>(obase + (size_t)row * D + chunk * 8));
    }
    if (!has_next) break;
    cur = nx;
    item = nxt_item;
    ++r;
  }
  wait_vmcnt<0>();   // no tile load may still be writing LDS when the wave ends
  // the last workgroup out (every other one has taken its last counter
  // entry by then) sets the call's counters back to zero for the next call
  if (dyn != nullptr && wave == 0 && lane == 0 &&
      __hip_atomic_fetch_add(dyn + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
          gridDim.x - 1) {
    __hip_atomic_store(dyn, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(dyn + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// Heads per workgroup: the largest of 8, 4, 2, 1 that divides g.
int pick_hwg(int g) {
  if (g % 8 == 0) return 8;
  if (g % 4 == 0) return 4;
  if (g % 2 == 0) return 2;
  return 1;
}

// MFMA shape of the forward kernel: 32 (v_mfma_f32_32x32x16_bf16) unless
// the environment variable ATTN_PREFILL_MFMA says 16 (or 32).  Both shapes
// compute the same attention (they differ in the order of the fp32 sums);
// the override exists for comparing them.
int pick_mfma() {
  const char* s = std::getenv("ATTN_PREFILL_MFMA");
  if (s && s[0] == '1' && s[1] == '6' && s[2] == 0) return 16;
  return 32;
}

// ---- the dynamic tail.  The eight XCDs of the chip do not run equally
// fast (their shares of one launch finish up to 5% apart, the same XCDs
// slow from launch to launch), which no static schedule can know.  The
// forward kernels therefore run the first rounds of their heavy-first
// schedule statically (each XCD on its own streams, for its L2) and hand out
// the items of the last, lightest rounds through a counter that every
// workgroup draws from when it is free, so that fast XCDs take more of them.
//
// Each call with a dynamic tail takes one pair of counters {next entry,
// workgroups finished} from a per-GPU pool; the call's last workgroup sets
// both back to zero, and a pair is handed out again only kDynSlots calls
// later, so calls in flight at once on several streams never share one.
// A call issued while its stream is being captured into a graph takes the
// static schedule and no counter (a replayed graph would reuse one pair).
constexpr int kDynSlots = 65536;
constexpr int kDynMaxDevices = 64;
static __device__ __align__(256) unsigned dyn_pool[2 * kDynSlots];
std::mutex dyn_mu;
unsigned* dyn_base[kDynMaxDevices] = {};
std::atomic<unsigned> dyn_next_slot{0};

// rounds of the static schedule before the dynamic tail: all of them when
// there are fewer than kDynMinRounds (a workgroup draws its next item when
// it starts the current one, so with a few large items per workgroup the
// first draws of the tail go to the workgroups that started the previous
// round first, which the zigzag gave a heavy item there: 3-12% slower at 4
// rounds, against 2.4-2.6% faster at 32 and 72);
// otherwise the tail holds the last 30% of the rounds of a causal schedule
// (about 9% of its work, the heavy-first rounds shrinking towards the end)
// or the last 10% of a non-causal one
constexpr long long kDynMinRounds = 16;
long long static_rounds(long long n_items, long long grid, int causal) {
  const long long R = (n_items + grid - 1) / grid;
  if (R < kDynMinRounds) return R;
  return R - (causal ? (3 * R + 9) / 10 : (R + 9) / 10);
}

// The counter pair of one call on the current GPU, or nullptr (static
// schedule) while the stream is being captured or if the pool's address
// cannot be had.
unsigned* dyn_counters(hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDynMaxDevices) return nullptr;
  unsigned* base = nullptr;
  {
    std::lock_guard<std::mutex> lock(dyn_mu);
    if (dyn_base[dev] == nullptr) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(dyn_pool)) != hipSuccess || p == nullptr)
        return nullptr;
      dyn_base[dev] = static_cast<unsigned*>(p);
    }
    base = dyn_base[dev];
  }
  return base + 2 * (dyn_next_slot.fetch_add(1, std::memory_order_relaxed) % kDynSlots);
}

// Balanced pairs (long causal schedules): the tail cut T, q-blocks 0 .. T - 1
// being the dynamic tail's share, nearest to 0.3 n_qblk within [0.2, 0.4]
// n_qblk (the tail then holds (T / n_qblk)^2 of the causal work, about 9%,
// as the last 30% of the rounds of a heavy-first list do) for which the pairs of
// q-blocks T .. n_qblk - 1 fill whole rounds: (n_qblk - T) / 2 pairs per
// item of a q-block, times ipq, a multiple of grid, i.e. (n_qblk - T) / 2 a
// multiple of m = grid / gcd(ipq, grid).  0 when no such T exists.
long long pair_cut(long long n_qblk, long long ipq, long long grid) {
  long long a = ipq, b = grid;
  while (b != 0) {
    const long long t = a % b;
    a = b;
    b = t;
  }
  const long long m = grid / a;
  const long long lo = std::max(1LL, (n_qblk + 4) / 5);
  const long long hi = 2 * n_qblk / 5;
  // T = n_qblk - 2 j m; the j nearest the target and its neighbours
  const long long j0 = 7 * n_qblk / (20 * m);
  long long best = 0, best_d = -1;
  for (long long j = j0 - 1; j <= j0 + 2; ++j) {
    const long long T = n_qblk - 2 * j * m;
    if (j < 1 || T < lo || T > hi) continue;
    const long long d = std::llabs(10 * T - 3 * n_qblk);
    if (best_d < 0 || d < best_d) {
      best = T;
      best_d = d;
    }
  }
  return best;
}

// The list form of a persistent forward launch and its static rounds when a
// counter pair is at hand (no GPU call): sg and pair_t as ItemList describes
// them; pair_rounds the balanced pairs' rounds; r_static the rounds before
// the dynamic tail (all of them when there is none).
struct ListForm {
  int sg, pair_t;
  long long pair_rounds, r_static;
};
ListForm list_form(long long n_items, long long ipq, long long n_qblk, long long ngroups,
                   long long grid, int causal) {
  ListForm f{0, 0, 0, 0};
  if (grid % 8 == 0) {
    const long long slots = grid / 8;
    // short sequences: whole heads per XCD and round when they fill every
    // round exactly and the rounds pair up (every round then holds heavy and
    // light q-blocks, and an unpaired last round would leave its heavy ones
    // running alone)
    if (slots % n_qblk == 0 && ipq % (8 * (slots / n_qblk)) == 0 && (n_items / grid) % 2 == 0) {
      f.sg = (int)n_qblk;
    } else if (n_items >= 16 * grid) {
      // long sequences: runs of one or two streams per XCD, as balanced
      // pairs when causal and the pairs fill whole rounds; otherwise plain
      // stream blocks, whose super-groups do not line up with the rounds, so
      // only when there are many rounds and many super-groups (each spanning
      // a small share of the causal weights) does the zigzag still even the
      // work out (within 0.1% over a sweep of shapes)
      const long long T = causal ? pair_cut(n_qblk, ipq, grid) : 0;
      if (T > 0) {
        f.pair_t = (int)T;
        f.sg = (int)std::min((n_qblk - T) / 2, std::max(1LL, slots / ngroups));
        f.pair_rounds = 2 * (((n_qblk - T) / 2) * ipq / grid);
      } else {
        const long long run = std::min(n_qblk, std::max(1LL, slots / ngroups));
        if (n_qblk >= 64 * run) f.sg = (int)run;
      }
    }
  }
  // the pairs' rounds static, q-blocks 0 .. T - 1 the tail; otherwise the
  // last rounds of the list
  f.r_static = f.pair_t > 0 ? f.pair_rounds : static_rounds(n_items, grid, causal);
  return f;
}

}  // namespace

__attribute__((visibility("hidden"))) ItemPlan attn_item_plan(long long n_items, long long ipq,
                                                              long long n_qblk, long long ngroups,
                                                              long long grid, int causal,
                                                              hipStream_t stream) {
  const ListForm f = list_form(n_items, ipq, n_qblk, ngroups, grid, causal);
  ItemPlan p{f.sg, f.pair_t, f.r_static, nullptr};
  if (p.r_static * grid < n_items) {
    p.dyn = dyn_counters(stream);
    if (p.dyn == nullptr) p.r_static = (n_items + grid - 1) / grid;
  }
  return p;
}

namespace {

// Sizes of one call; Lq = Lk and q_off = 0 for a whole-sequence prefill.
struct Shape {
  int B, Lq, Lk, q_off, n_q, n_kv, d_h;
};

template <int D, int HWG, int MS>
int launch(const void* q, const void* k, const void* v, void* out, float* lse, const Shape& sh,
           float scale, int causal, hipStream_t stream) {
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
  // the list form and the dynamic tail
  const ItemPlan plan = attn_item_plan(n_items, items_per_qblk, n_qblk,
                                       (sh.n_q / sh.n_kv) / HWG, grid, causal, stream);
  hipLaunchKernelGGL((attn_fwd_kernel<D, HWG, MS>), dim3((unsigned)grid), dim3(kWaves * 64), 0,
                     stream,
                     static_cast<const unsigned short*>(q), static_cast<const unsigned short*>(k),
                     static_cast<const unsigned short*>(v), static_cast<unsigned short*>(out), lse,
                     sh.Lq, sh.Lk, sh.q_off, sh.n_q, sh.n_kv, n_qblk, (int)items_per_qblk,
                     (int)n_items, scale, causal, plan.sg, plan.pair_t, plan.dyn,
                     (int)plan.r_static);
  return hipGetLastError() == hipSuccess ? ATTN_PREFILL_OK : ATTN_PREFILL_ERR_LAUNCH;
}

template <int D, int MS>
int launch_m(const void* q, const void* k, const void* v, void* out, float* lse, const Shape& sh,
             float scale, int causal, hipStream_t stream) {
  switch (pick_hwg(sh.n_q / sh.n_kv)) {
    case 8: return launch<D, 8, MS>(q, k, v, out, lse, sh, scale, causal, stream);
    case 4: return launch<D, 4, MS>(q, k, v, out, lse, sh, scale, causal, stream);
    case 2: return launch<D, 2, MS>(q, k, v, out, lse, sh, scale, causal, stream);
    default: return launch<D, 1, MS>(q, k, v, out, lse, sh, scale, causal, stream);
  }
}

template <int D>
int launch_d(const void* q, const void* k, const void* v, void* out, float* lse, const Shape& sh,
             float scale, int causal, hipStream_t stream) {
  if (pick_mfma() == 32) return launch_m<D, 32>(q, k, v, out, lse, sh, scale, causal, stream);
  return launch_m<D, 16>(q, k, v, out, lse, sh, scale, causal, stream);
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
constexpr int kDecMaxSplits = 4096;   // partials per row (bounds the workspace)

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
    v_src[s] = row * ROWB + ((pos ^ v_swz<D, 32>(row)) << 4);
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
      v_rd[tb] = TILE + key * ROWB + (((t >> 3) ^ v_swz<D, 32>(key)) << 4) + ((t >> 2) & 1) * 8;
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
// LSE = M + ln sum w_s.  Thread (sg, c4) owns four columns of the splits
// sg, sg + SG, ...; it loads a chunk of kCombChunk of its splits (LSEs and
// partial outputs together, one memory round trip per chunk) and folds
// them into a running maximum, weight sum and weighted sum, rescaled when
// the maximum grows; the SG groups then merge the same way through LDS.
constexpr int kCombChunk = 16;
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    unsigned short* __restrict__ out, float* __restrict__ lse, int n_split) {
  constexpr int C4 = D / 4;            // float4 columns of a row
  constexpr int SG = 256 / C4;         // split groups
  __shared__ float m_g[SG], l_g[SG];
  __shared__ float4 part[SG][C4];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const float* lrow = ws_lse + row * n_split;
  const float* orow = ws_o + row * n_split * D;
  const int c4 = tid % C4;
  const int sg = tid / C4;

  float m = -INFINITY;   // this group's running max of the LSEs
  float wsum = 0.0f;     // sum of exp(lse_s - m)
  float4 a = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = sg; s0 < n_split; s0 += SG * kCombChunk) {
    float x[kCombChunk];
    float4 o[kCombChunk];
#pragma unroll
    for (int u = 0; u < kCombChunk; ++u) {
      const int s = s0 + u * SG;
      x[u] = -INFINITY;
      o[u] = float4{0.0f, 0.0f, 0.0f, 0.0f};
      if (s < n_split) {
        x[u] = lrow[s];
        o[u] = *reinterpret_cast<const float4*>(orow + (size_t)s * D + 4 * c4);
      }
    }
#pragma unroll
    for (int u = 0; u < kCombChunk; ++u) {
      if (s0 + u * SG < n_split) {
        const float mn = fmaxf(m, x[u]);
        const float sc = __expf(m - mn);   // 0 for the group's first split
        const float w = __expf(x[u] - mn);
        wsum = wsum * sc + w;
        a.x = a.x * sc + w * o[u].x;
        a.y = a.y * sc + w * o[u].y;
        a.z = a.z * sc + w * o[u].z;
        a.w = a.w * sc + w * o[u].w;
        m = mn;
      }
    }
  }
  if (c4 == 0) {
    m_g[sg] = m;
    l_g[sg] = wsum;
  }
  part[sg][c4] = a;
  __syncthreads();
  if (tid < C4) {
    float M = m_g[0];   // group 0 holds split 0, so M is finite
#pragma unroll
    for (int g2 = 1; g2 < SG; ++g2) M = fmaxf(M, m_g[g2]);
    float W = 0.0f;
    float4 t = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g2 = 0; g2 < SG; ++g2) {
      if (g2 >= n_split) break;   // groups past the split count hold nothing
      const float e = __expf(m_g[g2] - M);
      const float4 u = part[g2][tid];
      W += l_g[g2] * e;
      t.x += u.x * e;
      t.y += u.y * e;
      t.z += u.z * e;
      t.w += u.w * e;
    }
    const float inv = 1.0f / W;
    bf16x4 y;
    y[0] = (__bf16)(t.x * inv);
    y[1] = (__bf16)(t.y * inv);
    y[2] = (__bf16)(t.z * inv);
    y[3] = (__bf16)(t.w * inv);
    *reinterpret_cast<u32x2*>(out + row * D + 4 * tid) = __builtin_bit_cast(u32x2, y);
    if (tid == 0) lse[row] = M + __logf(W);
  }
}

// Key ranges of a decode call.  Two workgroups fill a CU (their LDS), so the
// workgroups run in rounds of 512 and a call takes about (rounds) x (keys per
// range + a fixed cost per workgroup).  Ranges are multiples of 128 keys (each
// of the four waves gets the same number of whole 32-key tiles); the count per
// row is chosen to minimise that product, preferring fewer ranges (less to
// combine), and never exceeds kDecMaxSplits.
struct DecodeSplit {
  int n_split, split_keys;
};
DecodeSplit decode_split(int B, int Lk, int n_kv) {
  const long long pairs = (long long)B * n_kv;
  const long long chunks = ((long long)Lk + 127) / 128;   // 128-key pieces
  const long long max_n = chunks < kDecMaxSplits ? chunks : kDecMaxSplits;
  long long best_n = 1, best_per = chunks * 128, best_cost = -1;
  // visit each distinct range length once: q = ceil(chunks / n) 128-key pieces
  for (long long n = 1; n <= max_n;) {
    const long long q = (chunks + n - 1) / n;
    const long long per = q * 128;                                // keys per range
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

extern "C" int attn_prefill_schedule(int B, int Lq, int Lk, int q_offset, int n_q, int n_kv,
                                     int d_h, int causal, int n_cu, long long* plan, int* list,
                                     int* rounds) {
  if (!plan) return ATTN_PREFILL_ERR_NULL_PTR;
  if (B < 1 || Lq < 1 || Lk < 1 || n_q < 1 || n_kv < 1 || n_cu < 1)
    return ATTN_PREFILL_ERR_BAD_SHAPE;
  if (n_q % n_kv != 0) return ATTN_PREFILL_ERR_BAD_GQA;
  if (d_h != 64 && d_h != 128) return ATTN_PREFILL_ERR_BAD_HEADDIM;
  if (causal != 0 && causal != 1) return ATTN_PREFILL_ERR_BAD_CAUSAL;
  if (q_offset < 0 || (causal && (long long)q_offset + Lq > Lk)) return ATTN_PREFILL_ERR_BAD_OFFSET;
  const int hwg = pick_hwg(n_q / n_kv);
  const long long br = kCols / hwg;
  const long long n_qblk = (Lq + br - 1) / br;
  const long long ngroups = (n_q / n_kv) / hwg;
  const long long ipq = (long long)B * n_kv * ngroups;
  const long long n_items = ipq * n_qblk;
  if (ipq > INT_MAX || n_items > INT_MAX / 2) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  const long long grid = n_items < n_cu ? n_items : n_cu;
  const ListForm f = list_form(n_items, ipq, n_qblk, ngroups, grid, causal);
  const long long R = (n_items + grid - 1) / grid;
  plan[0] = grid;
  plan[1] = n_items;
  plan[2] = n_qblk;
  plan[3] = ipq;
  plan[4] = f.sg;
  plan[5] = f.pair_t;
  plan[6] = f.pair_rounds;
  plan[7] = f.r_static < R ? f.r_static : R;
  ItemList lst;
  lst.n_qblk = (int)n_qblk;
  lst.ipq = (int)ipq;
  lst.ngroups = (int)ngroups;
  lst.sg = f.sg;
  lst.pair_t = f.pair_t;
  lst.pair_rounds = (int)f.pair_rounds;
  if (list)
    for (long long e = 0; e < n_items; ++e)
      list_decode(lst, (int)e, (int)grid, list[3 * e], list[3 * e + 1], list[3 * e + 2]);
  if (rounds)
    for (long long r = 0; r < R; ++r)
      for (long long w = 0; w < grid; ++w) {
        const int it = list_item_at(lst, (int)r, (int)w, (int)grid);
        rounds[r * grid + w] = it < n_items ? it : -1;
      }
  return ATTN_PREFILL_OK;
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

extern "C" int attn_prefill_version(void) { return 400; }
