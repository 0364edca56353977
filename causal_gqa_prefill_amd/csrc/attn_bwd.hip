// attn_bwd.hip -- backward pass of causal GQA prefill attention for gfx950.
//
// The gradients of O with respect to Q, K and V for an upstream gradient dO,
// recomputed from the forward pass's row statistic LSE instead of a stored
// score matrix ("Long-Context Attention Explained", section "What
// FlashAttention does not change").  With P_ij = exp(s_ij - LSE_i),
// s_ij = scale q_i . k_j over the visible keys:
//     D_i   = dO_i . O_i
//     dV_j  = sum_i P_ij dO_i                 (over the group's query heads)
//     dS_ij = P_ij (dO_i . v_j - D_i)
//     dQ_i  = scale sum_j dS_ij k_j
//     dK_j  = scale sum_i dS_ij q_i           (over the group's query heads)
//
// Three kernels, no atomics:
//  * bwd_delta_kernel: D for every row (HBM-bound).
//  * bwd_dkdv_kernel: work item = (b, kv-head, 128-key block); four waves,
//    32 keys each (their K rows in registers, the item's V rows in LDS),
//    stream 32-row tiles of Q and dO (and the rows' LSE and D) of every query
//    head of the group through LDS and accumulate dK^T and dV^T in
//    registers; 65 KB of LDS and under 256 registers let two workgroups
//    share a CU.  Per tile and wave: S = Q K^T and dP = dO V^T with
//    queries as rows, so the accumulator holds one key per lane and 16
//    queries in the slot order of the B operand; then dV^T += dO^T P and
//    dK^T += Q^T dS with dO^T and Q^T read from LDS by the transpose read.
//  * bwd_dq_kernel: work item and query columns as the forward kernel; each
//    wave keeps its 32 rows of Q and dO in registers and streams K and V
//    tiles: S^T = K Q^T, dP^T = V dO^T (one query per lane), then
//    dQ^T += K^T dS^T with K^T from the transpose read.
// P and dS are rounded to bf16 (nearest even) for the products, everything
// accumulates in fp32, and the gradients are rounded to bf16 once.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "attn_prefill.h"
#include "device_common.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte chunk swizzles of rows of 2 D bytes (the LDS has 64 banks of 4
// bytes, so a 256-byte window spans them all; for D = 64 two rows share
// one).  "row": for tiles read only by 16-byte row reads, where a pass of 16
// lanes takes 16 consecutive rows at one chunk: the 16 rows must land on 16
// different chunk positions.  "tr": for tiles read both that way and by the
// transpose read, where a pass of 32 lanes takes an aligned group of 4 rows,
// 64 bytes (a 4-aligned group of 4 chunks) of each: besides the row-read
// condition the 4 rows must fall in 4 different 64-byte windows (D = 64:
// the two rows of each parity in 2 different ones).  It also maps the
// column block tb of row r + 8 (r % 16 < 8) to where block tb ^ 1 of row r
// sits, so the transpose read's second row group is the first one's address
// for tb ^ 1 plus 8 rows (no address of its own).  As 4 f + g (f: 64-byte
// window, g: chunk in it), with r = 8 r3 + 4 r2 + 2 r1 + r0:
//   D = 128: f = (2 r1 + r0) ^ r3, g = 2 r0 + r2;
//   D = 64:  f = r1 ^ r3,          g = 2 r2 + r1.
template <int D>
__device__ __forceinline__ int swz_row(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_tr(int row) {
  if (D == 128) return 4 * ((row & 3) ^ ((row >> 3) & 1)) + 2 * (row & 1) + ((row >> 2) & 1);
  return 4 * (((row >> 1) ^ (row >> 3)) & 1) + 2 * ((row >> 2) & 1) + ((row >> 1) & 1);
}

// A 16-byte operand fragment of row `row` (relative to a tile at `base`),
// logical chunk `chunk`, under swizzle `swz`.
template <int D>
__device__ __forceinline__ bf16x8 frag16(LDS_AS const unsigned char* base, int row, int chunk,
                                         int swz) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(base + row * (2 * D) + ((chunk ^ swz) << 4));
}

// Transposed operand: for lanes l (hi = l / 32) of a 32-row block at `base`
// (rows = the contraction dimension, in the slot order 16 ks + 8 (s / 4) +
// 4 hi + s % 4), the 8 values of column 32 tb + l % 32 for k-step ks.
// In each group of 16 lanes, lane 4 r + qq supplies four consecutive 16-bit
// values of row r and lane i receives column i of the four rows.
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(LDS_AS const unsigned char* base, int tb, int ks,
                                          int lane) {
  constexpr int ROWB = 2 * D;
  const int hi = lane >> 5;
  const int tr_r = (lane >> 2) & 3;
  const int tr_q = lane & 3;
  const int tr_g = (lane >> 4) & 1;
  const int key = 16 * ks + 4 * hi + tr_r;
  // this lane's 8 bytes of row key in column block c
  auto at = [&](int c) __attribute__((always_inline)) {
    const int t = 32 * c + 16 * tr_g + 4 * tr_q;
    return base + key * ROWB + (((t >> 3) ^ swz_tr<D>(key)) << 4) + ((t >> 2) & 1) * 8;
  };
  // rows key + 8: under the swizzle, block tb there is block tb ^ 1 of row key moved 8 rows
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)at(tb));
  const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(at(tb ^ 1) + 8 * ROWB));
  return __builtin_bit_cast(
      bf16x8, (u32x4){__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                      __builtin_bit_cast(u32x2, up)[0], __builtin_bit_cast(u32x2, up)[1]});
}

// Source offsets of one wave's share of a tile load (rows of 256 bytes,
// `loads` loads of 1 KB starting at LDS byte 1 KB * first), placing logical
// chunk c of row r at physical chunk c ^ swz(r).
template <int D, bool TR>
__device__ __forceinline__ int tile_src(int first, int s, int lane) {
  constexpr int ROWB = 2 * D;
  const int byte = (first + s) * 1024 + lane * 16;
  const int row = byte / ROWB;
  const int pos = (byte % ROWB) >> 4;
  return row * ROWB + ((pos ^ (TR ? swz_tr<D>(row) : swz_row<D>(row))) << 4);
}

// ---- D_i = dO_i . O_i, fp32: D / 8 lanes per row (8 elements each)
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const unsigned short* __restrict__ out,
                                                        const unsigned short* __restrict__ dout,
                                                        float* __restrict__ delta,
                                                        long long rows) {
  constexpr int PER_ROW = D / 8;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid / PER_ROW;
  const int part = threadIdx.x % PER_ROW;
  float acc = 0.0f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(out + row * D + part * 8);
    const u32x4 d = *reinterpret_cast<const u32x4*>(dout + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // copy the element out first: a bit cast of an ext-vector element
      // itself compiled to a cast of element 0 on this toolchain
      const unsigned ae = a[e], de = d[e];
      const bf16x2 x = __builtin_bit_cast(bf16x2, ae);
      const bf16x2 y = __builtin_bit_cast(bf16x2, de);
      acc = fmaf((float)x[0], (float)y[0], acc);
      acc = fmaf((float)x[1], (float)y[1], acc);
    }
  }
#pragma unroll
  for (int o = PER_ROW / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, PER_ROW);
  if (row < rows && part == 0) delta[row] = acc;
}

// ---- dK, dV
constexpr int kKvGroupWaves = 4;                // waves of a group: 32 keys each
constexpr int kKvKeys = 32 * kKvGroupWaves;     // keys per work item
constexpr int kKvAhead = 1;     // S / dP operand reads issued this many k-steps ahead
constexpr int kKvTrAhead = 2;   // dV / dK operand reads issued this many MFMAs ahead
constexpr int kQT = 32;                         // query rows per tile

// NG groups of four waves share the item's key block (the same K rows in
// each group's registers, one copy of its V rows in LDS) and take every
// NG-th query tile.  NG = 1: 65 KB of LDS and at most 256 registers, two
// workgroups per CU.  NG = 2: one workgroup per CU that a key block most
// queries see keeps busy on its own (for grids of a few rounds, where such
// a block would otherwise run alone at one wave per SIMD); at the end the
// second group's fp32 partial sums of dK^T and dV^T are added into the
// first group's through LDS and the first group writes the result.
template <int D, int NG>
__global__ __launch_bounds__(64 * kKvGroupWaves * NG) __attribute__((amdgpu_waves_per_eu(2))) void
bwd_dkdv_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, const unsigned short* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    unsigned short* __restrict__ dk, unsigned short* __restrict__ dv, int L, int n_q, int n_kv,
    int n_kblk, float scale, int causal) {
  constexpr int ROWB = 2 * D;
  constexpr int KSTEPS = D / 16;
  constexpr int TBLK = D / 32;
  constexpr int V_BYTES = kKvKeys * ROWB;         // 32 KB: the item's V rows
  constexpr int QT_BYTES = kQT * ROWB;            // 8 KB: one Q (or dO) tile
  constexpr int VOFF = 0;
  // per group: 2 buffers of Q tiles, 2 of dO tiles, 2 x (32 lse + 32 delta
  // floats, padded to 256 bytes each)
  constexpr int G_QOFF = 0;
  constexpr int G_DOOFF = 2 * QT_BYTES;
  constexpr int G_STOFF = 4 * QT_BYTES;
  constexpr int G_BYTES = G_STOFF + 2 * 512;
  constexpr int GOFF = V_BYTES;                   // group areas after the V rows
  constexpr int SMEM = GOFF + NG * G_BYTES;       // 65 or 98 KB (d_h = 128)
  constexpr int NWV = kKvGroupWaves * NG;         // waves per workgroup
  constexpr int V_LOADS = V_BYTES / (NWV * 1024);              // 8 or 4 per wave
  constexpr int QT_LOADS = QT_BYTES / (kKvGroupWaves * 1024);  // 2 per wave
  // the reduction (a group's dK^T or dV^T partials: 64 floats per lane per
  // wave) and the output staging (32 rows per wave) fit side by side
  constexpr int RED_BYTES = kKvGroupWaves * TBLK * 16 * 64 * 4;
  static_assert((NG == 2 ? RED_BYTES : 0) + kKvGroupWaves * 32 * ROWB <= SMEM,
                "reduction and staging must fit");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  LDS_AS unsigned char* const sl = (LDS_AS unsigned char*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / kKvGroupWaves;           // which group
  const int gw = wave % kKvGroupWaves;            // wave inside the group
  const int lane = tid & 63;
  const int hi = lane >> 5;
  const int col = lane & 31;

  // work item: key blocks in order (block 0, the one most queries see,
  // first), so the hardware's in-order dispatch places the heaviest first
  const int item = blockIdx.x;
  const int kb = item / (gridDim.x / n_kblk);
  const int rest = item % (gridDim.x / n_kblk);
  const int kvh = rest % n_kv;
  const int b = rest / n_kv;
  const int g = n_q / n_kv;
  const int k0 = kb * kKvKeys;
  const int kw0 = k0 + 32 * gw;                   // this wave's first key

  // this wave's K rows as the B operand of S = Q K^T, straight from memory
  // into registers (zero past L): key kw0 + col, elements 16 kk + 8 hi .. +8
  bf16x8 kf[KSTEPS];
  {
    const size_t kvrow = ((size_t)b * n_kv + kvh) * (size_t)L + (size_t)(kw0 + col);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 a = {0u, 0u, 0u, 0u};
      if (kw0 + col < L) a = *reinterpret_cast<const u32x4*>(k + kvrow * D + kk * 16 + hi * 8);
      kf[kk] = __builtin_bit_cast(bf16x8, a);
    }
  }
  // the item's V rows into LDS (rows past L read as zero), the B operand of
  // dP = dO V^T; every wave of the workgroup loads a share
  {
    int src[V_LOADS];
#pragma unroll
    for (int s = 0; s < V_LOADS; ++s) src[s] = tile_src<D, false>(wave * V_LOADS, s, lane);
    dma_tile(v + ((size_t)b * n_kv + kvh) * (size_t)L * D, src, V_LOADS, ROWB, k0, L, kKvKeys,
             smem + VOFF + wave * V_LOADS * 1024);
  }
  int qsrc[QT_LOADS];
#pragma unroll
  for (int s = 0; s < QT_LOADS; ++s) qsrc[s] = tile_src<D, true>(gw * QT_LOADS, s, lane);
  LDS_AS unsigned char* const gl = sl + GOFF + grp * G_BYTES;   // this group's area

  // query tiles: every head of the group, rows from the first tile that can
  // see a key of the block (causal) or from 0; group grp takes tiles
  // n = NG i + grp
  const int qt_first = causal ? k0 / kQT : 0;
  const int qt_per_head = (L + kQT - 1) / kQT - qt_first;
  const int n_qt = g * qt_per_head;
  const int n_iter = (n_qt + NG - 1) / NG;
  auto tile_head = [&] __device__ (int n) __attribute__((always_inline)) {
    return kvh * g + n / qt_per_head;
  };
  auto tile_q0 = [&] __device__ (int n) __attribute__((always_inline)) {
    return (qt_first + n % qt_per_head) * kQT;
  };
  // loads of this group's tile n into its buffer `buf`: Q and dO rows (zero
  // past L), and the rows' LSE and delta (the group's first wave, 4 bytes
  // per lane; zero past L)
  auto load_qtile = [&] __device__ (int n, int buf) __attribute__((always_inline)) {
    const int q0 = tile_q0(n);
    const size_t rowbase = ((size_t)b * n_q + tile_head(n)) * (size_t)L;
    dma_tile(q + rowbase * D, qsrc, QT_LOADS, ROWB, q0, L, kQT,
             smem + GOFF + grp * G_BYTES + G_QOFF + buf * QT_BYTES + gw * QT_LOADS * 1024);
    dma_tile(dout + rowbase * D, qsrc, QT_LOADS, ROWB, q0, L, kQT,
             smem + GOFF + grp * G_BYTES + G_DOOFF + buf * QT_BYTES + gw * QT_LOADS * 1024);
    if (gw == 0) {
      const int lim = max(min(L - q0, 64), 0) * 4;
      const unsigned st = lds_addr(smem + GOFF + grp * G_BYTES + G_STOFF + buf * 512);
      lds_load_b32(buffer_words(lse + rowbase + q0, lim), lane * 4, st);
      lds_load_b32(buffer_words(delta + rowbase + q0, lim), lane * 4, st + 256);
    }
  };

  f32x16 dkT[TBLK], dvT[TBLK];
#pragma unroll
  for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkT[tb][r] = dvT[tb][r] = 0.0f;
  const float c2 = scale * kLog2e;
  // the mask's per-lane limit plus the tile's first query q0 (< L): a key
  // at or past L is dead for every slot (key + 32 - q0 > 31), a causal key
  // kw0 + col for the queries before it (lanes of half hi hold queries
  // q0 + 4 hi + ...), otherwise none (0 - q0 <= 0)
  const int key_lim = kw0 + col >= L ? kw0 + col + 32 : (causal ? kw0 + col - 4 * hi : 0);

  if (grp < n_qt) load_qtile(grp, 0);
  for (int i = 0; i < n_iter; ++i) {
    // this wave's loads of tile NG i + grp (and the V rows) have landed;
    // after the barrier every wave's have, and every wave is done with the
    // buffer the next loads overwrite.  The group's first wave, which loaded
    // the tile's LSE, turns it into -log2(e) LSE in place before the barrier
    // (once per tile, instead of a multiply per score in every wave; the
    // same fp32 product either way)
    wait_vmcnt<0>();
    if (gw == 0 && NG * i + grp < n_qt) {
      LDS_AS float* const lse_t = (LDS_AS float*)(gl + G_STOFF + (i & 1) * 512);
      lse_t[lane] = -(lse_t[lane] * kLog2e);
      wait_lgkm0();
    }
    tile_barrier();
    const int n = NG * i + grp;
    if (n + NG < n_qt) load_qtile(n + NG, (i + 1) & 1);
    if (n >= n_qt) continue;
    const int q0 = tile_q0(n);
    const int buf = i & 1;
    // skip when every query of the tile is before every key of the wave
    if (causal && q0 + kQT - 1 < kw0) continue;
    LDS_AS const unsigned char* qt = gl + G_QOFF + buf * QT_BYTES;
    LDS_AS const unsigned char* dot = gl + G_DOOFF + buf * QT_BYTES;
    LDS_AS const unsigned char* vt = sl + VOFF + 32 * gw * ROWB;
    LDS_AS const float* st = (LDS_AS const float*)(gl + G_STOFF + buf * 512);

    // S = Q K^T and dP = dO V^T: rows = queries (A from the Q / dO tile),
    // columns = this wave's keys (B from its K registers / the V rows).  The
    // LDS fragments are read kKvAhead k-steps ahead of their MFMAs (the
    // scheduling barriers keep that order).
    f32x16 S, dP;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
    bf16x8 qa[KSTEPS], oa[KSTEPS], va[KSTEPS];
    auto load_qov = [&] __device__ (int kk) __attribute__((always_inline)) {
      const int ch = 2 * kk + hi;
      qa[kk] = frag16<D>(qt, col, ch, swz_tr<D>(col));
      oa[kk] = frag16<D>(dot, col, ch, swz_tr<D>(col));
      va[kk] = frag16<D>(vt, col, ch, swz_row<D>(col));
    };
#pragma unroll
    for (int kk = 0; kk < kKvAhead; ++kk) load_qov(kk);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (kk + kKvAhead < KSTEPS) load_qov(kk + kKvAhead);
      __builtin_amdgcn_sched_barrier(0);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], kf[kk], S, 0, 0, 0);
      dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[kk], va[kk], dP, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first transposed fragments of the dV / dK products, read while
    // the VALU forms P and dS: MFMA i of that phase is (ks, tb, which) =
    // (i / (2 TBLK), i / 2 % TBLK, i % 2), which = 0 for dV (dO^T), 1 for dK (Q^T)
    bf16x8 tf[4 * TBLK];
    auto load_tr = [&] __device__ (int i) __attribute__((always_inline)) {
      tf[i] = frag_tr<D>(i % 2 == 0 ? dot : qt, (i / 2) % TBLK, i / (2 * TBLK), lane);
    };
#pragma unroll
    for (int i = 0; i < kKvTrAhead; ++i) load_tr(i);
    __builtin_amdgcn_sched_barrier(0);
    // P = 2^(c2 s - log2e lse), dS = P (dP - D) (the tile's LSE already
    // scaled by -log2 e); lane (key col) holds
    // queries 8 (r / 4) + 4 hi + r % 4
    bf16x8 pk[2], dsk[2];
    // masked scores go in as -inf (2^-inf = 0): a select, where a
    // conditional exponential would become a branch per element.  Slot
    // r = 4 a + c holds query q0 + 4 hi + (8 a + c), dead when 8 a + c < lim.
    const int lim = key_lim - q0;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const f32x4 l4 = *reinterpret_cast<const LDS_AS f32x4*>(st + 8 * a + 4 * hi);
      const f32x4 d4 = *reinterpret_cast<const LDS_AS f32x4*>(st + 64 + 8 * a + 4 * hi);
      const float lv[4] = {l4[0], l4[1], l4[2], l4[3]};
      const float dv4[4] = {d4[0], d4[1], d4[2], d4[3]};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int r = 4 * a + c;
        const float x = fmaf(S[r], c2, lv[c]);   // lv: -log2(e) LSE
        const float p = __builtin_amdgcn_exp2f(8 * a + c < lim ? -INFINITY : x);
        const float ds = p * (dP[r] - dv4[c]);
        pk[r >> 3][r & 7] = (__bf16)p;
        dsk[r >> 3][r & 7] = (__bf16)ds;
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS (contraction over the tile's queries),
    // each fragment read kKvTrAhead MFMAs ahead
#pragma unroll
    for (int i = 0; i < 4 * TBLK; ++i) {
      if (i + kKvTrAhead < 4 * TBLK) load_tr(i + kKvTrAhead);
      __builtin_amdgcn_sched_barrier(0);
      const int tb = (i / 2) % TBLK, ks = i / (2 * TBLK);
      if (i % 2 == 0)
        dvT[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[i], pk[ks], dvT[tb], 0, 0, 0);
      else
        dkT[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[i], dsk[ks], dkT[tb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();

  // ---- the second group's partial sums into the first group's registers,
  // dK^T then dV^T, through LDS at [0, RED_BYTES): wave gw of each group
  // holds the same keys in the same lane layout, 16 bytes per lane and
  // store, laid out (wave, register quad, lane)
  LDS_AS unsigned char* const red = sl + gw * (TBLK * 16 * 64 * 4) + lane * 16;
#pragma unroll
  for (int which = 0; which < (NG == 2 ? 2 : 0); ++which) {
    tile_barrier();   // the area is free (loop done / previous part read)
    if (grp == 1) {
#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x16& a = which == 0 ? dkT[tb] : dvT[tb];
          const f32x4 v4 = {a[4 * qd], a[4 * qd + 1], a[4 * qd + 2], a[4 * qd + 3]};
          *reinterpret_cast<LDS_AS f32x4*>(red + (tb * 4 + qd) * 1024) = v4;
        }
    }
    tile_barrier();
    if (grp == 0) {
#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const f32x4 v4 = *reinterpret_cast<const LDS_AS f32x4*>(red + (tb * 4 + qd) * 1024);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (which == 0)
              dkT[tb][4 * qd + e] += v4[e];
            else
              dvT[tb][4 * qd + e] += v4[e];
          }
        }
    }
  }
  if (grp != 0) return;

  // ---- epilogue (first group): dK = scale dK^T^T, then dV = dV^T^T, in
  // bf16, each staged through LDS (8 KB per wave) as whole rows; a wave
  // reads back only the rows it wrote, in order, so no barrier is needed
  // after the one that ends the loop (or the reduction)
  if (NG == 1) tile_barrier();
  LDS_AS unsigned char* ot = sl + (NG == 2 ? RED_BYTES : 0) + gw * 32 * ROWB;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
      for (int grp4 = 0; grp4 < 4; ++grp4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o4[e] = (__bf16)(which == 0 ? dkT[tb][grp4 * 4 + e] * scale : dvT[tb][grp4 * 4 + e]);
        const int chunk = tb * 4 + grp4;
        *reinterpret_cast<LDS_AS u32x2*>(ot + col * ROWB + ((chunk ^ swz_row<D>(col)) << 4) +
                                         hi * 8) = __builtin_bit_cast(u32x2, o4);
      }
    unsigned short* gbase = (which == 0 ? dk : dv) + (((size_t)b * n_kv + kvh) * L + kw0) * D;
#pragma unroll
    for (int st = 0; st < 32 * ROWB / 1024; ++st) {
      const int byte = st * 1024 + lane * 16;
      const int row = byte / ROWB;
      const int chunk = (byte % ROWB) >> 4;
      const u32x4 v4 =
          *reinterpret_cast<const LDS_AS u32x4*>(ot + row * ROWB + ((chunk ^ swz_row<D>(row)) << 4));
      if (kw0 + row < L) *reinterpret_cast<u32x4*>(gbase + (size_t)row * D + chunk * 8) = v4;
    }
  }
}

// ---- dQ
constexpr int kDqCols = 256;   // query columns per workgroup (8 waves x 32)
constexpr int kDqWaves = 8;
constexpr int kDqKeys = 64;    // keys per K/V tile
constexpr int kDqAhead = 2;    // LDS operand reads issued this many MFMA steps ahead

template <int D, int HWG>
__global__ __launch_bounds__(64 * kDqWaves) void bwd_dq_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, const unsigned short* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta,
    unsigned short* __restrict__ dq, int L, int n_q, int n_kv, int n_qblk, int items_per_qblk,
    float scale, int causal) {
  constexpr int ROWB = 2 * D;
  constexpr int KSTEPS = D / 16;
  constexpr int TBLK = D / 32;
  constexpr int BR = kDqCols / HWG;
  constexpr int TILE = kDqKeys * ROWB;                  // 16 KB
  constexpr int LOADS = TILE / (kDqWaves * 1024);       // 2 per wave
  constexpr int KOFF = 0, VOFF = 2 * TILE;              // two buffers each
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TILE];
  LDS_AS unsigned char* const sl = (LDS_AS unsigned char*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int hi = lane >> 5;
  const int col = lane & 31;

  const int item = blockIdx.x;
  const int qb = n_qblk - 1 - item / items_per_qblk;
  int rest = item % items_per_qblk;
  const int g = n_q / n_kv;
  const int ngroups = g / HWG;
  const int hg = rest % ngroups;
  rest /= ngroups;
  const int kvh = rest % n_kv;
  const int b = rest / n_kv;
  const int c0 = 32 * wave;
  const int hh = kvh * g + hg * HWG + c0 / BR;
  const int q0 = qb * BR + c0 % BR;
  const int qi = q0 + col;

  const size_t rowbase = ((size_t)b * n_q + hh) * (size_t)L;
  const unsigned short* kbase = k + ((size_t)b * n_kv + kvh) * (size_t)L * D;
  const unsigned short* vbase = v + ((size_t)b * n_kv + kvh) * (size_t)L * D;

  const int wg_end = min(qb * BR + BR, L);
  const int n_tiles = causal ? (wg_end + kDqKeys - 1) / kDqKeys : (L + kDqKeys - 1) / kDqKeys;
  const int last_row = q0 < L ? min(q0 + 31, L - 1) : -1;
  const int wave_tiles = last_row < 0 ? 0 : (causal ? last_row / kDqKeys + 1 : n_tiles);

  // Q and dO rows of the wave's 32 columns as B operands (zero past L)
  bf16x8 qf[KSTEPS], of[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (qi < L) {
      a = *reinterpret_cast<const u32x4*>(q + (rowbase + qi) * D + kk * 16 + hi * 8);
      c = *reinterpret_cast<const u32x4*>(dout + (rowbase + qi) * D + kk * 16 + hi * 8);
    }
    qf[kk] = __builtin_bit_cast(bf16x8, a);
    of[kk] = __builtin_bit_cast(bf16x8, c);
  }
  const float lse2 = qi < L ? lse[rowbase + qi] * kLog2e : 0.0f;
  const float dlt = qi < L ? delta[rowbase + qi] : 0.0f;

  int ksrc[LOADS], vsrc[LOADS];
#pragma unroll
  for (int s = 0; s < LOADS; ++s) {
    ksrc[s] = tile_src<D, true>(wave * LOADS, s, lane);    // K: row reads and transpose reads
    vsrc[s] = tile_src<D, false>(wave * LOADS, s, lane);   // V: row reads
  }
  auto load_tiles = [&] __device__ (int t) __attribute__((always_inline)) {
    const int buf = t & 1;
    dma_tile(kbase, ksrc, LOADS, ROWB, t * kDqKeys, L, kDqKeys,
             smem + KOFF + buf * TILE + wave * LOADS * 1024);
    dma_tile(vbase, vsrc, LOADS, ROWB, t * kDqKeys, L, kDqKeys,
             smem + VOFF + buf * TILE + wave * LOADS * 1024);
  };

  f32x16 dqT[TBLK];
#pragma unroll
  for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqT[tb][r] = 0.0f;
  const float c2 = scale * kLog2e;

  if (n_tiles > 0) load_tiles(0);
  for (int t = 0; t < n_tiles; ++t) {
    wait_vmcnt<0>();
    tile_barrier();
    if (t + 1 < n_tiles) load_tiles(t + 1);
    if (t >= wave_tiles) continue;
    const int buf = t & 1;
    LDS_AS const unsigned char* kt = sl + KOFF + buf * TILE;
    LDS_AS const unsigned char* vt = sl + VOFF + buf * TILE;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      const int j0 = t * kDqKeys + 32 * jb;
      LDS_AS const unsigned char* kh = kt + 32 * jb * ROWB;
      LDS_AS const unsigned char* vh = vt + 32 * jb * ROWB;
      // S^T = K Q^T and dP^T = V dO^T: rows = keys, columns = queries.  The
      // K and V fragments are read kDqAhead k-steps ahead of their MFMAs
      // (the scheduling barriers keep that order), so the LDS latency
      // overlaps the MFMAs instead of preceding each one.
      f32x16 S, dP;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.0f;
      bf16x8 ka[KSTEPS], va[KSTEPS];
      auto load_kv = [&] __device__ (int kk) __attribute__((always_inline)) {
        ka[kk] = frag16<D>(kh, col, 2 * kk + hi, swz_tr<D>(col));
        va[kk] = frag16<D>(vh, col, 2 * kk + hi, swz_row<D>(col));
      };
#pragma unroll
      for (int kk = 0; kk < kDqAhead; ++kk) load_kv(kk);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        if (kk + kDqAhead < KSTEPS) load_kv(kk + kDqAhead);
        __builtin_amdgcn_sched_barrier(0);
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], S, 0, 0, 0);
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk], of[kk], dP, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the first K^T fragments of the dQ product, read while the VALU
      // forms dS
      bf16x8 kt_f[2 * TBLK];
#pragma unroll
      for (int i = 0; i < kDqAhead; ++i) kt_f[i] = frag_tr<D>(kh, i % TBLK, i / TBLK, lane);
      __builtin_amdgcn_sched_barrier(0);
      // dS^T = P^T (dP^T - D), lane (query col) holds keys 8 (r / 4) + 4 hi + r % 4
      bf16x8 dsk[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = fmaf(S[r], c2, -lse2);
      // masked scores go in as -inf (2^-inf = 0), only where some key of the
      // half lies past some query of the wave or past L (a test uniform over
      // the wave).  Slot r holds key j0 + 4 hi + (8 (r / 4) + r % 4), dead
      // past lim: the lane's query (causal) or L - 1, less j0 + 4 hi.
      if ((causal && j0 + 31 > q0) || j0 + 31 >= L) {
        const int lim = min(causal ? qi : INT_MAX, L - 1) - j0 - 4 * hi;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) > lim) S[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(S[r]);
        dsk[r >> 3][r & 7] = (__bf16)(p * (dP[r] - dlt));
      }
      // dQ^T += K^T dS^T (contraction over the half's keys), MFMA i = (ks,
      // tb) = (i / TBLK, i % TBLK), its fragment read kDqAhead MFMAs ahead
#pragma unroll
      for (int i = 0; i < 2 * TBLK; ++i) {
        if (i + kDqAhead < 2 * TBLK)
          kt_f[i + kDqAhead] = frag_tr<D>(kh, (i + kDqAhead) % TBLK, (i + kDqAhead) / TBLK, lane);
        __builtin_amdgcn_sched_barrier(0);
        dqT[i % TBLK] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt_f[i], dsk[i / TBLK],
                                                               dqT[i % TBLK], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  wait_vmcnt<0>();

  // ---- epilogue: dQ = scale dQ^T^T in bf16, staged through LDS as whole rows
  tile_barrier();
  LDS_AS unsigned char* ot = sl + wave * 32 * ROWB;   // 8 KB per wave
#pragma unroll
  for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(dqT[tb][grp * 4 + e] * scale);
      const int chunk = tb * 4 + grp;
      *reinterpret_cast<LDS_AS u32x2*>(ot + col * ROWB + ((chunk ^ swz_row<D>(col)) << 4) +
                                       hi * 8) = __builtin_bit_cast(u32x2, o4);
    }
  unsigned short* obase = dq + (rowbase + q0) * D;
#pragma unroll
  for (int st = 0; st < 32 * ROWB / 1024; ++st) {
    const int byte = st * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int chunk = (byte % ROWB) >> 4;
    const u32x4 v4 =
        *reinterpret_cast<const LDS_AS u32x4*>(ot + row * ROWB + ((chunk ^ swz_row<D>(row)) << 4));
    if (q0 + row < L) *reinterpret_cast<u32x4*>(obase + (size_t)row * D + chunk * 8) = v4;
  }
}

int bwd_pick_hwg(int g) {
  if (g % 8 == 0) return 8;
  if (g % 4 == 0) return 4;
  if (g % 2 == 0) return 2;
  return 1;
}

template <int D, int HWG>
int launch_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
              const float* delta, void* dq, int B, int L, int n_q, int n_kv, float scale,
              int causal, hipStream_t stream) {
  constexpr int BR = kDqCols / HWG;
  const int n_qblk = (L + BR - 1) / BR;
  const long long items_per_qblk = (long long)B * n_kv * ((n_q / n_kv) / HWG);
  const long long grid = items_per_qblk * n_qblk;
  if (items_per_qblk > INT_MAX || grid > INT_MAX) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  hipLaunchKernelGGL((bwd_dq_kernel<D, HWG>), dim3((unsigned)grid), dim3(64 * kDqWaves), 0,
                     stream, static_cast<const unsigned short*>(q),
                     static_cast<const unsigned short*>(k), static_cast<const unsigned short*>(v),
                     static_cast<const unsigned short*>(dout), lse, delta,
                     static_cast<unsigned short*>(dq), L, n_q, n_kv, n_qblk,
                     (int)items_per_qblk, scale, causal);
  return hipGetLastError() == hipSuccess ? ATTN_PREFILL_OK : ATTN_PREFILL_ERR_LAUNCH;
}

// The three kernels of one backward call for head size D.
template <int D>
int launch_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int L,
               int n_q, int n_kv, long long rows, float scale, int causal, hipStream_t stream) {
  const long long n_kblk = ((long long)L + kKvKeys - 1) / kKvKeys;
  const long long kv_grid = (long long)B * n_kv * n_kblk;
  const long long delta_blocks = (rows * (D / 8) + 255) / 256;
  if (kv_grid > INT_MAX || delta_blocks > INT_MAX) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((unsigned)delta_blocks), dim3(256), 0, stream,
                     static_cast<const unsigned short*>(out),
                     static_cast<const unsigned short*>(dout), delta, rows);
  if (hipGetLastError() != hipSuccess) return ATTN_PREFILL_ERR_LAUNCH;
  // A causal key block's work grows with the queries that see it (block 0:
  // all of them).  When the grid is only a few rounds of two workgroups per
  // CU, the heaviest blocks would end up running alone on a CU at one wave
  // per SIMD, well past the average load; then two groups share each block
  // in a workgroup that fills the CU (the same holds for a non-causal grid
  // that does not fill the CUs).
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu < 1)
    return ATTN_PREFILL_ERR_LAUNCH;
  const bool split = causal ? kv_grid <= 3LL * n_cu : kv_grid <= n_cu;
  if (split)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, 2>), dim3((unsigned)kv_grid), dim3(64 * kKvGroupWaves * 2),
                       0, stream, static_cast<const unsigned short*>(q),
                       static_cast<const unsigned short*>(k), static_cast<const unsigned short*>(v),
                       static_cast<const unsigned short*>(dout), lse, delta,
                       static_cast<unsigned short*>(dk), static_cast<unsigned short*>(dv), L, n_q,
                       n_kv, (int)n_kblk, scale, causal);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, 1>), dim3((unsigned)kv_grid), dim3(64 * kKvGroupWaves),
                       0, stream, static_cast<const unsigned short*>(q),
                       static_cast<const unsigned short*>(k), static_cast<const unsigned short*>(v),
                       static_cast<const unsigned short*>(dout), lse, delta,
                       static_cast<unsigned short*>(dk), static_cast<unsigned short*>(dv), L, n_q,
                       n_kv, (int)n_kblk, scale, causal);
  if (hipGetLastError() != hipSuccess) return ATTN_PREFILL_ERR_LAUNCH;
  switch (bwd_pick_hwg(n_q / n_kv)) {
    case 8: return launch_dq<D, 8>(q, k, v, dout, lse, delta, dq, B, L, n_q, n_kv, scale, causal, stream);
    case 4: return launch_dq<D, 4>(q, k, v, dout, lse, delta, dq, B, L, n_q, n_kv, scale, causal, stream);
    case 2: return launch_dq<D, 2>(q, k, v, dout, lse, delta, dq, B, L, n_q, n_kv, scale, causal, stream);
    default: return launch_dq<D, 1>(q, k, v, dout, lse, delta, dq, B, L, n_q, n_kv, scale, causal, stream);
  }
}

}  // namespace

extern "C" int attn_prefill_bwd(const void* q, const void* k, const void* v, const void* out,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                float* delta, int B, int L, int n_q, int n_kv, int d_h,
                                float scale, int causal, hipStream_t stream) {
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv || !delta)
    return ATTN_PREFILL_ERR_NULL_PTR;
  if (B < 1 || L < 1 || n_q < 1 || n_kv < 1) return ATTN_PREFILL_ERR_BAD_SHAPE;
  if (n_q % n_kv != 0) return ATTN_PREFILL_ERR_BAD_GQA;
  if (d_h != 64 && d_h != 128) return ATTN_PREFILL_ERR_BAD_HEADDIM;
  if (!std::isfinite(scale)) return ATTN_PREFILL_ERR_BAD_SCALE;
  if (causal != 0 && causal != 1) return ATTN_PREFILL_ERR_BAD_CAUSAL;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out) |
                          reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq) |
                          reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv);
  if ((align & 15) != 0 ||
      ((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(delta)) & 3) != 0)
    return ATTN_PREFILL_ERR_MISALIGNED;
  size_t rows, q_elems, kv_elems;
  if (__builtin_mul_overflow((size_t)B, (size_t)n_q, &rows) ||
      __builtin_mul_overflow(rows, (size_t)L, &rows) ||
      __builtin_mul_overflow(rows, (size_t)d_h, &q_elems) ||
      __builtin_mul_overflow((size_t)B, (size_t)n_kv, &kv_elems) ||
      __builtin_mul_overflow(kv_elems, (size_t)L, &kv_elems) ||
      __builtin_mul_overflow(kv_elems, (size_t)d_h, &kv_elems) ||
      q_elems > ((size_t)1 << 61) || kv_elems > ((size_t)1 << 61))
    return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  const size_t qb = q_elems * 2, kvb = kv_elems * 2, lb = rows * 4;
  // the outputs may overlap nothing
  const void* outs[4] = {dq, dk, dv, delta};
  const size_t osz[4] = {qb, kvb, kvb, lb};
  const void* ins[6] = {q, k, v, out, lse, dout};
  const size_t isz[6] = {qb, kvb, kvb, qb, lb, qb};
  for (int a = 0; a < 4; ++a) {
    for (int c = 0; c < 6; ++c)
      if (overlaps(outs[a], osz[a], ins[c], isz[c])) return ATTN_PREFILL_ERR_ALIASING;
    for (int c = a + 1; c < 4; ++c)
      if (overlaps(outs[a], osz[a], outs[c], osz[c])) return ATTN_PREFILL_ERR_ALIASING;
  }
  if (d_h == 128)
    return launch_bwd<128>(q, k, v, out, lse, dout, dq, dk, dv, delta, B, L, n_q, n_kv,
                           (long long)rows, scale, causal, stream);
  return launch_bwd<64>(q, k, v, out, lse, dout, dq, dk, dv, delta, B, L, n_q, n_kv,
                        (long long)rows, scale, causal, stream);
}
