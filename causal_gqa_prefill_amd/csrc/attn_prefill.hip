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
//  * Grouped-query heads: the g query heads of one key/value head read the
//    same K/V tile from LDS, so K and V bytes are amortised over g heads
//    ("flops / prefill-attention", section "Arithmetic intensity").
//
// CDNA4 mapping:
//  * A workgroup is 8 wave64s.  Each wave owns 32 query rows of one head.  A
//    workgroup covers HW heads of one group times BR = 256 / HW rows, so the
//    K/V tile it stages in LDS is used by HW heads.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (from LDS) is the A operand, Q (held in
//    VGPRs for the whole loop) the B operand.  In the 32x32 result, lane l
//    holds 16 keys of query column l % 32, so the row max and row sum are
//    lane-local except for one exchange between lanes l and l ^ 32.
//  * The output is accumulated transposed, O^T += V^T P^T, with V^T (from
//    LDS) as the A operand and P^T as the B operand.  The score result's
//    register layout is used directly as the B operand: the 16 keys a lane
//    holds form the contraction slots of two k-steps in a permuted order,
//    and V^T is written to LDS in that same key order, so P never leaves the
//    registers.
//  * LDS tiles are XOR-swizzled in 16-byte chunks so both the 16-byte MFMA
//    operand reads and the tile writes are free of bank conflicts (the V^T
//    transposing writes are 4-way conflicted but are few).
//  * K/V tiles are double-buffered: the global loads of tile t+1 are in
//    flight while tile t is computed; one barrier per tile.
//  * exp is done as exp2 with scale*log2(e) folded into one FMA; LSE is
//    converted back to the natural log at the end.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "attn_prefill.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;            // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kBC = 64;              // keys per K/V tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Byte offset of (row, 16-byte chunk) in a swizzled K tile [kBC][D].
template <int D>
__device__ __forceinline__ int k_off(int j, int chunk) {
  return j * (2 * D) + ((chunk ^ (j & 7)) << 4);
}

// Swizzle of V^T row t: differs for the 8 rows one 8-lane read group touches
// and for the 8 rows (spaced by 8) one transposing write touches.
__device__ __forceinline__ int vt_swz(int t) { return (t & 7) ^ ((t >> 3) & 7); }

// Byte offset of (row t, 16-byte chunk) in a swizzled V^T tile [D][kBC].
__device__ __forceinline__ int vt_off(int t, int chunk) {
  return t * (2 * kBC) + ((chunk ^ vt_swz(t)) << 4);
}

// Position of key j (0..63) of a tile inside a V^T row.  Inside each group
// of 16 keys, bits 2 and 3 are swapped: this is the order in which the score
// result's registers feed the P V contraction as a B operand.
__device__ __forceinline__ int key_slot(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

template <int D, int HW>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k,
    const unsigned short* __restrict__ v, unsigned short* __restrict__ out,
    float* __restrict__ lse, int L, int n_q, int n_kv, int n_qblk, int items_per_qblk,
    float scale, int causal) {
  constexpr int BR = 32 * kWaves / HW;        // query rows per workgroup
  constexpr int KT_BYTES = kBC * D * 2;       // K tile
  constexpr int VT_BYTES = D * kBC * 2;       // V^T tile
  constexpr int STAGE = KT_BYTES + VT_BYTES;
  constexpr int KSTEPS = D / 16;              // k-steps of Q K^T
  constexpr int TBLK = D / 32;                // 32-wide blocks of O^T rows
  constexpr int KCHUNKS = D / 8;              // 16-byte chunks per K row
  constexpr int K_LOADS = kBC * KCHUNKS / kThreads;  // K chunks per thread
  constexpr int V_UNITS = (kBC / 2) * KCHUNKS;       // (row pair, chunk) units

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hi = lane >> 5;     // which half of the wave
  const int col = lane & 31;    // query column inside the wave's 32 rows

  // ---- work item: heavy q-blocks first; neighbouring ids differ in head
  const int item = blockIdx.x;
  const int qb = n_qblk - 1 - item / items_per_qblk;
  int rest = item % items_per_qblk;
  const int g = n_q / n_kv;
  const int ngroups = g / HW;
  const int hg = rest % ngroups;
  rest /= ngroups;
  const int kvh = rest % n_kv;
  const int b = rest / n_kv;

  const int h = kvh * g + hg * HW + (wave % HW);
  const int q0 = qb * BR + (wave / HW) * 32;  // first row of this wave
  const int qi = q0 + col;                    // this lane's query row

  const size_t L64 = (size_t)L;
  const unsigned short* qrow = q + (((size_t)b * n_q + h) * L64 + (size_t)qi) * D;
  const unsigned short* kbase = k + ((size_t)b * n_kv + kvh) * L64 * D;
  const unsigned short* vbase = v + ((size_t)b * n_kv + kvh) * L64 * D;

  // ---- tiles this workgroup streams, and the tiles this wave computes
  const int wg_end = min(qb * BR + BR, L);  // one past the last valid row
  const int n_tiles = causal ? (wg_end + kBC - 1) / kBC : (L + kBC - 1) / kBC;
  int wave_tiles = 0;
  if (q0 < L) wave_tiles = causal ? (min(q0 + 31, L - 1) / kBC + 1) : n_tiles;

  // ---- Q fragment, the B operand of S^T = K Q^T: Q[qi][16 kk + 8 hi + 0..7]
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qi < L) raw = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hi * 8);
    qf[kk] = __builtin_bit_cast(bf16x8, raw);
  }

  // ---- K/V tile staging: global -> registers -> LDS
  u32x4 kreg[K_LOADS];
  u32x4 vreg[2];
  const int v_unit_ok = tid < V_UNITS;
  const int v_pair = tid / KCHUNKS;   // rows 2 v_pair, 2 v_pair + 1
  const int v_chunk = tid % KCHUNKS;  // columns 8 v_chunk .. + 7

  auto load_tile = [&](int tile) {
    const int j0 = tile * kBC;
#pragma unroll
    for (int s = 0; s < K_LOADS; ++s) {
      const int id = tid + s * kThreads;
      const int j = id / KCHUNKS, c = id % KCHUNKS;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (j0 + j < L)
        raw = *reinterpret_cast<const u32x4*>(kbase + (size_t)(j0 + j) * D + c * 8);
      kreg[s] = raw;
    }
    if (v_unit_ok) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int j = j0 + 2 * v_pair + r;
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (j < L) raw = *reinterpret_cast<const u32x4*>(vbase + (size_t)j * D + v_chunk * 8);
        vreg[r] = raw;
      }
    }
  };

  auto store_tile = [&](int buf) {
    unsigned char* ks = smem + buf * STAGE;
    unsigned char* vs = ks + KT_BYTES;
#pragma unroll
    for (int s = 0; s < K_LOADS; ++s) {
      const int id = tid + s * kThreads;
      const int j = id / KCHUNKS, c = id % KCHUNKS;
      *reinterpret_cast<u32x4*>(ks + k_off<D>(j, c)) = kreg[s];
    }
    if (v_unit_ok) {
      // V rows j, j+1 (8 columns each) -> 8 V^T rows, one dword per row
      // holding (V[j][t], V[j+1][t]).
      const int j = 2 * v_pair;
      const int slot = key_slot(j);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned int w0 = vreg[0][e >> 1], w1 = vreg[1][e >> 1];
        // low halves for even columns, high halves for odd ones
        const unsigned int packed = (e & 1) ? __builtin_amdgcn_perm(w1, w0, 0x07060302u)
                                            : __builtin_amdgcn_perm(w1, w0, 0x05040100u);
        const int t = v_chunk * 8 + e;
        *reinterpret_cast<unsigned int*>(vs + vt_off(t, slot >> 3) + (slot & 7) * 2) = packed;
      }
    }
  };

  // ---- running state (log2 domain, scaled): m, lane-partial row sum, acc
  f32x16 acc[TBLK];
#pragma unroll
  for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[tb][r] = 0.0f;
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float c2 = scale * kLog2e;   // score -> log2 domain
  const bool fast_scale = c2 > 0.0f;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < n_tiles) load_tile(tile + 1);
    __syncthreads();

    if (tile < wave_tiles) {
      const unsigned char* ks = smem + buf * STAGE;
      const unsigned char* vs = ks + KT_BYTES;
      const int j0 = tile * kBC;

      // S^T = K Q^T for the tile's two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[jb][r] = 0.0f;
        const int j = jb * 32 + col;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + k_off<D>(j, 2 * kk + hi));
          s[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[jb], 0, 0, 0);
        }
      }

      // mask: keys after the query (causal) and keys past the end
      const bool need_mask = (causal && j0 + kBC - 1 > q0) || (j0 + kBC > L);
      float c = c2;
      if (need_mask || !fast_scale) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = j0 + jb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
            const bool dead = (causal && j > qi) || j >= L;
            s[jb][r] = dead ? -INFINITY : s[jb][r] * c2;
          }
        c = 1.0f;
      }

      // tile max of this lane's 32 scores, then across lanes l and l^32
      float mx = s[0][0];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;

      // p = 2^(c s - m); P^T in bf16 as the B operand of the P V k-steps
      bf16x8 pk[4];
      float psum = 0.0f;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 frag;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[jb][half * 8 + e], c, -m_new));
            psum += p;
            frag[e] = (__bf16)p;
          }
          pk[jb * 2 + half] = frag;
        }
      l_run = l_run * alpha + psum;

#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tb][r] *= alpha;

      // O^T += V^T P^T
#pragma unroll
      for (int tb = 0; tb < TBLK; ++tb) {
        const int t = tb * 32 + col;
#pragma unroll
        for (int ks4 = 0; ks4 < 4; ++ks4) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + vt_off(t, 2 * ks4 + hi));
          acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[ks4], acc[tb], 0, 0, 0);
        }
      }
    }

    if (tile + 1 < n_tiles) store_tile(buf ^ 1);
  }

  // ---- epilogue: O = acc / l in bf16, LSE = ln 2 * (m + log2 l)
  if (wave_tiles == 0 || qi >= L) return;
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.0f / l_tot;
  unsigned short* orow = out + (((size_t)b * n_q + h) * L64 + (size_t)qi) * D;
#pragma unroll
  for (int tb = 0; tb < TBLK; ++tb)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int t0 = tb * 32 + grp * 8 + hi * 4;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[tb][grp * 4 + e] * inv);
      *reinterpret_cast<u32x2*>(orow + t0) = __builtin_bit_cast(u32x2, o4);
    }
  if (hi == 0)
    lse[((size_t)b * n_q + h) * L64 + (size_t)qi] = (m_run + __log2f(l_tot)) * kLn2;
}

// Heads per workgroup: the largest of 8, 4, 2, 1 that divides g.
int pick_hw(int g) {
  if (g % 8 == 0) return 8;
  if (g % 4 == 0) return 4;
  if (g % 2 == 0) return 2;
  return 1;
}

template <int D, int HW>
int launch(const void* q, const void* k, const void* v, void* out, float* lse, int B, int L,
           int n_q, int n_kv, float scale, int causal, hipStream_t stream) {
  constexpr int BR = 32 * kWaves / HW;
  const int n_qblk = (L + BR - 1) / BR;
  const long long items_per_qblk = (long long)B * n_kv * ((n_q / n_kv) / HW);
  const long long grid = items_per_qblk * n_qblk;
  if (items_per_qblk > INT_MAX || grid > INT_MAX) return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  hipLaunchKernelGGL((attn_fwd_kernel<D, HW>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     static_cast<const unsigned short*>(q), static_cast<const unsigned short*>(k),
                     static_cast<const unsigned short*>(v), static_cast<unsigned short*>(out), lse,
                     L, n_q, n_kv, n_qblk, (int)items_per_qblk, scale, causal);
  return hipGetLastError() == hipSuccess ? ATTN_PREFILL_OK : ATTN_PREFILL_ERR_LAUNCH;
}

template <int D>
int launch_d(const void* q, const void* k, const void* v, void* out, float* lse, int B, int L,
             int n_q, int n_kv, float scale, int causal, hipStream_t stream) {
  switch (pick_hw(n_q / n_kv)) {
    case 8: return launch<D, 8>(q, k, v, out, lse, B, L, n_q, n_kv, scale, causal, stream);
    case 4: return launch<D, 4>(q, k, v, out, lse, B, L, n_q, n_kv, scale, causal, stream);
    case 2: return launch<D, 2>(q, k, v, out, lse, B, L, n_q, n_kv, scale, causal, stream);
    default: return launch<D, 1>(q, k, v, out, lse, B, L, n_q, n_kv, scale, causal, stream);
  }
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bn && y < x + an;
}

}  // namespace

extern "C" int attn_prefill_fwd(const void* q, const void* k, const void* v, void* out,
                                float* lse, int B, int L, int n_q, int n_kv, int d_h,
                                float scale, int causal, hipStream_t stream) {
  if (!q || !k || !v || !out || !lse) return ATTN_PREFILL_ERR_NULL_PTR;
  if (B < 1 || L < 1 || n_q < 1 || n_kv < 1) return ATTN_PREFILL_ERR_BAD_SHAPE;
  if (n_q % n_kv != 0) return ATTN_PREFILL_ERR_BAD_GQA;
  if (d_h != 64 && d_h != 128) return ATTN_PREFILL_ERR_BAD_HEADDIM;
  if (!std::isfinite(scale)) return ATTN_PREFILL_ERR_BAD_SCALE;
  if (causal != 0 && causal != 1) return ATTN_PREFILL_ERR_BAD_CAUSAL;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
  if ((align & 15) != 0 || (reinterpret_cast<uintptr_t>(lse) & 3) != 0)
    return ATTN_PREFILL_ERR_MISALIGNED;

  // element counts, checked for 64-bit overflow (bytes must fit in 2^62)
  size_t lse_elems, q_elems, kv_rows, kv_elems;
  if (__builtin_mul_overflow((size_t)B, (size_t)n_q, &lse_elems) ||
      __builtin_mul_overflow(lse_elems, (size_t)L, &lse_elems) ||
      __builtin_mul_overflow(lse_elems, (size_t)d_h, &q_elems) ||
      __builtin_mul_overflow((size_t)B, (size_t)n_kv, &kv_rows) ||
      __builtin_mul_overflow(kv_rows, (size_t)L, &kv_rows) ||
      __builtin_mul_overflow(kv_rows, (size_t)d_h, &kv_elems) ||
      q_elems > ((size_t)1 << 61) || kv_elems > ((size_t)1 << 61))
    return ATTN_PREFILL_ERR_SIZE_OVERFLOW;
  const size_t q_bytes = q_elems * 2, kv_bytes = kv_elems * 2, lse_bytes = lse_elems * 4;
  if (overlaps(out, q_bytes, q, q_bytes) || overlaps(out, q_bytes, k, kv_bytes) ||
      overlaps(out, q_bytes, v, kv_bytes) || overlaps(out, q_bytes, lse, lse_bytes) ||
      overlaps(lse, lse_bytes, q, q_bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
      overlaps(lse, lse_bytes, v, kv_bytes))
    return ATTN_PREFILL_ERR_ALIASING;

  if (d_h == 128) return launch_d<128>(q, k, v, out, lse, B, L, n_q, n_kv, scale, causal, stream);
  return launch_d<64>(q, k, v, out, lse, B, L, n_q, n_kv, scale, causal, stream);
}

extern "C" const char* attn_prefill_strerror(int status) {
  switch (status) {
    case ATTN_PREFILL_OK: return "success";
    case ATTN_PREFILL_ERR_NULL_PTR: return "a buffer pointer is NULL";
    case ATTN_PREFILL_ERR_BAD_SHAPE: return "B, L, n_q and n_kv must be >= 1";
    case ATTN_PREFILL_ERR_BAD_GQA: return "n_q must be a multiple of n_kv";
    case ATTN_PREFILL_ERR_BAD_HEADDIM: return "d_h must be 64 or 128";
    case ATTN_PREFILL_ERR_BAD_SCALE: return "scale must be finite";
    case ATTN_PREFILL_ERR_BAD_CAUSAL: return "causal must be 0 or 1";
    case ATTN_PREFILL_ERR_MISALIGNED:
      return "q, k, v and out must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_PREFILL_ERR_SIZE_OVERFLOW: return "sizes overflow the supported range";
    case ATTN_PREFILL_ERR_ALIASING: return "out or lse overlaps another buffer";
    case ATTN_PREFILL_ERR_LAUNCH: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int attn_prefill_version(void) { return 100; }
