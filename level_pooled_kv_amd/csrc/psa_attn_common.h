// Pieces of the gfx950 attention kernel of the PSA forward path: LDS tile
// layout, staging geometry and the per-query-block tile lists.
#pragma once

#include "psa_device.h"
#include "psa_launch.h"

namespace psa {

// Raw global data of 8 consecutive d values of one key row (float32 I/O path only).
struct Raw8f {
  U128 r[2];
  __device__ __forceinline__ void load(const float* p) { r[0] = ld128(p); r[1] = ld128(p + 4); }
  __device__ __forceinline__ U128 bf16() const {
    U128 o;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      o.w[2 * i] = pack_bf16x2(__uint_as_float(r[i].w[0]), __uint_as_float(r[i].w[1]));
      o.w[2 * i + 1] = pack_bf16x2(__uint_as_float(r[i].w[2]), __uint_as_float(r[i].w[3]));
    }
    return o;
  }
};

template <int D, int NW>
struct AttnCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kCpr = D / 8;                // 16-byte chunks per 64-row tile row (bf16)
  static constexpr int kRpb = 64 / kCpr;            // rows per 1 KB block (one wave-wide 16 B load)
  static constexpr int kBlocks = 64 / kRpb;         // 1 KB blocks per tile and tensor
  static constexpr int kBpw = kBlocks / NW;         // blocks each wave stages per tensor
  static constexpr int kDt = D / 32;                // 32-wide d blocks of O^T
  static constexpr int kQc = D / 16;                // 16-deep d chunks of Q K^T
  static_assert(kBpw >= 1 && kBlocks % NW == 0, "staging layout");
};

// LDS tiles are row-major [64 keys][D] bf16 with the 16-byte chunks of row r XOR-ed by a
// row-dependent mask. For K the mask spreads the 16 rows one 128-bit operand read
// touches over distinct banks; for V it spreads the 4 rows x 32 bytes that one
// 16-lane group of a transposing read touches. Both are permutations within a row,
// so a wave-wide direct load of whole rows stays conflict-free.
template <int D> __device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D> __device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}
// Tiles read both ways (16-byte operand rows and transposing reads: the backward's Q,
// dO and K tiles). For D = 128 the two 2-bit fields of row & 15 are swapped: still a
// permutation over 16 consecutive rows, and the 4 rows x 2 chunks that one 16-lane
// group of a transposing read touches land on 8 distinct chunks.
template <int D> __device__ __forceinline__ int qt_swz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : k_swz<D>(row);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// s_waitcnt immediate that waits until at most n vector-memory operations are in
// flight (vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt left at
// their maxima).
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | 0x0F70; }


// Per-tile descriptor (built once per query block): level | first block-list index << 2 |
// valid segments << 16 | causal-diagonal << 30 | irregular << 31.
struct TileInfo { int lvl, base, nseg; bool diag, irr; };
__device__ __forceinline__ TileInfo decode_tile(uint32_t d) {
  return TileInfo{(int)(d & 3u), (int)((d >> 2) & 0x3fffu), (int)((d >> 16) & 15u), ((d >> 30) & 1u) != 0,
                  (d >> 31) != 0};
}

// Wave-level (call from one whole wave): compact one level-map row into level-major
// lists of block indices (blist, ascending within a level), the first tile of each
// level (s_tile[0..4], s_tile[4] = tile count) and one descriptor per tile (tdesc).
// A hardware tile is 64 key rows of ONE level: 1 block at level 0, 2 at level 1,
// 4 at level 2, 8 at level 3. A tile is irregular (needs per-key fixups) when it is
// the last of its level and has padding segments or holds the ragged final KV block.
// Under causal use a tile is diagonal (needs per-query masking) when its last block
// index is diag_from or more (the blocks reaching the query block's own rows; pass
// nkb for none).
__device__ __forceinline__ void build_tile_lists(const int8_t* __restrict__ lrow, int nkb, int L, int N,
                                                 int diag_from, int16_t* blist, uint32_t* tdesc,
                                                 int* s_tile) {
  const int lane = threadIdx.x & 63;
  // the row's levels, one entry per lane and 64-entry round, loaded once with every load
  // in flight before any is used (a load per round waited for in turn costs a memory
  // latency per round, twice)
  constexpr int KR = kMaxKvBlocks / 64;
  int lv[KR];
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const int j = 64 * k + lane;
    lv[k] = j < nkb ? (int)lrow[j] : -1;
  }
#pragma unroll
  for (int k = 0; k < KR; ++k)
    if (lv[k] >= L) lv[k] = -1;
  int cnt[4] = {0, 0, 0, 0};
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    if (64 * k >= nkb) break;
#pragma unroll
    for (int l = 0; l < 4; ++l) cnt[l] += __popcll(__ballot(lv[k] == l));
  }
  int pos[4];
  pos[0] = 0;
#pragma unroll
  for (int l = 1; l < 4; ++l) pos[l] = pos[l - 1] + cnt[l - 1];
  const int start[4] = {pos[0], pos[1], pos[2], pos[3]};
  int tfirst[5];
  tfirst[0] = 0;
#pragma unroll
  for (int l = 0; l < 4; ++l) tfirst[l + 1] = tfirst[l] + ((cnt[l] + (1 << l) - 1) >> l);
  if (lane == 0) {
#pragma unroll
    for (int l = 0; l < 5; ++l) s_tile[l] = tfirst[l];
  }
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    if (64 * k >= nkb) break;
    const int j = 64 * k + lane;
    const int lev = lv[k];
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const uint64_t m = __ballot(lev == l);
      if (lev == l) {
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        blist[pos[l] + below] = (int16_t)j;
      }
      pos[l] += __popcll(m);
    }
  }
  const int rem = N & 63;
#pragma unroll
  for (int l = 0; l < 4; ++l) {
    const int ntl = tfirst[l + 1] - tfirst[l];
    const bool tail = rem != 0 && cnt[l] > 0 && blist[start[l] + cnt[l] - 1] == nkb - 1;
    for (int u = lane; u < ntl; u += 64) {
      const int nseg = min(1 << l, cnt[l] - (u << l));
      const bool irr = u == ntl - 1 && (nseg < (1 << l) || tail);
      const bool diag = blist[start[l] + (u << l) + nseg - 1] >= diag_from;
      tdesc[tfirst[l] + u] = (uint32_t)l | ((uint32_t)(start[l] + (u << l)) << 2) | ((uint32_t)nseg << 16) |
                             (diag ? 0x40000000u : 0u) | (irr ? 0x80000000u : 0u);
    }
  }
}

// Last token a staged key row averages (for causal masking of diagonal tiles); padding
// rows and rows past the sequence get INT_MAX, so every query masks them.
__device__ __forceinline__ int key_last_token(bool ok, int lvl, int prow, int N) {
  return ok ? min((prow + 1) << lvl, N) - 1 : 0x7fffffff;
}

// Logit correction of one staged key row of an irregular tile, in units of the raw dot
// product: -inf for padding and rows past the sequence, (log2 c - l)/cs for a ragged pool
// group of c tokens, 0 otherwise.
__device__ __forceinline__ float key_correction(bool ok, int lvl, int prow, int N, float cs) {
  if (!ok) return -INFINITY;
  const int cnt = min(1 << lvl, N - (prow << lvl));
  return cnt == (1 << lvl) ? 0.f : (__log2f((float)cnt) - (float)lvl) / cs;
}

}  // namespace psa
