// Step 2 of the PSA forward path on gfx950: block importance and the multi-level mask.
//
// Importance of KV block j for query block i is the mean query of the block
// against the block's mean key (skillmd.com page, "Block importance scoring");
// levels are assigned per (query block, KV block) pair by thresholds on the
// importance (chatpaper.ai abstract; top168.com article, ablation paragraph).
// Reading taken for the threshold rule: softmax the scores of a query-block row
// into a probability mass, rank blocks by score (ties by index), and give block j
// the lowest level l whose threshold exceeds the mass ranked strictly ahead of j.
//
// Kernels:
//  * qblock_mean_kernel streams Q once (HBM-bound: every load of a thread is in
//    flight at once, 16-byte nontemporal loads, whole rows per wave, two query blocks per
//    workgroup) and writes the float32 mean query of each query block to the workspace.
//  * block_score_kernel: z = scale * qbar kbar^T + ln n_j per head on the float32
//    matrix cores (v_mfma_f32_32x32x2_f32), one 32 x 32 tile per wave, into a
//    workspace row of n_pad floats per query block.
//  * qblock_score_kernel (rows of more than 512 KV blocks): both of the above in one
//    pass, the mean queries kept in LDS, 16 x 16 score tiles per product.
//  * block_level_sel_kernel (no cumulative mass asked): one wave per query-block row:
//    a histogram of the blocks' weights (integer masses from the softmax of the row, or 1
//    under the ranked rule) over buckets of the score, and an exact ranking of only the
//    blocks of the buckets that hold the cuts; a row it cannot settle takes the exact sort
//    (in the same kernel for rows of up to 512 blocks, in block_level_kernel for longer).
//  * block_level_kernel: one wave per query-block row: softmax of the row, a bitonic
//    sort of 64-bit (score, index) keys held in registers (n_pad / 64 per lane; partners
//    in other lanes come through cross-lane shuffles, so no LDS and no workgroup
//    barrier), a wave-wide exclusive scan of the integer masses in rank order, the
//    threshold compares and the int8 level writes (and the cumulative mass when asked).
//  * The ranked rule (the quantile rule the top168.com ablation compares with
//    thresholds; fixed shares of the score-ranked blocks per level: skillmd.com, "Level
//    assignment") gives the block at rank r the lowest level l with r < K_l for
//    host-computed cumulative counts K_l: the same passes with rank in place of mass.
#include "psa_device.h"
#include "psa_launch.h"

#include <cmath>

namespace psa {

constexpr int kMaskThreads = 256;

template <typename T, int D, int QB>
__global__ void __launch_bounds__(kMaskThreads)
qblock_mean_kernel(const T* __restrict__ q, float* __restrict__ qbar, int N, int q_block, int nqb) {
  constexpr int E = io_traits<T>::per16;
  constexpr int CPR = D / E;                // 16-byte chunks per row
  constexpr int G = kMaskThreads / CPR;     // row groups
  constexpr int MAXR = 128 / G;             // rows per thread at the largest query block
  __shared__ float red[QB][G][D];
  const int t = threadIdx.x;
  const int chunk = t % CPR, g = t / CPR;
  const int64_t bh = blockIdx.y;
  const int i0 = blockIdx.x * QB;           // QB query blocks per workgroup: every load in flight at once

  U128 raw[QB][MAXR];
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    const int r0 = (i0 + u) * q_block;
    const int m = i0 + u < nqb ? min(q_block, N - r0) : 0;
    const T* src = q + (bh * N + r0) * (int64_t)D + chunk * E;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const int row = g + r * G;
      raw[u][r] = row < m ? ld128_stream(src + (int64_t)row * D) : U128{{0u, 0u, 0u, 0u}};
    }
  }
#pragma unroll
  for (int u = 0; u < QB; ++u) {
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      float x[E];
      unpack16<T>(raw[u][r], x);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) red[u][g][chunk * E + e] = acc[e];
  }
  __syncthreads();
  for (int x = t; x < QB * D; x += kMaskThreads) {
    const int u = x / D, c = x - u * D;
    const int i = i0 + u;
    if (i >= nqb) continue;
    float s = 0.f;
#pragma unroll 8
    for (int gg = 0; gg < G; ++gg) s += red[u][gg][c];
    qbar[(bh * nqb + i) * D + c] = s / (float)min(q_block, N - i * q_block);
  }
}

// One 32 (KV blocks) x 32 (query blocks) tile of scores per wave, kScoreWaves waves
// (consecutive KV tiles) per workgroup sharing one query tile. Operand tiles are
// staged through LDS with coalesced 16-byte loads (rows padded by 4 floats, so the
// per-lane row reads of the MFMA operands are free of bank conflicts). The
// contraction index is split between the two lane halves as [0, D/2) and
// [D/2, D), the same split for both operands.
constexpr int kScoreWaves = 2;

template <int D>
__global__ void __launch_bounds__(64 * kScoreWaves)
block_score_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar, float* __restrict__ z,
                   int N, int H, int H_kv, int nqb, int nkb, int zstride, float scale) {
  constexpr int S = D / 2;                  // MFMA steps (k = 2 each)
  constexpr int RS = D + 4;                 // padded LDS row (floats)
  constexpr int F4 = 32 * D / 4;            // float4 per 32-row tile
  __shared__ __align__(16) float qs[32 * RS];
  __shared__ __align__(16) float ks[kScoreWaves][32 * RS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int kt = blockIdx.x * kScoreWaves + wave;
  const bool active = kt * 32 < nkb;        // whole wave
  const int qt = blockIdx.y;
  const int bh = blockIdx.z;
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / H_kv);

  const float* qsrc = qbar + (int64_t)bh * nqb * D;
#pragma unroll
  for (int c = 0; c < F4 / (64 * kScoreWaves); ++c) {
    const int f = t + 64 * kScoreWaves * c;
    const int row = f / (D / 4), col = 4 * (f % (D / 4));
    const int qi = min(qt * 32 + row, nqb - 1);
    *reinterpret_cast<float4*>(&qs[row * RS + col]) = *reinterpret_cast<const float4*>(qsrc + (int64_t)qi * D + col);
  }
  if (active) {
    const float* ksrc = kbar + (int64_t)(b * H_kv + g) * nkb * D;
#pragma unroll
    for (int c = 0; c < F4 / 64; ++c) {
      const int f = lane + 64 * c;
      const int row = f / (D / 4), col = 4 * (f % (D / 4));
      const int key = min(kt * 32 + row, nkb - 1);
      *reinterpret_cast<float4*>(&ks[wave][row * RS + col]) =
          *reinterpret_cast<const float4*>(ksrc + (int64_t)key * D + col);
    }
  }
  __syncthreads();
  if (!active) return;

  const int l32 = lane & 31, half = lane >> 5;
  const float* ka = &ks[wave][l32 * RS + half * S];
  const float* qa = &qs[l32 * RS + half * S];
  f32x16 acc;
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.f;
#pragma unroll
  for (int c = 0; c < S / 4; ++c) {
    const float4 kv = *reinterpret_cast<const float4*>(ka + 4 * c);
    const float4 qv = *reinterpret_cast<const float4*>(qa + 4 * c);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.x, qv.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.y, qv.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.z, qv.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.w, qv.w, acc, 0, 0, 0);
  }
  // accumulator v of lane l: query block 32 qt + l%32, KV block 32 kt + 8 (v/4) + 4 (l/32) + v%4
  const int row = qt * 32 + l32;
  if (row >= nqb) return;
  float* zr = z + ((int64_t)bh * nqb + row) * zstride;
  // ln n_j: every block but the last holds min(64, N) tokens
  const float ln_full = logf((float)min(64, N)), ln_last = logf((float)(N - 64 * (nkb - 1)));
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const int j0 = kt * 32 + 8 * g4 + 4 * half;
    float out[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int j = j0 + x;
      out[x] = fmaf(scale, acc[4 * g4 + x], j == nkb - 1 ? ln_last : ln_full);
    }
    if (j0 + 3 < nkb) {
      *reinterpret_cast<float4*>(zr + j0) = make_float4(out[0], out[1], out[2], out[3]);
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (j0 + x < nkb) zr[j0 + x] = out[x];
    }
  }
}

// For rows of more than 512 KV blocks, where the score products dominate: query-block means
// and block scores in one pass, one workgroup per (b, h) and 16 consecutive query blocks.
// The workgroup streams the 16 blocks' rows of Q once (the next block's loads in flight
// while the current one is reduced), keeps the float32 mean queries in LDS (the B operand)
// and computes z = scale * qbar kbar^T + ln n_j on the float32 matrix cores
// (v_mfma_f32_16x16x4_f32: 16 KV blocks x 16 query blocks per product), k_bar coming
// straight from global memory as the A operand, so neither the mean queries nor a k_bar
// tile pass through LDS staging. Two tiles per step give each wave two independent
// product chains.
template <typename T, int D>
__global__ void __launch_bounds__(kMaskThreads)
qblock_score_kernel(const T* __restrict__ q, const float* __restrict__ kbar, float* __restrict__ z, int N,
                    int H, int H_kv, int q_block, int nqb, int nkb, int zstride, float scale) {
  constexpr int R = 16;                     // query blocks per workgroup (the 16 product columns)
  constexpr int E16 = io_traits<T>::per16;  // elements per 16-byte chunk
  constexpr int CPR = D / E16;              // chunks per row
  constexpr int G = kMaskThreads / CPR;     // row groups
  constexpr int MAXR = 128 / G;             // rows per thread per query block (q_block <= 128)
  constexpr int QS = D + 4;                 // padded LDS row of the mean queries (floats)
  __shared__ __align__(16) float qs[R * QS];
  __shared__ float red[G][D];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i0 = blockIdx.x * R;            // first query block of the workgroup
  const int bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / H_kv);
  const int nrow = min(R, nqb - i0);        // query blocks present
  const int chunk = t % CPR, grp = t / CPR;
  const T* qh = q + (int64_t)bh * N * D + chunk * E16;

  for (int x = t; x < R * QS; x += kMaskThreads)   // absent query blocks: zero columns
    if (x / QS >= nrow) qs[x] = 0.f;

  auto load_block = [&](int r, U128 (&raw)[MAXR]) {
    const int r0 = (i0 + r) * q_block;
    const int m = r < nrow ? min(q_block, N - r0) : 0;
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
      const int row = grp + k * G;
      raw[k] = row < m ? ld128_stream(qh + (int64_t)(r0 + row) * D) : U128{{0u, 0u, 0u, 0u}};
    }
  };
  U128 buf[2][MAXR];
  load_block(0, buf[0]);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r + 1 < R) load_block(r + 1, buf[(r + 1) & 1]);
    float acc[E16];
#pragma unroll
    for (int e = 0; e < E16; ++e) acc[e] = 0.f;
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
      float x[E16];
      unpack16<T>(buf[r & 1][k], x);
#pragma unroll
      for (int e = 0; e < E16; ++e) acc[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < E16; ++e) red[grp][chunk * E16 + e] = acc[e];
    __syncthreads();
    if (t < D && r < nrow) {
      float sum = 0.f;
#pragma unroll 8
      for (int gg = 0; gg < G; ++gg) sum += red[gg][t];
      qs[r * QS + t] = sum / (float)min(q_block, N - (i0 + r) * q_block);
    }
    __syncthreads();
  }

  // scores: wave w takes 16-block tiles w + 8u and w + 8u + 4. Lane l supplies KV block
  // 16 tile + l%16 (operand A) and query column l%16 (operand B) at d = 16c + 4(l/16) + 0..3
  // (one float4 of each feeds four products), and receives blocks 16 tile + 4(l/16) + 0..3
  // of query column l%16.
  const float* kb = kbar + (int64_t)(b * H_kv + g) * nkb * D;
  const int ntiles = (nkb + 15) / 16;
  const int n = lane & 15, kq = lane >> 4;
  const float* qcol = qs + n * QS + 4 * kq;
  float* zr = z + ((int64_t)bh * nqb + i0 + n) * zstride;
  // ln n_j: every block but the last holds min(64, N) tokens
  const float ln_full = logf((float)min(64, N)), ln_last = logf((float)(N - 64 * (nkb - 1)));
  auto store = [&](int tile, const f32x4& acc) {
    if (n >= nrow || tile >= ntiles) return;
    const int j0 = tile * 16 + 4 * kq;
    float out[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) out[x] = fmaf(scale, acc[x], j0 + x == nkb - 1 ? ln_last : ln_full);
    if (j0 + 3 < nkb) {
      *reinterpret_cast<float4*>(zr + j0) = make_float4(out[0], out[1], out[2], out[3]);
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (j0 + x < nkb) zr[j0 + x] = out[x];
    }
  };
  for (int tile = wave; tile < ntiles; tile += 2 * (kMaskThreads / 64)) {
    const int tile1 = tile + kMaskThreads / 64;
    const float* krow0 = kb + (int64_t)min(tile * 16 + n, nkb - 1) * D + 4 * kq;
    const float* krow1 = kb + (int64_t)min(tile1 * 16 + n, nkb - 1) * D + 4 * kq;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const float4 a0 = *reinterpret_cast<const float4*>(krow0 + 16 * c);
      const float4 a1 = *reinterpret_cast<const float4*>(krow1 + 16 * c);
      const float4 bq = *reinterpret_cast<const float4*>(qcol + 16 * c);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.x, bq.x, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.x, bq.x, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.y, bq.y, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.y, bq.y, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.z, bq.z, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.z, bq.z, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.w, bq.w, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.w, bq.w, acc1, 0, 0, 0);
    }
    store(tile, acc0);
    store(tile1, acc1);
  }
}

// Butterfly reductions over the wave with VALU cross-lane moves; every lane gets the result.
__device__ __forceinline__ float wave_max(float x) {
  const int lane = lane_id();
  x = fmaxf(x, __uint_as_float(xor_lane<1>(__float_as_uint(x), lane)));
  x = fmaxf(x, __uint_as_float(xor_lane<2>(__float_as_uint(x), lane)));
  x = fmaxf(x, __uint_as_float(xor_lane<4>(__float_as_uint(x), lane)));
  x = fmaxf(x, __uint_as_float(xor_lane<8>(__float_as_uint(x), lane)));
  x = fmaxf(x, __uint_as_float(xor_lane<16>(__float_as_uint(x), lane)));
  x = fmaxf(x, __uint_as_float(xor_lane<32>(__float_as_uint(x), lane)));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x, lane_id()); }

// Sort key: ascending key order = score descending, then block index ascending.
// The high word is an order-reversing bijection of the float's bits (so the score
// can be recovered from a sorted key), the low word the block index.
__device__ __forceinline__ uint64_t rank_key(float z, int j) {
  const uint32_t u = __float_as_uint(z + 0.0f);          // -0 -> +0
  const uint32_t key = (u & 0x80000000u) ? u : (~u & 0x7fffffffu);
  return ((uint64_t)key << 32) | (uint32_t)j;
}
__device__ __forceinline__ float key_score(uint64_t k) {
  const uint32_t key = (uint32_t)(k >> 32);
  return __uint_as_float((key & 0x80000000u) ? key : (~key & 0x7fffffffu));
}

template <int M>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t x, int lane) {
  const uint32_t lo = xor_lane<M>((uint32_t)x, lane);
  const uint32_t hi = xor_lane<M>((uint32_t)(x >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Ascending bitonic sort of the 64 E keys of one wave; element e = E * lane + r is
// key[r] of lane `lane`. Pairs at distance J < E are in one lane; at J >= E the
// partner is lane ^ (J / E), same r. Every exchange is a select on a compare, no
// branch; the network is unrolled at compile time, so every direction test folds to
// a per-lane constant.
template <int E, int M>
__device__ __forceinline__ void stage_cross64(uint64_t (&key)[E], int lane, int k) {
  const bool upper = (lane & M) != 0;                   // holds the higher element of its pair
  const bool asc = ((E * lane) & k) == 0;               // k >= 2E: the same for every r
  const bool keep_max = upper == asc;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const uint64_t y = xor_lane64<M>(key[r], lane);
    key[r] = ((y > key[r]) == keep_max) ? y : key[r];
  }
}
template <int E, int J>
__device__ __forceinline__ void stage_in64(uint64_t (&key)[E], int lane, int k) {
#pragma unroll
  for (int r = 0; r < E; ++r) {
    if (r & J) continue;
    const bool asc = ((E * lane + r) & k) == 0;
    const uint64_t a = key[r], c = key[r + J];
    const bool swap = (a > c) == asc;
    key[r] = swap ? c : a;
    key[r + J] = swap ? a : c;
  }
}
template <int E, int K, int J>
__device__ __forceinline__ void merge64(uint64_t (&key)[E], int lane) {
  if constexpr (J > 0) {
    if constexpr (J >= E) stage_cross64<E, J / E>(key, lane, K);
    else stage_in64<E, J>(key, lane, K);
    merge64<E, K, J / 2>(key, lane);
  }
}
template <int E, int K = 2>
__device__ __forceinline__ void wave_bitonic_sort(uint64_t (&key)[E], int lane) {
  if constexpr (K <= 64 * E) {
    merge64<E, K, K / 2>(key, lane);
    wave_bitonic_sort<E, 2 * K>(key, lane);
  }
}

// Block masses in fixed point: p * 2^31 rounded to an integer (p <= 1, and the masses of
// a row add up to about 2^31, so every partial sum fits 32 bits). Integer sums do not
// depend on the order of the additions, so every pass (sorted scan, bucket histogram)
// finds the same mass ranked ahead of a block, and C * 2^-31 < tau holds exactly when
// C < ceil(tau * 2^31) (the host's mass_threshold).
constexpr float kMassScale = 2147483648.0f;
__device__ __forceinline__ uint32_t mass_units(float p) { return __float2uint_rn(p * kMassScale); }

// Exclusive prefix, across the wave, of per-lane totals (exact).
__device__ __forceinline__ uint32_t wave_exclusive_sum_u32(uint32_t tot, int lane) {
  uint32_t incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, o);
    if (lane >= o) incl += y;
  }
  return incl - tot;
}

// Exact level pass, one wave per query-block row: a sort of the row's 64-bit (score,
// index) keys, a scan of the integer masses in rank order and the threshold compares (the
// ranked rule: the sorted position against K_l), writing the cumulative mass when asked.
// It runs over the rows flagged in need_exact by block_level_sel_kernel (rows of more
// than 512 blocks it could not settle; it sorts shorter ones itself), or over every row
// (need_exact null) when the cumulative mass is asked for.
template <int E, bool RANKED>
__global__ void __launch_bounds__(kMaskThreads)
block_level_kernel(const float* __restrict__ z, int8_t* __restrict__ level_map, float* __restrict__ cmass,
                   uint8_t* __restrict__ need_exact, int N, int nkb, int zstride, int nrows, int L,
                   int n_dense_prefix, uint32_t T0, uint32_t T1, uint32_t T2, uint32_t T3, RankFractions frac,
                   int q_block, int nqb, int causal) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * (kMaskThreads / 64) + wave;
  if (row >= nrows) return;                 // whole wave; no barrier in this kernel
  if (need_exact != nullptr && need_exact[row] == 0) return;
  // Causal use: the row ranks only the nvis blocks that hold a token at or before its
  // query block's last row; blocks from dfirst on reach the block's own rows and stay at
  // full resolution (a pooled key would mix in later tokens); later blocks are pruned.
  int nvis = nkb, dfirst = nkb;
  if (causal) {
    const int r0 = (row % nqb) * q_block;
    nvis = (min(N, r0 + q_block) - 1) / 64 + 1;
    dfirst = r0 / 64;
  }
  // the row's scores only (64 E may exceed the row stride; groups of 4 stay in the padded row)
  const float* zr = z + (int64_t)row * zstride + E * lane;
  float zz[E];
  if constexpr (E >= 4) {
#pragma unroll
    for (int c = 0; c < E / 4; ++c) {
      const float4 f = E * lane + 4 * c < nkb ? reinterpret_cast<const float4*>(zr)[c]
                                              : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      zz[4 * c] = f.x; zz[4 * c + 1] = f.y; zz[4 * c + 2] = f.z; zz[4 * c + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int r = 0; r < E; ++r) zz[r] = E * lane + r < nkb ? zr[r] : -INFINITY;
  }

  // ---- softmax statistics of the row (the ranked rule needs them only for cmass)
  const bool want_mass = !RANKED || cmass != nullptr;
  float mx = -INFINITY, inv_s = 0.f;
  if (want_mass) {
#pragma unroll
    for (int r = 0; r < E; ++r)
      if (E * lane + r < nvis) mx = fmaxf(mx, zz[r]);
    mx = wave_max(mx);
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < E; ++r)
      if (E * lane + r < nvis) s += __expf(zz[r] - mx);
    s = wave_sum(s);
    inv_s = 1.0f / s;
  }
  const uint32_t T[4] = {T0, T1, T2, T3};     // mass thresholds in mass units
  // ranked rule: K_l = floor(f_l * nvis) in double precision (the host's expression)
  int K[4];
#pragma unroll
  for (int l = 0; l < 4; ++l) K[l] = RANKED && l < L ? (int)floor(frac.f[l] * (double)nvis) : 0;
  int8_t* lrow = level_map + (int64_t)row * nkb;
  float* crow = cmass ? cmass + (int64_t)row * nkb : nullptr;
  if (nvis < nkb) {   // causal: blocks after the query block are pruned; all the mass lies ahead
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int j = E * lane + r;
      if (j >= nvis && j < nkb) {
        lrow[j] = -1;
        if (crow) crow[j] = 1.f;
      }
    }
  }

  // ---- exact path: sort (score, index) keys
  uint64_t key[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int j = E * lane + r;
    key[r] = j < nvis ? rank_key(zz[r], j) : ~0ull;   // padding (and invisible blocks) sort last
  }
  wave_bitonic_sort<E>(key, lane);
  uint32_t u[E], tot = 0u;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const uint32_t j = (uint32_t)key[r];
    u[r] = want_mass && j < (uint32_t)nvis ? mass_units(__expf(key_score(key[r]) - mx) * inv_s) : 0u;
    tot += u[r];
  }
  uint32_t run = want_mass ? wave_exclusive_sum_u32(tot, lane) : 0u;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const uint32_t j = (uint32_t)key[r];
    const uint32_t C = run;
    run += u[r];
    if (j < (uint32_t)nvis) {
      int lev = -1;
#pragma unroll
      for (int l = kMaxLevels - 1; l >= 0; --l) {
        const bool in = RANKED ? E * lane + r < K[l] : C < T[l];   // sorted position = rank
        if (l < L && in) lev = l;
      }
      if (64 * (int)j < n_dense_prefix || (int)j >= dfirst) lev = 0;
      lrow[j] = (int8_t)lev;
      if (crow) crow[j] = (float)C * (1.0f / kMassScale);
    }
  }
}

// Levels of one row from a sort of its (score, index) keys: the exact pass of
// block_level_kernel for a row the bucket pass could not settle. A block's weight is its
// integer mass (threshold rule) or 1 (ranked rule: the weight ranked ahead is the rank).
template <int E, bool RANKED>
__device__ __forceinline__ void exact_row_levels(const float (&zz)[E], float mx, float inv_s, int nvis,
                                                 int dfirst, int8_t* lrow, const uint32_t (&T)[kMaxLevels],
                                                 int L, int n_dense_prefix, int lane) {
  uint64_t key[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int j = E * lane + r;
    key[r] = j < nvis ? rank_key(zz[r], j) : ~0ull;
  }
  wave_bitonic_sort<E>(key, lane);
  uint32_t u[E], tot = 0u;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const uint32_t j = (uint32_t)key[r];
    u[r] = j < (uint32_t)nvis ? (RANKED ? 1u : mass_units(__expf(key_score(key[r]) - mx) * inv_s)) : 0u;
    tot += u[r];
  }
  uint32_t run = wave_exclusive_sum_u32(tot, lane);
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const uint32_t j = (uint32_t)key[r];
    const uint32_t C = run;
    run += u[r];
    if (j < (uint32_t)nvis) {
      int lev = -1;
#pragma unroll
      for (int l = kMaxLevels - 1; l >= 0; --l)
        if (l < L && C < T[l]) lev = l;
      if (64 * (int)j < n_dense_prefix || (int)j >= dfirst) lev = 0;
      lrow[j] = (int8_t)lev;
    }
  }
}

// Fast level pass (no cumulative mass asked), without a sort. The visible scores go into
// NB buckets by their distance below the row's top score (bucket 0 holds the top), with a
// histogram of the blocks' weights: their integer masses (threshold rule), or 1 (ranked
// rule, where the weight ranked ahead of a block is its rank). Bucket order follows the
// rank order, so the weight ranked ahead of a block of bucket b is F(b), the weight of the
// buckets before it, plus that of the blocks of bucket b ranked ahead of it; for level l
// (T_l: the mass threshold in mass units, or K_l blocks) the last bucket with F(b) < T_l
// holds the cut: every block of an earlier bucket takes level l or a finer one and no
// block of a later bucket does. Only the blocks of those (at most four) buckets are ranked
// exactly: their (score, index) keys are sorted across the wave, one per lane, and their
// weights scanned in that order. A row whose cut buckets hold more than 64 blocks (many
// equal scores) takes the exact pass's sort of the whole row: here for rows of up to 512
// blocks, in block_level_kernel's exact pass (flagged in need_exact) for longer ones,
// whose sort would weigh on every row of this kernel. The weights are the exact pass's
// integers, so all ways give the same levels.
template <int E, bool RANKED>
__global__ void __launch_bounds__(kMaskThreads)
block_level_sel_kernel(const float* __restrict__ z, int8_t* __restrict__ level_map,
                       uint8_t* __restrict__ need_exact, int N, int nkb, int nrows, int L, int n_dense_prefix,
                       uint32_t T0, uint32_t T1, uint32_t T2, uint32_t T3, RankFractions frac, int q_block,
                       int nqb, int causal) {
  constexpr int NP = 64 * E;
  constexpr int NB = 512;                   // buckets
  constexpr int BPL = NB / 64;              // buckets per lane
  __shared__ __align__(16) uint32_t hist[kMaskThreads / 64][NB];
  __shared__ uint64_t cbuf[kMaskThreads / 64][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * (kMaskThreads / 64) + wave;
  if (row >= nrows) return;                 // whole wave; wave-private LDS, no barrier
  int nvis = nkb, dfirst = nkb;
  if (causal) {
    const int r0 = (row % nqb) * q_block;
    nvis = (min(N, r0 + q_block) - 1) / 64 + 1;
    dfirst = r0 / 64;
  }
  const float* zr = z + (int64_t)row * NP + E * lane;
  float zz[E];
  if constexpr (E >= 4) {
#pragma unroll
    for (int c = 0; c < E / 4; ++c) {   // the row's scores only (groups of 4 stay in the padded row)
      const float4 f = E * lane + 4 * c < nkb ? reinterpret_cast<const float4*>(zr)[c]
                                              : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      zz[4 * c] = f.x; zz[4 * c + 1] = f.y; zz[4 * c + 2] = f.z; zz[4 * c + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int r = 0; r < E; ++r) zz[r] = E * lane + r < nkb ? zr[r] : -INFINITY;
  }
  int8_t* lrow = level_map + (int64_t)row * nkb;
  // softmax statistics in block_level_kernel's grouping, so every mass is the same float
  float mx = -INFINITY, zmin = INFINITY;
  const bool full = nvis == nkb;            // no causal cut in this row (the same in every lane)
  if (full) {
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const bool in = E * lane + r < nkb;
      mx = fmaxf(mx, in ? zz[r] : -INFINITY);
      zmin = fminf(zmin, in ? zz[r] : INFINITY);
    }
  } else {
#pragma unroll
    for (int r = 0; r < E; ++r) {
      const int j = E * lane + r;
      if (j < nvis) {
        mx = fmaxf(mx, zz[r]);
        zmin = fminf(zmin, zz[r]);
      } else if (j < nkb) {
        lrow[j] = -1;                       // causal: blocks after the query block
      }
    }
  }
  mx = wave_max(mx);
  zmin = -wave_max(-zmin);
  float inv_s = 0.f;
  if constexpr (!RANKED) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < E; ++r)
      if (E * lane + r < nvis) s += __expf(zz[r] - mx);
    s = wave_sum(s);
    inv_s = 1.0f / s;
  }
  const float bscale = mx > zmin ? (float)NB / (mx - zmin) : 0.f;
  auto bucket_of = [&](float zv) { return min(NB - 1, (int)((mx - zv) * bscale)); };
  // a visible block's weight: its integer mass, or 1 (ranked rule)
  auto weight_of = [&](float zv) { return RANKED ? 1u : mass_units(__expf(zv - mx) * inv_s); };

  // ---- weight histogram over the buckets
  uint32_t* h = hist[wave];
#pragma unroll
  for (int c = 0; c < BPL / 4; ++c) reinterpret_cast<uint4*>(h + BPL * lane)[c] = make_uint4(0u, 0u, 0u, 0u);
  __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  int bk[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const bool vis = E * lane + r < nvis;
    bk[r] = vis ? bucket_of(zz[r]) : NB;
    const uint32_t u = vis ? weight_of(zz[r]) : 0u;
    if (u != 0u) atomicAdd(&hist[wave][bk[r]], u);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  // F of this lane's buckets BPL*lane + k: an exclusive prefix in bucket order
  uint32_t F[BPL];
  {
    uint32_t hv[BPL];
#pragma unroll
    for (int c = 0; c < BPL / 4; ++c) {
      const uint4 v4 = reinterpret_cast<const uint4*>(h + BPL * lane)[c];
      hv[4 * c] = v4.x; hv[4 * c + 1] = v4.y; hv[4 * c + 2] = v4.z; hv[4 * c + 3] = v4.w;
    }
    uint32_t tot = 0u;
#pragma unroll
    for (int k = 0; k < BPL; ++k) {
      F[k] = tot;
      tot += hv[k];
    }
    const uint32_t base = wave_exclusive_sum_u32(tot, lane);
#pragma unroll
    for (int k = 0; k < BPL; ++k) F[k] += base;
  }
  uint32_t T[kMaxLevels] = {T0, T1, T2, T3};
  if constexpr (RANKED) {   // K_l = floor(f_l * nvis) in double precision (the host's expression)
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l) T[l] = l < L ? (uint32_t)floor(frac.f[l] * (double)nvis) : 0u;
  }
  // cut bucket of each threshold: the last bucket with F < T (F is nondecreasing)
  int dcut[kMaxLevels];
  uint32_t Fcut[kMaxLevels];
#pragma unroll
  for (int l = 0; l < kMaxLevels; ++l) {
    dcut[l] = -1;
    Fcut[l] = 0u;
    if (l < L && T[l] > 0u) {
      int D = 0;
#pragma unroll
      for (int k = 0; k < BPL; ++k) D += __popcll(__ballot(F[k] < T[l]));
      dcut[l] = D - 1;                      // >= 0: F(0) = 0 < T
      uint32_t v = F[0];
#pragma unroll
      for (int k = 1; k < BPL; ++k)
        if (dcut[l] % BPL == k) v = F[k];
      Fcut[l] = (uint32_t)__builtin_amdgcn_readlane((int)v, dcut[l] / BPL);
    }
  }

  // ---- the blocks of the cut buckets, ranked exactly (one per lane)
  int ncand = 0;
  uint64_t* cb = cbuf[wave];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    bool c = false;
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l) c |= bk[r] == dcut[l];
    const uint64_t m = __ballot(c);
    const int pos = ncand + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (c && pos < 64) cb[pos] = rank_key(zz[r], E * lane + r);
    ncand += __popcll(m);
  }
  const bool fail = ncand > 64;
  uint64_t kap[kMaxLevels];                 // key of the last block taking level l or finer
  bool has[kMaxLevels];
  if (!fail) {
    if (lane >= ncand) cb[lane] = ~0ull;
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    uint64_t ck[1] = {cb[lane]};
    wave_bitonic_sort<1>(ck, lane);
    const bool real = ck[0] != ~0ull;
    const float zc = key_score(ck[0]);
    const uint32_t uc = real ? weight_of(zc) : 0u;
    const int bc = real ? bucket_of(zc) : NB;
    const uint32_t G = wave_exclusive_sum_u32(uc, lane);
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l) {
      has[l] = dcut[l] >= 0;
      kap[l] = ~0ull;                       // an empty cut bucket (the last one): every block is in
      if (!has[l]) continue;
      const uint64_t mb = __ballot(bc == dcut[l]);
      if (mb == 0) continue;
      const int first = __builtin_ctzll(mb);
      const uint32_t start = (uint32_t)__builtin_amdgcn_readlane((int)G, first);
      const uint32_t C = Fcut[l] + (G - start);
      const uint64_t mi = __ballot(bc == dcut[l] && C < T[l]);   // never empty: the first has C = F < T
      const int last = 63 - __builtin_clzll(mi);
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)ck[0], last);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(ck[0] >> 32), last);
      kap[l] = ((uint64_t)hi << 32) | lo;
    }
    auto level_at = [&](int r) {
      const int j = E * lane + r;
      const uint64_t kr = rank_key(zz[r], j);
      int lev = -1;
#pragma unroll
      for (int l = kMaxLevels - 1; l >= 0; --l)
        if (has[l] && kr <= kap[l]) lev = l;
      if (64 * j < n_dense_prefix || j >= dfirst) lev = 0;
      return lev;
    };
    bool done = false;
    if constexpr (E % 4 == 0) {
      // every group of four whole; the map itself is 16-byte aligned (the library checks it),
      // so each group's 4-byte store is aligned
      if (full && (nkb & 3) == 0) {
#pragma unroll
        for (int c = 0; c < E / 4; ++c) {
          const int j0 = E * lane + 4 * c;
          if (j0 < nkb) {
            const uint32_t w4 = (uint32_t)(level_at(4 * c) & 0xff) | (uint32_t)(level_at(4 * c + 1) & 0xff) << 8 |
                                (uint32_t)(level_at(4 * c + 2) & 0xff) << 16 |
                                (uint32_t)(level_at(4 * c + 3) & 0xff) << 24;
            *reinterpret_cast<uint32_t*>(lrow + j0) = w4;
          }
        }
        done = true;
      }
    }
    if (!done) {
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const int j = E * lane + r;
        if (j < nvis) lrow[j] = (int8_t)level_at(r);
      }
    }
  }
  if constexpr (E <= 8) {
    if (fail) exact_row_levels<E, RANKED>(zz, mx, inv_s, nvis, dfirst, lrow, T, L, n_dense_prefix, lane);
  } else {
    if (lane == 0) need_exact[row] = fail ? 1 : 0;
  }
}

// C * 2^-31 < tau  <=>  C < ceil(tau * 2^31) for an integer mass C (tau * 2^31 is exact in
// double: tau is a float)
static uint32_t mass_threshold(float tau) {
  const double t = std::ceil((double)tau * 2147483648.0);
  return t <= 0.0 ? 0u : t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
}

// E: scores per lane of the bucket pass (the score-row stride / 64); the exact pass sorts
// 64 EP keys, EP the power of two >= E.
template <int E, bool RANKED>
static void launch_level_r(const MaskArgs& a, int nrows, hipStream_t stream) {
  constexpr int EP = E <= 8 ? E : E <= 16 ? 16 : 32;
  RankFractions frac;
  for (int l = 0; l < kMaxLevels; ++l) frac.f[l] = a.frac[l];
  uint32_t T[kMaxLevels];
  for (int l = 0; l < kMaxLevels; ++l) T[l] = mass_threshold(a.tau[l]);
  const dim3 grid((nrows + 3) / 4);
  const int causal = a.causal ? 1 : 0;
  uint8_t* flagged = nullptr;               // exact pass over these rows only (null: every row)
  if (a.cmass == nullptr) {
    hipLaunchKernelGGL((block_level_sel_kernel<E, RANKED>), grid, dim3(kMaskThreads), 0, stream, a.z,
                       a.level_map, a.need_exact, a.N, a.nkb, nrows, a.L, a.n_dense_prefix, T[0], T[1], T[2],
                       T[3], frac, a.q_block, a.nqb, causal);
    if constexpr (E <= 8) return;            // unsettled rows were sorted in the kernel
    flagged = a.need_exact;
  }
  hipLaunchKernelGGL((block_level_kernel<EP, RANKED>), grid, dim3(kMaskThreads), 0, stream, a.z, a.level_map,
                     a.cmass, flagged, a.N, a.nkb, mask_score_stride(a.nkb), nrows, a.L, a.n_dense_prefix, T[0],
                     T[1], T[2], T[3], frac, a.q_block, a.nqb, causal);
}

template <int E>
static void launch_level_e(const MaskArgs& a, int nrows, hipStream_t stream) {
  if (a.ranked) launch_level_r<E, true>(a, nrows, stream);
  else launch_level_r<E, false>(a, nrows, stream);
}

template <typename T, int D>
static hipError_t launch_mask_t(const MaskArgs& a, hipStream_t stream) {
  const int zstride = mask_score_stride(a.nkb);
  hipError_t e;
  if (a.nkb > 512) {
    hipLaunchKernelGGL((qblock_score_kernel<T, D>), dim3((a.nqb + 15) / 16, a.B * a.H), dim3(kMaskThreads), 0,
                       stream, static_cast<const T*>(a.q), a.k_bar, a.z, a.N, a.H, a.H_kv, a.q_block, a.nqb, a.nkb,
                       zstride, a.scale);
  } else {
    constexpr int QB = 2;
    hipLaunchKernelGGL((qblock_mean_kernel<T, D, QB>), dim3((a.nqb + QB - 1) / QB, a.B * a.H), dim3(kMaskThreads),
                       0, stream, static_cast<const T*>(a.q), a.qbar, a.N, a.q_block, a.nqb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ktiles = (a.nkb + 31) / 32;
    dim3 sgrid((ktiles + kScoreWaves - 1) / kScoreWaves, (a.nqb + 31) / 32, a.B * a.H);
    hipLaunchKernelGGL((block_score_kernel<D>), sgrid, dim3(64 * kScoreWaves), 0, stream, a.qbar, a.k_bar, a.z,
                       a.N, a.H, a.H_kv, a.nqb, a.nkb, zstride, a.scale);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = a.B * a.H * a.nqb;
  switch (zstride) {
    case 64: launch_level_e<1>(a, nrows, stream); break;
    case 128: launch_level_e<2>(a, nrows, stream); break;
    case 256: launch_level_e<4>(a, nrows, stream); break;
    case 512: launch_level_e<8>(a, nrows, stream); break;
    case 768: launch_level_e<12>(a, nrows, stream); break;
    case 1024: launch_level_e<16>(a, nrows, stream); break;
    case 1280: launch_level_e<20>(a, nrows, stream); break;
    case 1536: launch_level_e<24>(a, nrows, stream); break;
    case 1792: launch_level_e<28>(a, nrows, stream); break;
    case 2048: launch_level_e<32>(a, nrows, stream); break;
    default: return hipErrorInvalidValue;   // nkb above the supported maximum (checked by the ABI layer)
  }
  return hipGetLastError();
}

hipError_t launch_mask(const MaskArgs& a, hipStream_t stream) {
  if (a.bf16) return a.d == 128 ? launch_mask_t<bf16_t, 128>(a, stream) : launch_mask_t<bf16_t, 64>(a, stream);
  return a.d == 128 ? launch_mask_t<float, 128>(a, stream) : launch_mask_t<float, 64>(a, stream);
}

}  // namespace psa
