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
// Three kernels:
//  * qblock_mean_kernel streams Q once (HBM-bound: every load of a thread is in
//    flight at once, 16-byte loads, whole rows per wave) and writes the float32
//    mean query of each query block to the workspace.
//  * block_score_kernel: z = scale * qbar kbar^T + ln n_j per head on the float32
//    matrix cores (v_mfma_f32_32x32x2_f32), one 32 x 32 tile per wave, into a
//    workspace row of n_pad floats per query block.
//  * block_level_kernel: one wave per query-block row: softmax of the row, a
//    bitonic sort of score keys held in registers (n_pad / 64 per lane; partners
//    in other lanes come through cross-lane shuffles, so no LDS and no workgroup
//    barrier), a wave-wide exclusive scan of the masses in rank order, the
//    threshold compares and the int8 level writes. 32-bit keys settle a row unless
//    a cut splits a group of equal scores; such rows, and calls that want the
//    cumulative mass, sort 64-bit (score, index) keys (for rows of more than 512
//    blocks in a second kernel over the rows the first one flags).
//    Its ranked form (the quantile rule the top168.com ablation compares with
//    thresholds; fixed shares of the score-ranked blocks per level: skillmd.com,
//    "Level assignment") gives the block at rank r the lowest level l with
//    r < K_l for host-computed cumulative counts K_l, so it needs the sort but
//    neither the softmax nor the scan.
#include "psa_device.h"
#include "psa_launch.h"

namespace psa {

constexpr int kMaskThreads = 256;

template <typename T, int D>
__global__ void __launch_bounds__(kMaskThreads)
qblock_mean_kernel(const T* __restrict__ q, float* __restrict__ qbar, int N, int q_block, int nqb) {
  constexpr int E = io_traits<T>::per16;
  constexpr int CPR = D / E;                // 16-byte chunks per row
  constexpr int G = kMaskThreads / CPR;     // row groups
  constexpr int MAXR = 128 / G;             // rows per thread at the largest query block
  __shared__ float red[G][D];
  const int t = threadIdx.x;
  const int chunk = t % CPR, g = t / CPR;
  const int i = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int r0 = i * q_block;
  const int m = min(q_block, N - r0);
  const T* src = q + (bh * N + r0) * (int64_t)D + chunk * E;

  // rows g, g+G, g+2G, ...: all loads issued before any is used
  U128 raw[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    const int row = g + r * G;
    raw[r] = row < m ? ld128(src + (int64_t)row * D) : U128{{0u, 0u, 0u, 0u}};
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    float x[E];
    unpack16<T>(raw[r], x);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += x[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[g][chunk * E + e] = acc[e];
  __syncthreads();
  if (t < D) {
    float s = 0.f;
#pragma unroll 8
    for (int gg = 0; gg < G; ++gg) s += red[gg][t];
    qbar[(bh * nqb + i) * D + t] = s / (float)m;
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
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const int j0 = kt * 32 + 8 * g4 + 4 * half;
    float out[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int j = j0 + x;
      const float lnn = logf((float)min(64, N - 64 * j));
      out[x] = fmaf(scale, acc[4 * g4 + x], lnn);
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

// 32-bit keys: the order word alone (no index). Exchanges are v_med3_u32 against 0
// (minimum) or ~0 (maximum), one VALU op per element of a cross-lane stage.
__device__ __forceinline__ uint32_t med3u(uint32_t a, uint32_t b, uint32_t c) {
  return min(max(a, b), max(min(a, b), c));
}
__device__ __forceinline__ uint32_t score_key(float z) {
  const uint32_t u = __float_as_uint(z + 0.0f);
  return (u & 0x80000000u) ? u : (~u & 0x7fffffffu);
}
__device__ __forceinline__ float key32_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? key : (~key & 0x7fffffffu));
}
constexpr uint32_t kPadKey32 = 0xFFFFFFFFu;   // above every finite score's key

template <int E, int M>
__device__ __forceinline__ void stage_cross32(uint32_t (&key)[E], int lane, int k) {
  const bool upper = (lane & M) != 0;
  const bool asc = ((E * lane) & k) == 0;
  const uint32_t c = (upper == asc) ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int r = 0; r < E; ++r) key[r] = med3u(key[r], xor_lane<M>(key[r], lane), c);
}
template <int E, int J>
__device__ __forceinline__ void stage_in32(uint32_t (&key)[E], int lane, int k) {
#pragma unroll
  for (int r = 0; r < E; ++r) {
    if (r & J) continue;
    const uint32_t clo = ((E * lane + r) & k) == 0 ? 0u : 0xFFFFFFFFu;
    const uint32_t a = key[r], b = key[r + J];
    key[r] = med3u(a, b, clo);
    key[r + J] = med3u(a, b, ~clo);
  }
}
template <int E, int K, int J>
__device__ __forceinline__ void merge32(uint32_t (&key)[E], int lane) {
  if constexpr (J > 0) {
    if constexpr (J >= E) stage_cross32<E, J / E>(key, lane, K);
    else stage_in32<E, J>(key, lane, K);
    merge32<E, K, J / 2>(key, lane);
  }
}
template <int E, int K = 2>
__device__ __forceinline__ void wave_bitonic_sort32(uint32_t (&key)[E], int lane) {
  if constexpr (K <= 64 * E) {
    merge32<E, K, K / 2>(key, lane);
    wave_bitonic_sort32<E, 2 * K>(key, lane);
  }
}

// Exclusive prefix, across the wave, of per-lane totals.
__device__ __forceinline__ float wave_exclusive_sum(float tot, int lane) {
  float incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  return incl - tot;
}

// One wave per query-block row. Fast path (no cmass): sort the 32-bit score keys; the
// mass ranked ahead of a block is a prefix of the sorted masses, so level l takes the
// blocks whose key is at most the key at the last sorted position with prefix mass
// below tau_l, unless that key continues past the cut (equal scores, which the rule
// orders by block index). Exact path, for such rows and for calls that want the
// cumulative mass itself: sort 64-bit (score, index) keys. Both paths sum the same
// masses in the same order, so they give the same levels. MODE 0 runs both in one
// kernel (the exact path only for rows the fast one cannot settle); for long rows the
// two are separate kernels, which keeps the fast one small enough for several waves
// per SIMD: MODE 1 is the fast path, flagging such rows in need_exact, MODE 2 the exact
// path over the flagged rows (every row when need_exact is null).
template <int E, bool RANKED, int MODE>
__global__ void __launch_bounds__(kMaskThreads)
block_level_kernel(const float* __restrict__ z, int8_t* __restrict__ level_map, float* __restrict__ cmass,
                   uint8_t* __restrict__ need_exact, int N, int nkb, int nrows, int L, int n_dense_prefix,
                   float tau0, float tau1, float tau2, float tau3, RankFractions frac,
                   int q_block, int nqb, int causal) {
  constexpr int NP = 64 * E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * (kMaskThreads / 64) + wave;
  if (row >= nrows) return;                 // whole wave; no barrier in this kernel
  if constexpr (MODE == 2) {
    if (need_exact != nullptr && need_exact[row] == 0) return;
  }
  // Causal use: the row ranks only the nvis blocks that hold a token at or before its
  // query block's last row; blocks from dfirst on reach the block's own rows and stay at
  // full resolution (a pooled key would mix in later tokens); later blocks are pruned.
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
    for (int c = 0; c < E / 4; ++c) {
      const float4 f = reinterpret_cast<const float4*>(zr)[c];
      zz[4 * c] = f.x; zz[4 * c + 1] = f.y; zz[4 * c + 2] = f.z; zz[4 * c + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int r = 0; r < E; ++r) zz[r] = zr[r];
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
  const float tau[4] = {tau0, tau1, tau2, tau3};
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

  if (MODE == 1 || (MODE == 0 && cmass == nullptr)) {
    uint32_t orig[E], key[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
      orig[r] = E * lane + r < nvis ? score_key(zz[r]) : kPadKey32;
      key[r] = orig[r];
    }
    wave_bitonic_sort32<E>(key, lane);
    // equal scores anywhere in the row (neighbours in sorted order)?
    bool tie = false;
#pragma unroll
    for (int r = 0; r + 1 < E; ++r) tie |= key[r] == key[r + 1] && key[r] != kPadKey32;
    const uint32_t next_first = (uint32_t)__shfl_down((int)key[0], 1);
    tie |= lane < 63 && key[E - 1] == next_first && key[E - 1] != kPadKey32;
    const bool any_tie = __ballot(tie) != 0;
    // cnt[l]: how many blocks, in rank order, take level l or a finer one. Blocks with
    // equal scores have equal masses, so the prefix sums along the sorted keys do not
    // depend on how the sort ordered them among themselves.
    int cnt[kMaxLevels] = {0, 0, 0, 0};
    if constexpr (RANKED) {
#pragma unroll
      for (int l = 0; l < kMaxLevels; ++l) cnt[l] = K[l];
    } else {
      float p[E], tot = 0.f;
#pragma unroll
      for (int r = 0; r < E; ++r) {
        p[r] = key[r] != kPadKey32 ? __expf(key32_score(key[r]) - mx) * inv_s : 0.f;
        tot += p[r];
      }
      float run = wave_exclusive_sum(tot, lane);
      int lc[kMaxLevels] = {0, 0, 0, 0};   // this lane's blocks with C below each threshold
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const float C = run;
        run += p[r];
        const bool real = key[r] != kPadKey32;
#pragma unroll
        for (int l = 0; l < kMaxLevels; ++l) lc[l] += real && C < tau[l] ? 1 : 0;
      }
#pragma unroll
      for (int l = 0; l < kMaxLevels; ++l) cnt[l] = (int)wave_sum((float)lc[l]);   // exact: counts < 2^24
    }
    // cut[l]: key at sorted position cnt[l] - 1, the last block level l (or a finer one)
    // takes. Equal scores matter only where more than cnt[l] keys are <= cut[l], i.e. a
    // key after the cut equals it: then the index order decides which of them are in,
    // and the row takes the exact path.
    uint32_t cut[kMaxLevels];
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l) {
      const int pos = cnt[l] - 1;
      uint32_t v = key[0];
#pragma unroll
      for (int r = 1; r < E; ++r)
        if (pos >= 0 && pos % E == r) v = key[r];
      cut[l] = pos >= 0 ? (uint32_t)__builtin_amdgcn_readlane((int)v, pos / E) : 0u;
    }
    bool split = false;
    if (any_tie) {
      int le[kMaxLevels] = {0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < E; ++r)
#pragma unroll
        for (int l = 0; l < kMaxLevels; ++l) le[l] += orig[r] <= cut[l] ? 1 : 0;
#pragma unroll
      for (int l = 0; l < kMaxLevels; ++l)
        if (l < L && cnt[l] > 0) split |= (int)wave_sum((float)le[l]) > cnt[l];   // exact: counts < 2^24
    }
    if (MODE == 1 && lane == 0) need_exact[row] = split ? 1 : 0;
    if (!split) {
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const int j = E * lane + r;
        if (j < nvis) {
          int lev = -1;
#pragma unroll
          for (int l = kMaxLevels - 1; l >= 0; --l)
            if (l < L && cnt[l] > 0 && orig[r] <= cut[l]) lev = l;
          if (64 * j < n_dense_prefix || j >= dfirst) lev = 0;
          lrow[j] = (int8_t)lev;
        }
      }
      return;
    }
    if constexpr (MODE == 1) return;
  }

  // ---- exact path: sort (score, index) keys
  uint64_t key[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int j = E * lane + r;
    key[r] = j < nvis ? rank_key(zz[r], j) : ~0ull;   // padding (and invisible blocks) sort last
  }
  wave_bitonic_sort<E>(key, lane);
  float p[E], tot = 0.f;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const uint32_t j = (uint32_t)key[r];
    p[r] = want_mass && j < (uint32_t)nvis ? __expf(key_score(key[r]) - mx) * inv_s : 0.f;
    tot += p[r];
  }
  float run = want_mass ? wave_exclusive_sum(tot, lane) : 0.f;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const uint32_t j = (uint32_t)key[r];
    const float C = run;
    run += p[r];
    if (j < (uint32_t)nvis) {
      int lev = -1;
#pragma unroll
      for (int l = kMaxLevels - 1; l >= 0; --l) {
        const bool in = RANKED ? E * lane + r < K[l] : C < tau[l];   // sorted position = rank
        if (l < L && in) lev = l;
      }
      if (64 * (int)j < n_dense_prefix || (int)j >= dfirst) lev = 0;
      lrow[j] = (int8_t)lev;
      if (crow) crow[j] = C;
    }
  }
}

// Padded score-row length: the smallest power of two >= max(nkb, 64).
int mask_score_stride(int nkb) {
  int n = 64;
  while (n < nkb) n <<= 1;
  return n;
}

template <int E, bool RANKED>
static void launch_level_r(const MaskArgs& a, int nrows, hipStream_t stream) {
  RankFractions frac;
  for (int l = 0; l < kMaxLevels; ++l) frac.f[l] = a.frac[l];
  const dim3 grid((nrows + 3) / 4);
  const int causal = a.causal ? 1 : 0;
  if constexpr (E <= 8) {
    hipLaunchKernelGGL((block_level_kernel<E, RANKED, 0>), grid, dim3(kMaskThreads), 0, stream, a.z, a.level_map,
                       a.cmass, nullptr, a.N, a.nkb, nrows, a.L, a.n_dense_prefix, a.tau[0], a.tau[1], a.tau[2],
                       a.tau[3], frac, a.q_block, a.nqb, causal);
  } else {
    // without cmass: the fast pass, then the exact pass over the rows it flagged
    if (a.cmass == nullptr)
      hipLaunchKernelGGL((block_level_kernel<E, RANKED, 1>), grid, dim3(kMaskThreads), 0, stream, a.z,
                         a.level_map, a.cmass, a.need_exact, a.N, a.nkb, nrows, a.L, a.n_dense_prefix, a.tau[0],
                         a.tau[1], a.tau[2], a.tau[3], frac, a.q_block, a.nqb, causal);
    hipLaunchKernelGGL((block_level_kernel<E, RANKED, 2>), grid, dim3(kMaskThreads), 0, stream, a.z, a.level_map,
                       a.cmass, a.cmass == nullptr ? a.need_exact : nullptr, a.N, a.nkb, nrows, a.L,
                       a.n_dense_prefix, a.tau[0], a.tau[1], a.tau[2], a.tau[3], frac, a.q_block, a.nqb, causal);
  }
}

template <int E>
static void launch_level_e(const MaskArgs& a, int nrows, hipStream_t stream) {
  if (a.ranked) launch_level_r<E, true>(a, nrows, stream);
  else launch_level_r<E, false>(a, nrows, stream);
}

template <typename T, int D>
static hipError_t launch_mask_t(const MaskArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((qblock_mean_kernel<T, D>), dim3(a.nqb, a.B * a.H), dim3(kMaskThreads), 0, stream,
                     static_cast<const T*>(a.q), a.qbar, a.N, a.q_block, a.nqb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int zstride = mask_score_stride(a.nkb);
  const int ktiles = (a.nkb + 31) / 32;
  dim3 sgrid((ktiles + kScoreWaves - 1) / kScoreWaves, (a.nqb + 31) / 32, a.B * a.H);
  hipLaunchKernelGGL((block_score_kernel<D>), sgrid, dim3(64 * kScoreWaves), 0, stream, a.qbar, a.k_bar, a.z, a.N,
                     a.H, a.H_kv, a.nqb, a.nkb, zstride, a.scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nrows = a.B * a.H * a.nqb;
  switch (zstride) {
    case 64: launch_level_e<1>(a, nrows, stream); break;
    case 128: launch_level_e<2>(a, nrows, stream); break;
    case 256: launch_level_e<4>(a, nrows, stream); break;
    case 512: launch_level_e<8>(a, nrows, stream); break;
    case 1024: launch_level_e<16>(a, nrows, stream); break;
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
