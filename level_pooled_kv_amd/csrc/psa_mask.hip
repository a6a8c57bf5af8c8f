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
//    bitonic sort of (score, index) keys held in registers (n_pad / 64 per lane;
//    partners in other lanes come through cross-lane shuffles, so no LDS and no
//    workgroup barrier), a wave-wide exclusive scan of the masses in rank order,
//    the threshold compares and the int8 level writes.
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

// One 32 (KV blocks) x 32 (query blocks) tile of scores per wave. The contraction
// index is split between the two lane halves as [0, D/2) and [D/2, D) (the same
// split for both operands, so every product pairs matching elements).
template <int D>
__global__ void __launch_bounds__(kMaskThreads)
block_score_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar, float* __restrict__ z,
                   int N, int H, int H_kv, int nqb, int nkb, int zstride, float scale) {
  constexpr int S = D / 2;                  // MFMA steps (k = 2 each)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kt = blockIdx.x * (kMaskThreads / 64) + wave;
  if (kt * 32 >= nkb) return;               // whole wave; no barrier in this kernel
  const int qt = blockIdx.y;
  const int bh = blockIdx.z;
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / H_kv);
  const int l32 = lane & 31, half = lane >> 5;
  const int key = min(kt * 32 + l32, nkb - 1);
  const int qi = min(qt * 32 + l32, nqb - 1);
  const float4* ka = reinterpret_cast<const float4*>(kbar + ((int64_t)(b * H_kv + g) * nkb + key) * D + half * S);
  const float4* qa = reinterpret_cast<const float4*>(qbar + ((int64_t)bh * nqb + qi) * D + half * S);
  float4 kv[S / 4], qv[S / 4];
#pragma unroll
  for (int c = 0; c < S / 4; ++c) {
    kv[c] = ka[c];
    qv[c] = qa[c];
  }
  f32x16 acc;
#pragma unroll
  for (int x = 0; x < 16; ++x) acc[x] = 0.f;
#pragma unroll
  for (int c = 0; c < S / 4; ++c) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[c].x, qv[c].x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[c].y, qv[c].y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[c].z, qv[c].z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[c].w, qv[c].w, acc, 0, 0, 0);
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

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

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort, ascending, of the 64 E keys of one wave; element e = E * lane + r is
// key[r] of lane `lane`. Pairs at distance < E are in one lane; at distance >= E the
// partner is lane ^ (distance / E), same r.
template <int E>
__device__ __forceinline__ void wave_bitonic_sort(uint64_t (&key)[E], int lane) {
  constexpr int NP = 64 * E;
#pragma unroll
  for (int k = 2; k <= NP; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= E) {
        const int m = j / E;
        const bool upper = (lane & m) != 0;                 // holds the higher element of its pair
        const bool asc = ((E * lane) & k) == 0;             // k >= 2E: the same for every r
        const bool keep_max = upper == asc;
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const uint64_t y = shfl_xor_u64(key[r], m);
          const uint64_t x = key[r];
          const bool take = keep_max ? (y > x) : (y < x);
          key[r] = take ? y : x;
        }
      } else {
#pragma unroll
        for (int r = 0; r < E; ++r) {
          if (r & j) continue;
          const bool asc = ((E * lane + r) & k) == 0;
          const uint64_t a = key[r], c = key[r + j];
          const bool swap = (a > c) == asc;
          key[r] = swap ? c : a;
          key[r + j] = swap ? a : c;
        }
      }
    }
  }
}

template <int E>
__global__ void __launch_bounds__(kMaskThreads)
block_level_kernel(const float* __restrict__ z, int8_t* __restrict__ level_map, float* __restrict__ cmass,
                   int N, int nkb, int nrows, int L, int n_dense_prefix,
                   float tau0, float tau1, float tau2, float tau3) {
  constexpr int NP = 64 * E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * (kMaskThreads / 64) + wave;
  if (row >= nrows) return;                 // whole wave; no barrier in this kernel
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

  // ---- softmax statistics of the row
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < E; ++r)
    if (E * lane + r < nkb) mx = fmaxf(mx, zz[r]);
  mx = wave_max(mx);
  float s = 0.f;
  uint64_t key[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int j = E * lane + r;
    if (j < nkb) {
      s += expf(zz[r] - mx);
      key[r] = rank_key(zz[r], j);
    } else {
      key[r] = ~0ull;                        // padding sorts last
    }
  }
  s = wave_sum(s);
  const float inv_s = 1.0f / s;

  wave_bitonic_sort<E>(key, lane);

  // ---- exclusive prefix of the masses in rank order: lane-local, then across lanes
  float p[E], tot = 0.f;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const uint32_t j = (uint32_t)key[r];
    p[r] = j < (uint32_t)nkb ? expf(key_score(key[r]) - mx) * inv_s : 0.f;
    tot += p[r];
  }
  float incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  float run = incl - tot;

  const float tau[4] = {tau0, tau1, tau2, tau3};
  int8_t* lrow = level_map + (int64_t)row * nkb;
  float* crow = cmass ? cmass + (int64_t)row * nkb : nullptr;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const uint32_t j = (uint32_t)key[r];
    const float C = run;
    run += p[r];
    if (j < (uint32_t)nkb) {
      int lev = -1;
#pragma unroll
      for (int l = kMaxLevels - 1; l >= 0; --l)
        if (l < L && C < tau[l]) lev = l;
      if (64 * (int)j < n_dense_prefix) lev = 0;
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

template <int E>
static void launch_level_e(const MaskArgs& a, int nrows, hipStream_t stream) {
  hipLaunchKernelGGL((block_level_kernel<E>), dim3((nrows + 3) / 4), dim3(kMaskThreads), 0, stream, a.z,
                     a.level_map, a.cmass, a.N, a.nkb, nrows, a.L, a.n_dense_prefix, a.tau[0], a.tau[1],
                     a.tau[2], a.tau[3]);
}

template <typename T, int D>
static hipError_t launch_mask_t(const MaskArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((qblock_mean_kernel<T, D>), dim3(a.nqb, a.B * a.H), dim3(kMaskThreads), 0, stream,
                     static_cast<const T*>(a.q), a.qbar, a.N, a.q_block, a.nqb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int zstride = mask_score_stride(a.nkb);
  const int ktiles = (a.nkb + 31) / 32;
  dim3 sgrid((ktiles + 3) / 4, (a.nqb + 31) / 32, a.B * a.H);
  hipLaunchKernelGGL((block_score_kernel<D>), sgrid, dim3(kMaskThreads), 0, stream, a.qbar, a.k_bar, a.z, a.N,
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
