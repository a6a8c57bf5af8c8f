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
// Two kernels:
//  * qblock_mean_kernel streams Q once (HBM-bound, 16-byte loads, whole rows per
//    wave) and writes the float32 mean query of each query block to the workspace.
//  * block_mask_kernel takes R query blocks of one head per workgroup, computes
//    their R x nkb float32 scores against k_bar (k_bar is read once per R rows),
//    then per row: softmax, an LDS bitonic sort of (score, index) keys, a
//    deterministic exclusive prefix sum of the sorted masses, threshold compares,
//    and scattered int8 level writes.
#include "psa_device.h"
#include "psa_launch.h"

namespace psa {

constexpr int kMaskThreads = 256;
constexpr int kMaskWaves = kMaskThreads / 64;

template <typename T, int D>
__global__ void __launch_bounds__(kMaskThreads)
qblock_mean_kernel(const T* __restrict__ q, float* __restrict__ qbar, int N, int q_block, int nqb) {
  constexpr int E = io_traits<T>::per16;
  constexpr int CPR = D / E;
  constexpr int G = kMaskThreads / CPR;     // row groups
  __shared__ float red[G][D];
  const int t = threadIdx.x;
  const int chunk = t % CPR, g = t / CPR;
  const int i = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int r0 = i * q_block;
  const int m = min(q_block, N - r0);
  const T* src = q + (bh * N + r0) * (int64_t)D + chunk * E;

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  // rows g, g+G, g+2G, ...: one load instruction of a wave covers 64/CPR consecutive rows
  for (int r = g; r < m; r += 2 * G) {
    const bool two = r + G < m;
    U128 a = ld128(src + (int64_t)r * D);
    U128 b = two ? ld128(src + (int64_t)(r + G) * D) : U128{{0u, 0u, 0u, 0u}};
    float xa[E], xb[E];
    unpack16<T>(a, xa);
    unpack16<T>(b, xb);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += xa[e] + xb[e];
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
__device__ __forceinline__ uint64_t rank_key(float z, int j) {
  uint32_t u = __float_as_uint(z + 0.0f);          // -0 -> +0
  uint32_t key = (u & 0x80000000u) ? u : (~u & 0x7fffffffu);
  return ((uint64_t)key << 32) | (uint32_t)j;
}

template <int D>
__global__ void __launch_bounds__(kMaskThreads)
block_mask_kernel(const float* __restrict__ qbar, const float* __restrict__ kbar,
                  int8_t* __restrict__ level_map, float* __restrict__ cmass,
                  int N, int H, int H_kv, int nqb, int nkb, int L, int n_dense_prefix,
                  float scale, float tau0, float tau1, float tau2, float tau3, int R, int n_pad) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);                 // [n_pad]
  float* pbuf = reinterpret_cast<float*>(keys + n_pad);               // [n_pad]
  float* qs = pbuf + n_pad;                                           // [R][D]
  float* zs = qs + R * D;                                             // [R][nkb]
  __shared__ float red[kMaskWaves];
  __shared__ float scan_w[kMaskWaves];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int b = blockIdx.y / H, h = blockIdx.y % H;
  const int g = h / (H / H_kv);
  const int i0 = blockIdx.x * R;
  const int nr = min(R, nqb - i0);
  const float tau[4] = {tau0, tau1, tau2, tau3};

  // ---- scores z[r][j] = scale * <qbar_r, kbar_j> + ln n_j
  const float* qsrc = qbar + ((int64_t)(b * H + h) * nqb + i0) * D;
  for (int x = t; x < nr * D; x += kMaskThreads) qs[x] = qsrc[x];
  __syncthreads();
  const float* kb_head = kbar + (int64_t)(b * H_kv + g) * nkb * D;
  for (int j = t; j < nkb; j += kMaskThreads) {
    const float4* kr = reinterpret_cast<const float4*>(kb_head + (int64_t)j * D);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = 0; c < D / 4; ++c) {
      const float4 kv = kr[c];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < nr) {
          const float4 qv = *reinterpret_cast<const float4*>(qs + r * D + 4 * c);
          acc[r] = fmaf(kv.x, qv.x, acc[r]);
          acc[r] = fmaf(kv.y, qv.y, acc[r]);
          acc[r] = fmaf(kv.z, qv.z, acc[r]);
          acc[r] = fmaf(kv.w, qv.w, acc[r]);
        }
      }
    }
    const float lnn = logf((float)min(64, N - 64 * j));
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < nr) zs[r * nkb + j] = fmaf(scale, acc[r], lnn);
  }
  __syncthreads();

  const int per = (n_pad + kMaskThreads - 1) / kMaskThreads;   // sorted positions per thread
  for (int r = 0; r < nr; ++r) {
    const float* z = zs + r * nkb;
    // ---- row max and softmax denominator
    float mx = -INFINITY;
    for (int j = t; j < nkb; j += kMaskThreads) mx = fmaxf(mx, z[j]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = red[0];
#pragma unroll
    for (int w = 1; w < kMaskWaves; ++w) mx = fmaxf(mx, red[w]);
    __syncthreads();
    float s = 0.f;
    for (int j = t; j < nkb; j += kMaskThreads) {
      const float e = expf(z[j] - mx);
      pbuf[j] = e;
      s += e;
    }
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    s = red[0];
#pragma unroll
    for (int w = 1; w < kMaskWaves; ++w) s += red[w];
    const float inv_s = 1.0f / s;
    for (int j = t; j < n_pad; j += kMaskThreads) {
      if (j < nkb) {
        pbuf[j] *= inv_s;
        keys[j] = rank_key(z[j], j);
      } else {
        keys[j] = ~0ull;
      }
    }
    __syncthreads();

    // ---- bitonic sort of keys[0, n_pad), ascending
    for (int kk = 2; kk <= n_pad; kk <<= 1) {
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        for (int x = t; x < (n_pad >> 1); x += kMaskThreads) {
          const int lo = ((x & ~(jj - 1)) << 1) | (x & (jj - 1));
          const int hi = lo + jj;
          const bool up = (lo & kk) == 0;
          const uint64_t a = keys[lo], c = keys[hi];
          if ((a > c) == up) { keys[lo] = c; keys[hi] = a; }
        }
        __syncthreads();
      }
    }

    // ---- exclusive prefix sum of masses in rank order (fixed order: deterministic)
    const int p0 = t * per, p1 = min(p0 + per, nkb);
    float loc = 0.f;
    for (int x = p0; x < p1; ++x) loc += pbuf[(uint32_t)keys[x]];
    // exclusive scan of loc across threads
    float incl = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) scan_w[wave] = incl;
    __syncthreads();
    float run = incl - loc;
    for (int w = 0; w < wave; ++w) run += scan_w[w];

    int8_t* lrow = level_map + ((int64_t)(b * H + h) * nqb + i0 + r) * nkb;
    float* crow = cmass ? cmass + ((int64_t)(b * H + h) * nqb + i0 + r) * nkb : nullptr;
    for (int x = p0; x < p1; ++x) {
      const int j = (int)(uint32_t)keys[x];
      const float C = run;
      run += pbuf[j];
      int lev = -1;
      for (int l = L - 1; l >= 0; --l)
        if (C < tau[l]) lev = l;
      if (64 * j < n_dense_prefix) lev = 0;
      lrow[j] = (int8_t)lev;
      if (crow) crow[j] = C;
    }
    __syncthreads();
  }
}

template <typename T, int D>
static hipError_t launch_mask_t(const MaskArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((qblock_mean_kernel<T, D>), dim3(a.nqb, a.B * a.H), dim3(kMaskThreads), 0, stream,
                     static_cast<const T*>(a.q), a.qbar, a.N, a.q_block, a.nqb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int n_pad = 1;
  while (n_pad < a.nkb) n_pad <<= 1;
  const int R = 4;
  const size_t lds = (size_t)n_pad * (8 + 4) + (size_t)R * D * 4 + (size_t)R * a.nkb * 4;
  dim3 grid((a.nqb + R - 1) / R, a.B * a.H);
  hipLaunchKernelGGL((block_mask_kernel<D>), grid, dim3(kMaskThreads), lds, stream, a.qbar, a.k_bar,
                     a.level_map, a.cmass, a.N, a.H, a.H_kv, a.nqb, a.nkb, a.L, a.n_dense_prefix,
                     a.scale, a.tau[0], a.tau[1], a.tau[2], a.tau[3], R, n_pad);
  return hipGetLastError();
}

size_t mask_lds_bytes(int nkb, int d) {
  int n_pad = 1;
  while (n_pad < nkb) n_pad <<= 1;
  return (size_t)n_pad * 12 + 4 * (size_t)d * 4 + 4 * (size_t)nkb * 4;
}

hipError_t launch_mask(const MaskArgs& a, hipStream_t stream) {
  if (a.bf16) return a.d == 128 ? launch_mask_t<bf16_t, 128>(a, stream) : launch_mask_t<bf16_t, 64>(a, stream);
  return a.d == 128 ? launch_mask_t<float, 128>(a, stream) : launch_mask_t<float, 64>(a, stream);
}

}  // namespace psa
