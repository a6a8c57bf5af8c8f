// Step 1 of the PSA forward path on gfx950: the average-pooled K/V pyramid and the
// per-block mean key.
//
// Pooling by 2^l consecutive tokens ("PSA: Pyramid Sparse Attention ...",
// skillmd.com page, "Pooled KV cache creation"; progressive pooling, top168.com
// article, three-components paragraph). This step moves K and V through once and
// writes levels 1..L-1 plus k_bar, so it is bound by HBM bandwidth: loads are
// 16-byte per lane, a wave reads whole 256-byte rows, every level of a 64-token
// block is produced from registers without re-reading.
//
// One workgroup per (KV block j, batch*KV head): the first half of the threads
// pools K, the second half V. Thread (row group rg, chunk c) owns rows 8rg..8rg+7
// of the block for one 16-byte column chunk, so level 1 (pairs), level 2 (quads)
// and level 3 (the eight rows) are in-thread sums; k_bar needs one LDS reduction
// over the eight row groups. Sums are float32; results are rounded once.
#include "psa_device.h"
#include "psa_launch.h"

namespace psa {

template <typename T, int D>
__global__ void __launch_bounds__(16 * (D / io_traits<T>::per16))
pyramid_pool_kernel(const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ kp,
                    T* __restrict__ vp, float* __restrict__ kbar, int N, int nkb,
                    int64_t pyr_rows, int off1, int off2, int off3, int L) {
  constexpr int E = io_traits<T>::per16;   // elements per 16-byte chunk
  constexpr int CPR = D / E;               // chunks per row
  constexpr int HALF = 8 * CPR;            // threads per tensor
  __shared__ float red[8][D];

  const int t = threadIdx.x;
  const int tensor = t / HALF;             // 0: K, 1: V
  const int tt = t - tensor * HALF;
  const int chunk = tt % CPR;
  const int rg = tt / CPR;
  const int j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int n_j = min(64, N - 64 * j);
  const int nv = min(max(n_j - 8 * rg, 0), 8);   // valid rows of this thread's group

  const T* src = (tensor ? v : k) + ((bh * N) + 64 * j + 8 * rg) * (int64_t)D + chunk * E;
  U128 raw[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (r < nv) raw[r] = ld128(src + (int64_t)r * D);
    else raw[r] = U128{{0u, 0u, 0u, 0u}};
  }
  float x[8][E];
#pragma unroll
  for (int r = 0; r < 8; ++r) unpack16<T>(raw[r], x[r]);

  float s1[4][E], s2[2][E], s3[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s1[i][e] = x[2 * i][e] + x[2 * i + 1][e];
#pragma unroll
    for (int i = 0; i < 2; ++i) s2[i][e] = s1[2 * i][e] + s1[2 * i + 1][e];
    s3[e] = s2[0][e] + s2[1][e];
  }

  T* dst = (tensor ? vp : kp) + bh * pyr_rows * D + chunk * E;
  float out[E];
  if (L > 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cnt = min(max(nv - 2 * i, 0), 2);
      if (cnt > 0) {
        const float inv = cnt == 2 ? 0.5f : 1.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = s1[i][e] * inv;
        st128(dst + (int64_t)(off1 + 32 * j + 4 * rg + i) * D, pack16<T>(out));
      }
    }
  }
  if (L > 2) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cnt = min(max(nv - 4 * i, 0), 4);
      if (cnt > 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = cnt == 4 ? s2[i][e] * 0.25f : s2[i][e] / (float)cnt;
        st128(dst + (int64_t)(off2 + 16 * j + 2 * rg + i) * D, pack16<T>(out));
      }
    }
  }
  if (L > 3 && nv > 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = nv == 8 ? s3[e] * 0.125f : s3[e] / (float)nv;
    st128(dst + (int64_t)(off3 + 8 * j + rg) * D, pack16<T>(out));
  }

  // k_bar: mean of K over the block's n_j tokens.
  if (tensor == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) red[rg][chunk * E + e] = s3[e];
  }
  __syncthreads();
  if (t < D) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) s += red[g][t];
    kbar[(bh * nkb + j) * D + t] = s / (float)n_j;
  }
}

template <typename T, int D>
static hipError_t launch_pyramid_t(const PyramidArgs& a, hipStream_t stream) {
  constexpr int threads = 16 * (D / io_traits<T>::per16);
  dim3 grid(a.nkb, a.B * a.H_kv);
  hipLaunchKernelGGL((pyramid_pool_kernel<T, D>), grid, dim3(threads), 0, stream,
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), static_cast<T*>(a.k_pyr),
                     static_cast<T*>(a.v_pyr), a.k_bar, a.N, a.nkb, a.pyr_rows, a.off[1], a.off[2],
                     a.off[3], a.L);
  return hipGetLastError();
}

hipError_t launch_pyramid(const PyramidArgs& a, hipStream_t stream) {
  if (a.bf16) return a.d == 128 ? launch_pyramid_t<bf16_t, 128>(a, stream) : launch_pyramid_t<bf16_t, 64>(a, stream);
  return a.d == 128 ? launch_pyramid_t<float, 128>(a, stream) : launch_pyramid_t<float, 64>(a, stream);
}

}  // namespace psa
