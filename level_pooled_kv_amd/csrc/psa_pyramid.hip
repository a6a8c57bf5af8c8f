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
//
// Optionally (k_sim != NULL) the same registers give each block's key similarity per
// pooled level, for the cosine-similarity constraint of the ablation (top168.com
// article; the formula is this library's reading): a level-l pool group scores the
// mean over its tokens of cos(k_t, group mean), the block the smallest group score.
// Partial dot products over a thread's chunk are summed across the row's chunk
// lanes with DPP / lane-swap adds, so K is still read once.
#include "psa_device.h"
#include "psa_launch.h"

namespace psa {

template <typename T, int D, bool SIM>
__global__ void __launch_bounds__(16 * (D / io_traits<T>::per16))
pyramid_pool_kernel(const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ kp,
                    T* __restrict__ vp, float* __restrict__ kbar, float* __restrict__ ksim, int N, int nkb,
                    int64_t pyr_rows, int off1, int off2, int off3, int L) {
  constexpr int E = io_traits<T>::per16;   // elements per 16-byte chunk
  constexpr int CPR = D / E;               // chunks per row
  constexpr int HALF = 8 * CPR;            // threads per tensor
  static_assert(HALF % 64 == 0 && 64 % CPR == 0, "a wave holds whole row groups of one tensor");
  __shared__ float red[8][D];
  __shared__ float smin[8][3];

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

  // key similarity per pooled level (K half only; wave-uniform branch)
  if (SIM && L > 1 && tensor == 0) {
    const int lane = t & 63;
    float nt[8], d1[8], d2[8], d3[8], g1[4], g2[2], g3 = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      nt[r] = d1[r] = d2[r] = d3[r] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        nt[r] = fmaf(x[r][e], x[r][e], nt[r]);
        d1[r] = fmaf(x[r][e], s1[r >> 1][e], d1[r]);
        d2[r] = fmaf(x[r][e], s2[r >> 2][e], d2[r]);
        d3[r] = fmaf(x[r][e], s3[e], d3[r]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g1[i] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) g1[i] = fmaf(s1[i][e], s1[i][e], g1[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      g2[i] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) g2[i] = fmaf(s2[i][e], s2[i][e], g2[i]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) g3 = fmaf(s3[e], s3[e], g3);
    // totals over the row's CPR chunk lanes (consecutive, aligned lanes)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      nt[r] = group_sum<CPR>(nt[r], lane);
      d1[r] = group_sum<CPR>(d1[r], lane);
      d2[r] = group_sum<CPR>(d2[r], lane);
      d3[r] = group_sum<CPR>(d3[r], lane);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) g1[i] = group_sum<CPR>(g1[i], lane);
#pragma unroll
    for (int i = 0; i < 2; ++i) g2[i] = group_sum<CPR>(g2[i], lane);
    g3 = group_sum<CPR>(g3, lane);
    // cos(k_t, group sum) = cos(k_t, group mean); 0 when either vector is zero
    auto cosv = [](float dot, float na, float nb) {
      return na > 0.f && nb > 0.f ? dot * rsqrtf(na) * rsqrtf(nb) : 0.f;
    };
    float m1 = INFINITY, m2 = INFINITY, m3 = INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cnt = min(max(nv - 2 * i, 0), 2);
      if (cnt > 0) {
        float c = cosv(d1[2 * i], nt[2 * i], g1[i]);
        if (cnt == 2) c += cosv(d1[2 * i + 1], nt[2 * i + 1], g1[i]);
        m1 = fminf(m1, c / (float)cnt);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cnt = min(max(nv - 4 * i, 0), 4);
      if (cnt > 0) {
        float c = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r < cnt) c += cosv(d2[4 * i + r], nt[4 * i + r], g2[i]);
        m2 = fminf(m2, c / (float)cnt);
      }
    }
    if (nv > 0) {
      float c = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r < nv) c += cosv(d3[r], nt[r], g3);
      m3 = c / (float)nv;
    }
    if (chunk == 0) {
      smin[rg][0] = m1;
      smin[rg][1] = m2;
      smin[rg][2] = m3;
    }
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
  if (SIM && t < L - 1) {   // level t + 1: smallest group score over the row groups
    float m = INFINITY;
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (8 * g < n_j) m = fminf(m, smin[g][t]);
    ksim[(bh * nkb + j) * (L - 1) + t] = m;
  }
}

// Cosine-similarity cap: a retained block at level l > 0 drops to the coarsest level
// l' <= l whose levels 1..l' all have key similarity >= threshold (level 0 always).
__global__ void __launch_bounds__(256)
similarity_cap_kernel(int8_t* __restrict__ level_map, const float* __restrict__ ksim, float threshold, int H,
                      int H_kv, int nqb, int nkb, int L) {
  const int64_t row = blockIdx.x;                       // (b*H + h)*nqb + i: wave-uniform
  const int j = blockIdx.y * 256 + threadIdx.x;
  if (j >= nkb) return;
  int8_t* lp = level_map + row * nkb + j;
  const int lev = *lp;
  if (lev <= 0 || lev >= L) return;          // pruned, full resolution, or out of range: unchanged
  const int64_t bh = row / nqb;
  const int64_t b = bh / H;
  const int h = (int)(bh - b * H);
  const int64_t g = b * H_kv + h / (H / H_kv);
  const float* s = ksim + (g * nkb + j) * (L - 1);
  int cap = 0;
  for (int l = 1; l <= lev; ++l) {
    if (!(s[l - 1] >= threshold)) break;
    cap = l;
  }
  if (cap < lev) *lp = (int8_t)cap;
}

hipError_t launch_similarity_cap(const CapArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.nqb;   // < 2^31 (checked with the problem)
  if (rows == 0 || a.L < 2) return hipSuccess;
  hipLaunchKernelGGL(similarity_cap_kernel, dim3((unsigned)rows, (unsigned)((a.nkb + 255) / 256)), dim3(256), 0,
                     stream, a.level_map, a.k_sim, a.threshold, a.H, a.H_kv, a.nqb, a.nkb, a.L);
  return hipGetLastError();
}

template <typename T, int D, bool SIM>
static hipError_t launch_pyramid_s(const PyramidArgs& a, hipStream_t stream) {
  constexpr int threads = 16 * (D / io_traits<T>::per16);
  dim3 grid(a.nkb, a.B * a.H_kv);
  hipLaunchKernelGGL((pyramid_pool_kernel<T, D, SIM>), grid, dim3(threads), 0, stream,
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), static_cast<T*>(a.k_pyr),
                     static_cast<T*>(a.v_pyr), a.k_bar, a.k_sim, a.N, a.nkb, a.pyr_rows, a.off[1], a.off[2],
                     a.off[3], a.L);
  return hipGetLastError();
}

// The similarity registers would halve occupancy of the plain pyramid, so it is a
// separate instantiation.
template <typename T, int D>
static hipError_t launch_pyramid_t(const PyramidArgs& a, hipStream_t stream) {
  return a.k_sim ? launch_pyramid_s<T, D, true>(a, stream) : launch_pyramid_s<T, D, false>(a, stream);
}

hipError_t launch_pyramid(const PyramidArgs& a, hipStream_t stream) {
  if (a.bf16) return a.d == 128 ? launch_pyramid_t<bf16_t, 128>(a, stream) : launch_pyramid_t<bf16_t, 64>(a, stream);
  return a.d == 128 ? launch_pyramid_t<float, 128>(a, stream) : launch_pyramid_t<float, 64>(a, stream);
}

}  // namespace psa
