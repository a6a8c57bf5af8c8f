// Step 3 of the PSA forward path on gfx950: attention over mixed-resolution KV
// blocks under one online softmax.
//
// What is computed ("PSA: Pyramid Sparse Attention ...": chatpaper.ai abstract;
// top168.com article, three-components paragraph): query row r of query block i
// attends to every pooled row p of each KV block j the level map retains, at that
// block's level l; the logit of a pooled row is scale*<q_r, K^l_p> + ln c_p, c_p the
// number of tokens it averages, so one softmax over all rows keeps the probability
// of a pooled row equal to that of the c_p tokens it stands for.
//
// How (decoupled logical blocks / hardware tiles, chatpaper.ai abstract and the
// top168.com kernel paragraph, re-designed for CDNA4):
//  * One workgroup per (batch, head, query block); NW waves of 32 query rows each.
//    Workgroup ids are remapped so that the eight XCDs each take a contiguous run
//    of query blocks of the same heads (dispatch is round-robin over XCDs), which
//    keeps the K/V rows those blocks share in one XCD's L2.
//  * The level-map row is compacted in LDS into per-level lists of block indices.
//    A hardware tile is always 64 key rows of ONE level: 1 block at level 0,
//    2 at level 1, 4 at level 2, 8 at level 3. Within a tile every key carries the
//    same ln(2^l) bias, so the bias folds into the running max at no per-logit
//    cost; only the last tile of a level (padding, ragged tail) takes a per-key
//    correction path.
//  * Tiles are staged global -> registers -> LDS with one tile of prefetch (double
//    buffered LDS). K is stored row-major with an XOR swizzle of its 16-byte
//    chunks; V is stored transposed (V^T, key-contiguous) so it can feed the
//    matrix core as the A operand of O^T = V^T P^T.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as A, Q from registers
//    as B). In the 32x32 accumulator a lane owns one query column and 16 key rows;
//    the same registers, rounded to bf16, are the B operand of O^T = V^T P^T, once
//    the keys of V^T are laid out in the order the accumulator holds them (bits 2
//    and 3 of the key index swapped). O^T also leaves each lane with one query, so
//    the row max, row sum and rescale never leave the lane pair (l, l^32).
//  * Online softmax in base 2; the running max is only raised when a row's max
//    grows by more than 2^8, which keeps every P <= 256 and skips most rescales.
#include "psa_device.h"
#include "psa_launch.h"

namespace psa {

// Position of key kappa (0..63) of a tile inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int kappa) {
  return (kappa & 0x33) | ((kappa & 4) << 1) | ((kappa & 8) >> 1);
}

// Raw global data of 8 consecutive d values of one key row.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  U128 r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = ld128(p); }
  __device__ __forceinline__ U128 bf16() const { return r; }
};
template <> struct Raw8<float> {
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

template <typename T, int D, int NW>
struct AttnCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kCpr = D / 8;                // 16-byte bf16 chunks per K row
  static constexpr int kKpt = kCpr / NW;            // consecutive keys one thread stages
  static constexpr int kDt = D / 32;                // 32-wide d blocks of O^T
  static constexpr int kQc = D / 16;                // 16-deep d chunks of Q K^T
  static_assert(kKpt == 2 || kKpt == 4 || kKpt == 8, "staging layout");
};

__device__ __forceinline__ int k_swz(int row, int cpr) {
  return cpr == 16 ? (row & 15) : ((row >> 1) & 7);
}

template <typename T, int D, int NW>
__global__ void __launch_bounds__(NW * 64)
pyramid_attn_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                        const T* __restrict__ kp, const T* __restrict__ vp,
                        const int8_t* __restrict__ level_map, T* __restrict__ o, float* __restrict__ lse,
                        int H, int H_kv, int N, int nqb, int nkb, int L, int total_items, int per_xcd,
                        int64_t pyr_rows, int off1, int off2, int off3, int rows1, int rows2, int rows3,
                        float cs /* scale * log2(e) */) {
  using C = AttnCfg<T, D, NW>;
  constexpr int CPR = C::kCpr, KPT = C::kKpt;
  __shared__ __align__(16) uint16_t Ks[2][64 * D];
  __shared__ __align__(16) uint16_t Vt[2][D * 64];
  __shared__ float corr[2][64];
  __shared__ int16_t blist[kMaxKvBlocks];
  __shared__ int s_cnt[4], s_start[4], s_tile[5];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bid = blockIdx.x;
  const int item = (bid & 7) * per_xcd + (bid >> 3);
  if (item >= total_items) return;
  const int bh = item / nqb, qi = item - bh * nqb;
  const int b = bh / H, h = bh - b * H;
  const int bkv = b * H_kv + h / (H / H_kv);

  // ---- compact the level-map row into level-major block lists (wave 0)
  const int8_t* lrow = level_map + (int64_t)item * nkb;   // item == (b*H + h)*nqb + qi
  if (wave == 0) {
    int cnt[4] = {0, 0, 0, 0};
    for (int j0 = 0; j0 < nkb; j0 += 64) {
      const int j = j0 + lane;
      int lev = j < nkb ? (int)lrow[j] : -1;
      if (lev >= L) lev = -1;
#pragma unroll
      for (int l = 0; l < 4; ++l) cnt[l] += __popcll(__ballot(lev == l));
    }
    int pos[4];
    pos[0] = 0;
#pragma unroll
    for (int l = 1; l < 4; ++l) pos[l] = pos[l - 1] + cnt[l - 1];
    if (lane == 0) {
      int ts = 0;
#pragma unroll
      for (int l = 0; l < 4; ++l) {
        s_cnt[l] = cnt[l];
        s_start[l] = pos[l];
        s_tile[l] = ts;
        ts += (cnt[l] + (1 << l) - 1) >> l;
      }
      s_tile[4] = ts;
    }
    for (int j0 = 0; j0 < nkb; j0 += 64) {
      const int j = j0 + lane;
      int lev = j < nkb ? (int)lrow[j] : -1;
      if (lev >= L) lev = -1;
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
  }

  // ---- Q operand in registers: lane (row = lane%32, half = lane/32) holds d = 16c + 8*half + 0..7
  const int half = lane >> 5, l32 = lane & 31;
  const int q0 = qi * (32 * NW);
  const int my_row = q0 + 32 * wave + l32;
  bf16x8 qreg[C::kQc];
  {
    const T* qrow = q + ((int64_t)bh * N + min(my_row, N - 1)) * D;
#pragma unroll
    for (int c = 0; c < C::kQc; ++c) {
      Raw8<T> rw;
      rw.load(qrow + 16 * c + 8 * half);
      U128 u = rw.bf16();
      if (my_row >= N) u = U128{{0u, 0u, 0u, 0u}};
      qreg[c] = __builtin_bit_cast(bf16x8, make_uint4(u.w[0], u.w[1], u.w[2], u.w[3]));
    }
  }
  __syncthreads();

  const int T_total = s_tile[4];
  const T* kh = k + (int64_t)bkv * N * D;
  const T* vh = v + (int64_t)bkv * N * D;
  const T* kph = kp ? kp + (int64_t)bkv * pyr_rows * D : nullptr;
  const T* vph = vp ? vp + (int64_t)bkv * pyr_rows * D : nullptr;
  const int offs[4] = {0, off1, off2, off3};
  const int rows_l[4] = {N, rows1, rows2, rows3};
  const int rem = N & 63;

  // staging role: 16-byte chunk sc of keys KPT*sg .. KPT*sg + KPT-1
  const int sc = tid % CPR, sg = tid / CPR;
  const int key0 = KPT * sg;

  // tile t -> (level, index within level, irregular?)
  auto tile_info = [&](int t, int& lvl, int& u, bool& irregular) {
    lvl = 0;
#pragma unroll
    for (int l = 1; l < 4; ++l)
      if (t >= s_tile[l]) lvl = l;
    u = t - s_tile[lvl];
    const int cntl = s_cnt[lvl];
    const int ntl = s_tile[lvl + 1] - s_tile[lvl];
    const bool last = (u == ntl - 1);
    const bool pad = (cntl & ((1 << lvl) - 1)) != 0;
    const bool tail = rem != 0 && blist[s_start[lvl] + cntl - 1] == nkb - 1;
    irregular = last && (pad || tail);
  };

  Raw8<T> kr[KPT], vr[KPT];
  auto load_tile = [&](int t) {
    int lvl, u; bool irr;
    tile_info(t, lvl, u, irr);
    const int seglen = 64 >> lvl;
    const int li = (u << lvl) + (key0 >> (6 - lvl));
    const bool vseg = li < s_cnt[lvl];
    const int blk = vseg ? (int)blist[s_start[lvl] + li] : 0;
    const int prow0 = blk * seglen + (key0 & (seglen - 1));
    const T* kb = lvl == 0 ? kh : kph + (int64_t)offs[lvl] * D;
    const T* vb = lvl == 0 ? vh : vph + (int64_t)offs[lvl] * D;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int prow = prow0 + i;
      const bool ok = vseg && prow < rows_l[lvl];
      const int64_t r = ok ? prow : 0;
      kr[i].load(kb + r * D + 8 * sc);
      vr[i].load(vb + r * D + 8 * sc);
    }
  };
  auto store_tile = [&](int t, int buf) {
    int lvl, u; bool irr;
    tile_info(t, lvl, u, irr);
    uint16_t* kd = Ks[buf];
    uint16_t* vd = Vt[buf];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int row = key0 + i;
      const U128 x = kr[i].bf16();
      st128(kd + row * D + ((sc ^ k_swz(row, CPR)) * 8), x);
    }
    U128 xv[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) xv[i] = vr[i].bf16();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * sc + e;
      const int w = e >> 1;
      const bool hi = e & 1;
      uint16_t* vrow = vd + d * 64;
      const int swz = (d >> 1) & 7;
      if constexpr (KPT == 2) {
        const uint32_t a = xv[0].w[w], c = xv[1].w[w];
        const uint32_t pk = hi ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
        const int pos = vt_pos(key0);
        *reinterpret_cast<uint32_t*>(vrow + (((pos >> 3) ^ swz) * 8) + (pos & 7)) = pk;
      } else {
#pragma unroll
        for (int g4 = 0; g4 < KPT / 4; ++g4) {
          const uint32_t a0 = xv[4 * g4].w[w], a1 = xv[4 * g4 + 1].w[w];
          const uint32_t a2 = xv[4 * g4 + 2].w[w], a3 = xv[4 * g4 + 3].w[w];
          uint2 pk;
          pk.x = hi ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
          pk.y = hi ? ((a2 >> 16) | (a3 & 0xffff0000u)) : ((a2 & 0xffffu) | (a3 << 16));
          const int pos = vt_pos(key0 + 4 * g4);
          *reinterpret_cast<uint2*>(vrow + (((pos >> 3) ^ swz) * 8) + (pos & 7)) = pk;
        }
      }
    }
    if (irr && sc == 0) {
      // per-key logit correction (in units of the raw dot product):
      // -inf for padding / rows past the sequence, log2(c)-l for a ragged pool group
      const int seglen = 64 >> lvl;
      const int li = (u << lvl) + (key0 >> (6 - lvl));
      const bool vseg = li < s_cnt[lvl];
      const int blk = vseg ? (int)blist[s_start[lvl] + li] : 0;
      const int prow0 = blk * seglen + (key0 & (seglen - 1));
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int prow = prow0 + i;
        float cval = -INFINITY;
        if (vseg && prow < rows_l[lvl]) {
          const int cnt = min(1 << lvl, N - (prow << lvl));
          cval = cnt == (1 << lvl) ? 0.f : (__log2f((float)cnt) - (float)lvl) / cs;
        }
        corr[buf][key0 + i] = cval;
      }
    }
  };

  f32x16 oacc[C::kDt];
#pragma unroll
  for (int t = 0; t < C::kDt; ++t)
#pragma unroll
    for (int x = 0; x < 16; ++x) oacc[t][x] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (T_total > 0) {
    load_tile(0);
    store_tile(0, 0);
  }
  __syncthreads();

  for (int t = 0; t < T_total; ++t) {
    const int buf = t & 1;
    if (t + 1 < T_total) load_tile(t + 1);
    int lvl, u; bool irr;
    tile_info(t, lvl, u, irr);
    const uint16_t* Kb = Ks[buf];
    const uint16_t* Vb = Vt[buf];

    // S^T = K Q^T: two 32-key halves
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int x = 0; x < 16; ++x) sacc[kb][x] = 0.f;
      const int krow = 32 * kb + l32;
      const uint16_t* kr_l = Kb + krow * D;
      const int swz = k_swz(krow, CPR);
#pragma unroll
      for (int c = 0; c < C::kQc; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr_l + (((2 * c + half) ^ swz) * 8));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], sacc[kb], 0, 0, 0);
      }
    }
    if (irr) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x)
          sacc[kb][x] += corr[buf][32 * kb + 8 * (x >> 2) + 4 * half + (x & 3)];
    }

    // online softmax (base 2); this tile's keys all carry bias lvl
    float tmax = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int x = 0; x < 16; ++x) tmax = fmaxf(tmax, sacc[kb][x]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float lvlf = (float)lvl;
    const float mt = fmaf(tmax, cs, lvlf);
    const bool upd = mt > m_run + 8.0f;
    if (__ballot(upd)) {
      const float m_new = upd ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int tt = 0; tt < C::kDt; ++tt)
#pragma unroll
        for (int x = 0; x < 16; ++x) oacc[tt][x] *= alpha;
      m_run = m_new;
    }
    const float moff = lvlf - m_run;
    bf16x8 preg[4];
    float lsum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[c >> 1][8 * (c & 1) + e], cs, moff));
        lsum += p;
        preg[c][e] = (__bf16)p;
      }
    }
    l_run += lsum;

    // O^T += V^T P^T
#pragma unroll
    for (int tt = 0; tt < C::kDt; ++tt) {
      const int drow = 32 * tt + l32;
      const uint16_t* vr_l = Vb + drow * 64;
      const int swz = (drow >> 1) & 7;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vr_l + (((2 * c + half) ^ swz) * 8));
        oacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, preg[c], oacc[tt], 0, 0, 0);
      }
    }

    if (t + 1 < T_total) store_tile(t + 1, buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and write O (and LSE)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (my_row < N) {
    T* orow = o + ((int64_t)bh * N + my_row) * D;
#pragma unroll
    for (int tt = 0; tt < C::kDt; ++tt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * tt + 8 * g4 + 4 * half;
        const float y0 = oacc[tt][4 * g4] * inv, y1 = oacc[tt][4 * g4 + 1] * inv;
        const float y2 = oacc[tt][4 * g4 + 2] * inv, y3 = oacc[tt][4 * g4 + 3] * inv;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
        } else {
          *reinterpret_cast<float4*>(orow + d) = make_float4(y0, y1, y2, y3);
        }
      }
    }
    if (lse && half == 0)
      lse[(int64_t)bh * N + my_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  }
}

template <typename T, int D, int NW>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  const int total = a.B * a.H * a.nqb;
  const int per = (total + 7) / 8;
  const float cs = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((pyramid_attn_fwd_kernel<T, D, NW>), dim3(8 * per), dim3(NW * 64), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                     static_cast<const T*>(a.k_pyr), static_cast<const T*>(a.v_pyr), a.level_map,
                     static_cast<T*>(a.o), a.lse, a.H, a.H_kv, a.N, a.nqb, a.nkb, a.L, total, per,
                     a.pyr_rows, a.off[1], a.off[2], a.off[3], a.rows[1], a.rows[2], a.rows[3], cs);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_attn_dtype(const AttnArgs& a, hipStream_t stream) {
  if (a.d == 128) {
    return a.q_block == 128 ? launch_attn_t<T, 128, 4>(a, stream) : launch_attn_t<T, 128, 2>(a, stream);
  }
  return a.q_block == 128 ? launch_attn_t<T, 64, 4>(a, stream) : launch_attn_t<T, 64, 2>(a, stream);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_attn_dtype<bf16_t>(a, stream) : launch_attn_dtype<float>(a, stream);
}

}  // namespace psa
