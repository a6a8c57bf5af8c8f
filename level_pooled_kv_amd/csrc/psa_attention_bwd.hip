// Backward of the PSA attention step on gfx950: gradients of the output with respect to
// q, k and v, with the level map held fixed (it is a discrete choice).
//
// The pages describe no backward pass (the top168.com article implies training use:
// its models are fine-tuned and distilled with PSA); this is the gradient of the
// forward defined in psa_attention.hip. Per query row r and retained pooled key p,
// with P_rp = exp(a_rp - lse_r) and D_r = <dO_r, O_r>:
//   dV_p = sum_r P_rp dO_r,  dS_rp = P_rp (<dO_r, V_p> - D_r),
//   dq_r = scale sum_p dS_rp K_p,  dK_p = scale sum_r dS_rp q_r,
// and a pooled row, the mean of its c tokens, passes 1/c of its gradient to each.
//
// Four kernels:
//  * bwd_rowdot_kernel: D_r from O and dO (HBM-bound, one pass).
//  * pyramid_attn_bwd_dq_kernel: dq, one workgroup per (batch, head, query block) over
//    the same level-homogeneous 64-row key tiles as the forward (S^T = K Q^T and
//    dP^T = V dO^T on the matrix cores, dq^T += K^T dS^T with K^T read by LDS
//    transposing loads; 64-row query blocks split each tile's keys between two wave
//    pairs and sum their dq^T at the end). No atomics.
//  * pyramid_attn_bwd_dkdv_kernel: dK and dV of the pooled rows, key-outer: one
//    workgroup per (batch, KV head, level, 64-row tile of that level) walks every
//    (query head of the group, query block) that keeps any block of the tile at that
//    level (blocks it does not keep are masked per key), stages the query block's Q
//    and dO in LDS and accumulates dK^T and dV^T in registers. A head's tiles are
//    dispatched from the coarsest level down (the long items first). No atomics; each
//    pooled row is written once (float32, zero if unused).
//  * bwd_unpool_kernel: dk_t = dK^0_t + sum_l dK^l_{t >> l} / c, in the I/O dtype.
#include "psa_attn_common.h"

#include <type_traits>

namespace psa {

// ------------------------------------------------------------------ D_r = <dO_r, O_r>
// Row statistics of the backward, per (b, h) padded to Npad rows (a multiple of 64), stored
// as the dK/dV kernel uses them, the starting values of its S and dP accumulators:
// -lse2 / cs with lse2 the lse in base 2 and cs = scale * log2(e) (-inf for a row that saw
// no key and for padding, so its P is 0), and -D_r (0 on padding).
template <typename T, int D>
__global__ void __launch_bounds__(256)
bwd_rowdot_kernel(const T* __restrict__ o, const T* __restrict__ dout, const float* __restrict__ lse,
                  float* __restrict__ lse2, float* __restrict__ Dr, int N, int Npad, int64_t rows, float cs) {
  constexpr int E = io_traits<T>::per16, CPR = D / E, RPB = 256 / CPR;
  const int t = threadIdx.x, lane = t & 63, chunk = t % CPR;
  const int64_t prow = (int64_t)blockIdx.x * RPB + t / CPR;   // padded row index
  const int64_t bh = prow / Npad;
  const int r = (int)(prow - bh * Npad);
  const bool live = prow < rows && r < N;
  const int64_t row = bh * N + r;
  float s = 0.f;
  if (live) {
    float a[E], c[E];
    unpack16<T>(ld128(o + row * D + chunk * E), a);
    unpack16<T>(ld128(dout + row * D + chunk * E), c);
#pragma unroll
    for (int e = 0; e < E; ++e) s = fmaf(a[e], c[e], s);
  }
  s = group_sum<CPR>(s, lane);   // every lane takes part: no early exit above
  if (prow < rows && chunk == 0) {
    const float l = live ? lse[row] : -INFINITY;
    lse2[prow] = l > -INFINITY ? -(l * 1.4426950408889634f) / cs : -INFINITY;
    Dr[prow] = -s;
  }
}

// ------------------------------------------------------------------ dq (query-outer)
// KS = 2 (64-row query blocks): the NW = 4 waves are 2 row groups x 2 key halves of every
// tile, and the two halves' dq^T are summed through LDS at the end (four waves per
// workgroup keep two waves per SIMD).
template <typename T, int D, int NW, int KS>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
pyramid_attn_bwd_dq_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                           const T* __restrict__ kp, const T* __restrict__ vp,
                           const int8_t* __restrict__ level_map, const float* __restrict__ lse,
                           const float* __restrict__ Dr, const T* __restrict__ dout, T* __restrict__ dq,
                           int H, int H_kv, int N, int Npad, int nqb, int nkb, int L, int total_items, int per_xcd,
                           int64_t pyr_rows, int rows1, int rows2, float cs, float scale, int causal) {
  using C = AttnCfg<D, NW>;
  constexpr int CPR = C::kCpr, RPB = C::kRpb, BPW = C::kBpw;
  constexpr bool kDirect = sizeof(T) == 2;
  __shared__ __align__(16) uint16_t K0[64 * D], K1[64 * D];
  __shared__ __align__(16) uint16_t V0[64 * D], V1[64 * D];
  __shared__ float corr[2][64];
  __shared__ int ltok[2][64];
  __shared__ int16_t blist[kMaxKvBlocks];
  __shared__ uint32_t tdesc[kMaxKvBlocks + 4];
  __shared__ int s_tile[5];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar LDS destinations
  const int bid = blockIdx.x;
  const int item = (bid & 7) * per_xcd + (bid >> 3);
  if (item >= total_items) return;
  const int bh = item / nqb, qi = item - bh * nqb;
  const int b = bh / H, h = bh - b * H;
  const int bkv = b * H_kv + h / (H / H_kv);
  constexpr int RW = NW / KS;                 // row groups of 32 queries
  const int q0 = qi * (32 * RW);

  const int8_t* lrow = level_map + (int64_t)item * nkb;
  if (wave == 0) build_tile_lists(lrow, nkb, L, N, causal ? q0 / 64 : nkb, blist, tdesc, s_tile);

  // Q and dO as B operands: lane (row = lane%32, half = lane/32) holds d = 16c + 8*half + 0..7
  const int half = lane >> 5, l32 = lane & 31;
  const int khalf = KS == 1 ? 0 : wave / RW;   // key half of every tile
  const int my_row = q0 + 32 * (KS == 1 ? wave : wave % RW) + l32;
  bf16x8 qreg[C::kQc], doreg[C::kQc];
  {
    const int64_t roff = ((int64_t)bh * N + min(my_row, N - 1)) * D;
#pragma unroll
    for (int c = 0; c < C::kQc; ++c) {
      U128 uq, ud;
      if constexpr (kDirect) {
        uq = ld128(q + roff + 16 * c + 8 * half);
        ud = ld128(dout + roff + 16 * c + 8 * half);
      } else {
        Raw8f rq, rd;
        rq.load(reinterpret_cast<const float*>(q + roff) + 16 * c + 8 * half);
        rd.load(reinterpret_cast<const float*>(dout + roff) + 16 * c + 8 * half);
        uq = rq.bf16();
        ud = rd.bf16();
      }
      if (my_row >= N) uq = ud = U128{{0u, 0u, 0u, 0u}};
      qreg[c] = __builtin_bit_cast(bf16x8, make_uint4(uq.w[0], uq.w[1], uq.w[2], uq.w[3]));
      doreg[c] = __builtin_bit_cast(bf16x8, make_uint4(ud.w[0], ud.w[1], ud.w[2], ud.w[3]));
    }
  }
  // row statistics: lse in base 2, D; a row that saw no key (lse = -inf) gets no gradient
  const float lse_r = my_row < N ? lse[(int64_t)bh * N + my_row] : -INFINITY;
  const bool live = lse_r > -INFINITY;
  const float lse2 = live ? lse_r * 1.4426950408889634f : 0.f;
  const float d_r = my_row < N ? -Dr[(int64_t)bh * Npad + my_row] : 0.f;   // stored negated
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  const int T_total = __builtin_amdgcn_readfirstlane(s_tile[4]);
  const T* kh = k + (int64_t)bkv * N * D;
  const T* vh = v + (int64_t)bkv * N * D;
  const T* kph = kp ? kp + (int64_t)bkv * pyr_rows * D : nullptr;
  const T* vph = vp ? vp + (int64_t)bkv * pyr_rows * D : nullptr;
  auto tile_info = [&](int t) { return decode_tile(__builtin_amdgcn_readfirstlane(tdesc[t])); };
  auto level_rows = [&](int lvl) { return (N + (1 << lvl) - 1) >> lvl; };
  auto level_off = [&](int lvl) { return (lvl >= 2 ? rows1 : 0) + (lvl >= 3 ? rows2 : 0); };

  const int st_row0 = RPB * (wave * BPW) + lane / CPR;
  const int st_pchunk = lane % CPR;
  Raw8f fk[kDirect ? 1 : BPW], fv[kDirect ? 1 : BPW];
  auto kbuf = [&](auto P) -> uint16_t* { if constexpr (P() == 0) return K0; else return K1; };
  auto vbuf = [&](auto P) -> uint16_t* { if constexpr (P() == 0) return V0; else return V1; };
  // Per-key fixups of the rare tiles that need them (last of a level, causal diagonal),
  // out of the common path: logit corrections and last tokens of the staged key rows.
  auto tile_fixups = [&](const TileInfo& ti, int buf, const int* fprow, const bool* fok) {
    if (st_pchunk != 0) return;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int row = st_row0 + RPB * i;
      if (ti.irr) corr[buf][row] = key_correction(fok[i], ti.lvl, fprow[i], N, cs);
      if (ti.diag) ltok[buf][row] = key_last_token(fok[i], ti.lvl, fprow[i], N);
    }
  };
  // Both K and V are read row-wise (A operands) and K also transposed; both tiles use
  // the swizzle of tiles read both ways (qt_swz).
  auto issue_tile = [&](int t, auto P) {
    constexpr int buf = P();
    const TileInfo ti = tile_info(t);
    const int lvl = ti.lvl;
    const int sh = 6 - lvl, seglen = 64 >> lvl;
    const int rows_lv = level_rows(lvl);
    const int64_t loff = (int64_t)level_off(lvl) * D;
    const char* kb = reinterpret_cast<const char*>(lvl == 0 ? kh : kph + loff);
    const char* vb = reinterpret_cast<const char*>(lvl == 0 ? vh : vph + loff);
    uint32_t off[BPW];
    if (__builtin_expect(!(ti.irr || ti.diag), 1)) {
      // a regular tile: every segment is a whole block of full pooled rows, so each staged
      // row is valid (no per-row checks, no fixups)
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int row = st_row0 + RPB * i;
        const int blk = (int)blist[ti.base + (row >> sh)];
        off[i] = (uint32_t)((((blk << sh) + (row & (seglen - 1))) * D + 8 * (st_pchunk ^ qt_swz<D>(row))) *
                            (int)sizeof(T));
      }
    } else {
      int fx_prow[BPW];
      bool fx_ok[BPW];
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int row = st_row0 + RPB * i;
        const int seg = row >> sh;
        const bool vseg = seg < ti.nseg;
        const int blk = vseg ? (int)blist[ti.base + seg] : 0;
        const int prow = blk * seglen + (row & (seglen - 1));
        const bool ok = vseg && prow < rows_lv;
        const int rowel = (ok ? prow : 0) * D;
        off[i] = (uint32_t)((rowel + 8 * (st_pchunk ^ qt_swz<D>(row))) * (int)sizeof(T));
        fx_prow[i] = prow;
        fx_ok[i] = ok;
      }
      tile_fixups(ti, buf, fx_prow, fx_ok);
    }
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      if constexpr (kDirect) {
        const int blkoff = (wave * BPW + i) * 512;
        __builtin_amdgcn_global_load_lds((gbl_void*)(kb + off[i]), (lds_void*)(kbuf(P) + blkoff), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_void*)(vb + off[i]), (lds_void*)(vbuf(P) + blkoff), 16, 0, 0);
      } else {
        fk[i].load(reinterpret_cast<const float*>(kb + off[i]));
        fv[i].load(reinterpret_cast<const float*>(vb + off[i]));
      }
    }
  };
  auto commit_tile = [&](auto P) {
    if constexpr (!kDirect) {
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int off = (wave * BPW + i) * 512 + lane * 8;
        st128(kbuf(P) + off, fk[i].bf16());
        st128(vbuf(P) + off, fv[i].bf16());
      }
    }
  };

  f32x16 dqacc[C::kDt];
#pragma unroll
  for (int t = 0; t < C::kDt; ++t)
#pragma unroll
    for (int x = 0; x < 16; ++x) dqacc[t][x] = 0.f;

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if (T_total > 0) {
    issue_tile(0, P0{});
    commit_tile(P0{});
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  const int trg = lane >> 4, trs = lane & 15;
  const int tr_row = 4 * (trg >> 1) + (trs >> 2);
  const int tr_col = 16 * (trg & 1) + 4 * (trs & 3);

  auto body = [&](int t, auto P) {
    constexpr int buf = P();
    using PN = std::integral_constant<int, 1 - P()>;
    if (t + 1 < T_total) issue_tile(t + 1, PN{});
    const TileInfo ti = tile_info(t);
    const float lvlf = (float)ti.lvl;
    const uint16_t* Kb = kbuf(P);
    const uint16_t* Vb = vbuf(P);
    int zero;   // opaque: keeps the LDS address arithmetic in the loop (hoisted, it spilled)
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    // lane offsets of the S and dP operand reads (row 32 kb + l32, chunk (2c + half) ^ swz):
    // the swizzle depends on the row mod 16 only, so the 32-row step kb and the K / V tile
    // are immediate offsets
    int ko[C::kQc];
#pragma unroll
    for (int c = 0; c < C::kQc; ++c) ko[c] = (l32 + zero) * D + (((2 * c + half) ^ qt_swz<D>(l32)) * 8);
#pragma unroll
    for (int kbi = 0; kbi < 2 / KS; ++kbi) {
      const int kb = kbi + (2 / KS) * khalf;
      f32x16 sacc, dpacc;
#pragma unroll
      for (int x = 0; x < 16; ++x) sacc[x] = dpacc[x] = 0.f;
#pragma unroll
      for (int c = 0; c < C::kQc; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + 32 * kb * D + ko[c]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], sacc, 0, 0, 0);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(Vb + 32 * kb * D + ko[c]);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, doreg[c], dpacc, 0, 0, 0);
      }
      if (ti.irr) {
#pragma unroll
        for (int x = 0; x < 16; ++x) sacc[x] += corr[buf][32 * kb + 8 * (x >> 2) + 4 * half + (x & 3)];
      }
      if (ti.diag) {
#pragma unroll
        for (int x = 0; x < 16; ++x)
          if (ltok[buf][32 * kb + 8 * (x >> 2) + 4 * half + (x & 3)] > my_row) sacc[x] = -INFINITY;
      }
      // dS^T = P^T (dP^T - D), P^T = exp2(cs * S^T + lvl - lse2); keys in the order the
      // transposing K^T reads below deliver them
      bf16x8 dsr[2];
      // a row that saw no key takes an offset of -inf, so its P is 0 without a select
      const float off = live ? lvlf - lse2 : -INFINITY;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int x = 8 * cc + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[x], cs, off));
          dsr[cc][e] = (__bf16)(p * (dpacc[x] - d_r));
        }
      }
      // dq^T += K^T dS^T. The swizzle of row 16c + 8j + tr_row depends on the row mod 16 only,
      // so each (j, tt) takes one lane offset and the 16-row step c is an immediate offset
      int tro[2][C::kDt];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int tt = 0; tt < C::kDt; ++tt) {
          const int r = 8 * j + tr_row, col = 32 * tt + tr_col;
          tro[j][tt] = (r + zero) * D + ((col >> 3) ^ qt_swz<D>(r)) * 8 + (col & 7);
        }
#pragma unroll
      for (int tt = 0; tt < C::kDt; ++tt) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int c = 2 * kb + cc;
          bf16x4 part[2];
#pragma unroll
          for (int j = 0; j < 2; ++j)
            part[j] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Kb + tro[j][tt] + 16 * c * D));
          const bf16x8 a = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
          dqacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsr[cc], dqacc[tt], 0, 0, 0);
        }
      }
    }
    if (t + 1 < T_total) commit_tile(PN{});
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
  };
  for (int t = 0; t < T_total; t += 2) {
    body(t, P0{});
    if (t + 1 < T_total) body(t + 1, P1{});
  }

  if constexpr (KS == 2) {
    // sum the two key halves: the khalf = 1 waves hand their dq^T over through LDS (the
    // tile buffers are idle after the loop's last barrier)
    float* xq = reinterpret_cast<float*>((wave % RW) == 0 ? K0 : K1);   // [tt][x][lane]
    if (khalf == 1) {
#pragma unroll
      for (int tt = 0; tt < C::kDt; ++tt)
#pragma unroll
        for (int x = 0; x < 16; ++x) xq[(tt * 16 + x) * 64 + lane] = dqacc[tt][x];
    }
    __syncthreads();
    if (khalf == 0) {
#pragma unroll
      for (int tt = 0; tt < C::kDt; ++tt)
#pragma unroll
        for (int x = 0; x < 16; ++x) dqacc[tt][x] += xq[(tt * 16 + x) * 64 + lane];
    }
  }
  if (my_row < N && khalf == 0) {
    T* orow = dq + ((int64_t)bh * N + my_row) * D;
#pragma unroll
    for (int tt = 0; tt < C::kDt; ++tt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * tt + 8 * g4 + 4 * half;
        const float y0 = dqacc[tt][4 * g4] * scale, y1 = dqacc[tt][4 * g4 + 1] * scale;
        const float y2 = dqacc[tt][4 * g4 + 2] * scale, y3 = dqacc[tt][4 * g4 + 3] * scale;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
        } else {
          *reinterpret_cast<float4*>(orow + d) = make_float4(y0, y1, y2, y3);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ dK, dV (key-outer)
struct DkdvGeom {
  int tiles[kMaxLevels];     // 64-row tiles of level l: ceil(rows_l / 64)
  int first[kMaxLevels + 1]; // first tile index of level l among one head's tiles (coarsest level
                             // first); first[kMaxLevels] = tiles per head
  int rows[kMaxLevels];      // rows of level l (level 0: N)
  int woff[kMaxLevels];      // row offset of level l in a head's float32 gradient rows
  int poff[kMaxLevels];      // row offset of level l in the pyramid (l >= 1)
};

template <typename T, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
pyramid_attn_bwd_dkdv_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                             const T* __restrict__ kp, const T* __restrict__ vp,
                             const int8_t* __restrict__ level_map, const float* __restrict__ lse2p,
                             const float* __restrict__ Dp, const T* __restrict__ dout,
                             float* __restrict__ dkw, float* __restrict__ dvw, int H, int H_kv, int N, int Npad, int nqb,
                             int nkb, int L, int q_block, int total_items, int per_xcd, int64_t pyr_rows,
                             int64_t rows_all, DkdvGeom geo, float cs, float scale, int causal) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int E = io_traits<T>::per16;      // elements per 16-byte global chunk
  constexpr int kQc = D / 16, kDt = D / 32;
  constexpr int CH = D / 8;                   // 16-byte bf16 chunks per LDS row
  // LDS: K, V tiles (64 x D bf16) and Q, dO chunks (64 rows x D bf16); at the end the
  // same bytes hold the cross-wave reduction of dK^T, dV^T (2 x 2 x 32 x D floats).
  __shared__ __align__(16) uint16_t pool[4 * 64 * D];
  uint16_t* Ks = pool;
  uint16_t* Vs = pool + 64 * D;
  uint16_t* Qs = pool + 2 * 64 * D;
  uint16_t* Os = pool + 3 * 64 * D;
  __shared__ __align__(16) float s_lse2[64];
  __shared__ __align__(16) float s_D[64];
  __shared__ float s_keyb[64];
  __shared__ int s_ltok[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar LDS destinations
  const int bid = blockIdx.x;
  const int item = (bid & 7) * per_xcd + (bid >> 3);
  if (item >= total_items) return;
  const int tiles_head = geo.first[kMaxLevels];
  const int bg = item / tiles_head;
  const int rem = item - bg * tiles_head;
  // a head's tiles run from the coarsest level down: the coarse tiles, kept by many
  // query blocks, are the long items and start first
  int lvl = L - 1;
#pragma unroll
  for (int l = kMaxLevels - 2; l >= 0; --l)
    if (l < L - 1 && rem >= geo.first[l]) lvl = l;
  const int kt = rem - geo.first[lvl];
  const int b = bg / H_kv, g = bg - b * H_kv;
  const int G = H / H_kv;
  const int sh = 6 - lvl;
  const int nseg = 1 << lvl;
  const int rows_l = geo.rows[lvl];
  const int prow0 = kt * 64;
  const int j0 = kt << lvl;                   // first KV block of the tile

  // ---- stage the tile's pooled K and V rows (bf16, qt_swz swizzle), per-key constants
  {
    const T* ksrc = lvl == 0 ? k + (int64_t)bg * N * D : kp + ((int64_t)bg * pyr_rows + geo.poff[lvl]) * D;
    const T* vsrc = lvl == 0 ? v + (int64_t)bg * N * D : vp + ((int64_t)bg * pyr_rows + geo.poff[lvl]) * D;
    for (int u = tid; u < 64 * CH; u += 256) {
      const int row = u / CH, ch = u - row * CH;
      const int prow = prow0 + row;
      U128 kk{{0u, 0u, 0u, 0u}}, vv{{0u, 0u, 0u, 0u}};
      if (prow < rows_l) {
        if constexpr (sizeof(T) == 2) {
          kk = ld128(ksrc + (int64_t)prow * D + ch * 8);
          vv = ld128(vsrc + (int64_t)prow * D + ch * 8);
        } else {
          Raw8f rk, rv;
          rk.load(reinterpret_cast<const float*>(ksrc) + (int64_t)prow * D + ch * 8);
          rv.load(reinterpret_cast<const float*>(vsrc) + (int64_t)prow * D + ch * 8);
          kk = rk.bf16();
          vv = rv.bf16();
        }
      }
      const int pc = ch ^ qt_swz<D>(row);
      st128(Ks + row * D + pc * 8, kk);
      st128(Vs + row * D + pc * 8, vv);
    }
    if (tid < 64) {
      const int prow = prow0 + tid;
      const bool ok = prow < rows_l;
      const int cnt = ok ? min(1 << lvl, N - (prow << lvl)) : 1;
      s_keyb[tid] = ok ? __log2f((float)cnt) : -INFINITY;     // log2 of the pool count (ln c in base 2)
      s_ltok[tid] = key_last_token(ok, lvl, prow, N);
    }
  }
  __syncthreads();                            // s_keyb, s_ltok are read by every wave

  const int half = lane >> 5, l32 = lane & 31;
  const int kh = wave & 1, qh = wave >> 1;    // this wave's 32 keys and 32 queries of a 64-row chunk
  const int krow = 32 * kh + l32;             // key row of this lane's accumulator column
  const int trg = lane >> 4, trs = lane & 15;
  const int tr_row = 4 * (trg >> 1) + (trs >> 2);
  const int tr_col = 16 * (trg & 1) + 4 * (trs & 3);

  f32x16 dkacc[kDt], dvacc[kDt];
#pragma unroll
  for (int t = 0; t < kDt; ++t)
#pragma unroll
    for (int x = 0; x < 16; ++x) dkacc[t][x] = dvacc[t][x] = 0.f;

  const int npairs = G * nqb;
  for (int base = 0; base < npairs; base += 64) {
    // this lane's (query head, query block): the tile segments it keeps at this level
    const int pr = base + lane;
    uint32_t segm = 0;
    if (pr < npairs) {
      const int hh = pr / nqb, i = pr - hh * nqb;
      const int8_t* lm = level_map + (((int64_t)b * H + g * G + hh) * nqb + i) * nkb;
      for (int s = 0; s < nseg; ++s)
        if (j0 + s < nkb && lm[j0 + s] == lvl) segm |= 1u << s;
    }
    uint64_t todo = __ballot(segm != 0);      // the same in every wave of the workgroup
    while (todo) {
      const int sel = __builtin_ctzll(todo);
      todo &= todo - 1;
      const int pair = base + sel;
      const uint32_t mask = (uint32_t)__builtin_amdgcn_readlane((int)segm, sel);
      const int hh = pair / nqb, i = pair - hh * nqb;
      const int64_t bh = (int64_t)b * H + g * G + hh;
      const int key_used = (mask >> (krow >> sh)) & 1;
      // this wave's 32 keys: segments (32 kh) >> sh .. (32 kh + 31) >> sh
      const uint32_t hmask = lvl == 0 ? 1u : ((1u << (nseg >> 1)) - 1u) << (kh * (nseg >> 1));
      const bool active = (mask & hmask) != 0;   // wave-uniform: nothing to add otherwise
      const float kbias = key_used ? s_keyb[krow] : -INFINITY;   // log2 pool count; -inf: key not kept
      const int ktok = s_ltok[krow];
      for (int r0 = i * q_block; r0 < min((i + 1) * q_block, N); r0 += 64) {
        __syncthreads();                      // the previous chunk's reads are done
        // stage Q and dO rows r0..r0+63 (qt_swz swizzle; rows past N read row N-1 and are
        // never used: their lse2 is +inf, so P = dS = 0). bf16: direct global -> LDS
        // loads, each wave filling 1 KB blocks of RPK rows; all loads issued before any wait.
        {
          constexpr int RPK = 1024 / (2 * D);        // rows per 1 KB block
          constexpr int NBLK = 64 / RPK;             // blocks per tensor
          constexpr int BPWV = NBLK / 4;             // blocks per wave and tensor
          const int lrow = lane / CH, lch = lane % CH;
          if constexpr (sizeof(T) == 2) {
            // wave-uniform chunk bases plus 32-bit lane offsets (the scalar-base load form)
            const char* qc = reinterpret_cast<const char*>(q + (bh * N + r0) * D);
            const char* oc = reinterpret_cast<const char*>(dout + (bh * N + r0) * D);
            // an empty asm statement pins each base as one scalar value, so the compiler does not
            // re-associate the sums into per-lane 64-bit adds
            asm volatile("" : "+s"(qc), "+s"(oc));
            const int rlast = N - 1 - r0;                // last valid row of the chunk
#pragma unroll
            for (int bb = 0; bb < BPWV; ++bb) {
              const int blk = wave * BPWV + bb;
              const int row = blk * RPK + lrow;
              const int lc = lch ^ qt_swz<D>(row);     // logical chunk stored in physical slot lch
              const uint32_t off = (uint32_t)((min(row, rlast) * D + lc * 8) * (int)sizeof(T));
              __builtin_amdgcn_global_load_lds((gbl_void*)(qc + off), (lds_void*)(Qs + blk * 512), 16, 0, 0);
              __builtin_amdgcn_global_load_lds((gbl_void*)(oc + off), (lds_void*)(Os + blk * 512), 16, 0, 0);
            }
            const float* lc0 = lse2p + bh * Npad + r0;
            const float* dc0 = Dp + bh * Npad + r0;
            asm volatile("" : "+s"(lc0), "+s"(dc0));
            if (wave == 0) __builtin_amdgcn_global_load_lds((gbl_void*)(lc0 + lane), (lds_void*)s_lse2, 4, 0, 0);
            if (wave == 1) __builtin_amdgcn_global_load_lds((gbl_void*)(dc0 + lane), (lds_void*)s_D, 4, 0, 0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
          } else {
            Raw8f rq[BPWV], rd[BPWV];
#pragma unroll
            for (int bb = 0; bb < BPWV; ++bb) {
              const int row = (wave * BPWV + bb) * RPK + lrow;
              const int64_t r = min(r0 + row, N - 1);
              const int lc = lch ^ qt_swz<D>(row);
              rq[bb].load(reinterpret_cast<const float*>(q) + (bh * N + r) * D + lc * 8);
              rd[bb].load(reinterpret_cast<const float*>(dout) + (bh * N + r) * D + lc * 8);
            }
#pragma unroll
            for (int bb = 0; bb < BPWV; ++bb) {
              const int blk = wave * BPWV + bb;
              st128(Qs + blk * 512 + lane * 8, rq[bb].bf16());
              st128(Os + blk * 512 + lane * 8, rd[bb].bf16());
            }
          }
        }
        if constexpr (sizeof(T) != 2) {
          if (tid < 64) {
            s_lse2[tid] = lse2p[bh * Npad + r0 + tid];
            s_D[tid] = Dp[bh * Npad + r0 + tid];
          }
        }
        __syncthreads();

        if (!active) continue;                // the loop's barrier is at its top: no wave skips one
        // S = Q K^T and dP = dO V^T for 32 queries x 32 keys: lane holds key column krow,
        // rows = queries 32qh + 8(x>>2) + 4half + (x&3)
        // S starts from -lse2 / cs and dP from -D_r of its query row (the rows of accumulator
        // entries 4 g4 .. 4 g4 + 3 are 4 consecutive rows), so the exponent below is one FMA
        // and dS one product
        f32x16 sacc, dpacc;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 l4 = *reinterpret_cast<const float4*>(s_lse2 + 32 * qh + 8 * g4 + 4 * half);
          const float4 d4 = *reinterpret_cast<const float4*>(s_D + 32 * qh + 8 * g4 + 4 * half);
          sacc[4 * g4] = l4.x; sacc[4 * g4 + 1] = l4.y; sacc[4 * g4 + 2] = l4.z; sacc[4 * g4 + 3] = l4.w;
          dpacc[4 * g4] = d4.x; dpacc[4 * g4 + 1] = d4.y; dpacc[4 * g4 + 2] = d4.z; dpacc[4 * g4 + 3] = d4.w;
        }
        const int qrow = 32 * qh + l32;
        const int qswz = qt_swz<D>(qrow), kswz = qt_swz<D>(krow);
#pragma unroll
        for (int c = 0; c < kQc; ++c) {
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qs + qrow * D + (((2 * c + half) ^ qswz) * 8));
          const bf16x8 bk = *reinterpret_cast<const bf16x8*>(Ks + krow * D + (((2 * c + half) ^ kswz) * 8));
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, sacc, 0, 0, 0);
          const bf16x8 ad = *reinterpret_cast<const bf16x8*>(Os + qrow * D + (((2 * c + half) ^ qswz) * 8));
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(Vs + krow * D + (((2 * c + half) ^ kswz) * 8));
          dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, bv, dpacc, 0, 0, 0);
        }
        // the 16 query rows of this lane's accumulator entries come in 4 runs of 4
        bf16x8 preg[2], dsreg[2];
        // causal masking in its own copy of the loop (a scalar branch): the bidirectional
        // case does no per-pair compares
        auto probs = [&](auto CAUSAL) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int x = 4 * g4 + u;
              const int ql = 32 * qh + 8 * g4 + 4 * half + u;   // query row in the chunk
              // unseen pairs take an exponent of -inf (p = 0) instead of a branch
              float arg = fmaf(sacc[x], cs, kbias);
              if constexpr (CAUSAL()) arg = ktok > r0 + ql ? -INFINITY : arg;
              const float p = __builtin_amdgcn_exp2f(arg);
              preg[x >> 3][x & 7] = (__bf16)p;
              dsreg[x >> 3][x & 7] = (__bf16)(p * dpacc[x]);
            }
          }
        };
        if (causal) probs(std::true_type{});
        else probs(std::false_type{});
        // dV^T += dO^T P and dK^T += Q^T dS: A operands read transposed from LDS, the
        // query rows chosen in the order the S accumulator holds them
#pragma unroll
        for (int tt = 0; tt < kDt; ++tt) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            bf16x4 pd[2], pq[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int row = 32 * qh + 16 * cc + 8 * j + tr_row;
              const int col = 32 * tt + tr_col;
              const int chunk = (col >> 3) ^ qt_swz<D>(row);
              pd[j] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Os + row * D + chunk * 8 + (col & 7)));
              pq[j] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(Qs + row * D + chunk * 8 + (col & 7)));
            }
            const bf16x8 ad = __builtin_shufflevector(pd[0], pd[1], 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 aq = __builtin_shufflevector(pq[0], pq[1], 0, 1, 2, 3, 4, 5, 6, 7);
            dvacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, preg[cc], dvacc[tt], 0, 0, 0);
            dkacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, dsreg[cc], dkacc[tt], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- sum the two query halves of each key half and write the float32 rows
  __syncthreads();
  float* red = reinterpret_cast<float*>(pool);   // [kh][tensor][x][tt][lane]: 2 x 2 x 16 x kDt x 64 floats
  auto ridx = [&](int tensor, int tt, int x) { return (((kh * 2 + tensor) * 16 + x) * kDt + tt) * 64 + lane; };
  if (qh == 1) {
#pragma unroll
    for (int tt = 0; tt < kDt; ++tt)
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        red[ridx(0, tt, x)] = dkacc[tt][x];
        red[ridx(1, tt, x)] = dvacc[tt][x];
      }
  }
  __syncthreads();
  if (qh == 0) {
    const int prow = prow0 + krow;
    if (prow < rows_l) {
      const int64_t wrow = (int64_t)bg * rows_all + geo.woff[lvl] + prow;
      float* dkr = dkw + wrow * D;
      float* dvr = dvw + wrow * D;
#pragma unroll
      for (int tt = 0; tt < kDt; ++tt) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int d = 32 * tt + 8 * m + 4 * half;
          float4 kk, vv;
          kk.x = (dkacc[tt][4 * m] + red[ridx(0, tt, 4 * m)]) * scale;
          kk.y = (dkacc[tt][4 * m + 1] + red[ridx(0, tt, 4 * m + 1)]) * scale;
          kk.z = (dkacc[tt][4 * m + 2] + red[ridx(0, tt, 4 * m + 2)]) * scale;
          kk.w = (dkacc[tt][4 * m + 3] + red[ridx(0, tt, 4 * m + 3)]) * scale;
          vv.x = dvacc[tt][4 * m] + red[ridx(1, tt, 4 * m)];
          vv.y = dvacc[tt][4 * m + 1] + red[ridx(1, tt, 4 * m + 1)];
          vv.z = dvacc[tt][4 * m + 2] + red[ridx(1, tt, 4 * m + 2)];
          vv.w = dvacc[tt][4 * m + 3] + red[ridx(1, tt, 4 * m + 3)];
          *reinterpret_cast<float4*>(dkr + d) = kk;
          *reinterpret_cast<float4*>(dvr + d) = vv;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ pooled rows -> tokens
template <typename T, int D>
__global__ void __launch_bounds__(256)
bwd_unpool_kernel(const float* __restrict__ dkw, const float* __restrict__ dvw, T* __restrict__ dk,
                  T* __restrict__ dv, int N, int L, int64_t rows_all, DkdvGeom geo, int64_t total) {
  constexpr int E = io_traits<T>::per16, CPR = D / E;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= total) return;
  const int64_t row = u / CPR;                 // (bg, token)
  const int c = (int)(u - row * CPR);
  const int64_t bg = row / N;
  const int t = (int)(row - bg * N);
  float ak[E], av[E];
  const float* k0 = dkw + (bg * rows_all + t) * D + c * E;
  const float* v0 = dvw + (bg * rows_all + t) * D + c * E;
#pragma unroll
  for (int e = 0; e < E; ++e) { ak[e] = k0[e]; av[e] = v0[e]; }
#pragma unroll
  for (int l = 1; l < kMaxLevels; ++l) {
    if (l < L) {
      const int p = t >> l;
      const float inv = 1.0f / (float)min(1 << l, N - (p << l));
      const float* kl = dkw + (bg * rows_all + geo.woff[l] + p) * D + c * E;
      const float* vl = dvw + (bg * rows_all + geo.woff[l] + p) * D + c * E;
#pragma unroll
      for (int e = 0; e < E; ++e) { ak[e] = fmaf(kl[e], inv, ak[e]); av[e] = fmaf(vl[e], inv, av[e]); }
    }
  }
  st128(dk + row * D + c * E, pack16<T>(ak));
  st128(dv + row * D + c * E, pack16<T>(av));
}

// ------------------------------------------------------------------ launch
static DkdvGeom dkdv_geometry(const BwdArgs& a) {
  DkdvGeom g{};
  int woff = 0;
  for (int l = 0; l < kMaxLevels; ++l) {
    const int rows = l < a.L ? (a.N + (1 << l) - 1) >> l : 0;
    g.rows[l] = rows;
    g.tiles[l] = (rows + 63) / 64;
    g.woff[l] = woff;
    woff += rows;
    g.poff[l] = l >= 1 ? a.off[l] : 0;
  }
  int first = 0;   // levels L-1, ..., 0 in that order
  for (int l = a.L - 1; l >= 0; --l) {
    g.first[l] = first;
    first += g.tiles[l];
  }
  for (int l = a.L; l < kMaxLevels; ++l) g.first[l] = first;
  g.first[kMaxLevels] = first;
  return g;
}

template <typename T, int D, int NW, int KS>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  constexpr int E = io_traits<T>::per16, CPR = D / E;
  const T* q = static_cast<const T*>(a.q);
  const T* o = static_cast<const T*>(a.o);
  const T* dout = static_cast<const T*>(a.dout);
  const int64_t prows = (int64_t)a.B * a.H * a.Npad;
  const float cs = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((bwd_rowdot_kernel<T, D>), dim3((unsigned)((prows + 256 / CPR - 1) / (256 / CPR))), dim3(256), 0,
                     stream, o, dout, a.lse, a.lse2, a.Dr, a.N, a.Npad, prows, cs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int total = a.B * a.H * a.nqb;
  const int per = (total + 7) / 8;
  hipLaunchKernelGGL((pyramid_attn_bwd_dq_kernel<T, D, NW, KS>), dim3(8 * per), dim3(NW * 64), 0, stream, q,
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), static_cast<const T*>(a.k_pyr),
                     static_cast<const T*>(a.v_pyr), a.level_map, a.lse, a.Dr, dout, static_cast<T*>(a.dq), a.H,
                     a.H_kv, a.N, a.Npad, a.nqb, a.nkb, a.L, total, per, a.pyr_rows, a.rows[1], a.rows[2], cs, a.scale,
                     a.causal ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const DkdvGeom geo = dkdv_geometry(a);
  const int items = a.B * a.H_kv * geo.first[kMaxLevels];
  const int per2 = (items + 7) / 8;
  const int64_t rows_all = a.N + a.pyr_rows;
  hipLaunchKernelGGL((pyramid_attn_bwd_dkdv_kernel<T, D>), dim3(8 * per2), dim3(256), 0, stream, q,
                     static_cast<const T*>(a.k), static_cast<const T*>(a.v), static_cast<const T*>(a.k_pyr),
                     static_cast<const T*>(a.v_pyr), a.level_map, a.lse2, a.Dr, dout, a.dkw, a.dvw, a.H, a.H_kv, a.N,
                     a.Npad, a.nqb, a.nkb, a.L, a.q_block, items, per2, a.pyr_rows, rows_all, geo, cs, a.scale,
                     a.causal ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  const int64_t chunks = (int64_t)a.B * a.H_kv * a.N * CPR;
  hipLaunchKernelGGL((bwd_unpool_kernel<T, D>), dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                     a.dkw, a.dvw, static_cast<T*>(a.dk), static_cast<T*>(a.dv), a.N, a.L, rows_all, geo, chunks);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_dtype(const BwdArgs& a, hipStream_t stream) {
  // 64-row query blocks: dq with four waves as two row groups x two key halves
  if (a.d == 128) return a.q_block == 128 ? launch_bwd_t<T, 128, 4, 1>(a, stream) : launch_bwd_t<T, 128, 4, 2>(a, stream);
  return a.q_block == 128 ? launch_bwd_t<T, 64, 4, 1>(a, stream) : launch_bwd_t<T, 64, 4, 2>(a, stream);
}

hipError_t launch_attention_bwd(const BwdArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_bwd_dtype<bf16_t>(a, stream) : launch_bwd_dtype<float>(a, stream);
}

}  // namespace psa
