// Step 3 of the PSA forward path on gfx950, two-group ("ping-pong") attention kernel.
//
// Computes exactly what pyramid_attn_fwd_kernel computes (one softmax over the
// mixed-resolution keys a query block retains, each pooled key weighted by its pool
// size; "PSA: Pyramid Sparse Attention ...": chatpaper.ai abstract, top168.com
// three-components paragraph) with a different schedule, built so that the matrix
// cores and the vector ALUs of every SIMD work at the same time:
//
//  * One workgroup of two groups of NW waves per query block. Both groups hold the
//    block's Q rows; group g takes the block's tiles g, g+2, g+4, ... (split over the
//    key sequence) with its own LDS buffers, running max, row sums and O^T
//    accumulators. At the end group 1 hands (max, sums, O^T) to group 0 through LDS
//    and group 0 merges the two partial softmaxes and writes O.
//  * Execution alternates two phases separated by workgroup barriers. In a GEMM
//    phase a group issues the QK^T products of its tile i and the PV products of its
//    tile i-1 (32 MFMAs per wave at d = 128); in a softmax phase it turns tile i's
//    scores into bf16 probabilities and starts the direct global->LDS loads of later
//    tiles. The groups are half a step apart, so each SIMD holds one wave of each
//    group and always has one MFMA-phase wave and one VALU-phase wave.
//  * Buffers per group: K of tile i lives in K buffer i%2, V of tile i in V buffer
//    i%2. The softmax phase of tile i loads K(i+2) and V(i+1); each buffer is
//    overwritten only after the barrier that follows its last reader, and a wave
//    waits only for the loads of the previous softmax phase before a barrier.
//  * Tile packing, LDS layouts, the V^T operand fetch (LDS transpose reads), the
//    base-2 online softmax with its 2^8 lazy-rescale threshold and the per-key
//    corrections of irregular tiles are those of the single-group kernel.
#include "psa_attn_common.h"

#include <type_traits>

namespace psa {

template <typename T, int D, int NW>
__global__ void __launch_bounds__(2 * NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
pyramid_attn_fwd_pp_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                           const T* __restrict__ kp, const T* __restrict__ vp,
                           const int8_t* __restrict__ level_map, T* __restrict__ o, float* __restrict__ lse,
                           int H, int H_kv, int N, int nqb, int nkb, int L, int total_items, int per_xcd,
                           int64_t pyr_rows, int rows1, int rows2, float cs /* scale * log2(e) */) {
  using C = AttnCfg<D, NW>;
  constexpr int CPR = C::kCpr, RPB = C::kRpb, BPW = C::kBpw;
  constexpr bool kDirect = sizeof(T) == 2;     // bf16: global -> LDS without registers
  constexpr int TILE = 64 * D;                 // bf16 elements of one tile of one tensor
  // One LDS object per (tensor, group, buffer): the wait-count analysis can then tell
  // the direct loads into one buffer from operand reads of another and does not make
  // the reads wait for the prefetch. Group and buffer choices are compile-time.
  __shared__ __align__(16) uint16_t K00[TILE], K01[TILE], K10[TILE], K11[TILE];
  __shared__ __align__(16) uint16_t V00[TILE], V01[TILE], V10[TILE], V11[TILE];
  __shared__ float corr[2][2][64];
  __shared__ int16_t blist[kMaxKvBlocks];
  __shared__ uint32_t tdesc[kMaxKvBlocks + 4];
  __shared__ int s_tile[5];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave / NW, gw = wave - grp * NW;
  const int bid = blockIdx.x;
  const int item = (bid & 7) * per_xcd + (bid >> 3);
  if (item >= total_items) return;
  const int bh = item / nqb, qi = item - bh * nqb;
  const int b = bh / H, h = bh - b * H;
  const int bkv = b * H_kv + h / (H / H_kv);

  const int8_t* lrow = level_map + (int64_t)item * nkb;   // item == (b*H + h)*nqb + qi
  if (wave == 0) build_tile_lists(lrow, nkb, L, N, blist, tdesc, s_tile);

  // ---- Q operand in registers: lane (row = lane%32, half = lane/32) holds d = 16c + 8*half + 0..7
  const int half = lane >> 5, l32 = lane & 31;
  const int my_row = qi * (32 * NW) + 32 * gw + l32;
  bf16x8 qreg[C::kQc];
  {
    const T* qrow = q + ((int64_t)bh * N + min(my_row, N - 1)) * D;
#pragma unroll
    for (int c = 0; c < C::kQc; ++c) {
      U128 u;
      if constexpr (kDirect) {
        u = ld128(qrow + 16 * c + 8 * half);
      } else {
        Raw8f rw;
        rw.load(reinterpret_cast<const float*>(qrow) + 16 * c + 8 * half);
        u = rw.bf16();
      }
      if (my_row >= N) u = U128{{0u, 0u, 0u, 0u}};
      qreg[c] = __builtin_bit_cast(bf16x8, make_uint4(u.w[0], u.w[1], u.w[2], u.w[3]));
    }
  }
  // Retire the Q loads here so the wait-count analysis does not wait on later
  // prefetches inside the tile loop (0x0F70 = vmcnt(0)).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  const int T_total = __builtin_amdgcn_readfirstlane(s_tile[4]);
  const int n_iter = ((T_total + 1) >> 1) + 1;       // same trip count (and barriers) for both groups

  const T* kh = k + (int64_t)bkv * N * D;
  const T* vh = v + (int64_t)bkv * N * D;
  const T* kph = kp ? kp + (int64_t)bkv * pyr_rows * D : nullptr;
  const T* vph = vp ? vp + (int64_t)bkv * pyr_rows * D : nullptr;
  auto level_rows = [&](int lvl) { return (N + (1 << lvl) - 1) >> lvl; };
  auto level_off = [&](int lvl) { return (lvl >= 2 ? rows1 : 0) + (lvl >= 3 ? rows2 : 0); };

  // Staging: wave gw of the group fills 1 KB blocks gw*BPW .. gw*BPW+BPW-1 of each of
  // the group's tiles; in a block, lane i owns row RPB*blk + i/CPR, physical chunk i%CPR.
  const int st_row0 = RPB * (gw * BPW) + lane / CPR;
  const int st_pchunk = lane % CPR;
  Raw8f fk[kDirect ? 1 : BPW], fv[kDirect ? 1 : BPW];

  f32x16 oacc[C::kDt];
#pragma unroll
  for (int t = 0; t < C::kDt; ++t)
#pragma unroll
    for (int x = 0; x < 16; ++x) oacc[t][x] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 sacc[2];
  bf16x8 preg[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) preg[c][e] = (__bf16)0.0f;

  // V operand addressing for ds_read_b64_tr_b16 (see the single-group kernel)
  const int trg = lane >> 4, trs = lane & 15;
  const int tr_row = 4 * (trg >> 1) + (trs >> 2);
  const int tr_col = 16 * (trg & 1) + 4 * (trs & 3);

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto kbuf = [&](auto G, auto P) -> uint16_t* {
    if constexpr (G() == 0) { if constexpr (P() == 0) return K00; else return K01; }
    else { if constexpr (P() == 0) return K10; else return K11; }
  };
  auto vbuf = [&](auto G, auto P) -> uint16_t* {
    if constexpr (G() == 0) { if constexpr (P() == 0) return V00; else return V01; }
    else { if constexpr (P() == 0) return V10; else return V11; }
  };

  // GEMM phase i: S(i) = K(i) Q^T and O^T += V(i-1)^T P(i-1)^T. All K operands are read
  // up front; each QK^T MFMA is followed by the two transposing reads of one V operand
  // (which can take the registers the MFMA just consumed), then the PV MFMAs rotate
  // over the O^T accumulators so no two consecutive MFMAs depend on each other.
  constexpr int NK = 2 * C::kQc, NV = 4 * C::kDt;      // operands per product
  static_assert(NK == NV, "phase layout pairs one V operand with each QK^T MFMA");
  // (each LDS address is the buffer plus ONE integer offset, so the compiler can trace
  // every access to its buffer and keep the per-buffer alias information)
  auto k_operand = [&](const uint16_t* Kb, int j) {     // j = 2c + kb
    const int c = j >> 1, kb = j & 1;
    const int off = (32 * kb + l32) * D + (((2 * c + half) ^ k_swz<D>(l32)) * 8);
    return *reinterpret_cast<const bf16x8*>(&Kb[off]);
  };
  auto v_operand = [&](const uint16_t* Vb, int j) {     // j = c * kDt + tt
    const int c = j / C::kDt, tt = j % C::kDt;
    bf16x4 part[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int row = 16 * c + 8 * jj + tr_row;
      const int col = 32 * tt + tr_col;
      const int off = row * D + (((col >> 3) ^ v_swz<D>(row)) * 8) + (col & 7);
      part[jj] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)&Vb[off]);
    }
    return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto qk_mfma = [&](const bf16x8& a, int j) {
    const int c = j >> 1, kb = j & 1;
    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], c == 0 ? f32x16{} : sacc[kb], 0, 0, 0);
  };
  auto pv_mfma = [&](const bf16x8& a, int j) {
    const int c = j / C::kDt, tt = j % C::kDt;
    oacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, preg[c], oacc[tt], 0, 0, 0);
  };

  // Everything below runs with the group G as a compile-time constant.
  auto run = [&](auto G) {
    constexpr int g = G();
    const int T_g = (T_total + 1 - g) >> 1;            // tiles g, g+2, ... of this block
    auto tile_info = [&](int i) { return decode_tile(__builtin_amdgcn_readfirstlane(tdesc[2 * i + g])); };

    // Start moving K (is_v false) or V of the group's tile i into buffer P; issuing V also
    // writes the tile's per-key logit corrections when it is irregular.
    auto issue = [&](bool is_v, int i, auto P) {
      const TileInfo ti = tile_info(i);
      const int lvl = ti.lvl;
      const int sh = 6 - lvl, seglen = 64 >> lvl;
      const int rows_lv = level_rows(lvl);
      // wave-uniform base of the level + 32-bit per-lane byte offset (scalar-base addressing)
      const char* base = reinterpret_cast<const char*>(
          is_v ? (lvl == 0 ? vh : vph + (int64_t)level_off(lvl) * D)
               : (lvl == 0 ? kh : kph + (int64_t)level_off(lvl) * D));
#pragma unroll
      for (int r = 0; r < BPW; ++r) {
        const int row = st_row0 + RPB * r;
        const int seg = row >> sh;
        const bool vseg = seg < ti.nseg;
        const int blk = vseg ? (int)blist[ti.base + seg] : 0;
        const int prow = blk * seglen + (row & (seglen - 1));
        const bool ok = vseg && prow < rows_lv;
        const uint32_t boff = (uint32_t)(((ok ? prow : 0) * D + 8 * (st_pchunk ^ (is_v ? v_swz<D>(row) : k_swz<D>(row)))) *
                                         (int)sizeof(T));
        if constexpr (kDirect) {
          const int off = (gw * BPW + r) * 512;
          dma16(base, boff, (is_v ? vbuf(G, P) : kbuf(G, P)) + off);
        } else {
          (is_v ? fv : fk)[r].load(reinterpret_cast<const float*>(base + boff));
        }
        if (is_v && ti.irr && st_pchunk == 0) corr[g][P()][row] = key_correction(ok, lvl, prow, N, cs);
      }
    };
    // float32 path: convert the staged registers and write them to LDS.
    auto commit = [&](bool is_v, auto P) {
      if constexpr (!kDirect) {
        uint16_t* dst = is_v ? vbuf(G, P) : kbuf(G, P);
#pragma unroll
        for (int r = 0; r < BPW; ++r) st128(dst + (gw * BPW + r) * 512 + lane * 8, (is_v ? fv : fk)[r].bf16());
      }
    };

    // One code path for every GEMM phase 0..T_g (separate QK-only / PV-only variants of
    // the same LDS reads would let the optimizer merge them and drop the per-buffer alias
    // scopes the load-tracking relies on). Phase 0 multiplies a dummy V tile by P = 0;
    // the last phase's QK^T result is never used.
    auto gemm = [&](int i, auto P) {                   // P = i % 2
      using PN = std::integral_constant<int, 1 - P()>;
      if (T_g == 0 || i > T_g) return;
      const uint16_t* Kb = kbuf(G, P);
      const uint16_t* Vb = vbuf(G, PN{});
      // rolling pipeline: K operands PF steps ahead, each PV MFMA LAG steps behind the
      // read of its V operand; QK^T and PV MFMAs alternate
      constexpr int PF = 4, LAG = 3;
      bf16x8 kop[NK], vop[NV];
#pragma unroll
      for (int j = 0; j < PF; ++j) kop[j] = k_operand(Kb, j);
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        qk_mfma(kop[j], j);
        if (j + PF < NK) kop[j + PF] = k_operand(Kb, j + PF);
        vop[j] = v_operand(Vb, j);
        if (j >= LAG) pv_mfma(vop[j - LAG], j - LAG);
      }
#pragma unroll
      for (int j = NK - LAG; j < NK; ++j) pv_mfma(vop[j], j);
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);                  // K operand reads
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // QK^T MFMA
        if (j + PF < NK) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // next K + V reads
        else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);            // V reads
        if (j >= LAG) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // PV MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, LAG, 0);                 // last PV MFMAs
    };

    // Softmax phase i (P = i % 2): P(i) from S(i), then the loads of K(i+2) and V(i+1),
    // then wait for the loads the previous softmax phase started.
    auto softmax = [&](int i, auto P) {
      using PN = std::integral_constant<int, 1 - P()>;
      if (i < 0) return;
      if (i < T_g) {
        const TileInfo ti = tile_info(i);
        if (ti.irr) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int x = 0; x < 16; ++x)
              sacc[kb][x] += corr[g][P()][32 * kb + 8 * (x >> 2) + 4 * half + (x & 3)];
        }
        float tmax = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int x = 0; x < 16; ++x) tmax = fmaxf(tmax, sacc[kb][x]);
        {   // lanes l and l^32 hold the two key halves of one query
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
          tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float lvlf = (float)ti.lvl;          // every key of the tile carries bias log2(2^lvl)
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
      }
      const bool nk = i + 2 < T_g, nv = i + 1 < T_g;
      if (nk) {
        issue(false, i + 2, P);
        commit(false, P);
      }
      if (nv) {
        issue(true, i + 1, PN{});
        commit(true, PN{});
      }
      if constexpr (kDirect) {
        // wait until only this phase's loads may still be in flight
        if (nk && nv) wait_vmcnt<2 * BPW>();
        else if (nk || nv) wait_vmcnt<BPW>();
        else wait_vmcnt<0>();
      }
    };

    // prologue: K(0), V(0), K(1) of this group, and V(0) once more into V buffer 1 as the
    // finite dummy tile phase 0 multiplies by P = 0
    if (T_g > 0) {
      issue(false, 0, I0{});
      commit(false, I0{});
      issue(true, 0, I0{});
      commit(true, I0{});
      issue(true, 0, I1{});
      commit(true, I1{});
    }
    if (T_g > 1) {
      issue(false, 1, I1{});
      commit(false, I1{});
    }
    // a barrier whose fence the compiler drains itself: the tile loop then starts from a
    // state with no load in flight that it must assume aliases an operand buffer
    __syncthreads();

    // group 0 runs GEMM(i) then softmax(i); group 1 runs softmax(i-1) then GEMM(i).
    // The barriers leave the prefetch of later tiles in flight.
    auto iteration = [&](int i, auto P) {
      using PN = std::integral_constant<int, 1 - P()>;
      if constexpr (g == 0) gemm(i, P); else softmax(i - 1, PN{});
      lds_barrier();
      if constexpr (g == 0) softmax(i, P); else gemm(i, P);
      lds_barrier();
    };
    for (int i = 0; i < n_iter; i += 2) {
      iteration(i, I0{});
      if (i + 1 < n_iter) iteration(i + 1, I1{});
    }
  };
  if (grp == 0) run(I0{}); else run(I1{});

  // ---- merge the two groups' partial softmaxes (no load is in flight any more). Group 1
  // hands its max and row sums over through V00, then its O^T in rounds through K00 (one
  // LDS array each, addressed directly); group 0 merges each round and writes O.
  __syncthreads();
  float* xm = reinterpret_cast<float*>(V00);           // [NW][64] max, then [NW][64] sums
  if (grp == 1) {
    xm[gw * 64 + lane] = m_run;
    xm[(NW + gw) * 64 + lane] = l_run;
  }
  __syncthreads();
  float a0 = 0.f, a1 = 0.f, inv = 0.f, m = -INFINITY, l_tot = 0.f;
  if (grp == 0) {
    const float m1 = xm[gw * 64 + lane], l1 = xm[(NW + gw) * 64 + lane];
    m = fmaxf(m_run, m1);
    a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
    a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
    const float lpart = a0 * l_run + a1 * l1;
    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lpart), __float_as_uint(lpart), false, false);
    l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  }
  constexpr int NX = C::kDt * 4;                       // float4 slots of a lane's O^T (slot = 4 tt + g4)
  constexpr int SPR = NX < (TILE * 2) / (NW * 64 * 16) ? NX : (TILE * 2) / (NW * 64 * 16);   // slots per round
  float4* x4 = reinterpret_cast<float4*>(K00);         // [SPR][NW][64]
  T* orow = o + ((int64_t)bh * N + min(my_row, N - 1)) * D;
#pragma unroll
  for (int r0 = 0; r0 < NX; r0 += SPR) {
    if (grp == 1) {
#pragma unroll
      for (int x = r0; x < r0 + SPR && x < NX; ++x) {
        const int tt = x >> 2, g4 = x & 3;
        x4[((x - r0) * NW + gw) * 64 + lane] =
            make_float4(oacc[tt][4 * g4], oacc[tt][4 * g4 + 1], oacc[tt][4 * g4 + 2], oacc[tt][4 * g4 + 3]);
      }
    }
    __syncthreads();
    if (grp == 0 && my_row < N) {
#pragma unroll
      for (int x = r0; x < r0 + SPR && x < NX; ++x) {
        const int tt = x >> 2, g4 = x & 3;
        const float4 y1 = x4[((x - r0) * NW + gw) * 64 + lane];
        const int d = 32 * tt + 8 * g4 + 4 * half;
        const float z0 = (a0 * oacc[tt][4 * g4] + a1 * y1.x) * inv;
        const float z1 = (a0 * oacc[tt][4 * g4 + 1] + a1 * y1.y) * inv;
        const float z2 = (a0 * oacc[tt][4 * g4 + 2] + a1 * y1.z) * inv;
        const float z3 = (a0 * oacc[tt][4 * g4 + 3] + a1 * y1.w) * inv;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(z0, z1), pack_bf16x2(z2, z3));
        } else {
          *reinterpret_cast<float4*>(orow + d) = make_float4(z0, z1, z2, z3);
        }
      }
    }
    __syncthreads();
  }
  if (grp == 0 && my_row < N && lse && half == 0)
    lse[(int64_t)bh * N + my_row] = l_tot > 0.f ? (m + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
}

template <typename T, int D, int NW>
static hipError_t launch_pp_t(const AttnArgs& a, hipStream_t stream) {
  const int total = a.B * a.H * a.nqb;
  const int per = (total + 7) / 8;
  const float cs = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((pyramid_attn_fwd_pp_kernel<T, D, NW>), dim3(8 * per), dim3(2 * NW * 64), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                     static_cast<const T*>(a.k_pyr), static_cast<const T*>(a.v_pyr), a.level_map,
                     static_cast<T*>(a.o), a.lse, a.H, a.H_kv, a.N, a.nqb, a.nkb, a.L, total, per,
                     a.pyr_rows, a.rows[1], a.rows[2], cs);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_pp_dtype(const AttnArgs& a, hipStream_t stream) {
  if (a.d == 128) {
    return a.q_block == 128 ? launch_pp_t<T, 128, 4>(a, stream) : launch_pp_t<T, 128, 2>(a, stream);
  }
  return a.q_block == 128 ? launch_pp_t<T, 64, 4>(a, stream) : launch_pp_t<T, 64, 2>(a, stream);
}

hipError_t launch_attention_pp(const AttnArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_pp_dtype<bf16_t>(a, stream) : launch_pp_dtype<float>(a, stream);
}

}  // namespace psa
