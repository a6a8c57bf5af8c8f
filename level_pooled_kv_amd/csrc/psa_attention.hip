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
//  * One workgroup per (batch, head, query block) of four waves: 32 query rows each
//    for 128-row query blocks; for 64-row blocks two row groups x two key halves,
//    each wave with its own online softmax over its half of every tile, merged at
//    the end (four waves per workgroup keep two waves per SIMD).
//    Workgroup ids are remapped so that the eight XCDs each take a contiguous run
//    of query blocks of the same heads (dispatch is round-robin over XCDs), which
//    keeps the K/V rows those blocks share in one XCD's L2. Under causal use the
//    runs are made of (i, nqb-1-i) pairs of equal work, heavy halves first.
//  * The level-map row is compacted in LDS into per-level lists of block indices.
//    A hardware tile is always 64 key rows of ONE level: 1 block at level 0,
//    2 at level 1, 4 at level 2, 8 at level 3. Within a tile every key carries the
//    same ln(2^l) bias, so the bias folds into the running max at no per-logit
//    cost; only the last tile of a level (padding, ragged tail) takes a per-key
//    correction path.
//  * Tiles are double buffered in LDS with one tile of prefetch. bf16 K and V rows go
//    straight from global memory to LDS (16-byte direct loads, no registers); both
//    are stored row-major with an XOR swizzle of their 16-byte chunks.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from LDS as A, Q from registers
//    as B). In the 32x32 accumulator a lane owns one query column and 16 key rows;
//    the same registers, rounded to bf16, are the B operand of O^T = V^T P^T. Its A
//    operand (V^T) is read from row-major V with the LDS transpose read
//    (ds_read_b64_tr_b16: a 16-lane group reads a 4-key x 16-column block and each
//    lane receives the 4 keys of one column), two reads per operand, choosing the key
//    rows so the operand's k order matches the order the accumulator holds the keys
//    in. O^T also leaves each lane with one query, so the row max, row sum and
//    rescale never leave the lane pair (l, l^32).
//  * Online softmax in base 2; the running max is only raised when a row's max
//    grows by more than 2^8, which keeps every P <= 256 and skips most rescales.
#include "psa_attn_common.h"


#include <type_traits>

namespace psa {

// Waves per SIMD: two (two workgroups per CU) at d = 128; three at d = 64 with bf16 I/O,
// where the tiles and registers are small enough for three workgroups per CU (the
// 17776-token d = 64 layer: 815 -> 695 us).
template <typename T, int D, int NW>
constexpr int attn_waves_per_eu() { return D == 64 && sizeof(T) == 2 ? 3 : NW / 2; }

// KS = 1: NW waves of 32 query rows each over whole tiles. KS = 2 (64-row query blocks):
// the NW = 4 waves are 2 row groups x 2 key halves; each wave runs its own online
// softmax over its 32 keys of every tile, and the two halves' (max, sum, O) states are
// merged through LDS at the end. This keeps four waves per workgroup, hence two per
// SIMD, where two-wave workgroups would leave one (the LDS holds two per CU).
template <typename T, int D, int NW, int KS>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<T, D, NW>(), attn_waves_per_eu<T, D, NW>())))
pyramid_attn_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                        const T* __restrict__ kp, const T* __restrict__ vp,
                        const int8_t* __restrict__ level_map, T* __restrict__ o, float* __restrict__ lse,
                        int H, int H_kv, int N, int nqb, int nkb, int L, int total_items, int per_xcd,
                        int64_t pyr_rows, int rows1, int rows2, float cs /* scale * log2(e) */, int causal) {
  using C = AttnCfg<D, NW>;
  constexpr int RW = NW / KS;                    // waves per 32-key group: row groups of 32 queries
  constexpr int KB = 2 / KS;                     // 32-key halves of a tile each wave computes
  // d = 64: half the matrix work per exponential, so the softmax's VALU work counts for
  // more; there the tile max is taken only when a row's sum overflows (the 17776-token
  // d = 64 layer: 851 -> 817 us; no gain measured at d = 128, also with 64-row blocks)
  constexpr bool kSkipMax = D == 64;
  constexpr int CPR = C::kCpr, RPB = C::kRpb, BPW = C::kBpw;
  constexpr bool kDirect = sizeof(T) == 2;     // bf16: global -> LDS without registers
  // One LDS object per tile buffer: the wait-count analysis can then tell the direct
  // loads into one buffer from the operand reads of the other and does not make the
  // reads wait for the prefetch. Buffer choices are therefore compile-time (parity P).
  __shared__ __align__(16) uint16_t K0[64 * D], K1[64 * D];
  __shared__ __align__(16) uint16_t V0[64 * D], V1[64 * D];
  __shared__ float corr[2][64];
  __shared__ int ltok[2][64];                    // diagonal tiles: last token of each staged key row
  __shared__ __align__(16) int16_t blist[kMaxKvBlocks + 8];  // + 8: a tile's segment lookups stay in the array
  __shared__ uint32_t tdesc[kMaxKvBlocks + 4];   // per tile: level | list base << 2 | segs << 16 | irregular << 31
  __shared__ int s_tile[5];

  // wave index read as a wave-uniform value: every LDS destination of a direct load is then
  // formed in scalar registers (no vector-to-scalar moves per load)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  int bh, qi;
  if (causal && (nqb & 1) == 0) {
    // Causal: query block i sees about i + 1 blocks, so the pair (i, nqb-1-i) always
    // carries the same work. Each XCD takes a contiguous run of pairs (balanced work, one
    // head's K/V in one L2) and starts the heavy halves first, in decreasing order, so
    // the light halves fill the tail.
    const int ppx = per_xcd >> 1, k = bid >> 3;
    const int u = k < ppx ? k : 2 * ppx - 1 - k;
    const int pair = (bid & 7) * ppx + u;
    if (pair >= (total_items >> 1)) return;
    const int hq = nqb >> 1;
    bh = pair / hq;
    const int pi = pair - bh * hq;
    qi = k < ppx ? nqb - 1 - pi : pi;
  } else {
    const int slot = (bid & 7) * per_xcd + (bid >> 3);
    if (slot >= total_items) return;
    bh = slot / nqb;
    qi = slot - bh * nqb;
    if (causal) qi = nqb - 1 - qi;   // heavier (later) query blocks first
  }
  const int item = bh * nqb + qi;
  const int b = bh / H, h = bh - b * H;
  const int bkv = b * H_kv + h / (H / H_kv);

  // ---- compact the level-map row into level-major block lists (wave 0)
  const int8_t* lrow = level_map + (int64_t)item * nkb;   // item == (b*H + h)*nqb + qi
  const int q0 = qi * (32 * RW);
  if (wave == 0) build_tile_lists(lrow, nkb, L, N, causal ? q0 / 64 : nkb, blist, tdesc, s_tile);

  // ---- Q operand in registers: lane (row = lane%32, half = lane/32) holds d = 16c + 8*half + 0..7
  const int half = lane >> 5, l32 = lane & 31;
  const int khalf = KS == 1 ? 0 : wave / RW;        // key half of every tile
  const int my_row = q0 + 32 * (KS == 1 ? wave : wave % RW) + l32;
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
  // Retire the Q loads here: otherwise the wait-count analysis cannot prove them done
  // inside the tile loop and waits on every outstanding load (the next tile's prefetch)
  // before each QK^T product. 0x0F70 = vmcnt(0), expcnt and lgkmcnt unconstrained.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  const int T_total = __builtin_amdgcn_readfirstlane(s_tile[4]);

  const T* kh = k + (int64_t)bkv * N * D;
  const T* vh = v + (int64_t)bkv * N * D;
  const T* kph = kp ? kp + (int64_t)bkv * pyr_rows * D : nullptr;
  const T* vph = vp ? vp + (int64_t)bkv * pyr_rows * D : nullptr;
  // tile t -> level, first block-list index, valid segments, irregular flag
  auto tile_info = [&](int t) { return decode_tile(__builtin_amdgcn_readfirstlane(tdesc[t])); };
  // per-level constants: pooled rows, row offset in the pyramid, K/V base pointers
  auto level_rows = [&](int lvl) { return (N + (1 << lvl) - 1) >> lvl; };
  auto level_off = [&](int lvl) { return (lvl >= 2 ? rows1 : 0) + (lvl >= 3 ? rows2 : 0); };

  // Staging: wave w fills 1 KB blocks w*BPW .. w*BPW+BPW-1 of each tensor's tile; in a
  // block, lane i owns row RPB*blk + i/CPR and physical chunk i%CPR.
  const int st_row0 = RPB * (wave * BPW) + lane / CPR;
  const int st_pchunk = lane % CPR;
  Raw8f fk[kDirect ? 1 : BPW], fv[kDirect ? 1 : BPW];
  auto kbuf = [&](auto P) -> uint16_t* { if constexpr (P() == 0) return K0; else return K1; };
  auto vbuf = [&](auto P) -> uint16_t* { if constexpr (P() == 0) return V0; else return V1; };
  // Per-key fixups of a tile that needs them (rare: the last tile of a level, or a
  // causal diagonal tile), kept out of the common path: logit corrections of padding and
  // ragged pooled rows, and the last token of each staged key row.
  auto tile_fixups = [&](const TileInfo& ti, int buf, const int* fprow, const bool* fok) {
    if (st_pchunk != 0) return;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int row = st_row0 + RPB * i;
      if (ti.irr) corr[buf][row] = key_correction(fok[i], ti.lvl, fprow[i], N, cs);
      if (ti.diag) ltok[buf][row] = key_last_token(fok[i], ti.lvl, fprow[i], N);
    }
  };
  auto issue_tile = [&](int t, auto P) {
    constexpr int buf = P();
    const TileInfo ti = tile_info(t);
    const int lvl = ti.lvl;
    const int sh = 6 - lvl, seglen = 64 >> lvl;
    const int rows_lv = level_rows(lvl);
    const int64_t loff = (int64_t)level_off(lvl) * D;
    // wave-uniform bases of the level + 32-bit per-lane byte offsets (scalar-base addressing)
    const char* kb = reinterpret_cast<const char*>(lvl == 0 ? kh : kph + loff);
    const char* vb = reinterpret_cast<const char*>(lvl == 0 ? vh : vph + loff);
    int fx_prow[BPW];
    bool fx_ok[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int row = st_row0 + RPB * i;
      const int seg = row >> sh;
      const bool vseg = seg < ti.nseg;
      const int blk = (int)blist[ti.base + seg];     // unused (row not ok) past the valid segments
      const int prow = blk * seglen + (row & (seglen - 1));
      const bool ok = vseg && prow < rows_lv;
      const int rowel = (ok ? prow : 0) * D;
      const uint32_t koff = (uint32_t)((rowel + 8 * (st_pchunk ^ k_swz<D>(row))) * (int)sizeof(T));
      const uint32_t voff = (uint32_t)((rowel + 8 * (st_pchunk ^ v_swz<D>(row))) * (int)sizeof(T));
      if constexpr (kDirect) {
        const int blkoff = (wave * BPW + i) * 512;    // 1 KB block, in bf16 elements
        __builtin_amdgcn_global_load_lds((gbl_void*)(kb + koff), (lds_void*)(kbuf(P) + blkoff), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_void*)(vb + voff), (lds_void*)(vbuf(P) + blkoff), 16, 0, 0);
      } else {
        fk[i].load(reinterpret_cast<const float*>(kb + koff));
        fv[i].load(reinterpret_cast<const float*>(vb + voff));
      }
      fx_prow[i] = prow;
      fx_ok[i] = ok;
    }
    if (__builtin_expect(ti.irr || ti.diag, 0)) tile_fixups(ti, buf, fx_prow, fx_ok);
  };
  // Direct-load path: the byte offsets of tile t's staged rows are computed up front
  // (with the tile's logit corrections when irregular), and the loads themselves are
  // issued one at a time between the S-product MFMAs of the current tile, so no wave stalls
  // behind a burst of loads queued at the CU's load path. A wave stages 16 consecutive rows
  // of a tile, 16 w + q_i with q_i = RPB i + lane / CPR; its rows with q_i < 8 and those with
  // q_i >= 8 each lie in one segment (segments are 8 rows or more), so the block index of
  // every staged row is wave-uniform: one for the lower and one for the upper 8 rows. The
  // tile's descriptor and these two block indices are read from LDS one tile earlier
  // (prefetch_tile), so forming the offsets waits on no LDS round trip at the start of a
  // tile; a regular tile's row offset is then a scalar term plus the lane's own part (q_i
  // rows and the swizzled chunk slot), which is the same for every tile.
  static_assert(RPB * BPW == 16, "a wave stages 16 consecutive rows");
  constexpr int RB = D * (int)sizeof(T);          // bytes per K or V row
  uint32_t ck[BPW], cv[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int q = RPB * i + lane / CPR;
    ck[i] = (uint32_t)(q * RB + 8 * (st_pchunk ^ k_swz<D>(16 * wave + q)) * (int)sizeof(T));
    cv[i] = (uint32_t)(q * RB + 8 * (st_pchunk ^ v_swz<D>(16 * wave + q)) * (int)sizeof(T));
  }
  struct Stage { const char* kb; const char* vb; uint32_t koff[BPW], voff[BPW]; };
  struct Pref { uint32_t desc; int blk[2]; };
  auto prefetch_tile = [&](int t) {
    Pref pf;
    pf.desc = __builtin_amdgcn_readfirstlane(tdesc[t]);
    const TileInfo ti = decode_tile(pf.desc);
    const int sh = 6 - ti.lvl;
    // past the valid segments: unused (the rows are not ok)
    pf.blk[0] = __builtin_amdgcn_readfirstlane((int)blist[ti.base + ((16 * wave) >> sh)]);
    pf.blk[1] = __builtin_amdgcn_readfirstlane((int)blist[ti.base + ((16 * wave + 8) >> sh)]);
    return pf;
  };
  auto stage_addr = [&](const Pref& pf, auto P) {
    constexpr int buf = P();
    Stage st;
    const TileInfo ti = decode_tile(pf.desc);
    const int lvl = ti.lvl;
    const int sh = 6 - lvl, seglen = 64 >> lvl;
    const int rows_lv = level_rows(lvl);
    const int64_t loff = (int64_t)level_off(lvl) * D;
    st.kb = reinterpret_cast<const char*>(lvl == 0 ? kh : kph + loff);
    st.vb = reinterpret_cast<const char*>(lvl == 0 ? vh : vph + loff);
    if (__builtin_expect(!(ti.irr || ti.diag), 1)) {
      // a regular tile: every segment is a whole block of full pooled rows, so each staged
      // row is valid; pooled row of staged row i = U_u + q_i for its half u, with
      // U_u = (block << sh) + ((16 w + 8 u) mod seglen) - 8 u (wave-uniform). Unsigned
      // arithmetic: U_u * RB may wrap below zero, the sum with the lane part does not.
      uint32_t ub[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        ub[u] = (uint32_t)((pf.blk[u] << sh) + ((16 * wave + 8 * u) & (seglen - 1)) - 8 * u) * (uint32_t)RB;
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        st.koff[i] = ub[RPB * i >= 8 ? 1 : 0] + ck[i];
        st.voff[i] = ub[RPB * i >= 8 ? 1 : 0] + cv[i];
      }
      return st;
    }
    int fx_prow[BPW];
    bool fx_ok[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int row = st_row0 + RPB * i;
      const int seg = row >> sh;
      const bool vseg = seg < ti.nseg;
      const int prow = pf.blk[RPB * i >= 8 ? 1 : 0] * seglen + (row & (seglen - 1));
      const bool ok = vseg && prow < rows_lv;
      const int rowel = (ok ? prow : 0) * D;
      st.koff[i] = (uint32_t)((rowel + 8 * (st_pchunk ^ k_swz<D>(row))) * (int)sizeof(T));
      st.voff[i] = (uint32_t)((rowel + 8 * (st_pchunk ^ v_swz<D>(row))) * (int)sizeof(T));
      fx_prow[i] = prow;
      fx_ok[i] = ok;
    }
    tile_fixups(ti, buf, fx_prow, fx_ok);
    return st;
  };
  auto dma_k = [&](const Stage& st, int i, auto P) {
    __builtin_amdgcn_global_load_lds((gbl_void*)(st.kb + st.koff[i]), (lds_void*)(kbuf(P) + (wave * BPW + i) * 512), 16, 0, 0);
  };
  auto dma_v = [&](const Stage& st, int i, auto P) {
    __builtin_amdgcn_global_load_lds((gbl_void*)(st.vb + st.voff[i]), (lds_void*)(vbuf(P) + (wave * BPW + i) * 512), 16, 0, 0);
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

  f32x16 oacc[C::kDt];
#pragma unroll
  for (int t = 0; t < C::kDt; ++t)
#pragma unroll
    for (int x = 0; x < 16; ++x) oacc[t][x] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if (T_total > 0) {
    issue_tile(0, P0{});
    commit_tile(P0{});
  }
  // descriptor of the tile being computed, and the prefetched staging of the next one
  uint32_t dcur = T_total > 0 ? __builtin_amdgcn_readfirstlane(tdesc[0]) : 0u;
  Pref pf{};
  if (kDirect && T_total > 0) pf = prefetch_tile(min(1, T_total - 1));
  __syncthreads();

  // V operand addressing for ds_read_b64_tr_b16: in 16-lane group G, lane 4m+q points at
  // key row (16c + 8j + 4*(G/2) + m), columns 32tt + 16*(G%2) + 4q .. +3; the group then
  // holds, per lane, 4 consecutive keys of one d column.
  const int trg = lane >> 4, trs = lane & 15;
  const int tr_row = 4 * (trg >> 1) + (trs >> 2);
  const int tr_col = 16 * (trg & 1) + 4 * (trs & 3);
  // byte offset of the K operand read of chunk c: row l32 of the key half, 16-byte chunk
  // (2c + half) ^ swizzle
  int kro[C::kQc];
#pragma unroll
  for (int c = 0; c < C::kQc; ++c) kro[c] = (l32 * D + (((2 * c + half) ^ k_swz<D>(l32)) * 8)) * 2;   // bytes

  // tile t (t % 2 == P()): prefetch tile t+1 into the other buffers, then compute t
  auto body = [&](int t, auto P) {
    constexpr int buf = P();
    using PN = std::integral_constant<int, 1 - P()>;
    // the next tile's staging (past the last tile: a reload of the last tile into the
    // idle buffers, so the interleaved loads need no branch)
    Stage st{};
    if constexpr (kDirect) st = stage_addr(pf, PN{});
    else if (t + 1 < T_total) issue_tile(t + 1, PN{});
    const uint32_t dnext = kDirect ? pf.desc : 0u;
    // the next tile's K and V loads go out one per SK S-product MFMAs, K first: issued
    // early, they have the softmax and the P.V products to land before the tile's wait
    constexpr int SK = KB * C::kQc / (2 * BPW);
    // the compiler's interleaving of LDS reads with the matrix ops of this region
    // (about 1% on the 32760-token layer, interleaved A/B)
    __builtin_amdgcn_iglp_opt(0);
    const TileInfo ti = kDirect ? decode_tile(dcur) : tile_info(t);
    const int lvl = ti.lvl;
    const bool irr = ti.irr;
    const uint16_t* Kb = kbuf(P);
    const uint16_t* Vb = vbuf(P);

    // S^T = K Q^T: the wave's 32-key halves (kb + KB khalf of the tile). The lane offsets of
    // the K operand reads do not change from tile to tile (the swizzle depends on the row mod
    // 16 only; the key half and the buffer are immediate offsets); an empty asm statement
    // keeps them in registers instead of recomputing them every tile.
#pragma unroll
    for (int c = 0; c < C::kQc; ++c) asm volatile("" : "+v"(kro[c]));
    f32x16 sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int x = 0; x < 16; ++x) sacc[kb][x] = 0.f;
      const uint16_t* kr_l = Kb + 32 * (kb + KB * khalf) * D;
#pragma unroll
      for (int c = 0; c < C::kQc; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(kr_l) + kro[c]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], sacc[kb], 0, 0, 0);
        if constexpr (kDirect) {
          const int j = kb * C::kQc + c;
          if ((j + 1) % SK == 0) {
            const int u = j / SK;
            if (u < BPW) dma_k(st, u, PN{});
            else dma_v(st, u - BPW, PN{});
          }
        }
      }
    }
    // staging of tile t+2 (the last tile again past the end), read while the S products run
    if constexpr (kDirect) pf = prefetch_tile(min(t + 2, T_total - 1));
    if (irr) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x)
          sacc[kb][x] += corr[buf][32 * (kb + KB * khalf) + 8 * (x >> 2) + 4 * half + (x & 3)];
    }
    if (ti.diag) {   // causal: a key is seen only by rows at or after its last token
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x)
          if (ltok[buf][32 * (kb + KB * khalf) + 8 * (x >> 2) + 4 * half + (x & 3)] > my_row) sacc[kb][x] = -INFINITY;
    }

    // online softmax (base 2); this tile's keys all carry bias lvl
    bf16x8 preg[2 * KB];
    float lsum = 0.f;
    const float lvlf = (float)lvl;
    if constexpr (kSkipMax) {
      // the exponentials against the running max first; the tile max and a rescale only
      // where a row's partial sum reached 2^64 or is not a number (scores far above the
      // running max, or no running max yet), which then recomputes them
      {
        const float moff = lvlf - m_run;
#pragma unroll
        for (int c = 0; c < 2 * KB; ++c) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[c >> 1][8 * (c & 1) + e], cs, moff));
            lsum += p;
            preg[c][e] = (__bf16)p;
          }
        }
      }
      if (__ballot(!(lsum < 0x1p64f))) {
        float tmax = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int x = 0; x < 16; ++x) tmax = fmaxf(tmax, sacc[kb][x]);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
          tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float mn = fmaxf(m_run, fmaf(tmax, cs, lvlf));
        const float alpha = mn == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - mn);
        l_run *= alpha;
#pragma unroll
        for (int tt = 0; tt < C::kDt; ++tt)
#pragma unroll
          for (int x = 0; x < 16; ++x) oacc[tt][x] *= alpha;
        m_run = mn;
        const float moff = m_run == -INFINITY ? 0.f : lvlf - m_run;
        lsum = 0.f;
#pragma unroll
        for (int c = 0; c < 2 * KB; ++c) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[c >> 1][8 * (c & 1) + e], cs, moff));
            lsum += p;
            preg[c][e] = (__bf16)p;
          }
        }
      }
    } else {
      // tile max with the IEEE maximum (v_maximum3_f32), which needs no quieting of its
      // operands; the scores hold no NaN (masked ones are -inf)
      float tmax = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x) tmax = __builtin_elementwise_maximum(tmax, sacc[kb][x]);
      {   // lanes l and l^32 hold the two key halves of one query
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
        tmax = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float mt = fmaf(tmax, cs, lvlf);
      const bool upd = mt > m_run + 8.0f;
      if (__ballot(upd)) {
        // lanes that keep their max scale by 1 (also when it is still -inf after causal masking)
        const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int tt = 0; tt < C::kDt; ++tt)
#pragma unroll
          for (int x = 0; x < 16; ++x) oacc[tt][x] *= alpha;
        m_run = upd ? mt : m_run;
      }
      // a row that has seen no key yet keeps p = 0 (its logits here are all -inf: causal
      // masking, or with split keys a half tile of only padding rows)
      float moff = lvlf - m_run;
      if (KS == 2 || ti.diag) moff = m_run == -INFINITY ? 0.f : moff;
#pragma unroll
      for (int c = 0; c < 2 * KB; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[c >> 1][8 * (c & 1) + e], cs, moff));
          lsum += p;
          preg[c][e] = (__bf16)p;
        }
      }
    }
    l_run += lsum;

    // O^T += V^T P^T; the A operand is fetched transposed from row-major V
#pragma unroll
    for (int c = 0; c < 2 * KB; ++c) {
#pragma unroll
      for (int tt = 0; tt < C::kDt; ++tt) {
        bf16x4 part[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row = 16 * (c + 2 * KB * khalf) + 8 * j + tr_row;
          const int col = 32 * tt + tr_col;
          const int chunk = (col >> 3) ^ v_swz<D>(row);
          part[j] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)(Vb + row * D + chunk * 8 + (col & 7)));
        }
        const bf16x8 a = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, preg[c], oacc[tt], 0, 0, 0);

      }
    }

    if (t + 1 < T_total) commit_tile(PN{});
    if constexpr (kDirect) dcur = dnext;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // this wave's loads of tile t+1 have landed
    __syncthreads();
  };
  for (int t = 0; t < T_total; t += 2) {
    body(t, P0{});
    if (t + 1 < T_total) body(t + 1, P1{});
  }

  if constexpr (KS == 2) {
    // merge the two key halves' softmax states of each query: the khalf = 1 waves hand
    // (max, partial sums, O^T) to the khalf = 0 waves of the same rows through LDS (the
    // tile buffers are idle: the loop's last barrier follows its last loads)
    static_assert(RW <= 4, "one tile buffer per row group");
    const int rw = wave % RW;
    float* xo = reinterpret_cast<float*>(rw == 0 ? K0 : rw == 1 ? K1 : rw == 2 ? V0 : V1);   // [tt][x][lane]
    float* xs = reinterpret_cast<float*>(blist) + rw * 128;     // [m, l][lane]
    if (khalf == 1) {
#pragma unroll
      for (int tt = 0; tt < C::kDt; ++tt)
#pragma unroll
        for (int x = 0; x < 16; ++x) xo[(tt * 16 + x) * 64 + lane] = oacc[tt][x];
      xs[lane] = m_run;
      xs[64 + lane] = l_run;
    }
    __syncthreads();
    if (khalf == 0) {
      const float m1 = xs[lane], l1 = xs[64 + lane];
      const float m = fmaxf(m_run, m1);
      const float a0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
      const float a1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
      l_run = l_run * a0 + l1 * a1;
#pragma unroll
      for (int tt = 0; tt < C::kDt; ++tt)
#pragma unroll
        for (int x = 0; x < 16; ++x) oacc[tt][x] = oacc[tt][x] * a0 + xo[(tt * 16 + x) * 64 + lane] * a1;
      m_run = m;
    }
  }

  // ---- normalise and write O (and LSE)
  const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l_tot = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if constexpr (sizeof(T) == 2) {
    // bf16: a wave's 32 output rows go through LDS (the idle tile buffers, 16-byte chunks
    // XOR-swizzled by row) and leave as whole rows, four 256-byte rows per 16-byte store
    // instruction, instead of 8-byte pieces of 32 rows per instruction
    constexpr int CH = D / 8;                   // 16-byte chunks per row
    uint16_t* ost = KS == 1 ? (wave == 0 ? K0 : wave == 1 ? K1 : wave == 2 ? V0 : V1)
                            : (wave % RW == 0 ? V0 : V1);   // the key-half merge used K0, K1
    if (khalf == 0) {
#pragma unroll
      for (int tt = 0; tt < C::kDt; ++tt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int pc = (4 * tt + g4) ^ (l32 & (CH - 1));
          const float y0 = oacc[tt][4 * g4] * inv, y1 = oacc[tt][4 * g4 + 1] * inv;
          const float y2 = oacc[tt][4 * g4 + 2] * inv, y3 = oacc[tt][4 * g4 + 3] * inv;
          *reinterpret_cast<uint2*>(ost + l32 * D + pc * 8 + 4 * half) =
              make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
        }
      }
    }
    __syncthreads();
    if (khalf == 0) {
      const int rbase = q0 + 32 * (KS == 1 ? wave : wave % RW);
      T* obase = o + ((int64_t)bh * N + rbase) * D;
#pragma unroll
      for (int i = 0; i < 32 * CH / 64; ++i) {
        const int idx = 64 * i + lane, r = idx / CH, c = idx % CH;
        if (rbase + r < N) st128(obase + r * D + c * 8, ld128(ost + r * D + ((c ^ (r & (CH - 1))) * 8)));
      }
      if (lse && half == 0 && my_row < N)
        lse[(int64_t)bh * N + my_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    }
  } else if (my_row < N && khalf == 0) {
    T* orow = o + ((int64_t)bh * N + my_row) * D;
#pragma unroll
    for (int tt = 0; tt < C::kDt; ++tt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * tt + 8 * g4 + 4 * half;
        const float y0 = oacc[tt][4 * g4] * inv, y1 = oacc[tt][4 * g4 + 1] * inv;
        const float y2 = oacc[tt][4 * g4 + 2] * inv, y3 = oacc[tt][4 * g4 + 3] * inv;
        *reinterpret_cast<float4*>(orow + d) = make_float4(y0, y1, y2, y3);
      }
    }
    if (lse && half == 0)
      lse[(int64_t)bh * N + my_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  }
}

template <typename T, int D, int NW, int KS>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  const int total = a.B * a.H * a.nqb;
  // slots per XCD; causal with an even nqb hands out whole (i, nqb-1-i) pairs
  const int per = a.causal && a.nqb % 2 == 0 ? 2 * ((total / 2 + 7) / 8) : (total + 7) / 8;
  const float cs = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((pyramid_attn_fwd_kernel<T, D, NW, KS>), dim3(8 * per), dim3(NW * 64), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                     static_cast<const T*>(a.k_pyr), static_cast<const T*>(a.v_pyr), a.level_map,
                     static_cast<T*>(a.o), a.lse, a.H, a.H_kv, a.N, a.nqb, a.nkb, a.L, total, per,
                     a.pyr_rows, a.rows[1], a.rows[2], cs, a.causal ? 1 : 0);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_attn_dtype(const AttnArgs& a, hipStream_t stream) {
  // 64-row query blocks: four waves as two row groups x two key halves
  if (a.d == 128) {
    return a.q_block == 128 ? launch_attn_t<T, 128, 4, 1>(a, stream) : launch_attn_t<T, 128, 4, 2>(a, stream);
  }
  return a.q_block == 128 ? launch_attn_t<T, 64, 4, 1>(a, stream) : launch_attn_t<T, 64, 4, 2>(a, stream);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t stream) {
  return a.bf16 ? launch_attn_dtype<bf16_t>(a, stream) : launch_attn_dtype<float>(a, stream);
}

}  // namespace psa
