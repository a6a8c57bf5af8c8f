// Host-side launch descriptions passed from the C ABI layer to each step's launcher.
// Every field has already been validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psa {

constexpr int kKvBlock = 64;       // tokens per KV block
constexpr int kMaxLevels = 4;      // levels 0..3: pool factors 1, 2, 4, 8
constexpr int kMaxKvBlocks = 2048; // per sequence (LDS capacity of the mask sort and the attention block lists)

struct PyramidArgs {
  const void* k; const void* v; void* k_pyr; void* v_pyr; float* k_bar;
  float* k_sim;                  // nullable: [B, H_kv, nkb, L-1] key similarity per pooled level
  int B, H_kv, N, d, nkb, L;
  bool bf16;
  int64_t pyr_rows;              // rows of the concatenated pyramid
  int off[kMaxLevels];           // row offset of level l (l >= 1) in the pyramid
};

struct MaskArgs {
  const void* q; const float* k_bar; int8_t* level_map; float* cmass;
  float* qbar;                   // workspace: [B, H, nqb, d] mean queries
  float* z;                      // workspace: [B, H, nqb, mask_score_stride(nkb)] block scores
  uint8_t* need_exact;           // workspace: [B, H, nqb] rows the bucket pass left to the exact pass
  int B, H, H_kv, N, d, q_block, nqb, nkb, L, n_dense_prefix;
  bool bf16;
  float scale;
  float tau[kMaxLevels];
  bool ranked;                   // level by rank: rank < floor(frac[l] * visible blocks) instead of C < tau[l]
  double frac[kMaxLevels];       // cumulative block fractions of the ranked rule
  bool causal;                   // rank only the blocks a query block can see (see psa.h)
};

// Kernel argument: the ranked rule's cumulative fractions (double, as the host gives them).
struct RankFractions { double f[kMaxLevels]; };

struct AttnArgs {
  const void* q; const void* k; const void* v; const void* k_pyr; const void* v_pyr;
  const int8_t* level_map; void* o; float* lse;
  int B, H, H_kv, N, d, q_block, nqb, nkb, L;
  bool bf16;
  bool causal;                   // row r sees a pooled key only if all its tokens are <= r
  float scale;
  int64_t pyr_rows;
  int off[kMaxLevels];           // row offset of level l (l >= 1) in the pyramid
  int rows[kMaxLevels];          // ceil(N / 2^l)
};

struct CapArgs {
  int8_t* level_map; const float* k_sim; float threshold;
  int B, H, H_kv, nqb, nkb, L;
};

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* k_pyr; const void* v_pyr;
  const int8_t* level_map; const void* o; const float* lse; const void* dout;
  void* dq; void* dk; void* dv;
  float* lse2;                   // workspace: [B, H, Npad] lse in base 2 (+inf: no key, or padding)
  float* Dr;                     // workspace: [B, H, Npad] row dots <dO, O> (0 on padding)
  int Npad;                      // N rounded up to a multiple of 64
  float* dkw; float* dvw;        // workspace: [B, H_kv, N + pyr_rows, d] float32 per-level pooled gradients
  int B, H, H_kv, N, d, q_block, nqb, nkb, L;
  bool bf16;
  bool causal;
  float scale;
  int64_t pyr_rows;
  int off[kMaxLevels];           // row offset of level l (l >= 1) in the pyramid
  int rows[kMaxLevels];          // ceil(N / 2^l)
};

hipError_t launch_pyramid(const PyramidArgs& a, hipStream_t stream);
hipError_t launch_attention_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_similarity_cap(const CapArgs& a, hipStream_t stream);
hipError_t launch_mask(const MaskArgs& a, hipStream_t stream);
// Padded score-row length of the mask workspace: up to 512 blocks the smallest power of two
// >= max(nkb, 64); beyond, nkb rounded up to a multiple of 256 (64 lanes x a multiple of 4
// scores each, so the bucket level pass holds about one score per lane and slot).
inline int mask_score_stride(int nkb) {
  if (nkb > 512) return (nkb + 255) / 256 * 256;
  int n = 64;
  while (n < nkb) n <<= 1;
  return n;
}
// Device address of the static scratch of the allocation-free mask entry point on the
// current device (looked up once per device); hipSuccess or the lookup's error.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_attention(const AttnArgs& a, hipStream_t stream);

}  // namespace psa
