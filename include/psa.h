/*
 * psa.h — C ABI of the MI355X (gfx950) Pyramid Sparse Attention forward path.
 *
 * Pyramid Sparse Attention (PSA; "PSA: Pyramid Sparse Attention for Efficient
 * Video Understanding and Generation", abstract) replaces binary keep/drop block
 * masks with a multi-level pooled KV pyramid: every (query block, KV block) pair
 * gets a pool level, fine for important blocks, coarse for less important ones,
 * or is pruned. The forward pass has three steps, one entry point each:
 *
 *   psa_build_pyramid  — average-pooled K/V levels 1..L-1 and per-block mean keys
 *   psa_estimate_mask  — block importance and the threshold-based level map
 *   psa_estimate_mask_ranked — the same with a fixed share of ranked blocks per level
 *   psa_estimate_mask_noalloc — psa_estimate_mask with a static workspace (allocates nothing)
 *   psa_build_pyramid_sim, psa_apply_similarity_cap — the cosine-similarity constraint
 *   psa_attention_fwd  — attention over mixed-resolution keys, one softmax
 *   psa_attention_bwd  — its gradients with respect to q, k and v
 *
 * Tensors (all row-major, contiguous, head_dim innermost):
 *   q      [B, H,    N, d]          I/O dtype
 *   k, v   [B, H_kv, N, d]          I/O dtype; query head h reads KV head h / (H / H_kv)
 *   k_pyr, v_pyr [B, H_kv, R, d]    I/O dtype, R = psa_pyramid_rows(): level 1, then
 *                                   level 2, ... concatenated along the row axis;
 *                                   level l has ceil(N / 2^l) rows
 *   k_bar  [B, H_kv, nkb, d]        float32 mean key of each 64-token KV block
 *   level_map [B, H, nqb, nkb]      int8: level 0..L-1, or -1 = pruned
 *   o      [B, H, N, d]             I/O dtype;  lse [B, H, N] float32 (natural log)
 * with nqb = ceil(N / q_block), nkb = ceil(N / kv_block).
 *
 * Conventions shared by every entry point:
 *  - Device pointers point to memory of the current HIP device; the caller owns
 *    every buffer, keeps it alive until the work on `stream` has finished, and the
 *    library keeps no pointer after a call returns. Device pointers must be
 *    16-byte aligned. `thresholds` and `fractions` are host pointers.
 *  - Calls only enqueue kernels on `stream` and return without synchronising.
 *    The library allocates no memory and holds no state, except the static device
 *    scratch of psa_estimate_mask_noalloc (see there); calls are thread-safe, but
 *    overlapping psa_estimate_mask_noalloc calls on one device race on its scratch.
 *  - Arguments are checked before anything is launched: invalid values return
 *    PSA_ERR_INVALID_ARGUMENT, valid shapes outside the supported envelope
 *    PSA_ERR_UNSUPPORTED, a short workspace PSA_ERR_WORKSPACE_TOO_SMALL; a failed
 *    launch returns PSA_ERR_HIP. No call aborts, throws or prints;
 *    psa_last_error() gives the calling thread's detail message.
 *  - Arithmetic: pooling, block means and block scores accumulate in float32;
 *    attention multiplies bf16 operands on the matrix cores with float32
 *    accumulation and a float32 online softmax. float32 I/O is rounded to bf16
 *    on its way into the matrix cores.
 *
 * Causal use (PSA serves causal attention for generation and bidirectional attention
 * for understanding: top168.com article, paragraph on causal and bidirectional use):
 *  - mask: query block i (rows r0..r1-1) ranks only the KV blocks that hold a token
 *    at or before r1-1 (softmax, C and the ranked counts over those blocks); blocks
 *    that hold a token at or after r0 are then set to level 0 (a pooled key would
 *    mix in tokens later than some of the block's rows); later blocks are -1 and
 *    report C = 1 (also when n_dense_prefix covers them);
 *  - attention: row r sees a key only if every token it averages is at or before r
 *    (at level 0: token t <= r), whatever the level map says.
 */
#ifndef PSA_H_
#define PSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PSA_OK = 0,
  PSA_ERR_INVALID_ARGUMENT = 1,
  PSA_ERR_UNSUPPORTED = 2,
  PSA_ERR_WORKSPACE_TOO_SMALL = 3,
  PSA_ERR_HIP = 4
} psa_status_t;

typedef enum { PSA_F32 = 0, PSA_BF16 = 1 } psa_dtype_t;

/* Which call a workspace size is asked for. */
typedef enum { PSA_WS_ESTIMATE_MASK = 0, PSA_WS_ATTENTION_FWD = 1, PSA_WS_ATTENTION_BWD = 2 } psa_workspace_kind_t;

typedef struct {
  int32_t B, H, H_kv, N, d;   /* d in {64, 128}; H % H_kv == 0; B * H <= 65535        */
  int32_t q_block;            /* query block size: 64 or 128                           */
  int32_t kv_block;           /* KV block size: 64                                     */
  int32_t num_levels;         /* L in [1, 4]: level l pools 2^l tokens                 */
  psa_dtype_t dtype;          /* I/O dtype of q, k, v, k_pyr, v_pyr, o                 */
  float scale;                /* softmax scale; <= 0 selects 1/sqrt(d)                 */
  int32_t causal;             /* 0: bidirectional; 1: causal (query row r sees tokens
                                 0..r; rules under "Causal use" above)                 */
} psa_problem_t;

/* Rows of the concatenated pyramid: sum over l = 1..L-1 of ceil(N / 2^l).
 * Returns 0 for a NULL or malformed problem. */
size_t psa_pyramid_rows(const psa_problem_t* prob);

/* Device workspace, in bytes, that `kind`'s call needs (0 if none; also 0 for a
 * NULL or malformed problem). */
size_t psa_workspace_bytes(const psa_problem_t* prob, psa_workspace_kind_t kind);

/* Checks a problem description alone (no pointers): PSA_OK, INVALID_ARGUMENT or
 * UNSUPPORTED, with the reason in psa_last_error(). */
psa_status_t psa_check_problem(const psa_problem_t* prob);

/*
 * Step 1, the pyramid ("pyramid KV block construction by progressive pooling":
 * top168.com article, paragraph naming the three components; pool factor 2^level
 * and average pooling over tokens: skillmd.com page, "Pooled KV cache creation").
 * For l = 1..L-1, pooled row p of level l is the mean of K (and of V) over tokens
 * [p*2^l, min((p+1)*2^l, N)); a ragged last group is averaged over the tokens it
 * has. Results are rounded to the I/O dtype (ties to even). k_bar[j] is the
 * float32 mean of K over KV block j (its n_j = min(64, N - 64 j) tokens).
 * k_pyr and v_pyr may be NULL when num_levels == 1.
 */
psa_status_t psa_build_pyramid(const psa_problem_t* prob, const void* k, const void* v,
                               void* k_pyr, void* v_pyr, float* k_bar, hipStream_t stream);

/*
 * Step 1 plus the key similarity of the cosine-similarity constraint (the
 * top168.com ablation paragraph reports that such a constraint helps on some tasks
 * and gives no formula; this is the library's reading). Same outputs as
 * psa_build_pyramid, and for KV block j and level l = 1..L-1
 *   k_sim[b, g, j, l-1] = min over the level-l pool groups G of block j of
 *                         (1/|G|) sum_{t in G} cos(k_t, mean of G),
 * with cos = 0 when either vector is zero: 1 when every group's keys point the
 * same way, lower as they spread. Float32, computed from the same registers as
 * the pyramid (K is read once). k_sim [B, H_kv, nkb, L-1] float32; may be NULL
 * when num_levels == 1 (then nothing is written).
 */
psa_status_t psa_build_pyramid_sim(const psa_problem_t* prob, const void* k, const void* v,
                                   void* k_pyr, void* v_pyr, float* k_bar, float* k_sim,
                                   hipStream_t stream);

/*
 * The cosine-similarity constraint applied to a level map in place: a retained
 * block at level l > 0 of query head h takes the coarsest level l' <= l such that
 * k_sim[b, g(h), j, m-1] >= threshold for every m = 1..l' (level 0 if level 1
 * already fails). Pruned blocks, level-0 blocks and values outside [-1, L-1] are
 * left as they are; the map is then ready for psa_attention_fwd. Nothing to do when
 * num_levels == 1 (k_sim may then be NULL). threshold: any non-NaN float.
 */
psa_status_t psa_apply_similarity_cap(const psa_problem_t* prob, const float* k_sim, float threshold,
                                      int8_t* level_map, hipStream_t stream);

/*
 * Step 2, the multi-level mask ("a multi-level mask generator that assigns a
 * level by the importance of each query-block / KV-block pair": top168.com,
 * three-components paragraph; threshold-based assignment: same page, ablation
 * paragraph; scoring a block by the query against the block's mean key:
 * skillmd.com, "Block importance scoring").
 * For query block i of head h (mean query qbar_i over its rows) and KV block j:
 *   z_ij = scale * <qbar_i, k_bar_j> + ln n_j,   p_ij = softmax over j of z_ij.
 * Blocks are ranked by z descending, ties by j ascending; C_ij is the total p of
 * the blocks ranked strictly ahead of j. level_ij = min{l : C_ij < thresholds[l]},
 * or -1 (pruned) if there is none. Finally every KV block that overlaps tokens
 * [0, n_dense_prefix) is set to level 0 for every query block.
 * thresholds: host array of num_levels floats, nondecreasing, each in [0, 1].
 * cmass_out (nullable): C as float32 [B, H, nqb, nkb].
 * workspace: psa_workspace_bytes(prob, PSA_WS_ESTIMATE_MASK) bytes of device memory
 * (mean queries, then block scores with rows padded to the power of two >= max(nkb, 64)
 * up to nkb = 512 and to a multiple of 256 beyond, then one flag byte per score row),
 * 16-byte aligned; its contents on entry do not matter.
 * Supported: nkb <= 2048 (N <= 131072).
 */
psa_status_t psa_estimate_mask(const psa_problem_t* prob, const void* q, const float* k_bar,
                               const float* thresholds, int32_t n_dense_prefix,
                               int8_t* level_map, float* cmass_out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Step 2 with the ranked (quantile) rule in place of thresholds: the alternative
 * assignment the top168.com ablation paragraph compares with thresholds; a fixed
 * share of the score-ranked blocks at full resolution and the rest spread over the
 * pooled levels (skillmd.com page, "Level assignment", whose keep ratio is
 * fractions[0]). With num_levels == 1 it is the binary top-k block-sparse mask.
 * Scores and ranking are those of psa_estimate_mask. With K_l = floor(fractions[l]
 * * n) (the product in double precision; n = nkb, or under causal use the row's
 * visible blocks), the block of rank r (0 = most important) gets
 * level_ij = min{l : r < K_l}, or -1 (pruned) if there is none.
 * So each row has K_l - K_{l-1} blocks at level l (K_{-1} = 0) before the dense
 * prefix (and, under causal use, the level-0 rule for blocks reaching the query
 * block's rows) is applied as in psa_estimate_mask. cmass_out (nullable): C as
 * defined there.
 * fractions: host array of num_levels doubles, nondecreasing, each in [0, 1].
 * Workspace, supported sizes and errors as psa_estimate_mask.
 */
psa_status_t psa_estimate_mask_ranked(const psa_problem_t* prob, const void* q, const float* k_bar,
                                      const double* fractions, int32_t n_dense_prefix,
                                      int8_t* level_map, float* cmass_out,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Capacity, in bytes, of the library's static device scratch used by
 * psa_estimate_mask_noalloc. */
#define PSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * psa_estimate_mask for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * computation, kernels and results, with the workspace taken from a static device
 * array of PSA_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device it
 * runs on until the process ends. The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine. The caller still provides q, k_bar,
 * level_map and cmass_out (nullable) as for psa_estimate_mask.
 * The first call on a device looks up that device's copy of the array (with the
 * device current); later calls reuse the address.
 * Errors: as psa_estimate_mask; a problem whose workspace
 * (psa_workspace_bytes(prob, PSA_WS_ESTIMATE_MASK)) exceeds the array returns
 * PSA_ERR_WORKSPACE_TOO_SMALL before anything is launched.
 * Every call on one device shares that device's array: calls that overlap in time on
 * one device (several streams or threads) race on it and must be serialised by the
 * caller. Nothing in the array needs to be zero on entry (every byte a kernel reads is
 * written earlier in the same call).
 */
psa_status_t psa_estimate_mask_noalloc(const psa_problem_t* prob, const void* q, const float* k_bar,
                                       const float* thresholds, int32_t n_dense_prefix,
                                       int8_t* level_map, float* cmass_out, hipStream_t stream);

/*
 * Step 3, attention over mixed-resolution keys with one softmax ("adaptive
 * pyramid attention that keeps the probability distribution consistent":
 * top168.com, three-components paragraph; decoupled logical-block / hardware-tile
 * execution: chatpaper.ai abstract and top168.com kernel paragraph).
 * Query row r of block i attends to every pooled row p of every retained KV block
 * j (level l = level_map[.., i, j] >= 0; block j owns rows
 * [j*64/2^l, ceil((j*64 + n_j)/2^l)) of level l, level 0 being K/V themselves), with
 * logit a_rp = scale * <q_r, K^l_p> + ln c_p, c_p the number of tokens row p
 * averages. O_r = sum_p e^{a_rp} V^l_p / sum_p e^{a_rp}; lse_r = ln sum_p e^{a_rp}.
 * A row whose query block retains nothing gets O = 0 and lse = -inf.
 * lse may be NULL. workspace may be NULL when psa_workspace_bytes(prob,
 * PSA_WS_ATTENTION_FWD) is 0. k_pyr, v_pyr may be NULL when num_levels == 1.
 * level_map values outside [-1, L-1] are treated as -1 (pruned).
 */
psa_status_t psa_attention_fwd(const psa_problem_t* prob, const void* q, const void* k,
                               const void* v, const void* k_pyr, const void* v_pyr,
                               const int8_t* level_map, void* o, float* lse,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of step 3: gradients of the attention output with respect to q, k and v,
 * with the level map held fixed (it is a discrete choice). The pages describe no
 * backward pass; they imply training use (the top168.com article's models are
 * fine-tuned and distilled with PSA), and this is the exact gradient of the forward
 * defined by psa_attention_fwd. With P_rp = e^{a_rp - lse_r} over the pooled keys p of
 * row r (the causal rule applied as in the forward) and D_r = <dO_r, O_r>:
 *   dV_p = sum_r P_rp dO_r,  dA_rp = P_rp (<dO_r, V_p> - D_r),
 *   dq_r = scale sum_p dA_rp K_p,  dK_p = scale sum_r dA_rp q_r,
 * and a pooled row, the mean of its c tokens, passes 1/c of its gradient to each;
 * dk and dv sum over the query heads that share the KV head.
 * Inputs: q, k, v, k_pyr, v_pyr, level_map as given to psa_attention_fwd, and that
 * call's outputs o (I/O dtype) and lse (float32, required), d_o = dL/dO like o.
 * Outputs dq like q, dk and dv like k (I/O dtype), every element written.
 * workspace: psa_workspace_bytes(prob, PSA_WS_ATTENTION_BWD) bytes of device memory,
 * 16-byte aligned, contents on entry irrelevant (per query row the lse in base 2 and
 * the row dot <dO, O>, then float32 per-level gradients of K and of V). Arithmetic: bf16 operands on the matrix cores with
 * float32 accumulation (P and dA rounded to bf16 for their products), like the
 * forward.
 */
psa_status_t psa_attention_bwd(const psa_problem_t* prob, const void* q, const void* k, const void* v,
                               const void* k_pyr, const void* v_pyr, const int8_t* level_map,
                               const void* o, const float* lse, const void* d_o,
                               void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code ("PSA_OK", ...); never NULL. */
const char* psa_status_string(psa_status_t status);

/* Detail of the calling thread's last non-OK return ("" if none); valid until the
 * thread's next psa_* call. */
const char* psa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PSA_H_ */
