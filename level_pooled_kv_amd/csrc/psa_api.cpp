// C ABI of the PSA forward path: argument validation, derived sizes, launches.
// Nothing here allocates device memory, synchronises, prints or throws.
#include "psa.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "psa_launch.h"

namespace {

thread_local char g_err[512] = "";

psa_status_t fail(psa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = '\0'; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

psa_status_t check_problem(const psa_problem_t* p) {
  if (!p) return fail(PSA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->B <= 0 || p->H <= 0 || p->H_kv <= 0 || p->N <= 0 || p->d <= 0)
    return fail(PSA_ERR_INVALID_ARGUMENT, "B, H, H_kv, N, d must be positive (got %d, %d, %d, %d, %d)",
                p->B, p->H, p->H_kv, p->N, p->d);
  if (p->H % p->H_kv != 0)
    return fail(PSA_ERR_INVALID_ARGUMENT, "H (%d) must be a multiple of H_kv (%d)", p->H, p->H_kv);
  if (p->q_block <= 0 || p->kv_block <= 0)
    return fail(PSA_ERR_INVALID_ARGUMENT, "block sizes must be positive");
  if (p->num_levels < 1)
    return fail(PSA_ERR_INVALID_ARGUMENT, "num_levels must be >= 1 (got %d)", p->num_levels);
  if (p->dtype != PSA_F32 && p->dtype != PSA_BF16)
    return fail(PSA_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)p->dtype);
  if (isnan(p->scale) || isinf(p->scale))
    return fail(PSA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (p->causal != 0 && p->causal != 1)
    return fail(PSA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1 (got %d)", p->causal);
  if (p->d != 64 && p->d != 128)
    return fail(PSA_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", p->d);
  if (p->q_block != 64 && p->q_block != 128)
    return fail(PSA_ERR_UNSUPPORTED, "q_block %d not supported (64 or 128)", p->q_block);
  if (p->kv_block != psa::kKvBlock)
    return fail(PSA_ERR_UNSUPPORTED, "kv_block %d not supported (64)", p->kv_block);
  if (p->num_levels > psa::kMaxLevels)
    return fail(PSA_ERR_UNSUPPORTED, "num_levels %d not supported (1..4)", p->num_levels);
  if (ceil_div(p->N, psa::kKvBlock) > psa::kMaxKvBlocks)
    return fail(PSA_ERR_UNSUPPORTED, "N = %d gives more than %d KV blocks", p->N, psa::kMaxKvBlocks);
  const int64_t elems = (int64_t)p->B * p->H * p->N * p->d;
  if (elems >= ((int64_t)1 << 40))
    return fail(PSA_ERR_UNSUPPORTED, "tensor of %lld elements is too large", (long long)elems);
  if ((int64_t)p->B * p->H * ceil_div(p->N, p->q_block) >= ((int64_t)1 << 31) - 8)
    return fail(PSA_ERR_UNSUPPORTED, "too many query blocks");
  if ((int64_t)p->B * p->H > 65535)   // one grid dimension spans batch x heads
    return fail(PSA_ERR_UNSUPPORTED, "B * H = %lld exceeds 65535", (long long)p->B * p->H);
  return PSA_OK;
}

int64_t pyramid_rows(const psa_problem_t* p) {
  int64_t r = 0;
  for (int l = 1; l < p->num_levels; ++l) r += ceil_div(p->N, (int64_t)1 << l);
  return r;
}

void level_offsets(const psa_problem_t* p, int off[psa::kMaxLevels], int rows[psa::kMaxLevels]) {
  int64_t acc = 0;
  for (int l = 0; l < psa::kMaxLevels; ++l) {
    rows[l] = (int)ceil_div(p->N, (int64_t)1 << l);
    off[l] = 0;
  }
  for (int l = 1; l < psa::kMaxLevels; ++l) {
    off[l] = (int)acc;
    if (l < p->num_levels) acc += rows[l];
  }
}

float effective_scale(const psa_problem_t* p) {
  return p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->d);
}

// Mask workspace: mean queries [B, H, nqb, d] then block scores [B, H, nqb, stride],
// both float32 (the first part's size is a multiple of 256 bytes, so the second
// stays 16-byte aligned), then one byte per score row (rows the exact pass redoes).
size_t mask_qbar_bytes(const psa_problem_t* p) {
  return (size_t)p->B * p->H * ceil_div(p->N, p->q_block) * p->d * sizeof(float);
}
size_t mask_score_bytes(const psa_problem_t* p) {
  const int nkb = (int)ceil_div(p->N, psa::kKvBlock);
  return (size_t)p->B * p->H * ceil_div(p->N, p->q_block) * psa::mask_score_stride(nkb) * sizeof(float);
}
size_t mask_workspace(const psa_problem_t* p) {
  return mask_qbar_bytes(p) + mask_score_bytes(p) + (size_t)p->B * p->H * ceil_div(p->N, p->q_block);
}

#define REQUIRE_PTR(ptr, name)                                                        \
  do {                                                                                \
    if (!(ptr)) return fail(PSA_ERR_INVALID_ARGUMENT, "%s is NULL", name);            \
    if (!aligned16(ptr)) return fail(PSA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name); \
  } while (0)

psa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PSA_OK;
  return fail(PSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t psa_pyramid_rows(const psa_problem_t* prob) {
  if (check_problem(prob) != PSA_OK) return 0;
  return (size_t)pyramid_rows(prob);
}

// Backward workspace: per query row the lse in base 2 and the row dot D, each [B, H, Npad]
// with N padded to a multiple of 64 (padding rows: lse +inf, D 0), then the float32
// per-level gradients of K and of V [B, H_kv, N + pyramid rows, d]; each part starts on a
// 256-byte boundary.
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
int bwd_npad(const psa_problem_t* p) { return (int)ceil_div(p->N, 64) * 64; }
size_t bwd_dr_bytes(const psa_problem_t* p) { return round256((size_t)p->B * p->H * bwd_npad(p) * sizeof(float)); }
size_t bwd_grad_bytes(const psa_problem_t* p) {
  return round256((size_t)p->B * p->H_kv * (p->N + pyramid_rows(p)) * p->d * sizeof(float));
}
size_t bwd_workspace(const psa_problem_t* p) { return 2 * bwd_dr_bytes(p) + 2 * bwd_grad_bytes(p); }

size_t psa_workspace_bytes(const psa_problem_t* prob, psa_workspace_kind_t kind) {
  if (check_problem(prob) != PSA_OK) return 0;
  if (kind == PSA_WS_ESTIMATE_MASK) return mask_workspace(prob);
  if (kind == PSA_WS_ATTENTION_BWD) return bwd_workspace(prob);
  return 0;
}

psa_status_t psa_check_problem(const psa_problem_t* prob) {
  clear_error();
  return check_problem(prob);
}

static psa_status_t build_pyramid_common(const psa_problem_t* prob, const void* k, const void* v, void* k_pyr,
                                         void* v_pyr, float* k_bar, float* k_sim, hipStream_t stream,
                                         const char* what) {
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(k_bar, "k_bar");
  if (prob->num_levels > 1) {
    REQUIRE_PTR(k_pyr, "k_pyr");
    REQUIRE_PTR(v_pyr, "v_pyr");
  }
  psa::PyramidArgs a{};
  a.k = k; a.v = v; a.k_pyr = k_pyr; a.v_pyr = v_pyr; a.k_bar = k_bar;
  a.k_sim = prob->num_levels > 1 ? k_sim : nullptr;
  a.B = prob->B; a.H_kv = prob->H_kv; a.N = prob->N; a.d = prob->d;
  a.nkb = (int)ceil_div(prob->N, psa::kKvBlock);
  a.L = prob->num_levels;
  a.bf16 = prob->dtype == PSA_BF16;
  a.pyr_rows = pyramid_rows(prob);
  int rows[psa::kMaxLevels];
  level_offsets(prob, a.off, rows);
  return hip_status(psa::launch_pyramid(a, stream), what);
}

psa_status_t psa_build_pyramid(const psa_problem_t* prob, const void* k, const void* v, void* k_pyr,
                               void* v_pyr, float* k_bar, hipStream_t stream) {
  clear_error();
  psa_status_t s = check_problem(prob);
  if (s != PSA_OK) return s;
  return build_pyramid_common(prob, k, v, k_pyr, v_pyr, k_bar, nullptr, stream, "psa_build_pyramid launch");
}

psa_status_t psa_build_pyramid_sim(const psa_problem_t* prob, const void* k, const void* v, void* k_pyr,
                                   void* v_pyr, float* k_bar, float* k_sim, hipStream_t stream) {
  clear_error();
  psa_status_t s = check_problem(prob);
  if (s != PSA_OK) return s;
  if (prob->num_levels > 1) REQUIRE_PTR(k_sim, "k_sim");
  return build_pyramid_common(prob, k, v, k_pyr, v_pyr, k_bar, k_sim, stream, "psa_build_pyramid_sim launch");
}

psa_status_t psa_apply_similarity_cap(const psa_problem_t* prob, const float* k_sim, float threshold,
                                      int8_t* level_map, hipStream_t stream) {
  clear_error();
  psa_status_t s = check_problem(prob);
  if (s != PSA_OK) return s;
  if (isnan(threshold)) return fail(PSA_ERR_INVALID_ARGUMENT, "threshold is NaN");
  REQUIRE_PTR(level_map, "level_map");
  if (prob->num_levels < 2) return PSA_OK;   // nothing is pooled: nothing to cap
  REQUIRE_PTR(k_sim, "k_sim");
  psa::CapArgs a{};
  a.level_map = level_map; a.k_sim = k_sim; a.threshold = threshold;
  a.B = prob->B; a.H = prob->H; a.H_kv = prob->H_kv;
  a.nqb = (int)ceil_div(prob->N, prob->q_block);
  a.nkb = (int)ceil_div(prob->N, psa::kKvBlock);
  a.L = prob->num_levels;
  return hip_status(psa::launch_similarity_cap(a, stream), "psa_apply_similarity_cap launch");
}

static psa_status_t check_thresholds(const psa_problem_t* prob, const float* thresholds) {
  if (!thresholds) return fail(PSA_ERR_INVALID_ARGUMENT, "thresholds is NULL");
  for (int l = 0; l < prob->num_levels; ++l) {
    const float t = thresholds[l];
    if (!(t >= 0.f && t <= 1.f))
      return fail(PSA_ERR_INVALID_ARGUMENT, "thresholds[%d] = %g is not in [0, 1]", l, (double)t);
    if (l > 0 && t < thresholds[l - 1])
      return fail(PSA_ERR_INVALID_ARGUMENT, "thresholds must be nondecreasing (thresholds[%d] < thresholds[%d])",
                  l, l - 1);
  }
  return PSA_OK;
}

// Pointer and prefix checks of the mask entry points (the workspace is checked separately).
static psa_status_t check_mask_pointers(const psa_problem_t* prob, const void* q, const float* k_bar,
                                        int32_t n_dense_prefix, const int8_t* level_map, const float* cmass_out) {
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k_bar, "k_bar");
  REQUIRE_PTR(level_map, "level_map");
  if (cmass_out && !aligned16(cmass_out))
    return fail(PSA_ERR_INVALID_ARGUMENT, "cmass_out is not 16-byte aligned");
  if (n_dense_prefix < 0 || n_dense_prefix > prob->N)
    return fail(PSA_ERR_INVALID_ARGUMENT, "n_dense_prefix %d not in [0, N]", n_dense_prefix);
  return PSA_OK;
}

// Checks shared by both mask entry points, then the launch. Exactly one of tau and
// fractions is non-NULL: the threshold rule or the ranked rule.
static psa_status_t estimate_mask_common(const psa_problem_t* prob, const void* q, const float* k_bar,
                                         int32_t n_dense_prefix, int8_t* level_map, float* cmass_out,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                                         const float* tau, const double* fractions, const char* what) {
  psa_status_t s = check_mask_pointers(prob, q, k_bar, n_dense_prefix, level_map, cmass_out);
  if (s != PSA_OK) return s;
  const size_t need = mask_workspace(prob);
  if (workspace_bytes < need)
    return fail(PSA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  REQUIRE_PTR(workspace, "workspace");
  psa::MaskArgs a{};
  a.q = q; a.k_bar = k_bar; a.level_map = level_map; a.cmass = cmass_out;
  a.qbar = static_cast<float*>(workspace);
  a.z = reinterpret_cast<float*>(static_cast<char*>(workspace) + mask_qbar_bytes(prob));
  a.need_exact = reinterpret_cast<uint8_t*>(static_cast<char*>(workspace) + mask_qbar_bytes(prob) +
                                            mask_score_bytes(prob));
  a.B = prob->B; a.H = prob->H; a.H_kv = prob->H_kv; a.N = prob->N; a.d = prob->d;
  a.q_block = prob->q_block;
  a.nqb = (int)ceil_div(prob->N, prob->q_block);
  a.nkb = (int)ceil_div(prob->N, psa::kKvBlock);
  a.L = prob->num_levels;
  a.n_dense_prefix = n_dense_prefix;
  a.bf16 = prob->dtype == PSA_BF16;
  a.scale = effective_scale(prob);
  a.ranked = fractions != nullptr;
  a.causal = prob->causal != 0;
  for (int l = 0; l < psa::kMaxLevels; ++l) {
    a.tau[l] = tau && l < prob->num_levels ? tau[l] : 0.f;
    a.frac[l] = fractions && l < prob->num_levels ? fractions[l] : 0.0;
  }
  return hip_status(psa::launch_mask(a, stream), what);
}

psa_status_t psa_estimate_mask(const psa_problem_t* prob, const void* q, const float* k_bar,
                               const float* thresholds, int32_t n_dense_prefix, int8_t* level_map,
                               float* cmass_out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  clear_error();
  psa_status_t s = check_problem(prob);
  if (s != PSA_OK) return s;
  s = check_thresholds(prob, thresholds);
  if (s != PSA_OK) return s;
  return estimate_mask_common(prob, q, k_bar, n_dense_prefix, level_map, cmass_out, workspace, workspace_bytes,
                              stream, thresholds, nullptr, "psa_estimate_mask launch");
}

psa_status_t psa_estimate_mask_noalloc(const psa_problem_t* prob, const void* q, const float* k_bar,
                                       const float* thresholds, int32_t n_dense_prefix, int8_t* level_map,
                                       float* cmass_out, hipStream_t stream) {
  clear_error();
  psa_status_t s = check_problem(prob);
  if (s != PSA_OK) return s;
  s = check_thresholds(prob, thresholds);
  if (s != PSA_OK) return s;
  s = check_mask_pointers(prob, q, k_bar, n_dense_prefix, level_map, cmass_out);
  if (s != PSA_OK) return s;
  const size_t need = mask_workspace(prob);
  if (need > PSA_NOALLOC_SCRATCH_BYTES)
    return fail(PSA_ERR_WORKSPACE_TOO_SMALL,
                "psa_estimate_mask_noalloc: the problem needs %zu bytes of workspace, the static scratch holds %zu",
                need, (size_t)PSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const hipError_t e = psa::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "psa_estimate_mask_noalloc: scratch lookup");
  return estimate_mask_common(prob, q, k_bar, n_dense_prefix, level_map, cmass_out, ws, PSA_NOALLOC_SCRATCH_BYTES,
                              stream, thresholds, nullptr, "psa_estimate_mask_noalloc launch");
}

psa_status_t psa_estimate_mask_ranked(const psa_problem_t* prob, const void* q, const float* k_bar,
                                      const double* fractions, int32_t n_dense_prefix, int8_t* level_map,
                                      float* cmass_out, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  clear_error();
  psa_status_t s = check_problem(prob);
  if (s != PSA_OK) return s;
  if (!fractions) return fail(PSA_ERR_INVALID_ARGUMENT, "fractions is NULL");
  for (int l = 0; l < prob->num_levels; ++l) {
    const double f = fractions[l];
    if (!(f >= 0.0 && f <= 1.0))
      return fail(PSA_ERR_INVALID_ARGUMENT, "fractions[%d] = %g is not in [0, 1]", l, f);
    if (l > 0 && f < fractions[l - 1])
      return fail(PSA_ERR_INVALID_ARGUMENT, "fractions must be nondecreasing (fractions[%d] < fractions[%d])",
                  l, l - 1);
  }
  // the kernel takes K_l = floor(f_l * n) per row (n = nkb, or the row's visible blocks)
  return estimate_mask_common(prob, q, k_bar, n_dense_prefix, level_map, cmass_out, workspace, workspace_bytes,
                              stream, nullptr, fractions, "psa_estimate_mask_ranked launch");
}

psa_status_t psa_attention_fwd(const psa_problem_t* prob, const void* q, const void* k, const void* v,
                               const void* k_pyr, const void* v_pyr, const int8_t* level_map, void* o,
                               float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  (void)workspace;
  (void)workspace_bytes;
  psa_status_t s = check_problem(prob);
  if (s != PSA_OK) return s;
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(o, "o");
  REQUIRE_PTR(level_map, "level_map");
  if (prob->num_levels > 1) {
    REQUIRE_PTR(k_pyr, "k_pyr");
    REQUIRE_PTR(v_pyr, "v_pyr");
  }
  if (lse && !aligned16(lse)) return fail(PSA_ERR_INVALID_ARGUMENT, "lse is not 16-byte aligned");
  psa::AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.k_pyr = k_pyr; a.v_pyr = v_pyr; a.level_map = level_map; a.o = o; a.lse = lse;
  a.B = prob->B; a.H = prob->H; a.H_kv = prob->H_kv; a.N = prob->N; a.d = prob->d;
  a.q_block = prob->q_block;
  a.nqb = (int)ceil_div(prob->N, prob->q_block);
  a.nkb = (int)ceil_div(prob->N, psa::kKvBlock);
  a.L = prob->num_levels;
  a.bf16 = prob->dtype == PSA_BF16;
  a.causal = prob->causal != 0;
  a.scale = effective_scale(prob);
  a.pyr_rows = pyramid_rows(prob);
  level_offsets(prob, a.off, a.rows);
  return hip_status(psa::launch_attention(a, stream), "psa_attention_fwd launch");
}

psa_status_t psa_attention_bwd(const psa_problem_t* prob, const void* q, const void* k, const void* v,
                               const void* k_pyr, const void* v_pyr, const int8_t* level_map, const void* o,
                               const float* lse, const void* d_o, void* dq, void* dk, void* dv, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  psa_status_t s = check_problem(prob);
  if (s != PSA_OK) return s;
  REQUIRE_PTR(q, "q");
  REQUIRE_PTR(k, "k");
  REQUIRE_PTR(v, "v");
  REQUIRE_PTR(level_map, "level_map");
  REQUIRE_PTR(o, "o");
  REQUIRE_PTR(lse, "lse");
  REQUIRE_PTR(d_o, "d_o");
  REQUIRE_PTR(dq, "dq");
  REQUIRE_PTR(dk, "dk");
  REQUIRE_PTR(dv, "dv");
  if (prob->num_levels > 1) {
    REQUIRE_PTR(k_pyr, "k_pyr");
    REQUIRE_PTR(v_pyr, "v_pyr");
  }
  const size_t need = bwd_workspace(prob);
  if (workspace_bytes < need)
    return fail(PSA_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  REQUIRE_PTR(workspace, "workspace");
  psa::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.k_pyr = k_pyr; a.v_pyr = v_pyr; a.level_map = level_map;
  a.o = o; a.lse = lse; a.dout = d_o; a.dq = dq; a.dk = dk; a.dv = dv;
  char* ws = static_cast<char*>(workspace);
  a.lse2 = reinterpret_cast<float*>(ws);
  a.Dr = reinterpret_cast<float*>(ws + bwd_dr_bytes(prob));
  a.dkw = reinterpret_cast<float*>(ws + 2 * bwd_dr_bytes(prob));
  a.dvw = reinterpret_cast<float*>(ws + 2 * bwd_dr_bytes(prob) + bwd_grad_bytes(prob));
  a.Npad = bwd_npad(prob);
  a.B = prob->B; a.H = prob->H; a.H_kv = prob->H_kv; a.N = prob->N; a.d = prob->d;
  a.q_block = prob->q_block;
  a.nqb = (int)ceil_div(prob->N, prob->q_block);
  a.nkb = (int)ceil_div(prob->N, psa::kKvBlock);
  a.L = prob->num_levels;
  a.bf16 = prob->dtype == PSA_BF16;
  a.causal = prob->causal != 0;
  a.scale = effective_scale(prob);
  a.pyr_rows = pyramid_rows(prob);
  level_offsets(prob, a.off, a.rows);
  return hip_status(psa::launch_attention_bwd(a, stream), "psa_attention_bwd launch");
}

const char* psa_status_string(psa_status_t status) {
  switch (status) {
    case PSA_OK: return "PSA_OK";
    case PSA_ERR_INVALID_ARGUMENT: return "PSA_ERR_INVALID_ARGUMENT";
    case PSA_ERR_UNSUPPORTED: return "PSA_ERR_UNSUPPORTED";
    case PSA_ERR_WORKSPACE_TOO_SMALL: return "PSA_ERR_WORKSPACE_TOO_SMALL";
    case PSA_ERR_HIP: return "PSA_ERR_HIP";
  }
  return "PSA_ERR_UNKNOWN";
}

const char* psa_last_error(void) { return g_err; }

}  // extern "C"
