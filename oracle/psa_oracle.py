"""CPU oracle for the Pyramid Sparse Attention (PSA) forward pass.

TEST INFRASTRUCTURE ONLY. Tests, the smoke check and the benchmark's CPU
baseline may call this module; the product path (the HIP library and its
Python binding) never does, and this module imports nothing from it.

Plain, slow and float64 throughout. Each function follows one step of the
method as the pages describe it:

* "PSA: Pyramid Sparse Attention for Efficient Video Understanding and
  Generation" (chatpaper.ai), abstract: multi-level pooled KV, a level per
  (query block, KV block) pair, lower levels for critical blocks, pruning.
* top168.com article on arXiv:2512.04025, paragraph on the pyramid (average
  pooling, each level coarser) and the paragraph naming the three components
  (progressive pooling, a multi-level mask generator driven by query-block /
  KV-block importance, attention that keeps the probability distribution
  consistent); ablation paragraph (threshold-based assignment preferred to
  quantile-based; multi-level masks preferred to binary ones); paragraph on
  causal use (generation) and bidirectional use (understanding); the ablation's
  cosine-similarity constraint (no formula given: see key_similarity).
* skillmd.com "Psa Pyramid Sparse Attention", sections "Pooled KV cache
  creation" (pool factor 2**level, average pooling over tokens), "Block
  importance scoring" (query against the block's mean key) and "Level
  assignment" (fixed shares of the score-ranked blocks per level: the ranked
  rule that the top168.com ablation compares with thresholds).

Where the pages leave a step open, the reading taken is stated in the
function's docstring. The precise arithmetic of the probability-consistency
step (one softmax, each pooled key's logit raised by the log of its pool size)
is this project's reading of "probability distribution consistency".

Every function here has at least one independent pin in tests/ (closed forms,
brute force, invariants, a hand-worked example); the comparison with the
authors' own PSA outputs is "parity unpinned": the pages print no numeric
example and the authors' code is not available.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

LN2 = math.log(2.0)


# ----------------------------------------------------------------------------
# Rounding to the I/O dtype (the pyramid and O are typed outputs)
# ----------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits and float32's exponent range; values below
    the smallest normal are rounded on the fixed subnormal grid 2**-133."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    m, e = np.frexp(x[nz])                   # x = m * 2**e, 0.5 <= |m| < 1
    ulp_exp = np.maximum(e - 8, -133)        # 8 significant bits
    out[nz] = np.ldexp(np.rint(np.ldexp(x[nz], -ulp_exp)), ulp_exp)   # rint: ties to even
    out[~nz] = x[~nz]
    big = np.abs(out) > 3.3895313892515355e38   # largest finite bfloat16
    out[big] = np.sign(out[big]) * np.inf
    return out


def round_to_io(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "f64":          # no rounding (exact-arithmetic checks of the oracle itself)
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# O1: the pyramid
# ----------------------------------------------------------------------------

def pooled_rows(N: int, level: int) -> int:
    """Number of pooled rows at ``level``: ceil(N / 2**level)."""
    return -(-N // (1 << level))


def pool_counts(N: int, level: int) -> np.ndarray:
    """c_l[p] = number of tokens averaged into pooled row p (2**level except a ragged last row)."""
    P = 1 << level
    starts = np.arange(pooled_rows(N, level)) * P
    return (np.minimum(starts + P, N) - starts).astype(np.int64)


def pool_level(x: np.ndarray, level: int) -> np.ndarray:
    """Average pooling over tokens with factor 2**level (skillmd.com, "Pooled KV cache creation").

    x: [..., N, d]. Pooled row p is the mean of tokens [p*2**l, min((p+1)*2**l, N));
    a ragged last group is averaged over the tokens it has (reading: the pages are
    silent on it). Level 0 is x itself."""
    x = np.asarray(x, dtype=np.float64)
    if level == 0:
        return x.copy()
    N = x.shape[-2]
    P = 1 << level
    R = pooled_rows(N, level)
    pad = R * P - N
    xp = np.concatenate([x, np.zeros(x.shape[:-2] + (pad, x.shape[-1]))], axis=-2) if pad else x
    sums = xp.reshape(x.shape[:-2] + (R, P, x.shape[-1])).sum(axis=-2)
    return sums / pool_counts(N, level)[:, None]


def build_pyramid(x: np.ndarray, num_levels: int) -> List[np.ndarray]:
    """[level 0 (x itself), level 1, ..., level L-1] as exact float64 means.

    The article says the levels are built by progressive pooling; in exact
    arithmetic pooling each level from the one below equals pooling the tokens
    directly, so the oracle pools directly."""
    return [pool_level(x, l) for l in range(num_levels)]


def pyramid_concat(levels: Sequence[np.ndarray]) -> np.ndarray:
    """Level-major concatenation of levels 1..L-1 along the token axis ([..., sum_l R_l, d])."""
    if len(levels) <= 1:
        shape = levels[0].shape[:-2] + (0, levels[0].shape[-1])
        return np.zeros(shape)
    return np.concatenate(list(levels[1:]), axis=-2)


def pyramid_row_offsets(N: int, num_levels: int) -> List[int]:
    """Row offset of level l (l >= 1) in the concatenated pyramid; index 0 unused (0)."""
    offs = [0, 0]
    for l in range(1, num_levels):
        offs.append(offs[-1] + pooled_rows(N, l))
    return offs[:num_levels]


# ----------------------------------------------------------------------------
# O2: block means
# ----------------------------------------------------------------------------

def block_sizes(N: int, block: int) -> np.ndarray:
    """n_j: tokens in block j (block tokens [j*block, min((j+1)*block, N)))."""
    nb = -(-N // block)
    starts = np.arange(nb) * block
    return (np.minimum(starts + block, N) - starts).astype(np.int64)


def block_means(x: np.ndarray, block: int) -> np.ndarray:
    """Mean over the tokens of each block: [..., N, d] -> [..., nblocks, d].

    For keys this is the block's mean key that the scoring step dots the query
    with (skillmd.com, "Block importance scoring"); for queries it is the mean
    of the query block (reading: the mask is per query block, abstract)."""
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[-2]
    n = block_sizes(N, block)
    out = np.empty(x.shape[:-2] + (len(n), x.shape[-1]))
    for j in range(len(n)):
        out[..., j, :] = x[..., j * block: j * block + n[j], :].sum(axis=-2) / n[j]
    return out


# ----------------------------------------------------------------------------
# O3-O5: scores, mass, levels
# ----------------------------------------------------------------------------

def kv_head_of(h: int, H: int, H_kv: int) -> int:
    """Query head h reads KV head h // (H / H_kv) (consecutive groups; reading, pages silent)."""
    return h // (H // H_kv)


def block_scores(qbar: np.ndarray, kbar: np.ndarray, n_kv: np.ndarray, scale: float) -> np.ndarray:
    """z[b,h,i,j] = scale * <qbar[b,h,i], kbar[b,g(h),j]> + ln n_j.

    The dot product is the skillmd.com scoring step (query against the mean key);
    the + ln n_j term weights a block by its token count the same way the
    attention step weights a pooled key (equal for all full blocks)."""
    B, H, nqb, d = qbar.shape
    H_kv = kbar.shape[1]
    z = np.empty((B, H, nqb, kbar.shape[2]))
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, H_kv)
            z[b, h] = scale * (qbar[b, h] @ kbar[b, g].T) + np.log(n_kv.astype(np.float64))[None, :]
    return z


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """p = softmax over the last axis (the KV blocks of one query-block row)."""
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def importance_order(z_row: np.ndarray) -> np.ndarray:
    """Block indices from most to least important: z descending, ties by index ascending."""
    j = np.arange(z_row.shape[0])
    return np.lexsort((j, -z_row))


def cumulative_mass(z: np.ndarray, p: np.ndarray) -> np.ndarray:
    """C[..., j] = total p of the blocks strictly ahead of j in importance order (exclusive)."""
    C = np.empty_like(p)
    flat_z = z.reshape(-1, z.shape[-1])
    flat_p = p.reshape(-1, p.shape[-1])
    flat_C = C.reshape(-1, p.shape[-1])
    for r in range(flat_z.shape[0]):
        order = importance_order(flat_z[r])
        ps = flat_p[r][order]
        excl = np.concatenate([[0.0], np.cumsum(ps)[:-1]])
        flat_C[r, order] = excl
    return C


def assign_levels(C: np.ndarray, thresholds: Sequence[float], num_levels: int,
                  n_dense_prefix: int = 0, kv_block: int = 64) -> np.ndarray:
    """level_j = min{l : C_j < tau_l}, or -1 (pruned) if no level qualifies; then every
    KV block overlapping tokens [0, n_dense_prefix) is set to level 0.

    Thresholds are compared as the float32 numbers the library receives."""
    tau = np.asarray(thresholds, dtype=np.float32).astype(np.float64)[:num_levels]
    lev = np.full(C.shape, -1, dtype=np.int8)
    for l in range(num_levels - 1, -1, -1):
        lev[C < tau[l]] = l
    if n_dense_prefix > 0:
        nforce = -(-n_dense_prefix // kv_block)
        lev[..., :nforce] = 0
    return lev


def estimate_mask(q: np.ndarray, k: np.ndarray, q_block: int, kv_block: int,
                  thresholds: Sequence[float], num_levels: int, scale: float,
                  n_dense_prefix: int = 0, causal: bool = False) -> Dict[str, np.ndarray]:
    """The whole mask step: q/k [B,H(_kv),N,d] -> level map [B,H,nqb,nkb] int8 (+ intermediates).
    causal: see causal_blocks and apply_causal."""
    N = q.shape[-2]
    qbar = block_means(q, q_block)
    kbar = block_means(k, kv_block)
    n_kv = block_sizes(N, kv_block)
    z = block_scores(qbar, kbar, n_kv, scale)
    if causal:
        vis, _ = causal_blocks(N, q_block, kv_block)
        z = np.where(vis, z, -np.inf)
    p = softmax_rows(z)
    C = cumulative_mass(z, p)
    lev = assign_levels(C, thresholds, num_levels, n_dense_prefix, kv_block)
    if causal:
        C, lev = apply_causal(C, lev, N, q_block, kv_block)
    return {"qbar": qbar, "kbar": kbar, "z": z, "p": p, "cmass": C, "levels": lev}


# ----------------------------------------------------------------------------
# Causal use (top168.com article, paragraph on causal and bidirectional use)
# ----------------------------------------------------------------------------

def causal_blocks(N: int, q_block: int, kv_block: int) -> Tuple[np.ndarray, np.ndarray]:
    """vis[i, j]: KV block j holds a token at or before the last row of query block i;
    diag[i, j]: it is visible and holds a token at or after the block's first row (so it
    is not entirely in the past of every row of the block)."""
    nqb, nkb = -(-N // q_block), -(-N // kv_block)
    r0 = np.arange(nqb)[:, None] * q_block
    r1 = np.minimum(r0 + q_block, N)
    j0 = np.arange(nkb)[None, :] * kv_block
    j1 = np.minimum(j0 + kv_block, N)
    vis = j0 <= r1 - 1
    diag = vis & (j1 - 1 >= r0)
    return vis, diag


def apply_causal(C: np.ndarray, lev: np.ndarray, N: int, q_block: int, kv_block: int):
    """Causal reading of the mask: the mass and ranking run over the visible blocks only
    (the caller gives invisible blocks z = -inf); a block that reaches the query block's
    own rows is kept at full resolution, since a pooled key mixing in later tokens would
    leak them; invisible blocks are pruned and report C = 1 (all mass lies ahead)."""
    vis, diag = causal_blocks(N, q_block, kv_block)
    C = np.where(vis, C, 1.0)
    lev = lev.copy()
    lev[..., diag] = 0
    lev[..., ~vis] = -1
    return C, lev


# ----------------------------------------------------------------------------
# O4c: cosine-similarity constraint (top168.com, ablation paragraph)
# ----------------------------------------------------------------------------

def cosine(a: np.ndarray, b: np.ndarray) -> float:
    """cos(a, b); 0 when either vector is zero (a zero vector has no direction)."""
    na, nb = float(np.linalg.norm(a)), float(np.linalg.norm(b))
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b)) / (na * nb)


def key_similarity(k: np.ndarray, kv_block: int, num_levels: int) -> np.ndarray:
    """sim[b, g, j, l-1] for levels l = 1..L-1.

    The article reports that a cosine-similarity constraint helps on some tasks but
    gives no formula. Reading: a pooled key stands for its tokens well when it points
    the way they do, so a level-l pool group scores the mean over its tokens of
    cos(k_t, group mean); block j scores the smallest of its level-l groups (the
    worst pooled key it would contribute)."""
    k = np.asarray(k, dtype=np.float64)
    B, H_kv, N, _ = k.shape
    nkb = -(-N // kv_block)
    sim = np.ones((B, H_kv, nkb, max(num_levels - 1, 0)))
    for b in range(B):
        for g in range(H_kv):
            for j in range(nkb):
                lo, hi = j * kv_block, min((j + 1) * kv_block, N)
                for l in range(1, num_levels):
                    P = 1 << l
                    worst = np.inf
                    for s0 in range(lo, hi, P):
                        grp = k[b, g, s0:min(s0 + P, hi)]
                        mean = grp.mean(axis=0)
                        worst = min(worst, float(np.mean([cosine(t, mean) for t in grp])))
                    sim[b, g, j, l - 1] = worst
    return sim


def similarity_cap(sim: np.ndarray, threshold: float) -> np.ndarray:
    """cap[..., j] = the coarsest level l such that every level 1..l has sim >= threshold
    (level 0 always qualifies). The threshold is compared as the float32 the library gets."""
    thr = float(np.float32(threshold))
    cap = np.zeros(sim.shape[:-1], dtype=np.int8)
    ok = np.ones(sim.shape[:-1], dtype=bool)
    for l in range(1, sim.shape[-1] + 1):
        ok &= sim[..., l - 1] >= thr
        cap[ok] = l
    return cap


def apply_similarity_cap(levels: np.ndarray, sim: np.ndarray, threshold: float) -> np.ndarray:
    """A retained block takes min(level, cap of its KV block in the head's KV group);
    pruned blocks stay pruned. levels [B,H,nqb,nkb], sim [B,H_kv,nkb,L-1]."""
    B, H = levels.shape[:2]
    H_kv = sim.shape[1]
    cap = similarity_cap(sim, threshold)                        # [B, H_kv, nkb]
    out = levels.copy()
    for h in range(H):
        c = cap[:, kv_head_of(h, H, H_kv)][:, None, :]          # [B, 1, nkb]
        out[:, h] = np.where(levels[:, h] >= 0, np.minimum(levels[:, h], c), -1)
    return out


# ----------------------------------------------------------------------------
# O4b: ranked (quantile) level assignment, the ablation's alternative rule
# ----------------------------------------------------------------------------

def rank_counts(fractions: Sequence[float], num_levels: int, nkb: int) -> List[int]:
    """Cumulative block counts K_l = floor(f_l * nkb), the product taken in float64.

    skillmd.com "Level assignment" keeps int(num_blocks * keep_ratio) blocks at full
    resolution; a fraction per level generalises that keep ratio to every level."""
    return [int(math.floor(float(f) * nkb)) for f in list(fractions)[:num_levels]]


def block_ranks(z: np.ndarray) -> np.ndarray:
    """rank[..., j] = position of block j in importance order (0 = most important)."""
    R = np.empty(z.shape, dtype=np.int64)
    flat_z = z.reshape(-1, z.shape[-1])
    flat_R = R.reshape(-1, z.shape[-1])
    for r in range(flat_z.shape[0]):
        flat_R[r, importance_order(flat_z[r])] = np.arange(z.shape[-1])
    return R


def assign_levels_ranked(z: np.ndarray, fractions: Sequence[float], num_levels: int,
                         n_dense_prefix: int = 0, kv_block: int = 64, n_rank=None) -> np.ndarray:
    """level_j = min{l : rank_j < K_l}, or -1 (pruned) if no level qualifies; then the
    KV blocks overlapping tokens [0, n_dense_prefix) are set to level 0.

    The pages rank blocks by score and give fixed shares of them to each level
    (skillmd.com "Level assignment"; the top168.com ablation calls this the
    quantile-based rule). Reading: the blocks left after the keep ratio are taken
    in importance order, so a less important block never gets a finer level.

    n_rank: number of blocks the counts are taken of, per query-block row (broadcast
    against z[..., 0]); default: all nkb blocks."""
    rank = block_ranks(z)
    lev = np.full(z.shape, -1, dtype=np.int8)
    if n_rank is None:
        n_rank = np.full(z.shape[:-1], z.shape[-1])
    n_rank = np.broadcast_to(np.asarray(n_rank), z.shape[:-1])
    for l in range(num_levels - 1, -1, -1):
        K = np.vectorize(lambda n: rank_counts(fractions, num_levels, int(n))[l])(n_rank)
        lev[rank < np.asarray(K)[..., None]] = l
    if n_dense_prefix > 0:
        nforce = -(-n_dense_prefix // kv_block)
        lev[..., :nforce] = 0
    return lev


def estimate_mask_ranked(q: np.ndarray, k: np.ndarray, q_block: int, kv_block: int,
                         fractions: Sequence[float], num_levels: int, scale: float,
                         n_dense_prefix: int = 0, causal: bool = False) -> Dict[str, np.ndarray]:
    """The mask step with the ranked rule; scores, p and C as in estimate_mask. Causal:
    the counts are fractions of each row's visible blocks, then apply_causal."""
    N = q.shape[-2]
    qbar = block_means(q, q_block)
    kbar = block_means(k, kv_block)
    z = block_scores(qbar, kbar, block_sizes(N, kv_block), scale)
    n_rank = None
    if causal:
        vis, _ = causal_blocks(N, q_block, kv_block)
        z = np.where(vis, z, -np.inf)
        n_rank = vis.sum(axis=-1)
    p = softmax_rows(z)
    C = cumulative_mass(z, p)
    lev = assign_levels_ranked(z, fractions, num_levels, n_dense_prefix, kv_block, n_rank)
    if causal:
        C, lev = apply_causal(C, lev, N, q_block, kv_block)
    return {"qbar": qbar, "kbar": kbar, "z": z, "p": p, "cmass": C, "rank": block_ranks(z), "levels": lev}


# ----------------------------------------------------------------------------
# O6: pyramid attention under one softmax
# ----------------------------------------------------------------------------

def gather_keys(levels_row: np.ndarray, N: int, kv_block: int,
                kpyr: Sequence[np.ndarray], vpyr: Sequence[np.ndarray], with_last: bool = False,
                with_index: bool = False):
    """Keys, values and log pool sizes that one query block attends to.

    KV block j at level l contributes its pooled rows [j*b/2**l, ceil((j*b + n_j)/2**l))
    of level l (level 0: its tokens). kpyr/vpyr: per-level [N_l, d] arrays.
    with_last: also return the last token each key averages (for causal masking).
    with_index: also return each key's (level, pooled row) (for scattering gradients)."""
    n_kv = block_sizes(N, kv_block)
    ks, vs, lc, last, idx = [], [], [], [], []
    for j, l in enumerate(levels_row):
        l = int(l)
        if l < 0:
            continue
        P = 1 << l
        lo = (j * kv_block) // P
        hi = -(-(j * kv_block + int(n_kv[j])) // P)
        ks.append(kpyr[l][lo:hi])
        vs.append(vpyr[l][lo:hi])
        lc.append(np.log(pool_counts(N, l)[lo:hi].astype(np.float64)))
        last.append(np.minimum((np.arange(lo, hi) + 1) * P, N) - 1)
        idx.append(np.stack([np.full(hi - lo, l), np.arange(lo, hi)], axis=1))
    d = kpyr[0].shape[-1]
    if not ks:
        out = (np.zeros((0, d)), np.zeros((0, d)), np.zeros(0))
        extra = ((np.zeros(0, dtype=np.int64),) if with_last else ()) + \
                ((np.zeros((0, 2), dtype=np.int64),) if with_index else ())
        return out + extra
    out = (np.concatenate(ks), np.concatenate(vs), np.concatenate(lc))
    extra = ((np.concatenate(last),) if with_last else ()) + ((np.concatenate(idx),) if with_index else ())
    return out + extra


def attention_rows(qrows: np.ndarray, keys: np.ndarray, vals: np.ndarray, logc: np.ndarray,
                   scale: float, allowed: np.ndarray = None) -> Tuple[np.ndarray, np.ndarray]:
    """One softmax over mixed-resolution keys; logit = scale*<q, key> + ln(pool count).

    Two passes (max, then exp and sums). allowed [m, keys] (optional): False drops that
    key for that row. Returns (O [m, d], LSE [m]); a row with no key gives O = 0 and
    LSE = -inf."""
    m = qrows.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((m, qrows.shape[1])), np.full(m, -np.inf)
    a = scale * (qrows @ keys.T) + logc[None, :]
    if allowed is not None:
        a = np.where(allowed, a, -np.inf)
    M = a.max(axis=1, keepdims=True)
    empty = ~np.isfinite(M[:, 0])
    M = np.where(np.isfinite(M), M, 0.0)
    e = np.exp(a - M)
    s = e.sum(axis=1, keepdims=True)
    O = (e @ vals) / np.where(s > 0, s, 1.0)
    LSE = (M + np.log(np.where(s > 0, s, 1.0)))[:, 0]
    O[empty] = 0.0
    LSE[empty] = -np.inf
    return O, LSE


def pyramid_attention(q: np.ndarray, kpyr_levels: Sequence[np.ndarray], vpyr_levels: Sequence[np.ndarray],
                      level_map: np.ndarray, q_block: int, kv_block: int, scale: float,
                      items=None, causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Pyramid attention for all (or some) query blocks.

    q [B,H,N,d]; kpyr_levels[l] [B,H_kv,N_l,d] (level 0 = K); level_map [B,H,nqb,nkb].
    ``items``: optional iterable of (b, h, i) query blocks; other rows of the result are NaN.
    causal: query row r sees a key only if every token it averages is at or before r
    (for level 0: token t <= r).
    Returns O [B,H,N,d] and LSE [B,H,N] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    H_kv = kpyr_levels[0].shape[1]
    nqb = -(-N // q_block)
    O = np.full((B, H, N, d), np.nan)
    LSE = np.full((B, H, N), np.nan)
    if items is None:
        items = [(b, h, i) for b in range(B) for h in range(H) for i in range(nqb)]
    for (b, h, i) in items:
        g = kv_head_of(h, H, H_kv)
        keys, vals, logc, last = gather_keys(level_map[b, h, i], N, kv_block, [lv[b, g] for lv in kpyr_levels],
                                             [lv[b, g] for lv in vpyr_levels], with_last=True)
        r0, r1 = i * q_block, min((i + 1) * q_block, N)
        allowed = last[None, :] <= np.arange(r0, r1)[:, None] if causal else None
        O[b, h, r0:r1], LSE[b, h, r0:r1] = attention_rows(q[b, h, r0:r1], keys, vals, logc, scale, allowed)
    return O, LSE


def pyramid_attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, num_levels: int, level_map: np.ndarray,
                          q_block: int, kv_block: int, scale: float, dO: np.ndarray, io_dtype: str = "f32",
                          causal: bool = False) -> Dict[str, np.ndarray]:
    """Gradients of sum(O * dO) with respect to q, k and v, the level map held fixed
    (it is a discrete choice). The pages describe no backward pass; this is the
    gradient of the forward as defined here.

    Per query row r with weights P_rp = exp(a_rp - LSE_r) over its keys p:
      dV_p += P_rp dO_r;  dP_rp = <dO_r, V_p>;  D_r = <dO_r, O_r>;
      dA_rp = P_rp (dP_rp - D_r);  dq_r = scale sum_p dA_rp K_p;  dK_p += scale dA_rp q_r.
    A pooled row is the mean of its c tokens, so its gradient reaches each of them
    divided by c. The pooled keys and values are those the forward used (rounded to
    the I/O dtype). Returns dq [B,H,N,d], dk, dv [B,H_kv,N,d] and the per-level
    pooled gradients dk_levels / dv_levels (level 0 = the tokens' own share)."""
    q = np.asarray(q, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    kp = [np.asarray(k, np.float64)] + [round_to_io(x, io_dtype) for x in build_pyramid(k, num_levels)[1:]]
    vp = [np.asarray(v, np.float64)] + [round_to_io(x, io_dtype) for x in build_pyramid(v, num_levels)[1:]]
    O, LSE = pyramid_attention(q, kp, vp, level_map, q_block, kv_block, scale, causal=causal)
    dq = np.zeros_like(q)
    dkl = [np.zeros_like(x) for x in kp]
    dvl = [np.zeros_like(x) for x in vp]
    nqb = -(-N // q_block)
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, H_kv)
            for i in range(nqb):
                keys, vals, logc, last, idx = gather_keys(level_map[b, h, i], N, kv_block, [x[b, g] for x in kp],
                                                          [x[b, g] for x in vp], with_last=True, with_index=True)
                if keys.shape[0] == 0:
                    continue
                r0, r1 = i * q_block, min((i + 1) * q_block, N)
                qr, dOr, Or = q[b, h, r0:r1], dO[b, h, r0:r1], O[b, h, r0:r1]
                a = scale * (qr @ keys.T) + logc[None, :]
                if causal:
                    a = np.where(last[None, :] <= np.arange(r0, r1)[:, None], a, -np.inf)
                fin = np.isfinite(LSE[b, h, r0:r1])[:, None]
                P = np.where(fin, np.exp(a - np.where(fin, LSE[b, h, r0:r1][:, None], 0.0)), 0.0)
                dP = dOr @ vals.T
                Dr = np.sum(dOr * Or, axis=1, keepdims=True)
                dA = P * (dP - Dr)
                dq[b, h, r0:r1] = scale * (dA @ keys)
                dK = scale * (dA.T @ qr)
                dV = P.T @ dOr
                for l in range(num_levels):
                    sel = idx[:, 0] == l
                    np.add.at(dkl[l][b, g], idx[sel, 1], dK[sel])
                    np.add.at(dvl[l][b, g], idx[sel, 1], dV[sel])
    dk = dkl[0].copy()
    dv = dvl[0].copy()
    for l in range(1, num_levels):
        c = pool_counts(N, l).astype(np.float64)[:, None]
        up = np.arange(N) >> l
        dk += (dkl[l] / c)[:, :, up]
        dv += (dvl[l] / c)[:, :, up]
    return {"dq": dq, "dk": dk, "dv": dv, "dk_levels": dkl, "dv_levels": dvl, "O": O, "LSE": LSE}


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Textbook softmax(scale * Q K^T) V per head (KV head g(h) for query head h);
    causal: row r sees tokens 0..r only."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    O = np.empty((B, H, N, d))
    LSE = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, H_kv)
            allowed = np.tril(np.ones((N, N), dtype=bool)) if causal else None
            O[b, h], LSE[b, h] = attention_rows(q[b, h], np.asarray(k[b, g], np.float64),
                                                np.asarray(v[b, g], np.float64), np.zeros(N), scale, allowed)
    return O, LSE


# ----------------------------------------------------------------------------
# Work accounting
# ----------------------------------------------------------------------------

def effective_flops(level_map: np.ndarray, N: int, q_block: int, kv_block: int, d: int,
                    causal: bool = False) -> float:
    """sum over retained (b,h,i,j) of 4 * m_i * ceil(n_j / 2**l) * d: QK^T and PV on the
    pooled rows actually attended to (no padding, no exp). Causal: only the (query row,
    pooled row) pairs the causal rule lets through are counted."""
    m = block_sizes(N, q_block).astype(np.float64)
    n = block_sizes(N, kv_block)
    lm = level_map.reshape(-1, level_map.shape[-2], level_map.shape[-1])
    total = 0.0
    top = int(lm.max()) if lm.size else -1
    for l in range(top + 1):
        sel = (lm == l).astype(np.float64)                       # [B*H, nqb, nkb]
        if not causal:
            rows_l = (-(-n // (1 << l))).astype(np.float64)      # pooled rows of each block at level l
            total += float(np.einsum("xij,i,j->", sel, m, rows_l))
            continue
        P = 1 << l
        # last token of pooled row p of block j (p < kv_block / P); rows past the block: never seen
        p = np.arange(kv_block // P)
        last = (np.arange(len(n))[:, None] * kv_block + (p[None, :] + 1) * P).astype(np.int64)
        last = np.minimum(last, N) - 1
        last = np.where(p[None, :] * P < n[:, None], last, np.iinfo(np.int64).max // 2)
        # query rows r0 .. r1-1 of block i see pooled row p when r >= last: r1 - max(r0, last) rows
        r0 = (np.arange(len(m)) * q_block)[:, None, None]
        r1 = r0 + m.astype(np.int64)[:, None, None]
        seen = np.clip(r1 - np.maximum(r0, last[None, :, :]), 0, None)
        pairs = seen.sum(axis=-1).astype(np.float64)             # [nqb, nkb]
        total += float(np.einsum("xij,ij->", sel, pairs))
    return 4.0 * d * total


def run_forward(q, k, v, q_block, kv_block, thresholds, num_levels, scale, io_dtype,
                n_dense_prefix=0, items=None, ranked_fractions=None, causal=False):
    """All three steps chained: pyramid (rounded to the I/O dtype), mask, attention.
    With ranked_fractions the mask takes the ranked rule instead of the thresholds."""
    kp = build_pyramid(k, num_levels)
    vp = build_pyramid(v, num_levels)
    kp_io = [np.asarray(k, np.float64)] + [round_to_io(x, io_dtype) for x in kp[1:]]
    vp_io = [np.asarray(v, np.float64)] + [round_to_io(x, io_dtype) for x in vp[1:]]
    if ranked_fractions is None:
        mask = estimate_mask(q, k, q_block, kv_block, thresholds, num_levels, scale, n_dense_prefix, causal)
    else:
        mask = estimate_mask_ranked(q, k, q_block, kv_block, ranked_fractions, num_levels, scale, n_dense_prefix,
                                    causal)
    O, LSE = pyramid_attention(q, kp_io, vp_io, mask["levels"], q_block, kv_block, scale, items, causal)
    return {"kpyr": kp_io, "vpyr": vp_io, "mask": mask, "O": O, "LSE": LSE}
