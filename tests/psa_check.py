"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Tolerances:
  * pyramid: per level ||gpu - oracle||_2 / ||oracle||_2 <= 1e-3 and no element more
    than one unit in the last place of the I/O dtype away from the oracle's rounded mean;
  * block mean keys (float32 output): |gpu - oracle| <= 1e-5 * (1 + |oracle|);
  * level map: identical, except a mismatch at (b,h,i,j) is accepted when the GPU's
    level is one the oracle's own rule gives for some mass C in
    [C_lo - 1e-5, C_hi + 1e-5], where C_lo / C_hi are the oracle's mass ahead of j
    if every block whose score is within 1e-6*|z_j| of z_j were ranked behind /
    ahead of j (so: within 1e-5 of a threshold, or a near-tie reordering);
  * ranked level map: exact per-level counts in every row; a mismatch only where a
    near-tie (scores within 1e-6 relative) could move the block across a count;
  * attention output: max |gpu - oracle| <= 2e-2, mean <= 2e-3, no NaN.
"""
from __future__ import annotations

import numpy as np
import torch

PYR_REL_L2 = 1e-3
KBAR_TOL = 1e-5
MASK_C_TOL = 1e-5
MASK_Z_REL = 1e-6
ATT_MAX_ABS = 2e-2
ATT_MEAN_ABS = 2e-3


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda().contiguous()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    bits = 8 if dtype == "bf16" else 24
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - (bits - 1))


def check_pyramid(gpu_levels, ora_levels, dtype: str, label: str = "", amax: float = 0.0):
    """gpu_levels / ora_levels: lists of arrays for levels 1..L-1 (oracle already rounded).

    bf16 I/O: the float32 sums of bf16 tokens are exact, so every element must be within
    one bf16 ulp of the oracle's correctly rounded mean. float32 I/O: the float32 sum of
    2^l tokens carries up to 2^l roundings of size 2^-24 * amax (amax: largest |input|),
    added to the final rounding."""
    for l, (g, r) in enumerate(zip(gpu_levels, ora_levels), start=1):
        assert g.shape == r.shape, (label, l, g.shape, r.shape)
        assert np.all(np.isfinite(g)), (label, l, "non-finite pyramid values")
        num = np.linalg.norm((g - r).ravel())
        den = max(np.linalg.norm(r.ravel()), 1e-30)
        assert num / den <= PYR_REL_L2, (label, l, num / den)
        err = np.abs(g - r)
        tol = ulp(r, dtype) * 1.0000001
        if dtype == "f32":
            tol = tol + (2 ** l) * 2.0 ** -24 * amax
        bad = err > tol
        assert not bad.any(), (label, l, int(bad.sum()), float(err.max()))


def check_kbar(g: np.ndarray, r: np.ndarray, label: str = ""):
    err = np.abs(g - r)
    assert np.all(err <= KBAR_TOL * (1.0 + np.abs(r))), (label, float(err.max()))


def _level_of(C: float, tau, L: int) -> int:
    for l in range(L):
        if C < np.float64(np.float32(tau[l])):
            return l
    return L   # pruned, ordered as the coarsest


def check_mask(gpu_levels: np.ndarray, ora: dict, tau, L: int, n_dense_prefix: int, kv_block: int = 64,
               label: str = ""):
    """Returns (n_mismatch_accepted). Raises AssertionError on an unaccepted mismatch."""
    ref = ora["levels"]
    assert gpu_levels.shape == ref.shape, (label, gpu_levels.shape, ref.shape)
    diff = np.argwhere(gpu_levels != ref)
    nforce = -(-n_dense_prefix // kv_block) if n_dense_prefix > 0 else 0
    z, p, C = ora["z"], ora["p"], ora["cmass"]
    bad = []
    for (b, h, i, j) in diff:
        if j < nforce:
            bad.append((b, h, i, j, "forced block"))
            continue
        zr, pr = z[b, h, i], p[b, h, i]
        delta = MASK_Z_REL * abs(zr[j])
        others = np.arange(len(zr)) != j
        c_lo = pr[(zr > zr[j] + delta) & others].sum()
        c_hi = pr[(zr >= zr[j] - delta) & others].sum()
        finest = _level_of(c_lo - MASK_C_TOL, tau, L)
        coarsest = _level_of(c_hi + MASK_C_TOL, tau, L)
        gl = int(gpu_levels[b, h, i, j])
        gl = L if gl < 0 else gl
        if not (finest <= gl <= coarsest):
            bad.append((int(b), int(h), int(i), int(j), int(ref[b, h, i, j]), gl, float(C[b, h, i, j])))
    assert not bad, (label, f"{len(bad)} unaccepted level mismatches, first: {bad[:5]}")
    return len(diff)


def check_mask_ranked(gpu_levels: np.ndarray, ora: dict, counts, L: int, n_dense_prefix: int,
                      kv_block: int = 64, label: str = "", check_counts: bool = True):
    """Ranked rule. Every row must hold exactly K_l - K_{l-1} blocks at level l (checked
    on rows without forced blocks) -- unique whatever the order of near-ties. A block
    may differ from the oracle only when its level is the rule's level for some rank in
    [r_lo, r_hi], where r_lo / r_hi count the other blocks whose score is above
    z_j + 1e-6*|z_j| / at least z_j - 1e-6*|z_j| (a near-tie reordering).
    Returns the number of accepted mismatches."""
    ref = ora["levels"]
    assert gpu_levels.shape == ref.shape, (label, gpu_levels.shape, ref.shape)
    K = list(counts[:L])

    def level_of_rank(r):
        for l in range(L):
            if r < K[l]:
                return l
        return L

    if n_dense_prefix == 0 and check_counts:
        flat = gpu_levels.reshape(-1, gpu_levels.shape[-1])
        for l in range(L):
            want = K[l] - (K[l - 1] if l else 0)
            have = (flat == l).sum(axis=1)
            assert np.all(have == max(want, 0)), (label, l, want, np.unique(have))
    nforce = -(-n_dense_prefix // kv_block) if n_dense_prefix > 0 else 0
    z = ora["z"]
    bad = []
    diff = np.argwhere(gpu_levels != ref)
    for (b, h, i, j) in diff:
        if j < nforce:
            bad.append((b, h, i, j, "forced block"))
            continue
        zr = z[b, h, i]
        delta = MASK_Z_REL * abs(zr[j])
        others = np.arange(len(zr)) != j
        r_lo = int(((zr > zr[j] + delta) & others).sum())
        r_hi = int(((zr >= zr[j] - delta) & others).sum())
        gl = int(gpu_levels[b, h, i, j])
        gl = L if gl < 0 else gl
        if not (level_of_rank(r_lo) <= gl <= level_of_rank(r_hi)):
            bad.append((int(b), int(h), int(i), int(j), int(ref[b, h, i, j]), gl, r_lo, r_hi))
    assert not bad, (label, f"{len(bad)} unaccepted level mismatches, first: {bad[:5]}")
    return len(diff)


def check_cmass(gpu_C: np.ndarray, ora: dict, label: str = ""):
    """GPU cumulative mass vs the oracle's: within 1e-5, or inside the near-tie interval
    [C_lo - 1e-5, C_hi + 1e-5] (see check_mask) where a near-tie reorders blocks."""
    C, z, p = ora["cmass"], ora["z"], ora["p"]
    far = np.argwhere(np.abs(gpu_C - C) > MASK_C_TOL)
    bad = []
    for (b, h, i, j) in far:
        zr, pr = z[b, h, i], p[b, h, i]
        delta = MASK_Z_REL * abs(zr[j])
        others = np.arange(len(zr)) != j
        c_lo = pr[(zr > zr[j] + delta) & others].sum()
        c_hi = pr[(zr >= zr[j] - delta) & others].sum()
        g = gpu_C[b, h, i, j]
        if not (c_lo - MASK_C_TOL <= g <= c_hi + MASK_C_TOL):
            bad.append((int(b), int(h), int(i), int(j), float(g), float(C[b, h, i, j]), float(c_lo), float(c_hi)))
    assert not bad, (label, f"{len(bad)} cumulative masses off, first: {bad[:5]}")
    return len(far)


def lse_tolerance(q: np.ndarray, k: np.ndarray, scale: float, dtype: str) -> np.ndarray:
    """Per-row bound on |lse_gpu - lse_oracle| ([B, H, N]).

    bf16 I/O: the matrix cores multiply the exact bf16 inputs and accumulate in float32,
    so only float32 accumulation error remains (1e-3 is generous). float32 I/O: q and k are
    rounded to bf16 first, so every product q_c*k_c carries a relative error below 2^-8 and
    every logit of row r moves by at most 2^-8 * scale * sum_c |q_rc| * max_t |k_tc|;
    the log-sum-exp moves by at most the largest logit change."""
    B, H, N, d = q.shape
    tol = np.full((B, H, N), 1e-3)
    if dtype == "f32":
        H_kv = k.shape[1]
        kmax = np.abs(k).max(axis=2)                                   # [B, H_kv, d]
        kmax_h = np.repeat(kmax, H // H_kv, axis=1)                    # [B, H, d]
        tol += 2.0 ** -8 * scale * np.einsum("bhnd,bhd->bhn", np.abs(q), kmax_h)
    return tol


def check_attention(o_gpu: np.ndarray, o_ora: np.ndarray, label: str = "", rows=None):
    """Compare O on the rows the oracle computed (non-NaN rows of o_ora, or `rows` mask)."""
    sel = ~np.isnan(o_ora[..., 0]) if rows is None else rows
    g, r = o_gpu[sel], o_ora[sel]
    assert g.size > 0, (label, "no rows compared")
    assert not np.isnan(g).any(), (label, "NaN in GPU output")
    err = np.abs(g - r)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= ATT_MAX_ABS and mean <= ATT_MEAN_ABS, (label, mx, mean)
    return mx, mean
