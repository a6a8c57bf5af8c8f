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

from tests.oracle_heads import lse_tolerance  # noqa: F401  (re-exported for the GPU tests)

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


# ------------------------------------------------------------------------------ backward bounds

BF16_UNIT = 2.0 ** -8          # largest relative rounding error of a bf16 value (8 significant bits)
F32_UNIT = 2.0 ** -24          # relative rounding error of one float32 operation


def backward_bounds(q, k, v, L, level_map, q_block, scale, dO, dtype, causal=False):
    """Element-wise bounds on |gpu - oracle| for dq, dk, dv and the per-level pooled
    gradients of psa_attention_bwd, derived from the roundings the kernels make.

    Per query row r and pooled key p (P = softmax weight, dP = <dO_r, V_p>, D = <dO_r, O_r>,
    dA = P (dP - D), e = 2^-8 the largest relative error of a bf16 rounding (8 significant
    bits), u = 2^-24 of a float32 operation):
      * the forward's O carries |dO| <= e |O| (its bf16 rounding) + e sum_p P |V_p| (P is
        rounded to bf16 for the P.V product), so D is off by dD <= <|dO_r|, that bound>;
      * dP is a float32 sum of d exact bf16 products: ddP <= d u <|dO_r|, |V_p|>;
      * dA is computed in float32 and rounded to bf16: ddA <= e |dA| + P (dD + ddP)
        (+ the effect of an error in P: relative 1e-6 for bf16 I/O, where the logits are
        float32 sums of exact products and lse comes from the forward; for float32 I/O q and
        k are rounded to bf16 first, which moves a logit by up to eps = 2^-8 scale <|q_r|,|K_p|>
        and lse by up to the row's largest eps, so P moves by a factor up to e^(eps+max eps));
      * dq_r = scale sum_p dA K_p, dK_p = scale sum_r dA q_r, dV_p = sum_r P dO_r (P rounded
        to bf16: e P |dO_r|), each a float32 sum of n terms: + n u of its absolute sum; float32
        I/O also rounds K, q and dO to bf16 (+ e of the absolute sum);
      * a pooled row passes 1/c of its gradient to each of its c tokens (nonnegative weights:
        the bounds add the same way), and bf16 outputs add their own rounding, e |g|.
    Returns a dict with bounds "dq", "dk", "dv" [like the gradients] and "dk_levels",
    "dv_levels" (per level, before the 1/c spread; float32 in the library's workspace)."""
    from oracle import psa_oracle as o
    e, u = BF16_UNIT, F32_UNIT
    f32 = dtype == "f32"
    q = np.asarray(q, np.float64)
    dO = np.asarray(dO, np.float64)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    kp = [np.asarray(k, np.float64)] + [o.round_to_io(x, dtype) for x in o.build_pyramid(k, L)[1:]]
    vp = [np.asarray(v, np.float64)] + [o.round_to_io(x, dtype) for x in o.build_pyramid(v, L)[1:]]
    O, LSE = o.pyramid_attention(q, kp, vp, level_map, q_block, 64, scale, causal=causal)
    bq = np.zeros_like(q)
    bkl = [np.zeros_like(x) for x in kp]
    bvl = [np.zeros_like(x) for x in vp]
    nqb = -(-N // q_block)
    n_rows_k = (H // H_kv) * N          # terms summed into one pooled key's gradient, at most
    ext = e if f32 else 0.0
    for b in range(B):
        for h in range(H):
            g = o.kv_head_of(h, H, H_kv)
            for i in range(nqb):
                keys, vals, logc, last, idx = o.gather_keys(level_map[b, h, i], N, 64, [x[b, g] for x in kp],
                                                            [x[b, g] for x in vp], with_last=True, with_index=True)
                if keys.shape[0] == 0:
                    continue
                r0, r1 = i * q_block, min((i + 1) * q_block, N)
                qr, dOr, Or = q[b, h, r0:r1], dO[b, h, r0:r1], O[b, h, r0:r1]
                a = scale * (qr @ keys.T) + logc[None, :]
                if causal:
                    seen = last[None, :] <= np.arange(r0, r1)[:, None]
                    a = np.where(seen, a, -np.inf)
                fin = np.isfinite(LSE[b, h, r0:r1])[:, None]
                P = np.where(fin, np.exp(a - np.where(fin, LSE[b, h, r0:r1][:, None], 0.0)), 0.0)
                dP = dOr @ vals.T
                D = np.sum(dOr * Or, axis=1, keepdims=True)
                dA = P * (dP - D)
                aq, ak, av, ado = np.abs(qr), np.abs(keys), np.abs(vals), np.abs(dOr)
                fwd_err = e * np.abs(Or) + e * (P @ av)
                dD = np.sum(ado * fwd_err, axis=1, keepdims=True)
                ddP = (d * u + 2 * ext) * (ado @ av.T)
                if f32:
                    eps = scale * 2.0 ** -8 * (aq @ ak.T)
                    prel = np.expm1(eps + eps.max(axis=1, keepdims=True))
                else:
                    prel = 1e-6
                ddA = e * np.abs(dA) + P * (dD + ddP) + prel * P * np.abs(dP - D)
                adA = np.abs(dA)
                n = keys.shape[0]
                bq[b, h, r0:r1] = scale * (ddA @ ak) + scale * (n * u + ext) * (adA @ ak)
                bK = scale * (ddA.T @ aq) + scale * (n_rows_k * u + ext) * (adA.T @ aq)
                bV = (e + n_rows_k * u + ext) * (P.T @ ado) + (prel * P).T @ ado
                for l in range(L):
                    sel = idx[:, 0] == l
                    np.add.at(bkl[l][b, g], idx[sel, 1], bK[sel])
                    np.add.at(bvl[l][b, g], idx[sel, 1], bV[sel])
    bk, bv = bkl[0].copy(), bvl[0].copy()
    for l in range(1, L):
        c = o.pool_counts(N, l).astype(np.float64)[:, None]
        up = np.arange(N) >> l
        bk += (bkl[l] / c)[:, :, up]
        bv += (bvl[l] / c)[:, :, up]
    return {"dq": bq, "dk": bk, "dv": bv, "dk_levels": bkl, "dv_levels": bvl}


def check_grad_bound(g, r, bound, label, out_dtype=None):
    """|g - r| <= bound (+ the output's own bf16 rounding, e |r|, when out_dtype is bf16)
    element by element, with an absolute floor of 1e-6 of the largest reference entry.
    Returns the largest ratio of error to bound."""
    assert np.all(np.isfinite(g)), (label, "non-finite gradient")
    tol = bound + (BF16_UNIT * np.abs(r) if out_dtype == "bf16" else 0.0)
    tol = tol + 1e-6 * max(float(np.abs(r).max()), 1e-30)
    err = np.abs(g - r)
    bad = err > tol
    if bad.any():
        at = tuple(int(x) for x in np.argwhere(bad)[0])
        raise AssertionError((label, f"{int(bad.sum())} elements beyond their bound", at, float(err[at]),
                              float(tol[at]), float(r[at])))
    return float((err / tol).max())


def check_fast_vs_exact(lev_fast: np.ndarray, lev_exact: np.ndarray, cmass_exact: np.ndarray, tau, L: int,
                        label: str = ""):
    """The library's fast level pass (no cumulative mass requested) against its exact pass
    (cumulative mass requested). Both add the same integer block masses (p * 2^31 rounded),
    so they find the same mass ranked ahead of every block whatever order they add in, and
    the two level maps must be identical (both are also checked against the oracle by the
    caller). Returns the number of differing entries (0)."""
    diff = np.argwhere(lev_fast != lev_exact)
    bad = [(tuple(int(x) for x in idx), int(lev_fast[tuple(idx)]), int(lev_exact[tuple(idx)]),
            float(cmass_exact[tuple(idx)])) for idx in diff[:5]]
    assert len(diff) == 0, (label, f"{len(diff)} fast/exact level differences", bad)
    return len(diff)
