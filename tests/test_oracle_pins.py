"""Pins for the CPU oracle: every check here is independent of the oracle's own code
(closed forms, brute force with explicit loops, invariants the mathematics fixes,
a hand-derived worked example, library routines for textbook special cases)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import psa_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------- rounding

def test_bf16_rounding_matches_torch_on_float32_values():
    x = rng(0).standard_normal(20000).astype(np.float32) * np.float32(3.0)
    x = np.concatenate([x, np.float32([1.0, 65504.0, 1e-30, -7.5e-39, 3.0e38])])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = o.round_to_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even mantissa is 1.
    assert o.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert o.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert o.round_to_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7


# ----------------------------------------------------------------------------- pyramid (O1)

def brute_pool(x, level):
    N, d = x.shape
    P = 2 ** level
    rows = []
    for p in range(-(-N // P)):
        toks = list(range(p * P, min(p * P + P, N)))
        rows.append([math.fsum(x[t, c] for t in toks) / len(toks) for c in range(d)])
    return np.array(rows)


@pytest.mark.parametrize("N", [64, 130, 2045, 8])
def test_pool_brute_force(N):
    x = rng(N).standard_normal((N, 5))
    for l in range(4):
        np.testing.assert_allclose(o.pool_level(x, l), brute_pool(x, l), rtol=0, atol=1e-13)


def test_pool_constant_and_ramp_closed_forms():
    N = 2045
    const = np.full((1, 3, N, 4), 2.75)
    for lv in o.build_pyramid(const, 4):
        np.testing.assert_allclose(lv, 2.75, rtol=0, atol=1e-14)
    a, b = -1.5, 0.25
    t = np.arange(N, dtype=np.float64)
    ramp = (a + b * t)[:, None] * np.ones((1, 2))
    for l in range(4):
        P = 2 ** l
        starts = np.arange(-(-N // P)) * P
        c = np.minimum(starts + P, N) - starts
        expect = a + b * (starts + (c - 1) / 2.0)
        np.testing.assert_allclose(o.pool_level(ramp, l)[:, 0], expect, rtol=0, atol=1e-11)
        np.testing.assert_array_equal(o.pool_counts(N, l), c)


def test_progressive_equals_direct():
    x = rng(5).standard_normal((2, 2045, 3))
    prev, prev_c = x, np.ones(2045)
    for l in range(1, 4):
        R = prev.shape[-2]
        nxt = []
        cnt = []
        for p in range(-(-R // 2)):
            idx = [r for r in (2 * p, 2 * p + 1) if r < R]
            w = prev_c[idx]
            nxt.append(sum(prev[:, r] * prev_c[r] for r in idx) / w.sum())
            cnt.append(w.sum())
        prev, prev_c = np.stack(nxt, axis=1), np.array(cnt)
        np.testing.assert_allclose(o.pool_level(x, l), prev, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(o.pool_counts(2045, l), prev_c)


def test_pyramid_layout_offsets():
    N = 2045
    x = rng(1).standard_normal((1, 1, N, 2))
    levels = o.build_pyramid(x, 4)
    cat = o.pyramid_concat(levels)
    offs = o.pyramid_row_offsets(N, 4)
    assert cat.shape[-2] == sum(-(-N // 2 ** l) for l in (1, 2, 3))
    for l in (1, 2, 3):
        R = -(-N // 2 ** l)
        np.testing.assert_array_equal(cat[..., offs[l]:offs[l] + R, :], levels[l])


# ----------------------------------------------------------------------------- means, scores (O2, O3)

def test_block_means_brute_force():
    x = rng(2).standard_normal((130, 3))
    got = o.block_means(x, 64)
    for j, (lo, hi) in enumerate([(0, 64), (64, 128), (128, 130)]):
        for c in range(3):
            assert abs(got[j, c] - math.fsum(x[lo:hi, c]) / (hi - lo)) < 1e-14
    np.testing.assert_array_equal(o.block_sizes(130, 64), [64, 64, 2])


def test_scores_brute_force_and_softmax_sums_to_one():
    B, H, Hkv, d = 1, 4, 2, 6
    qbar = rng(3).standard_normal((B, H, 3, d))
    kbar = rng(4).standard_normal((B, Hkv, 5, d))
    n = np.array([64, 64, 64, 64, 7])
    s = 0.37
    z = o.block_scores(qbar, kbar, n, s)
    for h in range(H):
        g = h // 2
        for i in range(3):
            for j in range(5):
                ref = s * math.fsum(qbar[0, h, i, c] * kbar[0, g, j, c] for c in range(d)) + math.log(n[j])
                assert abs(z[0, h, i, j] - ref) < 1e-13
    p = o.softmax_rows(z)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-15)
    # softmax: ratios are exp of score differences
    np.testing.assert_allclose(p[..., 1] / p[..., 0], np.exp(z[..., 1] - z[..., 0]), rtol=1e-12)


def test_mask_shift_invariance():
    q = rng(6).standard_normal((1, 2, 256, 8))
    k = rng(7).standard_normal((1, 2, 256, 8))
    tau = (0.3, 0.5, 0.7, 0.9)
    m1 = o.estimate_mask(q, k, 64, 64, tau, 4, 0.35)
    m2 = o.estimate_mask(q, k + rng(8).standard_normal(8) * 3.0, 64, 64, tau, 4, 0.35)
    np.testing.assert_allclose(m1["p"], m2["p"], rtol=1e-10, atol=1e-14)
    np.testing.assert_array_equal(m1["levels"], m2["levels"])


# ----------------------------------------------------------------------------- mass and levels (O4, O5)

def brute_cmass(z_row, p_row):
    n = len(z_row)
    out = []
    for j in range(n):
        ahead = [p_row[k] for k in range(n)
                 if z_row[k] > z_row[j] or (z_row[k] == z_row[j] and k < j)]
        out.append(math.fsum(ahead))
    return np.array(out)


def test_cumulative_mass_brute_force_with_ties():
    z = rng(9).standard_normal((6, 40))
    z[:, 5] = z[:, 17]          # exact ties, broken by index
    z[:, 30] = z[:, 2]
    p = o.softmax_rows(z)
    C = o.cumulative_mass(z, p)
    for r in range(6):
        np.testing.assert_allclose(C[r], brute_cmass(z[r], p[r]), rtol=0, atol=1e-14)
    # the top block has no mass ahead of it
    top = np.argmax(z, axis=1)
    assert np.all(C[np.arange(6), top] == 0.0)


def test_levels_brute_force():
    C = rng(10).uniform(0, 1, size=(3, 50))
    tau = (0.1, 0.1, 0.45, 0.8)
    lev = o.assign_levels(C, tau, 4)
    for idx in np.ndindex(C.shape):
        ok = [l for l in range(4) if C[idx] < np.float32(tau[l])]
        assert lev[idx] == (min(ok) if ok else -1)
    assert not np.any(lev == 1)          # tau_1 == tau_0: level 1 is empty


def test_uniform_scores_closed_form():
    # Q = 0 and N a multiple of the block: every score equals ln 64, p = 1/nkb, ties broken
    # by index, so C_j = j/nkb and level_j = min{l : j/nkb < tau_l}.
    N, nkb = 2048, 32
    q = np.zeros((1, 1, N, 4))
    k = rng(11).standard_normal((1, 1, N, 4))
    tau = (0.25, 0.5, 0.625, 0.875)
    m = o.estimate_mask(q, k, 64, 64, tau, 4, 0.5)
    j = np.arange(nkb)
    np.testing.assert_allclose(m["cmass"][0, 0, 0], j / nkb, rtol=0, atol=1e-15)
    expect = np.array([min([l for l in range(4) if jj / nkb < tau[l]], default=-1) for jj in j])
    np.testing.assert_array_equal(m["levels"][0, 0, 0], expect)
    np.testing.assert_array_equal(m["levels"][0, 0, 0][:8], 0)
    np.testing.assert_array_equal(m["levels"][0, 0, 0][28:], -1)


def test_levels_monotone_in_thresholds_and_all_ones():
    q = rng(12).standard_normal((1, 2, 512, 8))
    k = rng(13).standard_normal((1, 2, 512, 8))
    base = np.array([0.2, 0.4, 0.6, 0.8])
    lev0 = o.estimate_mask(q, k, 64, 64, base, 4, 0.35)["levels"].astype(int)
    lev0[lev0 < 0] = 99
    for l in range(4):
        up = base.copy()
        up[l:] = np.minimum(up[l:] + 0.15, 1.0)
        lev1 = o.estimate_mask(q, k, 64, 64, up, 4, 0.35)["levels"].astype(int)
        lev1[lev1 < 0] = 99
        assert np.all(lev1 <= lev0)
    ones = o.estimate_mask(q, k, 64, 64, (1, 1, 1, 1), 4, 0.35)["levels"]
    assert np.all(ones == 0)


def test_dense_prefix_forced_after_ranking():
    q = rng(14).standard_normal((1, 1, 640, 8))
    k = rng(15).standard_normal((1, 1, 640, 8))
    tau = (0.1, 0.2, 0.3, 0.4)
    plain = o.estimate_mask(q, k, 128, 64, tau, 4, 0.35)
    forced = o.estimate_mask(q, k, 128, 64, tau, 4, 0.35, n_dense_prefix=130)
    assert np.all(forced["levels"][..., :3] == 0)
    np.testing.assert_array_equal(forced["levels"][..., 3:], plain["levels"][..., 3:])
    np.testing.assert_array_equal(forced["cmass"], plain["cmass"])


# ----------------------------------------------------------------------------- ranked rule (O4b)

def brute_rank(z_row, j):
    return sum(1 for k in range(len(z_row)) if z_row[k] > z_row[j] or (z_row[k] == z_row[j] and k < j))


def test_rank_counts_follow_the_keep_ratio_expression():
    # skillmd.com "Level assignment" keeps int(num_blocks * keep_ratio) blocks
    for nkb, f in [(10, 0.7), (100, 0.29), (30, 0.1), (512, 0.1), (278, 0.4), (7, 1.0), (7, 0.0)]:
        assert o.rank_counts([f], 1, nkb) == [int(nkb * f)]
    assert o.rank_counts([0.1, 0.4, 0.7, 1.0], 2, 30) == [3, 12]


def test_ranked_levels_brute_force_with_ties():
    z = np.round(rng(40).standard_normal((5, 37)), 1)       # many exact ties
    fr = (0.05, 0.3, 0.3, 0.8)                                # level 2 empty
    lev = o.assign_levels_ranked(z, fr, 4)
    K = [int(37 * f) for f in fr]
    for r in range(5):
        for j in range(37):
            rk = brute_rank(z[r], j)
            ok = [l for l in range(4) if rk < K[l]]
            assert lev[r, j] == (min(ok) if ok else -1)
    assert not np.any(lev == 2)
    for l, n in enumerate(np.diff([0] + K)):
        assert np.all((lev == l).sum(axis=1) == n)


def test_ranked_keep_ratio_split_into_thirds():
    # The page's rule: the top int(n * 0.1) blocks at level 0, the rest split into
    # thirds for levels 1..3 (taken in score order, the reading stated in the oracle).
    n = 30
    z = rng(41).standard_normal((1, n))
    order = np.argsort(-z[0], kind="stable")
    keep = order[:int(n * 0.1)]
    rest = order[int(n * 0.1):]
    expect = np.empty(n, dtype=int)
    expect[keep] = 0
    expect[rest[:len(rest) // 3]] = 1
    expect[rest[len(rest) // 3:2 * len(rest) // 3]] = 2
    expect[rest[2 * len(rest) // 3:]] = 3
    lev = o.assign_levels_ranked(z, (0.1, 0.4, 0.7, 1.0), 4)
    np.testing.assert_array_equal(lev[0], expect)


def test_ranked_binary_top_k_is_stable_argsort_prefix():
    z = rng(42).standard_normal((4, 3, 50))
    z[..., 7] = z[..., 11]
    for k in (0, 1, 13, 50):
        lev = o.assign_levels_ranked(z, [k / 50], 1)
        for idx in np.ndindex(4, 3):
            top = np.sort(np.argsort(-z[idx], kind="stable")[:k])
            np.testing.assert_array_equal(np.flatnonzero(lev[idx] == 0), top)
            assert np.all(lev[idx][lev[idx] != 0] == -1)
    zt = torch.from_numpy(rng(43).standard_normal((6, 40)))
    lev = o.assign_levels_ranked(zt.numpy(), [10 / 40], 1)
    for r in range(6):
        ti = np.sort(torch.topk(zt[r], 10).indices.numpy())
        np.testing.assert_array_equal(np.flatnonzero(lev[r] == 0), ti)


def test_ranked_uniform_scores_closed_form():
    # Q = 0: every score is ln 64, ranks follow the block index
    N, nkb = 2048, 32
    q = np.zeros((1, 1, N, 4))
    k = rng(44).standard_normal((1, 1, N, 4))
    fr = (0.125, 0.5, 0.5, 0.75)
    m = o.estimate_mask_ranked(q, k, 64, 64, fr, 4, 0.5)
    j = np.arange(nkb)
    K = [4, 16, 16, 24]
    expect = np.array([min([l for l in range(4) if jj < K[l]], default=-1) for jj in j])
    np.testing.assert_array_equal(m["levels"][0, 0, 0], expect)
    np.testing.assert_array_equal(m["rank"][0, 0, 0], j)


def test_ranked_equals_threshold_rule_at_equal_counts():
    # Both rules give each level a prefix of the same importance order, so with the
    # per-level counts the thresholds select, the ranked rule gives the same map.
    q = rng(45).standard_normal((1, 1, 128, 8))
    k = rng(46).standard_normal((1, 1, 2048, 8))
    q = np.concatenate([q] * 16, axis=2)
    tau = (0.3, 0.5, 0.7, 0.9)
    thr = o.estimate_mask(q, k, 2048, 64, tau, 4, 0.9)
    assert thr["levels"].shape == (1, 1, 1, 32)
    C = thr["cmass"][0, 0, 0]
    fr = [float(np.sum(C < np.float32(t))) / 32 for t in tau]
    ranked = o.estimate_mask_ranked(q, k, 2048, 64, fr, 4, 0.9)
    assert len(set(fr)) == 4
    np.testing.assert_array_equal(ranked["levels"], thr["levels"])


def test_ranked_dense_prefix_forced_after_ranking():
    q = rng(47).standard_normal((1, 2, 640, 8))
    k = rng(48).standard_normal((1, 2, 640, 8))
    fr = (0.2, 0.4, 0.6, 0.8)
    plain = o.estimate_mask_ranked(q, k, 128, 64, fr, 4, 0.35)
    forced = o.estimate_mask_ranked(q, k, 128, 64, fr, 4, 0.35, n_dense_prefix=129)
    assert np.all(forced["levels"][..., :3] == 0)
    np.testing.assert_array_equal(forced["levels"][..., 3:], plain["levels"][..., 3:])
    np.testing.assert_array_equal(forced["rank"], plain["rank"])


# ----------------------------------------------------------------------------- cosine-similarity constraint

def brute_group_score(keys):
    """mean over the group's tokens of cos(token, group mean), in plain float loops"""
    d = len(keys[0])
    mean = [math.fsum(k[c] for k in keys) / len(keys) for c in range(d)]
    nm = math.sqrt(math.fsum(x * x for x in mean))
    out = []
    for k in keys:
        nk = math.sqrt(math.fsum(x * x for x in k))
        out.append(0.0 if nk == 0 or nm == 0 else math.fsum(a * b for a, b in zip(k, mean)) / (nk * nm))
    return math.fsum(out) / len(out)


def test_similarity_brute_force_with_ragged_block():
    k = rng(70).standard_normal((1, 2, 150, 5))          # blocks of 64, 64, 22 tokens
    sim = o.key_similarity(k, 64, 4)
    assert sim.shape == (1, 2, 3, 3)
    for g, j, l in np.ndindex(2, 3, 3):
        lo, hi, P = 64 * j, min(64 * j + 64, 150), 2 ** (l + 1)
        ref = min(brute_group_score(list(k[0, g, s0:min(s0 + P, hi)])) for s0 in range(lo, hi, P))
        assert abs(sim[0, g, j, l] - ref) < 1e-12


def test_similarity_closed_forms():
    # level-1 pairs of unit keys at angle phi: the mean bisects them, each cosine is cos(phi/2)
    d, phis = 2, np.linspace(0.1, 3.0, 32)
    k = np.zeros((1, 1, 64, d))
    for p, phi in enumerate(phis):
        k[0, 0, 2 * p] = (1.0, 0.0)
        k[0, 0, 2 * p + 1] = (math.cos(phi), math.sin(phi))
    sim = o.key_similarity(k, 64, 2)
    assert abs(sim[0, 0, 0, 0] - math.cos(phis.max() / 2)) < 1e-12
    # identical keys: every level scores 1; opposite keys: the mean is zero, cosine 0
    same = np.tile(rng(71).standard_normal((1, 1, 1, 6)), (1, 1, 64, 1))
    np.testing.assert_allclose(o.key_similarity(same, 64, 4), 1.0, rtol=0, atol=1e-12)
    opp = same.copy()
    opp[0, 0, 1::2] *= -1
    assert np.all(o.key_similarity(opp, 64, 4)[0, 0, 0] == 0.0)


def test_similarity_invariances():
    k = rng(72).standard_normal((1, 1, 128, 6))
    base = o.key_similarity(k, 64, 4)
    Q, _ = np.linalg.qr(rng(73).standard_normal((6, 6)))
    np.testing.assert_allclose(o.key_similarity(k @ Q, 64, 4), base, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o.key_similarity(3.5 * k, 64, 4), base, rtol=0, atol=1e-12)


def test_similarity_cap_rules():
    sim = np.array([[[[0.9, 0.8, 0.7], [0.5, 0.95, 0.95], [0.99, 0.99, 0.2], [1.0, 1.0, 1.0]]]])
    np.testing.assert_array_equal(o.similarity_cap(sim, 0.75), [[[2, 0, 2, 3]]])
    np.testing.assert_array_equal(o.similarity_cap(sim, -1.0), [[[3, 3, 3, 3]]])
    np.testing.assert_array_equal(o.similarity_cap(sim, 1.5), [[[0, 0, 0, 0]]])
    lev = np.array([[[[3, 3, 3, 3], [-1, 1, 0, 2]]]], dtype=np.int8)          # B1 H1 nqb2 nkb4
    np.testing.assert_array_equal(o.apply_similarity_cap(lev, sim, 0.75), [[[[2, 0, 2, 3], [-1, 0, 0, 2]]]])


def test_similarity_cap_monotone_and_gqa():
    k = rng(74).standard_normal((1, 2, 512, 8))
    q = rng(75).standard_normal((1, 4, 512, 8))
    lev = o.estimate_mask(q, k, 64, 64, (0.2, 0.4, 0.6, 0.8), 4, 0.4)["levels"]
    sim = o.key_similarity(k, 64, 4)
    prev = lev.astype(int)
    for thr in (-1.0, 0.3, 0.5, 0.6, 0.7, 1.01):
        cur = o.apply_similarity_cap(lev, sim, thr).astype(int)
        assert np.all((cur >= 0) == (lev >= 0))                                 # pruning unchanged
        assert np.all(cur[lev >= 0] <= prev[lev >= 0])                          # never coarser
        prev = cur
    assert np.all(prev[lev >= 0] == 0)
    cap = o.similarity_cap(sim, 0.5)
    out = o.apply_similarity_cap(lev, sim, 0.5)
    for h in range(4):                                                          # heads 0,1 -> KV 0
        g = h // 2
        exp = np.where(lev[0, h] >= 0, np.minimum(lev[0, h], cap[0, g][None, :]), -1)
        np.testing.assert_array_equal(out[0, h], exp)


# ----------------------------------------------------------------------------- causal use

def test_causal_blocks_closed_form():
    vis, diag = o.causal_blocks(300, 128, 64)            # 3 query blocks, 5 KV blocks (last one ragged)
    np.testing.assert_array_equal(vis, [[1, 1, 0, 0, 0], [1, 1, 1, 1, 0], [1, 1, 1, 1, 1]])
    np.testing.assert_array_equal(diag, [[1, 1, 0, 0, 0], [0, 0, 1, 1, 0], [0, 0, 0, 0, 1]])
    vis, diag = o.causal_blocks(256, 64, 64)
    np.testing.assert_array_equal(vis, np.tril(np.ones((4, 4), bool)))
    np.testing.assert_array_equal(diag, np.eye(4, dtype=bool))


def test_causal_dense_map_equals_torch_causal_sdpa():
    q, k, v = small_case(60, N=200, d=8)
    s = 0.4
    O_ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=s).numpy()
    lev = np.zeros((1, 2, 4, 4), dtype=np.int8)           # every block at level 0: the causal rule masks
    kp, vp = o.build_pyramid(k, 4), o.build_pyramid(v, 4)
    O, LSE = o.pyramid_attention(q, kp, vp, lev, 64, 64, s, causal=True)
    np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
    Od, LSEd = o.dense_attention(q, k, v, s, causal=True)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, LSEd, rtol=0, atol=1e-12)
    # row 0 sees only token 0
    np.testing.assert_allclose(O[0, :, 0], v[0, :, 0], rtol=0, atol=1e-15)


def test_causal_row_equals_attention_on_truncated_sequence():
    # With the causal mask's map (blocks reaching the query block at level 0, earlier blocks
    # pooled or pruned), row r is pyramid attention over the first r+1 tokens only.
    N, d, bq = 333, 8, 128
    q, k, v = small_case(61, N=N, d=d)
    s = 0.35
    m = o.estimate_mask(q, k, bq, 64, (0.3, 0.5, 0.7, 0.8), 4, s, causal=True)
    lev = m["levels"]
    O, LSE = o.pyramid_attention(q, o.build_pyramid(k, 4), o.build_pyramid(v, 4), lev, bq, 64, s, causal=True)
    for r in (0, 5, 63, 64, 127, 128, 200, 255, 256, 300, 332):
        i = r // bq
        kt, vt = k[:, :, :r + 1], v[:, :, :r + 1]
        nkb_t = -(-(r + 1) // 64)
        lev_t = np.full((1, 2, 1, nkb_t), -1, dtype=np.int8)
        lev_t[..., 0, :] = lev[:, :, i, :nkb_t]
        qt = np.zeros((1, 2, r + 1, d))
        qt[:, :, r] = q[:, :, r]
        Ot, LSEt = o.pyramid_attention(qt, o.build_pyramid(kt, 4), o.build_pyramid(vt, 4), lev_t, r + 1, 64, s)
        np.testing.assert_allclose(O[:, :, r], Ot[:, :, r], rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[:, :, r], LSEt[:, :, r], rtol=0, atol=1e-12)


def test_causal_pooled_key_needs_all_its_tokens():
    # A pooled key is visible to row r only when every token it averages is <= r.
    N, d = 128, 4
    q, k, v = small_case(62, H=1, Hkv=1, N=N, d=d)
    lev = np.array([[[[0, -1], [0, 2]]]], dtype=np.int8)   # q-block 1 sees block 1 at level 2
    kp, vp = o.build_pyramid(k, 3), o.build_pyramid(v, 3)
    O, LSE = o.pyramid_attention(q, kp, vp, lev, 64, 64, 0.5, causal=True)
    for r in (64, 66, 67, 70, 127):
        keys = [k[0, 0, t] for t in range(64)]
        vals = [v[0, 0, t] for t in range(64)]
        wl = [0.0] * 64
        for p in range(16, 32):                            # level-2 rows of block 1: tokens 4p..4p+3
            if 4 * p + 3 <= r:
                keys.append(kp[2][0, 0, p])
                vals.append(vp[2][0, 0, p])
                wl.append(math.log(4))
        o_ref, lse_ref = brute_attention_row(q[0, 0, r], keys, vals, wl, 0.5)
        np.testing.assert_allclose(O[0, 0, r], o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(LSE[0, 0, r], lse_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("rule", ["threshold", "ranked"])
def test_causal_mask_equals_mask_of_truncated_problem(rule):
    # The causal mask row of query block i is the non-causal mask of the problem cut after
    # the last KV block that block can see, with the blocks reaching its rows set to level 0.
    N, d, bq = 700, 8, 128
    q = rng(63).standard_normal((1, 2, N, d))
    k = rng(64).standard_normal((1, 2, N, d))
    s, tau, fr = 0.45, (0.25, 0.5, 0.7, 0.85), (0.1, 0.3, 0.5, 0.7)
    if rule == "threshold":
        m = o.estimate_mask(q, k, bq, 64, tau, 4, s, causal=True)
    else:
        m = o.estimate_mask_ranked(q, k, bq, 64, fr, 4, s, causal=True)
    vis, diag = o.causal_blocks(N, bq, 64)
    assert np.all(m["levels"][..., ~vis] == -1) and np.all(m["levels"][..., diag] == 0)
    assert np.all(m["cmass"][..., ~vis] == 1.0)
    np.testing.assert_allclose(m["p"].sum(-1), 1.0, rtol=0, atol=1e-12)
    for i in range(vis.shape[0]):
        nv = int(vis[i].sum())
        Nt = min(N, 64 * nv)
        if rule == "threshold":
            t = o.estimate_mask(q[:, :, :Nt], k[:, :, :Nt], bq, 64, tau, 4, s)
        else:
            t = o.estimate_mask_ranked(q[:, :, :Nt], k[:, :, :Nt], bq, 64, fr, 4, s)
        np.testing.assert_allclose(m["cmass"][:, :, i, :nv], t["cmass"][:, :, i], rtol=0, atol=1e-13)
        expect = t["levels"][:, :, i].copy()
        expect[..., diag[i, :nv]] = 0
        np.testing.assert_array_equal(m["levels"][:, :, i, :nv], expect)


def test_causal_effective_flops_brute_force():
    r = rng(67)
    for N, bq in [(333, 128), (700, 64), (64, 128), (1, 64)]:
        nqb, nkb = -(-N // bq), -(-N // 64)
        lev = r.integers(-1, 4, size=(1, 2, nqb, nkb)).astype(np.int8)
        pairs = 0
        for h, i, j in np.ndindex(2, nqb, nkb):
            l = int(lev[0, h, i, j])
            if l < 0:
                continue
            P, nj = 1 << l, min(64, N - 64 * j)
            for prow in range((64 * j) // P, -(-(64 * j + nj) // P)):
                last = min((prow + 1) * P, N) - 1
                pairs += sum(1 for row in range(i * bq, min((i + 1) * bq, N)) if row >= last)
        assert o.effective_flops(lev, N, bq, 64, 8, causal=True) == 4 * 8 * pairs


def test_causal_effective_flops_closed_form():
    N, d = 300, 8
    lev = np.zeros((1, 1, 3, 5), dtype=np.int8)
    assert o.effective_flops(lev, N, 128, 64, d, causal=True) == 4 * d * N * (N + 1) / 2
    lev2 = o.estimate_mask(rng(65).standard_normal((1, 1, N, d)), rng(66).standard_normal((1, 1, N, d)),
                           128, 64, (0.2, 0.4, 0.6, 0.8), 4, 0.5, causal=True)["levels"]
    assert o.effective_flops(lev2, N, 128, 64, d, causal=True) < o.effective_flops(lev2, N, 128, 64, d)


# ----------------------------------------------------------------------------- attention (O6)

def brute_attention_row(qr, keys, vals, weights_log, scale):
    a = [scale * math.fsum(qr[c] * key[c] for c in range(len(qr))) + wl for key, wl in zip(keys, weights_log)]
    M = max(a)
    e = [math.exp(x - M) for x in a]
    s = math.fsum(e)
    out = [math.fsum(e[t] * vals[t][c] for t in range(len(e))) / s for c in range(len(vals[0]))]
    return np.array(out), M + math.log(s)


def small_case(seed, B=1, H=2, Hkv=2, N=256, d=8):
    r = rng(seed)
    return (r.standard_normal((B, H, N, d)), r.standard_normal((B, Hkv, N, d)),
            r.standard_normal((B, Hkv, N, d)))


def test_all_level0_equals_dense_brute_force():
    q, k, v = small_case(20, N=130, d=5)
    s = 0.41
    kp, vp = o.build_pyramid(k, 4), o.build_pyramid(v, 4)
    lev = np.zeros((1, 2, 3, 3), dtype=np.int8)
    O, L = o.pyramid_attention(q, kp, vp, lev, 64, 64, s)
    for h in range(2):
        for r in (0, 63, 64, 129):
            ref_o, ref_l = brute_attention_row(q[0, h, r], k[0, h], v[0, h], [0.0] * 130, s)
            np.testing.assert_allclose(O[0, h, r], ref_o, rtol=0, atol=1e-12)
            assert abs(L[0, h, r] - ref_l) < 1e-12
    Od, Ld = o.dense_attention(q, k, v, s)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-12)


def test_expanded_key_equivalence():
    # A pooled row of count c acts exactly like c copies of the pooled key/value in dense attention.
    N = 2045
    q, k, v = small_case(21, N=N, d=6)
    s = 0.3
    kp, vp = o.build_pyramid(k, 4), o.build_pyramid(v, 4)
    nkb = -(-N // 64)
    lev = rng(22).integers(-1, 4, size=(1, 2, 16, nkb)).astype(np.int8)
    lev[..., 0] = 0
    O, L = o.pyramid_attention(q, kp, vp, lev, 128, 64, s, items=[(0, 1, 3), (0, 0, 15)])
    for (h, i) in [(1, 3), (0, 15)]:
        ek, ev = [], []
        for j in range(nkb):
            l = int(lev[0, h, i, j])
            if l < 0:
                continue
            P = 2 ** l
            for t in range(j * 64, min(j * 64 + 64, N)):   # each token contributes its pooled row once
                ek.append(kp[l][0, h, t // P])
                ev.append(vp[l][0, h, t // P])
        for r in (i * 128, min(i * 128 + 127, N - 1)):
            ref_o, ref_l = brute_attention_row(q[0, h, r], ek, ev, [0.0] * len(ek), s)
            np.testing.assert_allclose(O[0, h, r], ref_o, rtol=0, atol=1e-11)
            assert abs(L[0, h, r] - ref_l) < 1e-11


def test_identical_keys_block_is_level_invariant():
    q, k, v = small_case(23, N=512, d=8)
    k[0, :, 128:192] = k[0, :, 128:129]     # block 2: identical keys and values
    v[0, :, 128:192] = v[0, :, 128:129]
    kp, vp = o.build_pyramid(k, 4), o.build_pyramid(v, 4)
    base = rng(24).integers(0, 4, size=(1, 2, 4, 8)).astype(np.int8)
    outs = []
    for l in range(4):
        lev = base.copy()
        lev[..., 2] = l
        outs.append(o.pyramid_attention(q, kp, vp, lev, 128, 64, 0.35))
    for l in range(1, 4):
        np.testing.assert_allclose(outs[l][0], outs[0][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(outs[l][1], outs[0][1], rtol=0, atol=1e-12)


def test_unit_values_give_unit_output():
    q, k, _ = small_case(25, N=300, d=4)
    v = np.ones_like(k)
    kp, vp = o.build_pyramid(k, 4), o.build_pyramid(v, 4)
    lev = rng(26).integers(-1, 4, size=(1, 2, 3, 5)).astype(np.int8)
    lev[..., 1] = 2
    O, _ = o.pyramid_attention(q, kp, vp, lev, 128, 64, 0.5)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-13)


def test_binary_mask_equals_masked_dense():
    # L = 1: PSA reduces to binary block-sparse attention = dense attention with -inf on pruned blocks.
    q, k, v = small_case(27, N=256, d=8)
    kp, vp = o.build_pyramid(k, 1), o.build_pyramid(v, 1)
    lev = rng(28).integers(-1, 1, size=(1, 2, 2, 4)).astype(np.int8)
    lev[..., 1] = 0
    O, L = o.pyramid_attention(q, kp, vp, lev, 128, 64, 0.35)
    for h in range(2):
        for i in range(2):
            keep = np.repeat(lev[0, h, i] >= 0, 64)
            for r in (i * 128, i * 128 + 77):
                wl = [0.0 if kk else -math.inf for kk in keep]
                idx = [t for t in range(256) if keep[t]]
                ref_o, ref_l = brute_attention_row(q[0, h, r], k[0, h, idx], v[0, h, idx], [0.0] * len(idx), 0.35)
                np.testing.assert_allclose(O[0, h, r], ref_o, rtol=0, atol=1e-12)
                assert abs(L[0, h, r] - ref_l) < 1e-12


def test_attention_key_shift_invariance():
    q, k, v = small_case(29, N=512, d=8)
    shift = rng(30).standard_normal(8)
    lev = rng(31).integers(-1, 4, size=(1, 2, 4, 8)).astype(np.int8)
    lev[..., 0] = 0
    a = o.pyramid_attention(q, o.build_pyramid(k, 4), o.build_pyramid(v, 4), lev, 128, 64, 0.35)[0]
    b = o.pyramid_attention(q, o.build_pyramid(k + shift, 4), o.build_pyramid(v, 4), lev, 128, 64, 0.35)[0]
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = small_case(32, H=4, Hkv=2, N=256, d=8)
    lev = rng(33).integers(-1, 4, size=(1, 4, 2, 4)).astype(np.int8)
    lev[..., 0] = 1
    tau = (0.3, 0.5, 0.7, 0.9)
    g = o.pyramid_attention(q, o.build_pyramid(k, 4), o.build_pyramid(v, 4), lev, 128, 64, 0.35)
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)   # heads [g0, g0, g1, g1]
    m = o.pyramid_attention(q, o.build_pyramid(kr, 4), o.build_pyramid(vr, 4), lev, 128, 64, 0.35)
    np.testing.assert_array_equal(g[0], m[0])
    mg = o.estimate_mask(q, k, 128, 64, tau, 4, 0.35)
    mm = o.estimate_mask(q, kr, 128, 64, tau, 4, 0.35)
    np.testing.assert_array_equal(mg["levels"], mm["levels"])


def test_all_pruned_row():
    q, k, v = small_case(34, N=128, d=4)
    lev = np.full((1, 2, 1, 2), -1, dtype=np.int8)
    O, L = o.pyramid_attention(q, o.build_pyramid(k, 4), o.build_pyramid(v, 4), lev, 128, 64, 0.5)
    assert np.all(O == 0) and np.all(np.isneginf(L))


def test_effective_flops_closed_forms():
    N, d = 2048, 64
    for l in range(4):
        lev = np.full((1, 2, 32, 32), l, dtype=np.int8)
        assert o.effective_flops(lev, N, 64, 64, d) == 4.0 * 2 * N * N * d / 2 ** l
    lev = np.full((1, 2, 32, 32), -1, dtype=np.int8)
    assert o.effective_flops(lev, N, 64, 64, d) == 0.0


# ----------------------------------------------------------------------------- backward

def loss_and_grads(q, k, v, L, lev, bq, s, dO, causal=False):
    g = o.pyramid_attention_bwd(q, k, v, L, lev, bq, 64, s, dO, io_dtype="f64", causal=causal)
    return float(np.sum(g["O"] * dO)), g


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal):
    # central differences of sum(O * dO) in float64 at a handful of coordinates per tensor
    r = rng(80)
    N, d, L, bq, s = 150, 3, 3, 64, 0.7
    q, k, v = r.standard_normal((1, 2, N, d)), r.standard_normal((1, 1, N, d)), r.standard_normal((1, 1, N, d))
    dO = r.standard_normal((1, 2, N, d))
    lev = r.integers(-1, L, size=(1, 2, 3, 3)).astype(np.int8)
    lev[..., 0] = np.maximum(lev[..., 0], 0)
    _, g = loss_and_grads(q, k, v, L, lev, bq, s, dO, causal)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for idx in [tuple(r.integers(0, n) for n in x.shape) for _ in range(12)] + [(0, 0, N - 1, 2)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            key = name[1:]
            fp = loss_and_grads(**{**args, key: xp}, L=L, lev=lev, bq=bq, s=s, dO=dO, causal=causal)[0]
            fm = loss_and_grads(**{**args, key: xm}, L=L, lev=lev, bq=bq, s=s, dO=dO, causal=causal)[0]
            assert abs((fp - fm) / (2 * eps) - g[name][idx]) < 1e-6, (name, idx, (fp - fm) / (2 * eps), g[name][idx])


def test_backward_dense_map_equals_torch_autograd():
    r = rng(81)
    N, d, s = 200, 8, 0.3
    q, k, v = r.standard_normal((1, 2, N, d)), r.standard_normal((1, 2, N, d)), r.standard_normal((1, 2, N, d))
    dO = r.standard_normal((1, 2, N, d))
    for causal in (False, True):
        lev = np.zeros((1, 2, 4, 4), dtype=np.int8)
        g = o.pyramid_attention_bwd(q, k, v, 4, lev, 64, 64, s, dO, io_dtype="f64", causal=causal)
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=s)
        out.backward(torch.from_numpy(dO))
        for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
            np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=0, atol=1e-11)


def test_backward_pooled_gradient_spreads_evenly():
    # With every block at level 3, a token's key gradient is its group's pooled gradient / 8
    r = rng(82)
    N, d = 128, 4
    q, k, v = r.standard_normal((1, 1, N, d)), r.standard_normal((1, 1, N, d)), r.standard_normal((1, 1, N, d))
    dO = r.standard_normal((1, 1, N, d))
    lev = np.full((1, 1, 2, 2), 3, dtype=np.int8)
    g = o.pyramid_attention_bwd(q, k, v, 4, lev, 64, 64, 0.5, dO, io_dtype="f64")
    for t in (0, 7, 8, 77, 127):
        np.testing.assert_allclose(g["dk"][0, 0, t], g["dk_levels"][3][0, 0, t // 8] / 8, rtol=0, atol=1e-14)
        np.testing.assert_allclose(g["dv"][0, 0, t], g["dv_levels"][3][0, 0, t // 8] / 8, rtol=0, atol=1e-14)
    # dV of a pooled row is the sum of its attention weights times dO: columns of P sum over rows
    np.testing.assert_allclose(g["dv_levels"][3].sum(axis=2), dO.sum(axis=2), rtol=0, atol=1e-10)


def test_backward_gqa_sums_heads():
    r = rng(83)
    N, d = 256, 4
    q, k, v = r.standard_normal((1, 4, N, d)), r.standard_normal((1, 2, N, d)), r.standard_normal((1, 2, N, d))
    dO = r.standard_normal((1, 4, N, d))
    lev = r.integers(-1, 4, size=(1, 4, 2, 4)).astype(np.int8)
    g = o.pyramid_attention_bwd(q, k, v, 4, lev, 128, 64, 0.5, dO, io_dtype="f64")
    rep = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    gm = o.pyramid_attention_bwd(q, rep[0], rep[1], 4, lev, 128, 64, 0.5, dO, io_dtype="f64")
    np.testing.assert_allclose(g["dq"], gm["dq"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dk"], gm["dk"].reshape(1, 2, 2, N, d).sum(axis=2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dv"], gm["dv"].reshape(1, 2, 2, N, d).sum(axis=2), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- hand-worked example

def test_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    N, bk, bq, L, s = ex["N"], ex["kv_block"], ex["q_block"], ex["num_levels"], ex["scale"]
    K = np.array(ex["K"], float).reshape(1, 1, N, 1)
    V = np.array(ex["V"], float).reshape(1, 1, N, 1)
    Q = np.array(ex["Q"], float).reshape(1, 1, N, 1)
    kp, vp = o.build_pyramid(K, L), o.build_pyramid(V, L)
    np.testing.assert_array_equal(kp[1][0, 0, :, 0], ex["level1_K"])
    np.testing.assert_array_equal(vp[1][0, 0, :, 0], ex["level1_V"])
    np.testing.assert_array_equal(o.pool_counts(N, 1), ex["level1_counts"])
    p0, p1 = 1 / (1 + math.exp(-1)), 1 / (1 + math.exp(1))
    for case in ex["cases"]:
        m = o.estimate_mask(Q, K, bq, bk, case["thresholds"], L, s)
        np.testing.assert_array_equal(m["kbar"][0, 0, :, 0], ex["kbar"])
        np.testing.assert_array_equal(m["qbar"][0, 0, :, 0], ex["qbar"])
        np.testing.assert_allclose(m["z"][0, 0, 0] - math.log(4), ex["z_minus_ln4"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(m["p"][0, 0, 0], [p0, p1], rtol=0, atol=1e-15)
        np.testing.assert_allclose(m["cmass"][0, 0, 0], [0.0, p0], rtol=0, atol=1e-15)
        np.testing.assert_array_equal(m["levels"][0, 0, 0], case["levels"])
        w = [c * math.exp(a) for a, c in case["weights_exp_args"]]
        o_ref = math.fsum(wi * vi for wi, vi in zip(w, case["values"])) / math.fsum(w)
        lse_ref = math.log(math.fsum(w))
        O, LSE = o.pyramid_attention(Q, kp, vp, m["levels"], bq, bk, s)
        np.testing.assert_allclose(O[0, 0, :, 0], o_ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(LSE[0, 0], lse_ref, rtol=0, atol=1e-13)


def test_whole_head_comparison_catches_planted_errors():
    """The whole-head parity helper of the GPU tests: the oracle's own output passes with zero
    error; one element off by 0.05, a NaN, or a wrong lse are each caught."""
    from synth import get as get_workload, generate
    from tests.oracle_heads import compare_heads
    w = get_workload("tiny")
    q, k, v = generate(w, "q"), generate(w, "k"), generate(w, "v")
    r = o.run_forward(q, k, v, w.q_block, w.kv_block, w.thresholds(), w.num_levels, w.scale, w.dtype)
    lev, O, LSE = r["mask"]["levels"], r["O"], r["LSE"]
    heads = [(0, 0), (0, 1)]
    mx, mean, cnt = compare_heads("tiny", heads, lev, O.astype(np.float32), LSE.astype(np.float32), say=lambda m: None)
    assert cnt == 2 * w.N * w.d and mx < 1e-5 and mean < 1e-6
    bad = O.astype(np.float32).copy()
    bad[0, 1, 1234, 5] += 0.05
    with pytest.raises(AssertionError, match="heads off"):
        compare_heads("tiny", heads, lev, bad, LSE.astype(np.float32), say=lambda m: None)
    bad = O.astype(np.float32).copy()
    bad[0, 0, 7, 0] = np.nan
    with pytest.raises(AssertionError, match="heads off"):
        compare_heads("tiny", heads, lev, bad, LSE.astype(np.float32), say=lambda m: None)
    bad_lse = LSE.astype(np.float32).copy()
    bad_lse[0, 1, 99] += 1.0     # float32 I/O: the bound allows the bf16 rounding of q and k
    with pytest.raises(AssertionError, match="heads off"):
        compare_heads("tiny", heads, lev, O.astype(np.float32), bad_lse, say=lambda m: None)


def test_run_forward_worked_example():
    """run_forward (the chain every GPU parity test and the smoke check call) on the
    hand-derived worked example: pyramid, levels, O and LSE equal the closed forms, in
    both I/O dtypes (every value of the example is exact in bf16)."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    N, bk, bq, L, s = ex["N"], ex["kv_block"], ex["q_block"], ex["num_levels"], ex["scale"]
    K = np.array(ex["K"], float).reshape(1, 1, N, 1)
    V = np.array(ex["V"], float).reshape(1, 1, N, 1)
    Q = np.array(ex["Q"], float).reshape(1, 1, N, 1)
    for io in ("f32", "bf16"):
        for case in ex["cases"]:
            r = o.run_forward(Q, K, V, bq, bk, case["thresholds"], L, s, io)
            np.testing.assert_array_equal(r["kpyr"][0][0, 0, :, 0], ex["K"])
            np.testing.assert_array_equal(r["kpyr"][1][0, 0, :, 0], ex["level1_K"])
            np.testing.assert_array_equal(r["vpyr"][1][0, 0, :, 0], ex["level1_V"])
            np.testing.assert_array_equal(r["mask"]["levels"][0, 0, 0], case["levels"])
            w = [c * math.exp(a) for a, c in case["weights_exp_args"]]
            o_ref = math.fsum(wi * vi for wi, vi in zip(w, case["values"])) / math.fsum(w)
            np.testing.assert_allclose(r["O"][0, 0, :, 0], o_ref, rtol=0, atol=1e-13)
            np.testing.assert_allclose(r["LSE"][0, 0], math.log(math.fsum(w)), rtol=0, atol=1e-13)


@pytest.mark.parametrize("io,causal,ranked", [("bf16", False, False), ("f32", False, False),
                                              ("bf16", True, False), ("bf16", False, True)])
def test_run_forward_equals_its_steps(io, causal, ranked):
    """run_forward against the step functions called one by one: the pyramid rounded to the
    I/O dtype (level 0 = the inputs themselves), the mask of the chosen rule, and attention
    over the rounded pyramid; GQA, a ragged tail and a partial pool group included."""
    from synth import random_qkv
    B, H, H_kv, N, d, bq, L = 2, 4, 2, 301, 8, 64, 4
    q, k, v = random_qkv(515, B, H, H_kv, N, d, io)
    k = k * 1.37          # pooled means no longer exact in bf16: the rounding step matters
    v = v * 0.91
    tau, fr, s = (0.2, 0.5, 0.7, 0.9), (0.1, 0.3, 0.6, 0.9), 0.3
    r = o.run_forward(q, k, v, bq, 64, tau, L, s, io, n_dense_prefix=70,
                      ranked_fractions=fr if ranked else None, causal=causal)
    for name, x in (("kpyr", k), ("vpyr", v)):
        lv = o.build_pyramid(x, L)
        np.testing.assert_array_equal(r[name][0], np.asarray(x, np.float64))
        for l in range(1, L):
            np.testing.assert_array_equal(r[name][l], o.round_to_io(lv[l], io))
            if io == "bf16":
                assert not np.array_equal(r[name][l], lv[l])   # the rounding changed something
    if ranked:
        m = o.estimate_mask_ranked(q, k, bq, 64, fr, L, s, 70, causal)
    else:
        m = o.estimate_mask(q, k, bq, 64, tau, L, s, 70, causal)
    np.testing.assert_array_equal(r["mask"]["levels"], m["levels"])
    O, LSE = o.pyramid_attention(q, r["kpyr"], r["vpyr"], m["levels"], bq, 64, s, causal=causal)
    np.testing.assert_array_equal(r["O"], O)
    np.testing.assert_array_equal(r["LSE"], LSE)
    # and attention over the unrounded pyramid differs (so the comparison above is not vacuous)
    if io == "bf16":
        kp_raw = [np.asarray(k, np.float64)] + o.build_pyramid(k, L)[1:]
        vp_raw = [np.asarray(v, np.float64)] + o.build_pyramid(v, L)[1:]
        O_raw, _ = o.pyramid_attention(q, kp_raw, vp_raw, m["levels"], bq, 64, s, causal=causal)
        assert np.abs(O_raw - O).max() > 0
