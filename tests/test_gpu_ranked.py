"""Parity of the ranked (keep-ratio / quantile) mask rule on MI355X with the CPU oracle.

The ranked rule shares the block-mean and score kernels with the threshold rule and
differs only in how the level kernel turns a sorted row into levels, so these cases
check the level maps (every element, against the oracle's scores), the per-level
counts, the 32-bit-key path against the exact path, and the end-to-end attention on
the map the GPU chose. Every case prints its name before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

from oracle import psa_oracle as o
from synth import generate, get as get_workload, random_qkv
from tests.psa_check import check_attention, check_cmass, check_kbar, check_mask_ranked, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def psa():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import level_pooled_kv_amd as lib
    return lib


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_ranked(psa, label, q, k, v, *, H, H_kv, d, q_block, L, dtype, fractions, n_dense_prefix=0,
               attention=True):
    B, _, N, _ = q.shape
    s = 1.0 / math.sqrt(d)
    prob = psa.Problem(B=B, H=H, H_kv=H_kv, N=N, d=d, q_block=q_block, kv_block=64, num_levels=L, dtype=dtype)
    say(f"{label}: B={B} H={H} H_kv={H_kv} N={N} d={d} q_block={q_block} L={L} {dtype} fractions={fractions}")
    ora = o.estimate_mask_ranked(q, k, q_block, 64, fractions, L, s, n_dense_prefix)
    counts = o.rank_counts(fractions, L, prob.nkb)
    qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    kp, vp, kbar = psa.psa_build_pyramid(prob, kd, vd)
    lev, cm = psa.psa_estimate_mask_ranked(prob, qd, kbar, fractions, n_dense_prefix, want_cmass=True)
    lev_fast, _ = psa.psa_estimate_mask_ranked(prob, qd, kbar, fractions, n_dense_prefix)
    torch.cuda.synchronize()
    check_kbar(to_host(kbar), ora["kbar"], label)
    lev_g = lev.cpu().numpy()
    assert np.array_equal(lev_fast.cpu().numpy(), lev_g), label
    nacc = check_mask_ranked(lev_g, ora, counts, L, n_dense_prefix, label=label)
    check_cmass(to_host(cm), ora, label)
    if attention:
        out, _ = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, lev)
        torch.cuda.synchronize()
        kpyr = [np.asarray(k, np.float64)] + [o.round_to_io(x, dtype) for x in o.build_pyramid(k, L)[1:]]
        vpyr = [np.asarray(v, np.float64)] + [o.round_to_io(x, dtype) for x in o.build_pyramid(v, L)[1:]]
        O, _ = o.pyramid_attention(q, kpyr, vpyr, lev_g, q_block, 64, s)
        check_attention(to_host(out), O, label + " e2e")
    say(f"{label}: ok (mask mismatches accepted: {nacc})")
    return ora, lev_g


CASES = [
    # label, N, d, q_block, L, dtype, H, H_kv, fractions, n_dense_prefix
    ("keep 0.1 + thirds N=2045 d128 gqa", 2045, 128, 128, 4, "bf16", 4, 2, (0.1, 0.4, 0.7, 1.0), 0),
    ("pruning N=4100 d64 bq128", 4100, 64, 128, 4, "bf16", 3, 3, (0.05, 0.15, 0.3, 0.5), 0),
    ("empty level 1 N=1000 d128 bq64", 1000, 128, 64, 4, "bf16", 2, 1, (0.2, 0.2, 0.5, 0.9), 0),
    ("binary top-k N=3000 d128 L=1", 3000, 128, 128, 1, "bf16", 2, 2, (0.25,), 0),
    ("N=777 d64 L=3 f32", 777, 64, 128, 3, "f32", 2, 2, (0.1, 0.3, 0.6), 0),
    ("N=130 d64 bq64", 130, 64, 64, 4, "bf16", 2, 2, (0.5, 0.5, 1.0, 1.0), 0),
    ("N=1 d64", 1, 64, 128, 4, "bf16", 1, 1, (0.0, 1.0, 1.0, 1.0), 0),
    ("dense prefix 226 N=1200 d64", 1200, 64, 128, 4, "bf16", 2, 2, (0.1, 0.2, 0.4, 0.6), 226),
    ("keep nothing N=700", 700, 64, 128, 2, "bf16", 1, 1, (0.0, 0.0), 0),
    # batches (optional last field B)
    ("B=2 ragged N=1500 d128 bq128 gqa", 1500, 128, 128, 4, "bf16", 6, 2, (0.1, 0.3, 0.6, 0.9), 0, 2),
    ("B=2 dense prefix 100 N=900 d64 bq64", 900, 64, 64, 4, "bf16", 2, 1, (0.05, 0.2, 0.4, 0.6), 100, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ranked_small(psa, case):
    label, N, d, bq, L, dtype, H, H_kv, fr, ndp, *rest = case
    B = rest[0] if rest else 1
    q, k, v = random_qkv(N + 3 * d + L + 1000 * (B - 1), B, H, H_kv, N, d, dtype)
    ora, lev = run_ranked(psa, label, q, k, v, H=H, H_kv=H_kv, d=d, q_block=bq, L=L, dtype=dtype,
                          fractions=fr, n_dense_prefix=ndp)
    if fr[-1] == 0.0:
        assert np.all(lev == -1)


def test_ranked_equal_scores(psa):
    # KV blocks 1..6 hold the same keys: equal scores, ordered by block index
    q, k, v = random_qkv(11, 1, 2, 2, 1024, 64, "bf16")
    k[:, :, 128:448] = np.tile(k[:, :, 64:128], (1, 1, 5, 1))
    ora, lev = run_ranked(psa, "ranked, equal scores (blocks 1..6)", q, k, v, H=2, H_kv=2, d=64, q_block=64,
                          L=4, dtype="bf16", fractions=(0.1, 0.25, 0.5, 0.75), attention=False)
    assert np.all(ora["z"][..., 1:7] == ora["z"][..., 1:2])
    # within the tied group the levels never decrease with the block index
    grp = lev[..., 1:7].astype(int)
    grp[grp < 0] = 9
    assert np.all(np.diff(grp, axis=-1) >= 0)


def test_ranked_equal_scores_long_rows(psa):
    # 1094 blocks per row (fast kernel plus exact kernel over flagged rows); 300 equal
    # scores in every row, which the rank cuts split
    N = 70000
    q, k, v = random_qkv(21, 1, 1, 1, N, 64, "bf16")
    k[:, :, 64:64 * 301] = np.tile(k[:, :, 64:128], (1, 1, 300, 1))
    ora, lev = run_ranked(psa, "ranked, 300 equal scores, 1094 blocks", q, k, v, H=1, H_kv=1, d=64, q_block=128,
                          L=4, dtype="bf16", fractions=(0.05, 0.15, 0.3, 0.5), attention=False)
    grp = lev[..., 1:301].astype(int)
    grp[grp < 0] = 9
    assert np.all(np.diff(grp, axis=-1) >= 0)


def test_ranked_all_blocks_level0_equals_threshold_one(psa):
    q, k, v = random_qkv(12, 1, 2, 2, 1500, 128, "bf16")
    prob = psa.Problem(B=1, H=2, H_kv=2, N=1500, d=128, q_block=128, num_levels=4, dtype="bf16")
    say("ranked fractions 1 == thresholds 1 (dense)")
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    _, _, kbar = psa.psa_build_pyramid(prob, kd, vd)
    a, _ = psa.psa_estimate_mask_ranked(prob, qd, kbar, (1.0, 1.0, 1.0, 1.0))
    b, _ = psa.psa_estimate_mask(prob, qd, kbar, (1.0, 1.0, 1.0, 1.0))
    torch.cuda.synchronize()
    assert torch.all(a == 0) and torch.equal(a, b)


@pytest.mark.parametrize("name,fractions", [("wan13b", (0.05, 0.15, 0.3, 0.5)),
                                            ("cogvx5b", (0.1, 0.4, 0.7, 1.0))])
def test_ranked_full_workload(psa, name, fractions):
    w = get_workload(name)
    L = w.num_levels
    say(f"{name} ranked: generating inputs B={w.B} H={w.H} H_kv={w.H_kv} N={w.N} d={w.d}")
    q, k = generate(w, "q"), generate(w, "k")
    prob = psa.Problem(B=w.B, H=w.H, H_kv=w.H_kv, N=w.N, d=w.d, q_block=w.q_block, kv_block=w.kv_block,
                       num_levels=L, dtype=w.dtype)
    qd, kd = to_device(q, w.dtype), to_device(k, w.dtype)
    say(f"{name} ranked: GPU pyramid + mask")
    _, _, kbar = psa.psa_build_pyramid(prob, kd, kd)
    lev, _ = psa.psa_estimate_mask_ranked(prob, qd, kbar, fractions, w.n_dense_prefix, want_cmass=True)
    lev_fast, _ = psa.psa_estimate_mask_ranked(prob, qd, kbar, fractions, w.n_dense_prefix)
    torch.cuda.synchronize()
    assert torch.equal(lev_fast, lev), name
    say(f"{name} ranked: oracle scores and ranks")
    kbar_o = np.concatenate([o.block_means(k[:, g:g + 1], w.kv_block) for g in range(w.H_kv)], axis=1)
    check_kbar(to_host(kbar), kbar_o, name)
    qbar = np.concatenate([o.block_means(q[:, h:h + 1], w.q_block) for h in range(w.H)], axis=1)
    z = o.block_scores(qbar, kbar_o, o.block_sizes(w.N, w.kv_block), w.scale)
    lev_o = o.assign_levels_ranked(z, fractions, L, w.n_dense_prefix, w.kv_block)
    counts = o.rank_counts(fractions, L, w.nkb)
    nacc = check_mask_ranked(lev.cpu().numpy(), {"z": z, "levels": lev_o}, counts, L, w.n_dense_prefix,
                             label=name)
    say(f"{name} ranked: ok (mask mismatches accepted: {nacc} of {lev_o.size})")
