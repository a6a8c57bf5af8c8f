"""Parity of the causal variant on MI355X with the CPU oracle (through the C ABI).

Causal use: the mask ranks only the KV blocks a query block can see and keeps the
blocks reaching its own rows at level 0; attention lets row r see a key only if every
token it averages is at or before r. Small cases compare every output element;
arbitrary level maps (pooled and future blocks on the diagonal) exercise the
attention rule by itself. Every case prints its name before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

from oracle import psa_oracle as o
from synth import generate, get as get_workload, random_qkv
from tests.oracle_heads import compare_heads
from tests.psa_check import (check_attention, check_cmass, check_fast_vs_exact, check_kbar, check_mask, check_mask_ranked,
                              lse_tolerance, to_device, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def psa():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import level_pooled_kv_amd as lib
    return lib


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def pyramid_io(x, L, dtype):
    return [np.asarray(x, np.float64)] + [o.round_to_io(a, dtype) for a in o.build_pyramid(x, L)[1:]]


def check_lse(lse_g, lse_r, q, k, s, dtype, label):
    fin = np.isfinite(lse_r)
    assert np.array_equal(np.isfinite(lse_g), fin), label
    if fin.any():
        tol = lse_tolerance(q, k, s, dtype)
        err = np.abs(lse_g[fin] - lse_r[fin])   # rows without a visible key hold -inf on both sides
        assert np.all(err <= tol[fin]), (label, err.max())


def run_causal(psa, label, q, k, v, *, H, H_kv, d, q_block, L, dtype, tau=None, fractions=None,
               n_dense_prefix=0):
    B, _, N, _ = q.shape
    s = 1.0 / math.sqrt(d)
    prob = psa.Problem(B=B, H=H, H_kv=H_kv, N=N, d=d, q_block=q_block, kv_block=64, num_levels=L, dtype=dtype,
                       causal=True)
    rule = f"tau={tau}" if fractions is None else f"fractions={fractions}"
    say(f"{label}: causal B={B} H={H} H_kv={H_kv} N={N} d={d} q_block={q_block} L={L} {dtype} {rule}")
    ora = o.run_forward(q, k, v, q_block, 64, tau, L, s, dtype, n_dense_prefix, ranked_fractions=fractions,
                        causal=True)
    m = ora["mask"]
    qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    kp, vp, kbar = psa.psa_build_pyramid(prob, kd, vd)
    if fractions is None:
        lev, cm = psa.psa_estimate_mask(prob, qd, kbar, tau, n_dense_prefix, want_cmass=True)
        lev_fast, _ = psa.psa_estimate_mask(prob, qd, kbar, tau, n_dense_prefix)
    else:
        lev, cm = psa.psa_estimate_mask_ranked(prob, qd, kbar, fractions, n_dense_prefix, want_cmass=True)
        lev_fast, _ = psa.psa_estimate_mask_ranked(prob, qd, kbar, fractions, n_dense_prefix)
    torch.cuda.synchronize()
    check_kbar(to_host(kbar), m["kbar"], label)
    lev_g = lev.cpu().numpy()
    assert np.array_equal(lev_fast.cpu().numpy(), lev_g), label
    vis, diag = o.causal_blocks(N, q_block, 64)
    assert np.all(lev_g[..., ~vis] == -1), label
    assert np.all(lev_g[..., diag] == 0), label
    if fractions is None:
        nacc = check_mask(lev_g, m, tau, L, n_dense_prefix, label=label)
    else:
        # counts are taken of each row's visible blocks; the forced blocks were checked above
        nacc = 0
        nvis = vis.sum(axis=-1)
        for i in range(lev_g.shape[2]):
            nv = int(nvis[i])
            sub = {"z": m["z"][:, :, i:i + 1, :nv], "levels": m["levels"][:, :, i:i + 1, :nv]}
            nacc += check_mask_ranked(lev_g[:, :, i:i + 1, :nv], sub, o.rank_counts(fractions, L, nv), L,
                                      n_dense_prefix, label=f"{label} row {i}", check_counts=False)
    check_cmass(to_host(cm), m, label)
    lev_o = torch.from_numpy(m["levels"]).cuda()
    out, lse = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, lev_o, want_lse=True)
    torch.cuda.synchronize()
    mx, mean = check_attention(to_host(out), ora["O"], label)
    check_lse(to_host(lse), ora["LSE"], q, k, s, dtype, label)
    if nacc:
        out2, _ = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, lev)
        torch.cuda.synchronize()
        O2, _ = o.pyramid_attention(q, ora["kpyr"], ora["vpyr"], lev_g, q_block, 64, s, causal=True)
        check_attention(to_host(out2), O2, label + " e2e")
    say(f"{label}: ok (mask mismatches: {nacc}, O max {mx:.2e} mean {mean:.2e})")


CASES = [
    # label, N, d, q_block, L, dtype, H, H_kv, tau, fractions, n_dense_prefix
    ("tiny shape f32 bq64", 2048, 64, 64, 4, "f32", 2, 2, (0.6, 0.8, 0.9, 0.95), None, 0),
    ("ragged N=2045 d128 bq128 gqa", 2045, 128, 128, 4, "bf16", 4, 2, (0.3, 0.55, 0.75, 0.9), None, 0),
    ("N=130 d64 bq64", 130, 64, 64, 4, "bf16", 2, 2, (0.3, 0.55, 0.75, 0.9), None, 0),
    ("N=1 d128", 1, 128, 128, 4, "bf16", 1, 1, (0.3, 0.55, 0.75, 0.9), None, 0),
    ("N=64 d64 bq128", 64, 64, 128, 4, "bf16", 1, 1, (0.3, 0.55, 0.75, 0.9), None, 0),
    ("N=1536 d128 L=1 binary", 1536, 128, 128, 1, "bf16", 2, 2, (0.5,), None, 0),
    ("N=900 d128 f32 L=3", 900, 128, 128, 3, "f32", 2, 1, (0.3, 0.6, 0.8), None, 0),
    ("dense prefix 226 N=1200 d64", 1200, 64, 128, 4, "bf16", 2, 2, (0.05, 0.2, 0.4, 0.6), None, 226),
    ("ranked N=3000 d128", 3000, 128, 128, 4, "bf16", 2, 2, None, (0.1, 0.3, 0.5, 0.7), 0),
    ("ranked top-k N=2500 d64 bq64", 2500, 64, 64, 1, "bf16", 2, 2, None, (0.25,), 0),
    ("N=1301 d128 bq64 gqa", 1301, 128, 64, 4, "bf16", 4, 2, (0.3, 0.55, 0.75, 0.9), None, 0),
    # batches (optional last field B)
    ("B=2 ragged N=1500 d128 bq128 gqa", 1500, 128, 128, 4, "bf16", 6, 2, (0.3, 0.55, 0.75, 0.9), None, 0, 2),
    ("B=2 ranked N=999 d64 bq64 gqa", 999, 64, 64, 4, "bf16", 4, 2, None, (0.1, 0.3, 0.5, 0.7), 0, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_causal_small(psa, case):
    label, N, d, bq, L, dtype, H, H_kv, tau, fr, ndp, *rest = case
    B = rest[0] if rest else 1
    q, k, v = random_qkv(N + 5 * d + L + 1000 * (B - 1), B, H, H_kv, N, d, dtype)
    run_causal(psa, label, q, k, v, H=H, H_kv=H_kv, d=d, q_block=bq, L=L, dtype=dtype, tau=tau, fractions=fr,
               n_dense_prefix=ndp)


ARBITRARY = [
    # label, N, d, q_block, dtype, H, H_kv
    ("arbitrary maps N=1000 d128 bq128", 1000, 128, 128, "bf16", 2, 2),
    ("arbitrary maps N=777 d64 bq64 f32", 777, 64, 64, "f32", 2, 1),
    ("arbitrary maps N=1301 d128 bq64 gqa", 1301, 128, 64, "bf16", 4, 2),
    ("arbitrary maps B=2 N=1100 d128 bq128 gqa", 1100, 128, 128, "bf16", 4, 2, 2),
]


@pytest.mark.parametrize("case", ARBITRARY, ids=[c[0] for c in ARBITRARY])
def test_causal_attention_arbitrary_maps(psa, case):
    # pooled blocks on the diagonal and blocks in the future: the per-key causal rule alone
    label, N, d, bq, dtype, H, H_kv, *rest = case
    B = rest[0] if rest else 1
    q, k, v = random_qkv(N + 17 + 1000 * (B - 1), B, H, H_kv, N, d, dtype)
    s = 1.0 / math.sqrt(d)
    prob = psa.Problem(B=B, H=H, H_kv=H_kv, N=N, d=d, q_block=bq, num_levels=4, dtype=dtype, causal=True)
    rng = np.random.default_rng(N)
    lev = rng.integers(-1, 4, size=(B, H, prob.nqb, prob.nkb)).astype(np.int8)
    lev[0, 0, 1] = 3                                  # a row whose first tiles are all in the future
    lev[0, 0, 1, :2] = -1
    say(f"{label}: causal attention on random level maps")
    qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    kp, vp, _ = psa.psa_build_pyramid(prob, kd, vd)
    out, lse = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, torch.from_numpy(lev).cuda(), want_lse=True)
    torch.cuda.synchronize()
    O, LSE = o.pyramid_attention(q, pyramid_io(k, 4, dtype), pyramid_io(v, 4, dtype), lev, bq, 64, s, causal=True)
    check_attention(to_host(out), O, label)
    check_lse(to_host(lse), LSE, q, k, s, dtype, label)
    assert not np.isfinite(LSE).all()                 # some rows see nothing: O = 0, lse = -inf
    say(f"{label}: ok")


def test_causal_dense_map_equals_causal_attention(psa):
    q, k, v = random_qkv(31, 1, 2, 2, 1500, 128, "bf16")
    prob = psa.Problem(B=1, H=2, H_kv=2, N=1500, d=128, q_block=128, num_levels=1, dtype="bf16", causal=True)
    say("causal all-level-0 map == causal dense attention")
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    lev = torch.zeros((1, 2, prob.nqb, prob.nkb), dtype=torch.int8, device="cuda")
    out, _ = psa.psa_attention_fwd(prob, qd, kd, vd, None, None, lev)
    torch.cuda.synchronize()
    Od, _ = o.dense_attention(q, k, v, 1 / math.sqrt(128), causal=True)
    check_attention(to_host(out), Od, "causal dense")


@pytest.mark.parametrize("ranked", [False, True], ids=["thresholds", "ranked"])
def test_causal_mask_long_rows(psa, ranked):
    # 625 KV blocks per row: the fast and exact level kernels (separate for rows this
    # long) under causal use, with 300 equal-score blocks so that some cuts split a tie
    N, d, L = 40000, 64, 4
    q, k, v = random_qkv(33, 1, 1, 1, N, d, "bf16")
    k[:, :, 64:64 * 301] = np.tile(k[:, :, 64:128], (1, 1, 300, 1))
    s = 1.0 / math.sqrt(d)
    prob = psa.Problem(B=1, H=1, H_kv=1, N=N, d=d, q_block=128, num_levels=L, dtype="bf16", causal=True)
    tau, fr = (0.02, 0.1, 0.3, 0.6), (0.05, 0.15, 0.3, 0.5)
    say(f"causal mask, {prob.nkb} blocks per row, {'ranked' if ranked else 'thresholds'}")
    qd, kd = to_device(q, "bf16"), to_device(k, "bf16")
    _, _, kbar = psa.psa_build_pyramid(prob, kd, to_device(v, "bf16"))
    if ranked:
        lev, _ = psa.psa_estimate_mask_ranked(prob, qd, kbar, fr)
        lev_c, _ = psa.psa_estimate_mask_ranked(prob, qd, kbar, fr, want_cmass=True)
    else:
        lev, _ = psa.psa_estimate_mask(prob, qd, kbar, tau)
        lev_c, cm_c = psa.psa_estimate_mask(prob, qd, kbar, tau, want_cmass=True)
    torch.cuda.synchronize()
    if ranked:
        assert torch.equal(lev, lev_c)       # ranks involve no mass sums: both passes agree exactly
    else:
        check_fast_vs_exact(lev.cpu().numpy(), lev_c.cpu().numpy(), to_host(cm_c), tau, L, label="causal long rows")
    lev_g = lev.cpu().numpy()
    vis, diag = o.causal_blocks(N, 128, 64)
    assert np.all(lev_g[..., ~vis] == -1) and np.all(lev_g[..., diag] == 0)
    if ranked:
        m = o.estimate_mask_ranked(q, k, 128, 64, fr, L, s, causal=True)
        nvis = vis.sum(axis=-1)
        for i in range(0, lev_g.shape[2], 7):
            nv = int(nvis[i])
            sub = {"z": m["z"][:, :, i:i + 1, :nv], "levels": m["levels"][:, :, i:i + 1, :nv]}
            check_mask_ranked(lev_g[:, :, i:i + 1, :nv], sub, o.rank_counts(fr, L, nv), L, 0,
                              label=f"causal ranked row {i}", check_counts=False)
    else:
        m = o.estimate_mask(q, k, 128, 64, tau, L, s, causal=True)
        check_mask(lev_g, m, tau, L, 0, label="causal, long rows")
        check_mask(lev_c.cpu().numpy(), m, tau, L, 0, label="causal, long rows, exact pass")
    say("causal mask, long rows: ok")


def test_causal_full_workload(psa):
    w = get_workload("wan13b_causal")
    L, s = w.num_levels, w.scale
    tau = w.thresholds()
    say(f"{w.name}: generating inputs B={w.B} H={w.H} N={w.N} d={w.d}")
    q, k, v = generate(w, "q"), generate(w, "k"), generate(w, "v")
    prob = psa.Problem(B=w.B, H=w.H, H_kv=w.H_kv, N=w.N, d=w.d, q_block=w.q_block, num_levels=L, dtype=w.dtype,
                       causal=True)
    qd, kd, vd = to_device(q, w.dtype), to_device(k, w.dtype), to_device(v, w.dtype)
    say(f"{w.name}: GPU pyramid + mask")
    kp, vp, kbar = psa.psa_build_pyramid(prob, kd, vd)
    lev, cm = psa.psa_estimate_mask(prob, qd, kbar, tau, want_cmass=True)
    lev_fast, _ = psa.psa_estimate_mask(prob, qd, kbar, tau)
    torch.cuda.synchronize()
    assert torch.equal(lev_fast, lev)
    say(f"{w.name}: oracle mask")
    kbar_o = np.concatenate([o.block_means(k[:, g:g + 1], w.kv_block) for g in range(w.H_kv)], axis=1)
    check_kbar(to_host(kbar), kbar_o, w.name)
    qbar = np.concatenate([o.block_means(q[:, h:h + 1], w.q_block) for h in range(w.H)], axis=1)
    z = o.block_scores(qbar, kbar_o, o.block_sizes(w.N, w.kv_block), s)
    vis, diag = o.causal_blocks(w.N, w.q_block, w.kv_block)
    z = np.where(vis, z, -np.inf)
    p = o.softmax_rows(z)
    C = o.cumulative_mass(z, p)
    C, lev_o = o.apply_causal(C, o.assign_levels(C, tau, L, 0, w.kv_block), w.N, w.q_block, w.kv_block)
    lev_g = lev.cpu().numpy()
    nacc = check_mask(lev_g, {"z": z, "p": p, "cmass": C, "levels": lev_o}, tau, L, 0, label=w.name)
    nfar = check_cmass(to_host(cm), {"z": z, "p": p, "cmass": C, "levels": lev_o}, w.name)
    say(f"{w.name}: GPU attention on the oracle's map, every query block (outputs prefilled with NaN)")
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=qd.device)
    psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, torch.from_numpy(lev_o).cuda(), o=out, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), (w.name, "output elements left unwritten or non-finite")
    assert not bool(torch.isnan(lse).any()), (w.name, "lse rows left unwritten")
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    mx, mean, cnt = compare_heads(w.name, heads, lev_o, out.float().cpu().numpy(), lse.cpu().numpy(), say=say)
    say(f"{w.name}: O over all {len(heads)} heads: max err {mx:.2e}, mean {mean:.2e}; cumulative masses "
        f"outside 1e-5 inside the near-tie interval: {nfar}")
    say(f"{w.name}: ok (mask mismatches accepted: {nacc} of {lev_o.size})")
