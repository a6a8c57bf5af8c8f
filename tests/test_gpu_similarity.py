"""Parity of the cosine-similarity constraint on MI355X with the CPU oracle (C ABI).

psa_build_pyramid_sim must give the pyramid of psa_build_pyramid bit for bit plus the
key similarity per pooled level (float32, within 2e-5 of the float64 oracle);
psa_apply_similarity_cap must cap a level map exactly as the oracle does, except where
a similarity lies within that tolerance of the threshold. Every case prints its name
before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

from oracle import psa_oracle as o
from synth import generate, get as get_workload, random_qkv
from tests.psa_check import check_attention, to_device, to_host

pytestmark = pytest.mark.gpu

SIM_TOL = 2e-5


@pytest.fixture(scope="module")
def psa():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import level_pooled_kv_amd as lib
    return lib


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def check_cap(gpu_map, lev_in, sim_ora, thr, H, label):
    """Exact, except where a level's similarity is within SIM_TOL of the threshold."""
    ref = o.apply_similarity_cap(lev_in, sim_ora, thr)
    diff = np.argwhere(gpu_map != ref)
    H_kv = sim_ora.shape[1]
    for (b, h, i, j) in diff:
        g = o.kv_head_of(h, H, H_kv)
        lo, hi = sorted((int(gpu_map[b, h, i, j]), int(ref[b, h, i, j])))
        near = [abs(sim_ora[b, g, j, l - 1] - np.float32(thr)) <= SIM_TOL for l in range(lo + 1, hi + 1)]
        assert lo >= 0 and any(near), (label, (b, h, i, j), int(gpu_map[b, h, i, j]), int(ref[b, h, i, j]))
    return len(diff)


def structured_keys(k, seed):
    """Make some KV blocks similar (one direction plus small noise), keep others random."""
    r = np.random.default_rng(seed)
    B, Hkv, N, d = k.shape
    for b in range(B):
        for g in range(Hkv):
            for j in range(b % 2, -(-N // 64), 3):
                lo, hi = 64 * j, min(64 * j + 64, N)
                base = r.standard_normal(d)
                k[b, g, lo:hi] = base + 0.05 * (j % 5) * r.standard_normal((hi - lo, d))
    return k


CASES = [
    # label, N, d, dtype, H, H_kv, L, q_block, threshold
    ("N=2045 d128 bf16 gqa", 2045, 128, "bf16", 4, 2, 4, 128, 0.6),
    ("N=777 d64 f32 L=3", 777, 64, "f32", 2, 2, 3, 128, 0.7),
    ("N=1000 d64 bf16 bq64", 1000, 64, "bf16", 2, 1, 4, 64, 0.5),
    ("N=1500 d128 f32 L=2", 1500, 128, "f32", 2, 2, 2, 128, 0.8),
    ("N=70 d128 bf16", 70, 128, "bf16", 1, 1, 4, 128, 0.9),
    # batches (optional last field B)
    ("B=2 N=1500 d128 bf16 gqa", 1500, 128, "bf16", 6, 2, 4, 128, 0.7),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_similarity_and_cap_small(psa, case):
    label, N, d, dtype, H, H_kv, L, bq, thr, *rest = case
    B = rest[0] if rest else 1
    q, k, v = random_qkv(N + 7 * d + L + 1000 * (B - 1), B, H, H_kv, N, d, dtype)
    k = structured_keys(k, N)
    k = o.round_to_bf16(k) if dtype == "bf16" else k.astype(np.float32).astype(np.float64)
    s = 1.0 / math.sqrt(d)
    prob = psa.Problem(B=B, H=H, H_kv=H_kv, N=N, d=d, q_block=bq, num_levels=L, dtype=dtype)
    say(f"{label}: similarity + cap, threshold {thr}")
    qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    kp0, vp0, kb0 = psa.psa_build_pyramid(prob, kd, vd)
    kp, vp, kb, ksim = psa.psa_build_pyramid_sim(prob, kd, vd)
    tau = (0.3, 0.55, 0.75, 0.9)[:L]
    lev, _ = psa.psa_estimate_mask(prob, qd, kb, tau)
    lev_in = lev.cpu().numpy()
    capped = psa.psa_apply_similarity_cap(prob, ksim, thr, lev.clone())
    torch.cuda.synchronize()
    assert torch.equal(kp, kp0) and torch.equal(vp, vp0) and torch.equal(kb, kb0), label
    sim_ora = o.key_similarity(k, 64, L)
    err = np.abs(to_host(ksim) - sim_ora)
    assert err.max() <= SIM_TOL, (label, float(err.max()))
    cap_g = capped.cpu().numpy()
    n = check_cap(cap_g, lev_in, sim_ora, thr, H, label)
    assert np.all((cap_g >= 0) == (lev_in >= 0)) and np.all(cap_g <= np.maximum(lev_in, -1))
    # attention on the capped map
    out, _ = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, capped)
    torch.cuda.synchronize()
    kpyr = [np.asarray(k, np.float64)] + [o.round_to_io(a, dtype) for a in o.build_pyramid(k, L)[1:]]
    vpyr = [np.asarray(v, np.float64)] + [o.round_to_io(a, dtype) for a in o.build_pyramid(v, L)[1:]]
    O, _ = o.pyramid_attention(q, kpyr, vpyr, cap_g, bq, 64, s)
    check_attention(to_host(out), O, label)
    changed = int((cap_g != lev_in).sum())
    say(f"{label}: ok (sim max err {err.max():.1e}, {changed} levels capped, {n} near-threshold differences)")


def test_similarity_cap_causal(psa):
    # the cap under causal use: diagonal blocks stay at level 0, invisible ones pruned,
    # and attention on the capped map matches the causal oracle
    N, d, bq, L, thr = 1500, 128, 128, 4, 0.7
    q, k, v = random_qkv(77, 1, 2, 2, N, d, "bf16")
    k = o.round_to_bf16(structured_keys(k, 3))
    s = 1.0 / math.sqrt(d)
    prob = psa.Problem(B=1, H=2, H_kv=2, N=N, d=d, q_block=bq, num_levels=L, dtype="bf16", causal=True)
    say(f"causal similarity cap, threshold {thr}")
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    kp, vp, kb, ksim = psa.psa_build_pyramid_sim(prob, kd, vd)
    lev, _ = psa.psa_estimate_mask(prob, qd, kb, (0.3, 0.55, 0.75, 0.9))
    lev_in = lev.cpu().numpy()
    capped = psa.psa_apply_similarity_cap(prob, ksim, thr, lev.clone())
    torch.cuda.synchronize()
    sim_ora = o.key_similarity(k, 64, L)
    cap_g = capped.cpu().numpy()
    check_cap(cap_g, lev_in, sim_ora, thr, 2, "causal cap")
    vis, diag = o.causal_blocks(N, bq, 64)
    assert np.all(cap_g[..., ~vis] == -1) and np.all(cap_g[..., diag] == 0)
    out, _ = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, capped)
    torch.cuda.synchronize()
    kpyr = [np.asarray(k, np.float64)] + [o.round_to_io(a, "bf16") for a in o.build_pyramid(k, L)[1:]]
    vpyr = [np.asarray(v, np.float64)] + [o.round_to_io(a, "bf16") for a in o.build_pyramid(v, L)[1:]]
    O, _ = o.pyramid_attention(q, kpyr, vpyr, cap_g, bq, 64, s, causal=True)
    check_attention(to_host(out), O, "causal cap attention")
    say("causal similarity cap: ok")


def test_cap_extremes(psa):
    q, k, v = random_qkv(5, 1, 2, 2, 900, 128, "bf16")
    prob = psa.Problem(B=1, H=2, H_kv=2, N=900, d=128, q_block=128, num_levels=4, dtype="bf16")
    say("cap with thresholds -2 (no change) and 2 (everything to level 0)")
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    _, _, kb, ksim = psa.psa_build_pyramid_sim(prob, kd, vd)
    lev, _ = psa.psa_estimate_mask(prob, qd, kb, (0.3, 0.55, 0.75, 0.9))
    same = psa.psa_apply_similarity_cap(prob, ksim, -2.0, lev.clone())
    flat = psa.psa_apply_similarity_cap(prob, ksim, 2.0, lev.clone())
    torch.cuda.synchronize()
    assert torch.equal(same, lev)
    assert torch.equal(flat, torch.where(lev >= 0, torch.zeros_like(lev), lev))


def test_similarity_full_workload_sampled(psa):
    w = get_workload("wan13b")
    L = w.num_levels
    say(f"{w.name}: key similarity at full size, sampled blocks")
    k, v = generate(w, "k"), generate(w, "v")
    prob = psa.Problem(B=w.B, H=w.H, H_kv=w.H_kv, N=w.N, d=w.d, q_block=w.q_block, num_levels=L, dtype=w.dtype)
    kd, vd = to_device(k, w.dtype), to_device(v, w.dtype)
    _, _, _, ksim = psa.psa_build_pyramid_sim(prob, kd, vd)
    torch.cuda.synchronize()
    sim_g = to_host(ksim)
    rng = np.random.default_rng(3)
    picks = {(0, w.nkb - 1), (w.H_kv - 1, 0)}
    while len(picks) < 48:
        picks.add((int(rng.integers(w.H_kv)), int(rng.integers(w.nkb))))
    for g, j in sorted(picks):
        blk = k[:, g:g + 1, 64 * j:min(64 * j + 64, w.N)]
        ref = o.key_similarity(blk, 64, L)[0, 0, 0]
        assert np.abs(sim_g[0, g, j] - ref).max() <= SIM_TOL, (g, j, sim_g[0, g, j], ref)
    say(f"{w.name}: ok; similarity per level, mean over blocks: "
        f"{[round(float(x), 3) for x in sim_g.reshape(-1, L - 1).mean(axis=0)]}")
