"""Parity of the attention backward (psa_attention_bwd, through the C ABI) with the
float64 oracle on MI355X.

Tolerance (derived, not fitted): every element of dq, dk, dv, and of the per-level
pooled gradients the library keeps in its workspace before spreading them over the
tokens, must lie within the bound tests.psa_check.backward_bounds derives from the
kernels' roundings (P and dA rounded to bf16 for their products, D_r = <dO_r, O_r> from
the bf16 output, float32 sums, bf16 outputs; float32 I/O also rounds its inputs to bf16
on the way into the matrix cores). As a whole-tensor sanity bound the relative L2 error
must stay within 1e-2 (bf16 I/O) or 2e-2 (float32 I/O).
Every case prints its name before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

from oracle import psa_oracle as o
from synth import generate, get as get_workload, random_qkv
from tests.psa_check import backward_bounds, check_grad_bound, to_device, to_host

pytestmark = pytest.mark.gpu

REL = {"bf16": 1e-2, "f32": 2e-2}
MAXREL = 5e-2


@pytest.fixture(scope="module")
def psa():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import level_pooled_kv_amd as lib
    return lib


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)


def check_grad(g, r, dtype, label):
    """Relative L2 error within REL[dtype] (a whole-tensor sanity bound next to the
    element-wise one)."""
    assert np.all(np.isfinite(g)), (label, "non-finite gradient")
    nr = np.linalg.norm(r.ravel())
    if nr == 0.0:   # e.g. a single key: dA = P (dP - D) vanishes up to float32 arithmetic
        assert np.abs(g).max() <= 1e-5, (label, "expected a zero gradient", float(np.abs(g).max()))
        return 0.0
    rel = np.linalg.norm((g - r).ravel()) / nr
    mx = np.abs(g - r).max() / max(np.abs(r).max(), 1e-30)
    assert rel <= REL[dtype] and mx <= MAXREL, (label, float(rel), float(mx))
    return float(rel)


def workspace_levels(ws, prob, which):
    """Per-level float32 gradients of K (which = 0) or V (1) from the backward's workspace:
    after two [B, H, N padded to 64] float32 arrays (each on a 256-byte boundary) come
    [B, H_kv, N + pyramid rows, d] for K, then for V (level 0 rows first, then level 1, ...)."""
    r256 = lambda x: (x + 255) // 256 * 256
    npad = -(-prob.N // 64) * 64
    rows = prob.N + prob.pyramid_rows
    off = 2 * r256(prob.B * prob.H * npad * 4) + which * r256(prob.B * prob.H_kv * rows * prob.d * 4)
    n = prob.B * prob.H_kv * rows * prob.d
    flat = ws[off:off + 4 * n].view(torch.float32).reshape(prob.B, prob.H_kv, rows, prob.d)
    out, r0 = [], 0
    for l in range(prob.num_levels):
        R = -(-prob.N // 2 ** l)
        out.append(to_host(flat[:, :, r0:r0 + R]))
        r0 += R
    return out


def run_bwd(psa, label, q, k, v, lev, *, H, H_kv, d, q_block, L, dtype, causal=False, seed=0):
    B, _, N, _ = q.shape
    s = 1.0 / math.sqrt(d)
    prob = psa.Problem(B=B, H=H, H_kv=H_kv, N=N, d=d, q_block=q_block, num_levels=L, dtype=dtype, causal=causal)
    dO = np.random.default_rng(seed).standard_normal(q.shape)
    if dtype == "bf16":
        dO = o.round_to_bf16(dO)
    say(f"{label}: backward B={B} H={H} H_kv={H_kv} N={N} d={d} q_block={q_block} L={L} {dtype} causal={causal}")
    qd, kd, vd, dod = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype), to_device(dO, dtype)
    kp, vp, _ = psa.psa_build_pyramid(prob, kd, vd)
    lev_d = torch.from_numpy(lev).cuda()
    out, lse = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, lev_d, want_lse=True)
    ws = torch.empty(prob.workspace_bytes(psa.PSA_WS_ATTENTION_BWD), dtype=torch.uint8, device=qd.device)
    dq, dk, dv = psa.psa_attention_bwd(prob, qd, kd, vd, kp, vp, lev_d, out, lse, dod, workspace=ws)
    torch.cuda.synchronize()
    ref = o.pyramid_attention_bwd(q, k, v, L, lev, q_block, 64, s, dO, io_dtype=dtype, causal=causal)
    bnd = backward_bounds(q, k, v, L, lev, q_block, s, dO, dtype, causal=causal)
    rels = [check_grad(to_host(x), ref[n], dtype, f"{label} {n}") for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    worst = max(check_grad_bound(to_host(x), ref[n], bnd[n], f"{label} {n}", dtype)
                for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")))
    # the pooled gradients per level, before they are spread over the tokens
    for which, name in ((0, "dk_levels"), (1, "dv_levels")):
        for l, gl in enumerate(workspace_levels(ws, prob, which)):
            worst = max(worst, check_grad_bound(gl, ref[name][l], bnd[name][l], f"{label} {name}[{l}]"))
    say(f"{label}: ok (relative L2 error dq {rels[0]:.1e} dk {rels[1]:.1e} dv {rels[2]:.1e}; largest "
        f"error / element bound {worst:.2f})")
    return ref


CASES = [
    # label, N, d, q_block, L, dtype, H, H_kv, causal
    ("tiny shape f32 bq64", 2048, 64, 64, 4, "f32", 2, 2, False),
    ("ragged N=2045 d128 bq128 gqa", 2045, 128, 128, 4, "bf16", 4, 2, False),
    ("N=130 d64 bq64", 130, 64, 64, 4, "bf16", 2, 2, False),
    ("N=1 d128", 1, 128, 128, 4, "bf16", 1, 1, False),
    ("N=1536 d128 L=1", 1536, 128, 128, 1, "bf16", 2, 2, False),
    ("N=900 d128 f32 L=3", 900, 128, 128, 3, "f32", 2, 1, False),
    ("causal N=1000 d128 bq128", 1000, 128, 128, 4, "bf16", 2, 2, True),
    ("causal N=777 d64 bq64 f32", 777, 64, 64, 4, "f32", 2, 1, True),
    ("N=1301 d128 bq64 gqa", 1301, 128, 64, 4, "bf16", 4, 2, False),
    ("causal N=1301 d128 bq64 gqa", 1301, 128, 64, 4, "bf16", 4, 2, True),
    # batches (optional last field B)
    ("B=2 ragged N=1500 d128 bq128 gqa", 1500, 128, 128, 4, "bf16", 6, 2, False, 2),
    ("B=2 causal N=999 d64 bq64 gqa", 999, 64, 64, 4, "bf16", 4, 2, True, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_on_mask(psa, case):
    label, N, d, bq, L, dtype, H, H_kv, causal, *rest = case
    B = rest[0] if rest else 1
    q, k, v = random_qkv(N + 11 * d + L + 1000 * (B - 1), B, H, H_kv, N, d, dtype)
    tau = (0.3, 0.55, 0.75, 0.9)[:L]
    lev = o.estimate_mask(q, k, bq, 64, tau, L, 1 / math.sqrt(d), causal=causal)["levels"]
    run_bwd(psa, label, q, k, v, lev, H=H, H_kv=H_kv, d=d, q_block=bq, L=L, dtype=dtype, causal=causal)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_arbitrary_maps(psa, causal):
    # every level anywhere (pooled blocks on the diagonal, rows that keep nothing)
    N, d, bq, H, H_kv = 1100, 128, 128, 2, 2
    q, k, v = random_qkv(N + 23, 1, H, H_kv, N, d, "bf16")
    nqb, nkb = -(-N // bq), -(-N // 64)
    lev = np.random.default_rng(5).integers(-1, 4, size=(1, H, nqb, nkb)).astype(np.int8)
    lev[0, 1, 2] = -1                                   # a query block that keeps nothing
    ref = run_bwd(psa, f"arbitrary maps causal={causal}", q, k, v, lev, H=H, H_kv=H_kv, d=d, q_block=bq, L=4,
                  dtype="bf16", causal=causal)
    assert np.all(ref["dq"][0, 1, 256:384] == 0)


def test_backward_dense_map_equals_dense_gradient(psa):
    N, d = 1000, 64
    q, k, v = random_qkv(41, 1, 2, 2, N, d, "bf16")
    lev = np.zeros((1, 2, 8, 16), dtype=np.int8)
    ref = run_bwd(psa, "dense map", q, k, v, lev, H=2, H_kv=2, d=d, q_block=128, L=1, dtype="bf16")
    qt, kt, vt = (torch.tensor(np.asarray(x, np.float64), requires_grad=True) for x in (q, k, v))
    dO = np.random.default_rng(0).standard_normal(q.shape)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=1 / math.sqrt(d))
    out.backward(torch.from_numpy(o.round_to_bf16(dO)).double())
    np.testing.assert_allclose(ref["dq"], qt.grad.numpy(), rtol=0, atol=1e-9)


def test_backward_full_workload_sampled(psa):
    # wan13b at full size: dq on sampled query blocks, dk and dv on sampled KV blocks
    w = get_workload("wan13b")
    L, s = w.num_levels, w.scale
    say(f"{w.name}: backward at full size, generating inputs")
    q, k, v = generate(w, "q"), generate(w, "k"), generate(w, "v")
    dO = o.round_to_bf16(np.random.default_rng(9).standard_normal(q.shape).astype(np.float32))
    prob = psa.Problem(B=w.B, H=w.H, H_kv=w.H_kv, N=w.N, d=w.d, q_block=w.q_block, num_levels=L, dtype=w.dtype)
    qd, kd, vd, dod = (to_device(x, w.dtype) for x in (q, k, v, dO))
    kp, vp, kbar = psa.psa_build_pyramid(prob, kd, vd)
    lev, _ = psa.psa_estimate_mask(prob, qd, kbar, w.thresholds())
    out, lse = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, lev, want_lse=True)
    say(f"{w.name}: GPU backward")
    dq, dk, dv = psa.psa_attention_bwd(prob, qd, kd, vd, kp, vp, lev, out, lse, dod)
    torch.cuda.synchronize()
    lev_h = lev.cpu().numpy()
    dq_g, dk_g, dv_g = to_host(dq), to_host(dk), to_host(dv)
    say(f"{w.name}: oracle on sampled blocks")
    pyr = {}
    for name, x in (("k", k), ("v", v)):
        for g in (0, 5):
            pyr[(name, g)] = [x[:, g:g + 1].astype(np.float64)] + \
                [o.round_to_io(a, w.dtype) for a in o.build_pyramid(x[:, g:g + 1], L)[1:]]
    # dq of sampled query blocks of heads 0 and 5: the oracle's backward restricted to one query block
    for h, i in ((0, 0), (0, 131), (5, 255), (5, 77)):
        r0, r1 = i * w.q_block, min((i + 1) * w.q_block, w.N)
        sub = lev_h[:, h:h + 1, i:i + 1]
        qs = np.zeros((1, 1, w.N, w.d))
        qs[:, :, r0:r1] = q[:, h:h + 1, r0:r1]
        dOs = np.zeros((1, 1, w.N, w.d))
        dOs[:, :, r0:r1] = dO[:, h:h + 1, r0:r1]
        levs = np.full((1, 1, w.nqb, w.nkb), -1, dtype=np.int8)
        levs[:, :, i] = sub[:, :, 0]
        ref = o.pyramid_attention_bwd(qs, k[:, h:h + 1], v[:, h:h + 1], L, levs, w.q_block, 64, s, dOs,
                                      io_dtype=w.dtype)
        bnd = backward_bounds(qs, k[:, h:h + 1], v[:, h:h + 1], L, levs, w.q_block, s, dOs, w.dtype)
        check_grad(dq_g[:, h:h + 1, r0:r1], ref["dq"][:, :, r0:r1], w.dtype, f"dq head {h} block {i}")
        check_grad_bound(dq_g[:, h:h + 1, r0:r1], ref["dq"][:, :, r0:r1], bnd["dq"][:, :, r0:r1],
                         f"dq head {h} block {i}", w.dtype)
    # dk, dv of sampled KV blocks: every query block of the head that keeps the block contributes
    for h, j in ((0, 3), (5, 400)):
        rows = [i for i in range(w.nqb) if lev_h[0, h, i, j] >= 0]
        levs = np.full((1, 1, w.nqb, w.nkb), -1, dtype=np.int8)
        levs[0, 0, rows] = lev_h[0, h, rows]
        ref = o.pyramid_attention_bwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], L, levs, w.q_block, 64, s,
                                      dO[:, h:h + 1], io_dtype=w.dtype)
        bnd = backward_bounds(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], L, levs, w.q_block, s,
                              dO[:, h:h + 1], w.dtype)
        t0, t1 = 64 * j, 64 * j + 64
        # only block j's own tokens are compared: other blocks also get contributions from
        # query blocks outside the sample
        for name, gg in (("dk", dk_g), ("dv", dv_g)):
            check_grad(gg[:, h:h + 1, t0:t1], ref[name][:, :, t0:t1], w.dtype, f"{name} head {h} block {j}")
            check_grad_bound(gg[:, h:h + 1, t0:t1], ref[name][:, :, t0:t1], bnd[name][:, :, t0:t1],
                             f"{name} head {h} block {j}", w.dtype)
    say(f"{w.name}: ok")


def test_backward_deterministic(psa):
    # no atomics anywhere in the backward: two calls give bit-identical gradients
    N, d = 3000, 128
    q, k, v = random_qkv(61, 1, 4, 2, N, d, "bf16")
    prob = psa.Problem(B=1, H=4, H_kv=2, N=N, d=d, q_block=128, num_levels=4, dtype="bf16")
    say("backward determinism, N=3000 gqa")
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    dod = to_device(o.round_to_bf16(np.random.default_rng(2).standard_normal(q.shape)), "bf16")
    kp, vp, kbar = psa.psa_build_pyramid(prob, kd, vd)
    lev, _ = psa.psa_estimate_mask(prob, qd, kbar, (0.3, 0.55, 0.75, 0.9))
    out, lse = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, lev, want_lse=True)
    g1 = psa.psa_attention_bwd(prob, qd, kd, vd, kp, vp, lev, out, lse, dod)
    g2 = psa.psa_attention_bwd(prob, qd, kd, vd, kp, vp, lev, out, lse, dod)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("wname", ["cogvx5b", "wan13b"])
def test_backward_repeatable_full_size(psa, wname):
    # At full size (thousands of dK/dV workgroups, whose per-key constants are shared
    # through LDS) three calls give bit-identical gradients: no read of shared state
    # races its write.
    w = get_workload(wname)
    say(f"{w.name}: backward repeatability at full size, generating inputs")
    q, k, v = generate(w, "q"), generate(w, "k"), generate(w, "v")
    dO = o.round_to_bf16(np.random.default_rng(11).standard_normal(q.shape).astype(np.float32))
    prob = psa.Problem(B=w.B, H=w.H, H_kv=w.H_kv, N=w.N, d=w.d, q_block=w.q_block, num_levels=w.num_levels,
                       dtype=w.dtype)
    qd, kd, vd, dod = (to_device(x, w.dtype) for x in (q, k, v, dO))
    kp, vp, kbar = psa.psa_build_pyramid(prob, kd, vd)
    lev, _ = psa.psa_estimate_mask(prob, qd, kbar, w.thresholds(), w.n_dense_prefix)
    out, lse = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, lev, want_lse=True)
    say(f"{w.name}: three GPU backward calls")
    g1 = psa.psa_attention_bwd(prob, qd, kd, vd, kp, vp, lev, out, lse, dod)
    for _ in range(2):
        g2 = psa.psa_attention_bwd(prob, qd, kd, vd, kp, vp, lev, out, lse, dod)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), g1, g2):
            assert torch.equal(a, b), (wname, name, float((a.float() - b.float()).abs().max()))
    say(f"{w.name}: ok")
