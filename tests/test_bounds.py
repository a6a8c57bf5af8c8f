"""The element-wise error bound of the backward GPU tests, checked on the CPU: a float64
emulation of the kernels' roundings (P and dA rounded to bf16 for their products, D from
the bf16 output, bf16 outputs) stays inside it, and plausible mistakes in the pooled
gradient's spread (a wrong 1/c, a dropped level) do not."""
import math

import numpy as np
import pytest

from oracle import psa_oracle as o
from synth import random_qkv
from tests.psa_check import backward_bounds, check_grad_bound

rb = o.round_to_bf16


def emulate_bwd(q, k, v, L, lev, bq, s, dO, spread=None, drop_level=None, io="bf16"):
    """The backward with the kernels' bf16 roundings. spread[l] replaces the 1/c of level l
    (a planted mistake); drop_level skips that level's pooled gradients. io="f32": float32
    inputs and outputs, every matrix-core operand (q, keys, values, dO) rounded to bf16."""
    mc = rb if io == "f32" else (lambda x: x)          # operand rounding on the way into the matrix cores
    out = rb if io == "bf16" else (lambda x: x)         # output rounding
    q = np.asarray(q, np.float64)
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    kp = [np.asarray(k, np.float64)] + [o.round_to_io(x, io) for x in o.build_pyramid(k, L)[1:]]
    vp = [np.asarray(v, np.float64)] + [o.round_to_io(x, io) for x in o.build_pyramid(v, L)[1:]]
    dq = np.zeros_like(q)
    dkl = [np.zeros_like(x) for x in kp]
    dvl = [np.zeros_like(x) for x in vp]
    for b in range(B):
        for h in range(H):
            g = o.kv_head_of(h, H, H_kv)
            for i in range(-(-N // bq)):
                keys, vals, logc, idx = o.gather_keys(lev[b, h, i], N, 64, [x[b, g] for x in kp],
                                                      [x[b, g] for x in vp], with_index=True)
                if keys.shape[0] == 0:
                    continue
                r0, r1 = i * bq, min((i + 1) * bq, N)
                qr, km, vm = mc(q[b, h, r0:r1]), mc(keys), mc(vals)
                a = s * (qr @ km.T) + logc[None, :]
                P = np.exp(a - a.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                O = out(rb(P) @ vm)                       # forward: bf16 P for P.V, output in the I/O dtype
                dOr = dO[b, h, r0:r1]
                D = np.sum(dOr * O, axis=1, keepdims=True)
                dA = rb(P * (mc(dOr) @ vm.T - D))
                dq[b, h, r0:r1] = s * (dA @ km)
                dK = s * (dA.T @ qr)
                dV = rb(P).T @ mc(dOr)
                for l in range(L):
                    sel = idx[:, 0] == l
                    np.add.at(dkl[l][b, g], idx[sel, 1], dK[sel])
                    np.add.at(dvl[l][b, g], idx[sel, 1], dV[sel])
    dk, dv = dkl[0].copy(), dvl[0].copy()
    for l in range(1, L):
        if l == drop_level:
            continue
        c = o.pool_counts(N, l).astype(np.float64)[:, None]
        w = 1.0 / c if spread is None or l not in spread else spread[l]
        up = np.arange(N) >> l
        dk += (dkl[l] * w)[:, :, up]
        dv += (dvl[l] * w)[:, :, up]
    return {"dq": out(dq), "dk": out(dk), "dv": out(dv), "dk_levels": dkl, "dv_levels": dvl}


@pytest.fixture(scope="module")
def case():
    B, H, H_kv, N, d, bq, L = 1, 2, 1, 300, 64, 64, 4
    q, k, v = random_qkv(4242, B, H, H_kv, N, d, "bf16")
    rng = np.random.default_rng(3)
    lev = rng.integers(-1, 4, size=(B, H, -(-N // bq), -(-N // 64))).astype(np.int8)
    lev[..., 0] = 0
    dO = rb(rng.standard_normal(q.shape))
    s = 1 / math.sqrt(d)
    ref = o.pyramid_attention_bwd(q, k, v, L, lev, bq, 64, s, dO, io_dtype="bf16")
    bnd = backward_bounds(q, k, v, L, lev, bq, s, dO, "bf16")
    return q, k, v, L, lev, bq, s, dO, ref, bnd


def test_emulated_roundings_stay_inside_the_bound(case):
    q, k, v, L, lev, bq, s, dO, ref, bnd = case
    emu = emulate_bwd(q, k, v, L, lev, bq, s, dO)
    for n in ("dq", "dk", "dv"):
        ratio = check_grad_bound(emu[n], ref[n], bnd[n], n, "bf16")
        assert ratio < 1.0
    for n in ("dk_levels", "dv_levels"):
        for l in range(L):
            check_grad_bound(emu[n][l], ref[n][l], bnd[n][l], f"{n}[{l}]")


@pytest.mark.parametrize("mistake", [{"spread": {3: 1.0 / 4}}, {"spread": {2: 1.0 / 8}}, {"drop_level": 3},
                                     {"drop_level": 1}],
                         ids=["level 3 spread 1/4", "level 2 spread 1/8", "level 3 dropped", "level 1 dropped"])
def test_spread_mistakes_leave_the_bound(case, mistake):
    q, k, v, L, lev, bq, s, dO, ref, bnd = case
    bad = emulate_bwd(q, k, v, L, lev, bq, s, dO, **mistake)
    with pytest.raises(AssertionError, match="beyond their bound"):
        for n in ("dk", "dv"):
            check_grad_bound(bad[n], ref[n], bnd[n], n, "bf16")


def test_bound_is_tight_enough_to_matter(case):
    # The bound is a worst case over signs (absolute sums), so it is loosest where the
    # gradient itself cancels most: dq and dk (dA has both signs), far less for dv (P >= 0).
    # It still stays well below each gradient's typical size.
    _, _, _, _, _, _, _, _, ref, bnd = case
    for n, frac in (("dq", 0.3), ("dk", 0.5), ("dv", 0.1)):
        assert np.median(bnd[n]) < frac * np.median(np.abs(ref[n])), n


def test_float32_io_emulation_stays_inside_the_bound():
    B, H, H_kv, N, d, bq, L = 1, 2, 2, 200, 64, 64, 4
    q, k, v = random_qkv(77, B, H, H_kv, N, d, "f32")
    rng = np.random.default_rng(8)
    lev = rng.integers(-1, 4, size=(B, H, -(-N // bq), -(-N // 64))).astype(np.int8)
    lev[..., 0] = 0
    dO = rng.standard_normal(q.shape).astype(np.float32).astype(np.float64)
    s = 1 / math.sqrt(d)
    ref = o.pyramid_attention_bwd(q, k, v, L, lev, bq, 64, s, dO, io_dtype="f32")
    bnd = backward_bounds(q, k, v, L, lev, bq, s, dO, "f32")
    emu = emulate_bwd(q, k, v, L, lev, bq, s, dO, io="f32")
    for n in ("dq", "dk", "dv"):
        check_grad_bound(emu[n], ref[n], bnd[n], n, "f32")
    for n in ("dk_levels", "dv_levels"):
        for l in range(L):
            check_grad_bound(emu[n][l], ref[n][l], bnd[n][l], f"{n}[{l}]")
