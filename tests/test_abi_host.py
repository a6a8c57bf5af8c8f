"""Host-only checks of the C ABI: the library loads, exports every function include/psa.h
declares, derives sizes correctly and rejects invalid arguments before launching anything
(these calls never reach the GPU, so they run without one)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psa.h")


@pytest.fixture(scope="module")
def psa():
    import level_pooled_kv_amd as lib
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(psa):
    names = declared_functions()
    assert len(names) >= 8
    assert set(names) == set(psa.EXPORTED)
    for n in names:
        assert hasattr(psa.lib, n), n


def prob(psa, **kw):
    base = dict(B=1, H=12, H_kv=12, N=32760, d=128, q_block=128, kv_block=64, num_levels=4, dtype="bf16")
    base.update(kw)
    return psa.Problem(**base)


def test_sizes(psa):
    p = prob(psa)
    assert p.pyramid_rows == sum(math.ceil(32760 / 2 ** l) for l in (1, 2, 3))
    # mean queries [B,H,nqb,d] + block scores [B,H,nqb,512] (512 KV blocks, already a power of two)
    # + one flag byte per score row
    assert p.workspace_bytes(psa.PSA_WS_ESTIMATE_MASK) == 12 * 256 * 128 * 4 + 12 * 256 * 512 * 4 + 12 * 256
    # score rows are padded to a power of two >= 64 up to 512 blocks: 278 KV blocks -> 512,
    # 32 -> 64; beyond, to a multiple of 256: 1182 -> 1280, 625 -> 768, 2048 -> 2048
    assert (prob(psa, H=48, H_kv=48, N=17776, d=64).workspace_bytes(psa.PSA_WS_ESTIMATE_MASK)
            == 48 * 139 * 64 * 4 + 48 * 139 * 512 * 4 + 48 * 139)
    assert (prob(psa, H=2, H_kv=2, N=2048, d=64, q_block=64).workspace_bytes(psa.PSA_WS_ESTIMATE_MASK)
            == 2 * 32 * 64 * 4 + 2 * 32 * 64 * 4 + 2 * 32)
    assert (prob(psa, H=40, H_kv=40, N=75600).workspace_bytes(psa.PSA_WS_ESTIMATE_MASK)
            == 40 * 591 * 128 * 4 + 40 * 591 * 1280 * 4 + 40 * 591)
    assert (prob(psa, H=1, H_kv=1, N=40000, d=64).workspace_bytes(psa.PSA_WS_ESTIMATE_MASK)
            == 313 * 64 * 4 + 313 * 768 * 4 + 313)
    assert (prob(psa, H=1, H_kv=1, N=64 * 2048).workspace_bytes(psa.PSA_WS_ESTIMATE_MASK)
            == 1024 * 128 * 4 + 1024 * 2048 * 4 + 1024)
    # backward: lse (base 2) and row dots [B,H,Npad] (N padded to 64 rows), each on a 256-byte
    # boundary, then float32 per-level gradients of K and V [B,H_kv,N+pyramid rows,d]
    r256 = lambda x: (x + 255) // 256 * 256
    rows_all = 32760 + p.pyramid_rows
    assert p.workspace_bytes(psa.PSA_WS_ATTENTION_BWD) == 2 * r256(12 * 32768 * 4) + 2 * r256(12 * rows_all * 128 * 4)
    assert p.workspace_bytes(psa.PSA_WS_ATTENTION_FWD) == 0
    assert prob(psa, num_levels=1).pyramid_rows == 0
    assert prob(psa, N=2045, num_levels=2).pyramid_rows == 1023
    assert prob(psa, d=96).pyramid_rows == 0          # malformed -> 0


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(N=-5), 1), (dict(H=12, H_kv=5), 1), (dict(num_levels=0), 1),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(causal=2), 1), (dict(causal=-1), 1),
    (dict(d=96), 2), (dict(q_block=32), 2), (dict(kv_block=128), 2), (dict(num_levels=5), 2),
    (dict(N=64 * 2048 + 1), 2), (dict(B=2, H=40000, H_kv=40000, N=64), 2),
])
def test_check_problem_rejects(psa, kw, status):
    p = prob(psa, **kw)
    st = psa.lib.psa_check_problem(ctypes.byref(p.c()))
    assert st == status, (kw, st, psa.last_error())
    assert psa.last_error() != ""


def test_check_problem_accepts_workloads(psa):
    from synth import WORKLOADS
    for w in WORKLOADS.values():
        p = psa.Problem(B=w.B, H=w.H, H_kv=w.H_kv, N=w.N, d=w.d, q_block=w.q_block, num_levels=w.num_levels,
                        dtype=w.dtype)
        assert psa.lib.psa_check_problem(ctypes.byref(p.c())) == 0, (w.name, psa.last_error())


FAKE = ctypes.c_void_p(4096)       # aligned, never dereferenced: every call below fails validation first
MISALIGNED = ctypes.c_void_p(4104)


def test_build_pyramid_rejects_bad_pointers(psa):
    p = prob(psa).c()
    f = psa.lib.psa_build_pyramid
    assert f(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert "k is NULL" in psa.last_error()
    assert f(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert f(ctypes.byref(p), FAKE, MISALIGNED, FAKE, FAKE, FAKE, None) == 1
    assert "aligned" in psa.last_error()
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    bad = prob(psa, d=80).c()
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2


def tau(*vals):
    return (ctypes.c_float * len(vals))(*vals)


def test_estimate_mask_rejects(psa):
    p = prob(psa)
    c = p.c()
    ws = p.workspace_bytes(psa.PSA_WS_ESTIMATE_MASK)
    f = psa.lib.psa_estimate_mask
    ok_tau = tau(0.1, 0.2, 0.3, 0.4)
    # thresholds: NaN, out of range, decreasing, NULL
    for t in (tau(0.1, float("nan"), 0.3, 0.4), tau(-0.1, 0.2, 0.3, 0.4), tau(0.1, 0.2, 1.5, 1.6),
              tau(0.3, 0.2, 0.4, 0.5)):
        assert f(ctypes.byref(c), FAKE, FAKE, t, 0, FAKE, None, FAKE, ws, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, None, 0, FAKE, None, FAKE, ws, None) == 1
    # n_dense_prefix outside [0, N]
    assert f(ctypes.byref(c), FAKE, FAKE, ok_tau, -1, FAKE, None, FAKE, ws, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, ok_tau, p.N + 1, FAKE, None, FAKE, ws, None) == 1
    # workspace too small
    assert f(ctypes.byref(c), FAKE, FAKE, ok_tau, 0, FAKE, None, FAKE, ws - 1, None) == 3
    assert "needed" in psa.last_error()
    # NULL / misaligned outputs
    assert f(ctypes.byref(c), FAKE, FAKE, ok_tau, 0, None, None, FAKE, ws, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, ok_tau, 0, FAKE, MISALIGNED, FAKE, ws, None) == 1


def fracs(*vals):
    return (ctypes.c_double * len(vals))(*vals)


def test_estimate_mask_ranked_rejects(psa):
    p = prob(psa)
    c = p.c()
    ws = p.workspace_bytes(psa.PSA_WS_ESTIMATE_MASK)
    f = psa.lib.psa_estimate_mask_ranked
    ok = fracs(0.1, 0.4, 0.7, 1.0)
    # fractions: NaN, out of range, decreasing, NULL
    for fr in (fracs(0.1, float("nan"), 0.7, 1.0), fracs(-0.01, 0.4, 0.7, 1.0), fracs(0.1, 0.4, 0.7, 1.01),
               fracs(0.4, 0.1, 0.7, 1.0)):
        assert f(ctypes.byref(c), FAKE, FAKE, fr, 0, FAKE, None, FAKE, ws, None) == 1
        assert "fractions" in psa.last_error()
    assert f(ctypes.byref(c), FAKE, FAKE, None, 0, FAKE, None, FAKE, ws, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, ok, -1, FAKE, None, FAKE, ws, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, ok, 0, FAKE, None, FAKE, ws - 1, None) == 3
    assert f(ctypes.byref(c), FAKE, FAKE, ok, 0, None, None, FAKE, ws, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, ok, 0, FAKE, MISALIGNED, FAKE, ws, None) == 1
    # only the first num_levels fractions are read
    c2 = prob(psa, num_levels=2).c()
    assert f(ctypes.byref(c2), FAKE, FAKE, fracs(0.1, 0.4, float("nan"), -3.0), 0, FAKE, MISALIGNED, FAKE, ws,
             None) == 1
    assert "cmass_out" in psa.last_error()


def test_similarity_entry_points_reject(psa):
    c = prob(psa).c()
    f = psa.lib.psa_build_pyramid_sim
    assert f(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1          # k_sim NULL with L = 4
    assert "k_sim" in psa.last_error()
    assert f(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, None) == 1
    assert f(ctypes.byref(c), None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    g = psa.lib.psa_apply_similarity_cap
    assert g(ctypes.byref(c), FAKE, ctypes.c_float(float("nan")), FAKE, None) == 1
    assert g(ctypes.byref(c), None, ctypes.c_float(0.5), FAKE, None) == 1
    assert g(ctypes.byref(c), FAKE, ctypes.c_float(0.5), None, None) == 1
    c1 = prob(psa, num_levels=1).c()                # nothing pooled: a no-op that launches nothing
    assert g(ctypes.byref(c1), None, ctypes.c_float(0.5), FAKE, None) == 0
    bad = prob(psa, d=96).c()
    assert g(ctypes.byref(bad), FAKE, ctypes.c_float(0.5), FAKE, None) == 2


def test_attention_rejects(psa):
    c = prob(psa).c()
    f = psa.lib.psa_attention_fwd
    assert f(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, 0, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    assert f(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, None, 0, None) == 1
    c1 = prob(psa, num_levels=1, d=64).c()     # pyramid pointers may be NULL at one level: passes
    # validation, so only check the unsupported path here (no launch without a GPU)
    bad = prob(psa, q_block=256).c()
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None, None, 0, None) == 2
    del c1


def test_status_strings(psa):
    names = [psa.status_string(s) for s in range(5)]
    assert names == ["PSA_OK", "PSA_ERR_INVALID_ARGUMENT", "PSA_ERR_UNSUPPORTED",
                     "PSA_ERR_WORKSPACE_TOO_SMALL", "PSA_ERR_HIP"]
    assert psa.status_string(99) == "PSA_ERR_UNKNOWN"


def test_binding_checks_attention_buffers(psa):
    """The binding rejects pyramid, output and lse buffers of the wrong shape or dtype before
    any pointer reaches the library (host tensors: the device check comes last)."""
    import torch
    p = prob(psa, B=1, H=2, H_kv=1, N=300, d=64, q_block=64)
    bf = torch.bfloat16
    q = torch.zeros((1, 2, 300, 64), dtype=bf)
    k = torch.zeros((1, 1, 300, 64), dtype=bf)
    lm = torch.zeros((1, 2, p.nqb, p.nkb), dtype=torch.int8)
    R = p.pyramid_rows
    kp = torch.zeros((1, 1, R, 64), dtype=bf)
    good = dict(k_pyr=kp, v_pyr=kp.clone(), o=torch.zeros_like(q), lse=torch.zeros((1, 2, 300)))
    bad = {
        "k_pyr": [None, torch.zeros((1, 1, R - 1, 64), dtype=bf), torch.zeros((1, 1, R, 64))],
        "v_pyr": [None, torch.zeros((1, 1, R, 128), dtype=bf)],
        "o": [torch.zeros((1, 2, 300, 64)), torch.zeros((1, 2, 299, 64), dtype=bf),
              torch.zeros((1, 2, 64, 300), dtype=bf).transpose(2, 3)],
        "lse": [torch.zeros((1, 2, 300), dtype=bf), torch.zeros((1, 1, 300))],
    }
    for name, cases in bad.items():
        for t in cases:
            kw = dict(good)
            kw[name] = t
            with pytest.raises(ValueError, match=name):
                psa.psa_attention_fwd(p, q, k, k, kw["k_pyr"], kw["v_pyr"], lm, o=kw["o"], lse=kw["lse"])
    # every shape right: only the device check is left, and it fails on host tensors
    with pytest.raises(ValueError, match="HIP device"):
        psa.psa_attention_fwd(p, q, k, k, good["k_pyr"], good["v_pyr"], lm, o=good["o"], lse=good["lse"])
    # one level: the pyramid may be omitted
    p1 = prob(psa, B=1, H=2, H_kv=1, N=300, d=64, q_block=64, num_levels=1)
    with pytest.raises(ValueError, match="HIP device"):
        psa.psa_attention_fwd(p1, q, k, k, None, None, lm)


def test_noalloc_rejects_problems_beyond_the_scratch(psa):
    """psa_estimate_mask_noalloc refuses, before anything else happens, a problem whose mask
    workspace exceeds the static scratch (the 75600-token, 40-head layer needs about 205 MB)."""
    f = psa.lib.psa_estimate_mask_noalloc
    big = prob(psa, H=40, H_kv=40, N=75600)
    need = big.workspace_bytes(psa.PSA_WS_ESTIMATE_MASK)
    assert need > psa.NOALLOC_SCRATCH_BYTES
    c = big.c()
    assert f(ctypes.byref(c), FAKE, FAKE, tau(0.1, 0.2, 0.3, 0.4), 0, FAKE, None, None) == 3
    assert "static scratch" in psa.last_error() and str(need) in psa.last_error()
    # argument errors come first, as in psa_estimate_mask
    small = prob(psa).c()
    assert f(ctypes.byref(small), FAKE, FAKE, tau(0.3, 0.2, 0.4, 0.5), 0, FAKE, None, None) == 1
    assert f(ctypes.byref(small), None, FAKE, tau(0.1, 0.2, 0.3, 0.4), 0, FAKE, None, None) == 1
    assert f(ctypes.byref(small), FAKE, FAKE, tau(0.1, 0.2, 0.3, 0.4), -1, FAKE, None, None) == 1
    # the bench workload fits
    assert prob(psa).workspace_bytes(psa.PSA_WS_ESTIMATE_MASK) <= psa.NOALLOC_SCRATCH_BYTES
