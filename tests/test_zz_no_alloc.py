"""psa_estimate_mask_noalloc (static device scratch, allocates nothing) against
psa_estimate_mask (caller's workspace) through the C ABI, on two calls in a row, the
second smaller than the first. Same kernels, so the level maps and cumulative masses
must be identical element for element."""

import numpy as np
import pytest
import torch

from synth import random_qkv
from tests.psa_check import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def psa():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import level_pooled_kv_amd as lib
    return lib


CALLS = [
    # B, H, H_kv, N, d, q_block, dtype, thresholds, n_dense_prefix, want_cmass
    (2, 4, 2, 20000, 128, 128, "bf16", (0.01, 0.1, 0.3, 0.6), 100, True),
    (1, 2, 1, 3000, 64, 64, "f32", (0.05, 0.2, 0.4, 0.7), 0, False),
]


def test_noalloc_matches_workspace_entry_point(psa):
    for n, (B, H, H_kv, N, d, bq, dtype, tau, ndp, want_c) in enumerate(CALLS):
        print(f"[gpu-case] noalloc call {n}: B={B} H={H} H_kv={H_kv} N={N} d={d} q_block={bq} {dtype} "
              f"cmass={want_c}", flush=True)
        prob = psa.Problem(B=B, H=H, H_kv=H_kv, N=N, d=d, q_block=bq, num_levels=4, dtype=dtype)
        assert prob.workspace_bytes(psa.PSA_WS_ESTIMATE_MASK) <= psa.NOALLOC_SCRATCH_BYTES
        q, k, v = random_qkv(300 + n, B, H, H_kv, N, d, dtype)
        qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
        _, _, kbar = psa.psa_build_pyramid(prob, kd, vd)
        shape = (B, H, prob.nqb, prob.nkb)
        lev_ref, cm_ref = psa.psa_estimate_mask(prob, qd, kbar, tau, ndp, want_cmass=want_c)
        lev = torch.full(shape, 99, dtype=torch.int8, device=qd.device)
        cm = torch.full(shape, float("nan"), dtype=torch.float32, device=qd.device) if want_c else None
        psa.psa_estimate_mask_noalloc(prob, qd, kbar, tau, ndp, lev, cm)
        torch.cuda.synchronize()
        assert torch.equal(lev, lev_ref), n
        if want_c:
            assert torch.equal(cm, cm_ref), n
        hist = np.bincount(lev.cpu().numpy().ravel().astype(np.int64) + 1, minlength=5)
        print(f"[gpu-case] noalloc call {n}: ok, levels -1..3 = {hist.tolist()}", flush=True)
