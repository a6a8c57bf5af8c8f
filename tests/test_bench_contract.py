"""The benchmark's contract: its algorithmic FLOP count (the numerator of `value` and of the
roofline) against brute-force pair counting, the refusal of more than one GPU, and (on a
GPU) the fields and internal consistency of the one JSON line it prints."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_force_flops(lev, N, q_block, kv_block, d, causal):
    """4 d x the (query row, pooled key row) pairs of every retained (head, query block,
    KV block, level); in causal use a pair counts when the pooled row's last token is at
    or before the query row. Pure loops over rows and tokens."""
    H, nqb, nkb = lev.shape
    pairs = 0
    for h in range(H):
        for i in range(nqb):
            rows = range(i * q_block, min((i + 1) * q_block, N))
            for j in range(nkb):
                l = int(lev[h, i, j])
                if l < 0:
                    continue
                t0, t1 = j * kv_block, min((j + 1) * kv_block, N)
                for p0 in range(t0, t1, 1 << l):
                    last = min(p0 + (1 << l), t1) - 1
                    pairs += sum(1 for r in rows if not causal or last <= r)
    return 4.0 * d * pairs


@pytest.mark.parametrize("causal", [False, True], ids=["bidirectional", "causal"])
@pytest.mark.parametrize("N,q_block", [(300, 64), (517, 128), (256, 64)])
def test_effective_flops_brute_force(N, q_block, causal):
    rng = np.random.default_rng(N + q_block)
    nqb, nkb = -(-N // q_block), -(-N // 64)
    lev = rng.integers(-1, 4, size=(3, nqb, nkb)).astype(np.int8)
    want = brute_force_flops(lev, N, q_block, 64, 8, causal)
    got = bench.effective_flops(lev[None], N, q_block, 64, 8, causal=causal)
    assert got == want


def test_tile_flops_cover_the_effective_ones():
    # The kernel packs 2^l blocks of level l into one 64-key tile and runs whole tiles for
    # all q_block rows: never less than the effective work, and equal to it when every
    # level's block count is a multiple of 2^l and no block or query block is short.
    rng = np.random.default_rng(5)
    N, q_block, d = 1024, 128, 16
    lev = rng.integers(-1, 4, size=(1, 2, N // q_block, N // 64)).astype(np.int8)
    assert bench.tile_matrix_flops(lev, N, q_block, d) >= bench.effective_flops(lev, N, q_block, 64, d)
    even = np.full((1, 1, N // q_block, N // 64), -1, dtype=np.int8)
    even[..., 0:8] = 3       # 8 level-3 blocks: one tile
    even[..., 8:12] = 2      # 4 level-2 blocks: one tile
    even[..., 12:14] = 1     # 2 level-1 blocks: one tile
    even[..., 14] = 0        # 1 level-0 block: one tile
    assert bench.tile_matrix_flops(even, N, q_block, d) == bench.effective_flops(even, N, q_block, 64, d)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_json_line():
    print("[gpu-case] bench.py --steps 3 --warmup 1 --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.strip()]
    assert len(lines) == 1, lines
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "effective_flops"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 1
    assert j["higher_is_better"] is True and j["data"] == "synthetic" and j["dtype"] == "bf16"
    assert j["unit"] == "TFLOP/s" and "workload" in j["config"]
    # value: the step's effective FLOPs over the wall-clock step time
    assert j["value"] == pytest.approx(j["effective_flops"] / (j["ms_per_step"] * 1e-3) / 1e12, rel=1e-3)
    roof = j["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "mfma" and roof["peak"] == 2500.0 and roof["unit"] == "TFLOP/s"
    attn_ms = j["calls_ms"]["attention_fwd"]
    assert roof["achieved"] == pytest.approx(j["effective_flops"] / (attn_ms * 1e-3) / 1e12, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert 0.0 < roof["frac"] < 1.0
    assert attn_ms < j["ms_per_step"]
