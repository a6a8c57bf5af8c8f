"""Benchmark of the MI355X Pyramid Sparse Attention forward path (one GPU).

    python bench.py [--steps K] [--warmup W] [--workload wan13b] [--no-cpu-baseline]
                    [--rule threshold|ranked] [--fractions f0,f1,f2,f3]
    python bench.py --compare-rules [--workload wan13b]   (accuracy of the mask rules)

A step is one pass of the whole forward path over one batch of resident inputs:
psa_build_pyramid, psa_estimate_mask (psa_estimate_mask_ranked with --rule ranked) and
psa_attention_fwd, enqueued on one stream.
W untimed steps, then K timed steps bracketed by device synchronisation (the "warm"
loop: `value` and ms_per_step come from its wall clock), with HIP events around the
attention call only (a single kernel launch, the roofline's kernel; an event record
leaves a gap on the stream). Then K untimed steps with events around every call (the
pyramid's and the mask's per-call times), then K more, each after a 512 MiB read that
evicts L2 and the MALL (the "cold" loop, outside `value`). Per call: mean, median, p10
and p90 of the warm and cold loops.

Throughput is effective TFLOP/s: FLOPs of QK^T and PV on the retained pooled rows
only (sum over retained blocks of 4 * rows * pooled_rows * d), divided by the step
time. The CPU baseline times the float64 oracle on ten heads of the same workload.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_wan13b_traffic.txt")
ATTN_SOURCES = [os.path.join(ROOT, "level_pooled_kv_amd", "csrc", f)
                for f in ("psa_attn_common.h", "psa_attention.hip")]
MASK_SOURCES = [os.path.join(ROOT, "level_pooled_kv_amd", "csrc", "psa_mask.hip")]


def attention_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for f in sources or ATTN_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def attention_kernel_name(d: int, q_block: int, dtype: str) -> str:
    t = "bf16" if dtype == "bf16" else "float"
    return f"pyramid_attn_fwd_kernel<{t},{d},4,{128 // q_block}>"


def effective_flops(level_map: np.ndarray, N: int, q_block: int, kv_block: int, d: int,
                    causal: bool = False) -> float:
    """sum over retained (b,h,i,j): 4 * d * (query row, pooled row) pairs, i.e.
    4 * m_i * ceil(n_j / 2^l) * d; in causal use only the pairs where the pooled row's last
    token is at or before the query row count."""
    nqb, nkb = level_map.shape[-2], level_map.shape[-1]
    m = np.minimum(q_block, N - np.arange(nqb) * q_block).astype(np.int64)
    n = np.minimum(kv_block, N - np.arange(nkb) * kv_block)
    lm = level_map.reshape(-1, nqb, nkb)
    total = 0.0
    for l in range(4):
        sel = (lm == l).astype(np.float64)
        if not sel.any():
            continue
        if not causal:
            rows = (-(-n // (1 << l))).astype(np.float64)
            total += float(np.einsum("xij,i,j->", sel, m.astype(np.float64), rows))
            continue
        P = 1 << l
        p = np.arange(kv_block // P)
        last = np.minimum(np.arange(nkb)[:, None] * kv_block + (p[None, :] + 1) * P, N) - 1
        last = np.where(p[None, :] * P < n[:, None], last, 1 << 40)
        r0 = (np.arange(nqb) * q_block)[:, None, None]
        pairs = np.clip(r0 + m[:, None, None] - np.maximum(r0, last[None]), 0, None).sum(-1).astype(np.float64)
        total += float(np.einsum("xij,ij->", sel, pairs))
    return 4.0 * d * total


def tile_matrix_flops(level_map: np.ndarray, N: int, q_block: int, d: int) -> float:
    """Matrix-core FLOPs the attention kernel executes: per query block, the tiles of its
    level lists (2^l blocks of level l share one 64-key tile, so a level's last tile may be
    part empty) times 64 keys x q_block query rows (a short last query block still runs whole
    tiles) x 4d for QK^T and PV."""
    lm = level_map.reshape(-1, level_map.shape[-1])
    tiles = 0
    for l in range(4):
        cnt = (lm == l).sum(axis=1)
        tiles += int(((cnt + (1 << l) - 1) >> l).sum())
    return 4.0 * d * 64 * q_block * tiles


def level_histogram(level_map: np.ndarray):
    return {str(l): int((level_map == l).sum()) for l in (-1, 0, 1, 2, 3)}


def traffic_from_profile(workload: str, plain_step: bool, key: str = "hbm_bytes_per_launch",
                         hash_key: str = "attention_source_sha256", sources=None):
    """HBM bytes from the committed rocprofv3 counter summary (per attention launch by
    default; key selects another figure), if it was taken on the current source of those
    kernels and on this workload's default step (else None)."""
    if workload != "wan13b" or not plain_step or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get(hash_key) != attention_source_hash(sources or ATTN_SOURCES):
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, q, k, v, tau, fractions=None):
    """Oracle (float64 NumPy) on a bounded sample: every step for about ten query heads (whole KV-head groups)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import psa_oracle as o

    cores = len(os.sched_getaffinity(0))        # the host cores this process may run on
    threadpool_limits(cores)                    # the oracle's BLAS uses exactly those
    t0 = time.perf_counter()
    group = w.H // w.H_kv                       # query heads per KV head
    nkv = max(1, min(w.H_kv, 10 // group))      # whole groups, about ten query heads
    nh = nkv * group
    qh = q[:, :nh].astype(np.float64)
    kh = k[:, :nkv].astype(np.float64)
    vh = v[:, :nkv].astype(np.float64)
    res = o.run_forward(qh, kh, vh, w.q_block, w.kv_block, tau, w.num_levels, w.scale, w.dtype,
                        w.n_dense_prefix, ranked_fractions=fractions, causal=w.causal)
    dt = time.perf_counter() - t0
    fl = o.effective_flops(res["mask"]["levels"], w.N, w.q_block, w.kv_block, w.d, causal=w.causal)
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "blas_threads": int(threads),
            "kind": "oracle",
            "sample": f"{w.name}: all three steps (pyramid, mask, attention) for heads 0..{nh - 1} of {w.H}, "
                      f"{fl:.3e} effective FLOPs in {dt:.1f} s, float64 NumPy"}


def compare_rules(psa, w, qd, kd, vd, steps: int):
    """Output error against dense attention for four level-assignment rules at nearly equal
    FLOP fractions: multi-level thresholds, multi-level ranked (matched block counts), and
    their binary (one-level) forms keeping as many blocks as the multi-level masks' FLOPs
    allow. Every step runs in the library's kernels; dense attention is the same attention
    kernel with every block at level 0. Prints one JSON line."""
    import torch
    if w.causal:
        raise SystemExit("--compare-rules covers bidirectional workloads only")
    dev = qd.device
    tau, fr = w.thresholds(), list(w.ranked_fractions())

    def problem(L):
        return psa.Problem(B=w.B, H=w.H, H_kv=w.H_kv, N=w.N, d=w.d, q_block=w.q_block, kv_block=w.kv_block,
                           num_levels=L, dtype=w.dtype)

    pL, p1 = problem(w.num_levels), problem(1)
    k_pyr, v_pyr, k_bar = psa.psa_build_pyramid(pL, kd, vd)
    dense_map = torch.zeros((w.B, w.H, pL.nqb, pL.nkb), dtype=torch.int8, device=dev)
    o_dense, _ = psa.psa_attention_fwd(p1, qd, kd, vd, None, None, dense_map)
    ref = o_dense.float()

    def measure(prob, lm, kp, vp):
        out, _ = psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, lm)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            psa.psa_attention_fwd(prob, qd, kd, vd, kp, vp, lm, o=out)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        x = out.float()
        rel = float(torch.linalg.vector_norm(x - ref) / torch.linalg.vector_norm(ref))
        cos = float(torch.nn.functional.cosine_similarity(x.reshape(-1, w.d), ref.reshape(-1, w.d), dim=1).mean())
        lmh = lm.cpu().numpy()
        rho = effective_flops(lmh, w.N, w.q_block, w.kv_block, w.d) / w.dense_flops()
        return {"rho": round(rho, 5), "rel_l2_err": round(rel, 5), "mean_cos": round(cos, 6),
                "attention_ms": round(ms, 4), "levels": level_histogram(lmh)}

    res = {}
    lm_t, _ = psa.psa_estimate_mask(pL, qd, k_bar, tau, w.n_dense_prefix)
    res["multi-level thresholds"] = measure(pL, lm_t, k_pyr, v_pyr)
    lm_r, _ = psa.psa_estimate_mask_ranked(pL, qd, k_bar, fr, w.n_dense_prefix)
    res["multi-level ranked"] = measure(pL, lm_r, k_pyr, v_pyr)
    # binary masks at the same FLOP fraction: keep rho * nkb blocks per row
    rho_t = res["multi-level thresholds"]["rho"]
    keep = int(round(rho_t * w.nkb))
    lm_b, _ = psa.psa_estimate_mask_ranked(p1, qd, k_bar, [(keep + 0.5) / w.nkb], w.n_dense_prefix)
    res["binary top-k"] = measure(p1, lm_b, None, None)
    lo, hi = 0.0, 1.0                      # binary threshold with the same mean kept count
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        lm, _ = psa.psa_estimate_mask(p1, qd, k_bar, [mid], w.n_dense_prefix)
        kept = float((lm >= 0).float().sum(-1).mean())
        lo, hi = (mid, hi) if kept < keep else (lo, mid)
    lm_bt, _ = psa.psa_estimate_mask(p1, qd, k_bar, [hi], w.n_dense_prefix)
    res["binary threshold"] = measure(p1, lm_bt, None, None)
    res["binary threshold"]["threshold"] = hi
    print(json.dumps({"metric": "relative L2 error of O against dense attention at equal FLOP fraction",
                      "workload": f"{w.name}: {w.description}", "data": "synthetic", "rules": res,
                      "thresholds": list(tau), "fractions": fr, "binary_keep_blocks": keep}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan13b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rule", choices=("threshold", "ranked"), default="threshold",
                    help="level assignment: the workload's thresholds, or fixed shares of the ranked blocks")
    ap.add_argument("--fractions", default=None,
                    help="ranked rule: comma-separated cumulative block fractions per level "
                         "(default: the workload's, matched to its threshold mask's mean level counts)")
    ap.add_argument("--similarity", type=float, default=None, metavar="THRESHOLD",
                    help="add the cosine-similarity constraint: the pyramid step also computes the key "
                         "similarity and the level map is capped at THRESHOLD before attention")
    ap.add_argument("--backward", action="store_true",
                    help="also time psa_attention_bwd on the step's output and report it under 'backward'")
    ap.add_argument("--compare-rules", action="store_true",
                    help="only compare the output error of threshold / ranked / binary masks at equal "
                         "FLOP fraction against dense attention, print that JSON line and exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (calibrates HBM byte counters) and exit")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        n = args.copy_probe * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "copies": 3}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the forward path has no cross-GPU step here; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import level_pooled_kv_amd as psa
    from synth import get as get_workload, generate

    w = get_workload(args.workload)
    tau = w.thresholds()
    fractions = None
    if args.rule == "ranked":
        fractions = ([float(x) for x in args.fractions.split(",")] if args.fractions
                     else list(w.ranked_fractions()))
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    q, k, v = generate(w, "q"), generate(w, "k"), generate(w, "v")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    qd = torch.from_numpy(q).to(dt).to(dev)
    kd = torch.from_numpy(k).to(dt).to(dev)
    vd = torch.from_numpy(v).to(dt).to(dev)
    if args.compare_rules:
        compare_rules(psa, w, qd, kd, vd, args.steps)
        return
    prob = psa.Problem(B=w.B, H=w.H, H_kv=w.H_kv, N=w.N, d=w.d, q_block=w.q_block, kv_block=w.kv_block,
                       num_levels=w.num_levels, dtype=w.dtype, causal=w.causal)
    R = prob.pyramid_rows
    k_pyr = torch.empty((w.B, w.H_kv, R, w.d), dtype=dt, device=dev)
    v_pyr = torch.empty_like(k_pyr)
    k_bar = torch.empty((w.B, w.H_kv, prob.nkb, w.d), dtype=torch.float32, device=dev)
    k_sim = torch.empty((w.B, w.H_kv, prob.nkb, max(w.num_levels - 1, 1)), dtype=torch.float32, device=dev)
    level_map = torch.empty((w.B, w.H, prob.nqb, prob.nkb), dtype=torch.int8, device=dev)
    ws = torch.empty(prob.workspace_bytes(psa.PSA_WS_ESTIMATE_MASK), dtype=torch.uint8, device=dev)
    o = torch.empty_like(qd)

    def step(ev=None):
        # ev: four events around the three calls (a None entry is not recorded)
        if ev and ev[0]: ev[0].record()
        if args.similarity is None:
            psa.psa_build_pyramid(prob, kd, vd, k_pyr, v_pyr, k_bar)
        else:
            psa.psa_build_pyramid_sim(prob, kd, vd, k_pyr, v_pyr, k_bar, k_sim)
        if ev and ev[1]: ev[1].record()
        if fractions is None:
            psa.psa_estimate_mask(prob, qd, k_bar, tau, w.n_dense_prefix, level_map=level_map, workspace=ws)
        else:
            psa.psa_estimate_mask_ranked(prob, qd, k_bar, fractions, w.n_dense_prefix, level_map=level_map,
                                         workspace=ws)
        if args.similarity is not None:
            psa.psa_apply_similarity_cap(prob, k_sim, args.similarity, level_map)
        if ev and ev[2]: ev[2].record()
        psa.psa_attention_fwd(prob, qd, kd, vd, k_pyr, v_pyr, level_map, o=o)
        if ev and ev[3]: ev[3].record()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # warm: K steps back to back (the timed region of `value` and ms_per_step), with events
    # around the attention call only (the roofline's live kernel time); every event record
    # leaves a gap on the stream, so the other calls are timed in a second warm loop
    att_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step([None, None, att_events[s][0], att_events[s][1]])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    attn_warm = np.array([e[0].elapsed_time(e[1]) for e in att_events])            # ms
    # warm, instrumented: K more steps with events around every call (untimed)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in events])   # ms
    per[:, 2] = attn_warm
    pyr_ms, mask_ms, attn_ms = (float(np.mean(per[:, i])) for i in range(3))
    # cold: K more steps, each after reading a 512 MiB buffer (evicts L2 and the 256 MB MALL,
    # so the step's inputs come from HBM). A read leaves only clean lines behind; a write
    # would leave dirty ones whose write-back the next step would pay for. The flush is
    # outside the per-call events.
    print(f"[bench] cold loop ({args.steps} steps, 512 MiB read before each)", file=sys.stderr, flush=True)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    cold_events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        torch.sum(flush, dim=0, out=sink)
        step(cold_events[s])
    torch.cuda.synchronize()
    per_cold = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(3)] for e in cold_events])
    del flush

    bwd = None
    if args.backward:
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        psa.psa_attention_fwd(prob, qd, kd, vd, k_pyr, v_pyr, level_map, o=o, lse=lse)
        d_o = torch.randn(qd.shape, generator=torch.Generator(device=dev).manual_seed(7), device=dev).to(dt)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        bws = torch.empty(prob.workspace_bytes(psa.PSA_WS_ATTENTION_BWD), dtype=torch.uint8, device=dev)
        for _ in range(max(args.warmup, 1)):
            psa.psa_attention_bwd(prob, qd, kd, vd, k_pyr, v_pyr, level_map, o, lse, d_o, dq, dk, dv, workspace=bws)
        torch.cuda.synchronize()
        bev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        bev[0].record()
        for s_ in range(args.steps):
            psa.psa_attention_bwd(prob, qd, kd, vd, k_pyr, v_pyr, level_map, o, lse, d_o, dq, dk, dv, workspace=bws)
            bev[s_ + 1].record()
        torch.cuda.synchronize()
        bwd = float(np.mean([bev[i].elapsed_time(bev[i + 1]) for i in range(args.steps)]))

    lm = level_map.cpu().numpy()
    flops = effective_flops(lm, w.N, w.q_block, w.kv_block, w.d, causal=w.causal)
    rho = flops / w.dense_flops()
    esz = 2 if w.dtype == "bf16" else 4
    kv_bytes = 2 * w.B * w.H_kv * w.N * w.d * esz
    pyr_bytes = kv_bytes + 2 * w.B * w.H_kv * R * w.d * esz + k_bar.numel() * 4
    mask_bytes = w.B * w.H * w.N * w.d * esz + k_bar.numel() * 4 + lm.size
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    traffic = traffic_from_profile(w.name, fractions is None and args.similarity is None)
    # measured bytes of the mask kernels, their float32 scratch (query means, score rows) included
    mask_traffic = traffic_from_profile(w.name, fractions is None and args.similarity is None,
                                        "mask_hbm_bytes_per_call", "mask_source_sha256", MASK_SOURCES)
    tile_flops = tile_matrix_flops(lm, w.N, w.q_block, w.d)

    def stats(x):
        return {"mean": round(float(np.mean(x)), 4), "median": round(float(np.median(x)), 4),
                "p10": round(float(np.percentile(x, 10)), 4), "p90": round(float(np.percentile(x, 90)), 4)}

    calls = {}
    for name, col in (("build_pyramid", 0), ("estimate_mask", 1), ("attention_fwd", 2)):
        calls[name] = {"warm": stats(per[:, col]), "cold": stats(per_cold[:, col])}
    step_cold = per_cold.sum(axis=1)

    result = {
        "metric": "PSA fwd ms/call + effective TFLOP/s (% MFMA peak) at 32760 tok, ~91% sparsity",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "B": w.B, "H": w.H, "H_kv": w.H_kv,
                   "N": w.N, "d": w.d, "q_block": w.q_block, "kv_block": w.kv_block,
                   "num_levels": w.num_levels, "causal": w.causal, "parallelism": "single GPU",
                   **({"rule": "threshold", "thresholds": list(tau)} if fractions is None
                      else {"rule": "ranked", "fractions": fractions}),
                   **({} if args.similarity is None else {"similarity_threshold": args.similarity})},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": attention_kernel_name(w.d, w.q_block, w.dtype)},
        "calls_ms": {"build_pyramid": round(pyr_ms, 4), "estimate_mask": round(mask_ms, 4),
                     "attention_fwd": round(attn_ms, 4)},
        "calls_ms_stats": calls,
        "step_ms_cold": stats(step_cold),
        "roofline_cold": {"achieved": round(flops / (float(np.median(per_cold[:, 2])) * 1e-3) / 1e12, 2),
                          "frac": round(flops / (float(np.median(per_cold[:, 2])) * 1e-3) / 1e12
                                        / PEAK_BF16_TFLOPS, 4),
                          "of": "median attention_fwd duration of the cold loop"},
        "tile_padding": {"matrix_flops": tile_flops, "effective_flops": flops,
                         "padding_frac": round(1.0 - flops / tile_flops, 4) if tile_flops else None,
                         "what": "matrix-core work the attention kernel's 64-key tiles and whole query "
                                 "blocks execute (QK^T and PV), against the effective FLOPs"},
        "effective_flops": flops, "flop_fraction_rho": round(rho, 5),
        "hbm": {"build_pyramid_GBps": round(pyr_bytes / (pyr_ms * 1e-3) / 1e9, 1),
                "build_pyramid_frac": round(pyr_bytes / (pyr_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "estimate_mask_GBps": round(mask_bytes / (mask_ms * 1e-3) / 1e9, 1),
                "estimate_mask_frac": round(mask_bytes / (mask_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "build_pyramid_frac_cold": round(
                    pyr_bytes / (float(np.median(per_cold[:, 0])) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "estimate_mask_frac_cold": round(
                    mask_bytes / (float(np.median(per_cold[:, 1])) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "build_pyramid_bytes": pyr_bytes, "estimate_mask_bytes": mask_bytes,
                "estimate_mask_traffic_bytes": mask_traffic},
        "levels": level_histogram(lm),
    }
    if bwd is not None:
        # algorithmic backward work: the five products of an attention backward (S and dP
        # recomputed once, dq, dK, dV), 2.5 x the forward's two
        bflops = 2.5 * flops
        result["backward"] = {"ms_per_call": round(bwd, 4), "effective_flops": bflops,
                              "achieved_tflops": round(bflops / (bwd * 1e-3) / 1e12, 2),
                              "frac_of_peak": round(bflops / (bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "call": "psa_attention_bwd (row dots, dq, dK/dV, unpool)"}
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a head sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, tau, fractions)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
