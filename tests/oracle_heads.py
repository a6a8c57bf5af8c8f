"""Whole-head attention parity at full size: the oracle's attention for every query block
of one (batch, head), computed in a worker process, against the GPU's output for that head.

Workers are started with 'spawn' and import only NumPy, the oracle and the input
generators (never torch, never the GPU); each regenerates its head's seeded inputs, so
only the level-map rows and the GPU output cross the process boundary."""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from oracle import psa_oracle as o
from synth import generate, get as get_workload

ATT_MAX_ABS = 2e-2
ATT_MEAN_ABS = 2e-3


def lse_tolerance(q: np.ndarray, k: np.ndarray, scale: float, dtype: str) -> np.ndarray:
    """Per-row bound on |lse_gpu - lse_oracle| ([B, H, N]).

    bf16 I/O: the matrix cores multiply the exact bf16 inputs and accumulate in float32,
    so only float32 accumulation error remains (1e-3 is generous). float32 I/O: q and k are
    rounded to bf16 first, so every product q_c*k_c carries a relative error below 2^-8 and
    every logit of row r moves by at most 2^-8 * scale * sum_c |q_rc| * max_t |k_tc|;
    the log-sum-exp moves by at most the largest logit change."""
    B, H, N, d = q.shape
    tol = np.full((B, H, N), 1e-3)
    if dtype == "f32":
        H_kv = k.shape[1]
        kmax = np.abs(k).max(axis=2)                                   # [B, H_kv, d]
        kmax_h = np.repeat(kmax, H // H_kv, axis=1)                    # [B, H, d]
        tol += 2.0 ** -8 * scale * np.einsum("bhnd,bhd->bhn", np.abs(q), kmax_h)
    return tol


def head_stats(task):
    """task = (workload name, b, h, level-map rows [nqb, nkb], GPU O [N, d], GPU lse [N]).
    Returns the error statistics of that head against the oracle."""
    wname, b, h, lev, out, lse = task
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                      # pragma: no cover
        threadpool_limits = None
    if threadpool_limits is None:
        return _head_stats(wname, b, h, lev, out, lse)
    with threadpool_limits(2):
        return _head_stats(wname, b, h, lev, out, lse)


def _head_stats(wname, b, h, lev, out, lse):
    w = get_workload(wname)
    g = o.kv_head_of(h, w.H, w.H_kv)
    q = generate(w, "q", heads=[h], batches=[b]).astype(np.float64)
    k = generate(w, "k", heads=[g], batches=[b])
    v = generate(w, "v", heads=[g], batches=[b])
    kp = [k.astype(np.float64)] + [o.round_to_io(x, w.dtype) for x in o.build_pyramid(k, w.num_levels)[1:]]
    vp = [v.astype(np.float64)] + [o.round_to_io(x, w.dtype) for x in o.build_pyramid(v, w.num_levels)[1:]]
    O, LSE = o.pyramid_attention(q, kp, vp, lev[None, None], w.q_block, w.kv_block, w.scale, causal=w.causal)
    O, LSE = O[0, 0], LSE[0, 0]
    g_out = out.astype(np.float64)
    err = np.abs(g_out - O)
    fin = np.isfinite(LSE)
    tol = lse_tolerance(q, k, w.scale, w.dtype)[0, 0]
    lse_err = np.abs(lse.astype(np.float64) - LSE)
    return {"b": b, "h": h, "max": float(np.nanmax(err)) if not np.isnan(err).all() else float("nan"),
            "sum": float(np.nansum(err)), "count": int(err.size), "nan": int(np.isnan(g_out).sum()),
            "worst_row": int(np.unravel_index(np.nanargmax(err), err.shape)[0]) if not np.isnan(err).all() else -1,
            "lse_pattern_ok": bool(np.array_equal(np.isfinite(lse), fin)),
            "lse_bad": int((lse_err[fin] > tol[fin]).sum()),
            "lse_max_err": float(lse_err[fin].max()) if fin.any() else 0.0}


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:                   # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(8, n))


def compare_heads(wname: str, heads, lev: np.ndarray, out: np.ndarray, lse: np.ndarray, say=print):
    """Oracle attention for every query block of each (b, h) in ``heads`` against the GPU's
    output ``out`` [B, H, N, d] and ``lse`` [B, H, N] (host arrays), computed on the level
    map ``lev`` [B, H, nqb, nkb]. Asserts max-abs <= 2e-2 on every element, mean-abs <= 2e-3
    over all compared elements, no NaN, and the lse bound on every row. Returns
    (max abs error, mean abs error, compared elements)."""
    tasks = [(wname, b, h, np.ascontiguousarray(lev[b, h]), np.ascontiguousarray(out[b, h], dtype=np.float32),
              np.ascontiguousarray(lse[b, h], dtype=np.float32)) for (b, h) in heads]
    n = min(workers(), len(tasks))
    say(f"{wname}: oracle attention on {len(tasks)} whole heads, {n} worker processes")
    ctx = mp.get_context("spawn")
    with ctx.Pool(n) as pool:
        res = pool.map(head_stats, tasks, chunksize=1)
    mx = max(r["max"] for r in res)
    tot = sum(r["sum"] for r in res)
    cnt = sum(r["count"] for r in res)
    mean = tot / cnt
    bad = [r for r in res if r["nan"] or r["max"] > ATT_MAX_ABS or not r["lse_pattern_ok"] or r["lse_bad"]]
    assert not bad, (wname, "heads off", bad[:3])
    assert mean <= ATT_MEAN_ABS, (wname, "mean abs error over all compared rows", mean)
    return mx, mean, cnt
