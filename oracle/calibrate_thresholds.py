"""Calibrate the cumulative-mass thresholds of the sparsity-targeted workloads.

TEST INFRASTRUCTURE (writes synth/thresholds.json; uses only the oracle and the
seeded input generator).

The workloads state a target FLOP fraction rho (computed FLOPs / dense FLOPs; for a
workload in causal use both count only the (query, key) pairs the causal rule lets through),
not thresholds. Reading taken: a one-parameter family tau_l(x) = tau0_l ** x with
tau0 = (0.6, 0.8, 0.9, 0.95) (the tiny workload's thresholds); rho is monotone
non-increasing in x, so bisection on log x finds x with |rho - target| <= 0.005
on the oracle's mask of the workload's seeded inputs. The thresholds are stored
as float32 values, since that is what the library receives.

With --ranked it instead matches the ranked rule to the stored thresholds: the
cumulative fraction of level l is the mean, over the query-block rows of the
threshold mask (before the dense prefix is forced), of the number of blocks at
level <= l, rounded to a whole count c and stored as (c + 0.5) / nkb so that
floor(f * nkb) = c exactly. Both rules then keep the same mean number of blocks
per level, which puts them at nearly equal FLOP fractions.

    python -m oracle.calibrate_thresholds [workload ...]
    python -m oracle.calibrate_thresholds --ranked [workload ...]
"""
from __future__ import annotations

import json
import math
import os
import sys
import time

import numpy as np

from oracle import psa_oracle as o
from synth import workloads as W
from synth.video_field import head_field


def block_means_streamed(w: W.Workload):
    """qbar [B,H,nqb,d] and kbar [B,H_kv,nkb,d] one head at a time (bounded memory)."""
    qbar = np.empty((w.B, w.H, w.nqb, w.d))
    kbar = np.empty((w.B, w.H_kv, w.nkb, w.d))
    for b in range(w.B):
        for h in range(w.H):
            qbar[b, h] = o.block_means(head_field(w, "q", b, h), w.q_block)
        for g in range(w.H_kv):
            kbar[b, g] = o.block_means(head_field(w, "k", b, g), w.kv_block)
    return qbar, kbar


def threshold_levels(w: W.Workload, C: np.ndarray, tau, n_dense_prefix: int) -> np.ndarray:
    lev = o.assign_levels(C, tau, w.num_levels, n_dense_prefix, w.kv_block)
    if w.causal:
        _, lev = o.apply_causal(C, lev, w.N, w.q_block, w.kv_block)
    return lev


def rho_of(w: W.Workload, lev: np.ndarray) -> float:
    return o.effective_flops(lev, w.N, w.q_block, w.kv_block, w.d, causal=w.causal) / w.dense_flops()


def rho_for(w: W.Workload, z: np.ndarray, C: np.ndarray, tau) -> float:
    return rho_of(w, threshold_levels(w, C, tau, w.n_dense_prefix))


def scores(w: W.Workload):
    """z (invisible blocks at -inf under causal use) and the cumulative mass C."""
    qbar, kbar = block_means_streamed(w)
    z = o.block_scores(qbar, kbar, o.block_sizes(w.N, w.kv_block), w.scale)
    if w.causal:
        vis, _ = o.causal_blocks(w.N, w.q_block, w.kv_block)
        z = np.where(vis, z, -np.inf)
    return z, o.cumulative_mass(z, o.softmax_rows(z))


def calibrate(w: W.Workload, tol: float = 0.005):
    t0 = time.time()
    z, C = scores(w)

    def tau_of(x):
        return tuple(float(np.float32(t ** x)) for t in W.TAU0[: w.num_levels])

    lo, hi = math.log(1e-3), math.log(1e3)     # rho(lo) high, rho(hi) low
    best = None
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        tau = tau_of(math.exp(mid))
        r = rho_for(w, z, C, tau)
        best = (math.exp(mid), tau, r)
        if abs(r - w.target_rho) <= tol * 0.5:
            break
        if r > w.target_rho:
            lo = mid
        else:
            hi = mid
    x, tau, r = best
    print(f"{w.name}: x={x:.6g} tau={tau} rho={r:.5f} (target {w.target_rho}) in {time.time()-t0:.1f}s",
          flush=True)
    if abs(r - w.target_rho) > tol:
        raise RuntimeError(f"{w.name}: could not reach rho={w.target_rho} (got {r})")
    return {"x": x, "thresholds": list(tau), "rho": r, "target_rho": w.target_rho}


def match_ranked(w: W.Workload, entry: dict) -> dict:
    t0 = time.time()
    if w.causal:
        raise ValueError("ranked fractions are matched for bidirectional workloads only")
    z, C = scores(w)
    tau = entry["thresholds"]
    lev = o.assign_levels(C, tau, w.num_levels, 0, w.kv_block)
    fr = []
    for l in range(w.num_levels):
        c = int(round(float(((lev >= 0) & (lev <= l)).sum(axis=-1).mean())))
        fr.append((c + 0.5) / w.nkb)
    lev_r = o.assign_levels_ranked(z, fr, w.num_levels, w.n_dense_prefix, w.kv_block)
    r = rho_of(w, lev_r)
    print(f"{w.name}: ranked fractions {fr} rho={r:.5f} (thresholds: {entry['rho']:.5f}) "
          f"in {time.time()-t0:.1f}s", flush=True)
    out = dict(entry)
    out.update({"ranked_fractions": fr, "ranked_rho": r})
    return out


def main(argv):
    ranked = "--ranked" in argv
    argv = [a for a in argv if a != "--ranked"]
    names = argv or [n for n, w in W.WORKLOADS.items() if w.target_rho is not None and not (ranked and w.causal)]
    table = {}
    if os.path.exists(W.THRESHOLDS_FILE):
        with open(W.THRESHOLDS_FILE) as f:
            table = json.load(f)
    for n in names:
        table[n] = match_ranked(W.WORKLOADS[n], table[n]) if ranked else calibrate(W.WORKLOADS[n])
        with open(W.THRESHOLDS_FILE, "w") as f:
            json.dump(table, f, indent=2, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:])
