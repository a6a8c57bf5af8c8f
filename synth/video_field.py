"""Seeded synthetic video-shaped Q/K/V (the only module both the HIP path's tests
and the oracle draw inputs from).

Recipe, per tensor X in {Q, K, V}, batch b, head h, channel c, for a token at
grid position (t, y, x) of a (T, H_grid, W) latent grid in raster order
n = n_text + (t*H_grid + y)*W + x:

    X = sum_{m=1..8} 0.5 * sin(2*pi*(ft*t/T + fy*y/H_grid + fx*x/W) + phi) + eps

with fy, fx ~ U[0, 2], ft ~ U[0, ft_max] (0.5 for the "stronger temporal
correlation" workload, else 2), phi ~ U[0, 2*pi), eps ~ N(0, 0.3^2). Amplitude
0.5 per sinusoid gives every channel unit RMS (8 * 0.5^2 / 2 = 1). Text tokens
(placed first) are i.i.d. N(0, 1). Every (workload, tensor, b, head) draws from
its own numpy PCG64 stream seeded by SeedSequence([20251203, workload index,
tensor index, b, h]); draw order: ft, fy, fx, phi (each [d, 8]), eps [N_grid, d]
float32, text [n_text, d] float32.

Values are returned as float32. For bf16 workloads they are rounded to the
nearest bf16 (ties to even) here, so a float32 array holds exactly the bf16 input.
Nothing in this module computes any step of the attention method.
"""
from __future__ import annotations

import numpy as np

from .workloads import Workload

SEED_ROOT = 20251203
TENSORS = {"q": 0, "k": 1, "v": 2}
N_SINUSOIDS = 8


def _round_f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def head_field(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """One (b, h) slice [N, d] of tensor 'q', 'k' or 'v', float32."""
    ti = TENSORS[tensor]
    rng = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, w.index, ti, b, h]))
    d = w.d
    T, Hg, W = w.grid
    ft = rng.uniform(0.0, w.ft_max, size=(d, N_SINUSOIDS))
    fy = rng.uniform(0.0, 2.0, size=(d, N_SINUSOIDS))
    fx = rng.uniform(0.0, 2.0, size=(d, N_SINUSOIDS))
    phi = rng.uniform(0.0, 2.0 * np.pi, size=(d, N_SINUSOIDS))
    n_grid = T * Hg * W
    eps = rng.standard_normal(size=(n_grid, d), dtype=np.float32)
    text = rng.standard_normal(size=(w.n_text, d), dtype=np.float32) if w.n_text else None

    # Separable evaluation: exp(i*(a+b+c+phi)) = exp(ia) exp(ib) exp(ic) exp(i*phi).
    two_pi = 2.0 * np.pi
    et = np.exp(1j * two_pi * ft[None, :, :] * (np.arange(T)[:, None, None] / T))     # [T, d, 8]
    ey = np.exp(1j * two_pi * fy[None, :, :] * (np.arange(Hg)[:, None, None] / Hg))   # [Hg, d, 8]
    ex = np.exp(1j * two_pi * fx[None, :, :] * (np.arange(W)[:, None, None] / W))     # [W, d, 8]
    amp = 0.5 * np.exp(1j * phi)                                                        # [d, 8]
    a = (et[:, None] * ey[None, :] * amp).reshape(T * Hg, d, N_SINUSOIDS)              # [T*Hg, d, 8]
    # field[c, ty, x] = Im(sum_m a[ty, c, m] * ex[x, c, m])
    a_c = np.ascontiguousarray(a.transpose(1, 0, 2)).astype(np.complex128)             # [d, T*Hg, 8]
    ex_c = np.ascontiguousarray(ex.transpose(1, 2, 0)).astype(np.complex128)           # [d, 8, W]
    field = np.matmul(a_c, ex_c).imag                                                   # [d, T*Hg, W]
    grid_vals = field.reshape(d, n_grid).T.astype(np.float32)                           # [n_grid, d]
    grid_vals += np.float32(0.3) * eps

    out = np.empty((w.N, d), dtype=np.float32)
    if text is not None:
        out[: w.n_text] = text
    out[w.n_text:] = grid_vals
    if w.dtype == "bf16":
        out = _round_f32_to_bf16(out)
    return out


def tensor_heads(w: Workload, tensor: str) -> int:
    return w.H if tensor == "q" else w.H_kv


def generate(w: Workload, tensor: str, heads=None, batches=None) -> np.ndarray:
    """Tensor 'q' [B,H,N,d] or 'k'/'v' [B,H_kv,N,d] as float32 (bf16-exact for bf16 workloads).

    ``heads`` / ``batches`` restrict the result to a subset (in that order)."""
    hs = list(range(tensor_heads(w, tensor))) if heads is None else list(heads)
    bs = list(range(w.B)) if batches is None else list(batches)
    out = np.empty((len(bs), len(hs), w.N, w.d), dtype=np.float32)
    for bi, b in enumerate(bs):
        for hi, h in enumerate(hs):
            out[bi, hi] = head_field(w, tensor, b, h)
    return out


def generate_qkv(w: Workload):
    return generate(w, "q"), generate(w, "k"), generate(w, "v")


def random_qkv(seed: int, B: int, H: int, H_kv: int, N: int, d: int, dtype: str = "bf16",
               scale: float = 1.0):
    """Small i.i.d. N(0, scale^2) inputs for edge-case tests (ragged N, odd shapes)."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED_ROOT, 1000 + seed]))
    q = (scale * rng.standard_normal((B, H, N, d))).astype(np.float32)
    k = (scale * rng.standard_normal((B, H_kv, N, d))).astype(np.float32)
    v = (scale * rng.standard_normal((B, H_kv, N, d))).astype(np.float32)
    if dtype == "bf16":
        q, k, v = _round_f32_to_bf16(q), _round_f32_to_bf16(k), _round_f32_to_bf16(v)
    return q, k, v
