"""Python binding of the MI355X Pyramid Sparse Attention forward library (libpsa.so).

Argument marshalling only: every step runs in the library's HIP kernels. Tensors
are torch tensors on the current HIP device (torch supplies device memory and the
current stream); each function passes their data pointers and sizes to the C ABI
declared in include/psa.h and raises PsaError on a non-OK status.

If libpsa.so has not been built this module raises ImportError: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PSA_LIBRARY may name another build of the same C ABI (the sanitizer host check loads its
# host-only build that way); by default the in-tree libpsa.so.
LIB_PATH = os.environ.get("PSA_LIBRARY") or os.path.join(_HERE, "libpsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python level_pooled_kv_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

PSA_OK, PSA_ERR_INVALID_ARGUMENT, PSA_ERR_UNSUPPORTED, PSA_ERR_WORKSPACE_TOO_SMALL, PSA_ERR_HIP = range(5)
PSA_F32, PSA_BF16 = 0, 1
PSA_WS_ESTIMATE_MASK, PSA_WS_ATTENTION_FWD, PSA_WS_ATTENTION_BWD = 0, 1, 2

EXPORTED = (
    "psa_pyramid_rows", "psa_workspace_bytes", "psa_check_problem", "psa_build_pyramid", "psa_build_pyramid_sim",
    "psa_apply_similarity_cap",
    "psa_estimate_mask", "psa_estimate_mask_ranked", "psa_estimate_mask_noalloc", "psa_attention_fwd", "psa_attention_bwd", "psa_status_string", "psa_last_error",
)


class psa_problem_t(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("H_kv", ctypes.c_int32),
        ("N", ctypes.c_int32), ("d", ctypes.c_int32),
        ("q_block", ctypes.c_int32), ("kv_block", ctypes.c_int32), ("num_levels", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float), ("causal", ctypes.c_int32),
    ]


_vp, _sz, _st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_P = ctypes.POINTER(psa_problem_t)
_lib.psa_pyramid_rows.argtypes, _lib.psa_pyramid_rows.restype = [_P], _sz
_lib.psa_workspace_bytes.argtypes, _lib.psa_workspace_bytes.restype = [_P, ctypes.c_int], _sz
_lib.psa_check_problem.argtypes, _lib.psa_check_problem.restype = [_P], _st
_lib.psa_build_pyramid.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.psa_build_pyramid.restype = _st
_lib.psa_build_pyramid_sim.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.psa_build_pyramid_sim.restype = _st
_lib.psa_apply_similarity_cap.argtypes = [_P, _vp, ctypes.c_float, _vp, _vp]
_lib.psa_apply_similarity_cap.restype = _st
_lib.psa_estimate_mask.argtypes = [_P, _vp, _vp, ctypes.POINTER(ctypes.c_float), ctypes.c_int32, _vp, _vp,
                                   _vp, _sz, _vp]
_lib.psa_estimate_mask.restype = _st
_lib.psa_estimate_mask_ranked.argtypes = [_P, _vp, _vp, ctypes.POINTER(ctypes.c_double), ctypes.c_int32, _vp,
                                          _vp, _vp, _sz, _vp]
_lib.psa_estimate_mask_ranked.restype = _st
_lib.psa_estimate_mask_noalloc.argtypes = [_P, _vp, _vp, ctypes.POINTER(ctypes.c_float), ctypes.c_int32, _vp, _vp,
                                           _vp]
_lib.psa_estimate_mask_noalloc.restype = _st
NOALLOC_SCRATCH_BYTES = 32 << 20     # PSA_NOALLOC_SCRATCH_BYTES
_lib.psa_attention_bwd.argtypes = [_P] + [_vp] * 13 + [_sz, _vp]
_lib.psa_attention_bwd.restype = _st
_lib.psa_attention_fwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.psa_attention_fwd.restype = _st
_lib.psa_status_string.argtypes, _lib.psa_status_string.restype = [_st], ctypes.c_char_p
_lib.psa_last_error.argtypes, _lib.psa_last_error.restype = [], ctypes.c_char_p


class PsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        name = _lib.psa_status_string(status).decode()
        super().__init__(f"{name}: {detail}")


def _check(status: int):
    if status != PSA_OK:
        raise PsaError(status, _lib.psa_last_error().decode())


@dataclass(frozen=True)
class Problem:
    """Shape of one PSA forward call (mirrors psa_problem_t)."""
    B: int
    H: int
    H_kv: int
    N: int
    d: int
    q_block: int = 128
    kv_block: int = 64
    num_levels: int = 4
    dtype: str = "bf16"           # "bf16" or "f32"
    scale: float = 0.0            # <= 0 selects 1/sqrt(d)
    causal: bool = False          # query row r sees tokens 0..r only

    def c(self) -> psa_problem_t:
        return psa_problem_t(self.B, self.H, self.H_kv, self.N, self.d, self.q_block, self.kv_block,
                             self.num_levels, PSA_BF16 if self.dtype == "bf16" else PSA_F32,
                             float(self.scale), int(self.causal))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def nqb(self) -> int:
        return -(-self.N // self.q_block)

    @property
    def nkb(self) -> int:
        return -(-self.N // self.kv_block)

    @property
    def pyramid_rows(self) -> int:
        return int(_lib.psa_pyramid_rows(ctypes.byref(self.c())))

    def workspace_bytes(self, kind: int) -> int:
        return int(_lib.psa_workspace_bytes(ctypes.byref(self.c()), kind))

    def check(self):
        _check(_lib.psa_check_problem(ctypes.byref(self.c())))


def _ptr(t: Optional[torch.Tensor]):
    """Device address of a tensor for the C ABI (after every shape and dtype check of the call)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a tensor on a HIP device, got one on {t.device}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, shape, dtype):
    """Shape, dtype and layout check (the device is checked when the pointer is taken)."""
    if t is None or tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        got = "None" if t is None else f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}"
        raise ValueError(f"{name}: expected contiguous {dtype} tensor of shape {tuple(shape)}, got {got}")


def _pyramid_buffers(prob: Problem, k, v, k_pyr, v_pyr, k_bar):
    dt = prob.torch_dtype
    kv_shape = (prob.B, prob.H_kv, prob.N, prob.d)
    _need(k, "k", kv_shape, dt)
    _need(v, "v", kv_shape, dt)
    R = prob.pyramid_rows
    if k_pyr is None:
        k_pyr = torch.empty((prob.B, prob.H_kv, max(R, 1), prob.d), dtype=dt, device=k.device)
    if v_pyr is None:
        v_pyr = torch.empty((prob.B, prob.H_kv, max(R, 1), prob.d), dtype=dt, device=k.device)
    if R > 0:
        _need(k_pyr, "k_pyr", (prob.B, prob.H_kv, R, prob.d), dt)
        _need(v_pyr, "v_pyr", (prob.B, prob.H_kv, R, prob.d), dt)
    if k_bar is None:
        k_bar = torch.empty((prob.B, prob.H_kv, prob.nkb, prob.d), dtype=torch.float32, device=k.device)
    _need(k_bar, "k_bar", (prob.B, prob.H_kv, prob.nkb, prob.d), torch.float32)
    return k_pyr, v_pyr, k_bar


def psa_build_pyramid(prob: Problem, k: torch.Tensor, v: torch.Tensor, k_pyr: Optional[torch.Tensor] = None,
                      v_pyr: Optional[torch.Tensor] = None, k_bar: Optional[torch.Tensor] = None, stream=None):
    """Step 1: pooled K/V levels 1..L-1 ([B,H_kv,R,d]) and block mean keys ([B,H_kv,nkb,d] float32).
    Missing outputs are allocated. Returns (k_pyr, v_pyr, k_bar)."""
    k_pyr, v_pyr, k_bar = _pyramid_buffers(prob, k, v, k_pyr, v_pyr, k_bar)
    _check(_lib.psa_build_pyramid(ctypes.byref(prob.c()), _ptr(k), _ptr(v), _ptr(k_pyr), _ptr(v_pyr),
                                  _ptr(k_bar), _stream(stream)))
    return k_pyr, v_pyr, k_bar


def psa_build_pyramid_sim(prob: Problem, k: torch.Tensor, v: torch.Tensor, k_pyr: Optional[torch.Tensor] = None,
                          v_pyr: Optional[torch.Tensor] = None, k_bar: Optional[torch.Tensor] = None,
                          k_sim: Optional[torch.Tensor] = None, stream=None):
    """Step 1 plus the key similarity per pooled level ([B,H_kv,nkb,L-1] float32).
    Returns (k_pyr, v_pyr, k_bar, k_sim)."""
    k_pyr, v_pyr, k_bar = _pyramid_buffers(prob, k, v, k_pyr, v_pyr, k_bar)
    shape = (prob.B, prob.H_kv, prob.nkb, max(prob.num_levels - 1, 0))
    if k_sim is None:
        k_sim = torch.empty(shape, dtype=torch.float32, device=k.device)
    _need(k_sim, "k_sim", shape, torch.float32)
    _check(_lib.psa_build_pyramid_sim(ctypes.byref(prob.c()), _ptr(k), _ptr(v), _ptr(k_pyr), _ptr(v_pyr),
                                      _ptr(k_bar), _ptr(k_sim) if k_sim.numel() else None, _stream(stream)))
    return k_pyr, v_pyr, k_bar, k_sim


def psa_apply_similarity_cap(prob: Problem, k_sim: torch.Tensor, threshold: float, level_map: torch.Tensor,
                             stream=None):
    """Caps the levels of level_map in place by the key similarity; returns level_map."""
    _need(k_sim, "k_sim", (prob.B, prob.H_kv, prob.nkb, max(prob.num_levels - 1, 0)), torch.float32)
    _need(level_map, "level_map", (prob.B, prob.H, prob.nqb, prob.nkb), torch.int8)
    _check(_lib.psa_apply_similarity_cap(ctypes.byref(prob.c()), _ptr(k_sim) if k_sim.numel() else None,
                                         ctypes.c_float(float(threshold)), _ptr(level_map), _stream(stream)))
    return level_map


def _mask_buffers(prob: Problem, q, k_bar, level_map, cmass, want_cmass, workspace):
    _need(q, "q", (prob.B, prob.H, prob.N, prob.d), prob.torch_dtype)
    _need(k_bar, "k_bar", (prob.B, prob.H_kv, prob.nkb, prob.d), torch.float32)
    shape = (prob.B, prob.H, prob.nqb, prob.nkb)
    if level_map is None:
        level_map = torch.empty(shape, dtype=torch.int8, device=q.device)
    _need(level_map, "level_map", shape, torch.int8)
    if cmass is None and want_cmass:
        cmass = torch.empty(shape, dtype=torch.float32, device=q.device)
    if cmass is not None:
        _need(cmass, "cmass", shape, torch.float32)
    ws_bytes = prob.workspace_bytes(PSA_WS_ESTIMATE_MASK)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    return level_map, cmass, workspace


def _per_level(prob: Problem, values: Sequence[float], name: str, ctype):
    if len(values) < prob.num_levels:
        raise ValueError(f"{name}: {len(values)} values for {prob.num_levels} levels")
    return (ctype * len(values))(*[float(x) for x in values])


def psa_estimate_mask(prob: Problem, q: torch.Tensor, k_bar: torch.Tensor, thresholds: Sequence[float],
                      n_dense_prefix: int = 0, level_map: Optional[torch.Tensor] = None,
                      cmass: Optional[torch.Tensor] = None, want_cmass: bool = False,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Step 2: level map [B,H,nqb,nkb] int8 (-1 = pruned); optionally the float32 cumulative mass.
    Returns (level_map, cmass or None)."""
    level_map, cmass, workspace = _mask_buffers(prob, q, k_bar, level_map, cmass, want_cmass, workspace)
    tau = _per_level(prob, thresholds, "thresholds", ctypes.c_float)
    _check(_lib.psa_estimate_mask(ctypes.byref(prob.c()), _ptr(q), _ptr(k_bar), tau, int(n_dense_prefix),
                                  _ptr(level_map), _ptr(cmass), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return level_map, cmass


def psa_estimate_mask_noalloc(prob: Problem, q: torch.Tensor, k_bar: torch.Tensor, thresholds: Sequence[float],
                              n_dense_prefix: int, level_map: torch.Tensor, cmass: Optional[torch.Tensor] = None,
                              stream=None):
    """Step 2 with the library's static device scratch as workspace (the C call allocates
    nothing; the caller passes every output). Returns (level_map, cmass or None)."""
    _need(q, "q", (prob.B, prob.H, prob.N, prob.d), prob.torch_dtype)
    _need(k_bar, "k_bar", (prob.B, prob.H_kv, prob.nkb, prob.d), torch.float32)
    shape = (prob.B, prob.H, prob.nqb, prob.nkb)
    _need(level_map, "level_map", shape, torch.int8)
    if cmass is not None:
        _need(cmass, "cmass", shape, torch.float32)
    tau = _per_level(prob, thresholds, "thresholds", ctypes.c_float)
    _check(_lib.psa_estimate_mask_noalloc(ctypes.byref(prob.c()), _ptr(q), _ptr(k_bar), tau, int(n_dense_prefix),
                                          _ptr(level_map), _ptr(cmass), _stream(stream)))
    return level_map, cmass


def psa_estimate_mask_ranked(prob: Problem, q: torch.Tensor, k_bar: torch.Tensor, fractions: Sequence[float],
                             n_dense_prefix: int = 0, level_map: Optional[torch.Tensor] = None,
                             cmass: Optional[torch.Tensor] = None, want_cmass: bool = False,
                             workspace: Optional[torch.Tensor] = None, stream=None):
    """Step 2, ranked rule: the top floor(fractions[l] * nkb) blocks of each row take level l
    or a finer one. Returns (level_map, cmass or None)."""
    level_map, cmass, workspace = _mask_buffers(prob, q, k_bar, level_map, cmass, want_cmass, workspace)
    fr = _per_level(prob, fractions, "fractions", ctypes.c_double)
    _check(_lib.psa_estimate_mask_ranked(ctypes.byref(prob.c()), _ptr(q), _ptr(k_bar), fr, int(n_dense_prefix),
                                         _ptr(level_map), _ptr(cmass), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))
    return level_map, cmass


def psa_attention_fwd(prob: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      k_pyr: Optional[torch.Tensor], v_pyr: Optional[torch.Tensor], level_map: torch.Tensor,
                      o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      want_lse: bool = False, stream=None):
    """Step 3: O [B,H,N,d] (I/O dtype) and optionally LSE [B,H,N] float32. Returns (o, lse or None)."""
    dt = prob.torch_dtype
    _need(q, "q", (prob.B, prob.H, prob.N, prob.d), dt)
    _need(k, "k", (prob.B, prob.H_kv, prob.N, prob.d), dt)
    _need(v, "v", (prob.B, prob.H_kv, prob.N, prob.d), dt)
    _need(level_map, "level_map", (prob.B, prob.H, prob.nqb, prob.nkb), torch.int8)
    if prob.num_levels > 1:
        for t, name in ((k_pyr, "k_pyr"), (v_pyr, "v_pyr")):
            _need(t, name, (prob.B, prob.H_kv, prob.pyramid_rows, prob.d), dt)
    if o is None:
        o = torch.empty_like(q)
    _need(o, "o", (prob.B, prob.H, prob.N, prob.d), dt)
    if lse is None and want_lse:
        lse = torch.empty((prob.B, prob.H, prob.N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", (prob.B, prob.H, prob.N), torch.float32)
    _check(_lib.psa_attention_fwd(ctypes.byref(prob.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(k_pyr), _ptr(v_pyr),
                                  _ptr(level_map), _ptr(o), _ptr(lse), None, 0, _stream(stream)))
    return o, lse


def psa_attention_bwd(prob: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      k_pyr: Optional[torch.Tensor], v_pyr: Optional[torch.Tensor], level_map: torch.Tensor,
                      o: torch.Tensor, lse: torch.Tensor, d_o: torch.Tensor, dq: Optional[torch.Tensor] = None,
                      dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Backward of step 3 with the level map fixed: returns (dq, dk, dv)."""
    dt = prob.torch_dtype
    q_shape = (prob.B, prob.H, prob.N, prob.d)
    kv_shape = (prob.B, prob.H_kv, prob.N, prob.d)
    for t, name, shape in ((q, "q", q_shape), (k, "k", kv_shape), (v, "v", kv_shape), (o, "o", q_shape),
                           (d_o, "d_o", q_shape)):
        _need(t, name, shape, dt)
    _need(lse, "lse", (prob.B, prob.H, prob.N), torch.float32)
    _need(level_map, "level_map", (prob.B, prob.H, prob.nqb, prob.nkb), torch.int8)
    if prob.num_levels > 1:
        for t, name in ((k_pyr, "k_pyr"), (v_pyr, "v_pyr")):
            _need(t, name, (prob.B, prob.H_kv, prob.pyramid_rows, prob.d), dt)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", q_shape, dt)
    _need(dk, "dk", kv_shape, dt)
    _need(dv, "dv", kv_shape, dt)
    ws_bytes = prob.workspace_bytes(PSA_WS_ATTENTION_BWD)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    _check(_lib.psa_attention_bwd(ctypes.byref(prob.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(k_pyr), _ptr(v_pyr),
                                  _ptr(level_map), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv


def psa_forward(prob: Problem, q, k, v, thresholds, n_dense_prefix: int = 0, stream=None):
    """The three steps chained. Returns a dict with k_pyr, v_pyr, k_bar, level_map, o."""
    k_pyr, v_pyr, k_bar = psa_build_pyramid(prob, k, v, stream=stream)
    level_map, _ = psa_estimate_mask(prob, q, k_bar, thresholds, n_dense_prefix, stream=stream)
    o, _ = psa_attention_fwd(prob, q, k, v, k_pyr, v_pyr, level_map, stream=stream)
    return {"k_pyr": k_pyr, "v_pyr": v_pyr, "k_bar": k_bar, "level_map": level_map, "o": o}


def status_string(status: int) -> str:
    return _lib.psa_status_string(status).decode()


def last_error() -> str:
    return _lib.psa_last_error().decode()


lib = _lib
