"""Thin Python binding of libflowcache.so (argument marshalling only).

Every function here has the name of the C entry point it calls, takes torch
tensors that already live on the GPU, passes their device pointers and the
current HIP stream through ctypes, and raises ``FlowCacheError`` on a non-OK
status.  torch provides device memory and streams; all arithmetic runs in the
library's HIP kernels.  Importing this module loads the library and fails
loudly when it has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libflowcache.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
        "or python kv_cache_compression_fc_amd/csrc/build.py). There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

FC_OK, FC_ERR_INVALID_ARG, FC_ERR_UNSUPPORTED, FC_ERR_WORKSPACE, FC_ERR_HIP = range(5)
FC_F32, FC_BF16 = 0, 1
FC_MAX_CHUNKS = 128

EXPORTS = (
    "fc_status_string", "fc_kv_compress_workspace_bytes", "fc_kv_compress", "fc_kv_importance",
    "fc_kv_importance_lse", "fc_kv_importance_colsum", "fc_kv_importance_redundancy",
    "fc_kv_redundancy", "fc_kv_select", "fc_topb_select_workspace_bytes", "fc_topb_select",
    "fc_chunk_rel_l1_workspace_bytes", "fc_chunk_rel_l1_decide",
    "fc_cache_commit_workspace_bytes", "fc_cache_commit", "fc_euler_step_l1_decide",
    "fc_uniform_rel_l1_decide", "fc_history_rel_l1_decide", "fc_chunk_rel_l1_decide_noalloc",
)
FC_NOALLOC_SCRATCH_BYTES = 256 * 1024


class fc_kv_params(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("d", ctypes.c_int32), ("L_q", ctypes.c_int32),
                ("L_k", ctypes.c_int32), ("B_budget", ctypes.c_int32), ("lambda_", ctypes.c_float),
                ("pool_window", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int)]


class fc_cache_params(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("d", ctypes.c_int32), ("B_budget", ctypes.c_int32),
                ("B_active", ctypes.c_int32), ("lambda_", ctypes.c_float), ("pool_window", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int)]


class fc_l1_params(ctypes.Structure):
    _fields_ = [("n_chunks", ctypes.c_int32), ("m", ctypes.c_int32), ("eps", ctypes.c_float),
                ("dtype", ctypes.c_int)]


_vp, _sz = ctypes.c_void_p, ctypes.c_size_t
_i64p = ctypes.POINTER(ctypes.c_int64)
_lib.fc_status_string.restype = ctypes.c_char_p
_lib.fc_status_string.argtypes = [ctypes.c_int]
_lib.fc_kv_compress_workspace_bytes.restype = _sz
_lib.fc_kv_compress_workspace_bytes.argtypes = [ctypes.POINTER(fc_kv_params)]
_lib.fc_kv_compress.restype = ctypes.c_int
_lib.fc_kv_compress.argtypes = [ctypes.POINTER(fc_kv_params)] + [_vp] * 9 + [_vp, _sz, _vp]
_lib.fc_kv_importance.restype = ctypes.c_int
_lib.fc_kv_importance.argtypes = [ctypes.POINTER(fc_kv_params), _vp, _vp, _vp, _vp, _sz, _vp]
_lib.fc_kv_importance_redundancy.restype = ctypes.c_int
_lib.fc_kv_importance_redundancy.argtypes = [ctypes.POINTER(fc_kv_params), _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.fc_kv_importance_lse.restype = ctypes.c_int
_lib.fc_kv_importance_lse.argtypes = [ctypes.POINTER(fc_kv_params), _vp, _vp, _vp, _vp, _sz, _vp]
_lib.fc_kv_importance_colsum.restype = ctypes.c_int
_lib.fc_kv_importance_colsum.argtypes = [ctypes.POINTER(fc_kv_params), _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.fc_kv_redundancy.restype = ctypes.c_int
_lib.fc_kv_redundancy.argtypes = [ctypes.POINTER(fc_kv_params), _vp, _vp, _vp, _sz, _vp]
_lib.fc_kv_select.restype = ctypes.c_int
_lib.fc_kv_select.argtypes = [ctypes.POINTER(fc_kv_params)] + [_vp] * 10 + [_vp, _sz, _vp]
_lib.fc_topb_select_workspace_bytes.restype = _sz
_lib.fc_topb_select_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
_lib.fc_topb_select.restype = ctypes.c_int
_lib.fc_topb_select.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _sz, _vp]
_lib.fc_chunk_rel_l1_workspace_bytes.restype = _sz
_lib.fc_chunk_rel_l1_workspace_bytes.argtypes = [ctypes.POINTER(fc_l1_params), _i64p]
_lib.fc_chunk_rel_l1_decide.restype = ctypes.c_int
_lib.fc_chunk_rel_l1_decide.argtypes = [ctypes.POINTER(fc_l1_params), _i64p, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _sz, _vp]
_lib.fc_chunk_rel_l1_decide_noalloc.restype = ctypes.c_int
_lib.fc_chunk_rel_l1_decide_noalloc.argtypes = [ctypes.POINTER(fc_l1_params), _i64p, _vp, _vp, _vp, _vp, _vp, _vp,
                                                _vp]

_lib.fc_cache_commit_workspace_bytes.restype = _sz
_lib.fc_cache_commit_workspace_bytes.argtypes = [ctypes.POINTER(fc_cache_params), ctypes.c_int32]
_lib.fc_cache_commit.restype = ctypes.c_int
_lib.fc_cache_commit.argtypes = [ctypes.POINTER(fc_cache_params), ctypes.POINTER(ctypes.c_int32), _vp, _vp,
                                 ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp,
                                 ctypes.POINTER(ctypes.c_int32), _vp, _sz, _vp]
_lib.fc_euler_step_l1_decide.restype = ctypes.c_int
_lib.fc_euler_step_l1_decide.argtypes = [ctypes.POINTER(fc_l1_params), _i64p] + [_vp] * 8 + [_vp, _sz, _vp]
_lib.fc_uniform_rel_l1_decide.restype = ctypes.c_int
_lib.fc_uniform_rel_l1_decide.argtypes = [ctypes.POINTER(fc_l1_params), _i64p] + [_vp] * 7 + [_vp, _sz, _vp]
_lib.fc_history_rel_l1_decide.restype = ctypes.c_int
_lib.fc_history_rel_l1_decide.argtypes = [ctypes.POINTER(fc_l1_params), _i64p] + [_vp] * 6 + [_vp, _sz, _vp]


class FlowCacheError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {fc_status_string(status)} (status {status})")
        self.status = status


def fc_status_string(status: int) -> str:
    return _lib.fc_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != FC_OK:
        raise FlowCacheError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(name: str, t: Optional[torch.Tensor], shape, dtype=None) -> None:
    """The library reads and writes exactly the extents its arguments imply;
    a tensor of another shape or dtype would be accessed out of bounds, so it
    is refused here, before any pointer crosses the boundary."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _expect_flat(name: str, t: Optional[torch.Tensor], min_numel: int, dtype) -> None:
    """A flat state: any shape, at least min_numel elements of dtype."""
    if t is None:
        return
    if t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, the offsets need {min_numel}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == FC_BF16 else torch.float32


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FC_BF16
    if t.dtype == torch.float32:
        return FC_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def kv_params(Q: torch.Tensor, K: torch.Tensor, B_budget: int, lam: float, pool_window: int,
              softmax_scale: float = 0.0) -> fc_kv_params:
    """Parameters of Q [H][L_q][d] and K [H][L_k][d] (same dtype)."""
    if Q.dim() != 3 or K.dim() != 3:
        raise ValueError("Q and K must be [H][L][d]")
    H, Lq, d = Q.shape
    _expect("K", K, (H, K.shape[1], d), Q.dtype)
    return fc_kv_params(H, d, Lq, K.shape[1], int(B_budget), float(lam), int(pool_window),
                        float(softmax_scale), _dtype_code(K))


def fc_kv_compress_workspace_bytes(p: fc_kv_params) -> int:
    return int(_lib.fc_kv_compress_workspace_bytes(ctypes.byref(p)))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    return workspace


def _nbytes(t: Optional[torch.Tensor]) -> int:
    """Size in bytes of a workspace tensor of any dtype (0 for None, which the
    library answers with FC_ERR_WORKSPACE)."""
    return 0 if t is None else t.numel() * t.element_size()


def _chunk_workspace(p: fc_l1_params, chunk_offsets: Sequence[int], workspace: Optional[torch.Tensor],
                     device) -> torch.Tensor:
    """The caller's workspace, or one sized by the query when none is given."""
    if workspace is not None:
        return workspace
    return torch.empty(max(fc_chunk_rel_l1_workspace_bytes(p, chunk_offsets), 1), dtype=torch.uint8, device=device)


def fc_kv_compress(Q, K, V, B_budget: int, lam: float, pool_window: int, softmax_scale: float = 0.0,
                   want_scores: bool = False, out: Optional[Dict[str, torch.Tensor]] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> Dict[str, torch.Tensor]:
    """Whole compression step.  Returns K_out, V_out, idx (+ score,
    imp_pooled, red when want_scores).  ``out`` may hold preallocated outputs."""
    p = kv_params(Q, K, B_budget, lam, pool_window, softmax_scale)
    H, Lk, d = K.shape
    Bp = min(int(B_budget), Lk)
    out = dict(out or {})
    dev = K.device
    out.setdefault("K_out", torch.empty((H, Bp, d), dtype=K.dtype, device=dev))
    out.setdefault("V_out", torch.empty((H, Bp, d), dtype=V.dtype, device=dev))
    out.setdefault("idx", torch.empty((H, Bp), dtype=torch.int32, device=dev))
    if want_scores:
        for k in ("score", "imp_pooled", "red"):
            out.setdefault(k, torch.empty((H, Lk), dtype=torch.float32, device=dev))
    _expect("V", V, (H, Lk, d), K.dtype)
    for k in ("K_out", "V_out"):
        _expect(k, out[k], (H, Bp, d), K.dtype)
    _expect("idx", out["idx"], (H, Bp), torch.int32)
    for k in ("score", "imp_pooled", "red"):
        _expect(k, out.get(k), (H, Lk), torch.float32)
    nbytes = fc_kv_compress_workspace_bytes(p)
    ws = _workspace(nbytes, dev, workspace)
    _check("fc_kv_compress", _lib.fc_kv_compress(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(out["K_out"]), _ptr(out["V_out"]), _ptr(out["idx"]),
        _ptr(out.get("score")), _ptr(out.get("imp_pooled")), _ptr(out.get("red")),
        _ptr(ws), _nbytes(ws), _stream(stream)))
    return out


def fc_kv_importance(Q, K, softmax_scale: float = 0.0, imp_out=None, workspace=None, stream=None) -> torch.Tensor:
    p = kv_params(Q, K, 1, 0.5, 1, softmax_scale)
    H, Lk, _ = K.shape
    if imp_out is None:
        imp_out = torch.empty((H, Lk), dtype=torch.float32, device=K.device)
    _expect("imp_out", imp_out, (H, Lk), torch.float32)
    ws = _workspace(fc_kv_compress_workspace_bytes(p), K.device, workspace)
    _check("fc_kv_importance", _lib.fc_kv_importance(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(imp_out), _ptr(ws),
                                                     _nbytes(ws), _stream(stream)))
    return imp_out


def fc_kv_importance_redundancy(Q, K, softmax_scale: float = 0.0, imp_out=None, r_out=None, workspace=None,
                                stream=None):
    """(importance before the pool, redundancy mean), both [H][L_k] f32, from
    the launches of fc_kv_compress's first half."""
    p = kv_params(Q, K, 1, 0.5, 1, softmax_scale)
    H, Lk, _ = K.shape
    if imp_out is None:
        imp_out = torch.empty((H, Lk), dtype=torch.float32, device=K.device)
    if r_out is None:
        r_out = torch.empty((H, Lk), dtype=torch.float32, device=K.device)
    _expect("imp_out", imp_out, (H, Lk), torch.float32)
    _expect("r_out", r_out, (H, Lk), torch.float32)
    ws = _workspace(fc_kv_compress_workspace_bytes(p), K.device, workspace)
    _check("fc_kv_importance_redundancy", _lib.fc_kv_importance_redundancy(
        ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(imp_out), _ptr(r_out), _ptr(ws), _nbytes(ws), _stream(stream)))
    return imp_out, r_out


def fc_kv_importance_lse(Q, K, softmax_scale: float = 0.0, lse_out=None, workspace=None, stream=None):
    p = kv_params(Q, K, 1, 0.5, 1, softmax_scale)
    H, Lq, _ = Q.shape
    if lse_out is None:
        lse_out = torch.empty((H, Lq), dtype=torch.float32, device=Q.device)
    _expect("lse_out", lse_out, (H, Lq), torch.float32)
    ws = _workspace(fc_kv_compress_workspace_bytes(p), K.device, workspace)
    _check("fc_kv_importance_lse", _lib.fc_kv_importance_lse(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(lse_out),
                                                             _ptr(ws), _nbytes(ws), _stream(stream)))
    return lse_out


def fc_kv_importance_colsum(Q, K, lse, softmax_scale: float = 0.0, imp_out=None, workspace=None, stream=None):
    p = kv_params(Q, K, 1, 0.5, 1, softmax_scale)
    H, Lk, _ = K.shape
    if imp_out is None:
        imp_out = torch.empty((H, Lk), dtype=torch.float32, device=K.device)
    _expect("lse", lse, (H, Q.shape[1]), torch.float32)
    _expect("imp_out", imp_out, (H, Lk), torch.float32)
    ws = _workspace(fc_kv_compress_workspace_bytes(p), K.device, workspace)
    _check("fc_kv_importance_colsum", _lib.fc_kv_importance_colsum(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(lse),
                                                                   _ptr(imp_out), _ptr(ws), _nbytes(ws),
                                                                   _stream(stream)))
    return imp_out


def fc_kv_redundancy(K, r_out=None, workspace=None, stream=None) -> torch.Tensor:
    H, Lk, d = K.shape
    p = fc_kv_params(H, d, 1, Lk, 1, 0.5, 1, 0.0, _dtype_code(K))
    if r_out is None:
        r_out = torch.empty((H, Lk), dtype=torch.float32, device=K.device)
    _expect("r_out", r_out, (H, Lk), torch.float32)
    ws = _workspace(fc_kv_compress_workspace_bytes(p), K.device, workspace)
    _check("fc_kv_redundancy", _lib.fc_kv_redundancy(ctypes.byref(p), _ptr(K), _ptr(r_out), _ptr(ws), _nbytes(ws),
                                                     _stream(stream)))
    return r_out


def fc_kv_select(imp, r, B_budget: int, lam: float, pool_window: int, K=None, V=None, want_scores: bool = True,
                 workspace=None, stream=None) -> Dict[str, torch.Tensor]:
    H, Lk = imp.shape
    _expect("r", r, (H, Lk), torch.float32)
    _expect("imp", imp, (H, Lk), torch.float32)
    if (K is None) != (V is None):
        raise ValueError("K and V are given together or not at all")
    d = K.shape[2] if K is not None else 64
    _expect("K", K, (H, Lk, d))
    _expect("V", V, (H, Lk, d), K.dtype if K is not None else None)
    dt = _dtype_code(K) if K is not None else FC_F32
    p = fc_kv_params(H, d, 1, Lk, int(B_budget), float(lam), int(pool_window), 0.0, dt)
    Bp = min(int(B_budget), Lk)
    dev = imp.device
    out = {"idx": torch.empty((H, Bp), dtype=torch.int32, device=dev)}
    if K is not None:
        out["K_out"] = torch.empty((H, Bp, d), dtype=K.dtype, device=dev)
        out["V_out"] = torch.empty((H, Bp, d), dtype=V.dtype, device=dev)
    if want_scores:
        for k in ("score", "imp_pooled", "red"):
            out[k] = torch.empty((H, Lk), dtype=torch.float32, device=dev)
    ws = _workspace(fc_kv_compress_workspace_bytes(p), dev, workspace)
    _check("fc_kv_select", _lib.fc_kv_select(
        ctypes.byref(p), _ptr(imp), _ptr(r), _ptr(K), _ptr(V), _ptr(out.get("K_out")), _ptr(out.get("V_out")),
        _ptr(out["idx"]), _ptr(out.get("score")), _ptr(out.get("imp_pooled")), _ptr(out.get("red")),
        _ptr(ws), _nbytes(ws), _stream(stream)))
    return out


def fc_topb_select_workspace_bytes(H: int, L: int) -> int:
    return int(_lib.fc_topb_select_workspace_bytes(int(H), int(L)))


def fc_topb_select(scores: torch.Tensor, B: int, idx_out=None, workspace=None, stream=None) -> torch.Tensor:
    H, L = scores.shape
    _expect("scores", scores, (H, L), torch.float32)
    if idx_out is None:
        idx_out = torch.empty((H, min(int(B), L)), dtype=torch.int32, device=scores.device)
    _expect("idx_out", idx_out, (H, min(int(B), L)), torch.int32)
    ws = _workspace(fc_topb_select_workspace_bytes(H, L), scores.device, workspace)
    _check("fc_topb_select", _lib.fc_topb_select(H, L, int(B), _ptr(scores), _ptr(idx_out), _ptr(ws), _nbytes(ws),
                                                 _stream(stream)))
    return idx_out


def _offsets(chunk_offsets: Sequence[int]):
    arr = (ctypes.c_int64 * len(chunk_offsets))(*[int(x) for x in chunk_offsets])
    return arr


def fc_chunk_rel_l1_workspace_bytes(p: fc_l1_params, chunk_offsets: Sequence[int]) -> int:
    return int(_lib.fc_chunk_rel_l1_workspace_bytes(ctypes.byref(p), _offsets(chunk_offsets)))


# The (m, eps) settings the FlowCache page reports (Key designs item 2): m
# forced-recompute steps (5 for MAGI-1, 4 for SkyReels-V2) and the reuse
# threshold of its slow (quality) and fast (speed) settings.
DECISION_PRESETS = {
    "magi-slow": (5, 0.01),
    "magi-fast": (5, 0.015),
    "skyreels-slow": (4, 0.1),
    "skyreels-fast": (4, 0.15),
}


class ChunkDecider:
    """Holds the per-chunk state (step, f) and the workspace on the device and
    calls fc_chunk_rel_l1_decide once per denoising step."""

    @classmethod
    def preset(cls, name: str, chunk_offsets: Sequence[int], dtype: torch.dtype, device="cuda") -> "ChunkDecider":
        """A decider with one of DECISION_PRESETS' (m, eps) settings."""
        if name not in DECISION_PRESETS:
            raise ValueError(f"unknown preset {name!r}; one of {sorted(DECISION_PRESETS)}")
        m, eps = DECISION_PRESETS[name]
        return cls(chunk_offsets, m, eps, dtype, device)

    def __init__(self, chunk_offsets: Sequence[int], m: int, eps: float, dtype: torch.dtype, device="cuda"):
        self.offsets = [int(x) for x in chunk_offsets]
        n = len(self.offsets) - 1
        self.p = fc_l1_params(n, int(m), float(eps), FC_BF16 if dtype == torch.bfloat16 else FC_F32)
        nbytes = fc_chunk_rel_l1_workspace_bytes(self.p, self.offsets)
        if nbytes == 0:
            raise FlowCacheError("fc_chunk_rel_l1_workspace_bytes", FC_ERR_INVALID_ARG)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.step = torch.full((n,), -1, dtype=torch.int32, device=device)
        self.f = torch.zeros(n, dtype=torch.float32, device=device)
        self.recompute = torch.zeros(n, dtype=torch.uint8, device=device)
        self.l1 = torch.zeros(n, dtype=torch.float32, device=device)

    def decide(self, X_t: torch.Tensor, X_tm1: torch.Tensor, stream=None) -> None:
        fc_chunk_rel_l1_decide(self.p, self.offsets, X_t, X_tm1, self.step, self.f, self.recompute, self.l1,
                               self.workspace, stream)

    def euler_step(self, X_t: torch.Tensor, v: torch.Tensor, dt: torch.Tensor, X_next: torch.Tensor,
                   stream=None) -> None:
        """X_next = X_t + v dt per chunk (dt: device f32 [n_chunks]) and the decision on that pair."""
        fc_euler_step_l1_decide(self.p, self.offsets, X_t, v, dt, X_next, self.step, self.f, self.recompute, self.l1,
                                self.workspace, stream)


def _expect_chunk_state(p: fc_l1_params, chunk_offsets: Sequence[int], states, per_chunk) -> None:
    """states: (name, tensor) laid out as the flat chunks; per_chunk: (name,
    tensor, length, dtype) of the per-chunk (or shared) device arrays."""
    if len(chunk_offsets) != p.n_chunks + 1:
        raise ValueError(f"{len(chunk_offsets)} offsets for {p.n_chunks} chunks")
    need = max(int(x) for x in chunk_offsets)
    for name, t in states:
        _expect_flat(name, t, need, _torch_dtype(p.dtype))
    for name, t, n, dt in per_chunk:
        _expect(name, t, (n,), dt)


def fc_chunk_rel_l1_decide(p: fc_l1_params, chunk_offsets: Sequence[int], X_t, X_tm1, step, f, recompute,
                           l1_rel_out=None, workspace=None, stream=None) -> None:
    n = p.n_chunks
    _expect_chunk_state(p, chunk_offsets, (("X_t", X_t), ("X_tm1", X_tm1)),
                        (("step", step, n, torch.int32), ("f", f, n, torch.float32),
                         ("recompute", recompute, n, torch.uint8), ("l1_rel_out", l1_rel_out, n, torch.float32)))
    workspace = _chunk_workspace(p, chunk_offsets, workspace, X_t.device)
    _check("fc_chunk_rel_l1_decide", _lib.fc_chunk_rel_l1_decide(
        ctypes.byref(p), _offsets(chunk_offsets), _ptr(X_t), _ptr(X_tm1), _ptr(step), _ptr(f), _ptr(recompute),
        _ptr(l1_rel_out), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def fc_chunk_rel_l1_decide_noalloc(p: fc_l1_params, chunk_offsets: Sequence[int], X_t, X_tm1, step, f, recompute,
                                   l1_rel_out=None, stream=None) -> None:
    """fc_chunk_rel_l1_decide without a workspace: the library's static
    per-device scratch holds the slab partials (nothing is allocated)."""
    n = p.n_chunks
    _expect_chunk_state(p, chunk_offsets, (("X_t", X_t), ("X_tm1", X_tm1)),
                        (("step", step, n, torch.int32), ("f", f, n, torch.float32),
                         ("recompute", recompute, n, torch.uint8), ("l1_rel_out", l1_rel_out, n, torch.float32)))
    _check("fc_chunk_rel_l1_decide_noalloc", _lib.fc_chunk_rel_l1_decide_noalloc(
        ctypes.byref(p), _offsets(chunk_offsets), _ptr(X_t), _ptr(X_tm1), _ptr(step), _ptr(f), _ptr(recompute),
        _ptr(l1_rel_out), _stream(stream)))


def fc_cache_commit_workspace_bytes(c: fc_cache_params, L_q: int) -> int:
    return int(_lib.fc_cache_commit_workspace_bytes(ctypes.byref(c), int(L_q)))


def fc_cache_commit(c: fc_cache_params, L_clean: int, K_chunk, V_chunk, pos0: int, Q, K_cur, V_cur, pos_cur=None,
                    K_spare=None, V_spare=None, pos_spare=None, workspace=None, stream=None,
                    L_c: Optional[int] = None) -> Tuple[int, bool]:
    """One commit; returns (the new clean length, whether the clean tokens
    moved to the spare region).  The regions are [H][B_budget + B_active][d]
    (positions [H][B_budget + B_active]).  K_chunk = V_chunk = None commits
    the L_c rows that already sit behind the clean rows of the current
    region."""
    H, d, dt = c.H, c.d, _torch_dtype(c.dtype)
    Bt = c.B_budget + c.B_active
    if K_chunk is None or V_chunk is None:
        if K_chunk is not None or V_chunk is not None or L_c is None:
            raise FlowCacheError("fc_cache_commit", FC_ERR_INVALID_ARG)
        L_c = int(L_c)
    else:
        L_c = int(K_chunk.shape[1])
        _expect("K_chunk", K_chunk, (H, L_c, d), dt)
        _expect("V_chunk", V_chunk, (H, L_c, d), dt)
    for name, t in (("K_cur", K_cur), ("V_cur", V_cur), ("K_spare", K_spare), ("V_spare", V_spare)):
        _expect(name, t, (H, Bt, d), dt)
    _expect("pos_cur", pos_cur, (H, Bt), torch.int32)
    _expect("pos_spare", pos_spare, (H, Bt), torch.int32)
    if Q is not None:
        _expect("Q", Q, (H, Q.shape[1], d), dt)
    n = ctypes.c_int32(int(L_clean))
    sw = ctypes.c_int32(0)
    L_q = int(Q.shape[1]) if Q is not None else 0
    _check("fc_cache_commit", _lib.fc_cache_commit(
        ctypes.byref(c), ctypes.byref(n), _ptr(K_chunk), _ptr(V_chunk), L_c, int(pos0), _ptr(Q), L_q, _ptr(K_cur),
        _ptr(V_cur), _ptr(pos_cur), _ptr(K_spare), _ptr(V_spare), _ptr(pos_spare), ctypes.byref(sw), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))
    return int(n.value), bool(sw.value)


class KvCache:
    """A fixed-size KV cache on the device: two regions of the fixed buffer
    (K, V [H][B_budget + B_active][d], positions [H][B_budget + B_active])
    and the commit workspace, allocated once.  ``commit`` adds a completed
    chunk (its tokens take the next positions) and compresses when the budget
    overflows, from the current region into the other one.  ``K``, ``V`` and
    ``pos`` are views of the clean rows; ``active(L_c)`` gives the rows a
    producer may write a chunk into before ``commit(None, None, Q, L_c=L_c)``."""

    def __init__(self, H: int, d: int, B_budget: int, B_active: int, L_q: int, lam: float, pool_window: int,
                 dtype: torch.dtype, softmax_scale: float = 0.0, device="cuda"):
        self.p = fc_cache_params(int(H), int(d), int(B_budget), int(B_active), float(lam), int(pool_window),
                                 float(softmax_scale), FC_BF16 if dtype == torch.bfloat16 else FC_F32)
        nbytes = fc_cache_commit_workspace_bytes(self.p, L_q)
        if nbytes == 0:
            raise FlowCacheError("fc_cache_commit_workspace_bytes", FC_ERR_INVALID_ARG)
        Bt = B_budget + B_active
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self._K = [torch.zeros((H, Bt, d), dtype=dtype, device=device) for _ in range(2)]
        self._V = [torch.zeros((H, Bt, d), dtype=dtype, device=device) for _ in range(2)]
        self._pos = [torch.full((H, Bt), -1, dtype=torch.int32, device=device) for _ in range(2)]
        self.cur = 0           # region holding the clean tokens
        self.length = 0        # clean tokens per head
        self.next_pos = 0      # position of the next committed token

    @property
    def K(self):
        return self._K[self.cur][:, :self.length]

    @property
    def V(self):
        return self._V[self.cur][:, :self.length]

    @property
    def pos(self):
        return self._pos[self.cur][:, :self.length]

    def active(self, L_c: int):
        """Views (K, V) of the L_c rows behind the clean rows of the current region."""
        if not 1 <= L_c <= self.p.B_active:
            raise FlowCacheError("KvCache.active", FC_ERR_INVALID_ARG)
        return (self._K[self.cur][:, self.length:self.length + L_c],
                self._V[self.cur][:, self.length:self.length + L_c])

    def commit(self, K_chunk, V_chunk, Q=None, stream=None, L_c: Optional[int] = None) -> int:
        c, o = self.cur, 1 - self.cur
        self.length, swapped = fc_cache_commit(self.p, self.length, K_chunk, V_chunk, self.next_pos, Q, self._K[c],
                                               self._V[c], self._pos[c], self._K[o], self._V[o], self._pos[o],
                                               self.workspace, stream, L_c)
        if swapped:
            self.cur = o
        self.next_pos += int(K_chunk.shape[1]) if K_chunk is not None else int(L_c)
        return self.length


def fc_euler_step_l1_decide(p: fc_l1_params, chunk_offsets: Sequence[int], X_t, v, dt, X_next, step, f, recompute,
                            l1_rel_out=None, workspace=None, stream=None) -> None:
    n = p.n_chunks
    _expect_chunk_state(p, chunk_offsets, (("X_t", X_t), ("v", v), ("X_next", X_next)),
                        (("dt", dt, n, torch.float32), ("step", step, n, torch.int32), ("f", f, n, torch.float32),
                         ("recompute", recompute, n, torch.uint8), ("l1_rel_out", l1_rel_out, n, torch.float32)))
    workspace = _chunk_workspace(p, chunk_offsets, workspace, X_t.device)
    _check("fc_euler_step_l1_decide", _lib.fc_euler_step_l1_decide(
        ctypes.byref(p), _offsets(chunk_offsets), _ptr(X_t), _ptr(v), _ptr(dt), _ptr(X_next), _ptr(step), _ptr(f),
        _ptr(recompute), _ptr(l1_rel_out), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def fc_uniform_rel_l1_decide(p: fc_l1_params, chunk_offsets: Sequence[int], X_t, X_tm1, chunk_step, step, f,
                             recompute, l1_rel_out=None, workspace=None, stream=None) -> None:
    n = p.n_chunks
    _expect_chunk_state(p, chunk_offsets, (("X_t", X_t), ("X_tm1", X_tm1)),
                        (("chunk_step", chunk_step, n, torch.int32), ("step", step, 1, torch.int32),
                         ("f", f, 1, torch.float32), ("recompute", recompute, n, torch.uint8),
                         ("l1_rel_out", l1_rel_out, 1, torch.float32)))
    workspace = _chunk_workspace(p, chunk_offsets, workspace, X_t.device)
    _check("fc_uniform_rel_l1_decide", _lib.fc_uniform_rel_l1_decide(
        ctypes.byref(p), _offsets(chunk_offsets), _ptr(X_t), _ptr(X_tm1), _ptr(chunk_step), _ptr(step), _ptr(f),
        _ptr(recompute), _ptr(l1_rel_out), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def fc_history_rel_l1_decide(p: fc_l1_params, segment_offsets: Sequence[int], h_prev, h_cur, step, acc, refresh,
                             dev_out=None, workspace=None, stream=None) -> None:
    n = p.n_chunks
    _expect_chunk_state(p, segment_offsets, (("h_prev", h_prev), ("h_cur", h_cur)),
                        (("step", step, n, torch.int32), ("acc", acc, n, torch.float32),
                         ("refresh", refresh, n, torch.uint8), ("dev_out", dev_out, n, torch.float32)))
    workspace = _chunk_workspace(p, segment_offsets, workspace, h_prev.device)
    _check("fc_history_rel_l1_decide", _lib.fc_history_rel_l1_decide(
        ctypes.byref(p), _offsets(segment_offsets), _ptr(h_prev), _ptr(h_cur), _ptr(step), _ptr(acc), _ptr(refresh),
        _ptr(dev_out), _ptr(workspace), _nbytes(workspace), _stream(stream)))
