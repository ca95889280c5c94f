"""fp64 CPU oracle for the FlowCache per-step hot path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
reference that the GPU library is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it.  It shares no code with the HIP library and never imports it; its
inputs are the seeded synthetic tensors (converted exactly to float64), never
values produced by the GPU.

The method is the one described on the page "Flow Caching for Autoregressive
Video Generation" (papernotes.org ICLR 2026 digest), section 方法详解 /
关键设计 ("Key designs"):

* item 1 -- chunk relative L1 distance
  L1_rel(X, t, i) = ||X^i_{t-1} - X^i_t||_1 / ||X^i_t||_1;
* item 2 -- chunkwise adaptive caching: per-chunk accumulator f, forced
  recompute (f = 0) for the first m steps, then recompute and reset when
  f + L1_rel > eps, else accumulate and reuse;
* item 3 -- joint importance-redundancy KV compression:
  Imp = query-mean of the attention softmax over the clean keys, then a 1-D
  max-pool; Red_j = softmax_j((1/L_k) sum_i S_ij) with S the cosine similarity
  of l2-normalised keys and a zeroed diagonal;
  Score_j = lambda * Imp~_j - (1 - lambda) * Red_j; each head keeps its top-B
  tokens.  The flowchart under 整体框架 ("Overall framework") shows the same
  two parts and the "cache full -> score, keep top-B per head" step;
* the cache manager of item 3: a fixed buffer split into a compressed clean
  region of B_budget tokens and the denoising region; a completed chunk is
  merged into the clean tokens and, when they no longer fit, compressed back
  to B_budget.

Readings where the page leaves a step open:

* softmax temperature: the usual attention scale 1/sqrt(d) unless a scale is
  given;                                                    (parity unpinned)
* max-pool: window w (odd), stride 1, "same" padding that ignores positions
  outside [0, L_k), along the flattened token order, no renormalisation after
  the pool;                                                 (parity unpinned)
* redundancy mean: literally 1/L_k times the sum over all i with S_jj = 0;
* zero-norm keys: normalised with max(||k||, 1e-12), so they contribute 0;
* top-B ties: the lower token index wins; output indices ascending;
  B' = min(B, L_k) (L_k <= B keeps every token);
* V follows K: the same indices select both;
* forced steps count from each chunk's own first step; f = 0 during them;
  ">" recomputes and "<=" reuses; ||X_t||_1 = 0 gives L1_rel = +inf;
* cache "full": the clean tokens plus the completed chunk exceed B_budget;
  the merged order is clean tokens (as kept) then the chunk, and the pool
  runs along that order; the queries that score a compression are the
  caller's.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.orc_lse.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double, dp, dp, dp]
        lib.orc_importance.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double, dp, dp, dp]
        lib.orc_redundancy_bruteforce.argtypes = [ctypes.c_int] * 3 + [dp, dp]
        lib.orc_redundancy_closed.argtypes = [ctypes.c_int] * 3 + [dp, dp]
        lib.orc_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the C half uses (OpenMP default: all host cores)."""
    return int(_load().orc_num_threads())


def as_f64(x) -> np.ndarray:
    """Exact conversion of a float32/bfloat16 tensor or array to float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_scale(d: int) -> float:
    """Attention temperature 1/sqrt(d) (the page gives none; see header)."""
    return 1.0 / math.sqrt(d)


# ---------------------------------------------------------------------------
# KV compression (Key designs, item 3)
# ---------------------------------------------------------------------------

def lse(Q, K, scale: float) -> np.ndarray:
    """Per-query log-sum-exp of scale * q_i . k_j over the clean keys, [H][Lq]."""
    Q, K = as_f64(Q), as_f64(K)
    H, Lq, d = Q.shape
    Lk = K.shape[1]
    out = np.empty((H, Lq), np.float64)
    _load().orc_lse(H, Lq, Lk, d, float(scale), _ptr(Q), _ptr(K), _ptr(out))
    return out


def importance(Q, K, scale: float) -> np.ndarray:
    """Imp[h][j] = mean over queries of the row softmax of scale * Q K^T.

    The softmax runs over the clean keys only and is taken before the mean
    (Key designs item 3: attention softmax, then the average across queries).
    """
    Q, K = as_f64(Q), as_f64(K)
    H, Lq, d = Q.shape
    assert K.shape[0] == H and K.shape[2] == d
    Lk = K.shape[1]
    out = np.empty((H, Lk), np.float64)
    _load().orc_importance(H, Lq, Lk, d, float(scale), _ptr(Q), _ptr(K), _ptr(out))
    return out


def maxpool1d(x: np.ndarray, w: int) -> np.ndarray:
    """1-D max-pool along the last axis: window w (odd), stride 1, same size.

    out_j = max{ x_k : |k - j| <= (w-1)/2, 0 <= k < L }  (out-of-range
    positions are ignored).  Key designs item 3 names the max-pool; window,
    stride and padding are this oracle's reading.
    """
    assert w >= 1 and w % 2 == 1
    x = np.asarray(x, np.float64)
    out = x.copy()
    for s in range(1, (w - 1) // 2 + 1):
        out[..., s:] = np.maximum(out[..., s:], x[..., :-s])    # neighbour j - s
        out[..., :-s] = np.maximum(out[..., :-s], x[..., s:])   # neighbour j + s
    return out


def redundancy_mean(K, method: str = "closed") -> np.ndarray:
    """r[h][j] = (1/Lk) sum_i S_ij, S = cosine similarity, S_jj = 0.

    method="bruteforce" evaluates the definition (O(Lk^2 d));
    method="closed" uses sum_{i!=j} khat_i.khat_j = u.khat_j - khat_j.khat_j
    with u = sum_i khat_i (O(Lk d)).
    """
    K = as_f64(K)
    H, Lk, d = K.shape
    out = np.empty((H, Lk), np.float64)
    if method == "bruteforce":
        _load().orc_redundancy_bruteforce(H, Lk, d, _ptr(K), _ptr(out))
    elif method == "closed":
        _load().orc_redundancy_closed(H, Lk, d, _ptr(K), _ptr(out))
    else:
        raise ValueError(method)
    return out


def softmax_lastdim(x: np.ndarray) -> np.ndarray:
    """softmax over the token axis: e^{x_j - max x} / sum_k e^{x_k - max x}."""
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def redundancy(K, method: str = "closed") -> np.ndarray:
    """Red[h][j] = softmax_j(r[h][j])."""
    return softmax_lastdim(redundancy_mean(K, method))


def joint_score(imp_pooled: np.ndarray, red: np.ndarray, lam: float) -> np.ndarray:
    """Score = lambda * Imp~ - (1 - lambda) * Red."""
    return lam * np.asarray(imp_pooled, np.float64) - (1.0 - lam) * np.asarray(red, np.float64)


def select_topb(score: np.ndarray, B: int) -> np.ndarray:
    """Per head, the B' = min(B, L) tokens with the largest score.

    Order: j before k iff score_j > score_k, or they are equal and j < k.
    Returns int64 indices [H][B'] in ascending token order.
    """
    score = np.asarray(score, np.float64)
    H, L = score.shape
    Bp = min(int(B), L)
    out = np.empty((H, Bp), np.int64)
    idx = np.arange(L)
    for h in range(H):
        order = np.lexsort((idx, -score[h]))   # primary: score desc; secondary: index asc
        out[h] = np.sort(order[:Bp])
    return out


def gather_rows(X, idx: np.ndarray):
    """X_out[h][b] = X[h][idx[h][b]] (an exact copy of the rows)."""
    import torch
    if isinstance(X, torch.Tensor):
        ii = torch.as_tensor(idx, dtype=torch.int64)
        return torch.stack([X[h].index_select(0, ii[h]) for h in range(X.shape[0])])
    return np.stack([np.asarray(X)[h][idx[h]] for h in range(len(idx))])


def kv_compress(Q, K, V, B: int, lam: float, w: int, scale: Optional[float] = None,
                imp: Optional[np.ndarray] = None, r: Optional[np.ndarray] = None) -> Dict[str, object]:
    """Whole compression step for one set of heads, in the page's order.

    ``imp``/``r`` may be passed in (values this oracle computed earlier, e.g.
    reused across a lambda sweep); they are never GPU outputs.
    """
    d = K.shape[2]
    if scale is None:
        scale = default_scale(d)
    if imp is None:
        imp = importance(Q, K, scale)
    if r is None:
        r = redundancy_mean(K, "closed")
    imp_p = maxpool1d(imp, w)
    red = softmax_lastdim(r)
    score = joint_score(imp_p, red, lam)
    idx = select_topb(score, B)
    return {"imp": imp, "imp_pooled": imp_p, "r": r, "red": red, "score": score,
            "idx": idx, "K_out": gather_rows(K, idx), "V_out": gather_rows(V, idx)}


# ---------------------------------------------------------------------------
# Chunkwise relative L1 and reuse decision (Key designs, items 1 and 2)
# ---------------------------------------------------------------------------

def chunk_l1_sums(x_t, x_tm1, offsets: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Per chunk i: A_i = sum |X_{t-1} - X_t| and N_i = sum |X_t| in fp64."""
    n = len(offsets) - 1
    A = np.zeros(n)
    N = np.zeros(n)
    for i in range(n):
        a = as_f64(x_t[offsets[i]:offsets[i + 1]])
        b = as_f64(x_tm1[offsets[i]:offsets[i + 1]])
        A[i] = np.abs(b - a).sum()
        N[i] = np.abs(a).sum()
    return A, N


def chunk_l1_rel(x_t, x_tm1, offsets: Sequence[int]) -> np.ndarray:
    """L1_rel_i = ||X^i_{t-1} - X^i_t||_1 / ||X^i_t||_1 (+inf when ||X^i_t||_1 = 0)."""
    A, N = chunk_l1_sums(x_t, x_tm1, offsets)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(N > 0, A / np.where(N > 0, N, 1.0), np.inf)
    return out


def decide(n: int, f: float, l1_rel: float, m: int, eps: float) -> Tuple[bool, float]:
    """One chunk's decision at its local step n (0-based).

    n < m: forced recompute, f = 0.  Otherwise a = f + L1_rel; a > eps:
    recompute and f = 0; else reuse and f = a.  Returns (recompute, new f).
    """
    if n < m:
        return True, 0.0
    a = f + l1_rel
    if a > eps:
        return True, 0.0
    return False, a


# ---------------------------------------------------------------------------
# KV cache manager (flowchart under 整体框架; Key designs, item 3)
# ---------------------------------------------------------------------------

def cache_merge(K_clean, V_clean, pos_clean: np.ndarray, K_chunk, V_chunk, pos0: int):
    """A completed chunk enters the cache: per head, the clean tokens (oldest
    first, as kept) followed by the chunk's tokens, whose positions are
    pos0, pos0 + 1, ...  K and V are torch CPU tensors [H][L][d] (their values
    are kept exactly); positions int64 [H][L]."""
    import torch
    H, Lc = K_chunk.shape[0], K_chunk.shape[1]
    K = torch.cat([K_clean, K_chunk], dim=1)
    V = torch.cat([V_clean, V_chunk], dim=1)
    new_pos = np.broadcast_to(pos0 + np.arange(Lc, dtype=np.int64), (H, Lc))
    pos = np.concatenate([np.asarray(pos_clean, np.int64).reshape(H, -1), new_pos], axis=1)
    return K, V, pos


def cache_commit(K_clean, V_clean, pos_clean, K_chunk, V_chunk, pos0: int, Q, B_budget: int, lam: float, w: int,
                 scale: Optional[float] = None) -> Dict[str, object]:
    """One commit of a completed chunk into the clean region of B_budget
    tokens per head.

    The flowchart's branch: when the merged tokens fit the budget the cache is
    not full and every token is kept as is; otherwise the merged set is
    scored with the queries Q and each head keeps its top-B_budget tokens
    (kv_compress), in ascending merged order, so the cache stays in temporal
    order.  Returns the new K, V, positions, and, after a compression, the
    compression's intermediate values ("comp", merged indices in comp["idx"])
    and the merged set ("merged": K, V, pos).
    """
    Km, Vm, pm = cache_merge(K_clean, V_clean, pos_clean, K_chunk, V_chunk, pos0)
    if Km.shape[1] <= B_budget:
        return {"K": Km, "V": Vm, "pos": pm, "comp": None, "merged": (Km, Vm, pm)}
    comp = kv_compress(Q, Km, Vm, B_budget, lam, w, scale)
    idx = comp["idx"]
    pos = np.stack([pm[h][idx[h]] for h in range(pm.shape[0])])
    return {"K": comp["K_out"], "V": comp["V_out"], "pos": pos, "comp": comp, "merged": (Km, Vm, pm)}


# ---------------------------------------------------------------------------
# The sampler's Euler step with the decision fused (Key designs, item 1: the
# L1 numerator is ||v dt||_1, the update itself)
# ---------------------------------------------------------------------------

def euler_step(x_t, v, offsets: Sequence[int], dt: Sequence[float], active: Sequence[bool]):
    """X_{t-1} = X_t + v * dt_i over each active chunk i; inactive chunks keep
    X_t's values.  The stored state is a rounded value, so this follows the
    kernel's precision: the product and the sum each rounded to float32 (no
    fused multiply-add), then the result rounded to the storage type of x_t
    (bf16: to nearest, ties to even).  x_t, v: torch CPU tensors, flat."""
    import torch
    x32 = x_t.to(torch.float32).numpy()
    v32 = v.to(torch.float32).numpy()
    y = x32.copy()
    for i in range(len(offsets) - 1):
        if not active[i]:
            continue
        s, e = offsets[i], offsets[i + 1]
        p = v32[s:e] * np.float32(dt[i])          # float32 product, rounded
        y[s:e] = x32[s:e] + p                     # float32 sum, rounded
    out = torch.from_numpy(y)
    return out.to(x_t.dtype)


# ---------------------------------------------------------------------------
# Other decision policies over the same relative L1
# ---------------------------------------------------------------------------

def uniform_l1_rel(x_t, x_tm1, offsets: Sequence[int], active: Sequence[bool]) -> float:
    """One relative L1 over every active chunk: the sum of the chunks'
    ||X_{t-1} - X_t||_1 over the sum of their ||X_t||_1 (+inf when that sum
    is 0).  The uniform policy the FlowCache page contrasts with
    (背景与动机: one decision for all content at a timestep)."""
    A, N = chunk_l1_sums(x_t, x_tm1, offsets)
    a = float(sum(A[i] for i in range(len(A)) if active[i]))
    n = float(sum(N[i] for i in range(len(N)) if active[i]))
    return a / n if n > 0 else math.inf


def decide_history(n: int, acc: float, dev: float, m: int, delta: float) -> Tuple[bool, float]:
    """ARCache's History-Guided Cache ("Accelerating Autoregressive Video
    Diffusion via History-Guided Cache and Residual Correction", papernotes
    digest, Key designs item 1): the cache is reused while the deviations
    summed from the last refresh step t_ref, that step included, through the
    current one stay <= delta; otherwise it refreshes and t_ref becomes the
    current step.  acc holds the sum through the previous step; returns
    (refresh, the sum through this step from the new t_ref).  The first m
    steps refresh."""
    if n < m:
        return True, dev
    a = acc + dev
    if a > delta:
        return True, dev
    return False, a
