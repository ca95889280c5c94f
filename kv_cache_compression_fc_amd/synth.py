"""Seeded synthetic inputs for the FlowCache hot path.

This module only draws numbers: it holds none of the method's arithmetic, and
both the GPU tests and the oracle take their inputs from it.  The real
workloads (MAGI-1 and SkyReels-V2 activations on VBench prompts) need trained
weights, so these generators stand in with the same shapes:

* queries and values ~ N(0, 1);
* keys are either clustered around a few base vectors (tiny case) or a smooth
  random field over the (frame, y, x) token grid -- Gaussian-blurred N(0, 1)
  noise, standardised per (head, channel), plus white noise -- so that
  neighbouring tokens are near-duplicates, as in real video latents;
* chunk states follow a straight flow-matching path
  X_t = X_N - v * (1 - sigma(t)),  sigma(t) = (t/N)^p,  v = s_i * N(0, 1),
  s_i ~ U(0.5, 2) per chunk, then rounded once to the storage dtype.

Token order is (frame, y, x) with x fastest, older chunks first.  bf16 values
are produced by rounding float32 once, to nearest-even (torch CPU cast); the
oracle receives exactly those values.

Every stream comes from ``numpy.random.SeedSequence(seed).spawn`` in a fixed
order, with one child per head, so any subset of heads is reproducible on its
own.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch


def _to_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# KV-compression workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class KVConfig:
    name: str
    H: int
    d: int
    Lq: int
    Lk: int
    B: int
    lam: Tuple[float, ...]
    w: int
    dtype: str                     # "f32" or "bf16"
    key_kind: str                  # "clustered" or "field"
    frames: int = 0                # clean-key volume, field keys only
    ny: int = 0
    nx: int = 0
    sigma: float = 0.0
    noise: float = 0.1
    dup: Optional[Tuple[Tuple[int, int], Tuple[int, int]]] = None  # ((src0, src1), (dst0, dst1)) frame ranges
    n_base: int = 32               # clustered keys only
    base_repeat: int = 8
    base_noise: float = 0.05


KV_CONFIGS = {
    # Tiny: H=2, d=64, Lq=64, Lk=256, B=64, lambda=0.5, window 5, fp32,
    # K = base[j // 8] + 0.05 N(0,1) with 32 base vectors.
    "tiny": KVConfig("tiny", H=2, d=64, Lq=64, Lk=256, B=64, lam=(0.5,), w=5, dtype="f32",
                     key_kind="clustered"),
    # MAGI-1-like: 24 heads, d=128, active chunk 4 x 30 x 30 = 3600 queries,
    # 20 clean latent frames of 30 x 30 = 18000 keys, B = 7200, window 7.
    "magi": KVConfig("magi", H=24, d=128, Lq=3600, Lk=18000, B=7200, lam=(0.5,), w=7, dtype="bf16",
                     key_kind="field", frames=20, ny=30, nx=30, sigma=3.0),
    # SkyReels-V2-like: 40 heads, 52 x 30 tokens per frame, chunk of 5 frames
    # (7800 queries), 30 clean frames (46800 keys), B = 15600.
    "skyreels": KVConfig("skyreels", H=40, d=128, Lq=7800, Lk=46800, B=15600, lam=(0.5,), w=7,
                         dtype="bf16", key_kind="field", frames=30, ny=52, nx=30, sigma=4.0),
    # Long video: 45 x 45 tokens per frame, 4-frame chunks (8100 queries),
    # 16 clean chunks = 64 frames (129600 keys), B = 32400, lambda sweep;
    # clean chunks 12-15 (frames 48-63) are exact copies of chunks 4-7
    # (frames 16-31), keys and values, to create exact duplicates.
    "long": KVConfig("long", H=24, d=128, Lq=8100, Lk=129600, B=32400, lam=(0.3, 0.5, 0.7), w=7,
                     dtype="bf16", key_kind="field", frames=64, ny=45, nx=45, sigma=3.0,
                     dup=((16, 32), (48, 64))),
}


def _head_streams(seed: int, H: int):
    """Independent generators per (tensor, head), fixed spawn order."""
    q_ss, kf_ss, kn_ss, v_ss = np.random.SeedSequence(seed).spawn(4)
    return (q_ss.spawn(H), kf_ss.spawn(H), kn_ss.spawn(H), v_ss.spawn(H))


def _field_keys(cfg: KVConfig, rng_field: np.random.Generator, rng_noise: np.random.Generator) -> np.ndarray:
    """One head of smooth-field keys, float32 [Lk][d]."""
    from scipy.ndimage import gaussian_filter
    vol = rng_field.standard_normal((cfg.d, cfg.frames, cfg.ny, cfg.nx), dtype=np.float32)
    vol = gaussian_filter(vol, sigma=(0.0, cfg.sigma, cfg.sigma, cfg.sigma), mode="reflect", truncate=4.0)
    flat = vol.reshape(cfg.d, -1)
    flat = (flat - flat.mean(axis=1, keepdims=True)) / flat.std(axis=1, keepdims=True)
    k = flat.T + cfg.noise * rng_noise.standard_normal((cfg.Lk, cfg.d), dtype=np.float32)
    return np.ascontiguousarray(k, dtype=np.float32)


def _apply_dup(cfg: KVConfig, x: np.ndarray) -> None:
    if cfg.dup is None:
        return
    (s0, s1), (d0, d1) = cfg.dup
    tpf = cfg.ny * cfg.nx
    x[d0 * tpf:d1 * tpf] = x[s0 * tpf:s1 * tpf]


def _kv_head(cfg: KVConfig, seed: int, h: int):
    """Head h's (Q, K, V), float32, from its own streams."""
    qs, kfs, kns, vs = _head_streams(seed, cfg.H)
    Q = np.random.default_rng(qs[h]).standard_normal((cfg.Lq, cfg.d), dtype=np.float32)
    V = np.random.default_rng(vs[h]).standard_normal((cfg.Lk, cfg.d), dtype=np.float32)
    rf, rn = np.random.default_rng(kfs[h]), np.random.default_rng(kns[h])
    if cfg.key_kind == "clustered":
        base = rf.standard_normal((cfg.n_base, cfg.d), dtype=np.float32)
        K = base[np.arange(cfg.Lk) // cfg.base_repeat] + \
            cfg.base_noise * rn.standard_normal((cfg.Lk, cfg.d), dtype=np.float32)
    elif cfg.key_kind == "field":
        K = _field_keys(cfg, rf, rn)
    else:
        raise ValueError(cfg.key_kind)
    _apply_dup(cfg, K)
    _apply_dup(cfg, V)
    return Q, K, V


def kv_inputs(cfg: KVConfig, seed: int = 0, heads: Optional[Sequence[int]] = None, workers: int = 1):
    """(Q, K, V) as CPU tensors in the config's storage dtype, head-major
    [H'][L][d], for the given heads (default: all).  With workers > 1 the
    heads are drawn on that many threads (the random draws and the filter
    release the GIL); every head has its own streams, so the values do not
    depend on the worker count."""
    if heads is None:
        heads = range(cfg.H)
    heads = list(heads)
    n_h = len(heads)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    Q = torch.empty((n_h, cfg.Lq, cfg.d), dtype=dt)
    K = torch.empty((n_h, cfg.Lk, cfg.d), dtype=dt)
    V = torch.empty((n_h, cfg.Lk, cfg.d), dtype=dt)

    def one(n):
        for dst, x in zip((Q, K, V), _kv_head(cfg, seed, heads[n])):
            dst[n] = _to_storage(x, cfg.dtype)

    if workers > 1 and n_h > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(workers, n_h)) as ex:
            list(ex.map(one, range(n_h)))
    else:
        for n in range(n_h):
            one(n)
    return Q, K, V


def random_kv(H: int, Lq: int, Lk: int, d: int, dtype: str, seed: int):
    """Plain N(0,1) Q, K, V of any shape (edge-case and tiling tests)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    Q = rng.standard_normal((H, Lq, d), dtype=np.float32)
    K = rng.standard_normal((H, Lk, d), dtype=np.float32)
    V = rng.standard_normal((H, Lk, d), dtype=np.float32)
    return _to_storage(Q, dtype), _to_storage(K, dtype), _to_storage(V, dtype)


def random_scores(H: int, L: int, seed: int, n_levels: int = 0) -> torch.Tensor:
    """float32 scores [H][L]; with n_levels > 0 they take only that many
    distinct values, so many exact ties occur."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    if n_levels > 0:
        levels = rng.standard_normal(n_levels).astype(np.float32) * np.float32(1e-4)
        s = levels[rng.integers(0, n_levels, size=(H, L))]
    else:
        s = rng.standard_normal((H, L), dtype=np.float32) * np.float32(1e-4)
    return torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32))


# ---------------------------------------------------------------------------
# Chunk-state trajectories
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class ChunkConfig:
    name: str
    n_chunks: int
    chunk_elems: int
    N: int                 # denoising steps per chunk
    m: int
    eps: Tuple[float, ...]
    dtype: str
    start_stride: int      # chunk i starts at global step i * start_stride
    p: float = 2.0         # power-law schedule sigma(t) = (t/N)^p


CHUNK_CONFIGS = {
    # 4 chunks x 256 fp32, 10 steps, all aligned, m=2, eps=0.01.
    "tiny": ChunkConfig("tiny", 4, 256, 10, 2, (0.01,), "f32", 0),
    # 16 chunks, each a [64][8][90][160] bf16 latent (7,372,800 elements),
    # 50 steps, chunk i offset by i steps, m=5, eps in {0.01, 0.015}.
    "scale": ChunkConfig("scale", 16, 64 * 8 * 90 * 160, 50, 5, (0.01, 0.015), "bf16", 1),
}


class ChunkTrajectory:
    """X^i_t = X^i_N - v_i (1 - sigma(t)) for every chunk i, float32 math,
    rounded to the storage dtype on output."""

    def __init__(self, cfg: ChunkConfig, seed: int = 0):
        self.cfg = cfg
        x_ss, s_ss, v_ss = np.random.SeedSequence(seed).spawn(3)
        n, e = cfg.n_chunks, cfg.chunk_elems
        self.x_noise = np.empty((n, e), np.float32)
        self.v = np.empty((n, e), np.float32)
        scales = np.random.default_rng(s_ss).uniform(0.5, 2.0, size=n).astype(np.float32)
        xs, vs = x_ss.spawn(n), v_ss.spawn(n)
        for i in range(n):
            self.x_noise[i] = np.random.default_rng(xs[i]).standard_normal(e, dtype=np.float32)
            self.v[i] = scales[i] * np.random.default_rng(vs[i]).standard_normal(e, dtype=np.float32)
        self.scales = scales
        self.offsets = [i * e for i in range(n + 1)]

    def sigma(self, t: int) -> float:
        return (t / self.cfg.N) ** self.cfg.p

    def state_f32(self, i: int, t: int) -> np.ndarray:
        c = np.float32(1.0 - self.sigma(t))
        return self.x_noise[i] - self.v[i] * c

    def state(self, i: int, t: int) -> torch.Tensor:
        return _to_storage(self.state_f32(i, t), self.cfg.dtype)

    def velocity(self) -> torch.Tensor:
        """The path's velocity, flat over the chunks, in the storage dtype:
        X_{t-1} - X_t = v (sigma(t-1) - sigma(t))."""
        return _to_storage(self.v.reshape(-1), self.cfg.dtype)

    def step_size(self, n: int) -> float:
        """sigma(t-1) - sigma(t) at local step n (t = N - n): the Euler step."""
        t = self.cfg.N - n
        return self.sigma(t - 1) - self.sigma(t)

    def noise_states(self) -> torch.Tensor:
        """X_N of every chunk, flat, in the storage dtype."""
        return _to_storage(self.x_noise.reshape(-1), self.cfg.dtype)

    def n_global_steps(self) -> int:
        return self.cfg.N + (self.cfg.n_chunks - 1) * self.cfg.start_stride

    def local_step(self, i: int, g: int) -> int:
        """Chunk i's local step at global step g (-1 when not denoising)."""
        n = g - i * self.cfg.start_stride
        return n if 0 <= n < self.cfg.N else -1

    def pair(self, g: int) -> Tuple[torch.Tensor, torch.Tensor, List[int]]:
        """(X_t, X_{t-1}, local steps) at global step g, all chunks concatenated;
        inactive chunks hold zeros."""
        cfg = self.cfg
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        xt = torch.zeros(cfg.n_chunks * cfg.chunk_elems, dtype=dt)
        xtm1 = torch.zeros_like(xt)
        steps = []
        for i in range(cfg.n_chunks):
            n = self.local_step(i, g)
            steps.append(n)
            if n < 0:
                continue
            t = cfg.N - n
            s, e = self.offsets[i], self.offsets[i + 1]
            xt[s:e] = self.state(i, t)
            xtm1[s:e] = self.state(i, t - 1)
        return xt, xtm1, steps


# ---------------------------------------------------------------------------
# Multi-chunk runs of the KV cache (a chunk completes, its keys join the cache)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class CacheConfig:
    name: str
    H: int
    d: int
    n_chunks: int          # chunks committed, oldest first
    fpc: int               # latent frames per chunk
    ny: int
    nx: int
    B_budget: int          # clean tokens each head keeps
    B_active: int          # tokens of one chunk (the denoising region)
    Lq: int                # queries that score each compression
    lam: float
    w: int
    dtype: str
    sigma: float = 3.0
    noise: float = 0.1

    @property
    def tokens_per_chunk(self) -> int:
        return self.fpc * self.ny * self.nx


CACHE_CONFIGS = {
    # Small: 2 heads, d=64, chunks of 2 frames x 8 x 6 = 96 tokens, a budget of
    # 160 tokens (the cache overflows from the second chunk on), fp32.
    "tiny": CacheConfig("tiny", H=2, d=64, n_chunks=6, fpc=2, ny=8, nx=6, B_budget=160, B_active=96, Lq=96,
                        lam=0.5, w=5, dtype="f32"),
    # MAGI-1-like run: 24 heads, d=128, chunks of 4 latent frames of 30 x 30
    # (3600 tokens), a budget of two chunks (7200), the active chunk's 3600
    # queries, ten chunks.  Every commit from the third on merges 10800 tokens
    # and keeps 7200.
    "magi": CacheConfig("magi", H=24, d=128, n_chunks=10, fpc=4, ny=30, nx=30, B_budget=7200, B_active=3600,
                        Lq=3600, lam=0.5, w=7, dtype="bf16"),
    # Long-video-like run: 24 heads, chunks of 4 latent frames of 45 x 45
    # (8100 tokens), a budget of four chunks (32400), an active region of
    # 9000 rows (above the chunk, so the cache's head stride exceeds every
    # merged length), 8100 queries, six chunks: commits five and six merge
    # 40500 tokens and keep 32400.
    "long": CacheConfig("long", H=24, d=128, n_chunks=6, fpc=4, ny=45, nx=45, B_budget=32400, B_active=9000,
                        Lq=8100, lam=0.5, w=7, dtype="bf16"),
}


def cache_inputs(cfg: CacheConfig, seed: int = 0, heads: Optional[Sequence[int]] = None):
    """Keys and values of every chunk of the run and the queries of every
    commit, as CPU tensors in the storage dtype:
      K, V  [H'][n_chunks * T][d]   (chunk c = rows [c T, (c+1) T), T tokens per chunk)
      Q     [n_chunks][H'][Lq][d]   (the queries that score commit c)
    Keys are one smooth random field over the whole video, so neighbouring
    chunks are correlated as consecutive frames are."""
    T = cfg.tokens_per_chunk
    frames = cfg.n_chunks * cfg.fpc
    kcfg = KVConfig(cfg.name, H=cfg.H, d=cfg.d, Lq=cfg.Lq, Lk=cfg.n_chunks * T, B=cfg.B_budget, lam=(cfg.lam,),
                    w=cfg.w, dtype=cfg.dtype, key_kind="field", frames=frames, ny=cfg.ny, nx=cfg.nx,
                    sigma=cfg.sigma, noise=cfg.noise)
    _, K, V = kv_inputs(kcfg, seed, heads)
    if heads is None:
        heads = range(cfg.H)
    heads = list(heads)
    q_ss = np.random.SeedSequence([seed, 1]).spawn(cfg.n_chunks)
    Q = np.empty((cfg.n_chunks, len(heads), cfg.Lq, cfg.d), np.float32)
    for c in range(cfg.n_chunks):
        per_head = q_ss[c].spawn(cfg.H)
        for n, h in enumerate(heads):
            Q[c, n] = np.random.default_rng(per_head[h]).standard_normal((cfg.Lq, cfg.d), dtype=np.float32)
    return _to_storage(Q, cfg.dtype), K, V


def group_labels(H: int, n_chunks: int, T: int, seed: int, spread: int = 3) -> np.ndarray:
    """int64 [H][n_chunks * T]: each token of chunk c draws its group from
    {c, c-1, ..., c-spread+1} (clipped at 0), so groups have varied sizes and
    later chunks repeat earlier ones."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 2]))
    g = np.empty((H, n_chunks * T), np.int64)
    for c in range(n_chunks):
        lo = max(0, c - spread + 1)
        g[:, c * T:(c + 1) * T] = rng.integers(lo, c + 1, size=(H, T))
    return g


def group_keys(groups: np.ndarray, d: int, dtype: str, scale: float = 1.0) -> torch.Tensor:
    """Keys [H][L][d] with k[h][j] = scale * e_{groups[h][j]} (unit vectors):
    keys of one group are exact duplicates, keys of different groups are
    orthogonal."""
    H, L = groups.shape
    assert int(groups.max()) < d
    K = np.zeros((H, L, d), np.float32)
    K[np.arange(H)[:, None], np.arange(L)[None, :], groups] = scale
    return _to_storage(K, dtype)
