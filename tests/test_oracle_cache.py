"""Pins for the KV cache manager of the fp64 oracle (CPU only).

The cache of Key designs item 3 ("Flow Caching for Autoregressive Video
Generation", papernotes digest; flowchart under 整体框架): a completed chunk
joins the clean tokens; when they no longer fit the budget B, every head
keeps its top-B tokens by the joint score.  The pins are closed forms that do
not go through the oracle's own arithmetic:

* not full: the cache is the plain concatenation of the chunks;
* lambda = 1 with zero queries: importance is uniform, every score ties, and
  the lower merged index wins, so the cache always holds the B oldest tokens;
* lambda = 0 with keys that are unit vectors of a few groups: the redundancy
  of a token grows with the size of its group (r_j = (count_j - 1)/L), so a
  head keeps the tokens of the smallest groups first, ties to the lower
  merged index -- a counting model with no floating point at all.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_fc_amd import synth


def _empty(H, d, dtype=torch.float64):
    return torch.zeros((H, 0, d), dtype=dtype), torch.zeros((H, 0, d), dtype=dtype), np.zeros((H, 0), np.int64)


def _run(K_all, V_all, Q_all, T, B, lam, w, n_chunks):
    """Commit chunks 0..n_chunks-1 through the oracle; yields each state."""
    H, _, d = K_all.shape
    K, V, pos = _empty(H, d, K_all.dtype)
    for c in range(n_chunks):
        sl = slice(c * T, (c + 1) * T)
        st = oracle.cache_commit(K, V, pos, K_all[:, sl], V_all[:, sl], c * T,
                                 None if Q_all is None else Q_all[c], B, lam, w)
        K, V, pos = st["K"], st["V"], st["pos"]
        yield c, st


def test_not_full_is_concatenation():
    rng = np.random.default_rng(0)
    H, d, T, n = 2, 8, 5, 4
    K_all = torch.from_numpy(rng.standard_normal((H, n * T, d)))
    V_all = torch.from_numpy(rng.standard_normal((H, n * T, d)))
    for c, st in _run(K_all, V_all, None, T, n * T, 0.5, 3, n):
        L = (c + 1) * T
        assert st["comp"] is None
        assert torch.equal(st["K"], K_all[:, :L]) and torch.equal(st["V"], V_all[:, :L])
        assert (st["pos"] == np.arange(L)).all()


@pytest.mark.parametrize("T,B", [(7, 10), (6, 18), (9, 4)])
def test_uniform_importance_keeps_the_oldest(T, B):
    rng = np.random.default_rng(1)
    H, d, n, Lq = 2, 16, 6, 5
    K_all = torch.from_numpy(rng.standard_normal((H, n * T, d)))
    V_all = torch.from_numpy(rng.standard_normal((H, n * T, d)))
    Q_all = torch.zeros((n, H, Lq, d), dtype=torch.float64)
    for c, st in _run(K_all, V_all, Q_all, T, B, 1.0, 3, n):
        L = min(B, (c + 1) * T)
        assert (st["pos"] == np.arange(L)).all(), f"commit {c}: {st['pos']}"
        assert torch.equal(st["K"], K_all[:, :L])


def _count_model(groups_h, T, B, n_chunks):
    """Kept positions after each commit for lambda = 0 and group keys: order
    the merged tokens by (size of their group among the merged tokens, merged
    index) and keep the first B, in merged order."""
    kept = []  # positions, in merged (= temporal) order
    out = []
    for c in range(n_chunks):
        merged = kept + list(range(c * T, (c + 1) * T))
        if len(merged) > B:
            g = [groups_h[p] for p in merged]
            count = {x: g.count(x) for x in set(g)}
            order = sorted(range(len(merged)), key=lambda i: (count[g[i]], i))
            merged = [merged[i] for i in sorted(order[:B])]
        kept = merged
        out.append(list(kept))
    return out


@pytest.mark.parametrize("T,B,scale,spread", [(10, 24, 1.0, 3), (12, 20, 3.0, 2), (8, 30, 0.5, 4)])
def test_group_keys_follow_the_count_model(T, B, scale, spread):
    H, d, n, Lq = 2, 16, 8, 4
    groups = synth.group_labels(H, n, T, seed=T + B, spread=spread)
    K_all = synth.group_keys(groups, d, "f32", scale).double()
    V_all = torch.from_numpy(np.random.default_rng(3).standard_normal((H, n * T, d)))
    Q_all = torch.from_numpy(np.random.default_rng(4).standard_normal((n, H, Lq, d)))
    want = [_count_model(groups[h].tolist(), T, B, n) for h in range(H)]
    n_comp = 0
    for c, st in _run(K_all, V_all, Q_all, T, B, 0.0, 5, n):
        n_comp += st["comp"] is not None
        for h in range(H):
            assert st["pos"][h].tolist() == want[h][c], f"head {h}, commit {c}"
            assert torch.equal(st["V"][h], V_all[h][st["pos"][h]])
    assert n_comp >= n - 3


def test_field_run_invariants():
    cfg = synth.CACHE_CONFIGS["tiny"]
    Q_all, K_all, V_all = synth.cache_inputs(cfg, seed=0)
    T, B = cfg.tokens_per_chunk, cfg.B_budget
    n_comp = 0
    prev = set()
    for c, st in _run(K_all, V_all, Q_all, T, B, cfg.lam, cfg.w, cfg.n_chunks):
        L = min(B, (c + 1) * T)
        assert st["pos"].shape == (cfg.H, L)
        for h in range(cfg.H):
            p = st["pos"][h]
            assert np.all(np.diff(p) > 0), "positions stay in temporal order"
            assert p[0] >= 0 and p[-1] < (c + 1) * T
            assert torch.equal(st["K"][h], K_all[h][p]) and torch.equal(st["V"][h], V_all[h][p])
        # kept tokens are a subset of the previous cache plus the new chunk
        now = {(h, int(x)) for h in range(cfg.H) for x in st["pos"][h]}
        new = {(h, x) for h in range(cfg.H) for x in range(c * T, (c + 1) * T)}
        assert now <= prev | new
        prev = now
        if st["comp"] is not None:
            n_comp += 1
            # the compression saw exactly the merged tokens: clean first, then the chunk
            Km, _, pm = st["merged"]
            assert Km.shape[1] == (L if c == 0 else min(B, c * T) + T)
            assert (pm[:, -T:] == np.arange(c * T, (c + 1) * T)).all()
    assert n_comp == cfg.n_chunks - 1  # 96 tokens fit the budget of 160; every later commit overflows it
