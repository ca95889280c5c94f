"""GPU parity of the KV cache manager (fc_cache_commit) against the fp64
oracle's cache_commit, run in lockstep over multi-chunk synthetic runs.

After every commit the GPU cache's length, positions and rows are compared
with the oracle's.  Where a compression keeps a different set, every token
that differs must lie in the tie band of the oracle's score (parity.py); the
oracle then adopts the GPU's set (both are correct results) and the run goes
on from the same state on both sides.  Kept rows must be bit-exact copies of
the merged rows at their positions.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
from kv_cache_compression_fc_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def fc():
    from kv_cache_compression_fc_amd import binding
    return binding


def say(msg):
    print(msg, flush=True)


class Lockstep:
    """Oracle state of the sampled heads, advanced beside the GPU cache."""

    def __init__(self, heads, d, dtype):
        H = len(heads)
        self.heads = list(heads)
        self.K = torch.zeros((H, 0, d), dtype=dtype)
        self.V = torch.zeros((H, 0, d), dtype=dtype)
        self.pos = np.zeros((H, 0), np.int64)
        self.n_band = self.n_diff = self.n_comp = 0

    def step(self, cache, K_chunk, V_chunk, pos0, Q, B, lam, w, scale=None):
        """K_chunk, V_chunk, Q: host tensors of the sampled heads."""
        st = oracle.cache_commit(self.K, self.V, self.pos, K_chunk, V_chunk, pos0, Q, B, lam, w, scale)
        L = st["pos"].shape[1]
        assert cache.length == L, f"GPU length {cache.length}, oracle {L}"
        hs = self.heads
        gpos = cache.pos[hs, :L].cpu().numpy().astype(np.int64)
        gK = cache.K[hs, :L].cpu()
        gV = cache.V[hs, :L].cpu()
        if st["comp"] is None:
            assert (gpos == st["pos"]).all(), "positions differ without a compression"
        else:
            self.n_comp += 1
            Km, Vm, pm = st["merged"]
            gidx = np.stack([np.searchsorted(pm[n], gpos[n]) for n in range(len(hs))])
            assert (gidx < pm.shape[1]).all() and (np.take_along_axis(pm, gidx, 1) == gpos).all(), \
                "GPU kept a position that is not in the merged set"
            nb, nd = parity.check_selection(torch.from_numpy(gidx.astype(np.int32)), st["comp"]["score"], B)
            self.n_band += nb
            self.n_diff += nd
            # adopt the GPU's set (identical unless inside the tie band)
            st["K"] = torch.stack([Km[n].index_select(0, torch.from_numpy(gidx[n])) for n in range(len(hs))])
            st["V"] = torch.stack([Vm[n].index_select(0, torch.from_numpy(gidx[n])) for n in range(len(hs))])
            st["pos"] = gpos
        assert torch.equal(gK, st["K"]), "kept K rows differ from the merged rows at their positions"
        assert torch.equal(gV, st["V"]), "kept V rows differ from the merged rows at their positions"
        self.K, self.V, self.pos = st["K"], st["V"], st["pos"]


def run_config(fc, cfg, Q_all, K_all, V_all, heads=None, sizes=None, label="", in_place=False):
    """Commit the run's chunks (sizes: tokens per commit, default whole
    chunks) into a KvCache and the oracle side by side.  Q_all, K_all, V_all
    are device tensors with every head; the oracle reads the sampled heads.
    in_place: each chunk is written into the cache's active rows first and
    committed where it lies (else the commit copies it in)."""
    dt = K_all.dtype
    H = K_all.shape[0]
    heads = list(range(H)) if heads is None else list(heads)
    T = cfg.tokens_per_chunk
    if sizes is None:
        sizes = [T] * cfg.n_chunks
    cache = fc.KvCache(H, cfg.d, cfg.B_budget, cfg.B_active, cfg.Lq, cfg.lam, cfg.w, dt)
    ls = Lockstep(heads, cfg.d, dt)
    hK, hV = K_all[heads].cpu(), V_all[heads].cpu()
    p0 = 0
    for c, n in enumerate(sizes):
        say(f"  {label} commit {c}: {n} tokens at position {p0}, clean {cache.length}")
        Kc = K_all[:, p0:p0 + n].contiguous()
        Vc = V_all[:, p0:p0 + n].contiguous()
        Q = Q_all[c % Q_all.shape[0]]
        if in_place:
            Ka, Va = cache.active(n)
            Ka.copy_(Kc)
            Va.copy_(Vc)
            cache.commit(None, None, Q, L_c=n)
        else:
            cache.commit(Kc, Vc, Q)
        torch.cuda.synchronize()
        ls.step(cache, hK[:, p0:p0 + n], hV[:, p0:p0 + n], p0, Q[heads].cpu(), cfg.B_budget, cfg.lam, cfg.w)
        p0 += n
    say(f"  {label}: {ls.n_comp} compressions, band population {ls.n_band}, tokens differing (all in band) "
        f"{ls.n_diff}")
    return cache, ls


def test_tiny_run(fc):
    cfg = synth.CACHE_CONFIGS["tiny"]
    say("case: cache run, tiny (H=2 d=64 fp32, chunks of 96, budget 160)")
    Q, K, V = synth.cache_inputs(cfg, seed=0)
    _, ls = run_config(fc, cfg, Q.to(DEV), K.to(DEV), V.to(DEV), label="tiny")
    assert ls.n_comp == cfg.n_chunks - 1


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_ragged_commits(fc, dtype, d):
    # commits of uneven sizes (tile tails, a one-token chunk, a chunk as
    # large as the active region), a first commit that already overflows
    cfg = synth.CacheConfig("ragged", H=3, d=d, n_chunks=8, fpc=1, ny=12, nx=10, B_budget=101, B_active=130,
                            Lq=70, lam=0.3, w=7, dtype=dtype)
    sizes = [120, 1, 37, 130, 64, 65, 2, 129, 96, 100]
    say(f"case: cache run, ragged commits ({dtype}, d={d}): {sizes}")
    total = sum(sizes)
    Q, K, V = synth.random_kv(cfg.H, cfg.Lq, total, d, dtype, seed=11)
    Qs = torch.stack([torch.roll(Q, shifts=c, dims=1) for c in range(3)])
    cache, _ = run_config(fc, cfg, Qs.to(DEV), K.to(DEV), V.to(DEV), sizes=sizes, label="ragged")
    # the commit's compression is fc_kv_compress on the merged set: replay the
    # last commit through fc_kv_compress and compare bit for bit
    n_last = sizes[-1]
    p0 = total - n_last
    Kd, Vd = K.to(DEV), V.to(DEV)
    before = fc.KvCache(cfg.H, d, cfg.B_budget, cfg.B_active, cfg.Lq, cfg.lam, cfg.w, Kd.dtype)
    pos = 0
    for c, n in enumerate(sizes[:-1]):
        before.commit(Kd[:, pos:pos + n].contiguous(), Vd[:, pos:pos + n].contiguous(), Qs[c % 3].to(DEV))
        pos += n
    Km = torch.cat([before.K[:, :before.length], Kd[:, p0:]], dim=1).contiguous()
    Vm = torch.cat([before.V[:, :before.length], Vd[:, p0:]], dim=1).contiguous()
    out = fc.fc_kv_compress(Qs[(len(sizes) - 1) % 3].to(DEV), Km, Vm, cfg.B_budget, cfg.lam, cfg.w)
    torch.cuda.synchronize()
    assert torch.equal(out["K_out"], cache.K) and torch.equal(out["V_out"], cache.V)
    pm = torch.cat([before.pos[:, :before.length],
                    torch.arange(p0, total, dtype=torch.int32, device=DEV).expand(cfg.H, -1)], dim=1)
    assert torch.equal(pm.gather(1, out["idx"].long()), cache.pos)


def test_in_place_commits_match_copies(fc):
    # a chunk written into the active rows and committed where it lies gives
    # the same cache, bit for bit, as the chunk handed over for copying; a
    # compressing commit moves the clean tokens to the other region
    cfg = synth.CacheConfig("inplace", H=3, d=128, n_chunks=8, fpc=1, ny=12, nx=10, B_budget=150, B_active=120,
                            Lq=50, lam=0.4, w=5, dtype="bf16")
    sizes = [120, 7, 64, 1, 120, 33, 90, 120]
    say(f"case: cache run, in-place commits against copied ones: {sizes}")
    total = sum(sizes)
    Q, K, V = synth.random_kv(cfg.H, cfg.Lq, total, cfg.d, "bf16", seed=21)
    Qd, Kd, Vd = Q.to(DEV), K.to(DEV), V.to(DEV)
    a = fc.KvCache(cfg.H, cfg.d, cfg.B_budget, cfg.B_active, cfg.Lq, cfg.lam, cfg.w, torch.bfloat16)
    b = fc.KvCache(cfg.H, cfg.d, cfg.B_budget, cfg.B_active, cfg.Lq, cfg.lam, cfg.w, torch.bfloat16)
    p0 = 0
    for n in sizes:
        Kc, Vc = Kd[:, p0:p0 + n].contiguous(), Vd[:, p0:p0 + n].contiguous()
        full = a.length + n > cfg.B_budget
        cur = b.cur
        a.commit(Kc, Vc, Qd)
        Ka, Va = b.active(n)
        Ka.copy_(Kc)
        Va.copy_(Vc)
        b.commit(None, None, Qd, L_c=n)
        torch.cuda.synchronize()
        assert b.cur == (1 - cur if full else cur)
        assert a.cur == b.cur and a.length == b.length == min(p0 + n, cfg.B_budget) and b.next_pos == p0 + n
        assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V) and torch.equal(a.pos, b.pos)
        p0 += n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_group_keys_count_model(fc, dtype):
    # lambda = 0 and unit-vector keys of a few groups: the kept tokens follow
    # the counting model of the oracle's pins exactly (exact ties included)
    H, d, n, T, B = 3, 64, 10, 40, 100
    cfg = synth.CacheConfig("groups", H=H, d=d, n_chunks=n, fpc=1, ny=T, nx=1, B_budget=B, B_active=T, Lq=33,
                            lam=0.0, w=5, dtype=dtype)
    say(f"case: cache run, group keys, lambda = 0 ({dtype})")
    groups = synth.group_labels(H, n, T, seed=5)
    K = synth.group_keys(groups, d, dtype)
    Q, _, V = synth.random_kv(H, cfg.Lq, n * T, d, dtype, seed=6)
    _, ls = run_config(fc, cfg, Q.unsqueeze(0).to(DEV), K.to(DEV), V.to(DEV), label="groups")
    assert ls.n_diff == 0


def test_append_only_and_no_queries(fc):
    # the budget holds the whole run: no compression, no queries, no workspace use
    H, d, T, n = 2, 128, 50, 4
    say("case: cache run that never fills")
    _, K, V = synth.random_kv(H, 1, n * T, d, "bf16", seed=3)
    Kd, Vd = K.to(DEV), V.to(DEV)
    cache = fc.KvCache(H, d, n * T, T, 16, 0.5, 7, torch.bfloat16)
    for c in range(n):
        cache.commit(Kd[:, c * T:(c + 1) * T].contiguous(), Vd[:, c * T:(c + 1) * T].contiguous(), None)
    torch.cuda.synchronize()
    assert cache.length == n * T
    assert torch.equal(cache.K, Kd) and torch.equal(cache.V, Vd)
    assert torch.equal(cache.pos.cpu(), torch.arange(n * T, dtype=torch.int32).expand(H, -1))
    with pytest.raises(fc.FlowCacheError):
        cache.commit(Kd[:, :T].contiguous(), Vd[:, :T].contiguous(), None)  # full now: queries required


def test_magi_like_run(fc):
    # the MAGI-like run at full size (24 heads, chunks of 3600, budget 7200,
    # 3600 queries); the oracle follows two heads, the other heads carry
    # seeded N(0,1) values drawn on the device
    cfg = synth.CACHE_CONFIGS["magi"]
    heads = [0, 13]
    say("case: cache run, MAGI-like (H=24 d=128 bf16, 10 chunks of 3600, budget 7200), oracle on heads 0 and 13")
    T = cfg.tokens_per_chunk
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    K = torch.randn((cfg.H, cfg.n_chunks * T, cfg.d), generator=g, device=DEV).to(torch.bfloat16)
    V = torch.randn((cfg.H, cfg.n_chunks * T, cfg.d), generator=g, device=DEV).to(torch.bfloat16)
    Q = torch.randn((cfg.n_chunks, cfg.H, cfg.Lq, cfg.d), generator=g, device=DEV).to(torch.bfloat16)
    hQ, hK, hV = synth.cache_inputs(cfg, seed=0, heads=heads)
    for n, h in enumerate(heads):
        K[h].copy_(hK[n].to(DEV))
        V[h].copy_(hV[n].to(DEV))
        Q[:, h].copy_(hQ[:, n].to(DEV))
    torch.cuda.synchronize()
    _, ls = run_config(fc, cfg, Q, K, V, heads=heads, label="magi")
    assert ls.n_comp == cfg.n_chunks - 2


def test_long_like_run(fc):
    # the long-video-like run (24 heads, chunks of 8100, budget 32400, 8100
    # queries): merged sets of 40500 keys take the multi-workgroup selection
    # and the persistent pass 1, read with a head stride of 41400 rows; the
    # oracle follows head 7, the other heads carry seeded N(0,1) values
    cfg = synth.CACHE_CONFIGS["long"]
    heads = [7]
    say("case: cache run, long-video-like (H=24 d=128 bf16, 6 chunks of 8100, budget 32400, active 9000), "
        "oracle on head 7")
    T = cfg.tokens_per_chunk
    g = torch.Generator(device=DEV)
    g.manual_seed(78)
    K = torch.randn((cfg.H, cfg.n_chunks * T, cfg.d), generator=g, device=DEV).to(torch.bfloat16)
    V = torch.randn((cfg.H, cfg.n_chunks * T, cfg.d), generator=g, device=DEV).to(torch.bfloat16)
    Q = torch.randn((cfg.n_chunks, cfg.H, cfg.Lq, cfg.d), generator=g, device=DEV).to(torch.bfloat16)
    hQ, hK, hV = synth.cache_inputs(cfg, seed=0, heads=heads)
    for n, h in enumerate(heads):
        K[h].copy_(hK[n].to(DEV))
        V[h].copy_(hV[n].to(DEV))
        Q[:, h].copy_(hQ[:, n].to(DEV))
    torch.cuda.synchronize()
    _, ls = run_config(fc, cfg, Q, K, V, heads=heads, label="long", in_place=True)
    assert ls.n_comp == cfg.n_chunks - 4


def test_degenerate_budget_and_positions(fc):
    # a budget of one token, single-token chunks, positions that end at 2^31 - 1
    H, d = 2, 64
    say("case: cache with B_budget = 1, one-token chunks, positions near 2^31")
    cfg = synth.CacheConfig("one", H=H, d=d, n_chunks=6, fpc=1, ny=1, nx=1, B_budget=1, B_active=1, Lq=5, lam=0.5,
                            w=3, dtype="f32")
    Q, K, V = synth.random_kv(H, cfg.Lq, cfg.n_chunks, d, "f32", seed=12)
    Qs = torch.stack([Q] * cfg.n_chunks)
    run_config(fc, cfg, Qs.to(DEV), K.to(DEV), V.to(DEV), label="one")
    # positions: the last token of the run takes position 2^31 - 1
    cache = fc.KvCache(H, d, 4, 3, cfg.Lq, 0.5, 3, torch.float32)
    cache.next_pos = 2 ** 31 - 1 - 5
    Kd, Vd = K.to(DEV), V.to(DEV)
    cache.commit(Kd[:, :3].contiguous(), Vd[:, :3].contiguous(), Q.to(DEV))
    cache.commit(Kd[:, 3:6].contiguous(), Vd[:, 3:6].contiguous(), Q.to(DEV))
    torch.cuda.synchronize()
    p = cache.pos.cpu()
    assert cache.length == 4 and int(p.max()) <= 2 ** 31 - 1 and int(p.min()) >= 2 ** 31 - 1 - 5
    assert all((p[h][1:] > p[h][:-1]).all() for h in range(H))
    with pytest.raises(fc.FlowCacheError):   # one more token would pass 2^31 - 1
        cache.commit(Kd[:, :1].contiguous(), Vd[:, :1].contiguous(), Q.to(DEV))


def test_commit_without_positions(fc):
    # positions are optional: the same commits with pos_cur = pos_spare = NULL
    # leave the same K and V as KvCache, which tracks positions
    H, d, B, Ba = 2, 128, 90, 70
    sizes = [70, 10, 33, 70, 5]
    say(f"case: commits without positions, {sizes}")
    total = sum(sizes)
    Q, K, V = synth.random_kv(H, 40, total, d, "bf16", seed=31)
    Qd, Kd, Vd = Q.to(DEV), K.to(DEV), V.to(DEV)
    ref = fc.KvCache(H, d, B, Ba, 40, 0.5, 5, torch.bfloat16)
    regs = [(torch.zeros((H, B + Ba, d), dtype=torch.bfloat16, device=DEV),
             torch.zeros((H, B + Ba, d), dtype=torch.bfloat16, device=DEV)) for _ in range(2)]
    cur, length, p0 = 0, 0, 0
    for n in sizes:
        Kc, Vc = Kd[:, p0:p0 + n].contiguous(), Vd[:, p0:p0 + n].contiguous()
        ref.commit(Kc, Vc, Qd)
        (Kcur, Vcur), (Ksp, Vsp) = regs[cur], regs[1 - cur]
        length, swapped = fc.fc_cache_commit(ref.p, length, Kc, Vc, p0, Qd, Kcur, Vcur, None, Ksp, Vsp, None,
                                             ref.workspace)
        if swapped:
            cur = 1 - cur
        p0 += n
        torch.cuda.synchronize()
        assert length == ref.length and cur == ref.cur
        assert torch.equal(regs[cur][0][:, :length], ref.K) and torch.equal(regs[cur][1][:, :length], ref.V)
