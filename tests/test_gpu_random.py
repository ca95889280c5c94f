"""Seeded random sweeps through the C ABI against the fp64 oracle:
compressions over every dtype, head size, window, lambda and temperature
the boundary accepts (small ones, wider ones up to 700 queries and 60000
keys, and one-query, one-key and budget-above-L_k corners),
chunk decisions (chunkwise, fused Euler, uniform, history-guided) over
random, unaligned chunk tables with random states, step counters and
accumulators, and cache runs with random budgets and commit sizes.  The
configurations come from fixed seeds, so every run draws the same ones."""
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


def kv_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ("bf16", "f32")[int(rng.integers(2))]
        d = (64, 128)[int(rng.integers(2))]
        H = int(rng.integers(1, 5))
        Lq = 1 if rng.uniform() < 0.15 else int(rng.integers(2, 400))
        Lk = 1 if rng.uniform() < 0.1 else int(rng.integers(2, 3000))
        B = int(rng.integers(1, Lk + 10))
        w = int(rng.choice([1, 3, 5, 7, 9]))
        u = rng.uniform()
        lam = 0.0 if u < 0.15 else (1.0 if u < 0.3 else round(float(rng.uniform()), 3))
        scale = 0.0 if rng.uniform() < 0.5 else round(float(rng.uniform(0.02, 0.3)), 4)
        out.append((dtype, d, H, Lq, Lk, B, w, lam, scale, 1000 + i))
    return out


def wide_configs(n, seed):
    """Larger and more varied shapes: up to 700 queries, 6 heads and 60000
    keys (a third of them past one 18432-key chunk), windows up to 129."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ("bf16", "f32")[int(rng.integers(2))] if rng.uniform() < 0.5 else "bf16"
        d = (64, 128)[int(rng.integers(2))]
        H = int(rng.integers(1, 7))
        Lq = 1 if rng.uniform() < 0.08 else int(rng.integers(2, 700))
        Lk = int(rng.choice([int(rng.integers(1, 5000)), int(rng.integers(5000, 20000)),
                             int(rng.integers(18000, 60000))]))
        B = int(rng.integers(1, Lk + 50))
        w = int(rng.choice([1, 3, 5, 7, 9, 15, 33, 129]))
        u = rng.uniform()
        lam = 0.0 if u < 0.1 else (1.0 if u < 0.2 else round(float(rng.uniform()), 3))
        scale = 0.0 if rng.uniform() < 0.5 else round(float(rng.uniform(0.02, 0.3)), 4)
        out.append((dtype, d, H, Lq, Lk, B, w, lam, scale, 5000 + i))
    return out


# shapes whose heads exceed one 18432-key chunk (the split selection), small
# query counts so the oracle stays fast
SPLIT = [
    ("bf16", 128, 2, 40, 18433, 6000, 7, 0.5, 0.0, 951),
    ("bf16", 64, 3, 17, 50000, 25001, 9, 0.3, 0.0, 952),
    ("f32", 128, 1, 9, 37000, 36999, 129, 0.7, 0.0, 953),
    ("bf16", 128, 5, 33, 24000, 1, 1, 0.0, 0.0, 954),
]

CORNERS = [
    # one query and one key; one key, budget above it; every token kept with
    # lambda = 1; lambda = 0 with a wide window; a 1-wide window at B = 1
    ("bf16", 128, 2, 1, 1, 1, 1, 1.0, 0.0, 901),
    ("f32", 64, 3, 50, 1, 5, 3, 0.5, 0.0, 902),
    ("bf16", 128, 1, 300, 500, 600, 7, 1.0, 0.0, 903),
    ("bf16", 64, 2, 129, 777, 100, 9, 0.0, 0.2, 904),
    ("f32", 128, 2, 64, 1000, 1, 1, 0.5, 0.0, 905),
]


@pytest.mark.parametrize("dtype,d,H,Lq,Lk,B,w,lam,scale,seed", kv_configs(16, 2026) + CORNERS + SPLIT + wide_configs(64, 11))
def test_random_compress(fc, dtype, d, H, Lq, Lk, B, w, lam, scale, seed):
    say(f"case: {dtype} d={d} H={H} Lq={Lq} Lk={Lk} B={B} w={w} lambda={lam} scale={scale} seed={seed}")
    Q, K, V = synth.random_kv(H, Lq, Lk, d, dtype, seed=seed)
    out = fc.fc_kv_compress(Q.to(DEV), K.to(DEV), V.to(DEV), B, lam, w, scale, want_scores=True)
    torch.cuda.synchronize()
    ref = oracle.kv_compress(Q, K, V, B, lam, w, None if scale == 0.0 else scale)
    parity.check_scores(out, ref, lam)
    parity.check_selection(out["idx"], ref["score"], B)
    parity.check_gather(K.to(DEV), V.to(DEV), out["idx"], out["K_out"], out["V_out"])
    parity.check_selection_consistent(out["idx"], out["score"], B)


@pytest.mark.parametrize("seed", range(8))
def test_random_chunk_decisions(fc, seed):
    rng = np.random.default_rng(3000 + seed)
    n = int(rng.integers(1, 12))
    sizes = [0 if rng.uniform() < 0.15 else int(rng.integers(1, 50000)) for _ in range(n)]
    offs = [int(rng.integers(0, 9))]
    for s in sizes:
        offs.append(offs[-1] + s)
    total = offs[-1] + int(rng.integers(0, 9))
    dtype = (torch.bfloat16, torch.float32)[int(rng.integers(2))]
    m = int(rng.integers(0, 4))
    eps = float(np.float32(rng.uniform(0.001, 0.05)))
    noise = rng.uniform(0.0005, 0.05, size=n)
    say(f"case: seed {seed}, {n} chunks {sizes} from {offs[0]}, {dtype}, m={m} eps={eps:.4g}")
    x32 = rng.standard_normal(total).astype(np.float32)
    y32 = x32.copy()
    for i in range(n):
        y32[offs[i]:offs[i + 1]] += (noise[i] * rng.standard_normal(sizes[i])).astype(np.float32)
    x = torch.from_numpy(x32).to(dtype)
    y = torch.from_numpy(y32).to(dtype)
    steps = [int(v) for v in rng.integers(-1, 6, size=n)]
    f0 = [float(np.float32(v)) for v in rng.uniform(0.0, eps, size=n)]
    dec = fc.ChunkDecider(offs, m, eps, dtype, DEV)
    dec.step.copy_(torch.tensor(steps, dtype=torch.int32))
    dec.f.copy_(torch.tensor(f0, dtype=torch.float32))
    dec.recompute.fill_(9)
    dec.decide(x.to(DEV), y.to(DEV))
    torch.cuda.synchronize()
    l1 = oracle.chunk_l1_rel(x, y, offs)
    got_l1, got_f = dec.l1.cpu().numpy(), dec.f.cpu().numpy()
    got_rec, got_step = dec.recompute.cpu().tolist(), dec.step.cpu().tolist()
    for i in range(n):
        if steps[i] < 0:  # inactive: untouched
            assert got_rec[i] == 9 and got_step[i] == steps[i] and got_f[i] == np.float32(f0[i]), i
            continue
        assert got_step[i] == steps[i] + 1, i
        if np.isinf(l1[i]):
            assert np.isinf(got_l1[i]), i
        else:
            assert abs(got_l1[i] - l1[i]) <= parity.L1_RTOL * l1[i] + 1e-12, (i, got_l1[i], l1[i])
        want_rec, want_f = oracle.decide(steps[i], f0[i], l1[i], m, eps)
        if steps[i] >= m and abs(f0[i] + l1[i] - eps) <= parity.EPS_BAND:
            continue  # inside the band either branch is correct
        assert got_rec[i] == int(want_rec), (i, got_rec[i], want_rec)
        assert abs(got_f[i] - want_f) <= 1e-6 * max(1.0, abs(want_f)), (i, got_f[i], want_f)


@pytest.mark.parametrize("seed", range(6))
def test_random_euler_steps(fc, seed):
    # the fused update is bit-exact against the oracle's update on every
    # active chunk, leaves inactive chunks and the gaps between chunks alone,
    # and decides exactly as the plain pass on (X_t, the stored X_{t-1})
    rng = np.random.default_rng(4000 + seed)
    n = int(rng.integers(1, 9))
    sizes = [0 if rng.uniform() < 0.1 else int(rng.integers(1, 40000)) for _ in range(n)]
    offs = [int(rng.integers(0, 9))]
    for s in sizes:
        offs.append(offs[-1] + s)
    total = offs[-1] + int(rng.integers(0, 9))
    dtype = (torch.bfloat16, torch.float32)[int(rng.integers(2))]
    m, eps = int(rng.integers(0, 3)), float(np.float32(rng.uniform(0.002, 0.05)))
    dts = [float(np.float32(v)) for v in -rng.uniform(1e-4, 0.05, size=n)]
    steps = [int(v) for v in rng.integers(-1, 5, size=n)]
    say(f"case: seed {seed}, {n} chunks {sizes} from {offs[0]}, {dtype}, steps {steps}")
    x = torch.from_numpy(rng.standard_normal(total).astype(np.float32)).to(dtype)
    v = torch.from_numpy((rng.uniform(0.5, 2.0) * rng.standard_normal(total)).astype(np.float32)).to(dtype)
    y = torch.full((total,), 5.0, dtype=dtype, device=DEV)
    fused = fc.ChunkDecider(offs, m, eps, dtype, DEV)
    fused.step.copy_(torch.tensor(steps, dtype=torch.int32))
    fused.euler_step(x.to(DEV), v.to(DEV), torch.tensor(dts, dtype=torch.float32, device=DEV), y)
    torch.cuda.synchronize()
    active = [s >= 0 for s in steps]
    want = oracle.euler_step(x, v, offs, dts, active)
    got = y.cpu()
    for i in range(n):
        lo, hi = offs[i], offs[i + 1]
        if active[i]:
            assert torch.equal(got[lo:hi], want[lo:hi]), i
        else:
            assert bool((got[lo:hi] == 5.0).all()), i
    assert bool((got[:offs[0]] == 5.0).all()) and bool((got[offs[-1]:] == 5.0).all())
    plain = fc.ChunkDecider(offs, m, eps, dtype, DEV)
    plain.step.copy_(torch.tensor(steps, dtype=torch.int32))
    plain.decide(x.to(DEV), y)
    torch.cuda.synchronize()
    for name in ("recompute", "f", "step"):
        assert torch.equal(getattr(fused, name).cpu(), getattr(plain, name).cpu()), name
    act = torch.tensor(active)
    assert torch.equal(fused.l1.cpu()[act], plain.l1.cpu()[act])


@pytest.mark.parametrize("seed", range(4))
def test_random_cache_runs(fc, seed):
    # random budgets, active sizes, commit sizes (1 .. B_active), query
    # counts, lambda and windows through KvCache, in lockstep with the
    # oracle's cache_commit (tests/test_gpu_cache.py)
    from test_gpu_cache import run_config
    rng = np.random.default_rng(5000 + seed)
    dtype = ("bf16", "f32")[int(rng.integers(2))]
    d = (64, 128)[int(rng.integers(2))]
    H = int(rng.integers(1, 4))
    B_budget, B_active = int(rng.integers(1, 300)), int(rng.integers(1, 300))
    sizes = [int(rng.integers(1, B_active + 1)) for _ in range(int(rng.integers(3, 9)))]
    Lq = int(rng.integers(1, 100))
    lam = round(float(rng.uniform()), 3)
    w = int(rng.choice([1, 3, 5, 7]))
    cfg = synth.CacheConfig("random", H=H, d=d, n_chunks=len(sizes), fpc=1, ny=1, nx=1, B_budget=B_budget,
                            B_active=B_active, Lq=Lq, lam=lam, w=w, dtype=dtype)
    say(f"case: seed {seed}, {dtype} d={d} H={H} budget {B_budget} active {B_active} commits {sizes} Lq={Lq} "
        f"lambda={lam} w={w}")
    total = sum(sizes)
    Q, K, V = synth.random_kv(H, Lq, total, d, dtype, seed=6000 + seed)
    Qs = torch.stack([torch.roll(Q, shifts=c, dims=1) for c in range(3)])
    cache, _ = run_config(fc, cfg, Qs.to(DEV), K.to(DEV), V.to(DEV), sizes=sizes, label=f"random {seed}",
                          in_place=seed % 2 == 1)
    assert cache.length == min(total, B_budget)


@pytest.mark.parametrize("seed", range(4))
def test_random_policies(fc, seed):
    # the uniform rule (one decision for all active chunks) and the
    # history-guided rule on random tables and states
    rng = np.random.default_rng(7000 + seed)
    n = int(rng.integers(1, 10))
    sizes = [0 if rng.uniform() < 0.1 else int(rng.integers(1, 30000)) for _ in range(n)]
    offs = [int(rng.integers(0, 9))]
    for s in sizes:
        offs.append(offs[-1] + s)
    total = offs[-1] + 3
    dtype = (torch.bfloat16, torch.float32)[int(rng.integers(2))]
    m, eps = int(rng.integers(0, 3)), float(np.float32(rng.uniform(0.005, 0.3)))
    say(f"case: seed {seed}, {n} chunks {sizes}, {dtype}, m={m} eps={eps:.4g}")
    x32 = rng.standard_normal(total).astype(np.float32)
    y32 = x32 + (rng.uniform(0.001, 0.1) * rng.standard_normal(total)).astype(np.float32)
    x, y = torch.from_numpy(x32).to(dtype), torch.from_numpy(y32).to(dtype)
    xd, yd = x.to(DEV), y.to(DEV)
    p = fc.fc_l1_params(n, m, eps, fc.FC_BF16 if dtype == torch.bfloat16 else fc.FC_F32)
    ws = torch.empty(fc.fc_chunk_rel_l1_workspace_bytes(p, offs), dtype=torch.uint8, device=DEV)
    # uniform
    cstep = [int(v) for v in rng.integers(-1, 3, size=n)]
    g0, f0 = int(rng.integers(0, 4)), float(np.float32(rng.uniform(0.0, eps)))
    cs = torch.tensor(cstep, dtype=torch.int32, device=DEV)
    gs = torch.tensor([g0], dtype=torch.int32, device=DEV)
    f = torch.tensor([f0], dtype=torch.float32, device=DEV)
    rec = torch.full((n,), 9, dtype=torch.uint8, device=DEV)
    l1 = torch.zeros(1, dtype=torch.float32, device=DEV)
    fc.fc_uniform_rel_l1_decide(p, offs, xd, yd, cs, gs, f, rec, l1, ws)
    torch.cuda.synchronize()
    active = [c >= 0 for c in cstep]
    got = rec.cpu().tolist()
    assert all(got[i] == 9 for i in range(n) if not active[i])
    assert gs.item() == g0 + 1
    want_l1 = oracle.uniform_l1_rel(x, y, offs, active)
    if np.isinf(want_l1):
        assert np.isinf(l1.item())
    else:
        assert abs(l1.item() - want_l1) <= parity.L1_RTOL * want_l1 + 1e-12
    r, fw = oracle.decide(g0, f0, want_l1, m, eps)
    if not (g0 >= m and abs(f0 + want_l1 - eps) <= parity.EPS_BAND):
        assert all(got[i] == int(r) for i in range(n) if active[i])
        assert abs(f.item() - fw) <= 1e-6 * max(1.0, abs(fw))
    # history-guided
    hsteps = [int(v) for v in rng.integers(-1, 4, size=n)]
    acc0 = [float(np.float32(v)) for v in rng.uniform(0.0, eps, size=n)]
    st = torch.tensor(hsteps, dtype=torch.int32, device=DEV)
    acc = torch.tensor(acc0, dtype=torch.float32, device=DEV)
    ref = torch.full((n,), 9, dtype=torch.uint8, device=DEV)
    dev = torch.zeros(n, dtype=torch.float32, device=DEV)
    fc.fc_history_rel_l1_decide(p, offs, xd, yd, st, acc, ref, dev, ws)
    torch.cuda.synchronize()
    want = oracle.chunk_l1_rel(x, y, offs)
    g_ref, g_acc, g_st = ref.cpu().tolist(), acc.cpu().numpy(), st.cpu().tolist()
    for i in range(n):
        if hsteps[i] < 0:
            assert g_ref[i] == 9 and g_st[i] == hsteps[i], i
            continue
        assert g_st[i] == hsteps[i] + 1, i
        r, a = oracle.decide_history(hsteps[i], acc0[i], want[i], m, eps)
        if hsteps[i] >= m and abs(acc0[i] + want[i] - eps) <= parity.EPS_BAND:
            continue
        assert g_ref[i] == int(r), (i, g_ref[i], r)
        if np.isinf(a):
            assert np.isinf(g_acc[i]), i
        else:
            assert abs(g_acc[i] - a) <= 1e-6 * max(1.0, abs(a)), (i, g_acc[i], a)
