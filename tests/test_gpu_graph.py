"""The library's entry points queue kernels only (no memset, copy or
allocation), so a caller can capture them in a HIP graph.  These tests
capture fc_kv_compress and the chunk decision, replay the graphs several
times with eager work and synchronisations in between, and compare every
replay bit for bit with eager calls on the same inputs; and it runs calls on
two streams at once, each with its own workspace."""
import pytest
import torch

from kv_cache_compression_fc_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def fc():
    from kv_cache_compression_fc_amd import binding
    return binding


def say(msg):
    print(msg, flush=True)


def test_compress_graph_replays(fc):
    say("case: fc_kv_compress captured in a graph (H=4 d=128 bf16 Lq=300 Lk=2000 B=700), 4 replays")
    Q, K, V = (x.to(DEV) for x in synth.random_kv(4, 300, 2000, 128, "bf16", seed=21))
    B, lam, w = 700, 0.5, 7
    p = fc.kv_params(Q, K, B, lam, w)
    ws = torch.empty(fc.fc_kv_compress_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    want = fc.fc_kv_compress(Q, K, V, B, lam, w, want_scores=True, workspace=ws)
    torch.cuda.synchronize()
    out = {k: torch.empty_like(v) for k, v in want.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fc.fc_kv_compress(Q, K, V, B, lam, w, want_scores=True, out=out, workspace=ws)   # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fc.fc_kv_compress(Q, K, V, B, lam, w, want_scores=True, out=out, workspace=ws)
    for r in range(4):
        for v in out.values():
            v.fill_(0)                      # eager work between replays
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in want:
            assert torch.equal(out[k], want[k]), f"replay {r}: {k} differs from the eager call"


def test_compress_graph_replays_persistent_split(fc):
    # a shape large enough for the persistent importance passes (their work
    # counters are zeroed by a kernel each call) and the multi-workgroup
    # selection (per-workgroup histograms over four launches)
    H, Lq, Lk, d, B = 8, 2048, 131072, 128, 40000
    say(f"case: fc_kv_compress captured in a graph (H={H} d={d} bf16 Lq={Lq} Lk={Lk} B={B}), 3 replays")
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(5)
    Q = torch.randn((H, Lq, d), generator=g0, device=DEV).to(torch.bfloat16)
    K = torch.randn((H, Lk, d), generator=g0, device=DEV).to(torch.bfloat16)
    V = torch.randn((H, Lk, d), generator=g0, device=DEV).to(torch.bfloat16)
    lam, w = 0.5, 7
    p = fc.kv_params(Q, K, B, lam, w)
    ws = torch.empty(fc.fc_kv_compress_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    want = fc.fc_kv_compress(Q, K, V, B, lam, w, want_scores=True, workspace=ws)
    torch.cuda.synchronize()
    out = {k: torch.empty_like(v) for k, v in want.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fc.fc_kv_compress(Q, K, V, B, lam, w, want_scores=True, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fc.fc_kv_compress(Q, K, V, B, lam, w, want_scores=True, out=out, workspace=ws)
    for r in range(3):
        for v in out.values():
            v.fill_(0)
        ws.fill_(0xAB)                       # counters and histograms must be rebuilt by the replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in want:
            assert torch.equal(out[k], want[k]), f"replay {r}: {k} differs from the eager call"


def test_decision_graph_replays(fc):
    say("case: fc_chunk_rel_l1_decide captured in a graph, 6 replays against an eager twin")
    cfg = synth.ChunkConfig("g", n_chunks=5, chunk_elems=20000, N=12, m=2, eps=(0.05,), dtype="bf16", start_stride=0)
    tr = synth.ChunkTrajectory(cfg, seed=8)
    xt, xtm1, steps = tr.pair(0)
    xt_d, xtm1_d = xt.to(DEV), xtm1.to(DEV)
    dec = fc.ChunkDecider(tr.offsets, cfg.m, 0.05, torch.bfloat16, DEV)
    twin = fc.ChunkDecider(tr.offsets, cfg.m, 0.05, torch.bfloat16, DEV)
    st = torch.tensor(steps, dtype=torch.int32)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dec.decide(xt_d, xtm1_d)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dec.decide(xt_d, xtm1_d)
    for d in (dec, twin):
        d.step.copy_(st)
        d.f.zero_()
    torch.cuda.synchronize()
    for r in range(6):
        g.replay()
        twin.decide(xt_d, xtm1_d)
        torch.cuda.synchronize()
        for name in ("step", "f", "recompute", "l1"):
            assert torch.equal(getattr(dec, name), getattr(twin, name)), f"replay {r}: {name} differs"
    # the replays advanced the device state: six steps counted from 0
    assert dec.step.cpu().tolist() == [6] * cfg.n_chunks


def test_concurrent_streams(fc):
    # calls on different streams with their own workspaces may overlap: two
    # compressions and two decisions in flight at once give the results of
    # the same calls made one after the other
    say("case: fc_kv_compress and the chunk decision on two streams at once")
    Q, K, V = (x.to(DEV) for x in synth.random_kv(3, 257, 3001, 128, "bf16", seed=31))
    Q2, K2, V2 = (x.to(DEV) for x in synth.random_kv(3, 257, 3001, 128, "bf16", seed=32))
    want1 = fc.fc_kv_compress(Q, K, V, 1000, 0.4, 7, want_scores=True)
    want2 = fc.fc_kv_compress(Q2, K2, V2, 1000, 0.6, 5, want_scores=True)
    cfg = synth.ChunkConfig("s", n_chunks=4, chunk_elems=50000, N=8, m=1, eps=(0.05,), dtype="bf16", start_stride=0)
    tr = synth.ChunkTrajectory(cfg, seed=9)
    xt, xtm1, steps = tr.pair(2)
    xt_d, xtm1_d = xt.to(DEV), xtm1.to(DEV)
    ref = fc.ChunkDecider(tr.offsets, cfg.m, 0.05, torch.bfloat16, DEV)
    ref.step.copy_(torch.tensor(steps, dtype=torch.int32))
    ref.decide(xt_d, xtm1_d)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    dec = fc.ChunkDecider(tr.offsets, cfg.m, 0.05, torch.bfloat16, DEV)
    dec.step.copy_(torch.tensor(steps, dtype=torch.int32))
    torch.cuda.synchronize()
    for _ in range(3):
        with torch.cuda.stream(s1):
            got1 = fc.fc_kv_compress(Q, K, V, 1000, 0.4, 7, want_scores=True, stream=s1)
        with torch.cuda.stream(s2):
            got2 = fc.fc_kv_compress(Q2, K2, V2, 1000, 0.6, 5, want_scores=True, stream=s2)
            dec.step.copy_(torch.tensor(steps, dtype=torch.int32, device=DEV))
            dec.f.zero_()
            dec.decide(xt_d, xtm1_d, stream=s2)
        torch.cuda.synchronize()
        for k in want1:
            assert torch.equal(got1[k], want1[k]) and torch.equal(got2[k], want2[k]), k
        for name in ("f", "recompute", "l1", "step"):
            assert torch.equal(getattr(dec, name), getattr(ref, name)), name
