"""The allocation-free chunk decision (fc_chunk_rel_l1_decide_noalloc) against
the workspace form (fc_chunk_rel_l1_decide) through the C ABI: the same
kernels on the same inputs, so step counters, accumulators, recompute flags
and L1_rel must agree bit for bit.  Two calls in a row share the library's
static scratch, the second with a smaller input (fewer chunks, other dtype),
so stale partials of the first call must not leak into the second; then a
few decisions in a row on one trajectory of states."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def fc():
    from kv_cache_compression_fc_amd import binding
    return binding


def say(msg):
    print(msg, flush=True)


def _case(rng, n, max_size, dtype):
    sizes = [int(rng.integers(1, max_size)) for _ in range(n)]
    offs = [int(rng.integers(0, 9))]
    for s in sizes:
        offs.append(offs[-1] + s)
    total = offs[-1] + int(rng.integers(0, 9))
    xt = torch.from_numpy(rng.standard_normal(total).astype(np.float32))
    xtm1 = xt + torch.from_numpy((0.01 * rng.standard_normal(total)).astype(np.float32))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    steps = torch.from_numpy(rng.integers(-1, 8, size=n).astype(np.int32))
    f0 = torch.from_numpy(rng.uniform(0, 0.01, size=n).astype(np.float32))
    return offs, xt.to(tdt).to(DEV), xtm1.to(tdt).to(DEV), steps.to(DEV), f0.to(DEV)


def _both(fc, p, offs, xt, xtm1, steps, f0):
    n = p.n_chunks
    out = []
    for noalloc in (False, True):
        st, f = steps.clone(), f0.clone()
        rec = torch.full((n,), 7, dtype=torch.uint8, device=DEV)
        l1 = torch.full((n,), -1.0, dtype=torch.float32, device=DEV)
        if noalloc:
            fc.fc_chunk_rel_l1_decide_noalloc(p, offs, xt, xtm1, st, f, rec, l1)
        else:
            fc.fc_chunk_rel_l1_decide(p, offs, xt, xtm1, st, f, rec, l1)
        torch.cuda.synchronize()
        out.append((st.cpu(), f.cpu(), rec.cpu(), l1.cpu()))
    return out


def _equal(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.float32 else x,
                           y.view(torch.uint8) if y.dtype == torch.float32 else y)


def test_noalloc_matches_workspace_form_two_calls(fc):
    rng = np.random.default_rng(77)
    # first call: 12 bf16 chunks of up to 900k elements (several slabs each)
    case1 = _case(rng, 12, 900_000, "bf16")
    say(f"call 1: 12 bf16 chunks, {case1[0][-1]} elements")
    p1 = fc.fc_l1_params(12, 3, 0.02, fc.FC_BF16)
    ws_form, na_form = _both(fc, p1, *case1)
    _equal(ws_form, na_form)
    # second call, smaller: 3 float32 chunks of up to 40k elements
    case2 = _case(rng, 3, 40_000, "f32")
    say(f"call 2: 3 f32 chunks, {case2[0][-1]} elements")
    p2 = fc.fc_l1_params(3, 2, 0.015, fc.FC_F32)
    ws_form, na_form = _both(fc, p2, *case2)
    _equal(ws_form, na_form)


def test_noalloc_trajectory(fc):
    """Ten decisions in a row on drifting states: the device counters and
    accumulators of both forms stay identical."""
    rng = np.random.default_rng(78)
    offs, xt, xtm1, steps, f0 = _case(rng, 5, 300_000, "bf16")
    say(f"trajectory: 5 bf16 chunks, {offs[-1]} elements")
    p = fc.fc_l1_params(5, 2, 0.01, fc.FC_BF16)
    sa, fa = steps.clone().clamp_min(0), f0.clone()
    sb, fb = sa.clone(), fa.clone()
    ra = torch.zeros(5, dtype=torch.uint8, device=DEV)
    rb = torch.zeros_like(ra)
    for k in range(10):
        x0 = xt.float() * (1.0 - 0.03 * k)
        x1 = xtm1.float() * (1.0 - 0.03 * k)
        a, b = x0.to(torch.bfloat16), x1.to(torch.bfloat16)
        fc.fc_chunk_rel_l1_decide(p, offs, a, b, sa, fa, ra)
        fc.fc_chunk_rel_l1_decide_noalloc(p, offs, a, b, sb, fb, rb)
        torch.cuda.synchronize()
        assert torch.equal(sa, sb) and torch.equal(ra, rb)
        assert torch.equal(fa.view(torch.int32), fb.view(torch.int32))
