"""GPU parity of fc_euler_step_l1_decide: the sampler's Euler update with the
chunk decision fused ("Flow Caching for Autoregressive Video Generation",
papernotes digest, Key designs item 1 writes the L1 numerator as ||v dt||_1).

The updated state must equal the oracle's bit for bit (the storage rounding
is a quantisation, taken in the kernel's float32 precision on both sides);
the decisions follow the oracle in lockstep under the tolerances of
parity.py; and the fused call must decide exactly as fc_chunk_rel_l1_decide
does on (X_t, the state it wrote).
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_fc_amd import synth
from parity import DecisionLockstep

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def fc():
    from kv_cache_compression_fc_amd import binding
    return binding


def say(msg):
    print(msg, flush=True)


def run_fused(fc, cfg, eps, in_place, seed=0, check_unfused=True):
    """Integrate every chunk from X_N with the fused call (chunk i starts at
    global step i * start_stride), beside the oracle."""
    tr = synth.ChunkTrajectory(cfg, seed=seed)
    dt_t = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    x_ref = tr.noise_states()
    v = tr.velocity()
    v_d = v.to(DEV)
    X = x_ref.to(DEV)
    Y = X if in_place else X.clone()   # out of place: inactive chunks keep their values in both
    dec = fc.ChunkDecider(tr.offsets, cfg.m, eps, dt_t, DEV)
    twin = fc.ChunkDecider(tr.offsets, cfg.m, eps, dt_t, DEV) if check_unfused else None
    lk = DecisionLockstep(cfg.n_chunks, cfg.m, eps)
    for g in range(tr.n_global_steps()):
        steps = [tr.local_step(i, g) for i in range(cfg.n_chunks)]
        active = [n >= 0 for n in steps]
        dts = [tr.step_size(n) if n >= 0 else 0.0 for n in steps]
        st = torch.tensor(steps, dtype=torch.int32, device=DEV)
        dec.step.copy_(st)
        x_before = X.clone() if (check_unfused or not in_place) else None
        if twin is not None:
            twin.step.copy_(st)
            twin.f.copy_(dec.f)
        dec.euler_step(X, v_d, torch.tensor(dts, dtype=torch.float32, device=DEV), Y)
        torch.cuda.synchronize()
        y_ref = oracle.euler_step(x_ref, v, tr.offsets, dts, active)
        got = Y.cpu()
        assert torch.equal(got.view(torch.int16 if cfg.dtype == "bf16" else torch.int32),
                           y_ref.view(torch.int16 if cfg.dtype == "bf16" else torch.int32)), f"state differs at step {g}"
        l1_ref = oracle.chunk_l1_rel(x_ref, y_ref, tr.offsets)
        lk.step(steps, l1_ref, dec.recompute.cpu().numpy(), dec.f.cpu().numpy(), dec.l1.cpu().numpy())
        if twin is not None:
            twin.decide(x_before, Y)
            torch.cuda.synchronize()
            act = torch.tensor(active, device=DEV)
            assert torch.equal(twin.l1[act], dec.l1[act]), "fused L1 differs from the two-state pass"
            assert torch.equal(twin.f[act], dec.f[act]) and torch.equal(twin.recompute[act], dec.recompute[act])
        x_ref = y_ref
        if not in_place:
            X.copy_(Y)
    return lk


@pytest.mark.parametrize("in_place", [True, False])
def test_tiny_fused(fc, in_place):
    cfg = synth.CHUNK_CONFIGS["tiny"]
    say(f"case: fused Euler + decision, tiny 4 x 256 fp32, in place {in_place}")
    lk = run_fused(fc, cfg, 0.01, in_place)
    say(f"  decisions {lk.decisions}, exempt {lk.exempt}")


@pytest.mark.parametrize("seed", [1, 2])
def test_staggered_bf16_fused(fc, seed):
    cfg = synth.ChunkConfig("stag", n_chunks=5, chunk_elems=1000 + 37 * seed, N=30, m=3, eps=(0.02,), dtype="bf16",
                            start_stride=4)
    say(f"case: fused Euler + decision, 5 chunks x {cfg.chunk_elems} bf16, staggered, seed {seed}")
    lk = run_fused(fc, cfg, cfg.eps[0], in_place=(seed == 1), seed=seed)
    say(f"  decisions {lk.decisions}, exempt {lk.exempt}")


def test_rounding_cases_in_head_tail_and_body(fc):
    # the oracle's pins, on the device: no fused multiply-add (f32), ties to
    # even (bf16), in the unaligned head and tail of a slab and in its body
    a = 1.0 + 2.0 ** -23
    for dtype, x0, v0, dt0, want in ((torch.float32, -(1.0 + 2.0 ** -22), a, a, 0.0),
                                     (torch.bfloat16, 1.0 + 2.0 ** -7, 1.0, 2.0 ** -8, 1.0 + 2.0 ** -6),
                                     (torch.bfloat16, 1.0, 1.0, 2.0 ** -8, 1.0)):
        say(f"case: rounding of the fused update, {dtype}, x={x0!r} v={v0!r} dt={dt0!r}")
        n = 3 + 8 * 40 + 6   # an unaligned head (from 3) and tail (the last element)
        offs = [3, n]
        x = torch.full((n,), x0, dtype=dtype)
        v = torch.full((n,), v0, dtype=dtype)
        p = fc.fc_l1_params(1, 0, 0.5, fc.FC_BF16 if dtype == torch.bfloat16 else fc.FC_F32)
        ws = torch.empty(fc.fc_chunk_rel_l1_workspace_bytes(p, offs), dtype=torch.uint8, device=DEV)
        step = torch.zeros(1, dtype=torch.int32, device=DEV)
        f = torch.zeros(1, dtype=torch.float32, device=DEV)
        rec = torch.zeros(1, dtype=torch.uint8, device=DEV)
        y = torch.full((n,), 7.0, dtype=dtype, device=DEV)
        fc.fc_euler_step_l1_decide(p, offs, x.to(DEV), v.to(DEV), torch.tensor([dt0], device=DEV), y, step, f, rec,
                                   workspace=ws)
        torch.cuda.synchronize()
        got = y.cpu()
        assert got[:3].tolist() == [7.0] * 3, "elements before the first chunk were written"
        assert (got[3:] == want).all(), got[3:].unique()
        assert torch.equal(got, torch.cat([torch.full((3,), 7.0, dtype=dtype),
                                           oracle.euler_step(x[3:], v[3:], [0, n - 3], [dt0], [True])]))


def test_inactive_chunks_untouched(fc):
    say("case: fused update leaves inactive chunks unread and unwritten")
    offs = [0, 1000, 2500, 2501, 4000]
    g = torch.Generator(device=DEV)
    g.manual_seed(23)
    x = torch.randn(4000, generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn(4000, generator=g, device=DEV).to(torch.bfloat16)
    y = torch.full((4000,), 3.0, dtype=torch.bfloat16, device=DEV)
    dec = fc.ChunkDecider(offs, 0, 0.1, torch.bfloat16, DEV)
    dec.step.copy_(torch.tensor([0, -1, 5, -1], dtype=torch.int32))
    dec.f.fill_(0.25)
    dec.recompute.fill_(9)
    dec.euler_step(x, v, torch.tensor([0.1, 0.2, 0.3, 0.4], device=DEV), y)
    torch.cuda.synchronize()
    yc = y.cpu()
    assert (yc[1000:2500] == 3.0).all() and (yc[2501:] == 3.0).all()
    ref = oracle.euler_step(x.cpu(), v.cpu(), offs, [0.1, 0.2, 0.3, 0.4], [True, False, True, False])
    assert torch.equal(yc[:1000], ref[:1000]) and torch.equal(yc[2500:2501], ref[2500:2501])
    assert dec.step.cpu().tolist() == [1, -1, 6, -1]
    assert dec.f.cpu()[1].item() == 0.25 and dec.recompute.cpu()[3].item() == 9


def test_scale_fused_steady_state(fc):
    # 16 chunks x 64x8x90x160 bf16, every chunk active at its own local step
    # (the steady state of the staggered schedule), updated in place
    cfg = synth.CHUNK_CONFIGS["scale"]
    say("case: fused Euler + decision at scale, 16 x 7,372,800 bf16, steady state, in place")
    tr = synth.ChunkTrajectory(cfg, seed=0)
    g = cfg.n_chunks - 1
    xt, _, steps = tr.pair(g)
    dts = [tr.step_size(n) for n in steps]
    v = tr.velocity()
    for eps in cfg.eps:
        dec = fc.ChunkDecider(tr.offsets, cfg.m, eps, torch.bfloat16, DEV)
        dec.step.copy_(torch.tensor(steps, dtype=torch.int32))
        f0 = torch.linspace(0, eps, cfg.n_chunks)
        dec.f.copy_(f0)
        X = xt.to(DEV)
        dec.euler_step(X, v.to(DEV), torch.tensor(dts, dtype=torch.float32, device=DEV), X)
        torch.cuda.synchronize()
        y_ref = oracle.euler_step(xt, v, tr.offsets, dts, [True] * cfg.n_chunks)
        assert torch.equal(X.cpu().view(torch.int16), y_ref.view(torch.int16))
        l1_ref = oracle.chunk_l1_rel(xt, y_ref, tr.offsets)
        lk = DecisionLockstep(cfg.n_chunks, cfg.m, eps)
        lk.f[:] = f0.numpy()
        lk.step(steps, l1_ref, dec.recompute.cpu().numpy(), dec.f.cpu().numpy(), dec.l1.cpu().numpy())
        say(f"  eps {eps}: recompute {dec.recompute.cpu().tolist()}, exempt {lk.exempt}")
