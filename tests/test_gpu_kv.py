"""GPU parity of the KV-compression path (fc_kv_compress and its stages)
against the fp64 oracle, through the C ABI.  Tolerances: see parity.py."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import parity
from kv_cache_compression_fc_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def fc():
    from kv_cache_compression_fc_amd import binding
    return binding


def say(msg):
    print(msg, flush=True)


def gpu_compress(fc, Q, K, V, B, lam, w, scale=0.0):
    out = fc.fc_kv_compress(Q.to(DEV), K.to(DEV), V.to(DEV), B, lam, w, scale, want_scores=True)
    torch.cuda.synchronize()
    return out


def full_check(fc, Q, K, V, B, lam, w, scale=None):
    d = K.shape[2]
    out = gpu_compress(fc, Q, K, V, B, lam, w, 0.0 if scale is None else scale)
    ref = oracle.kv_compress(Q, K, V, B, lam, w, scale)
    parity.check_scores(out, ref, lam)
    parity.check_selection(out["idx"], ref["score"], B)
    parity.check_gather(K.to(DEV), V.to(DEV), out["idx"], out["K_out"], out["V_out"])
    parity.check_selection_consistent(out["idx"], out["score"], B)
    return out, ref


def test_tiny_config(fc):
    cfg = synth.KV_CONFIGS["tiny"]
    say("case: tiny config (H=2 d=64 Lq=64 Lk=256 B=64 fp32)")
    Q, K, V = synth.kv_inputs(cfg, seed=0)
    full_check(fc, Q, K, V, cfg.B, cfg.lam[0], cfg.w)


def test_hand_example_padded(fc):
    # the golden example, embedded in d=64 by zero padding (dot products and
    # norms unchanged), float32 inputs
    g = json.load(open(os.path.join(GOLDEN, "kv_hand_example.json")))
    say("case: hand-worked example padded to d=64")

    def pad(x):
        a = np.zeros((1, len(x[0]), 64), np.float32)
        a[0, :, :2] = np.array(x[0], np.float32)
        return torch.from_numpy(a)
    Q, K, V = pad(g["Q"]), pad(g["K"]), pad(g["V"])
    out = gpu_compress(fc, Q, K, V, g["B"], g["lam"], g["w"], g["scale"])
    ev = lambda e: float(eval(e, {"__builtins__": {}}, {"sqrt": math.sqrt, "exp": math.exp}))
    for key in ("imp_pooled", "red", "score"):
        want = np.array([ev(e) for e in g["expect"][key]])
        np.testing.assert_allclose(out[key][0].cpu().double().numpy(), want, rtol=1e-5, atol=1e-6, err_msg=key)
    assert out["idx"][0].tolist() == g["expect"]["idx"]
    np.testing.assert_array_equal(out["V_out"][0, :, :2].cpu().numpy(), np.array(g["expect"]["V_out"]))


RAGGED = [
    # dtype, d, H, Lq, Lk, B, w
    ("bf16", 128, 3, 100, 700, 200, 7),
    ("bf16", 128, 2, 129, 2049, 1000, 5),
    ("bf16", 64, 2, 257, 4097, 3000, 3),
    ("bf16", 128, 1, 1, 300, 17, 7),
    ("f32", 64, 2, 37, 333, 100, 5),
    ("f32", 128, 1, 70, 190, 50, 1),
    ("bf16", 64, 5, 31, 65, 64, 9),
    # few key blocks, many queries: pass 2 splits the queries into ranges
    # (partial importance planes added by the select)
    ("bf16", 128, 2, 2000, 700, 300, 7),
    ("f32", 64, 1, 1000, 300, 100, 5),
]


@pytest.mark.parametrize("dtype,d,H,Lq,Lk,B,w", RAGGED)
def test_ragged_shapes(fc, dtype, d, H, Lq, Lk, B, w):
    say(f"case: ragged {dtype} d={d} H={H} Lq={Lq} Lk={Lk} B={B} w={w}")
    Q, K, V = synth.random_kv(H, Lq, Lk, d, dtype, seed=Lq * 7 + Lk)
    full_check(fc, Q, K, V, B, 0.5, w)


def test_explicit_scale_and_lambda_extremes(fc):
    cfg = synth.KV_CONFIGS["tiny"]
    Q, K, V = synth.kv_inputs(cfg, seed=1)
    for lam in (0.0, 1.0, 0.3):
        say(f"case: tiny seed 1, scale 0.2, lambda {lam}")
        full_check(fc, Q, K, V, cfg.B, lam, cfg.w, scale=0.2)


def test_budget_covers_all_tokens(fc):
    Q, K, V = synth.random_kv(2, 40, 90, 128, "bf16", seed=5)
    for B in (90, 500):
        for scores in (True, False):  # without score outputs the call only copies the rows
            say(f"case: B={B} >= Lk=90 keeps every token (score outputs: {scores})")
            out = fc.fc_kv_compress(Q.to(DEV), K.to(DEV), V.to(DEV), B, 0.5, 7, want_scores=scores)
            torch.cuda.synchronize()
            assert torch.equal(out["idx"].cpu(), torch.arange(90, dtype=torch.int32).repeat(2, 1))
            assert torch.equal(out["K_out"].cpu(), K) and torch.equal(out["V_out"].cpu(), V)
    # larger, fp32, ragged: rows past several gather blocks
    Q, K, V = synth.random_kv(3, 5, 1001, 64, "f32", seed=6)
    say("case: B=1001 = Lk, f32 d=64, no score outputs")
    out = fc.fc_kv_compress(Q.to(DEV), K.to(DEV), V.to(DEV), 1001, 0.5, 7)
    torch.cuda.synchronize()
    assert torch.equal(out["idx"].cpu(), torch.arange(1001, dtype=torch.int32).repeat(3, 1))
    assert torch.equal(out["K_out"].cpu(), K) and torch.equal(out["V_out"].cpu(), V)


def test_single_key_and_single_budget(fc):
    Q, K, V = synth.random_kv(2, 8, 1, 64, "bf16", seed=6)
    say("case: Lk=1")
    out = gpu_compress(fc, Q, K, V, 4, 0.5, 3)
    assert out["idx"].cpu().tolist() == [[0], [0]]
    np.testing.assert_allclose(out["imp_pooled"].cpu().numpy(), 1.0, rtol=1e-6)
    Q, K, V = synth.random_kv(3, 50, 500, 128, "bf16", seed=7)
    say("case: B=1")
    full_check(fc, Q, K, V, 1, 0.5, 7)


def test_zero_and_duplicate_keys(fc):
    Q, K, V = synth.random_kv(2, 64, 600, 128, "bf16", seed=8)
    K[0, 10] = 0
    K[1, 100:200] = K[1, 300:400]
    V[1, 100:200] = V[1, 300:400]
    say("case: zero key and duplicated keys")
    out, ref = full_check(fc, Q, K, V, 150, 0.5, 7)
    assert torch.isfinite(out["score"]).all()


@pytest.mark.parametrize("H,Lq,Lk", [(3, 300, 1000), (2, 2500, 500)])
def test_importance_stage(fc, H, Lq, Lk):
    # the second shape splits pass 2 into query ranges (planes added after)
    Q, K, _ = synth.random_kv(H, Lq, Lk, 128, "bf16", seed=9)
    say(f"case: fc_kv_importance bf16 H={H} Lq={Lq} Lk={Lk}")
    imp = fc.fc_kv_importance(Q.to(DEV), K.to(DEV))
    torch.cuda.synchronize()
    want = oracle.importance(Q, K, 1 / math.sqrt(128))
    assert parity.max_rel_err(imp.cpu().numpy(), want) <= parity.REL
    np.testing.assert_allclose(imp.double().sum(dim=1).cpu().numpy(), 1.0, rtol=1e-4)


def test_redundancy_stage(fc):
    _, K, _ = synth.random_kv(2, 1, 3000, 128, "bf16", seed=10)
    K[0, 7] = 0
    say("case: fc_kv_redundancy bf16 H=2 Lk=3000")
    r = fc.fc_kv_redundancy(K.to(DEV))
    torch.cuda.synchronize()
    want = oracle.redundancy_mean(K)
    assert float(np.max(np.abs(r.cpu().double().numpy() - want))) <= 1e-5
    assert float(r[0, 7]) == 0.0


# Heads of more than 18432 scores take the selection split over several
# workgroups per head: just above that size, many exact ties, B = 1,
# B = L - 1, B = L, many heads, and one head of 4.5M scores (more workgroups
# per head than threads in one, so the compaction loops over the earlier ones).
SPLIT_CASES = [(1, 18433, 9000, 0), (3, 129600, 32400, 3), (24, 40000, 1, 0), (5, 30000, 29999, 2),
               (2, 20000, 20000, 0), (1, 4_500_000, 1_000_000, 20), (40, 46800, 15600, 0)]


@pytest.mark.parametrize("H,L,B,levels", [(1, 10, 3, 0), (4, 5000, 1234, 0), (3, 5000, 2500, 7), (2, 70000, 20000, 50),
                                          (2, 4096, 4096, 3), (2, 100, 400, 0), (3, 2049, 1, 2), (1, 3, 2, 1)]
                         + SPLIT_CASES)
def test_topb_select_exact(fc, H, L, B, levels):
    s = synth.random_scores(H, L, seed=H * 1000 + L, n_levels=levels)
    if levels == 0 and L >= 10:
        s[0, :5] = -0.0
        s[0, 5:10] = 0.0
    say(f"case: fc_topb_select H={H} L={L} B={B} levels={levels}")
    idx = fc.fc_topb_select(s.to(DEV), B)
    torch.cuda.synchronize()
    want = oracle.select_topb(s.double().numpy(), B)
    np.testing.assert_array_equal(idx.cpu().numpy(), want)


def test_select_stage_from_oracle_inputs(fc):
    # importance and redundancy means given as float32 inputs
    cfg = synth.KV_CONFIGS["magi"]
    Q, K, V = synth.kv_inputs(cfg, seed=0, heads=[3])
    imp = oracle.importance(Q, K, 1 / math.sqrt(cfg.d)).astype(np.float32)
    r = oracle.redundancy_mean(K).astype(np.float32)
    say("case: fc_kv_select from float32 importance/redundancy, one MAGI-like head")
    out = fc.fc_kv_select(torch.from_numpy(imp).to(DEV), torch.from_numpy(r).to(DEV), cfg.B, 0.5, cfg.w,
                          K.to(DEV), V.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.kv_compress(Q, K, V, cfg.B, 0.5, cfg.w, imp=imp.astype(np.float64), r=r.astype(np.float64))
    parity.check_scores(out, ref, 0.5)
    parity.check_selection(out["idx"], ref["score"], cfg.B)
    parity.check_gather(K.to(DEV), V.to(DEV), out["idx"], out["K_out"], out["V_out"])


def test_deterministic(fc):
    Q, K, V = synth.random_kv(4, 500, 5000, 128, "bf16", seed=11)
    say("case: two identical calls give identical bits")
    a = gpu_compress(fc, Q, K, V, 1500, 0.5, 7)
    b = gpu_compress(fc, Q, K, V, 1500, 0.5, 7)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype,d,H,Lq,Lk", [("bf16", 128, 3, 200, 3000), ("f32", 64, 2, 65, 513),
                                             ("bf16", 64, 1, 3000, 400)])
def test_importance_two_stages(fc, dtype, d, H, Lq, Lk):
    # pass 1 (lse) against the oracle's log-sum-exp, then pass 2 fed with it
    Q, K, _ = synth.random_kv(H, Lq, Lk, d, dtype, seed=12)
    say(f"case: fc_kv_importance_lse + fc_kv_importance_colsum {dtype} d={d} H={H} Lq={Lq} Lk={Lk}")
    lse = fc.fc_kv_importance_lse(Q.to(DEV), K.to(DEV))
    imp = fc.fc_kv_importance_colsum(Q.to(DEV), K.to(DEV), lse)
    torch.cuda.synchronize()
    want_lse = oracle.lse(Q, K, 1 / math.sqrt(d))
    # an absolute lse error e is a relative error e on every exp(s - lse)
    assert float(np.max(np.abs(lse.cpu().double().numpy() - want_lse))) <= 1e-4
    assert parity.max_rel_err(imp.cpu().numpy(), oracle.importance(Q, K, 1 / math.sqrt(d))) <= parity.REL


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 64), ("bf16", 128)])
def test_importance_wide_logit_range(fc, dtype, d):
    # a later key scores ~150 binary orders above the first keys of its range,
    # which the fixed shift of pass 1 cannot hold: the exact path must take over
    H, Lq, Lk = 2, 70, 700
    rng = np.random.default_rng(13)
    Q = rng.standard_normal((H, Lq, d)).astype(np.float32)
    K = 0.01 * rng.standard_normal((H, Lk, d)).astype(np.float32)
    Q[:, :, 0] = 10.0
    K[0, 600, 0] = 10.0          # logit 100 (scale 1) against ~0 for the rest
    K[1, 333, 0] = -10.0         # and a very negative one
    Qt, Kt = torch.from_numpy(Q), torch.from_numpy(K)
    if dtype == "bf16":
        Qt, Kt = Qt.to(torch.bfloat16), Kt.to(torch.bfloat16)
    say(f"case: importance with a 100-nat logit spread ({dtype}, d={d})")
    imp = fc.fc_kv_importance(Qt.to(DEV), Kt.to(DEV), softmax_scale=1.0)
    lse = fc.fc_kv_importance_lse(Qt.to(DEV), Kt.to(DEV), softmax_scale=1.0)
    torch.cuda.synchronize()
    assert torch.isfinite(imp).all() and torch.isfinite(lse).all()
    want = oracle.importance(Qt, Kt, 1.0)
    # relative error on the entries that carry the mass; tiny ones absolutely
    got = imp.cpu().double().numpy()
    big = want > 1e-30
    assert float(np.max(np.abs(got[big] - want[big]) / want[big])) <= parity.REL or \
        float(np.max(np.abs(got - want))) <= 1e-6
    np.testing.assert_allclose(lse.cpu().double().numpy(), oracle.lse(Qt, Kt, 1.0), rtol=0, atol=1e-3)


@pytest.mark.parametrize("dtype,d,H,Lq,Lk", [("bf16", 128, 3, 300, 5000), ("f32", 64, 2, 70, 777),
                                             ("bf16", 64, 2, 2500, 500)])
def test_importance_redundancy_stage(fc, dtype, d, H, Lq, Lk):
    """The compression's first half as a stage: the importance bit-identical to
    fc_kv_importance's, the redundancy against the oracle (as the stand-alone
    stage is), and both fed to fc_kv_select give fc_kv_compress's result."""
    Q, K, V = synth.random_kv(H, Lq, Lk, d, dtype, seed=21)
    say(f"case: fc_kv_importance_redundancy {dtype} d={d} H={H} Lq={Lq} Lk={Lk}")
    Qd, Kd, Vd = Q.to(DEV), K.to(DEV), V.to(DEV)
    imp, r = fc.fc_kv_importance_redundancy(Qd, Kd)
    imp_alone = fc.fc_kv_importance(Qd, Kd)
    torch.cuda.synchronize()
    assert torch.equal(imp.view(torch.int32), imp_alone.view(torch.int32))
    want_imp = oracle.importance(Q, K, 1 / math.sqrt(d))
    assert parity.max_rel_err(imp.cpu().numpy(), want_imp) <= parity.REL
    want_r = oracle.redundancy_mean(K)
    assert float(np.max(np.abs(r.cpu().double().numpy() - want_r))) <= 1e-5
    B = Lk // 3
    sel = fc.fc_kv_select(imp, r, B, 0.5, 7, Kd, Vd, want_scores=False)
    full = fc.fc_kv_compress(Qd, Kd, Vd, B, 0.5, 7)
    torch.cuda.synchronize()
    ref = oracle.kv_compress(Q, K, V, B, 0.5, 7)
    parity.check_selection(sel["idx"], ref["score"], B)
    parity.check_selection(full["idx"], ref["score"], B)
