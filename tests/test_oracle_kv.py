"""Pins for the KV-compression half of the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a worked
example, a closed form, an invariant, a special case that reduces to a library
routine, or brute force.  Definitions: "Flow Caching for Autoregressive Video
Generation" (papernotes digest), Key designs item 3.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from kv_cache_compression_fc_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _eval(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"sqrt": math.sqrt, "exp": math.exp, "log": math.log}))


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------- worked example

def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "kv_hand_example.json")))
    Q, K, V = (np.array(g[k], np.float64) for k in ("Q", "K", "V"))
    out = oracle.kv_compress(Q, K, V, B=g["B"], lam=g["lam"], w=g["w"], scale=g["scale"])
    for key in ("imp", "imp_pooled", "r", "red", "score"):
        want = np.array([_eval(e) for e in g["expect"][key]])
        np.testing.assert_allclose(out[key][0], want, rtol=0, atol=1e-14, err_msg=key)
    assert out["idx"][0].tolist() == g["expect"]["idx"]
    np.testing.assert_array_equal(out["V_out"][0], np.array(g["expect"]["V_out"]))
    np.testing.assert_array_equal(out["K_out"][0], K[0][g["expect"]["idx"]])


# --------------------------------------------------------------- importance

def test_importance_rows_sum_to_one():
    Q, K = _rand((3, 17, 16), 1), _rand((3, 41, 16), 2)
    imp = oracle.importance(Q, K, 0.37)
    np.testing.assert_allclose(imp.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (imp > 0).all()


def test_importance_zero_queries_is_uniform():
    Q, K = np.zeros((2, 5, 8)), _rand((2, 13, 8), 3)
    imp = oracle.importance(Q, K, 1.0)
    np.testing.assert_array_equal(imp, np.full((2, 13), 1.0 / 13))


def test_importance_two_keys_is_mean_logistic():
    # softmax over two logits = logistic of their difference
    Q, K = _rand((1, 9, 4), 4), _rand((1, 2, 4), 5)
    s = 0.8 * Q[0] @ K[0].T
    want0 = scipy.special.expit(s[:, 0] - s[:, 1]).mean()
    imp = oracle.importance(Q, K, 0.8)
    np.testing.assert_allclose(imp[0], [want0, 1 - want0], rtol=1e-13)


def test_importance_single_query_is_softmax_row():
    Q, K = _rand((2, 1, 8), 6), _rand((2, 30, 8), 7)
    imp = oracle.importance(Q, K, 0.5)
    for h in range(2):
        np.testing.assert_allclose(imp[h], scipy.special.softmax(0.5 * K[h] @ Q[h, 0]), rtol=1e-13)


def test_importance_matches_torch_softmax_on_tiny_config():
    cfg = synth.KV_CONFIGS["tiny"]
    Q, K, _ = synth.kv_inputs(cfg, seed=0)
    scale = 1.0 / math.sqrt(cfg.d)
    q64, k64 = Q.double(), K.double()
    want = torch.softmax(scale * (q64 @ k64.transpose(1, 2).contiguous()), dim=-1).mean(dim=1).numpy()
    got = oracle.importance(Q, K, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)


def test_importance_permutation_equivariant():
    Q, K = _rand((1, 7, 8), 8), _rand((1, 25, 8), 9)
    perm = np.random.default_rng(10).permutation(25)
    a = oracle.importance(Q, K, 0.9)
    b = oracle.importance(Q, K[:, perm], 0.9)
    np.testing.assert_allclose(b[0], a[0][perm], rtol=1e-13)


def test_lse_matches_scipy():
    Q, K = _rand((2, 6, 8), 11), _rand((2, 19, 8), 12)
    got = oracle.lse(Q, K, 0.7)
    for h in range(2):
        np.testing.assert_allclose(got[h], scipy.special.logsumexp(0.7 * Q[h] @ K[h].T, axis=1), rtol=1e-14)


def test_importance_equals_exp_minus_lse_mean():
    # Imp_j = mean_i exp(s_ij - lse_i): ties the two-pass formulation to the definition
    Q, K = _rand((1, 11, 8), 13), _rand((1, 23, 8), 14)
    lse = oracle.lse(Q, K, 0.6)
    p = np.exp(0.6 * Q[0] @ K[0].T - lse[0][:, None])
    np.testing.assert_allclose(oracle.importance(Q, K, 0.6)[0], p.mean(axis=0), rtol=1e-13)


# --------------------------------------------------------------- max-pool

@pytest.mark.parametrize("w", [1, 3, 5, 7])
def test_maxpool_matches_torch(w):
    x = _rand((3, 50), 20 + w)
    want = F.max_pool1d(torch.from_numpy(x)[:, None, :], w, 1, (w - 1) // 2)[:, 0, :].numpy()
    np.testing.assert_array_equal(oracle.maxpool1d(x, w), want)


def test_maxpool_properties():
    x = _rand((2, 40), 30)
    np.testing.assert_array_equal(oracle.maxpool1d(x, 1), x)
    assert (oracle.maxpool1d(x, 7) >= x).all()
    c = np.full((1, 9), 0.25)
    np.testing.assert_array_equal(oracle.maxpool1d(c, 5), c)
    # a single spike spreads to exactly its window, clipped at the edges
    s = np.zeros((1, 10)); s[0, 1] = 1.0
    np.testing.assert_array_equal(oracle.maxpool1d(s, 5)[0], [1, 1, 1, 1, 0, 0, 0, 0, 0, 0])


# --------------------------------------------------------------- redundancy

def test_redundancy_closed_form_equals_bruteforce_tiny():
    cfg = synth.KV_CONFIGS["tiny"]
    _, K, _ = synth.kv_inputs(cfg, seed=0)
    a = oracle.redundancy_mean(K, "bruteforce")
    b = oracle.redundancy_mean(K, "closed")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_redundancy_closed_form_equals_bruteforce_field_keys():
    # two heads of the MAGI-like generator at full key count
    cfg = synth.KV_CONFIGS["magi"]
    _, K, _ = synth.kv_inputs(cfg, seed=0, heads=[0, 7])
    a = oracle.redundancy_mean(K, "bruteforce")
    b = oracle.redundancy_mean(K, "closed")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_redundancy_matches_torch_definition():
    K = _rand((2, 37, 8), 40)
    kt = F.normalize(torch.from_numpy(K), dim=-1)
    S = kt @ kt.transpose(1, 2)
    S = S - torch.diag_embed(torch.diagonal(S, dim1=1, dim2=2))
    want_r = S.mean(dim=1).numpy()          # (1/Lk) sum over i of S_ij
    np.testing.assert_allclose(oracle.redundancy_mean(K, "closed"), want_r, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.redundancy(K), torch.softmax(S.mean(dim=1), -1).numpy(), rtol=1e-13)


def test_redundancy_orthonormal_keys_uniform():
    Qm, _ = np.linalg.qr(_rand((16, 16), 41))
    K = (Qm[:10] * 3.0)[None]               # 10 orthogonal keys of norm 3
    np.testing.assert_allclose(oracle.redundancy_mean(K), 0.0, atol=1e-15)
    np.testing.assert_allclose(oracle.redundancy(K), 0.1, rtol=1e-14)


def test_redundancy_identical_keys():
    K = np.tile(_rand((1, 1, 8), 42), (1, 12, 1))
    np.testing.assert_allclose(oracle.redundancy_mean(K), 11.0 / 12.0, rtol=1e-14)


def test_redundancy_scale_invariant_and_zero_key():
    K = _rand((1, 20, 8), 43)
    s = np.abs(_rand((1, 20, 1), 44)) + 0.1
    np.testing.assert_allclose(oracle.redundancy_mean(K * s), oracle.redundancy_mean(K), atol=1e-14)
    Kz = K.copy(); Kz[0, 5] = 0.0
    r = oracle.redundancy_mean(Kz, "closed")
    assert r[0, 5] == 0.0
    np.testing.assert_allclose(r, oracle.redundancy_mean(Kz, "bruteforce"), atol=1e-14)


# --------------------------------------------------------------- selection

def test_select_matches_full_sort_and_topk():
    s = _rand((4, 300), 50)
    idx = oracle.select_topb(s, 77)
    for h in range(4):
        order = sorted(range(300), key=lambda j: (-s[h, j], j))
        assert idx[h].tolist() == sorted(order[:77])
        tk = torch.topk(torch.from_numpy(s[h]), 77).indices.numpy()
        assert set(tk.tolist()) == set(idx[h].tolist())


def test_select_ties_prefer_lower_index():
    s = np.array([[1.0, 2.0, 2.0, 0.5, 2.0, 2.0]])
    assert oracle.select_topb(s, 3)[0].tolist() == [1, 2, 4]
    assert oracle.select_topb(-np.zeros((1, 5)), 2)[0].tolist() == [0, 1]


def test_select_budget_at_least_length_keeps_all():
    s = _rand((2, 9), 51)
    np.testing.assert_array_equal(oracle.select_topb(s, 9), np.tile(np.arange(9), (2, 1)))
    np.testing.assert_array_equal(oracle.select_topb(s, 100), np.tile(np.arange(9), (2, 1)))


def test_lambda_extremes():
    cfg = synth.KV_CONFIGS["tiny"]
    Q, K, V = synth.kv_inputs(cfg, seed=0)
    one = oracle.kv_compress(Q, K, V, B=64, lam=1.0, w=5)
    np.testing.assert_array_equal(one["idx"], oracle.select_topb(one["imp_pooled"], 64))
    zero = oracle.kv_compress(Q, K, V, B=64, lam=0.0, w=5)
    np.testing.assert_array_equal(zero["idx"], oracle.select_topb(-zero["red"], 64))


def test_duplicate_keys_get_equal_redundancy():
    cfg = synth.KV_CONFIGS["long"]
    small = synth.KVConfig("dup", H=1, d=16, Lq=8, Lk=64 * 4 * 4, B=10, lam=(0.5,), w=7, dtype="bf16",
                           key_kind="field", frames=64, ny=4, nx=4, sigma=1.0, dup=cfg.dup)
    _, K, _ = synth.kv_inputs(small, seed=3)
    r = oracle.redundancy_mean(K)
    tpf = 16
    np.testing.assert_array_equal(r[0, 48 * tpf:64 * tpf], r[0, 16 * tpf:32 * tpf])


def test_gather_rows():
    X = torch.arange(2 * 5 * 3, dtype=torch.float32).reshape(2, 5, 3)
    idx = np.array([[0, 4], [1, 2]])
    out = oracle.gather_rows(X, idx)
    assert torch.equal(out[0], X[0, [0, 4]]) and torch.equal(out[1], X[1, [1, 2]])
