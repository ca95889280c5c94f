"""Comparison helpers for the GPU parity tests (tolerances in one place).

Tolerances (float32 accumulation on bf16 or fp32 inputs, compared with the
fp64 oracle on identical input values):
  * pooled importance, redundancy softmax: elementwise relative error <= 1e-3;
  * score: |dScore_j| <= 1e-3 * (lambda Imp~_j + (1-lambda) Red_j)  -- the
    score is a difference of two ~1/L_k terms, so the bound is relative to
    the magnitude of its parts;
  * top-B sets: equal except for tokens whose normalised oracle score lies in
    the band |L_k (Score_j - Score_(B'))| <= 1e-4 around the B'-th largest;
  * kept K/V rows: bit-exact copies of the input rows;
  * decisions: bit-exact unless |f + L1_rel - eps| <= 1e-6 on the oracle side;
  * states written by the fused Euler update: bit-exact (the storage rounding
    is taken in float32 on both sides).
"""
import numpy as np
import torch

import oracle

REL = 1e-3
BAND = 1e-4
L1_RTOL = 1e-5       # float32 slab sums vs fp64 (reported value only)
EPS_BAND = 1e-6      # decisions within this distance of eps are exempt


def max_rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.max(np.abs(got - want) / np.abs(want)))


def check_scores(out, ref, lam, heads=None):
    """out: GPU dict (torch, [H][L]); ref: oracle dict (numpy, [H'][L]) for
    `heads` (default all)."""
    H = ref["imp_pooled"].shape[0]
    heads = list(range(H)) if heads is None else list(heads)
    imp_p = out["imp_pooled"][heads].cpu().double().numpy()
    red = out["red"][heads].cpu().double().numpy()
    score = out["score"][heads].cpu().double().numpy()
    e_imp = max_rel_err(imp_p, ref["imp_pooled"])
    e_red = max_rel_err(red, ref["red"])
    mag = lam * ref["imp_pooled"] + (1 - lam) * ref["red"]
    e_score = float(np.max(np.abs(score - ref["score"]) / mag))
    assert e_imp <= REL, f"pooled importance rel err {e_imp:.3g}"
    assert e_red <= REL, f"redundancy rel err {e_red:.3g}"
    assert e_score <= REL, f"score err {e_score:.3g} (relative to its parts)"
    return e_imp, e_red, e_score


def check_selection(idx_gpu, ref_score, B, heads=None):
    """idx_gpu: torch [H][B'] int32; ref_score: oracle scores [H'][L] (fp64).
    Returns (band population, tokens that differ) summed over heads."""
    idx = idx_gpu.cpu().numpy()
    H, L = ref_score.shape
    heads = list(range(H)) if heads is None else list(heads)
    Bp = min(B, L)
    n_band = n_diff = 0
    for n, h in enumerate(heads):
        g = idx[h]
        assert np.all(np.diff(g) > 0), "indices must be strictly ascending"
        assert g.min() >= 0 and g.max() < L
        s = ref_score[n]
        sb = np.sort(s)[::-1][Bp - 1]
        band = np.abs(L * (s - sb)) <= BAND
        want = set(np.lexsort((np.arange(L), -s))[:Bp].tolist())
        diff = set(g.tolist()) ^ want
        bad = [j for j in diff if not band[j]]
        assert not bad, f"head {h}: {len(bad)} tokens differ outside the tie band, e.g. {bad[:5]}"
        n_band += int(band.sum())
        n_diff += len(diff)
    return n_band, n_diff


def check_gather(K_in, V_in, idx_gpu, K_out, V_out, heads=None):
    """Kept rows are exact copies of the input rows named by idx."""
    H = idx_gpu.shape[0]
    heads = range(H) if heads is None else heads
    for h in heads:
        ii = idx_gpu[h].long()
        assert torch.equal(K_out[h], K_in[h].index_select(0, ii)), f"K rows differ, head {h}"
        assert torch.equal(V_out[h], V_in[h].index_select(0, ii)), f"V rows differ, head {h}"


def check_selection_consistent(idx_gpu, score_gpu, B):
    """Property of the GPU's own output: every kept token's float32 score is
    >= every dropped token's, with ties kept at lower indices."""
    idx = idx_gpu.cpu().numpy()
    sc = score_gpu.cpu().numpy()
    H, L = sc.shape
    for h in range(H):
        keep = np.zeros(L, bool)
        keep[idx[h]] = True
        if keep.all():
            continue
        kmin = sc[h][keep].min()
        dmax = sc[h][~keep].max()
        assert kmin >= dmax, f"head {h}: kept min {kmin} < dropped max {dmax}"
        if kmin == dmax:  # ties: every kept tie has a lower index than every dropped tie
            kt = np.nonzero(keep & (sc[h] == kmin))[0]
            dt = np.nonzero(~keep & (sc[h] == kmin))[0]
            assert kt.max() < dt.min()


class DecisionLockstep:
    """Oracle state per chunk, advanced beside the GPU's.  `rule` is the
    oracle's decision function (oracle.decide for FlowCache's chunkwise rule,
    oracle.decide_history for ARCache's history-guided one)."""

    def __init__(self, n, m, eps, rule=None):
        self.f = np.zeros(n)
        self.m, self.eps = m, eps
        self.rule = oracle.decide if rule is None else rule
        self.exempt = 0
        self.decisions = 0

    def step(self, steps, l1_ref, rec_gpu, f_gpu, l1_gpu):
        for i, n in enumerate(steps):
            if n < 0:
                continue
            f_prev = self.f[i]
            r, f_new = self.rule(n, f_prev, l1_ref[i], self.m, self.eps)
            if np.isfinite(l1_ref[i]):
                assert abs(l1_gpu[i] - l1_ref[i]) <= L1_RTOL * l1_ref[i] + 1e-12, (i, n, l1_gpu[i], l1_ref[i])
            else:
                assert l1_gpu[i] == np.inf
            exempt = n >= self.m and abs(f_prev + l1_ref[i] - self.eps) <= EPS_BAND
            self.decisions += 1
            if exempt:
                self.exempt += 1
            else:
                assert bool(rec_gpu[i]) == r, f"chunk {i} local step {n}: gpu {rec_gpu[i]} oracle {r}"
                assert abs(f_gpu[i] - f_new) <= 1e-6 or (np.isinf(f_new) and f_gpu[i] == f_new), (i, n, f_gpu[i], f_new)
            self.f[i] = f_new if bool(rec_gpu[i]) == r else float(f_gpu[i])
