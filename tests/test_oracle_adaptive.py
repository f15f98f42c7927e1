"""Pins of the oracle's near-tie adaptive budget (value-of-information router
abstract, automata-index page: the gap between the k-th and (k+1)-th best
block scores decides whether a query's kept set is doubled).

The rule is pinned to its two limits (a threshold of 0 is plain top-k, an
infinite one is plain top-2k), to the pure-Python brute force (exact
rational scores) on random inputs with mixed decisions, and to a hand-worked
example with exact scores that puts one gap exactly on the threshold.
Planted mistakes (<= for <, the gap one slot off, doubling the widest gaps)
must each fail one of the pins."""
import math

import numpy as np
import pytest

from oracle import brute
from oracle import hsa_oracle as O
from tests.test_oracle_pins import rand_qkv


def run_adaptive(Q, K, V, S, k, tau, dtype):
    """Oracle over every row of [B, Hq, T, D] inputs; returns stacked arrays."""
    B, Hq, T, D = Q.shape
    Hkv = K.shape[1]
    L = O.landmarks(K, S, dtype)
    outs, sels, dbl, gaps = [], [], [], []
    pos = np.arange(T)
    for b in range(B):
        for h in range(Hq):
            g = O.kv_head_of(h, Hq, Hkv)
            r, d, gp = O.hsa_rows_adaptive(Q[b, h], pos, K[b, g], V[b, g], L[b, g], S, k, tau)
            outs.append(r.out)
            sels.append(r.sel_idx)
            dbl.append(d)
            gaps.append(gp)
    return np.stack(outs), np.stack(sels), np.stack(dbl), np.stack(gaps)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_zero_threshold_is_plain_topk_and_infinite_is_top_2k(dtype):
    S, k, T, D = 4, 3, 64, 8
    Q, K, V = rand_qkv(31, 1, 2, 1, T, D, dtype)
    out0, sel0, dbl0, _ = run_adaptive(Q, K, V, S, k, 0.0, dtype)
    ref_k, sel_k, _, _ = O.prefill(Q, K, V, S, k, dtype)
    assert not dbl0.any()
    assert np.array_equal(out0, ref_k.reshape(out0.shape))
    assert np.array_equal(sel0[..., :k], sel_k.reshape(-1, T, k)) and np.all(sel0[..., k:] == -1)
    outi, seli, dbli, _ = run_adaptive(Q, K, V, S, k, math.inf, dtype)
    ref_2k, sel_2k, _, _ = O.prefill(Q, K, V, S, 2 * k, dtype)
    assert np.array_equal(outi, ref_2k.reshape(outi.shape))
    assert np.array_equal(seli, sel_2k.reshape(seli.shape))
    n = np.minimum(np.arange(T) // S, T // S)
    assert np.array_equal(dbli[0], n > k)


@pytest.mark.parametrize("case", [(1, 2, 1, 48, 4, 4, 2, "fp32"), (1, 2, 2, 40, 8, 2, 3, "bf16")])
def test_adaptive_matches_brute_force(case):
    B, Hq, Hkv, T, D, S, k, dtype = case
    Q, K, V = rand_qkv(41 + k, B, Hq, Hkv, T, D, dtype)
    _, _, _, gaps = run_adaptive(Q, K, V, S, k, 0.0, dtype)
    g = gaps[~np.isnan(gaps)]
    # a threshold between two observed gaps, far from both: about half the rows double
    srt = np.sort(g)
    i = len(srt) // 2
    tau = 0.5 * (srt[i - 1] + srt[i])
    assert srt[i] - srt[i - 1] > 1e-9
    out, sel, dbl, _ = run_adaptive(Q, K, V, S, k, tau, dtype)
    assert 0 < dbl.sum() < (~np.isnan(gaps)).sum()
    for b in range(B):
        for h in range(Hq):
            g_ = (h * Hkv) // Hq
            for p in range(T):
                bo, bs, bc, bd = brute.hsa_query_adaptive(Q[b, h, p].tolist(), p, K[b, g_].tolist(),
                                                          V[b, g_].tolist(), S, k, tau, dtype)
                row = b * Hq + h
                assert bool(dbl[row, p]) == bd
                m = len(bs)
                assert list(sel[row, p, :m]) == bs and np.all(sel[row, p, m:] == -1)
                np.testing.assert_allclose(out[row, p], bo, rtol=0, atol=1e-12)


def hand_case():
    """D = 4 (scale 1/2), S = 2, chunks of two equal keys: landmark = that key.
    Query e0; first key components 10, 8, 7, 7, 3, so the exact scores are
    5, 4, 3.5, 3.5, 1.5 (chunk order 0..4).  Values are constant per chunk."""
    firsts = [10, 8, 7, 7, 3]
    K = np.zeros((10, 4))
    V = np.zeros((10, 4))
    for c, f in enumerate(firsts):
        K[2 * c:2 * c + 2, 0] = f
        V[2 * c:2 * c + 2, :] = c + 1  # chunk c's attention output is (c+1) * ones
    q = np.array([[1.0, 0.0, 0.0, 0.0]])
    L = O.landmarks(K, 2, "fp32")
    return q, K, V, L


def fused(chunks, scores):
    w = np.exp(np.array(scores) - max(scores))
    w /= w.sum()
    return float(sum(wi * (c + 1) for wi, c in zip(w, chunks))) * np.ones(4)


@pytest.mark.parametrize("k,tau,expect", [
    (2, 0.5, [0, 1]),                  # gap s2 - s3 = 0.5, not < 0.5: keep k
    (2, 0.5000001, [0, 1, 2, 3]),      # just above: keep 2k; the 3.5 tie goes lower index first
    (3, 0.0, [0, 1, 2]),               # gap s3 - s4 = 0 (a tie), threshold 0: keep k
    (3, 1e-300, [0, 1, 2, 3, 4]),      # any positive threshold doubles; only 5 candidates
    (1, 1.0, [0]),                     # gap 1.0
    (1, 1.5, [0, 1]),
    (5, math.inf, [0, 1, 2, 3, 4]),    # n <= k: no cut, all kept
])
def test_hand_worked_gaps(k, tau, expect):
    q, K, V, L = hand_case()
    r, dbl, gap = O.hsa_rows_adaptive(q, np.array([10]), K, V, L, 2, k, tau)
    m = len(expect)
    assert list(r.sel_idx[0, :m]) == expect and np.all(r.sel_idx[0, m:] == -1)
    scores = [[5, 4, 3.5, 3.5, 1.5][c] for c in expect]
    np.testing.assert_allclose(r.sel_score[0, :m], scores, rtol=0, atol=0)
    np.testing.assert_allclose(r.out[0], fused(expect, scores), rtol=0, atol=1e-14)
    assert bool(dbl[0]) == (m > k)
    assert (np.isnan(gap[0]) if k >= 5 else gap[0] == [1.0, 0.5, 0.0][k - 1])


def test_planted_mistakes_are_caught(monkeypatch):
    good = O.adaptive_keep_count

    def le_instead_of_lt(s, k, tau):
        n = len(s)
        if n <= k:
            return n, float("nan")
        gap = float(s[k - 1] - s[k])
        return (min(2 * k, n) if gap <= tau else k), gap

    def gap_one_off(s, k, tau):
        n = len(s)
        if n <= k + 1:
            return n if n <= k else k, float("nan")
        gap = float(s[k] - s[k + 1])
        return (min(2 * k, n) if gap < tau else k), gap

    def widest_gaps(s, k, tau):
        m, gap = good(s, k, tau)
        if np.isnan(gap):
            return m, gap
        return (min(2 * k, len(s)) if gap > tau else k), gap

    cases = [(2, 0.5, [0, 1]), (2, 0.5000001, [0, 1, 2, 3]), (3, 0.0, [0, 1, 2]), (1, 1.0, [0]),
             (1, 1.5, [0, 1])]
    for bad in (le_instead_of_lt, gap_one_off, widest_gaps):
        failed = 0
        with monkeypatch.context() as m:
            m.setattr(O, "adaptive_keep_count", bad)
            for c in cases:
                try:
                    test_hand_worked_gaps(*c)
                except AssertionError:
                    failed += 1
        assert failed >= 1, bad.__name__
    assert O.adaptive_keep_count is good
