"""Pins of the oracle's backward pass (hsa_rows_backward, prefill_backward).

* finite differences of the oracle's forward (fp64 storage, so the forward is
  smooth; the selection is held fixed, as the backward defines it);
* S = 1 with every chunk kept: the layer is dense causal attention without
  the diagonal, whose gradients torch's autograd gives (fp64);
* S = 1 with a sparse kept set: masked attention over the kept keys;
* the two-chunk case: rows with one candidate are plain attention over
  chunk 0 (in-chunk softmax path only).
Source mutations of the backward (a dropped landmark term, a missing 1/S, a
missing fusion-softmax term) must each fail one of the pins."""
import inspect
import math
import textwrap

import numpy as np
import pytest
import torch

from oracle import hsa_oracle as O
from tests.test_oracle_pins import rand_qkv


def forward_fixed(Q, K, V, S, sel, dtype="fp64"):
    """Oracle forward with the selection fixed to sel [B,Hq,T,k]."""
    B, Hq, T, D = Q.shape
    Hkv = K.shape[1]
    L = O.landmarks(K, S, dtype)
    out = np.zeros_like(Q)
    pos = np.arange(T)
    for b in range(B):
        for h in range(Hq):
            g = O.kv_head_of(h, Hq, Hkv)
            lists = [[c for c in sel[b, h, t] if c >= 0] for t in range(T)]
            for t in range(T):  # hsa_rows stacks overrides of equal length per candidate count
                if lists[t]:
                    out[b, h, t] = O.hsa_rows(Q[b, h, t:t + 1], pos[t:t + 1], K[b, g], V[b, g], L[b, g], S,
                                              len(lists[t]), sel_override=[lists[t]]).out[0]
    return out


def finite_difference_check(Q, K, V, S, k, G, eps=1e-6, rtol=2e-6):
    _, sel, _, _ = O.prefill(Q, K, V, S, k, "fp64")
    dQ, dK, dV, _, _, _ = O.prefill_backward(Q, K, V, S, k, "fp64", G, sel_idx=sel)

    def loss(Q_, K_, V_):
        return float(np.sum(G * forward_fixed(Q_, K_, V_, S, sel)))

    for name, X, grad in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        num = np.zeros_like(X)
        it = np.nditer(X, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = X[i]
            X[i] = old + eps
            lp = loss(Q, K, V)
            X[i] = old - eps
            lm = loss(Q, K, V)
            X[i] = old
            num[i] = (lp - lm) / (2 * eps)
        scale = max(np.abs(num).max(), 1e-12)
        np.testing.assert_allclose(grad, num, rtol=0, atol=rtol * scale * 50, err_msg=f"d{name}")


@pytest.mark.parametrize("case", [(1, 1, 1, 20, 3, 4, 2), (1, 2, 1, 18, 4, 3, 3), (1, 2, 2, 16, 2, 2, 8)])
def test_backward_matches_finite_differences(case):
    B, Hq, Hkv, T, D, S, k = case
    Q, K, V = rand_qkv(50 + T, B, Hq, Hkv, T, D, "fp32")
    G = np.random.default_rng(60 + T).standard_normal(Q.shape)
    finite_difference_check(Q, K, V, S, k, G)


def torch_attention_grads(q, k, v, mask, g):
    """Autograd of masked softmax attention (fp64): gradients w.r.t. q, k, v."""
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    m = torch.from_numpy(mask)
    logits = (tq @ tk.T) / math.sqrt(q.shape[1])
    logits = logits.masked_fill(~m, float("-inf"))
    out = torch.softmax(logits, dim=-1) @ tv
    out.backward(torch.from_numpy(g))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def test_chunk1_dense_causal_gradients():
    T, D = 24, 6
    Q, K, V = rand_qkv(70, 1, 1, 1, T, D, "fp32")
    G = np.random.default_rng(71).standard_normal(Q.shape)
    dQ, dK, dV, _, _, _ = O.prefill_backward(Q, K, V, 1, T + 3, "fp64", G)
    mask = np.tril(np.ones((T, T), dtype=bool), k=-1)[1:]
    rq, rk, rv = torch_attention_grads(Q[0, 0, 1:], K[0, 0], V[0, 0], mask, G[0, 0, 1:])
    np.testing.assert_allclose(dQ[0, 0, 1:], rq, rtol=0, atol=1e-12)
    assert np.all(dQ[0, 0, 0] == 0)
    np.testing.assert_allclose(dK[0, 0], rk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV[0, 0], rv, rtol=0, atol=1e-12)


def test_chunk1_sparse_gradients_are_masked_attention():
    T, D, k = 30, 4, 5
    Q, K, V = rand_qkv(72, 1, 1, 1, T, D, "fp32")
    G = np.random.default_rng(73).standard_normal(Q.shape)
    _, sel, _, _ = O.prefill(Q, K, V, 1, k, "fp64")
    dQ, dK, dV, _, _, _ = O.prefill_backward(Q, K, V, 1, k, "fp64", G, sel_idx=sel)
    mask = np.zeros((T, T), dtype=bool)
    for t in range(T):
        mask[t, [c for c in sel[0, 0, t] if c >= 0]] = True
    rows = mask.any(axis=1)
    rq, rk, rv = torch_attention_grads(Q[0, 0, rows], K[0, 0], V[0, 0], mask[rows], G[0, 0, rows])
    np.testing.assert_allclose(dQ[0, 0, rows], rq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK[0, 0], rk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV[0, 0], rv, rtol=0, atol=1e-12)


@pytest.mark.parametrize("S", [4, 8])
def test_two_chunk_gradients_are_plain_attention_over_chunk0(S):
    D = 5
    Q, K, V = rand_qkv(74 + S, 1, 1, 1, 2 * S, D, "bf16")
    G = np.random.default_rng(75).standard_normal(Q.shape)
    dQ, dK, dV, _, _, _ = O.prefill_backward(Q, K, V, S, 3, "bf16", G)
    rq, rk, rv = torch_attention_grads(Q[0, 0, S:], K[0, 0, :S], V[0, 0, :S], np.ones((S, S), dtype=bool),
                                       G[0, 0, S:])
    np.testing.assert_allclose(dQ[0, 0, S:], rq, rtol=0, atol=1e-12)
    assert np.all(dQ[0, 0, :S] == 0)
    np.testing.assert_allclose(dK[0, 0, :S], rk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV[0, 0, :S], rv, rtol=0, atol=1e-12)
    assert np.all(dK[0, 0, S:] == 0) and np.all(dV[0, 0, S:] == 0)


def test_planted_mistakes_are_caught(monkeypatch):
    src = textwrap.dedent(inspect.getsource(O.hsa_rows_backward))
    mutations = {
        "landmark term of dK dropped": ("gk = (dlogit + ds[:, None] / S)", "gk = (dlogit + 0 * ds[:, None] / S)"),
        "landmark 1/S missing": ("gk = (dlogit + ds[:, None] / S)", "gk = (dlogit + ds[:, None])"),
        "score path of dq dropped": ("+ ds @ Lg[chunks]) * sig", "+ 0 * (ds @ Lg[chunks])) * sig"),
        "fusion softmax centring dropped": ("ds = w * (o @ g - out @ g)", "ds = w * (o @ g)"),
        "in-chunk softmax centring dropped": ("dlogit = a * (da - np.sum(a * da, axis=1, keepdims=True))",
                                              "dlogit = a * da"),
    }
    for name, (a, b) in mutations.items():
        assert a in src, name
        ns = dict(O.__dict__)
        exec(compile(src.replace(a, b), "<mutant>", "exec"), ns)
        failed = 0
        with monkeypatch.context() as m:
            m.setattr(O, "hsa_rows_backward", ns["hsa_rows_backward"])
            for fn in (lambda: test_backward_matches_finite_differences((1, 2, 1, 18, 4, 3, 3)),
                       test_chunk1_dense_causal_gradients,
                       lambda: test_two_chunk_gradients_are_plain_attention_over_chunk0(4)):
                try:
                    fn()
                except AssertionError:
                    failed += 1
        assert failed >= 1, name
