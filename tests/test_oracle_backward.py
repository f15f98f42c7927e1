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


# ---------------------------------------------------------------------------
# the error scales the GPU bounds are built from
# ---------------------------------------------------------------------------

from oracle import brute  # noqa: E402

SCALE_CASES = [
    # B, Hq, Hkv, T, D, S, k, dtype
    (1, 1, 1, 14, 3, 2, 3, "fp32"),
    (1, 2, 1, 13, 4, 3, 2, "bf16"),
    (1, 2, 2, 16, 2, 4, 1, "bf16"),
    (1, 4, 2, 12, 3, 2, 8, "fp32"),   # k above the candidate count
]


def _oracle_rows(Q, K, V, S, k, dtype, G, b, h):
    Hq, Hkv, T = Q.shape[1], K.shape[1], Q.shape[2]
    g = O.kv_head_of(h, Hq, Hkv)
    L = O.landmarks(K, S, dtype)
    _, sel, _, _ = O.prefill(Q, K, V, S, k, dtype, L=L)
    res = O.hsa_rows_backward(Q[b, h], np.arange(T), K[b, g], V[b, g], L[b, g], S, sel[b, h], G[b, h])
    return g, sel[b, h], res


@pytest.mark.parametrize("case", SCALE_CASES)
def test_backward_scales_equal_brute_term_sums(case):
    """Gradients, magnitude sums and output sensitivities of the numpy
    backward equal the term-by-term pure-Python sums of oracle.brute, row by
    row (dq) and accumulated over rows (dK, dV)."""
    B, Hq, Hkv, T, D, S, k, dtype = case
    Q, K, V = rand_qkv(80 + T, B, Hq, Hkv, T, D, dtype)
    G = np.random.default_rng(81 + T).standard_normal(Q.shape)
    for h in range(Hq):
        g, sel, res = _oracle_rows(Q, K, V, S, k, dtype, G, 0, h)
        Kl, Vl = K[0, g].tolist(), V[0, g].tolist()
        bK = np.zeros((T, D, 3))
        bV = np.zeros((T, D, 3))
        for p in range(T):
            dq, dK, dV = brute.backward_query(Q[0, h, p].tolist(), Kl, Vl, S, sel[p].tolist(), G[0, h, p].tolist(),
                                              dtype)
            dq = np.array(dq)
            for arr, got in ((res.dq[p], dq[:, 0]), (res.abs_dq[p], dq[:, 1]), (res.out_dq[p], dq[:, 2])):
                np.testing.assert_allclose(arr, got, rtol=1e-11, atol=1e-14)
            for t, v in dK.items():
                bK[t] += np.array(v)
            for t, v in dV.items():
                bV[t] += np.array(v)
        for arr, got in ((res.dK, bK[..., 0]), (res.abs_dK, bK[..., 1]), (res.out_dK, bK[..., 2]),
                         (res.dV, bV[..., 0]), (res.abs_dV, bV[..., 1])):
            np.testing.assert_allclose(arr, got, rtol=1e-11, atol=1e-14)
        assert np.all(bV[..., 2] == 0)


def test_magnitude_sums_bound_the_gradients():
    B, Hq, Hkv, T, D, S, k = 1, 2, 1, 64, 6, 4, 3
    Q, K, V = rand_qkv(90, B, Hq, Hkv, T, D, "bf16")
    G = np.random.default_rng(91).standard_normal(Q.shape)
    for h in range(Hq):
        _, _, r = _oracle_rows(Q, K, V, S, k, "bf16", G, 0, h)
        for grad, mag in ((r.dq, r.abs_dq), (r.dK, r.abs_dK), (r.dV, r.abs_dV)):
            assert np.all(np.abs(grad) <= mag * (1 + 1e-12))
        assert np.all(r.out_dq >= 0) and np.all(r.out_dK >= 0)


def test_output_sensitivity_bounds_perturbed_outputs():
    """dq and dK given output rows off by at most eps stay within eps times
    the sensitivities; with one kept chunk per row and the error eps*sign(g)
    the bound is reached exactly."""
    B, Hq, Hkv, T, D, S, k = 1, 1, 1, 40, 5, 4, 2
    eps = 1e-3
    Q, K, V = rand_qkv(92, B, Hq, Hkv, T, D, "fp32")
    G = np.random.default_rng(93).standard_normal(Q.shape)
    L = O.landmarks(K, S, "fp32")
    _, sel, _, _ = O.prefill(Q, K, V, S, k, "fp32", L=L)
    pos = np.arange(T)
    args = (Q[0, 0], pos, K[0, 0], V[0, 0], L[0, 0], S)
    base = O.hsa_rows_backward(*args, sel[0, 0], G[0, 0])
    rng = np.random.default_rng(94)
    for _ in range(5):
        pert = O.hsa_rows_backward(*args, sel[0, 0], G[0, 0],
                                   delta_out=base.out + rng.uniform(-eps, eps, base.out.shape))
        assert np.all(np.abs(pert.dq - base.dq) <= eps * base.out_dq * (1 + 1e-9) + 1e-15)
        assert np.all(np.abs(pert.dK - base.dK) <= eps * base.out_dK * (1 + 1e-9) + 1e-15)
        assert np.array_equal(pert.dV, base.dV)
    # one kept chunk: the sign of the error chosen against g reaches the bound
    one = [[c for c in row if c >= 0][:1] for row in sel[0, 0]]
    b1 = O.hsa_rows_backward(*args, one, G[0, 0])
    p1 = O.hsa_rows_backward(*args, one, G[0, 0], delta_out=b1.out + eps * np.sign(G[0, 0]))
    np.testing.assert_allclose(np.abs(p1.dq - b1.dq), eps * b1.out_dq, rtol=1e-8, atol=1e-15)
    # dK reaches it on the chunks that a single row kept
    rows_of_chunk = {}
    for p, lst in enumerate(one):
        for c in lst:
            rows_of_chunk.setdefault(c, []).append(p)
    for c, rows in rows_of_chunk.items():
        if len(rows) == 1:
            t = slice(c * S, (c + 1) * S)
            np.testing.assert_allclose(np.abs(p1.dK[t] - b1.dK[t]), eps * b1.out_dK[t], rtol=1e-8, atol=1e-15)


def _bf16(x):
    return O.round_to_bf16(np.asarray(x, dtype=np.float64))


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def test_bf16_operand_evaluation_within_bounds():
    """A model of the kernels' arithmetic stays inside the tests' bounds:
    dV and dK contract bf16-rounded probabilities, dO and dlogit + ds/S
    (9e-3 of the magnitude sums); dq contracts dlogit as a bf16 head + tail
    pair and ds in fp32 (2e-4).  Products are summed in fp32.  This pins
    that the bounds are not tighter than the arithmetic they describe."""
    S, D, k = 8, 16, 3
    T = 8 * S + 5
    Q, K, V = rand_qkv(95, 1, 1, 1, T, D, "bf16")
    Gd = np.random.default_rng(96).standard_normal(Q.shape).astype(np.float32).astype(np.float64)
    L = O.landmarks(K, S, "bf16")
    _, sel, _, _ = O.prefill(Q, K, V, S, k, "bf16", L=L)
    ref = O.hsa_rows_backward(Q[0, 0], np.arange(T), K[0, 0], V[0, 0], L[0, 0], S, sel[0, 0], Gd[0, 0])
    sig = 1.0 / np.sqrt(D)
    dK = np.zeros((T, D), dtype=np.float32)
    dV = np.zeros((T, D), dtype=np.float32)
    dq = np.zeros((T, D), dtype=np.float32)
    for p in range(T):
        chunks = np.array([c for c in sel[0, 0, p] if c >= 0], dtype=np.int64)
        if chunks.size == 0:
            continue
        q, g = Q[0, 0, p], Gd[0, 0, p]
        s = L[0, 0, chunks] @ q * sig
        w = np.exp(s - s.max()); w /= w.sum()
        for j, c in enumerate(chunks):
            t = slice(c * S, (c + 1) * S)
            lg = K[0, 0, t] @ q * sig
            a = np.exp(lg - lg.max()); a /= a.sum()
            do = w[j] * g
            da = V[0, 0, t] @ do
            dl = a * (da - a @ da)
            ds = a @ da - w[j] * (ref.out[p] @ g)       # u - w delta
            dV[t] += _f32(np.outer(_bf16(a), _bf16(do))).astype(np.float32)
            dK[t] += _f32(np.outer(_bf16(dl + ds / S), q) * sig).astype(np.float32)
            head = _bf16(dl)
            tail = _bf16(dl - head)
            dq[p] += _f32((head @ K[0, 0, t] + tail @ K[0, 0, t] + ds * L[0, 0, c]) * sig).astype(np.float32)
    for name, got, want, mag, tol in (("dV", dV, ref.dV, ref.abs_dV, 9e-3), ("dK", dK, ref.dK, ref.abs_dK, 9e-3),
                                      ("dq", dq, ref.dq, ref.abs_dq, 2e-4)):
        err = np.abs(got.astype(np.float64) - want)
        assert np.all(err <= tol * mag + 1e-6), name
        assert err.max() > 0, name
        print(name, "worst error / magnitude sum", float((err / np.maximum(mag, 1e-300)).max()))


def test_planted_scale_mistakes_are_caught(monkeypatch):
    """Mistakes in the error scales (inflated, a term dropped, the 1/S
    missing) each fail the comparison with the brute-force term sums."""
    src = textwrap.dedent(inspect.getsource(O.hsa_rows_backward))
    mutations = {
        "dq scale inflated": ("abs_dq[r] = (", "abs_dq[r] = 10 * ("),
        "dK scale inflated": ("abs_dK[ti] += (", "abs_dK[ti] += 10 * ("),
        "dV scale inflated": ("abs_dV[ti] += (", "abs_dV[ti] += 2 * ("),
        "U term dropped": ("mag_l = a * (A + U[:, None])", "mag_l = a * A"),
        "delta term dropped": ("mag_s = U + w * (np.abs(out) @ np.abs(g))", "mag_s = U"),
        "dq sensitivity doubled": ("out_dq[r] = (w @ np.abs(Lg[chunks])) * g1 * sig",
                                   "out_dq[r] = 2 * (w @ np.abs(Lg[chunks])) * g1 * sig"),
        "dK sensitivity 1/S missing": ("* (g1 * sig / S)", "* (g1 * sig)"),
    }
    for name, (a, b) in mutations.items():
        assert a in src, name
        ns = dict(O.__dict__)
        exec(compile(src.replace(a, b), "<mutant>", "exec"), ns)
        with monkeypatch.context() as m:
            m.setattr(O, "hsa_rows_backward", ns["hsa_rows_backward"])
            with pytest.raises(AssertionError):
                test_backward_scales_equal_brute_term_sums(SCALE_CASES[1])
