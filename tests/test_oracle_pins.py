"""Pins of the CPU oracle against things other than itself.

Each test checks ``oracle.hsa_oracle`` against brute force (``oracle.brute``,
exact rationals), a closed form, a library routine (torch's attention and
bf16 cast), a hand-derived example or an invariant of the method.  The
mutation tests at the end plant plausible mistakes in the oracle and check
that these pins catch them.
"""
import math
import zlib

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import hsa_oracle as O


def rng(seed):
    return np.random.default_rng(seed)


def bf16_values(a):
    """Round fp64 samples to exact bf16 values (input generation for tests)."""
    t = torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def rand_qkv(seed, B, Hq, Hkv, T, D, dtype="fp32", scale=1.0):
    r = rng(seed)
    Q = r.standard_normal((B, Hq, T, D)) * scale
    K = r.standard_normal((B, Hkv, T, D)) * scale
    V = r.standard_normal((B, Hkv, T, D)) * scale
    if dtype == "bf16":
        return bf16_values(Q), bf16_values(K), bf16_values(V)
    f = lambda x: x.astype(np.float32).astype(np.float64)
    return f(Q), f(K), f(V)


# ---------------------------------------------------------------- rounding

def test_round_bf16_hand_cases():
    one = 1.0
    assert O.round_to_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0            # tie -> even
    assert O.round_to_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6  # tie -> even (up)
    # just above the halfway point: one rounding goes up; rounding via fp32 first would tie to 1.0
    x = one + 2.0 ** -8 + 2.0 ** -30
    assert O.round_to_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert O.round_to_bf16(np.array([-x]))[0] == -(1.0 + 2.0 ** -7)
    assert O.round_to_bf16(np.array([0.0]))[0] == 0.0
    # carry into the exponent
    assert O.round_to_bf16(np.array([2.0 - 2.0 ** -9]))[0] == 2.0


def test_round_bf16_matches_torch_cast_on_fp32_values():
    """For fp32-representable inputs one RNE step from fp64 equals torch's fp32->bf16 cast."""
    x = rng(1).standard_normal(200_000).astype(np.float32)
    x[:1000] = (np.arange(1000, dtype=np.float32) + 0.5) * np.float32(2.0 ** -7) + 1  # many exact ties
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(ref, got)
    bits = O.f32_to_bf16_bits(got)
    assert np.array_equal(bits, torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(O.bf16_bits_to_f64(bits), got)


def test_round_bf16_matches_exact_rational_rounding():
    vals = rng(2).standard_normal(3000) * 10.0 ** rng(3).integers(-8, 8, 3000)
    got = O.round_to_bf16(vals)
    from fractions import Fraction
    ref = [float(brute.round_fraction(Fraction(v), 8)) for v in vals]
    assert np.array_equal(got, np.array(ref))


# ---------------------------------------------------------------- landmarks

@pytest.mark.parametrize("S", [1, 2, 4, 8, 64])
def test_landmarks_bf16_bit_exact_vs_fractions(S):
    _, K, _ = rand_qkv(4 + S, 1, 1, 2, 3 * S + 1, 8, dtype="bf16")
    L = O.landmarks(K, S, "bf16")
    Nc = (3 * S + 1) // S
    assert L.shape == (1, 2, Nc, 8)
    for g in range(2):
        for c in range(Nc):
            ref = brute.landmark(K[0, g, c * S:(c + 1) * S].tolist(), "bf16")
            assert np.array_equal(L[0, g, c], np.array(ref))


def test_landmarks_constant_chunk_and_S1():
    _, K, _ = rand_qkv(5, 1, 1, 1, 16, 8, dtype="bf16")
    K[0, 0, 4:8] = K[0, 0, 4]
    L = O.landmarks(K, 4, "bf16")
    assert np.array_equal(L[0, 0, 1], K[0, 0, 4])
    assert np.array_equal(O.landmarks(K, 1, "bf16"), K)
    assert np.array_equal(O.landmarks(K, 1, "fp32"), K)


def test_landmarks_fp32_within_one_ulp_of_exact():
    _, K, _ = rand_qkv(6, 1, 1, 1, 5 * 64, 4, dtype="fp32")
    L = O.landmarks(K, 64, "fp32")
    for c in range(5):
        ref = np.array(brute.landmark(K[0, 0, c * 64:(c + 1) * 64].tolist(), "fp32"))
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(L[0, 0, c] - ref) <= ulp)


# ---------------------------------------------------------------- brute force

CASES = [
    # B, Hq, Hkv, T, D, S, k, dtype
    (1, 1, 1, 12, 4, 2, 1, "fp32"),
    (1, 2, 1, 17, 4, 3, 2, "fp32"),
    (2, 4, 2, 24, 8, 4, 3, "bf16"),
    (1, 2, 2, 20, 4, 1, 5, "bf16"),
    (1, 4, 1, 48, 8, 8, 2, "bf16"),
    (2, 2, 1, 30, 4, 4, 100, "fp32"),  # k > Nc
]


@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_brute_force(case):
    B, Hq, Hkv, T, D, S, k, dtype = case
    Q, K, V = rand_qkv(zlib.crc32(repr(case).encode()) % 1000, B, Hq, Hkv, T, D, dtype)
    out, sel, sc, L = O.prefill(Q, K, V, S, k, dtype)
    bo, bs, bc = brute.prefill(Q.tolist(), K.tolist(), V.tolist(), S, k, dtype)
    for b in range(B):
        for h in range(Hq):
            for p in range(T):
                m = len(bs[b][h][p])
                assert list(sel[b, h, p, :m]) == bs[b][h][p]
                assert np.all(sel[b, h, p, m:] == -1)
                np.testing.assert_allclose(sc[b, h, p, :m], bc[b][h][p], rtol=0, atol=1e-12)
                np.testing.assert_allclose(out[b, h, p], bo[b][h][p], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def torch_attention(q, k, v, mask=None):
    """Library attention (fp64, CPU) used as the textbook reference."""
    tq = torch.from_numpy(q)[None, None]
    tk = torch.from_numpy(k)[None, None]
    tv = torch.from_numpy(v)[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m)[0, 0].numpy()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_closed_form_chunk1_is_dense_causal_attention_without_diagonal(dtype):
    T, D = 40, 8
    Q, K, V = rand_qkv(7, 1, 2, 1, T, D, dtype)
    out, _, _, _ = O.prefill(Q, K, V, 1, T + 5, dtype)
    mask = np.tril(np.ones((T, T), dtype=bool), k=-1)  # j < p only
    for h in range(2):
        ref = torch_attention(Q[0, h, 1:], K[0, 0], V[0, 0], mask[1:])
        np.testing.assert_allclose(out[0, h, 1:], ref, rtol=0, atol=1e-12)
        assert np.all(out[0, h, 0] == 0)


@pytest.mark.parametrize("S,k", [(4, 1), (8, 3), (16, 16)])
def test_two_chunk_case_is_plain_attention_over_chunk0(S, k):
    D = 8
    Q, K, V = rand_qkv(8 + S, 1, 1, 1, 2 * S, D, "bf16")
    out, sel, _, _ = O.prefill(Q, K, V, S, k, "bf16")
    assert np.all(out[0, 0, :S] == 0) and np.all(sel[0, 0, :S] == -1)
    ref = torch_attention(Q[0, 0, S:], K[0, 0, :S], V[0, 0, :S])
    np.testing.assert_allclose(out[0, 0, S:], ref, rtol=0, atol=1e-12)
    assert np.all(sel[0, 0, S:, 0] == 0)


def test_hand_worked_example():
    """D=2, S=2: landmarks, selection and fusion worked out by hand."""
    K = np.array([[1, 0], [1, 0], [0, 1], [0, 1], [2, 2], [0, 0]], dtype=np.float64)
    V = np.array([[1, 2], [3, 4], [5, 6], [7, 8], [9, 9], [9, 9]], dtype=np.float64)
    q = np.array([[2.0, 0.0]])
    L = O.landmarks(K[None, None], 2, "fp32")[0, 0]
    assert np.array_equal(L, np.array([[1, 0], [0, 1], [1, 1]], dtype=np.float64))
    r1 = O.hsa_rows(q, np.array([4]), K, V, L, 2, 1)
    # scores: chunk0 = 2/sqrt2, chunk1 = 0; keys inside each chunk are equal -> uniform softmax
    assert list(r1.sel_idx[0]) == [0]
    np.testing.assert_allclose(r1.out[0], [2.0, 3.0], atol=1e-15)
    r2 = O.hsa_rows(q, np.array([4]), K, V, L, 2, 2)
    w0 = math.exp(math.sqrt(2)) / (math.exp(math.sqrt(2)) + 1)
    np.testing.assert_allclose(r2.out[0], [w0 * 2 + (1 - w0) * 6, w0 * 3 + (1 - w0) * 7], atol=1e-14)
    np.testing.assert_allclose(r2.sel_score[0], [math.sqrt(2), 0.0], atol=1e-15)
    # position 3 sits in chunk 1: only chunk 0 is a candidate
    r3 = O.hsa_rows(q, np.array([3]), K, V, L, 2, 2)
    assert list(r3.sel_idx[0]) == [0, -1]


# ---------------------------------------------------------------- special cases

def test_k1_output_is_best_chunk_attention():
    S, D, T = 4, 8, 32
    Q, K, V = rand_qkv(9, 1, 1, 1, T, D, "bf16")
    out, sel, _, L = O.prefill(Q, K, V, S, 1, "bf16")
    for p in range(S, T):
        n = p // S
        s = L[0, 0, :n] @ Q[0, 0, p]
        c = int(np.argmax(s))
        assert sel[0, 0, p, 0] == c
        ref = torch_attention(Q[0, 0, p][None], K[0, 0, c * S:(c + 1) * S], V[0, 0, c * S:(c + 1) * S])
        np.testing.assert_allclose(out[0, 0, p], ref[0], atol=1e-12)


def test_no_candidates_gives_zero_and_padding():
    Q, K, V = rand_qkv(10, 1, 2, 1, 7, 4, "fp32")
    out, sel, sc, _ = O.prefill(Q, K, V, 8, 3, "fp32")  # T < S: no complete chunk at all
    assert np.all(out == 0) and np.all(sel == -1) and np.all(np.isneginf(sc))


def test_gqa_replication_matches_mha():
    B, Hq, Hkv, T, D, S, k = 1, 8, 2, 40, 8, 4, 3
    Q, K, V = rand_qkv(11, B, Hq, Hkv, T, D, "bf16")
    out, sel, _, _ = O.prefill(Q, K, V, S, k, "bf16")
    rep = [O.kv_head_of(h, Hq, Hkv) for h in range(Hq)]
    assert rep == [0, 0, 0, 0, 1, 1, 1, 1]
    out2, sel2, _, _ = O.prefill(Q, K[:, rep], V[:, rep], S, k, "bf16")
    assert np.array_equal(sel, sel2)
    np.testing.assert_allclose(out, out2, atol=1e-12)


def test_duplicate_chunk_keeps_lower_index():
    S, D, T = 4, 8, 40
    Q, K, V = rand_qkv(12, 1, 1, 1, T, D, "bf16")
    K[0, 0, 20:24] = K[0, 0, 4:8]  # chunk 5 := chunk 1
    V[0, 0, 20:24] = V[0, 0, 4:8]
    out, sel, sc, L = O.prefill(Q, K, V, S, 1, "bf16")
    assert np.array_equal(L[0, 0, 1], L[0, 0, 5])
    hits = 0
    for p in range(24, T):
        s = L[0, 0, :p // S] @ Q[0, 0, p]
        if np.argmax(s) in (1, 5) or s[1] == s.max():
            hits += 1
            assert sel[0, 0, p, 0] == 1
        assert sel[0, 0, p, 0] != 5
    # force ties with negative zero as well
    s = np.array([[0.0, -0.0, 0.0]])
    assert list(O.select_topk(s, 2)[0]) == [0, 1]
    assert list(O.select_topk(np.array([[-0.0, 0.0, 1.0]]), 2)[0]) == [2, 0]


# ---------------------------------------------------------------- invariants

def test_convexity_scaling_and_shift():
    S, D, T, k = 4, 8, 48, 3
    Q, K, V = rand_qkv(13, 1, 2, 1, T, D, "fp32")
    out, sel, _, L = O.prefill(Q, K, V, S, k, "fp32")
    for h in range(2):
        for p in range(S, T):
            toks = np.concatenate([np.arange(c * S, c * S + S) for c in sel[0, h, p] if c >= 0])
            lo, hi = V[0, 0, toks].min(axis=0), V[0, 0, toks].max(axis=0)
            assert np.all(out[0, h, p] >= lo - 1e-12) and np.all(out[0, h, p] <= hi + 1e-12)
    out2, sel2, _, _ = O.prefill(Q, K, 2.5 * V, S, k, "fp32", L=L)
    np.testing.assert_allclose(out2, 2.5 * out, atol=1e-12)
    b = rng(14).standard_normal(D)
    out3, _, _, _ = O.prefill(Q, K, V + b, S, k, "fp32", L=L)
    np.testing.assert_allclose(out3[:, :, S:], out[:, :, S:] + b, atol=1e-12)
    assert np.all(out3[:, :, :S] == 0)


def test_position_independence_under_chunk_permutation():
    """Retrieval depends on landmark similarity, not on absolute position
    (card, "Core Technique", length generalisation)."""
    S, D, k = 4, 8, 3
    n = 6
    T = (n + 1) * S
    Q, K, V = rand_qkv(15, 1, 1, 1, T, D, "bf16")
    perm = rng(16).permutation(n)
    tok = np.concatenate([np.arange(c * S, c * S + S) for c in perm] + [np.arange(n * S, T)])
    K2, V2 = K[:, :, tok], V[:, :, tok]
    rows = np.arange(n * S, T)  # queries in the last chunk see all n candidates
    out, sel, _, _ = O.prefill(Q, K, V, S, k, "bf16", rows=rows)
    out2, sel2, _, _ = O.prefill(Q, K2, V2, S, k, "bf16", rows=rows)
    # new chunk i holds original chunk perm[i]
    assert np.array_equal(sel, perm[sel2])
    np.testing.assert_allclose(out, out2, atol=1e-12)


def test_prefill_row_equals_decode():
    S, D, T, k = 4, 8, 44, 3
    Q, K, V = rand_qkv(17, 2, 4, 2, T, D, "bf16")
    out, sel, sc, L = O.prefill(Q, K, V, S, k, "bf16")
    for p in [0, 3, 4, 9, 23, 43]:
        Lp = O.landmarks(K[:, :, :p], S, "bf16")
        o2, s2, c2 = O.decode(Q[:, :, p], K[:, :, :p], V[:, :, :p], Lp, S, k)
        assert np.array_equal(s2, sel[:, :, p])
        np.testing.assert_allclose(o2, out[:, :, p], atol=1e-12)


# ---------------------------------------------------------------- acceptance rule

def test_check_selection_rules():
    r = rng(18)
    D, n, k = 16, 40, 5
    q = r.standard_normal(D)
    L = r.standard_normal((n, D))
    ok, exact, _ = O.check_selection(list(O.select_topk(((L @ q) / 4.0)[None], k)[0]), q, L, n, k)
    assert ok and exact
    s = (L @ q) / 4.0
    order = np.lexsort((np.arange(n), -s))
    bad = list(order[:k - 1]) + [int(order[k + 3])]
    assert not O.check_selection(bad, q, L, n, k)[0]
    assert not O.check_selection(list(order[:k - 1]) + [int(order[0])], q, L, n, k)[0]  # duplicate
    assert not O.check_selection(list(order[:k]) + [-1], q, L, n, k + 1)[0]  # too few
    # make the k-th and (k+1)-th a near tie: nudge landmark order[k] toward order[k-1]
    L2 = L.copy()
    a, b = order[k - 1], order[k]
    L2[b] = L2[a] * (1 - 1e-9)
    s2 = (L2 @ q) / 4.0
    o2 = np.lexsort((np.arange(n), -s2))
    tie, band, _ = O.near_tie_info(q, L2, n, k)
    assert tie
    swapped = list(o2[:k - 1]) + [int(o2[k])]
    ok, exact, _ = O.check_selection(swapped, q, L2, n, k)
    assert ok and not exact


# ---------------------------------------------------------------- mutation tests

def _pins_that_must_fail(monkeypatch, name, bad):
    monkeypatch.setattr(O, name, bad)
    failures = 0
    for fn in (lambda: test_oracle_matches_brute_force(CASES[2]),
               lambda: test_two_chunk_case_is_plain_attention_over_chunk0(8, 3),
               lambda: test_closed_form_chunk1_is_dense_causal_attention_without_diagonal("fp32"),
               test_hand_worked_example):
        try:
            fn()
        except AssertionError:
            failures += 1
    return failures


def test_planted_mistakes_are_caught(monkeypatch):
    good_attn, good_fuse, good_sel, good_lm = O.chunk_attention, O.fuse, O.select_topk, O.landmarks

    def attn_no_scale(q, Kc, Vc):
        return good_attn(q * math.sqrt(q.shape[-1]), Kc, Vc)

    def fuse_raw_scores(s_sel, o):  # the literal "sum of score * output" reading
        return np.einsum("rm,rmd->rd", s_sel, o) if s_sel.shape[1] else good_fuse(s_sel, o)

    def sel_reversed(s, k):
        return good_sel(-s, k)

    def lm_first_key(K, S, dtype):
        Nc = K.shape[-2] // S
        return O.round_to_dtype(K[..., : Nc * S: S, :], dtype)

    for name, bad in [("chunk_attention", attn_no_scale), ("fuse", fuse_raw_scores),
                      ("select_topk", sel_reversed), ("landmarks", lm_first_key)]:
        with monkeypatch.context() as m:
            assert _pins_that_must_fail(m, name, bad) >= 1, name
    assert O.chunk_attention is good_attn and O.landmarks is good_lm
