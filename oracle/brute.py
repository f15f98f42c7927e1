"""Pure-Python brute-force HSA forward layer for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Written independently of ``hsa_oracle`` (no numpy,
no shared helpers) so that the two pin each other.  Inputs are nested Python
lists of floats holding the stored values exactly.

Follows the skill card "Every Token Counts 16m Context", sections "Core
Technique" and "Implementation", one query at a time:
landmark = exact mean of the chunk's keys (Fraction arithmetic) rounded once,
half-to-even, to the storage precision; scores = exact dot products (the
common positive 1/sqrt(D) factor cannot change the order, so the selection is
decided on exact rationals); top-k under (score desc, index asc); softmax
attention inside each kept chunk; softmax fusion over the kept scores.
"""
from __future__ import annotations

import math
from fractions import Fraction

PRECISION_BITS = {"bf16": 8, "fp32": 24}


def round_fraction(x: Fraction, bits: int) -> Fraction:
    """Round a rational to the nearest binary float with ``bits`` significant
    bits, ties to even (normal range only)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = -x if x < 0 else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # adjust so that 2**e <= a < 2**(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - bits + 1)
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def landmark(chunk_keys, dtype: str):
    """Mean of a chunk's keys, rounded once to the storage precision."""
    S = len(chunk_keys)
    D = len(chunk_keys[0])
    out = []
    for d in range(D):
        tot = sum((Fraction(row[d]) for row in chunk_keys), Fraction(0))
        out.append(float(round_fraction(tot / S, PRECISION_BITS[dtype])))
    return out


def _softmax(xs):
    mx = max(xs)
    es = [math.exp(x - mx) for x in xs]
    tot = sum(es)
    return [e / tot for e in es]


def hsa_query(q, p: int, K, V, S: int, k: int, dtype: str):
    """Output, selected chunks (in order) and their scores for the query row q
    at position p, against one KV head (K, V: lists of T rows)."""
    D = len(q)
    T = len(K)
    Nc = T // S
    n = min(p // S, Nc)
    if n == 0:
        return [0.0] * D, [], []
    exact = _exact_scores(q, K, S, n, dtype)
    order = sorted(range(n), key=lambda c: (-exact[c], c))
    sel = order[:min(k, n)]
    return _attend_and_fuse(q, sel, exact, K, V, S)


def hsa_query_adaptive(q, p: int, K, V, S: int, k: int, tau: float, dtype: str):
    """As hsa_query, with the near-tie adaptive budget of the value-of-
    information router abstract (automata-index page): when the query has
    more than k candidates and its k-th best score exceeds its (k+1)-th by
    less than tau (scores scaled by 1/sqrt(D)), it keeps its best 2k chunks
    (or all, if fewer) instead of k.  The gap is taken from the exact dot
    products.  Returns (out, sel, scores, doubled)."""
    D = len(q)
    n = min(p // S, len(K) // S)
    if n == 0:
        return [0.0] * D, [], [], False
    exact = _exact_scores(q, K, S, n, dtype)
    order = sorted(range(n), key=lambda c: (-exact[c], c))
    m = min(k, n)
    if n > k and float(exact[order[k - 1]] - exact[order[k]]) / math.sqrt(D) < tau:
        m = min(2 * k, n)
    out, sel, scores = _attend_and_fuse(q, order[:m], exact, K, V, S)
    return out, sel, scores, m > k


def _exact_scores(q, K, S: int, n: int, dtype: str):
    """Exact (unscaled) q . landmark for the first n chunks."""
    D = len(q)
    lms = [landmark(K[c * S:(c + 1) * S], dtype) for c in range(n)]
    return [sum((Fraction(q[d]) * Fraction(lm[d]) for d in range(D)), Fraction(0)) for lm in lms]


def _attend_and_fuse(q, sel, exact, K, V, S: int):
    """Softmax attention inside every chunk of sel, fused by a softmax over
    the kept scaled scores."""
    D = len(q)
    scale = 1.0 / math.sqrt(D)
    scores = [float(exact[c]) * scale for c in sel]
    outs = []
    for c in sel:
        logits = [sum(q[d] * K[t][d] for d in range(D)) * scale for t in range(c * S, c * S + S)]
        a = _softmax(logits)
        outs.append([sum(a[i] * V[c * S + i][d] for i in range(S)) for d in range(D)])
    w = _softmax(scores)
    out = [sum(w[j] * outs[j][d] for j in range(len(sel))) for d in range(D)]
    return out, sel, scores


def prefill(Q, K, V, S: int, k: int, dtype: str):
    """Q: [B][Hq][T][D]; K, V: [B][Hkv][T][D] nested lists.
    Returns (out, sel, scores) nested as [B][Hq][T]."""
    B, Hq, T = len(Q), len(Q[0]), len(Q[0][0])
    Hkv = len(K[0])
    outs, sels, scs = [], [], []
    for b in range(B):
        ob, sb, cb = [], [], []
        for h in range(Hq):
            g = (h * Hkv) // Hq
            oh, sh, ch = [], [], []
            for p in range(T):
                o, s, c = hsa_query(Q[b][h][p], p, K[b][g], V[b][g], S, k, dtype)
                oh.append(o)
                sh.append(s)
                ch.append(c)
            ob.append(oh)
            sb.append(sh)
            cb.append(ch)
        outs.append(ob)
        sels.append(sb)
        scs.append(cb)
    return outs, sels, scs


# ---------------------------------------------------------------------------
# backward of one query row, term by term
# ---------------------------------------------------------------------------

def backward_query(q, K, V, S: int, sel, g, dtype: str):
    """Gradient of one query row's output with respect to q, K and V, written
    as explicit sums of elementary products (pure Python, no shared helpers).

    Forward of the row (card "Core Technique" / "Implementation"): landmark
    L_c = mean of chunk c's keys (stored rounded; the rounding is taken as
    the identity for the gradient, so each of the chunk's keys receives 1/S
    of the landmark's gradient), s_c = q.L_c/sqrt(D) over the kept chunks
    sel (fixed: selection is piecewise constant), w = softmax(s), in-chunk
    probabilities a_ct = softmax_t(q.k_t/sqrt(D)), o_c = sum_t a_ct v_t,
    out = sum_c w_c o_c.  g is dLoss/dout of the row.

    Each gradient entry is the sum of a list of products; the chain rule
    gives, with every dot product opened into its D products:
      dv_te   <- a_ct w_c g_e
      dlogit_ct = sum_e a_ct w_c g_e v_te - sum_t' sum_e a_ct a_ct' w_c g_e v_t'e
      ds_c      = sum_t sum_e a_ct w_c g_e v_te - sum_e w_c g_e out_e
      dq_d    = (sum_c sum_t dlogit_ct k_td + sum_c ds_c L_cd) / sqrt(D)
      dk_td  <- (dlogit_ct + ds_c / S) q_d / sqrt(D)
    For every entry this returns three numbers: the sum of the products (the
    gradient), the sum of their absolute values (the magnitude sum that
    bounds the error of a lower-precision evaluation of the same products),
    and the sum of |product / out_e| over the products holding a factor
    out_e (how much an error in the row's output, as used for the
    gradient, can move the entry per unit of max-abs output error).

    Returns (dq, dK, dV): dq is a list of D triples (value, magnitude,
    out_sensitivity); dK and dV map a token index to such a list.
    """
    D = len(q)
    sig = 1.0 / math.sqrt(D)
    sel = [c for c in sel if c >= 0]
    zero = [(0.0, 0.0, 0.0)] * D
    if not sel:
        return list(zero), {}, {}
    lms = {c: landmark(K[c * S:(c + 1) * S], dtype) for c in sel}
    s = [sum(q[d] * lms[c][d] for d in range(D)) * sig for c in sel]
    w = _softmax(s)
    a, o = {}, {}
    for c in sel:
        logits = [sum(q[d] * K[t][d] for d in range(D)) * sig for t in range(c * S, c * S + S)]
        pr = _softmax(logits)
        for i in range(S):
            a[c, c * S + i] = pr[i]
        o[c] = [sum(pr[i] * V[c * S + i][e] for i in range(S)) for e in range(D)]
    out = [sum(w[j] * o[c][e] for j, c in enumerate(sel)) for e in range(D)]

    # the products of dlogit_ct and of ds_c, each as (value, |value|, |value / out_e| if it holds out_e)
    def dlogit_terms(j, c, t):
        terms = []
        for e in range(D):
            terms.append(a[c, t] * w[j] * g[e] * V[t][e])
        for t2 in range(c * S, c * S + S):
            for e in range(D):
                terms.append(-a[c, t] * a[c, t2] * w[j] * g[e] * V[t2][e])
        return [(x, abs(x), 0.0) for x in terms]

    def ds_terms(j, c):
        terms = []
        for t in range(c * S, c * S + S):
            for e in range(D):
                x = a[c, t] * w[j] * g[e] * V[t][e]
                terms.append((x, abs(x), 0.0))
        for e in range(D):
            x = -w[j] * g[e] * out[e]
            terms.append((x, abs(x), abs(w[j] * g[e])))
        return terms

    def scaled(terms, f):
        return [(x * f, m * abs(f), o_ * abs(f)) for x, m, o_ in terms]

    def total(terms):
        return (sum(x for x, _, _ in terms), sum(m for _, m, _ in terms), sum(o_ for _, _, o_ in terms))

    dq = []
    for d in range(D):
        terms = []
        for j, c in enumerate(sel):
            for t in range(c * S, c * S + S):
                terms += scaled(dlogit_terms(j, c, t), K[t][d] * sig)
            terms += scaled(ds_terms(j, c), lms[c][d] * sig)
        dq.append(total(terms))
    dK, dV = {}, {}
    for j, c in enumerate(sel):
        ds = ds_terms(j, c)
        for t in range(c * S, c * S + S):
            dl = dlogit_terms(j, c, t)
            dK[t] = [total(scaled(dl, q[d] * sig) + scaled(ds, q[d] * sig / S)) for d in range(D)]
            dV[t] = [(a[c, t] * w[j] * g[e], abs(a[c, t] * w[j] * g[e]), 0.0) for e in range(D)]
    return dq, dK, dV
