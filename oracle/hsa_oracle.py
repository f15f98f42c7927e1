"""numpy float64 oracle of the Hierarchical Sparse Attention (HSA) forward layer.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What HSA computes (skill card "Every Token Counts 16m Context", sections
"Core Technique" and "Implementation"; abstract page "Every Token Counts:
Generalizing 16M Ultra-Long Context in Large Language Models"):

  1. split the keys into non-overlapping chunks of a fixed length S;
  2. give every chunk a landmark, read here as the plain mean of the chunk's
     keys (the card's learned encoder needs trained weights, so this layer
     fixes the mean pool);
  3. score every earlier landmark against the query (scaled dot product);
  4. keep the top-k chunks;
  5. attend inside each kept chunk with ordinary softmax attention;
  6. fuse the per-chunk outputs with weights taken from the retrieval scores
     (read as a softmax over the kept scores).

Readings of points the pages leave open (each is listed in the design doc):

* candidates of a query at position p are the complete chunks strictly before
  the query's own chunk: c < n_p = min(floor(p / S), Nc); a decode query sits at
  position T (just after its cache).  A query with no candidate outputs zero.
* GQA: query head h reads KV head g(h) = floor(h * Hkv / Hq) (contiguous groups);
  every query head scores and selects on its own.
* ties in the top-k go to the lower chunk index (total order: score
  descending, then index ascending); -0.0 and +0.0 compare equal.
* landmarks are rounded once, round-to-nearest-even, to the storage dtype.
* the in-chunk softmax and the fusion softmax both use the 1/sqrt(D) scale;
  each chunk output is normalised on its own.
* the output is float (fp64 here; fp32 on the GPU) even for bf16 inputs.
* near-tie adaptive budget (value-of-information router abstract): a row
  whose k-th best score beats its (k+1)-th by less than a threshold tau keeps
  its best 2k chunks instead of k (adaptive_keep_count).
* backward: the selection is held fixed (piecewise constant) and the
  landmark's rounding is taken as the identity (hsa_rows_backward).

Every input array handed to this module holds the exact values of the stored
tensors as float64 (bf16 and fp32 upcast exactly).  Parity unpinned: nothing.
Every function below is pinned by the CPU tests (brute force, closed forms,
special cases, invariants and a library-routine cross-check).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "f32_to_bf16_bits", "round_to_bf16", "round_to_f32",
    "round_to_dtype", "landmarks", "num_candidates", "scores_for_rows",
    "select_topk", "chunk_attention", "fuse", "hsa_rows", "prefill", "decode",
    "near_tie_info", "check_selection", "HSARowsResult", "adaptive_keep_count",
    "hsa_rows_adaptive", "hsa_rows_backward", "prefill_backward", "BackwardResult",
]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns: the 16 bits are the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, in ONE step.

    bf16 keeps 8 significant bits; float64 keeps 53.  The low 45 significand
    bits of the float64 are rounded away with round-half-even directly (no
    intermediate fp32, which would round twice).  Only the normal bf16 range
    is supported (|x| >= 2**-126 or x == 0, no overflow); anything else raises.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    if np.any((ax != 0) & (ax < 2.0 ** -126)) or np.any(ax >= 3.3895313892515355e38):
        raise ValueError("round_to_bf16: value outside the normal bf16 range")
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_bf16: non-finite input")
    u = x.view(np.uint64)
    drop = np.uint64(45)
    lsb = (u >> drop) & np.uint64(1)
    u = u + (np.uint64((1 << 44) - 1) + lsb)
    u = u & ~np.uint64((1 << 45) - 1)
    return u.view(np.float64)


def f32_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit pattern of values that are already exactly representable in bf16."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("f32_to_bf16_bits: value not representable")
    bits = f.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("f32_to_bf16_bits: value not representable in bf16")
    return (bits >> np.uint32(16)).astype(np.uint16)


def round_to_f32(x) -> np.ndarray:
    """Round float64 to the nearest fp32 value (numpy's cast is one RNE step)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round to the storage dtype; "fp64" keeps float64 (no rounding), which
    the gradient pins use so that the forward is smooth in its inputs."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "fp32":
        return round_to_f32(x)
    if dtype == "fp64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# step 1-2: chunks and landmarks
# ---------------------------------------------------------------------------

def landmarks(K: np.ndarray, S: int, dtype: str) -> np.ndarray:
    """Mean-pooled landmark of every complete chunk of S keys.

    Skill card "Every Token Counts 16m Context", section "Implementation"
    (landmark from mean pooling of the chunk's tokens) and "Core Technique"
    (non-overlapping fixed-length chunks).  K: [..., T, D] float64 holding the
    stored key values.  Returns [..., floor(T/S), D] float64 whose values are
    exactly representable in ``dtype``.  A trailing partial chunk gets no
    landmark.  The chunk sum is taken in float64 (exact for bf16 inputs of the
    magnitudes used here), divided by S and rounded once to ``dtype``.
    """
    K = np.asarray(K, dtype=np.float64)
    T, D = K.shape[-2], K.shape[-1]
    Nc = T // S
    chunks = K[..., : Nc * S, :].reshape(K.shape[:-2] + (Nc, S, D))
    mean = chunks.sum(axis=-2) / S
    return round_to_dtype(mean, dtype)


def num_candidates(p, S: int, Nc: int):
    """n_p = min(floor(p/S), Nc): complete chunks strictly before position p's chunk."""
    return np.minimum(np.asarray(p) // S, Nc)


# ---------------------------------------------------------------------------
# step 3-4: scoring and selection
# ---------------------------------------------------------------------------

def scores_for_rows(q: np.ndarray, L: np.ndarray, n: int) -> np.ndarray:
    """s[r, c] = (q[r] . L[c]) / sqrt(D) for c < n (card, "Implementation":
    similarity of the query with every landmark; read as the scaled dot product)."""
    D = q.shape[-1]
    return (q @ L[:n].T) * (1.0 / math.sqrt(D))


def select_topk(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the top-min(k, n) entries of each row of s under the order
    (score descending, chunk index ascending); rows of s are [R, n].

    Card "Implementation": keep the k best-scoring chunks.  The card's argsort
    expression leaves ties open; this layer breaks them toward the lower index.
    Returned in that order, shape [R, min(k, n)].
    """
    R, n = s.shape
    m = min(k, n)
    if m == 0:
        return np.zeros((R, 0), dtype=np.int64)
    s0 = s + 0.0  # -0.0 -> +0.0, so the two zeros tie
    idx = np.broadcast_to(np.arange(n), (R, n))
    order = np.lexsort((idx, -s0), axis=-1)
    return order[:, :m]


# ---------------------------------------------------------------------------
# step 5-6: in-chunk attention and fusion
# ---------------------------------------------------------------------------

def chunk_attention(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray) -> np.ndarray:
    """Softmax attention of query rows over the S tokens of one chunk each.

    Card "Implementation": attend to each selected chunk with standard
    attention.  q: [R, D]; Kc, Vc: [R, m, S, D] (the m chunks of each row).
    Returns o: [R, m, D]; each chunk output is normalised on its own, with the
    1/sqrt(D) scale and no mask (every token of a candidate chunk precedes q).
    """
    D = q.shape[-1]
    logits = np.einsum("rd,rmtd->rmt", q, Kc) * (1.0 / math.sqrt(D))
    logits = logits - logits.max(axis=-1, keepdims=True)
    a = np.exp(logits)
    a = a / a.sum(axis=-1, keepdims=True)
    return np.einsum("rmt,rmtd->rmd", a, Vc)


def fuse(s_sel: np.ndarray, o: np.ndarray) -> np.ndarray:
    """out = sum_c w_c o_c with w = softmax of the kept retrieval scores.

    Card "Core Technique" / "Implementation": results are fused with the
    retrieval scores as weights; read as a softmax over the kept scores (the
    scores already carry 1/sqrt(D)).  s_sel: [R, m]; o: [R, m, D].
    Rows with m == 0 give zeros.
    """
    R, m = s_sel.shape
    if m == 0:
        return np.zeros((R, o.shape[-1]))
    z = s_sel - s_sel.max(axis=-1, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=-1, keepdims=True)
    return np.einsum("rm,rmd->rd", w, o)


# ---------------------------------------------------------------------------
# the layer over a set of query rows sharing one KV head
# ---------------------------------------------------------------------------

@dataclass
class HSARowsResult:
    out: np.ndarray        # [R, D] float64
    sel_idx: np.ndarray    # [R, k] int64, -1 padded
    sel_score: np.ndarray  # [R, k] float64, -inf padded
    n: np.ndarray          # [R] number of candidates


def hsa_rows(q: np.ndarray, pos: np.ndarray, Kg: np.ndarray, Vg: np.ndarray,
             Lg: np.ndarray, S: int, k: int, sel_override=None) -> HSARowsResult:
    """HSA output of query rows q[r] at positions pos[r] against one KV head.

    q: [R, D]; Kg, Vg: [T, D]; Lg: [Nc', D] (landmarks of at least the needed
    chunks).  ``sel_override`` (list of index arrays, one per row) replaces the
    selection step, for checking a different but equally valid selection.
    """
    q = np.asarray(q, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    R, D = q.shape
    T = Kg.shape[0]
    Nc = T // S
    n_all = num_candidates(pos, S, Nc)
    out = np.zeros((R, D))
    sel_idx = np.full((R, k), -1, dtype=np.int64)
    sel_score = np.full((R, k), -np.inf)
    # rows with the same candidate count share the whole candidate set
    for n in np.unique(n_all):
        rows = np.nonzero(n_all == n)[0]
        if n == 0:
            continue
        s = scores_for_rows(q[rows], Lg, int(n))
        if sel_override is None:
            sel = select_topk(s, k)
        else:
            sel = np.stack([np.asarray(sel_override[r], dtype=np.int64) for r in rows])
        m = sel.shape[1]
        s_sel = np.take_along_axis(s, sel, axis=1)
        tok = sel[:, :, None] * S + np.arange(S)[None, None, :]  # [r, m, S]
        o = chunk_attention(q[rows], Kg[tok], Vg[tok])
        out[rows] = fuse(s_sel, o)
        sel_idx[rows, :m] = sel
        sel_score[rows, :m] = s_sel
    return HSARowsResult(out, sel_idx, sel_score, n_all)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Contiguous GQA grouping: g(h) = floor(h * Hkv / Hq)."""
    return (h * Hkv) // Hq


def prefill(Q, K, V, S: int, k: int, dtype: str, L=None, rows=None):
    """Causal HSA over a whole sequence.  Q: [B, Hq, T, D]; K, V: [B, Hkv, T, D].

    Query row p uses chunks strictly before its own.  ``rows`` optionally
    restricts the computation to a subset of positions (same for every head).
    Returns (out [B,Hq,R,D], sel_idx, sel_score, L).
    """
    Q = np.asarray(Q, dtype=np.float64)
    B, Hq, T, D = Q.shape
    Hkv = K.shape[1]
    if L is None:
        L = landmarks(K, S, dtype)
    pos = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    R = pos.shape[0]
    out = np.zeros((B, Hq, R, D))
    sel_idx = np.full((B, Hq, R, k), -1, dtype=np.int64)
    sel_score = np.full((B, Hq, R, k), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            r = hsa_rows(Q[b, h, pos], pos, K[b, g], V[b, g], L[b, g], S, k)
            out[b, h], sel_idx[b, h], sel_score[b, h] = r.out, r.sel_idx, r.sel_score
    return out, sel_idx, sel_score, L


def decode(q, Kc, Vc, L, S: int, k: int):
    """Single-token queries after their caches.  q: [B, Hq, D]; Kc, Vc: [B, Hkv, T, D];
    L: [B, Hkv, >= floor(T/S), D].  The query sits at position T."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, T = Kc.shape[1], Kc.shape[2]
    out = np.zeros((B, Hq, D))
    sel_idx = np.full((B, Hq, k), -1, dtype=np.int64)
    sel_score = np.full((B, Hq, k), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            r = hsa_rows(q[b, h][None], np.array([T]), Kc[b, g], Vc[b, g], L[b, g], S, k)
            out[b, h], sel_idx[b, h], sel_score[b, h] = r.out[0], r.sel_idx[0], r.sel_score[0]
    return out, sel_idx, sel_score


# ---------------------------------------------------------------------------
# near-tie adaptive budget
# ---------------------------------------------------------------------------

def adaptive_keep_count(s_sorted: np.ndarray, k: int, tau: float):
    """Kept count of one row under the near-tie adaptive budget, and its gap.

    Value-of-information router abstract (automata-index page): a row whose
    k-th and (k+1)-th best scores lie close together gets a doubled budget.
    Read here as a per-row threshold tau on that gap (in score units, the
    1/sqrt(D) scale included): s_sorted holds a
    row's candidate scores in selection order (score descending, index
    ascending), n = len(s_sorted).  With n > k the row keeps min(2k, n)
    chunks when s_sorted[k-1] - s_sorted[k] < tau and k otherwise; with
    n <= k no cut is made and all n are kept.  Strict comparison: tau = 0
    never doubles (a gap is never negative), tau = +inf always does.
    Returns (m, gap); gap is nan when n <= k.
    """
    n = len(s_sorted)
    if n <= k:
        return n, float("nan")
    gap = float(s_sorted[k - 1] - s_sorted[k])
    return (min(2 * k, n) if gap < tau else k), gap


def hsa_rows_adaptive(q: np.ndarray, pos: np.ndarray, Kg: np.ndarray, Vg: np.ndarray,
                      Lg: np.ndarray, S: int, k: int, tau: float):
    """HSA with the near-tie adaptive budget (adaptive_keep_count) for query
    rows q[r] at positions pos[r] against one KV head.

    Each row ranks its candidates as in select_topk, keeps its first m chunks
    (m from the gap rule) and then attends and fuses exactly as hsa_rows
    does over those m chunks.  Returns (result, doubled, gap): result is an
    HSARowsResult whose selection arrays have 2k columns (-1 / -inf
    padding), doubled[r] says whether row r kept more than k chunks, gap[r]
    is its k-th minus (k+1)-th score (nan when it has at most k candidates).
    """
    q = np.asarray(q, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    R = q.shape[0]
    Nc = Kg.shape[0] // S
    n_all = num_candidates(pos, S, Nc)
    keep = []
    doubled = np.zeros(R, dtype=bool)
    gap = np.full(R, np.nan)
    for r in range(R):
        n = int(n_all[r])
        if n == 0:
            keep.append(np.zeros(0, dtype=np.int64))
            continue
        s = scores_for_rows(q[r:r + 1], Lg, n)
        order = select_topk(s, 2 * k)[0]
        m, gap[r] = adaptive_keep_count(s[0, order], k, tau)
        doubled[r] = m > k
        keep.append(order[:m])
    out = np.zeros_like(q)
    sel_idx = np.full((R, 2 * k), -1, dtype=np.int64)
    sel_score = np.full((R, 2 * k), -np.inf)
    # rows keeping the same number of chunks go through hsa_rows together
    for m in sorted({len(c) for c in keep}):
        rows = np.array([r for r in range(R) if len(keep[r]) == m])
        res = hsa_rows(q[rows], pos[rows], Kg, Vg, Lg, S, 2 * k, sel_override=[keep[r] for r in rows])
        out[rows], sel_idx[rows], sel_score[rows] = res.out, res.sel_idx, res.sel_score
    return HSARowsResult(out, sel_idx, sel_score, n_all), doubled, gap


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------

@dataclass
class BackwardResult:
    dq: np.ndarray    # [R, D]
    dK: np.ndarray    # [T, D]
    dV: np.ndarray    # [T, D]
    # element-wise error scales of a lower-precision evaluation: sums of the
    # magnitudes of the terms each gradient entry adds up, every dot product
    # inside (da, u, delta) taken over absolute values, so that the scales
    # also bound the cancellation errors of dlogit and ds
    abs_dK: np.ndarray
    abs_dV: np.ndarray
    abs_dq: np.ndarray
    # how far an error in the rows' outputs, as the gradient uses them (in
    # delta = g.out), can move each entry per unit of max-abs output error
    out_dK: np.ndarray
    out_dq: np.ndarray
    # the rows' outputs under the given selection (the forward, fp64)
    out: np.ndarray


def hsa_rows_backward(q: np.ndarray, pos: np.ndarray, Kg: np.ndarray, Vg: np.ndarray, Lg: np.ndarray,
                      S: int, sel, dout: np.ndarray, delta_out=None) -> BackwardResult:
    """Gradients of the layer's output rows with respect to q, K and V.

    The forward (hsa_rows) for a row is: s_c = q.L_c/sqrt(D) over its kept
    chunks c (a fixed list sel[r]: the selection is piecewise constant, so
    no gradient flows through it), w = softmax(s), a_c = softmax over the
    chunk's tokens of q.k_t/sqrt(D), o_c = sum_t a_ct v_t, out = sum_c w_c o_c,
    with L_c the mean of the chunk's keys (its rounding to the storage dtype
    is taken as the identity, so every key of the chunk receives 1/S of the
    landmark's gradient).  The derivation is the chain rule on those steps
    (card, "Core Technique" / "Implementation"; training the landmarks and
    attention end to end is what the abstract describes):

      do_c = w_c g                         (g = dL/dout of the row)
      ds_c = w_c (g.o_c - g.out)           (softmax of the fusion weights)
      dv_t += a_ct do_c
      dlogit_ct = a_ct (do_c.v_t - do_c.o_c)
      dq = (sum_c sum_t dlogit_ct k_t + sum_c ds_c L_c) / sqrt(D)
      dk_t += (dlogit_ct q + ds_c q / S) / sqrt(D)    for t in chunk c

    q: [R, D] rows at positions pos; Kg, Vg: [T, D]; Lg: landmarks; sel: one
    index list per row (its kept chunks); dout: [R, D]; delta_out: [R, D]
    output rows to use in delta = g.out in place of the forward's own (the
    sensitivity pins perturb them).  Returns dq [R, D] and
    the rows' contributions dK, dV [T, D], plus the magnitude sums
    abs_dV = sum a_ct |do_c|,
    abs_dK = sum (a_ct (A_ct + U_c) + (U_c + w_c E) / S) |q| / sqrt(D),
    abs_dq = (sum a_ct (A_ct + U_c) |k_t| + sum (U_c + w_c E) |L_c|) / sqrt(D)
    with A_ct = |do_c| . |v_t|, U_c = sum_t a_ct A_ct and E = |g| . |out|:
    the sums of the absolute values of the elementary products each entry
    adds up once every dot product (da, u, delta) is opened, which bound the
    error of evaluating those products in lower precision (cancellation
    inside dlogit and ds included); and the output sensitivities
    out_dq = sum_c w_c |L_c| (sum_e |g_e|) / sqrt(D),
    out_dK = sum w_c (sum_e |g_e|) / S |q| / sqrt(D),
    the bound on how much an output row that is off by at most eps in every
    element moves dq and dK (through delta = g.out inside ds), per unit eps.
    """
    q = np.asarray(q, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    R, D = q.shape
    T = Kg.shape[0]
    sig = 1.0 / math.sqrt(D)
    dq = np.zeros((R, D))
    dK = np.zeros((T, D))
    dV = np.zeros((T, D))
    abs_dK = np.zeros((T, D))
    abs_dV = np.zeros((T, D))
    abs_dq = np.zeros((R, D))
    out_dK = np.zeros((T, D))
    out_dq = np.zeros((R, D))
    out_rows = np.zeros((R, D))
    for r in range(R):
        chunks = np.asarray(sel[r], dtype=np.int64)
        chunks = chunks[chunks >= 0]
        if chunks.size == 0:
            continue
        g = dout[r]
        tok = chunks[:, None] * S + np.arange(S)[None, :]     # [m, S]
        Kc, Vc = Kg[tok], Vg[tok]                             # [m, S, D]
        s = (Lg[chunks] @ q[r]) * sig                         # [m]
        w = np.exp(s - s.max())
        w /= w.sum()
        logits = (Kc @ q[r]) * sig                            # [m, S]
        a = np.exp(logits - logits.max(axis=1, keepdims=True))
        a /= a.sum(axis=1, keepdims=True)
        o = np.einsum("mt,mtd->md", a, Vc)                    # [m, D]
        out = w @ o
        out_rows[r] = out
        if delta_out is not None:
            out = np.asarray(delta_out[r], dtype=np.float64)
        do = w[:, None] * g[None, :]                          # [m, D]
        ds = w * (o @ g - out @ g)                            # [m]
        da = np.einsum("mtd,md->mt", Vc, do)                  # do_c . v_t
        dlogit = a * (da - np.sum(a * da, axis=1, keepdims=True))
        dq[r] = (np.einsum("mt,mtd->d", dlogit, Kc) + ds @ Lg[chunks]) * sig
        gk = (dlogit + ds[:, None] / S)                       # [m, S]
        ti = tok.reshape(-1)  # distinct tokens (the kept chunks are distinct)
        dK[ti] += (gk.reshape(-1, 1) * q[r][None, :]) * sig
        dV[ti] += (a[:, :, None] * do[:, None, :]).reshape(-1, D)
        A = np.einsum("mtd,md->mt", np.abs(Vc), np.abs(do))  # >= |da|
        U = np.sum(a * A, axis=1)                             # >= |u|
        mag_l = a * (A + U[:, None])                          # >= |dlogit|
        mag_s = U + w * (np.abs(out) @ np.abs(g))             # >= |ds|
        abs_dK[ti] += ((mag_l + mag_s[:, None] / S).reshape(-1, 1) * np.abs(q[r])[None, :]) * sig
        abs_dV[ti] += (a[:, :, None] * np.abs(do)[:, None, :]).reshape(-1, D)
        abs_dq[r] = (np.einsum("mt,mtd->d", mag_l, np.abs(Kc)) + mag_s @ np.abs(Lg[chunks])) * sig
        g1 = np.abs(g).sum()                                  # |g . err| <= eps * g1
        out_dq[r] = (w @ np.abs(Lg[chunks])) * g1 * sig
        out_dK[ti] += (np.repeat(w, S)[:, None] * np.abs(q[r])[None, :]) * (g1 * sig / S)
    return BackwardResult(dq, dK, dV, abs_dK, abs_dV, abs_dq, out_dK, out_dq, out_rows)


def prefill_backward(Q, K, V, S: int, k: int, dtype: str, dOut, sel_idx=None):
    """Gradients of the causal prefill with respect to Q [B,Hq,T,D] and K, V
    [B,Hkv,T,D] for the upstream gradient dOut [B,Hq,T,D].  The selection is
    the forward's (prefill) unless sel_idx [B,Hq,T,k'] is given.  Returns
    (dQ, dK, dV, abs_dK, abs_dV, abs_dQ)."""
    Q = np.asarray(Q, dtype=np.float64)
    B, Hq, T, D = Q.shape
    Hkv = K.shape[1]
    L = landmarks(K, S, dtype)
    if sel_idx is None:
        _, sel_idx, _, _ = prefill(Q, K, V, S, k, dtype, L=L)
    dQ = np.zeros_like(Q)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    aK = np.zeros(K.shape)
    aV = np.zeros(V.shape)
    aQ = np.zeros_like(Q)
    pos = np.arange(T)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            r = hsa_rows_backward(Q[b, h], pos, K[b, g], V[b, g], L[b, g], S, sel_idx[b, h], dOut[b, h])
            dQ[b, h] = r.dq
            dK[b, g] += r.dK
            dV[b, g] += r.dV
            aK[b, g] += r.abs_dK
            aV[b, g] += r.abs_dV
            aQ[b, h] = r.abs_dq
    return dQ, dK, dV, aK, aV, aQ


# ---------------------------------------------------------------------------
# near-tie acceptance for a selection computed in lower precision
# ---------------------------------------------------------------------------

def near_tie_info(q: np.ndarray, Lg: np.ndarray, n: int, k: int, rel: float = 1e-5):
    """For one query row: (is_near_tie, band, s) where s are the fp64 scores of
    the n candidates.

    The cut between the m-th and (m+1)-th best (m = min(k, n)) is a near tie
    when their gap is below rel * mu, mu = max(|s_m|, |s_m+1|, A_m, A_m+1) and
    A_c = sum_d |q_d| |L_cd| / sqrt(D) bounds the rounding error of a
    lower-precision dot product (a plain relative test is ill-posed near 0).
    The block-sparse router page (value-of-information router abstract) names
    this k-th versus (k+1)-th gap.
    """
    D = q.shape[-1]
    s = (Lg[:n] @ q) / math.sqrt(D)
    m = min(k, n)
    if m >= n:
        return False, 0.0, s
    order = np.lexsort((np.arange(n), -(s + 0.0)))
    a, b = order[m - 1], order[m]
    A = (np.abs(Lg[:n]) @ np.abs(q)) / math.sqrt(D)
    mu = max(abs(s[a]), abs(s[b]), A[a], A[b])
    band = rel * mu
    return bool(s[a] - s[b] < band), band, s


def check_selection(gpu_sel, q, Lg, n: int, k: int, rel: float = 1e-5):
    """Accept or reject a GPU selection for one row (indices, -1 padded).

    Returns (ok, exact_match, message).  Non-near-tie rows must match the
    oracle's set exactly; near-tie rows must be a top-m set up to the band.
    """
    g = [int(c) for c in gpu_sel if int(c) >= 0]
    m = min(k, n)
    pad = [int(c) for c in gpu_sel[len(g):]]
    if len(g) != m or any(c != -1 for c in pad):
        return False, False, f"expected {m} indices then -1 padding, got {list(gpu_sel)}"
    if len(set(g)) != m or any(c < 0 or c >= n for c in g):
        return False, False, f"invalid indices {g} for n={n}"
    if m == 0:
        return True, True, ""
    tie, band, s = near_tie_info(q, Lg, n, k, rel)
    ref = select_topk(s[None, :], k)[0]
    if set(ref.tolist()) == set(g):
        return True, True, ""
    if not tie:
        return False, False, f"selection {sorted(g)} != oracle {sorted(ref.tolist())}"
    inside = min(s[c] for c in g)
    outside = [s[c] for c in range(n) if c not in set(g)]
    ok = (not outside) or inside >= max(outside) - band
    return ok, False, "" if ok else "near-tie selection outside the band"
