"""GPU parity of decoding with the near-tie adaptive budget
(hsa_forward_decode_adaptive; value-of-information router abstract: the
k-th versus (k+1)-th score gap decides whether a query head keeps 2k chunks).

Each (query, head) row is checked against the oracle's adaptive rule: its
kept count must be the oracle's unless the oracle's fp64 gap lies within the
fp32 score error of the threshold (then either count is valid), its kept set
must be a valid top-m set for that count, and its output must match the
oracle's for that set.  The limits are checked bit for bit against the plain
decode: threshold 0 gives hsa_forward_decode with k, +inf gives it with 2k,
and any threshold gives every row exactly one of the two."""
import math

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs
from oracle import hsa_oracle as O
from tests.gpu_util import TOL, Mismatch, check_rows_adaptive, f64, new_stats

pytestmark = pytest.mark.gpu
S = 64

CASES = [
    # B, Hq, Hkv, T, D, k, dtype, lengths (None: fixed length T)
    (4, 16, 4, 64 * 3000, 128, 16, "bf16", None),
    (3, 8, 2, 64 * 500 + 17, 64, 8, "fp32", None),
    (2, 8, 1, 64 * 5000, 128, 32, "bf16", None),
    (4, 8, 2, 64 * 900, 128, 16, "bf16", [64 * 900, 20, 64 * 16 + 3, 64 * 451]),
]


def oracle_gaps(q, Kc, Lc, lens, k):
    """fp64 k-th minus (k+1)-th score of every (b, h) row (nan: <= k candidates)."""
    B, Hq, D = q.shape
    Hkv = Kc.shape[1]
    gaps = np.full((B, Hq), np.nan)
    for b in range(B):
        n = int(lens[b]) // S
        for h in range(Hq):
            g = O.kv_head_of(h, Hq, Hkv)
            if n > k:
                s = O.scores_for_rows(q[b, h][None], Lc[b, g], n)[0]
                order = O.select_topk(s[None], k + 1)[0]
                gaps[b, h] = s[order[k - 1]] - s[order[k]]
    return gaps


def pick_threshold(gaps):
    """A threshold halfway between two neighbouring observed gaps near the
    median, so that about half of the rows with a cut double."""
    g = np.sort(gaps[~np.isnan(gaps)])
    i = max(1, len(g) // 2)
    while i < len(g) - 1 and g[i] - g[i - 1] < 1e-4 * abs(g[i]):
        i += 1
    return float(0.5 * (g[i - 1] + g[i]))


def run(fn_args, lens_t, k, tau, B, Hq, kk):
    q, kd, vd, L = fn_args
    sel = torch.full((B, Hq, kk), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Hq, kk), 7.0, dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_decode_adaptive(q, kd, vd, L, S, k, tau, cache_lens=lens_t, sel_idx=sel, sel_score=sc)
    return out, sel, sc


def plain(fn_args, lens_t, kk):
    q, kd, vd, L = fn_args
    if lens_t is None:
        return hsa.hsa_forward_decode(q, kd, vd, L, S, kk)
    return hsa.hsa_forward_decode_varlen(q, kd, vd, L, lens_t, S, kk)


@pytest.mark.parametrize("case", CASES)
def test_adaptive_decode(case):
    B, Hq, Hkv, T, D, k, dtype, lens = case
    print(f"adaptive case {case}", flush=True)
    lens = [T] * B if lens is None else lens
    q, kc, vc = small_inputs(B, Hq, Hkv, T, D, dtype, seed=1000 + T % 977 + k, decode=True)
    Q, K, V = f64(q), f64(kc), f64(vc)
    Lc = O.landmarks(K, S, dtype)
    gaps = oracle_gaps(Q, K, Lc, lens, k)
    tau = pick_threshold(gaps)
    args = (q.cuda(), kc.cuda(), vc.cuda(), None)
    L = torch.empty((B, Hkv, T // S, D), dtype=kc.dtype, device="cuda")
    hsa.hsa_build_landmarks(args[1], L, S)
    args = args[:3] + (L,)
    lens_t = torch.tensor(lens, dtype=torch.int64, device="cuda") if case[7] is not None else None

    ref_k = plain(args, lens_t, k)
    ref_2k = plain(args, lens_t, 2 * k)
    out0, sel0, _ = run(args, lens_t, k, 0.0, B, Hq, 2 * k)
    outi, seli, _ = run(args, lens_t, k, math.inf, B, Hq, 2 * k)
    out, sel, sc = run(args, lens_t, k, tau, B, Hq, 2 * k)
    torch.cuda.synchronize()
    assert torch.equal(out0, ref_k) and torch.all(sel0[..., k:] == -1)
    assert torch.equal(outi, ref_2k)
    m_gpu = (sel >= 0).sum(-1).cpu().numpy()
    same_k = (out == ref_k).all(-1).cpu().numpy()
    same_2k = (out == ref_2k).all(-1).cpu().numpy()
    assert np.all(np.where(m_gpu > k, same_2k, same_k)), "rows must equal the plain decode at their budget"

    sel_h, sc_h, out_h = sel.cpu().numpy(), f64(sc), f64(out)
    stats = new_stats()
    for b in range(B):
        for h in range(Hq):
            g = O.kv_head_of(h, Hq, Hkv)
            try:
                check_rows_adaptive(Q[b, h][None], [lens[b]], K[b, g, :lens[b]], V[b, g, :lens[b]], Lc[b, g], S,
                                    k, tau, out_h[b, h][None], sel_h[b, h][None], sc_h[b, h][None], TOL[dtype],
                                    stats)
            except Mismatch as e:
                raise Mismatch(f"(b {b}, h {h}): {e}") from None
    print(stats, f"tau {tau:.3e}", flush=True)
    rows_with_cut = int((~np.isnan(gaps)).sum())
    assert 0 < stats.get("doubled", 0) < rows_with_cut


PREFILL_CASES = [
    # B, Hq, Hkv, T, D, k, dtype
    (1, 8, 2, 64 * 70 + 13, 128, 8, "bf16"),  # 2k = 16
    (1, 4, 4, 64 * 80, 64, 16, "fp32"),       # 2k = 32, past one 64-chunk window
    (2, 4, 1, 64 * 140, 128, 16, "bf16"),     # two windows: remote pairs
    (1, 4, 1, 64 * 90 + 3, 128, 32, "bf16"),  # 2k = 64 (64-entry lists), past one window
    (1, 2, 2, 64 * 70, 64, 24, "fp32"),       # 2k = 48, G = 1
]


@pytest.mark.parametrize("case", PREFILL_CASES)
def test_adaptive_prefill(case):
    B, Hq, Hkv, T, D, k, dtype = case
    print(f"adaptive prefill case {case}", flush=True)
    q, kc, vc = small_inputs(B, Hq, Hkv, T, D, dtype, seed=2000 + T % 991 + k)
    Q, K, V = f64(q), f64(kc), f64(vc)
    Lc = O.landmarks(K, S, dtype)
    # threshold from the oracle's gaps of every row with a cut
    pos = np.arange(T)
    gaps = []
    for b in range(B):
        for h in range(Hq):
            g = O.kv_head_of(h, Hq, Hkv)
            _, _, gp = O.hsa_rows_adaptive(Q[b, h], pos, K[b, g], V[b, g], Lc[b, g], S, k, 0.0)
            gaps.append(gp)
    tau = pick_threshold(np.concatenate(gaps))
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    L = torch.empty((B, Hkv, T // S, D), dtype=kc.dtype, device="cuda")
    hsa.hsa_build_landmarks(kd, L, S)

    def adaptive(t):
        sel = torch.full((B, Hq, T, 2 * k), -7, dtype=torch.int32, device="cuda")
        sc = torch.full((B, Hq, T, 2 * k), 7.0, dtype=torch.float32, device="cuda")
        out = hsa.hsa_forward_prefill_adaptive(qd, kd, vd, L, S, k, t, sel_idx=sel, sel_score=sc)
        return out, sel, sc

    ref_k = hsa.hsa_forward_prefill(qd, kd, vd, L, S, k)
    ref_2k = hsa.hsa_forward_prefill(qd, kd, vd, L, S, 2 * k)
    out0, sel0, _ = adaptive(0.0)
    outi, _, _ = adaptive(math.inf)
    out, sel, sc = adaptive(tau)
    torch.cuda.synchronize()
    assert torch.equal(out0, ref_k) and torch.all(sel0[..., k:] == -1)
    assert torch.equal(outi, ref_2k)
    # a row's selection equals the plain prefill's at its budget; its output
    # matches up to fp32 rounding (a window chunk that fewer rows of the
    # row's 32-row block select is attended by the other path, and the
    # block's selections differ between the runs)
    m_gpu = (sel >= 0).sum(-1)
    sel_k = torch.empty((B, Hq, T, k), dtype=torch.int32, device="cuda")
    sel_2k = torch.empty((B, Hq, T, 2 * k), dtype=torch.int32, device="cuda")
    hsa.hsa_forward_prefill(qd, kd, vd, L, S, k, sel_idx=sel_k,
                            sel_score=torch.empty(sel_k.shape, dtype=torch.float32, device="cuda"))
    hsa.hsa_forward_prefill(qd, kd, vd, L, S, 2 * k, sel_idx=sel_2k,
                            sel_score=torch.empty(sel_2k.shape, dtype=torch.float32, device="cuda"))
    wide = (m_gpu > k)[..., None]
    ref_sel = torch.where(wide, sel_2k, torch.cat([sel_k, torch.full_like(sel_k, -1)], -1))
    assert torch.equal(sel, ref_sel), "rows must select as the plain prefill at their budget"
    ref = torch.where(wide, ref_2k, ref_k)
    assert float((out - ref).abs().max()) <= (1e-4 if dtype == "bf16" else 1e-6)

    sel_h, sc_h, out_h = sel.cpu().numpy(), f64(sc), f64(out)
    stats = new_stats()
    for b in range(B):
        for h in range(Hq):
            g = O.kv_head_of(h, Hq, Hkv)
            try:
                check_rows_adaptive(Q[b, h], pos, K[b, g], V[b, g], Lc[b, g], S, k, tau, out_h[b, h], sel_h[b, h],
                                    sc_h[b, h], TOL[dtype], stats)
            except Mismatch as e:
                raise Mismatch(f"(b {b}, h {h}): {e}") from None
    print(stats, f"tau {tau:.3e}", flush=True)
    assert 0 < stats.get("doubled", 0) < int(sum((~np.isnan(x)).sum() for x in gaps))
