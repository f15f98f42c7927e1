"""GPU parity of hsa_forward_decode against the oracle, through the C-ABI
binding: selected chunk indices exact except near ties, outputs within
2e-3 (bf16) / 1e-5 (fp32) max-abs."""
import zlib

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs
from oracle import hsa_oracle as O
from tests.gpu_util import TOL, check_rows, f64, new_stats

pytestmark = pytest.mark.gpu


def run_decode(q, k, v, S, topk, L=None):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    B, Hkv, T, D = k.shape
    if L is None:
        L = torch.empty((B, Hkv, T // S, D), dtype=k.dtype, device="cuda")
        hsa.hsa_build_landmarks(kd, L, S)
    Hq = q.shape[1]
    sel = torch.full((B, Hq, topk), -7, dtype=torch.int32, device="cuda")
    score = torch.full((B, Hq, topk), 7.0, dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_decode(qd, kd, vd, L, S, topk, sel_idx=sel, sel_score=score)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), sel.cpu().numpy(), score.cpu().double().numpy()


def compare(q, k, v, S, topk, dtype, out, sel, score):
    Q, K, V = f64(q), f64(k), f64(v)
    B, Hq, D = Q.shape
    Hkv, T = K.shape[1], K.shape[2]
    L = O.landmarks(K, S, dtype)
    stats = new_stats()
    for b in range(B):
        for h in range(Hq):
            g = O.kv_head_of(h, Hq, Hkv)
            check_rows(Q[b, h][None], np.array([T]), K[b, g], V[b, g], L[b, g], S, topk, out[b, h][None],
                       sel[b, h][None], score[b, h][None], TOL[dtype], stats)
    return stats


CASES = [
    # B, Hq, Hkv, T, D, k, dtype
    (2, 8, 2, 64 * 40 + 17, 128, 8, "bf16"),
    (3, 32, 8, 64 * 300, 128, 32, "bf16"),
    (2, 4, 4, 64 * 75 + 63, 64, 8, "fp32"),
    (1, 8, 1, 64 * 100, 64, 16, "bf16"),      # G = 8
    (1, 8, 1, 64 * 200 + 9, 128, 64, "bf16"),  # G = 8, k = 64: 512 group entries in the merge
    (2, 4, 2, 64 * 129, 128, 64, "fp32"),     # G = 2, k = 64
    (1, 4, 4, 64 * 5, 128, 16, "bf16"),       # fewer chunks than k
    (2, 8, 2, 63, 128, 4, "bf16"),            # no complete chunk: zeros
    (1, 4, 1, 64 * 5000, 128, 32, "bf16"),    # many scan splits
]


@pytest.mark.parametrize("case", CASES)
def test_decode_matches_oracle(case):
    B, Hq, Hkv, T, D, topk, dtype = case
    print(f"decode case {case}", flush=True)
    q, k, v = small_inputs(B, Hq, Hkv, T, D, dtype, seed=zlib.crc32(repr(case).encode()) % 10000, decode=True)
    out, sel, score = run_decode(q, k, v, 64, topk)
    stats = compare(q, k, v, 64, topk, dtype, out, sel, score)
    print(stats)
    if T < 64:
        assert np.all(out == 0) and np.all(sel == -1) and np.all(np.isneginf(score))


def test_decode_duplicate_chunks_keep_lower_index():
    B, Hq, Hkv, T, D = 1, 4, 1, 64 * 50, 128
    q, k, v = small_inputs(B, Hq, Hkv, T, D, "bf16", seed=11, decode=True)
    # make chunk 40 a copy of chunk 9 and chunk 30 a copy of chunk 2
    for dst, src in ((40, 9), (30, 2)):
        k[0, 0, dst * 64:(dst + 1) * 64] = k[0, 0, src * 64:(src + 1) * 64]
        v[0, 0, dst * 64:(dst + 1) * 64] = v[0, 0, src * 64:(src + 1) * 64]
    for topk in (1, 3, 8):
        out, sel, score = run_decode(q, k, v, 64, topk)
        compare(q, k, v, 64, topk, "bf16", out, sel, score)
        for h in range(Hq):
            s = list(sel[0, h])
            if 40 in s:
                assert 9 in s
            if 30 in s:
                assert 2 in s


def test_decode_is_deterministic():
    q, k, v = small_inputs(2, 32, 8, 64 * 700, 128, "bf16", seed=5, decode=True)
    a = run_decode(q, k, v, 64, 32)
    b = run_decode(q, k, v, 64, 32)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_decode_all_scores_equal_keep_lowest_indices():
    """Every chunk identical (all retrieval scores equal): the kept set is the
    k lowest chunk indices, in index order (ties toward the lower index)."""
    B, Hq, Hkv, T, D, topk = 1, 4, 1, 64 * 300, 128, 32
    q, k, v = small_inputs(B, Hq, Hkv, T, D, "bf16", seed=13, decode=True)
    for c in range(1, T // 64):
        k[0, 0, c * 64:(c + 1) * 64] = k[0, 0, 0:64]
    out, sel, score = run_decode(q, k, v, 64, topk)
    assert np.array_equal(sel[0], np.tile(np.arange(topk), (Hq, 1)))
    compare(q, k, v, 64, topk, "bf16", out, sel, score)


def test_decode_few_distinct_scores():
    """Chunks drawn from a handful of distinct ones: many exact ties around
    the k-th score, resolved toward the lower index."""
    B, Hq, Hkv, T, D, topk = 2, 8, 2, 64 * 2000, 128, 64
    q, k, v = small_inputs(B, Hq, Hkv, T, D, "bf16", seed=17, decode=True)
    r = np.random.default_rng(3)
    for b in range(B):
        for g in range(Hkv):
            src = r.integers(0, 5, size=T // 64)
            for c in range(5, T // 64):
                s0 = int(src[c])
                k[b, g, c * 64:(c + 1) * 64] = k[b, g, s0 * 64:(s0 + 1) * 64]
    out, sel, score = run_decode(q, k, v, 64, topk)
    compare(q, k, v, 64, topk, "bf16", out, sel, score)
