"""The prefill at its largest supported length: 65,536 chunks (T = 4,194,304
tokens; one head, D = 64, k = 16).  The selection stores chunk indices in 16
bits and marks up to 2,048 landmark tiles per row, so this is the boundary
of both.  A needle planted at chunk 65,534 (the last candidate of the last
query chunk) must be selected there, and sampled rows of the last, a middle
and an early query chunk match the oracle."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs
from oracle import hsa_oracle as O
from gpu_util import TOL, check_rows, f64, new_stats

pytestmark = pytest.mark.gpu

S, NC, D, TOPK = 64, 65536, 64, 16
T = S * NC
NEEDLE = NC - 2


def inputs():
    q, k, v = small_inputs(1, 1, 1, T, D, "bf16", seed=65536)
    # the last query row's direction, scaled, added to the needle chunk's keys
    qd = q[0, 0, T - 1].float()
    kn = k[0, 0, NEEDLE * S:(NEEDLE + 1) * S].float() + 3.0 * qd / qd.norm() * np.sqrt(D)
    k[0, 0, NEEDLE * S:(NEEDLE + 1) * S] = kn.to(torch.bfloat16)
    return q, k, v


def test_prefill_at_the_largest_chunk_count():
    q, k, v = inputs()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    L = torch.empty((1, 1, NC, D), dtype=torch.bfloat16, device="cuda")
    hsa.hsa_build_landmarks(kd, L, S)
    sel = torch.empty((1, 1, T, TOPK), dtype=torch.int32, device="cuda")
    sc = torch.empty((1, 1, T, TOPK), dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_prefill(qd, kd, vd, L, S, TOPK, sel_idx=sel, sel_score=sc)
    torch.cuda.synchronize()
    pos = np.concatenate([np.arange(T - S, T), np.arange(32768 * S, 32768 * S + 8), np.arange(S, S + 8)])
    pt = torch.from_numpy(pos).cuda()
    g_out = out[0, 0, pt].double().cpu().numpy()
    g_sel = sel[0, 0, pt].cpu().numpy()
    g_sc = sc[0, 0, pt].double().cpu().numpy()
    del qd, kd, vd, out, sel, sc
    assert NEEDLE in g_sel[S - 1], "the needle at chunk 65,534 must be kept by the last row"
    assert g_sel[:S].max() >= 32768, "the last rows keep chunks above 2^15"
    Kg = f64(k[0, 0])
    Lg = O.landmarks(Kg[None, None], S, "bf16")[0, 0]
    np.testing.assert_array_equal(f64(L[0, 0, -4:]), Lg[-4:])
    stats = new_stats()
    check_rows(f64(q[0, 0, torch.from_numpy(pos)]), pos, Kg, f64(v[0, 0]), Lg, S, TOPK, g_out, g_sel, g_sc,
               TOL["bf16"], stats)
    print(stats)
