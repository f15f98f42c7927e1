"""GPU parity of chunked prefill over a cached prefix
(hsa_forward_prefill_cached): the rows of the new tokens must equal, bit for
bit, the same rows of a full-sequence hsa_forward_prefill (the kernels do the
same work per query chunk), and match the oracle under the acceptance rule."""
import zlib

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs
from oracle import hsa_oracle as O
from tests.gpu_util import TOL, check_rows, f64, new_stats

pytestmark = pytest.mark.gpu
S = 64

CASES = [
    # B, Hq, Hkv, T, D, k, dtype, q_offset
    (1, 8, 2, 64 * 150 + 17, 128, 16, "bf16", 64 * 100),   # prefix past one window
    (2, 4, 4, 64 * 70, 64, 8, "fp32", 64 * 60),
    (1, 8, 1, 64 * 40 + 5, 128, 32, "bf16", 64 * 3),
    (1, 4, 1, 64 * 90, 128, 4, "bf16", 0),                # no prefix: same as prefill
]


@pytest.mark.parametrize("case", CASES)
def test_prefill_cached_matches_full_prefill_and_oracle(case):
    B, Hq, Hkv, T, D, topk, dtype, off = case
    print(f"prefill_cached case {case}", flush=True)
    q, k, v = small_inputs(B, Hq, Hkv, T, D, dtype, seed=zlib.crc32(repr(case).encode()) % 10000)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    L = torch.empty((B, Hkv, T // S, D), dtype=k.dtype, device="cuda")
    hsa.hsa_build_landmarks(kd, L, S)
    Tq = T - off
    sel = torch.full((B, Hq, Tq, topk), -7, dtype=torch.int32, device="cuda")
    score = torch.full((B, Hq, Tq, topk), 7.0, dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_prefill_cached(qd[:, :, off:].contiguous(), kd, vd, L, off, S, topk, sel_idx=sel,
                                         sel_score=score)
    full_sel = torch.empty((B, Hq, T, topk), dtype=torch.int32, device="cuda")
    full_score = torch.empty((B, Hq, T, topk), dtype=torch.float32, device="cuda")
    full = hsa.hsa_forward_prefill(qd, kd, vd, L, S, topk, sel_idx=full_sel, sel_score=full_score)
    torch.cuda.synchronize()
    assert torch.equal(out, full[:, :, off:])
    assert torch.equal(sel, full_sel[:, :, off:]) and torch.equal(score, full_score[:, :, off:])
    # and the oracle on a sample of the new rows
    rows = np.unique(np.concatenate([np.arange(off, min(T, off + 70)), np.arange(max(off, T - 70), T)]))
    Q, K, V = f64(q), f64(k), f64(v)
    Lo = O.landmarks(K, S, dtype)
    o, sl, sc = out.cpu().double().numpy(), sel.cpu().numpy(), score.cpu().double().numpy()
    stats = new_stats()
    for b in range(B):
        for h in range(Hq):
            g = O.kv_head_of(h, Hq, Hkv)
            check_rows(Q[b, h, rows], rows, K[b, g], V[b, g], Lo[b, g], S, topk, o[b, h, rows - off],
                       sl[b, h, rows - off], sc[b, h, rows - off], TOL[dtype], stats)
    print(stats)
