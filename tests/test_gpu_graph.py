"""The decode and prefill calls captured in a HIP graph (as a serving loop
runs them): every replay, with new query values written into the captured
input between replays and eager work in between, equals the eager call on
the same inputs bit for bit (outputs, selections and scores)."""
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs

pytestmark = pytest.mark.gpu
S = 64


def _capture(fn):
    """Capture fn() on a side stream after one warm-up call (torch's graph
    capture protocol)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_replays_in_a_graph():
    B, Hq, Hkv, T, D, k = 2, 8, 2, 64 * 40 + 17, 128, 8
    print(f"graph decode case {(B, Hq, Hkv, T, D, k)}", flush=True)
    q0, kc, vc = small_inputs(B, Hq, Hkv, T, D, "bf16", seed=31)
    kd, vd = kc.cuda(), vc.cuda()
    L = torch.empty((B, Hkv, T // S, D), dtype=kd.dtype, device="cuda")
    hsa.hsa_build_landmarks(kd, L, S)
    dims = hsa.make_dims(B, Hq, Hkv, D, S, k, T, 1)
    ws = torch.empty(hsa.hsa_attn_workspace_size(dims, 1), dtype=torch.uint8, device="cuda")
    q = torch.empty((B, Hq, D), dtype=kd.dtype, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, Hq, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hq, k), dtype=torch.float32, device="cuda")
    q.copy_(q0[:, :, T - 1])
    g = _capture(lambda: hsa.hsa_forward_decode(q, kd, vd, L, S, k, out=out, sel_idx=sel, sel_score=sc,
                                                workspace=ws))
    for rep in range(4):
        q.copy_(q0[:, :, T - 1 - 37 * rep])   # a new query in the captured buffer
        out.fill_(float("nan"))
        sel.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), sel.clone(), sc.clone())
        ref_sel = torch.empty_like(sel)
        ref_sc = torch.empty_like(sc)
        ref = hsa.hsa_forward_decode(q.clone(), kd, vd, L, S, k, sel_idx=ref_sel, sel_score=ref_sc)
        torch.cuda.synchronize()
        assert torch.equal(got[1], ref_sel), f"replay {rep}: selection differs"
        assert torch.equal(got[2], ref_sc), f"replay {rep}: scores differ"
        assert torch.equal(got[0], ref), f"replay {rep}: output differs"


def test_prefill_replays_in_a_graph():
    B, Hq, Hkv, T, D, k = 1, 4, 1, 64 * 70 + 9, 128, 8
    print(f"graph prefill case {(B, Hq, Hkv, T, D, k)}", flush=True)
    q0, kc, vc = small_inputs(B, Hq, Hkv, T, D, "bf16", seed=32)
    kd, vd = kc.cuda(), vc.cuda()
    L = torch.empty((B, Hkv, T // S, D), dtype=kd.dtype, device="cuda")
    hsa.hsa_build_landmarks(kd, L, S)
    dims = hsa.make_dims(B, Hq, Hkv, D, S, k, T, 1)
    ws = torch.empty(hsa.hsa_attn_workspace_size(dims, 0), dtype=torch.uint8, device="cuda")
    q = q0.cuda()
    out = torch.empty((B, Hq, T, D), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, Hq, T, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hq, T, k), dtype=torch.float32, device="cuda")
    g = _capture(lambda: hsa.hsa_forward_prefill(q, kd, vd, L, S, k, out=out, sel_idx=sel, sel_score=sc,
                                                 workspace=ws))
    for rep in range(3):
        q.copy_(torch.roll(q0, shifts=rep, dims=1).cuda())   # new queries in the captured buffer
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = (out.clone(), sel.clone(), sc.clone())
        ref_sel = torch.empty_like(sel)
        ref_sc = torch.empty_like(sc)
        ref = hsa.hsa_forward_prefill(q.clone(), kd, vd, L, S, k, sel_idx=ref_sel, sel_score=ref_sc)
        torch.cuda.synchronize()
        assert torch.equal(got[1], ref_sel), f"replay {rep}: selection differs"
        assert torch.equal(got[2], ref_sc), f"replay {rep}: scores differ"
        assert torch.equal(got[0], ref), f"replay {rep}: output differs"
