"""Empty inputs through the binding and the C ABI.  A sequence of no tokens,
a chunked prefill with no new rows and a backward over no tokens do nothing
and succeed (empty tensors hand the library NULL data pointers); decode
caches of no tokens, or with no complete chunk, give every query no
candidate, so its output is zero and its slots are padding (index -1,
score -inf), through the plain, adaptive-budget and no-allocation calls."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefill_over_no_tokens(dtype):
    dt = DT[dtype]
    q = torch.empty((1, 4, 0, 128), dtype=dt, device="cuda")
    k = torch.empty((1, 2, 0, 128), dtype=dt, device="cuda")
    v = torch.empty_like(k)
    L = torch.empty((1, 2, 0, 128), dtype=dt, device="cuda")
    hsa.hsa_build_landmarks(k, L, 64)
    sel = torch.empty((1, 4, 0, 8), dtype=torch.int32, device="cuda")
    sc = torch.empty((1, 4, 0, 8), dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_prefill(q, k, v, L, 64, 8, sel_idx=sel, sel_score=sc)
    out2 = hsa.hsa_forward_prefill_adaptive(q, k, v, L, 64, 8, 0.5)
    torch.cuda.synchronize()
    assert out.shape == (1, 4, 0, 128) and out2.shape == (1, 4, 0, 128)


def test_cached_prefill_with_no_new_rows_and_backward_over_no_tokens():
    torch.manual_seed(3)
    T = 64 * 5
    k = torch.randn((1, 2, T, 64), device="cuda").to(torch.bfloat16)
    v = torch.randn((1, 2, T, 64), device="cuda").to(torch.bfloat16)
    L = torch.empty((1, 2, T // 64, 64), dtype=torch.bfloat16, device="cuda")
    hsa.hsa_build_landmarks(k, L, 64)
    q = torch.empty((1, 4, 0, 64), dtype=torch.bfloat16, device="cuda")
    out = hsa.hsa_forward_prefill_cached(q, k, v, L, T, 64, 8)
    # backward over a sequence of no tokens
    e = torch.empty((1, 4, 0, 64), dtype=torch.bfloat16, device="cuda")
    ke = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    Le = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    f = torch.empty((1, 4, 0, 64), dtype=torch.float32, device="cuda")
    si = torch.empty((1, 4, 0, 8), dtype=torch.int32, device="cuda")
    ss = torch.empty((1, 4, 0, 8), dtype=torch.float32, device="cuda")
    dq, dk, dv = hsa.hsa_backward_prefill(e, ke, ke, Le, f, f, si, ss, 64)
    torch.cuda.synchronize()
    assert out.shape == (1, 4, 0, 64) and dq.shape == (1, 4, 0, 64) and dk.shape == (1, 2, 0, 64)


@pytest.mark.parametrize("T", [0, 1, 63])
def test_decode_without_a_complete_chunk_outputs_zero(T):
    torch.manual_seed(4 + T)
    B, Hq, Hkv, D, topk = 3, 8, 2, 128, 16
    q = torch.randn((B, Hq, D), device="cuda").to(torch.bfloat16)
    k = torch.randn((B, Hkv, T, D), device="cuda").to(torch.bfloat16)
    v = torch.randn((B, Hkv, T, D), device="cuda").to(torch.bfloat16)
    L = torch.empty((B, Hkv, 0, D), dtype=torch.bfloat16, device="cuda")
    outs = []
    for call in ("plain", "adaptive", "noalloc"):
        out = torch.full((B, Hq, D), 5.0, dtype=torch.float32, device="cuda")
        sel = torch.full((B, Hq, topk * (2 if call == "adaptive" else 1)), 7, dtype=torch.int32, device="cuda")
        sc = torch.full(sel.shape, 7.0, dtype=torch.float32, device="cuda")
        if call == "plain":
            hsa.hsa_forward_decode(q, k, v, L, 64, topk, out=out, sel_idx=sel, sel_score=sc)
        elif call == "adaptive":
            hsa.hsa_forward_decode_adaptive(q, k, v, L, 64, topk, 0.25, out=out, sel_idx=sel, sel_score=sc)
        else:
            hsa.hsa_forward_decode_noalloc(q, k, v, L, 64, topk, out, sel_idx=sel, sel_score=sc)
        torch.cuda.synchronize()
        assert float(out.abs().max()) == 0.0, call
        assert bool((sel == -1).all()), call
        assert bool(torch.isneginf(sc).all()), call
        outs.append(out)
    assert np.array_equal(outs[0].cpu().numpy(), outs[2].cpu().numpy())
