"""hsa_forward_decode_noalloc (the decode entry point that allocates
nothing and keeps its scratch in a fixed per-GPU array of the library)
against hsa_forward_decode with a workspace, through the C ABI: two calls in
a row, the second on a smaller input, each bit-identical to the workspace
call on the same inputs (same kernels, same plan); a shape whose scratch
would not fit is rejected before any launch."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs

pytestmark = pytest.mark.gpu
S = 64


def run_both(B, Hq, Hkv, T, D, k, dtype, seed, with_sel):
    print(f"no-alloc decode case B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} k={k} {dtype} sel={with_sel}", flush=True)
    q, kc, vc = small_inputs(B, Hq, Hkv, T, D, dtype, seed=seed, decode=True)
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    L = torch.empty((B, Hkv, T // S, D), dtype=kc.dtype, device="cuda")
    hsa.hsa_build_landmarks(kd, L, S)
    res = []
    for fn in ("workspace", "noalloc"):
        out = torch.full((B, Hq, D), 7.0, device="cuda")
        sel = torch.full((B, Hq, k), -7, dtype=torch.int32, device="cuda") if with_sel else None
        sc = torch.full((B, Hq, k), 7.0, device="cuda") if with_sel else None
        if fn == "workspace":
            hsa.hsa_forward_decode(qd, kd, vd, L, S, k, out=out, sel_idx=sel, sel_score=sc)
        else:
            hsa.hsa_forward_decode_noalloc(qd, kd, vd, L, S, k, out, sel_idx=sel, sel_score=sc)
        torch.cuda.synchronize()
        res.append([t.cpu() for t in (out, sel, sc) if t is not None])
    for a, b in zip(*res):
        assert torch.equal(a, b)
    assert torch.isfinite(res[1][0]).all()


def test_noalloc_decode_equals_workspace_decode_twice():
    # a larger call, then a smaller one that reuses the same scratch array
    run_both(8, 32, 8, 64 * 4096 + 21, 128, 32, "bf16", seed=5, with_sel=True)
    run_both(2, 8, 2, 64 * 40 + 3, 64, 16, "bf16", seed=6, with_sel=False)
    run_both(3, 4, 4, 64 * 70, 64, 8, "fp32", seed=7, with_sel=True)


def test_noalloc_decode_rejects_shapes_beyond_its_scratch():
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    T = 1 << 22  # 64 caches of 4M tokens: ~100 MiB of candidates alone
    dims = hsa.make_dims(64, 32, 8, 128, S, 64, T, hsa.HSA_ATTN_BF16)
    need = hsa.hsa_attn_workspace_size(dims, 1)
    assert need > 64 << 20
    lib = hsa.load_library()
    p = q.data_ptr()
    out = torch.empty((64, 32, 128), device="cuda")
    st = lib.hsa_forward_decode_noalloc(hsa.ctypes.byref(dims), p, p, p, p, out.data_ptr(), None, None, None)
    assert st == hsa.HSA_ATTN_WORKSPACE_TOO_SMALL
    assert "64" in hsa.hsa_attn_last_error() or "67108864" in hsa.hsa_attn_last_error()
