"""The debug library (libhsa_attn_debug.so, the same kernels built with
HSA_ATTN_DEBUG=1) on the GPU.  Each of its calls fills the workspace and the
outputs with a NaN pattern before its kernels and checks every index the
kernels read back from the workspace.  Every entry point, on shapes that take
every kernel path (chunk-major pairs, several slabs, adaptive budgets, ragged
caches), must leave the flag word at 0 and reproduce the release library's
results bit for bit: no result depends on memory a call did not write, and
no workspace index was out of range."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs

pytestmark = pytest.mark.gpu
S = 64


def _ws(dims, kind):
    return torch.empty(hsa.hsa_attn_workspace_size(dims, kind), dtype=torch.uint8, device="cuda")


def _same(name, a, b):
    a, b = a.cpu(), b.cpu()
    assert a.shape == b.shape and a.dtype == b.dtype, name
    same = torch.equal(a, b) if not a.is_floating_point() else bool(
        ((a == b) | (torch.isnan(a) & torch.isnan(b))).all())
    assert same, f"{name}: debug and release results differ (max |diff| " \
                 f"{(a.double() - b.double()).abs().nan_to_num(float('inf')).max().item():.3e})"
    if a.is_floating_point():
        assert not torch.isnan(a).any(), f"{name}: NaN from unwritten memory"


def _both(run):
    """run(debug) -> (results dict, workspace or None); returns the release
    and debug results after checking the debug call's flag word."""
    rel, _ = run(False)
    with hsa.debug_library():
        dbg, ws = run(True)
        flags = hsa.hsa_attn_debug_flags(ws)
    assert flags == 0, f"debug checks failed: flags 0x{flags:x}"
    for key in rel:
        _same(key, dbg[key], rel[key])
    return rel, dbg


def _landmarks(k):
    B, Hkv, T, D = k.shape
    L = torch.empty((B, Hkv, T // S, D), dtype=k.dtype, device="cuda")
    hsa.hsa_build_landmarks(k, L, S)
    return L


PREFILL = [
    # B, Hq, Hkv, T, D, k, dtype, slabs (None: the default workspace)
    (1, 8, 2, 64 * 140 + 13, 128, 16, "bf16", None),   # chunk-major pairs before the window
    (1, 8, 2, 64 * 140 + 13, 128, 16, "bf16", 3),      # the same in three slabs
    (1, 2, 1, 64 * 90 + 40, 128, 32, "bf16", None),    # 32-entry lists
    (1, 4, 2, 64 * 80 + 5, 64, 64, "bf16", None),      # 64-entry lists
    (2, 2, 2, 64 * 75 + 1, 64, 8, "fp32", None),
    (1, 4, 1, 50, 128, 4, "bf16", None),               # no complete chunk
]


@pytest.mark.parametrize("case", PREFILL)
def test_debug_prefill_matches_release(case):
    B, Hq, Hkv, T, D, k, dt, slabs = case
    q, kk, v = (x.cuda() for x in small_inputs(B, Hq, Hkv, T, D, dt, seed=11 + T))
    L = _landmarks(kk)

    def run(debug):
        dims = hsa.make_dims(B, Hq, Hkv, D, S, k, T, hsa.HSA_ATTN_BF16 if dt == "bf16" else hsa.HSA_ATTN_FP32)
        ws = _ws(dims, 0)
        if slabs:
            # the smallest workspace that still holds rows / slabs query rows per slab
            want = -(-(-(-T // 64)) // slabs) * 64
            lo, hi = 0, ws.numel()
            while lo < hi:
                mid = (lo + hi) // 2
                if hsa.hsa_attn_prefill_slab_rows(dims, mid, False, True) >= want:
                    hi = mid
                else:
                    lo = mid + 1
            ws = torch.empty(lo, dtype=torch.uint8, device="cuda")
        sel = torch.empty((B, Hq, T, k), dtype=torch.int32, device="cuda")
        sc = torch.empty((B, Hq, T, k), dtype=torch.float32, device="cuda")
        out = hsa.hsa_forward_prefill(q, kk, v, L, S, k, sel_idx=sel, sel_score=sc, workspace=ws)
        return {"out": out, "sel_idx": sel, "sel_score": sc}, ws

    _both(run)


def test_debug_prefill_library_selection_cached_and_adaptive():
    B, Hq, Hkv, T, D, k = 1, 8, 2, 64 * 100 + 9, 128, 16
    q, kk, v = (x.cuda() for x in small_inputs(B, Hq, Hkv, T, D, "bf16", seed=5))
    L = _landmarks(kk)
    dims = hsa.make_dims(B, Hq, Hkv, D, S, k, T, hsa.HSA_ATTN_BF16)

    def plain(debug):  # the selection kept in the (poisoned) workspace
        ws = _ws(dims, 0)
        return {"out": hsa.hsa_forward_prefill(q, kk, v, L, S, k, workspace=ws)}, ws

    def cached(debug):
        off = 64 * 40
        ws = _ws(dims, 0)
        out = hsa.hsa_forward_prefill_cached(q[:, :, off:].contiguous(), kk, v, L, off, S, k, workspace=ws)
        return {"out": out}, ws

    def adaptive(debug):
        ws = _ws(dims, 3)
        sel = torch.empty((B, Hq, T, 2 * k), dtype=torch.int32, device="cuda")
        sc = torch.empty((B, Hq, T, 2 * k), dtype=torch.float32, device="cuda")
        out = hsa.hsa_forward_prefill_adaptive(q, kk, v, L, S, k, 1e-2, sel_idx=sel, sel_score=sc, workspace=ws)
        return {"out": out, "sel_idx": sel, "sel_score": sc}, ws

    for run in (plain, cached, adaptive):
        _both(run)


def test_debug_decode_paths_match_release():
    B, Hq, Hkv, T, D, k = 3, 8, 2, 64 * 300 + 5, 128, 32
    _, kk, v = (x.cuda() for x in small_inputs(B, Hq, Hkv, T, D, "bf16", seed=21))
    q = small_inputs(B, Hq, Hkv, T, D, "bf16", seed=22, decode=True)[0].cuda()
    L = _landmarks(kk)
    dims = hsa.make_dims(B, Hq, Hkv, D, S, k, T, hsa.HSA_ATTN_BF16)
    lens = torch.tensor([64 * 300 + 5, 64 * 17 + 3, 30], dtype=torch.int64, device="cuda")

    def decode(debug):
        ws = _ws(dims, 1)
        sel = torch.empty((B, Hq, k), dtype=torch.int32, device="cuda")
        sc = torch.empty((B, Hq, k), dtype=torch.float32, device="cuda")
        out = hsa.hsa_forward_decode(q, kk, v, L, S, k, sel_idx=sel, sel_score=sc, workspace=ws)
        return {"out": out, "sel_idx": sel, "sel_score": sc}, ws

    def varlen(debug):
        ws = _ws(dims, 1)
        return {"out": hsa.hsa_forward_decode_varlen(q, kk, v, L, lens, S, k, workspace=ws)}, ws

    def adaptive(debug):
        ws = _ws(dims, 2)
        out = hsa.hsa_forward_decode_adaptive(q, kk, v, L, S, 16, 1e-3, cache_lens=lens, workspace=ws)
        return {"out": out}, ws

    def noalloc(debug):
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        hsa.hsa_forward_decode_noalloc(q, kk, v, L, S, k, out)
        return {"out": out}, None  # the flag word sits in the scratch

    for run in (decode, varlen, adaptive, noalloc):
        _both(run)


def test_debug_backward_matches_release():
    B, Hq, Hkv, T, D, k = 1, 4, 1, 64 * 90 + 5, 128, 8
    q, kk, v = (x.cuda() for x in small_inputs(B, Hq, Hkv, T, D, "bf16", seed=31))
    L = _landmarks(kk)
    sel = torch.empty((B, Hq, T, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hq, T, k), dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_prefill(q, kk, v, L, S, k, sel_idx=sel, sel_score=sc)
    g = torch.from_numpy(np.random.default_rng(32).standard_normal((B, Hq, T, D)).astype(np.float32)).cuda()
    dims = hsa.make_dims(B, Hq, Hkv, D, S, k, T, hsa.HSA_ATTN_BF16)

    def run(debug):
        ws = _ws(dims, 4)
        dq, dk, dv = hsa.hsa_backward_prefill(q, kk, v, L, out, g, sel, sc, S, workspace=ws)
        # the chunk kernel's dK/dV sums follow the bucket order its atomics
        # leave, so they are compared within rounding; dq is summed in slot
        # order and must match exactly
        return {"dq": dq, "dk": dk, "dv": dv}, ws

    rel, _ = run(False)
    with hsa.debug_library():
        dbg, ws = run(True)
        flags = hsa.hsa_attn_debug_flags(ws)
    assert flags == 0, f"debug checks failed: flags 0x{flags:x}"
    _same("dq", dbg["dq"], rel["dq"])
    for key in ("dk", "dv"):
        a, b = dbg[key].cpu().double(), rel[key].cpu().double()
        assert not torch.isnan(a).any(), f"{key}: NaN from unwritten memory"
        assert (a - b).abs().max().item() <= 1e-5 * max(1.0, b.abs().max().item()), key
