"""GPU parity of hsa_backward_prefill against the oracle's backward.

The forward selection, scores and output given to the GPU backward are the
oracle's (the backward takes them as inputs); dOut is seeded N(0, 1).
Bounds, derived from the arithmetic of the kernels (the oracle supplies the
magnitude sums of the terms, abs_*):
* dK, dV: every product contracts bf16-rounded probabilities, dlogit and
  dO (8 significant bits: relative error up to 2^-8 each, 2^-7 per
  product) with fp32 accumulation: |err| <= 9e-3 abs + 1e-6;
* dq: dO and dlogit enter as bf16 head + tail pairs (the tail rounds a
  remainder below 2^-7 |x| to 8 bits: relative error below 2^-15 per
  operand) against exact bf16 K, V with fp32 accumulation:
  |err| <= 2e-4 abs + 1e-6."""
import zlib

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs
from oracle import hsa_oracle as O
from tests.gpu_util import f64

pytestmark = pytest.mark.gpu
S = 64
TOL_KV = (9e-3, 1e-6)
TOL_Q = (2e-4, 1e-6)

CASES = [
    # B, Hq, Hkv, T, D, k
    (1, 4, 1, 64 * 12 + 30, 128, 4),
    (1, 4, 2, 64 * 24, 128, 16),
    (2, 4, 4, 64 * 20 + 1, 64, 8),      # G = 1, one ragged token
    (1, 8, 1, 64 * 10 + 40, 128, 8),    # G = 8
    (1, 2, 1, 64 * 66 + 40, 128, 16),   # past one 64-chunk window
    (1, 2, 2, 50, 64, 4),               # no complete chunk
    (1, 2, 2, 64 * 33, 128, 32),
]


def check_bound(name, got, ref, scale, tol):
    err = np.abs(got - ref)
    bound = tol[0] * scale + tol[1]
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} entries over the bound; worst at {i}: "
                             f"got {got[i]:.6e} ref {ref[i]:.6e} bound {bound[i]:.3e}")
    return float((err / np.maximum(scale, 1e-30)).max()) if err.size else 0.0


def run_case(case):
    B, Hq, Hkv, T, D, k = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    q, kc, vc = small_inputs(B, Hq, Hkv, T, D, "bf16", seed=seed)
    dout = np.random.default_rng(seed + 1).standard_normal((B, Hq, T, D)).astype(np.float32)
    Q, K, V = f64(q), f64(kc), f64(vc)
    G64 = dout.astype(np.float64)
    out, sel, score, _ = O.prefill(Q, K, V, S, k, "bf16")
    dQ, dK, dV, aK, aV, aQ = O.prefill_backward(Q, K, V, S, k, "bf16", G64, sel_idx=sel)
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    L = torch.empty((B, Hkv, T // S, D), dtype=torch.bfloat16, device="cuda")
    hsa.hsa_build_landmarks(kd, L, S)
    sel_t = torch.from_numpy(sel.astype(np.int32)).cuda()
    score_t = torch.from_numpy(score.astype(np.float32)).cuda()
    out_t = torch.from_numpy(out.astype(np.float32)).cuda()
    dout_t = torch.from_numpy(dout).cuda()
    dq = torch.full((B, Hq, T, D), 7.0, device="cuda")
    dk = torch.full((B, Hkv, T, D), 7.0, device="cuda")
    dv = torch.full((B, Hkv, T, D), 7.0, device="cuda")
    hsa.hsa_backward_prefill(qd, kd, vd, L, out_t, dout_t, sel_t, score_t, S, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return (f64(dq), f64(dk), f64(dv)), (dQ, dK, dV), (aQ, aK, aV)


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_oracle(case):
    print(f"backward case {case}", flush=True)
    (gq, gk, gv), (rq, rk, rv), (aq, ak, av) = run_case(case)
    worst = {"dq": check_bound("dq", gq, rq, aq, TOL_Q), "dk": check_bound("dk", gk, rk, ak, TOL_KV),
             "dv": check_bound("dv", gv, rv, av, TOL_KV)}
    print("worst error / scale:", worst)


def test_backward_is_linear_in_dout():
    """Twice the upstream gradient gives twice the gradients (a property of
    the layer's backward that holds at any size), checked within rounding."""
    B, Hq, Hkv, T, D, k = 1, 4, 1, 64 * 30, 128, 8
    q, kc, vc = small_inputs(B, Hq, Hkv, T, D, "bf16", seed=91)
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    L = torch.empty((B, Hkv, T // S, D), dtype=torch.bfloat16, device="cuda")
    hsa.hsa_build_landmarks(kd, L, S)
    sel = torch.empty((B, Hq, T, k), dtype=torch.int32, device="cuda")
    sc = torch.empty((B, Hq, T, k), dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_prefill(qd, kd, vd, L, S, k, sel_idx=sel, sel_score=sc)
    g = torch.randn((B, Hq, T, D), device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    a = hsa.hsa_backward_prefill(qd, kd, vd, L, out, g, sel, sc, S)
    b = hsa.hsa_backward_prefill(qd, kd, vd, L, out, 2 * g, sel, sc, S)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.allclose(2 * x, y, rtol=1e-2, atol=1e-5)


def test_rows_without_pairs_do_not_leak():
    """Lanes past the end of a bucket load the first pair's rows and mask
    the values where they are used.  Rows of the first 64 tokens keep no
    pair (no complete chunk lies before them); filling their q with +inf and
    their dOut with NaN must leave every gradient as it is with finite
    values there (dq bit for bit: its partials do not depend on the order
    of a bucket's pairs; dK, dV within the order's rounding), and their dq
    rows zero."""
    B, Hq, Hkv, T, D, k = 1, 4, 1, 64 * 12 + 30, 128, 4
    print(f"backward poisoned-row case {(B, Hq, Hkv, T, D, k)}", flush=True)
    q, kc, vc = small_inputs(B, Hq, Hkv, T, D, "bf16", seed=321)
    dout = np.random.default_rng(322).standard_normal((B, Hq, T, D)).astype(np.float32)
    out, sel, score, _ = O.prefill(f64(q), f64(kc), f64(vc), S, k, "bf16")
    assert (sel[:, :, :S] < 0).all()
    qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
    L = torch.empty((B, Hkv, T // S, D), dtype=torch.bfloat16, device="cuda")
    hsa.hsa_build_landmarks(kd, L, S)
    sel_t = torch.from_numpy(sel.astype(np.int32)).cuda()
    score_t = torch.from_numpy(score.astype(np.float32)).cuda()
    out_t = torch.from_numpy(out.astype(np.float32)).cuda()

    def run(qx, gx):
        grads = [torch.full((B, h, T, D), 7.0, device="cuda") for h in (Hq, Hkv, Hkv)]
        hsa.hsa_backward_prefill(qx, kd, vd, L, out_t, gx, sel_t, score_t, S, dq=grads[0], dk=grads[1],
                                 dv=grads[2])
        torch.cuda.synchronize()
        return [g.cpu().numpy() for g in grads]

    clean = run(qd, torch.from_numpy(dout).cuda())
    qp = qd.clone()
    qp[:, :, :S] = float("inf")
    gp = torch.from_numpy(dout).cuda()
    gp[:, :, :S] = float("nan")
    poisoned = run(qp, gp)
    for g in poisoned:
        assert np.isfinite(g).all()
    assert np.array_equal(poisoned[0], clean[0])
    assert (poisoned[0][:, :, :S] == 0).all()
    for name, a, b in (("dk", poisoned[1], clean[1]), ("dv", poisoned[2], clean[2])):
        scale = np.abs(b).max() + 1e-30
        assert np.abs(a - b).max() <= 1e-5 * scale, name
