"""Parity of prefill and decode against the oracle on seeded random shapes:
query-group size, head dim, dtype, k (1 .. 64 within the supported
envelope), ragged sequence lengths (including fewer tokens than one chunk)
and batch drawn from a fixed generator, so that combinations the hand-picked
cases leave out are checked too.  The backward and the adaptive-budget
decode and prefill get the same treatment within their own envelopes."""
import numpy as np
import pytest

from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs
from tests import test_gpu_decode as dec
from tests import test_gpu_prefill as pre

pytestmark = pytest.mark.gpu


def _cases(kind, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        D = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "fp32"]))
        kmax = 32 if (kind == "prefill" and G > 4) else 64
        k = int(rng.integers(1, kmax + 1))
        T = int(rng.integers(10, 64 * 40 + 64))
        B = int(rng.choice([1, 2]))
        out.append((B, G * Hkv, Hkv, T, D, k, dtype))
    return out


@pytest.mark.parametrize("case", _cases("prefill", 16, 2026))
def test_random_prefill_matches_oracle(case):
    B, Hq, Hkv, T, D, topk, dtype = case
    print(f"prefill case {case}", flush=True)
    q, k, v = small_inputs(B, Hq, Hkv, T, D, dtype, seed=pre.case_seed(case))
    out, sel, score = pre.run_prefill(q, k, v, 64, topk)
    print(pre.compare(q, k, v, 64, topk, dtype, out, sel, score))


@pytest.mark.parametrize("case", _cases("decode", 16, 2027))
def test_random_decode_matches_oracle(case):
    B, Hq, Hkv, T, D, topk, dtype = case
    print(f"decode case {case}", flush=True)
    q, k, v = small_inputs(B, Hq, Hkv, T, D, dtype, seed=pre.case_seed(case), decode=True)
    out, sel, score = dec.run_decode(q, k, v, 64, topk)
    print(dec.compare(q, k, v, 64, topk, dtype, out, sel, score))
    if T < 64:
        assert np.all(out == 0) and np.all(sel == -1)


def _backward_cases(n, seed):
    # bf16 storage, k up to 32 (the backward's envelope), shorter sequences:
    # the oracle's backward is the slow part
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        D = int(rng.choice([64, 128]))
        k = int(rng.integers(1, 33))
        T = int(rng.integers(10, 64 * 16 + 64))
        B = int(rng.choice([1, 2]))
        out.append((B, G * Hkv, Hkv, T, D, k))
    return out


@pytest.mark.parametrize("case", _backward_cases(8, 2028))
def test_random_backward_within_bounds(case):
    from tests import test_gpu_backward as bwd
    print(f"backward case {case}", flush=True)
    (gq, gk, gv), (rq, rk, rv), (aq, ak, av) = bwd.run_case(case)
    bwd.check_bound("dq", gq, rq, aq, bwd.TOL_Q)
    bwd.check_bound("dk", gk, rk, ak, bwd.TOL_KV)
    bwd.check_bound("dv", gv, rv, av, bwd.TOL_KV)


def _adaptive_cases(kind, n, seed):
    # base k with 2k <= 64 (2k <= 32 for prefill groups above four heads);
    # sequences long enough that rows have a k-th/(k+1)-th cut; for decode,
    # ragged cache lengths (some below one chunk) in about half the cases
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.choice([1, 2]))
        D = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "fp32"]))
        kmax = 16 if (kind == "prefill" and G > 4) else 32
        k = int(rng.integers(1, kmax + 1))
        B = int(rng.choice([1, 2])) if kind == "prefill" else int(rng.integers(2, 5))
        hi = 64 * 60 if kind == "prefill" else 64 * 2000
        T = int(rng.integers(64 * (2 * k + 3), hi))
        if kind == "prefill":
            out.append((B, G * Hkv, Hkv, T, D, k, dtype))
            continue
        lens = None
        if rng.random() < 0.5:
            lens = [T] + [int(x) for x in rng.integers(1, T + 1, size=B - 1)]
        out.append((B, G * Hkv, Hkv, T, D, k, dtype, lens))
    return out


@pytest.mark.parametrize("case", _adaptive_cases("decode", 6, 2029))
def test_random_adaptive_decode(case):
    from tests import test_gpu_adaptive as ada
    ada.test_adaptive_decode(case)


@pytest.mark.parametrize("case", _adaptive_cases("prefill", 4, 2030))
def test_random_adaptive_prefill(case):
    from tests import test_gpu_adaptive as ada
    ada.test_adaptive_prefill(case)
