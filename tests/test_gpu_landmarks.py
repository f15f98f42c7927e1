"""GPU parity of the landmark builder against the oracle (bit-exact for bf16,
within one fp32 ulp for fp32), through the C-ABI binding."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import small_inputs
from oracle import hsa_oracle as O
from tests.gpu_util import f64

pytestmark = pytest.mark.gpu


def run_landmarks(k, S, c0=0, c1=None, fill=None):
    B, Hkv, T, D = k.shape
    L = torch.empty((B, Hkv, T // S, D), dtype=k.dtype, device="cuda")
    if fill is not None:
        L.fill_(fill)
    hsa.hsa_build_landmarks(k, L, S, c0, c1)
    torch.cuda.synchronize()
    return L


@pytest.mark.parametrize("dtype,D,S,T", [
    ("bf16", 128, 64, 64 * 37 + 5),
    ("bf16", 64, 64, 64 * 9),
    ("bf16", 128, 16, 16 * 50 + 3),
    ("bf16", 128, 1, 40),
    ("bf16", 64, 3, 3 * 33 + 2),
    ("fp32", 64, 64, 64 * 20 + 63),
    ("fp32", 128, 32, 32 * 11),
])
def test_landmarks_match_oracle(dtype, D, S, T):
    print(f"landmarks dtype={dtype} D={D} S={S} T={T}", flush=True)
    _, k, _ = small_inputs(2, 2, 3, T, D, dtype, seed=T + S)
    L = run_landmarks(k.cuda(), S)
    ref = O.landmarks(f64(k), S, dtype)
    got = f64(L)
    if dtype == "bf16":
        assert np.array_equal(got, ref)
    else:
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= ulp)


def test_landmark_subrange_leaves_other_chunks_untouched():
    _, k, _ = small_inputs(1, 1, 2, 64 * 10, 128, "bf16", seed=3)
    L = run_landmarks(k.cuda(), 64, 3, 7, fill=5.0)
    ref = O.landmarks(f64(k), 64, "bf16")
    got = f64(L)
    assert np.array_equal(got[:, :, 3:7], ref[:, :, 3:7])
    assert np.all(got[:, :, :3] == 5.0) and np.all(got[:, :, 7:] == 5.0)


def test_landmark_of_constant_chunk_is_the_key():
    _, k, _ = small_inputs(1, 1, 1, 64 * 4, 128, "bf16", seed=4)
    k[0, 0, 64:128] = k[0, 0, 64]
    L = run_landmarks(k.cuda(), 64)
    assert torch.equal(L[0, 0, 1].cpu(), k[0, 0, 64])
