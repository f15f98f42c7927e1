"""The worker pool of the full-size parity tests, exercised on the CPU: the
oracle's own results fed through it as if they were the layer's pass every
row; a planted wrong selection fails; landmarks built slab by slab in the
workers equal the oracle's landmarks of the whole array."""
import numpy as np
import pytest

from oracle import hsa_oracle as O
from tests.oracle_pool import (OraclePool, check_prefill_rows_task, gather_landmarks, merge_stats,
                               oracle_landmarks)
from tests.test_oracle_pins import rand_qkv


def bits(x):
    return O.f32_to_bf16_bits(x)


def test_pool_checks_rows_and_builds_landmarks():
    B, Hq, Hkv, T, D, S, k = 1, 4, 2, 64 * 9 + 17, 8, 64, 3
    Q, K, V = rand_qkv(11, B, Hq, Hkv, T, D, "bf16")
    out, sel, sc, L = O.prefill(Q, K, V, S, k, "bf16")
    with OraclePool(workers=2) as P:
        for name, a in (("q", bits(Q)), ("k", bits(K)), ("v", bits(V)), ("out", out.astype(np.float32)),
                        ("sel", sel.astype(np.int32)), ("sc", sc.astype(np.float32))):
            m = P.array(name, a.shape, a.dtype)
            m[:] = a
            m.flush()
        futs = [P.submit(check_prefill_rows_task, P.dir, 0, h, O.kv_head_of(h, Hq, Hkv), np.arange(r0, min(T, r0 + 200)),
                         S, k, "bf16", 2e-3) for h in range(Hq) for r0 in range(0, T, 200)]
        stats = {}
        for f in futs:
            merge_stats(stats, f.result())
        assert stats["rows"] == Hq * T and stats["max_err"] < 1e-6
        # slabs of 128 rows (two chunks) give the same landmarks as one call
        lm = gather_landmarks(oracle_landmarks(P, P.path("k"), (0, 1), T, S, "bf16", slab=128), D)
        assert np.array_equal(lm, L[0, 1])
        # a wrong selection in one row is caught
        m = np.load(P.path("sel"), mmap_mode="r+")
        row = 64 * 8 + 3
        m[0, 2, row, 0] = (m[0, 2, row, 0] + 1) % 8
        m.flush()
        with pytest.raises(AssertionError):
            P.submit(check_prefill_rows_task, P.dir, 0, 2, 1, np.arange(row, row + 1), S, k, "bf16",
                     2e-3).result()
