"""The numpy oracle against stored brute-force results (tests/golden/*.json,
written by tests/golden/make_golden.py, which calls only the pure-Python oracle)."""
import json
import os

import numpy as np
import pytest

from oracle import hsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("name", ["tiny_gqa_bf16.json", "tiny_mha_fp32.json"])
def test_oracle_reproduces_golden(name):
    doc = json.load(open(os.path.join(GOLDEN, name)))
    sh = doc["shape"]
    Q, K, V = (np.array(doc[x], dtype=np.float64) for x in ("Q", "K", "V"))
    out, sel, sc, L = O.prefill(Q, K, V, sh["S"], sh["k"], sh["dtype"])
    assert np.array_equal(L, np.array(doc["landmarks"]).reshape(L.shape))
    for b in range(sh["B"]):
        for h in range(sh["Hq"]):
            for p in range(sh["T"]):
                ref = doc["sel"][b][h][p]
                assert list(sel[b, h, p, :len(ref)]) == ref
                assert np.all(sel[b, h, p, len(ref):] == -1)
                np.testing.assert_allclose(sc[b, h, p, :len(ref)], doc["sel_score"][b][h][p], atol=1e-12)
                np.testing.assert_allclose(out[b, h, p], doc["out"][b][h][p], atol=1e-12)
