"""Writes the stored expected values under tests/golden/ from the oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
It calls only ``oracle.brute`` (pure Python, exact-rational landmarks and
selection) on small seeded inputs whose values are exact in bf16 (fp32 cases
use dyadic values with few bits).  The inputs are stored next to the outputs,
so the fixture does not depend on any random-number library's stream.
"""
import json
import os
import random
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from oracle import brute  # noqa: E402


def dyadic(r):
    # multiples of 1/32 in [-4, 4): exact in bf16 (at most 8 significant bits)
    return r.randrange(-128, 128) / 32.0


def make(name, seed, B, Hq, Hkv, T, D, S, k, dtype):
    r = random.Random(seed)
    Q = [[[[dyadic(r) for _ in range(D)] for _ in range(T)] for _ in range(Hq)] for _ in range(B)]
    K = [[[[dyadic(r) for _ in range(D)] for _ in range(T)] for _ in range(Hkv)] for _ in range(B)]
    V = [[[[dyadic(r) for _ in range(D)] for _ in range(T)] for _ in range(Hkv)] for _ in range(B)]
    out, sel, sc = brute.prefill(Q, K, V, S, k, dtype)
    lms = [[[brute.landmark(K[b][g][c * S:(c + 1) * S], dtype) for c in range(T // S)]
            for g in range(Hkv)] for b in range(B)]
    doc = {"about": "HSA forward on dyadic inputs; expected values from oracle.brute",
           "shape": dict(B=B, Hq=Hq, Hkv=Hkv, T=T, D=D, S=S, k=k, dtype=dtype),
           "Q": Q, "K": K, "V": V, "landmarks": lms,
           "out": out, "sel": sel, "sel_score": sc}
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(doc, f)


if __name__ == "__main__":
    make("tiny_gqa_bf16.json", 20251128, 1, 4, 2, 20, 4, 4, 2, "bf16")
    make("tiny_mha_fp32.json", 11, 2, 2, 2, 13, 4, 3, 3, "fp32")
