"""Seeded synthetic inputs for tests and the benchmark.

Holds none of the layer's arithmetic: it only draws Q, K and V with the
shapes and value structure of the workloads below, and is shared by the
tests, the benchmark and (through the tests) the oracle.  Values are drawn in
fp32 and rounded once (round-to-nearest-even) to the storage dtype.

Workloads (all with chunk size 64):

  prefill_4k_fp32    B=1, T=4096, Hq=Hkv=4, D=64, k=8, fp32, N(0,1)
  prefill_32k_bf16   B=1, T=32768, Hq=32, Hkv=8, D=128, k=16, bf16, N(0,1)/sqrt(128)
  decode_1m_bf16     B=64 queries, each after its own 2^20-token cache, Hq=32,
                     Hkv=8, D=128, k=32, bf16, N(0,1), 8 needle chunks per cache
  prefill_256k_bf16  B=1, T=262144, Hq=32, Hkv=8, D=128, k=16, bf16, N(0,1)
                     plus a rank-8 component shared per 4096-token segment
  decode_16m_bf16    B=4 queries, 2^24-token caches, k=64, 16 needles per cache
  decode_1m_varlen_bf16  as decode_1m_bf16 in caches of capacity 2^20 that
                     hold seeded lengths in [2^19, 2^20) (cache_lengths)
  decode_1m_adaptive_bf16  decode_1m_bf16's inputs with the near-tie adaptive
                     budget, base k=16 (2k=32), gap threshold 1.25e-3 (the
                     0.25 quantile of these heads' k-th vs (k+1)-th gaps)
  prefill_256k_adaptive_bf16  prefill_256k_bf16's inputs with the near-tie
                     adaptive budget, base k=16 (2k=32), gap threshold 1e-2
                     (about the 0.25 quantile of the rows' 16th vs 17th gaps)
  backward_256k_bf16  the backward pass of prefill_256k_bf16 (its inputs,
                     selection and output; dOut ~ N(0, 1) fp32, seed 4100)
  prefill_256k_chunk_bf16  the last 65536 tokens of prefill_256k_bf16 over
                     its cached first 196608 tokens

Needles: per cache, distinct chunk indices drawn uniformly; every key of a
needle chunk gets 3 * u added (before rounding), u = the normalised sum of
the G query vectors of the KV group, the same chunks for every KV head.
Low-rank component: for segment s and KV head g, B_sg has N(0, 1/8) entries
(D x 8) and a_sg ~ N(0, I_8); token t of s draws e_t ~ N(0, I_8) and
B_sg (a_sg + e_t) is added to K[g, t], V[g, t] and Q[h, t] for h in group g.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "small_inputs", "prefill_inputs", "decode_inputs", "needle_chunks",
           "cache_lengths"]


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    Hq: int
    Hkv: int
    T: int
    D: int
    S: int
    k: int
    dtype: str           # "bf16" or "fp32"
    seed: int
    scale: float = 1.0   # multiplies the N(0,1) draws
    needles: int = 0     # decode only
    lowrank: int = 0     # prefill only: rank of the per-segment component
    segment: int = 4096
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    w.name: w for w in [
        Workload("prefill_4k_fp32", "prefill", 1, 4, 4, 4096, 64, 64, 8, "fp32", 1000),
        Workload("prefill_32k_bf16", "prefill", 1, 32, 8, 32768, 128, 64, 16, "bf16", 2000,
                 scale=1.0 / math.sqrt(128)),
        Workload("decode_1m_bf16", "decode", 64, 32, 8, 1 << 20, 128, 64, 32, "bf16", 3000, needles=8),
        Workload("prefill_256k_bf16", "prefill", 1, 32, 8, 262144, 128, 64, 16, "bf16", 4000, lowrank=8),
        Workload("decode_16m_bf16", "decode", 4, 32, 8, 1 << 24, 128, 64, 64, "bf16", 5000, needles=16),
        # incremental decoding: caches of capacity 2^20 holding 2^19 .. 2^20
        # tokens each; every step decodes one query per sequence and appends
        # one token
        Workload("decode_1m_varlen_bf16", "decode", 64, 32, 8, 1 << 20, 128, 64, 32, "bf16", 6000, needles=8,
                 extra={"min_len": 1 << 19}),
        # decode_1m with the near-tie adaptive budget: base k = 16 (2k = 32);
        # the gap threshold doubles about a quarter of the heads here
        Workload("decode_1m_adaptive_bf16", "decode", 64, 32, 8, 1 << 20, 128, 64, 16, "bf16", 3000, needles=8,
                 extra={"gap_threshold": 1.25e-3}),
        # prefill_256k with the near-tie adaptive budget: base k = 16 (2k =
        # 32); the gap threshold doubles about a quarter of the rows here
        Workload("prefill_256k_adaptive_bf16", "prefill", 1, 32, 8, 262144, 128, 64, 16, "bf16", 4000, lowrank=8,
                 extra={"gap_threshold": 1e-2}),
        # backward pass of prefill_256k (same inputs; dOut seeded N(0, 1))
        Workload("backward_256k_bf16", "backward", 1, 32, 8, 262144, 128, 64, 16, "bf16", 4000, lowrank=8),
        # chunked prefill: the last 64K tokens of the 256K sequence after a
        # cached prefix of 192K tokens (same inputs as prefill_256k_bf16)
        Workload("prefill_256k_chunk_bf16", "prefill", 1, 32, 8, 262144, 128, 64, 16, "bf16", 4000, lowrank=8,
                 extra={"q_offset": 196608}),
    ]
}


def _torch():
    import torch
    return torch


def _storage(dtype: str):
    torch = _torch()
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def small_inputs(B, Hq, Hkv, T, D, dtype="bf16", seed=0, scale=1.0, decode=False):
    """Small seeded inputs drawn with numpy on the host; returns CPU torch
    tensors (q, k, v) in the storage dtype.  decode=True gives q [B, Hq, D]."""
    torch = _torch()
    r = np.random.default_rng(seed)
    qshape = (B, Hq, D) if decode else (B, Hq, T, D)
    q = r.standard_normal(qshape, dtype=np.float32) * np.float32(scale)
    k = r.standard_normal((B, Hkv, T, D), dtype=np.float32) * np.float32(scale)
    v = r.standard_normal((B, Hkv, T, D), dtype=np.float32) * np.float32(scale)
    st = _storage(dtype)
    return tuple(torch.from_numpy(x).to(st) for x in (q, k, v))


def _gen(device, seed):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def prefill_inputs(w: Workload, device="cuda"):
    """Q [B,Hq,T,D], K, V [B,Hkv,T,D] in the storage dtype, drawn on `device`."""
    torch = _torch()
    st = _storage(w.dtype)
    G = w.Hq // w.Hkv
    gq, gk, gv, gl = (_gen(device, w.seed + i) for i in (0, 1, 2, 4))
    q = torch.empty((w.B, w.Hq, w.T, w.D), dtype=st, device=device)
    k = torch.empty((w.B, w.Hkv, w.T, w.D), dtype=st, device=device)
    v = torch.empty((w.B, w.Hkv, w.T, w.D), dtype=st, device=device)
    for b in range(w.B):
        for g in range(w.Hkv):
            kf = torch.randn((w.T, w.D), generator=gk, device=device) * w.scale
            vf = torch.randn((w.T, w.D), generator=gv, device=device) * w.scale
            qf = torch.randn((G, w.T, w.D), generator=gq, device=device) * w.scale
            if w.lowrank:
                nseg = (w.T + w.segment - 1) // w.segment
                for s in range(nseg):
                    t0, t1 = s * w.segment, min(w.T, (s + 1) * w.segment)
                    Bm = torch.randn((w.D, w.lowrank), generator=gl, device=device) / math.sqrt(w.lowrank)
                    a = torch.randn((w.lowrank,), generator=gl, device=device)
                    e = torch.randn((t1 - t0, w.lowrank), generator=gl, device=device)
                    comp = (a[None, :] + e) @ Bm.T
                    kf[t0:t1] += comp
                    vf[t0:t1] += comp
                    qf[:, t0:t1] += comp[None]
            k[b, g] = kf.to(st)
            v[b, g] = vf.to(st)
            q[b, g * G:(g + 1) * G] = qf.to(st)
    return q, k, v


def needle_chunks(w: Workload, b: int, device="cpu"):
    """The needle chunk indices of cache b (same for every KV head)."""
    r = np.random.default_rng([w.seed + 3, b])
    return np.sort(r.choice(w.T // w.S, size=w.needles, replace=False))


def decode_inputs(w: Workload, device="cuda", slab_tokens=1 << 21, progress=None):
    """q [B,Hq,D] and caches K, V [B,Hkv,T,D] in the storage dtype, drawn on
    `device` in slabs of `slab_tokens` tokens (no full-size fp32 temporaries),
    with needle chunks planted in K."""
    torch = _torch()
    st = _storage(w.dtype)
    G = w.Hq // w.Hkv
    gq, gk, gv = (_gen(device, w.seed + i) for i in (0, 1, 2))
    q = (torch.randn((w.B, w.Hq, w.D), generator=gq, device=device) * w.scale).to(st)
    k = torch.empty((w.B, w.Hkv, w.T, w.D), dtype=st, device=device)
    v = torch.empty((w.B, w.Hkv, w.T, w.D), dtype=st, device=device)
    qf = q.float()
    for b in range(w.B):
        chunks = needle_chunks(w, b) if w.needles else np.zeros(0, dtype=np.int64)
        for g in range(w.Hkv):
            u = qf[b, g * G:(g + 1) * G].sum(dim=0)
            u = u / u.norm()
            for t0 in range(0, w.T, slab_tokens):
                t1 = min(w.T, t0 + slab_tokens)
                kf = torch.randn((t1 - t0, w.D), generator=gk, device=device) * w.scale
                for c in chunks:
                    c0, c1 = int(c) * w.S, int(c) * w.S + w.S
                    if c0 < t1 and c1 > t0:
                        kf[max(c0, t0) - t0:min(c1, t1) - t0] += 3.0 * u
                k[b, g, t0:t1] = kf.to(st)
                del kf
                vf = torch.randn((t1 - t0, w.D), generator=gv, device=device) * w.scale
                v[b, g, t0:t1] = vf.to(st)
                del vf
        if progress:
            progress(b)
    return q, k, v


def cache_lengths(w: Workload):
    """Seeded per-sequence cache lengths of a varlen decode workload."""
    r = np.random.default_rng([w.seed + 5])
    return r.integers(w.extra.get("min_len", w.T), w.T, size=w.B, endpoint=False).astype(np.int64)
