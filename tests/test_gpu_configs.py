"""GPU parity at the five full workload sizes, in the launch configuration the
benchmark times: the whole layer runs at full size and sampled rows (all
rows for the 4K prefill) are checked against the oracle under the layer's
acceptance rule.  Landmarks of the sampled KV heads are checked bit for bit
(bf16) or to within one ulp (fp32).

Inputs come from the seeded generators in workloads.py; the oracle reads
them from the device (the same values the kernels read), never any output of
the HIP path."""
import gc

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd.workloads import WORKLOADS, decode_inputs, prefill_inputs
from oracle import hsa_oracle as O
from tests.gpu_util import TOL, check_rows, check_rows_adaptive, new_stats
from tests.oracle_pool import OraclePool, check_prefill_rows_task, gather_landmarks, merge_stats
from tests.oracle_pool import oracle_landmarks as pool_landmarks

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.fixture(autouse=True)
def release_device_memory():
    """Each workload needs most of the device: return what earlier tests
    left in torch's cache before the next one sizes itself."""
    gc.collect()
    torch.cuda.empty_cache()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def host64(t):
    return t.detach().float().cpu().double().numpy()


class DeviceRows:
    """[T, D] view of a device tensor for the oracle: fancy indexing fetches
    just the indexed rows as float64 (the caches are too large to copy)."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        idx = np.asarray(idx)
        rows = self.t[torch.as_tensor(idx.reshape(-1), device=self.t.device)]
        return host64(rows).reshape(idx.shape + (self.shape[-1],))


def oracle_landmarks(kg, S, dtype, slab=1 << 20):
    """Oracle landmarks of one KV head [T, D] on the device, slab by slab."""
    T = kg.shape[0]
    Nc = T // S
    parts = []
    for t0 in range(0, Nc * S, slab):
        t1 = min(Nc * S, t0 + slab)
        parts.append(O.landmarks(host64(kg[t0:t1]), S, dtype))
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, kg.shape[1]))


def host_stored(t):
    """Host copy of a device tensor as stored: bf16 as its uint16 bit
    patterns, everything else unchanged."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_landmarks(L_gpu, L_ref, dtype):
    got = host64(L_gpu)
    if dtype == "bf16":
        assert np.array_equal(got, L_ref), "bf16 landmarks must match the oracle bit for bit"
    else:
        ulp = np.spacing(np.abs(L_ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - L_ref) <= ulp), "fp32 landmarks must be within one ulp"


def run_prefill_workload(name, chunks, heads=None):
    w = WORKLOADS[name]
    off = int(w.extra.get("q_offset", 0))  # chunked prefill after a cached prefix
    print(f"workload {name}: sampled query chunks {chunks}", flush=True)
    q, k, v = prefill_inputs(w, "cuda")
    Nc = w.T // w.S
    Tq = w.T - off
    tau = w.extra.get("gap_threshold")  # near-tie adaptive budget
    kk = w.k if tau is None else 2 * w.k
    L = torch.empty((w.B, w.Hkv, Nc, w.D), dtype=k.dtype, device="cuda")
    out = torch.empty((w.B, w.Hq, Tq, w.D), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.B, w.Hq, Tq, kk), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, Tq, kk), dtype=torch.float32, device="cuda")
    if off:  # prefix landmarks first, then the new tokens' chunks, as the benchmark does
        hsa.hsa_build_landmarks(k, L, w.S, 0, off // w.S)
        hsa.hsa_build_landmarks(k, L, w.S, off // w.S, Nc)
        hsa.hsa_forward_prefill_cached(q[:, :, off:].contiguous(), k, v, L, off, w.S, w.k, out=out, sel_idx=sel,
                                       sel_score=sc)
    elif tau is not None:
        hsa.hsa_build_landmarks(k, L, w.S)
        hsa.hsa_forward_prefill_adaptive(q, k, v, L, w.S, w.k, tau, out=out, sel_idx=sel, sel_score=sc)
    else:
        hsa.hsa_build_landmarks(k, L, w.S)
        hsa.hsa_forward_prefill(q, k, v, L, w.S, w.k, out=out, sel_idx=sel, sel_score=sc)
    torch.cuda.synchronize()
    pos = np.concatenate([np.arange(c * w.S, min(w.T, (c + 1) * w.S)) for c in chunks]) if chunks is not None \
        else np.arange(off, w.T)
    assert pos.min() >= off
    pos_t = torch.as_tensor(pos, device="cuda")
    row_t = pos_t - off  # rows of the outputs
    G = w.Hq // w.Hkv
    stats = new_stats()
    for b in range(w.B):
        for g in range(w.Hkv):
            Kg, Vg = host64(k[b, g]), host64(v[b, g])
            Lg = O.landmarks(Kg, w.S, w.dtype)
            check_landmarks(L[b, g], Lg, w.dtype)
            for h in range(g * G, (g + 1) * G):
                if heads is not None and h not in heads:
                    continue
                args = (host64(q[b, h, pos_t]), pos, Kg, Vg, Lg, w.S, w.k)
                res = (host64(out[b, h, row_t]), sel[b, h, row_t].cpu().numpy(), host64(sc[b, h, row_t]))
                if tau is None:
                    check_rows(*args, *res, TOL[w.dtype], stats)
                else:
                    check_rows_adaptive(*args, tau, *res, TOL[w.dtype], stats)
    print(name, stats, flush=True)
    del q, k, v, L, out, sel, sc
    torch.cuda.empty_cache()
    return stats


def test_prefill_4k_fp32_every_row():
    stats = run_prefill_workload("prefill_4k_fp32", None)
    assert stats["rows"] == 4 * 4096


def test_prefill_32k_bf16_every_row():
    """Every row of every head of the 32K prefill, the oracle side split over
    a pool of worker processes (blocks of 1024 rows of one head)."""
    w = WORKLOADS["prefill_32k_bf16"]
    print(f"workload {w.name}: every row", flush=True)
    q, k, v = prefill_inputs(w, "cuda")
    Nc = w.T // w.S
    L = torch.empty((w.B, w.Hkv, Nc, w.D), dtype=k.dtype, device="cuda")
    out = torch.empty((w.B, w.Hq, w.T, w.D), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.B, w.Hq, w.T, w.k), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, w.T, w.k), dtype=torch.float32, device="cuda")
    hsa.hsa_build_landmarks(k, L, w.S)
    hsa.hsa_forward_prefill(q, k, v, L, w.S, w.k, out=out, sel_idx=sel, sel_score=sc)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    stats = new_stats()
    with OraclePool() as P:
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("sel", sel), ("sc", sc)):
            a = host_stored(t)
            m = P.array(name, a.shape, a.dtype)
            m[:] = a
            m.flush()
            del m, a
        futs = []
        for b in range(w.B):
            for h in range(w.Hq):
                for r0 in range(0, w.T, 1024):
                    futs.append(P.submit(check_prefill_rows_task, P.dir, b, h, h // G,
                                         np.arange(r0, min(w.T, r0 + 1024)), w.S, w.k, w.dtype, TOL[w.dtype]))
        for b in range(w.B):
            for g in range(w.Hkv):
                check_landmarks(L[b, g], O.landmarks(host64(k[b, g]), w.S, w.dtype), w.dtype)
        for i, f in enumerate(futs):
            merge_stats(stats, f.result())
            if (i + 1) % 128 == 0:
                print(f"{i + 1}/{len(futs)} row blocks checked: {stats}", flush=True)
    print(w.name, stats, flush=True)
    assert stats["rows"] == w.B * w.Hq * w.T


def test_prefill_256k_bf16_sampled():
    # the special chunks, chunks around window and segment edges, and chunks
    # spread over the sequence
    run_prefill_workload("prefill_256k_bf16", [0, 1, 16, 17, 63, 64, 65, 1000, 2047, 3333, 4095])


def test_prefill_256k_adaptive_bf16_sampled():
    stats = run_prefill_workload("prefill_256k_adaptive_bf16", [0, 1, 16, 17, 63, 64, 65, 2047, 4095])
    assert stats.get("doubled", 0) > 0


def test_prefill_256k_chunk_bf16_sampled():
    # the first new chunk, chunks at window edges, and the last
    run_prefill_workload("prefill_256k_chunk_bf16", [3072, 3073, 3135, 3136, 3500, 4095])


def test_prefill_256k_chunk_bf16_equals_full_prefill_rows():
    """Every output row of the chunked prefill equals the full-sequence
    prefill's row at the same position, bit for bit (same selection, same
    per-chunk arithmetic and fusion order)."""
    w = WORKLOADS["prefill_256k_chunk_bf16"]
    off = w.extra["q_offset"]
    Tq = w.T - off
    q, k, v = prefill_inputs(w, "cuda")
    Nc = w.T // w.S
    L = torch.empty((w.B, w.Hkv, Nc, w.D), dtype=k.dtype, device="cuda")
    hsa.hsa_build_landmarks(k, L, w.S)
    sel_f = torch.empty((w.B, w.Hq, w.T, w.k), dtype=torch.int32, device="cuda")
    sc_f = torch.empty((w.B, w.Hq, w.T, w.k), dtype=torch.float32, device="cuda")
    full = hsa.hsa_forward_prefill(q, k, v, L, w.S, w.k, sel_idx=sel_f, sel_score=sc_f)[:, :, off:].clone()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    sel = torch.empty((w.B, w.Hq, Tq, w.k), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, Tq, w.k), dtype=torch.float32, device="cuda")
    part = hsa.hsa_forward_prefill_cached(q[:, :, off:].contiguous(), k, v, L, off, w.S, w.k, sel_idx=sel,
                                          sel_score=sc)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_f[:, :, off:]) and torch.equal(sc, sc_f[:, :, off:])
    assert torch.equal(part, full)


def run_decode_workload(name, queries):
    w = WORKLOADS[name]
    esz = 2 if w.dtype == "bf16" else 4
    Nc = w.T // w.S
    need = 2 * w.B * w.Hkv * w.T * w.D * esz + w.B * w.Hkv * Nc * w.D * esz
    free, _ = torch.cuda.mem_get_info()
    if need + (2 << 30) > free:
        pytest.skip(f"{name} needs {need / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} GiB free")
    print(f"workload {name}: sampled queries {queries}", flush=True)
    tau = w.extra.get("gap_threshold")  # near-tie adaptive budget
    kk = w.k if tau is None else 2 * w.k
    q, k, v = decode_inputs(w, "cuda")
    L = torch.empty((w.B, w.Hkv, Nc, w.D), dtype=k.dtype, device="cuda")
    hsa.hsa_build_landmarks(k, L, w.S)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.B, w.Hq, kk), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, kk), dtype=torch.float32, device="cuda")
    if tau is None:
        hsa.hsa_forward_decode(q, k, v, L, w.S, w.k, out=out, sel_idx=sel, sel_score=sc)
    else:
        hsa.hsa_forward_decode_adaptive(q, k, v, L, w.S, w.k, tau, out=out, sel_idx=sel, sel_score=sc)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    stats = new_stats()

    def check_group(b, g, Lg):
        check_landmarks(L[b, g], Lg, w.dtype)
        hs = slice(g * G, (g + 1) * G)
        if tau is None:
            check_rows(host64(q[b, hs]), np.full(G, w.T), DeviceRows(k[b, g]), DeviceRows(v[b, g]), Lg, w.S,
                       w.k, host64(out[b, hs]), sel[b, hs].cpu().numpy(), host64(sc[b, hs]), TOL[w.dtype], stats)
        else:
            check_rows_adaptive(host64(q[b, hs]), np.full(G, w.T), DeviceRows(k[b, g]), DeviceRows(v[b, g]), Lg,
                                w.S, w.k, tau, host64(out[b, hs]), sel[b, hs].cpu().numpy(), host64(sc[b, hs]),
                                TOL[w.dtype], stats)
        if g == w.Hkv - 1:
            print(name, "query", b, stats, flush=True)

    # the oracle's landmarks of each (query, KV head) are built by the pool
    # from a shared-memory copy of the cache's keys, a few caches ahead of
    # the checks, which run here
    items = [(b, g) for b in queries for g in range(w.Hkv)]
    per_item = max(1, (Nc * w.S) // (1 << 20))               # slab tasks per cache
    depth = max(2, min(16, -(-28 // per_item), (8 << 30) // max(1, w.T * w.D * esz)))
    pending = []
    with OraclePool() as P:
        for i, (b, g) in enumerate(items):
            tag = f"k_{b}_{g}"
            m = P.array(tag, (w.T, w.D), np.uint16 if w.dtype == "bf16" else np.float32)
            m[:] = host_stored(k[b, g])
            m.flush()
            del m
            pending.append((b, g, tag, pool_landmarks(P, P.path(tag), (), w.T, w.S, w.dtype)))
            while len(pending) >= depth or (i == len(items) - 1 and pending):
                b0, g0, tag0, futs = pending.pop(0)
                Lg = gather_landmarks(futs, w.D)
                P.remove(tag0)
                check_group(b0, g0, Lg)
    print(name, stats, flush=True)
    del q, k, v, L, out, sel, sc
    torch.cuda.empty_cache()
    return stats


def test_decode_1m_bf16_sampled():
    # 16 of the 64 queries, spread over the batch
    stats = run_decode_workload("decode_1m_bf16", list(range(0, 64, 4)))
    assert stats["rows"] == 16 * 32


def test_decode_1m_adaptive_bf16_sampled():
    stats = run_decode_workload("decode_1m_adaptive_bf16", [0, 41])
    assert stats.get("doubled", 0) > 0


def test_decode_16m_bf16_every_query():
    stats = run_decode_workload("decode_16m_bf16", [0, 1, 2, 3])
    assert stats["rows"] == 4 * 32


def test_decode_1m_varlen_bf16_sampled():
    """Caches of seeded lengths inside the 2^20 capacity: each sampled query
    against the oracle on its own prefix."""
    from hierarchical_sparse_attention_hsa_amd.workloads import cache_lengths
    w = WORKLOADS["decode_1m_varlen_bf16"]
    Nc = w.T // w.S
    lens = cache_lengths(w)
    q, k, v = decode_inputs(w, "cuda")
    L = torch.empty((w.B, w.Hkv, Nc, w.D), dtype=k.dtype, device="cuda")
    hsa.hsa_build_landmarks(k, L, w.S)
    lens_t = torch.as_tensor(lens, device="cuda")
    sel = torch.empty((w.B, w.Hq, w.k), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, w.k), dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_decode_varlen(q, k, v, L, lens_t, w.S, w.k, sel_idx=sel, sel_score=sc)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    stats = new_stats()
    for b in (int(np.argmin(lens)), int(np.argmax(lens)), 5):
        n = int(lens[b])
        print(f"query {b}: cache length {n}", flush=True)
        for g in range(w.Hkv):
            Lg = oracle_landmarks(k[b, g, :n], w.S, w.dtype)
            check_landmarks(L[b, g, :n // w.S], Lg, w.dtype)
            hs = slice(g * G, (g + 1) * G)
            check_rows(host64(q[b, hs]), np.full(G, n), DeviceRows(k[b, g, :n]), DeviceRows(v[b, g, :n]), Lg, w.S,
                       w.k, host64(out[b, hs]), sel[b, hs].cpu().numpy(), host64(sc[b, hs]), TOL[w.dtype], stats)
    print(stats, flush=True)


def test_backward_256k_bf16_sampled():
    """The backward at full size in the benchmark's configuration.  The
    selection it is given is the forward's; every row used below has its
    selection validated against the oracle's rule first (exact, or a valid
    set within the near-tie band), and the oracle then differentiates with
    that same selection.  The GPU backward uses the GPU forward's output for
    delta = dOut . out, so the forward's own error enters ds; the bounds are
    those of the backward's arithmetic (dq: 2e-4 of the magnitude sums, the
    head + tail operands; dK, dV: 9e-3, the bf16 operands; plus 1e-6) plus
    that forward error: the max-abs difference eps between the GPU output
    row and the oracle's, measured per row (and itself held to the forward
    tolerance), times the oracle's output sensitivities (out_dq, out_dK),
    for dq of sampled rows and for dK, dV of two chunks summed over every
    row that kept them."""
    w = WORKLOADS["backward_256k_bf16"]
    S, D = w.S, w.D
    G = w.Hq // w.Hkv
    Nc = w.T // S
    q, k, v = prefill_inputs(w, "cuda")
    dout = torch.randn((w.B, w.Hq, w.T, D), dtype=torch.float32, device="cuda",
                       generator=torch.Generator("cuda").manual_seed(w.seed + 100))
    L = torch.empty((w.B, w.Hkv, Nc, D), dtype=k.dtype, device="cuda")
    hsa.hsa_build_landmarks(k, L, S)
    sel = torch.empty((w.B, w.Hq, w.T, w.k), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, w.T, w.k), dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_prefill(q, k, v, L, S, w.k, sel_idx=sel, sel_score=sc)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    dq, dk, dv = hsa.hsa_backward_prefill(q, k, v, L, out, dout, sel, sc, S)
    torch.cuda.synchronize()

    def rows_of(b, h, pos):
        pos_t = torch.as_tensor(pos, device="cuda")
        return host64(q[b, h, pos_t]), sel[b, h, pos_t].cpu().numpy(), host64(dout[b, h, pos_t])

    def forward_error(b, h, pos, ref):
        """Per-row max-abs error of the GPU forward output the backward used."""
        eps = np.abs(host64(out[b, h, torch.as_tensor(pos, device="cuda")]) - ref.out).max(axis=1)
        assert eps.max() <= 2e-3, f"forward output error {eps.max():.3e}"
        return eps

    def validated(qr, pos, Lg, sl):
        for r in range(len(pos)):
            n = int(O.num_candidates(np.array([pos[r]]), S, Nc)[0])
            ok, _, msg = O.check_selection(sl[r], qr[r], Lg, n, w.k)
            assert ok, f"position {pos[r]}: {msg}"

    b = 0
    Lh = {}
    for g in range(w.Hkv):
        Lh[g] = O.landmarks(host64(k[b, g]), S, w.dtype)
    # dq of sampled rows
    pos = np.concatenate([np.arange(c * S, (c + 1) * S) for c in (1, 17, 64, 1000, 4095)])
    for h in (0, 13, 31):
        g = O.kv_head_of(h, w.Hq, w.Hkv)
        qr, sl, gr = rows_of(b, h, pos)
        validated(qr, pos, Lh[g], sl)
        ref = O.hsa_rows_backward(qr, pos, DeviceRows(k[b, g]), DeviceRows(v[b, g]), Lh[g], S, sl, gr)
        eps = forward_error(b, h, pos, ref)
        got = host64(dq[b, h, torch.as_tensor(pos, device="cuda")])
        err = np.abs(got - ref.dq)
        bound = 2e-4 * ref.abs_dq + eps[:, None] * ref.out_dq + 1e-6
        print(f"dq head {h}: forward error {eps.max():.3e}, worst error / bound {(err / bound).max():.3f}", flush=True)
        assert np.all(err <= bound), f"dq head {h}: worst {err.max():.3e}"
    # dK, dV of two chunks of KV head 2: every (head, row) that kept them
    g = 2
    for c in (100, 3000):
        acc_k = np.zeros((S, D))
        acc_v = np.zeros((S, D))
        abs_k = np.zeros((S, D))
        abs_v = np.zeros((S, D))
        fwd_k = np.zeros((S, D))
        for h in range(g * G, (g + 1) * G):
            rows = torch.nonzero((sel[b, h] == c).any(dim=-1)).flatten().cpu().numpy()
            if rows.size == 0:
                continue
            qr, sl, gr = rows_of(b, h, rows)
            validated(qr, rows, Lh[g], sl)
            ref = O.hsa_rows_backward(qr, rows, DeviceRows(k[b, g]), DeviceRows(v[b, g]), Lh[g], S, sl, gr)
            fwd_k += forward_error(b, h, rows, ref).max() * ref.out_dK[c * S:(c + 1) * S]
            acc_k += ref.dK[c * S:(c + 1) * S]
            acc_v += ref.dV[c * S:(c + 1) * S]
            abs_k += ref.abs_dK[c * S:(c + 1) * S]
            abs_v += ref.abs_dV[c * S:(c + 1) * S]
        got_k = host64(dk[b, g, c * S:(c + 1) * S])
        got_v = host64(dv[b, g, c * S:(c + 1) * S])
        print(f"chunk {c}: max |dK| {np.abs(acc_k).max():.3e}, |dV| {np.abs(acc_v).max():.3e}", flush=True)
        assert np.all(np.abs(got_k - acc_k) <= 9e-3 * abs_k + fwd_k + 1e-6), f"dK chunk {c}"
        assert np.all(np.abs(got_v - acc_v) <= 9e-3 * abs_v + 1e-6), f"dV chunk {c}"
    del q, k, v, L, sel, sc, out, dq, dk, dv, dout
