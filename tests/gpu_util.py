"""Helpers shared by the GPU parity tests: run the HIP path through the C-ABI
binding and compare with the CPU oracle under the layer's acceptance rule
(exact selected chunk indices except near ties, max-abs output tolerance)."""
import numpy as np

from oracle import hsa_oracle as O

TOL = {"bf16": 2e-3, "fp32": 1e-5}


def f64(t):
    """Exact float64 values of a (CPU or GPU) torch tensor."""
    return t.detach().float().cpu().double().numpy()


def storage_name(t):
    import torch
    return "bf16" if t.dtype == torch.bfloat16 else "fp32"


class Mismatch(AssertionError):
    pass


def check_rows(q_rows, pos, Kg, Vg, Lg, S, k, gpu_out, gpu_sel, gpu_score, tol, stats):
    """Compare a set of query rows of one (b, h) against the oracle.

    q_rows [R, D], pos [R]: query values and positions; Kg, Vg [T, D] and Lg
    the oracle's landmarks of the KV head; gpu_* are the GPU outputs of those
    rows.  Updates stats (rows, near_tie_rows, exact) and raises on failure.
    """
    ref = O.hsa_rows(q_rows, pos, Kg, Vg, Lg, S, k)
    override = {}
    for r in range(q_rows.shape[0]):
        n = int(ref.n[r])
        ok, exact, msg = O.check_selection(gpu_sel[r], q_rows[r], Lg, n, k)
        if not ok:
            raise Mismatch(f"row {r} (pos {pos[r]}): {msg}")
        stats["rows"] += 1
        if not exact:
            stats["near_tie_rows"] += 1
            override[r] = [int(c) for c in gpu_sel[r] if c >= 0]
        else:
            m = min(k, n)
            # slot order: scores non-increasing, exact score ties by index
            sc = gpu_score[r, :m]
            if m > 1 and np.any(np.diff(sc) > 0):
                raise Mismatch(f"row {r}: slot scores not sorted: {sc}")
            ids = gpu_sel[r, :m]
            if m > 1 and np.any((np.diff(sc) == 0) & (np.diff(ids) < 0)):
                raise Mismatch(f"row {r}: equal scores not in ascending chunk order: {list(ids)} {list(sc)}")
            np.testing.assert_allclose(np.sort(sc), np.sort(ref.sel_score[r, :m]), rtol=1e-4, atol=1e-5,
                                       err_msg=f"row {r} retrieval scores")
    expect = ref.out.copy()
    if override:
        rows = np.array(sorted(override))
        alt = O.hsa_rows(q_rows[rows], pos[rows], Kg, Vg, Lg, S, k, sel_override=[override[r] for r in rows])
        expect[rows] = alt.out
    err = np.abs(gpu_out - expect)
    stats["max_err"] = max(stats.get("max_err", 0.0), float(err.max()) if err.size else 0.0)
    if err.size and err.max() > tol:
        r = int(np.argmax(err.max(axis=1)))
        raise Mismatch(f"output error {err.max():.3e} > {tol} at row {r} (pos {pos[r]})")


def new_stats():
    return {"rows": 0, "near_tie_rows": 0, "max_err": 0.0}


def check_rows_adaptive(q_rows, pos, Kg, Vg, Lg, S, k, tau, gpu_out, gpu_sel, gpu_score, tol, stats):
    """Query rows of one (b, h) under the near-tie adaptive budget (base k,
    threshold tau); gpu_sel/gpu_score have 2k slots per row.  A row's kept
    count (its valid slots) must be the oracle's unless the oracle's fp64
    k-th vs (k+1)-th gap lies within the fp32 score error band of tau, where
    either count is valid; the kept sets and outputs are then checked as
    plain top-m rows (check_rows), grouped by m."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    D = q_rows.shape[1]
    n_all = O.num_candidates(pos, S, Kg.shape[0] // S)
    m_gpu = (gpu_sel >= 0).sum(axis=1)
    for r in range(len(pos)):
        if np.any(gpu_sel[r, m_gpu[r]:] != -1):
            raise Mismatch(f"row {r} (pos {pos[r]}): padding expected after slot {m_gpu[r]}: {gpu_sel[r]}")
    for n in np.unique(n_all):
        rows = np.nonzero(n_all == n)[0]
        n = int(n)
        if n <= k:
            bad = rows[m_gpu[rows] != n]
            if bad.size:
                raise Mismatch(f"row {bad[0]} (pos {pos[bad[0]]}): kept {m_gpu[bad[0]]}, expected all {n}")
            continue
        s = O.scores_for_rows(q_rows[rows], Lg, n)
        order = O.select_topk(s, 2 * k)
        ss = np.take_along_axis(s, order, axis=1)
        A = (np.abs(q_rows[rows]) @ np.abs(Lg[:n]).T) / np.sqrt(D)  # fp32 error scale of each score
        for i, r in enumerate(rows):
            want, gap = O.adaptive_keep_count(ss[i], k, tau)
            a, b = order[i, k - 1], order[i, k]
            band = 1e-5 * max(abs(s[i, a]), abs(s[i, b]), A[i, a], A[i, b])
            allowed = {want}
            if abs(gap - tau) <= 2 * band:
                allowed = {k, min(2 * k, n)}
                stats["ambiguous"] = stats.get("ambiguous", 0) + 1
            if int(m_gpu[r]) not in allowed:
                raise Mismatch(f"row {r} (pos {pos[r]}): kept {m_gpu[r]}, expected {sorted(allowed)} "
                               f"(gap {gap}, tau {tau})")
    stats["doubled"] = stats.get("doubled", 0) + int((m_gpu > k).sum())
    for m in np.unique(m_gpu):
        rows = np.nonzero(m_gpu == m)[0]
        mm = max(int(m), 1)
        check_rows(q_rows[rows], pos[rows], Kg, Vg, Lg, S, mm, gpu_out[rows], gpu_sel[rows, :mm],
                   gpu_score[rows, :mm], tol, stats)
