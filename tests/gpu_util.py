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


def check_rows_adaptive(q_row, pos, Kg, Vg, Lg, S, k, tau, gpu_out, gpu_sel, gpu_score, tol, stats):
    """One query row under the near-tie adaptive budget (base k, threshold
    tau).  The kept count (valid entries of gpu_sel, 2k slots) must be the
    oracle's unless the oracle's fp64 k-th vs (k+1)-th gap lies within the
    fp32 score error band of tau, where either count is valid; the kept set
    and output are then checked as a plain top-m row."""
    n = int(O.num_candidates(np.array([pos]), S, Kg.shape[0] // S)[0])
    m = int((gpu_sel >= 0).sum())
    if n <= k:
        allowed = {n}
    else:
        s = O.scores_for_rows(q_row[None], Lg, n)[0]
        order = O.select_topk(s[None], 2 * k)[0]
        want, gap = O.adaptive_keep_count(s[order], k, tau)
        allowed = {want}
        _, band, _ = O.near_tie_info(q_row, Lg, n, k)
        if abs(gap - tau) <= 2 * band:
            allowed = {k, min(2 * k, n)}
            stats["ambiguous"] = stats.get("ambiguous", 0) + 1
    if m not in allowed:
        raise Mismatch(f"kept {m} chunks, expected {sorted(allowed)} (tau {tau})")
    if np.any(gpu_sel[m:] != -1):
        raise Mismatch(f"padding expected after slot {m}: {gpu_sel}")
    stats["doubled"] = stats.get("doubled", 0) + int(m > k)
    mm = max(m, 1)
    check_rows(q_row[None], np.array([pos]), Kg, Vg, Lg, S, mm, gpu_out[None], gpu_sel[:mm][None],
               gpu_score[:mm][None], tol, stats)
