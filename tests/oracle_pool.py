"""A pool of CPU worker processes for the oracle side of the full-size parity
tests.

The oracle is plain numpy, one row group at a time; checking every row of the
32K-token prefill, or building the oracle's landmarks of 16M-token caches,
serially would take far longer than the GPU work it checks.  Workers are
spawned (fresh interpreters that import numpy, the oracle and the row
checker only: never torch, never the library), take their inputs from files
in shared memory written by the test process, and return plain results.
Each worker runs numpy with one BLAS thread.  The arithmetic is the
oracle's own; the pool only splits rows and landmark ranges among processes.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

WORKERS = 14  # the GPU machine gives one GPU's run 16 host cores: 14 workers and the test process


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


class OraclePool:
    """Context manager: a spawned process pool plus a scratch directory in
    shared memory for the arrays the tasks read."""

    def __init__(self, workers: int = WORKERS):
        base = "/dev/shm" if os.path.isdir("/dev/shm") else tempfile.gettempdir()
        self.dir = tempfile.mkdtemp(prefix="hsa_oracle_", dir=base)
        self.ex = cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                                         initializer=_init_worker)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.ex.shutdown(wait=True, cancel_futures=True)
        shutil.rmtree(self.dir, ignore_errors=True)

    def array(self, name: str, shape, dtype) -> np.memmap:
        """A writable array in shared memory that tasks open by name."""
        return np.lib.format.open_memmap(os.path.join(self.dir, name + ".npy"), mode="w+", dtype=dtype,
                                         shape=tuple(shape))

    def path(self, name: str) -> str:
        return os.path.join(self.dir, name + ".npy")

    def remove(self, name: str):
        try:
            os.remove(self.path(name))
        except FileNotFoundError:
            pass

    def submit(self, fn, *args):
        return self.ex.submit(fn, *args)


def _load(path):
    return np.load(path, mmap_mode="r")


def values64(a, dtype: str) -> np.ndarray:
    """Exact float64 values of stored data: bf16 arrives as its uint16 bit
    patterns, fp32 as float32."""
    from oracle import hsa_oracle as O
    a = np.asarray(a)
    if dtype == "bf16":
        return O.bf16_bits_to_f64(a)
    return a.astype(np.float64)


def landmarks_task(path: str, index, r0: int, r1: int, S: int, dtype: str) -> np.ndarray:
    """Oracle landmarks of rows [r0, r1) of the key array at path[index]
    (r0 and r1 multiples of S)."""
    from oracle import hsa_oracle as O
    k = values64(_load(path)[index][r0:r1], dtype)
    return O.landmarks(k, S, dtype)


def oracle_landmarks(pool: OraclePool, path: str, index, T: int, S: int, dtype: str, slab: int = 1 << 20):
    """Futures of the oracle landmarks of one KV head's keys, slab by slab;
    join with gather_landmarks."""
    Nc = T // S
    return [pool.submit(landmarks_task, path, index, t0, min(Nc * S, t0 + slab), S, dtype)
            for t0 in range(0, Nc * S, slab)]


def gather_landmarks(futs, D: int) -> np.ndarray:
    parts = [f.result() for f in futs]
    return np.concatenate(parts, axis=0) if parts else np.zeros((0, D))


_LM_CACHE = {}


def check_prefill_rows_task(d: str, b: int, h: int, g: int, rows: np.ndarray, S: int, k: int, dtype: str,
                            tol: float, off: int = 0):
    """Check query rows `rows` (positions) of head h against the oracle under
    the layer's acceptance rule (tests.gpu_util.check_rows).  Inputs are the
    .npy files in directory d: q [B,Hq,Tq,D] and k, v [B,Hkv,T,D] (bf16 bits
    or fp32), out [B,Hq,Tq,D] float32, sel [B,Hq,Tq,k] int32, sc float32;
    q and the outputs hold positions off.. .  The oracle's landmarks of (b, g)
    are built once per worker process.  Returns the row statistics."""
    from oracle import hsa_oracle as O
    from tests.gpu_util import check_rows, new_stats
    key = (d, b, g)
    if key not in _LM_CACHE:
        _LM_CACHE.clear()
        K = values64(_load(os.path.join(d, "k.npy"))[b, g], dtype)
        _LM_CACHE[key] = (K, values64(_load(os.path.join(d, "v.npy"))[b, g], dtype), O.landmarks(K, S, dtype))
    K, V, L = _LM_CACHE[key]
    rows = np.asarray(rows, dtype=np.int64)
    r = rows - off
    q = values64(_load(os.path.join(d, "q.npy"))[b, h][r], dtype)
    out = np.asarray(_load(os.path.join(d, "out.npy"))[b, h][r], dtype=np.float64)
    sel = np.asarray(_load(os.path.join(d, "sel.npy"))[b, h][r])
    sc = np.asarray(_load(os.path.join(d, "sc.npy"))[b, h][r], dtype=np.float64)
    stats = new_stats()
    check_rows(q, rows, K, V, L, S, k, out, sel, sc, tol, stats)
    return stats


def merge_stats(total: dict, part: dict):
    for key, v in part.items():
        if key == "max_err":
            total[key] = max(total.get(key, 0.0), v)
        else:
            total[key] = total.get(key, 0) + v
    return total
