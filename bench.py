"""Benchmark of the HSA forward layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME|all] [--no-cpu-baseline]

Workloads (seeded, synthetic, shapes of the layer's published use: 1M- and
16M-token decode, 256K-token prefill; see hierarchical_sparse_attention_hsa_amd/workloads.py):
  decode_1m_bf16     step = hsa_forward_decode over 64 queries (landmarks
                     precomputed, as the workload defines), metric queries/s
  prefill_256k_bf16  step = hsa_build_landmarks + hsa_forward_prefill over
                     the 262144-token sequence, metric tokens/s
  decode_16m_bf16, prefill_32k_bf16, prefill_4k_fp32 on request.

The default (`all`) times prefill_256k_bf16 and then decode_1m_bf16 and prints
ONE JSON line: `value` is the 1M decode throughput (queries/s); the prefill
result rides along under "prefill".  Each timed region: W warm-up steps, then
K steps bracketed by torch.cuda.synchronize(); inputs are resident in HBM.
The step rate comes from K steps without timing events; per-kernel durations
come from K more steps in which the library records HIP events around each
of its launches on the same stream (hsa_attn_set_timing_events).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "HSA layer queries/s + achieved HBM GB/s (1M decode); tokens/s + MFMA% (256K prefill)"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
# the prefill kernels' split of window chunks between the local and the
# chunk-major attention (HSA_LOCAL_MIN_ROWS in csrc/prefill_kernels.hpp)
LOCAL_MIN_ROWS = 8
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- HIP events
class HipEvents:
    """Raw hipEvent_t handles (created with the HIP runtime) so that the
    library can record them on its own launch stream."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            out.append(e.value)
        self.pool += out
        return out

    def ms(self, a, b):
        t = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(t.value)


def timed_steps(step, steps, warmup, n_launch, events):
    """Run `warmup` untimed steps, then `steps` steps with timing events
    recorded around every launch, then the `steps` timed steps without them.
    Returns (seconds of the plain timed steps, per-launch mean durations in
    ms, seconds of the instrumented steps).  The step rate comes from the
    plain steps: the events add a few microseconds per launch (about 4% of a
    1M decode step), which the kernels themselves do not see; running the
    instrumented steps first also lets the GPU reach its steady clocks
    before the timed region (the first 20 decode steps after 5 warm-up steps
    run about 3% slower than the following ones)."""
    import torch
    import hierarchical_sparse_attention_hsa_amd as hsa
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    evs = [events.create(2 * n_launch) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t_events = time.perf_counter() - t0
    hsa.hsa_attn_set_timing_events(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(None)
    torch.cuda.synchronize()
    t_plain = time.perf_counter() - t0
    per = np.zeros(n_launch)
    for i in range(steps):
        for j in range(n_launch):
            per[j] += events.ms(evs[i][2 * j], evs[i][2 * j + 1])
    return t_plain, per / steps, t_events


def library_digest():
    """Digest of the built library (the build is deterministic for a given
    checkout path, and comments do not change it)."""
    import hashlib
    path = os.path.join(ROOT, "hierarchical_sparse_attention_hsa_amd", "libhsa_attn.so")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def device_code_digest():
    """Digest of the library's device code: its .hip_fatbin section, every
    kernel as compiled.  Host-side changes (argument checks, workspace
    planning) leave it unchanged, so counters taken for the kernels stay
    valid across them; any kernel change alters it.  (hipcc embeds
    compilation-unit ids derived from the source paths, so a build from
    another checkout path differs and reads as changed.)"""
    import hashlib
    import struct
    path = os.path.join(ROOT, "hierarchical_sparse_attention_hsa_amd", "libhsa_attn.so")
    data = open(path, "rb").read()
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)

    def header(i):  # name, type, flags, addr, offset, size, ...
        return struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize)

    names = header(shstrndx)[4]
    for i in range(shnum):
        h = header(i)
        if data[names + h[0]: data.index(b"\0", names + h[0])] == b".hip_fatbin":
            return hashlib.sha256(data[h[4]: h[4] + h[5]]).hexdigest()[:16]
    return None


def profile_is_current(rec):
    """A committed counter record applies to the built kernels: same device
    code (or, for a record without that key, the same library)."""
    if "device_code_sha256_16" in rec:
        return rec["device_code_sha256_16"] == device_code_digest()
    return rec.get("library_sha256_16") == library_digest()


def profiled_traffic(workload, kernel_prefix):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    record (profiles/<workload>.traffic.json: 128-byte read requests and
    WRITE_SIZE), or None when the built kernels differ from the profiled ones."""
    path = os.path.join(ROOT, "profiles", f"{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if not profile_is_current(rec):
        return None
    for name, b in rec["traffic_bytes_per_launch"].items():
        if kernel_prefix in name:
            return b
    return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def host_info():
    """Where the oracle baseline ran: host cores this process may use (its
    affinity set), the CPU model, and numpy with the BLAS it calls (and that
    BLAS's thread count, the threads the oracle actually uses)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [f"{p.get('internal_api')} {p.get('version')} ({p.get('num_threads')} threads)"
                for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:
        pass
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model, "numpy": np.__version__,
            "blas": blas}


def near_tie_rows(q_rows, Lg, n, k, rel=1e-5):
    """Rows whose cut is a near tie under the layer's acceptance rule, counted
    by rescoring in fp64 on the device: with m = min(k, n) < n, the m-th and
    (m+1)-th best scores s_m, s_m+1 (q.L/sqrt(D)) differ by less than
    rel * max(|s_m|, |s_m+1|, A_m, A_m+1), A_c = sum_d |q_d| |L_cd| / sqrt(D).
    q_rows [R, D] and Lg [Nc, D] are device tensors in the storage dtype,
    n [R] the rows' candidate counts (a device int64 tensor).  Returns
    (near-tie rows, rows with a cut)."""
    import torch
    D = q_rows.shape[-1]
    qd = q_rows.double()
    Ld = Lg.double()
    s = (qd @ Ld.T) / math.sqrt(D)
    cols = torch.arange(Ld.shape[0], device=s.device)
    s.masked_fill_(cols[None, :] >= n[:, None], -math.inf)
    m = torch.clamp(n, max=k)
    cut = m < n
    if not bool(cut.any()):
        return 0, 0
    kk = min(k + 1, Ld.shape[0])
    top, idx = torch.topk(s, kk, dim=1)
    r = torch.arange(s.shape[0], device=s.device)
    mi = (m - 1).clamp(min=0, max=kk - 2)
    a, b = top[r, mi], top[r, mi + 1]
    ia, ib = idx[r, mi], idx[r, mi + 1]
    A = lambda i: (qd.abs() * Ld[i].abs()).sum(-1) / math.sqrt(D)  # noqa: E731
    mu = torch.maximum(torch.maximum(a.abs(), b.abs()), torch.maximum(A(ia), A(ib)))
    tie = cut & (a - b < rel * mu)
    return int(tie.sum().item()), int(cut.sum().item())


def summarize_profile(workload, prof_dir, command, kernel, out_dir=None):
    """Turn the rocprofv3 CSVs of one workload (<workload>_kernel_stats.csv,
    _RDREQ.csv, _WRITE_SIZE.csv and _MFMA.csv in prof_dir) into
    profiles/<kernel>.<workload>.md, named for the dominant kernel (kernel
    times, HBM bytes, MFMA counters), and profiles/<workload>.traffic.json
    (bytes per launch, read by the benchmark).

    Bytes follow from the counters' definitions.  Reads: the L2 of gfx950
    sends 128-byte read requests to memory (TCC_EA0_RDREQ) and 32-byte ones
    (TCC_EA0_RDREQ_32B, counted among the former), so read bytes =
    128 (RDREQ - RDREQ_32B) + 32 RDREQ_32B.  (FETCH_SIZE prices every request
    that TCC_BUBBLE does not flag at 64 bytes, and TCC_BUBBLE flags only a few
    of the 128-byte requests on this chip, so FETCH_SIZE reads about half.)
    Writes: WRITE_SIZE (KiB).  A device copy of exactly 1 GiB run in the same
    process is the check: it must read and write 1 GiB."""
    import csv
    from collections import defaultdict

    def short(name):
        return name.replace("void ", "").split("(")[0]

    stats = [r for r in csv.DictReader(open(os.path.join(prof_dir, f"{workload}_kernel_stats.csv")))
             if "hsa_attn" in r["Name"]]
    per = {"RDREQ": defaultdict(lambda: defaultdict(float)), "WRITE_SIZE": defaultdict(lambda: defaultdict(float))}
    for c in per:
        for r in csv.DictReader(open(os.path.join(prof_dir, f"{workload}_{c}.csv"))):
            per[c][(int(r["Dispatch_Id"]), r["Kernel_Name"])][r["Counter_Name"]] += float(r["Counter_Value"])
    reads = {k: 128.0 * (v["TCC_EA0_RDREQ_sum"] - v["TCC_EA0_RDREQ_32B_sum"]) + 32.0 * v["TCC_EA0_RDREQ_32B_sum"]
             for k, v in per["RDREQ"].items()}
    writes = {k: 1024.0 * v["WRITE_SIZE"] for k, v in per["WRITE_SIZE"].items()}
    gib = float(1 << 30)

    def copy_of(counts):
        # the calibration copy: the non-library dispatch whose count is nearest 1 GiB
        cands = [k for k in counts if "hsa_attn" not in k[1] and "copy" in k[1].lower()]
        return min(cands, key=lambda k: abs(counts[k] - gib)) if cands else None

    cr, cw = copy_of(reads), copy_of(writes)
    check = {"copy_read_GiB": reads[cr] / gib if cr else None, "copy_written_GiB": writes[cw] / gib if cw else None}
    rd_per, wr_per = defaultdict(list), defaultdict(list)  # per library kernel, one entry per dispatch
    for k, rb in reads.items():
        if "hsa_attn" in k[1]:
            rd_per[short(k[1])].append(rb)
    for k, wb in writes.items():
        if "hsa_attn" in k[1]:
            wr_per[short(k[1])].append(wb)
    rd_avg = {n: float(np.mean(v)) for n, v in rd_per.items()}
    wr_avg = {n: float(np.mean(v)) for n, v in wr_per.items()}
    traffic = {n: rd_avg.get(n, 0.0) + wr_avg.get(n, 0.0) for n in set(rd_avg) | set(wr_avg)}
    rec = {"workload": workload, "library_sha256_16": library_digest(), "device_code_sha256_16": device_code_digest(),
           "bytes": "reads 128 x (TCC_EA0_RDREQ - TCC_EA0_RDREQ_32B) + 32 x TCC_EA0_RDREQ_32B; writes 1024 x WRITE_SIZE",
           "check_copy_1GiB": check, "traffic_bytes_per_launch": traffic}
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    with open(os.path.join(out_dir, f"{workload}.traffic.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    lines = [f"# {kernel} and the other library kernels: {workload}", "",
             "Commands (repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp`; REPO = the root):", ""]
    lines += [f"    {c}" for c in command] + ["", "## Kernel trace (--stats), library kernels", "",
                                               "| kernel | calls | average ns | total ns |", "|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['TotalDurationNs']):.0f} |")
    fmt = lambda x: f"{x:.3f}" if x is not None else "-"  # noqa: E731
    lines += ["", "## HBM bytes per dispatch (--pmc, averaged)", "",
              "Reads = 128 B x (TCC_EA0_RDREQ_sum - TCC_EA0_RDREQ_32B_sum) + 32 B x TCC_EA0_RDREQ_32B_sum (the L2 "
              "of gfx950 reads memory in 128-byte requests); writes = WRITE_SIZE. Check: the 1 GiB device copy "
              f"run in the same process reads {fmt(check['copy_read_GiB'])} GiB and writes "
              f"{fmt(check['copy_written_GiB'])} GiB by these definitions.", "",
              "| kernel | dispatches | read GiB | written GiB | HBM bytes |", "|---|---|---|---|---|"]
    for n in sorted(traffic, key=lambda n: -traffic[n]):
        lines.append(f"| {n} | {len(rd_per.get(n, []))} | {rd_avg.get(n, 0.0) / gib:.3f} | "
                     f"{wr_avg.get(n, 0.0) / gib:.3f} | {traffic[n] / gib:.3f} GiB |")
    mfma_csv = os.path.join(prof_dir, f"{workload}_MFMA.csv")
    if os.path.exists(mfma_csv):
        lines += mfma_summary(workload, mfma_csv, stats, short, out_dir)
    with open(os.path.join(out_dir, f"{kernel}.{workload}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SIMD_NUM = 1024  # MI355X: 256 CUs x 4 SIMDs


def mfma_summary(workload, csv_path, stats, short, out_dir):
    """MFMA counters of one --pmc pass (SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE and rocprofv3's derived
    MfmaUtil = sum of the busy cycles / (max GRBM_GUI_ACTIVE x SIMD_NUM)) per
    library kernel: the fraction of SIMD-cycles the matrix cores were busy,
    and the bf16 flops they executed (512 per MOPS count) over the kernel's
    average duration from the trace.  Written to profiles/<workload>.mfma.json
    (keyed to the built library, read by the benchmark) and returned as
    summary lines."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(csv_path)):
        if "hsa_attn" not in r["Kernel_Name"]:
            continue
        vals[(int(r["Dispatch_Id"]), short(r["Kernel_Name"]))][r["Counter_Name"]] += float(r["Counter_Value"])
    avg_ns = {short(r["Name"]): float(r["AverageNs"]) for r in stats}
    per = defaultdict(list)
    for (_, name), c in vals.items():
        per[name].append(c)
    out = {}
    for name, rows in per.items():
        util = float(np.mean([c.get("MfmaUtil", 0.0) for c in rows])) / 100.0
        flops = float(np.mean([512.0 * c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for c in rows]))
        ns = avg_ns.get(name)
        out[name] = {"mfma_busy_frac": util, "mfma_bf16_flops": flops, "avg_ns": ns,
                     "counter_tflops": flops / ns / 1e3 if ns else None,
                     "busy_cycles": float(np.mean([c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for c in rows])),
                     "grbm_gui_active": float(np.mean([c.get("GRBM_GUI_ACTIVE", 0.0) for c in rows]))}
    rec = {"workload": workload, "library_sha256_16": library_digest(), "device_code_sha256_16": device_code_digest(), "simd_num": SIMD_NUM, "kernels": out}
    with open(os.path.join(out_dir, f"{workload}.mfma.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    lines = ["", "## MFMA counters (--pmc, one dispatch per kernel)", "",
             "MfmaUtil (rocprofv3's derived counter) = sum of SQ_VALU_MFMA_BUSY_CYCLES / (max GRBM_GUI_ACTIVE x "
             f"SIMD_NUM); bf16 MFMA flops = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16, over the trace's average duration, "
             f"against 2.5 PFLOP/s dense bf16.", "",
             "| kernel | MfmaUtil | bf16 MFMA flops | flops / duration | of 2.5 PFLOP/s |", "|---|---|---|---|---|"]
    for name, o in sorted(out.items(), key=lambda kv: -(kv[1]["mfma_bf16_flops"])):
        if o["mfma_bf16_flops"] <= 0:
            continue
        tf = o["counter_tflops"]
        lines.append(f"| {name} | {100 * o['mfma_busy_frac']:.1f}% | {o['mfma_bf16_flops']:.3e} | "
                     f"{tf:.0f} TFLOP/s | {tf / PEAK_BF16_TFLOPS:.3f} |" if tf else f"| {name} | "
                     f"{100 * o['mfma_busy_frac']:.1f}% | {o['mfma_bf16_flops']:.3e} | - | - |")
    return lines


def profiled_mfma(workload, kernel_prefix):
    """Counter-based MFMA figures of a kernel from profiles/<workload>.mfma.json,
    or None when the built kernels differ from the profiled ones."""
    path = os.path.join(ROOT, "profiles", f"{workload}.mfma.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if not profile_is_current(rec):
        return None
    for name, o in rec["kernels"].items():
        if kernel_prefix in name:
            return {"mfma_busy_frac": o["mfma_busy_frac"],
                    "counter_flops_frac": (o["counter_tflops"] / PEAK_BF16_TFLOPS) if o["counter_tflops"] else None,
                    "counter_tflops": o["counter_tflops"]}
    return None


# ---------------------------------------------------------------- decode
def bench_decode(wname, steps, warmup, cpu_baseline):
    import torch
    import hierarchical_sparse_attention_hsa_amd as hsa
    from hierarchical_sparse_attention_hsa_amd.workloads import WORKLOADS, decode_inputs

    w = WORKLOADS[wname]
    G = w.Hq // w.Hkv
    esz = 2 if w.dtype == "bf16" else 4
    Nc = w.T // w.S
    kv_bytes = 2 * w.B * w.Hkv * w.T * w.D * esz
    lm_bytes = w.B * w.Hkv * Nc * w.D * esz
    free, total = torch.cuda.mem_get_info()
    log(f"[{wname}] device memory free {free / 2**30:.1f} GiB of {total / 2**30:.1f} GiB; "
        f"needs {(kv_bytes + lm_bytes) / 2**30:.1f} GiB")
    if kv_bytes + lm_bytes + (2 << 30) > free:
        raise SystemExit(f"{wname}: inputs ({(kv_bytes + lm_bytes) / 2**30:.1f} GiB) do not fit in free device "
                         f"memory ({free / 2**30:.1f} GiB)")
    t0 = time.perf_counter()
    q, k, v = decode_inputs(w, "cuda", progress=lambda b: (b + 1) % 16 == 0 and log(f"[{wname}] generated {b + 1}/{w.B} caches"))
    torch.cuda.synchronize()
    log(f"[{wname}] generated inputs in {time.perf_counter() - t0:.1f} s")
    L = torch.empty((w.B, w.Hkv, Nc, w.D), dtype=k.dtype, device="cuda")
    hsa.hsa_build_landmarks(k, L, w.S)
    adaptive = "gap_threshold" in w.extra  # near-tie adaptive budget
    kk = 2 * w.k if adaptive else w.k  # selection slots per head
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.B, w.Hq, kk), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, kk), dtype=torch.float32, device="cuda")
    dims = hsa.make_dims(w.B, w.Hq, w.Hkv, w.D, w.S, w.k, w.T, hsa.HSA_ATTN_BF16 if esz == 2 else hsa.HSA_ATTN_FP32)
    ws = torch.empty(hsa.hsa_attn_workspace_size(dims, 2 if adaptive else 1), dtype=torch.uint8, device="cuda")
    tau = float(w.extra["gap_threshold"]) if adaptive else None
    torch.cuda.synchronize()

    def step(ev):
        if ev is not None:
            hsa.hsa_attn_set_timing_events(ev)
        if adaptive:
            hsa.hsa_forward_decode_adaptive(q, k, v, L, w.S, w.k, tau, out=out, sel_idx=sel, sel_score=sc,
                                            workspace=ws)
        else:
            hsa.hsa_forward_decode(q, k, v, L, w.S, w.k, out=out, sel_idx=sel, sel_score=sc, workspace=ws)

    secs, per, secs_ev = timed_steps(step, steps, warmup, 4, HipEvents())
    ms_step = 1e3 * secs / steps
    # distinct selected (b, g, chunk) tiles
    attn_bytes = distinct_tile_bytes(sel, w)
    alg_bytes = lm_bytes + attn_bytes
    names = ["decode_scan", "decode_merge", "decode_attn", "decode_fuse"]
    dom, other = decode_roofline(wname, per[0], lm_bytes, per[2], attn_bytes)
    res = {
        "workload": wname, "value": w.B / (ms_step / 1e3), "unit": "queries/s", "ms_per_step": ms_step,
        "ms_per_step_timed_kernels": 1e3 * secs_ev / steps,
        "kernel_ms": {n: float(x) for n, x in zip(names, per)},
        "step_alg_bytes": alg_bytes, "step_alg_GBps": alg_bytes / (ms_step / 1e3) / 1e9,
        "config": {"workload": wname, "batch_queries": w.B, "cache_tokens": w.T, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.D, "chunk": w.S, "top_k": w.k, "needles": w.needles},
        "dtype": w.dtype,
        "roofline": dom,
        "roofline_other": other,
    }
    if adaptive:
        res["gap_threshold"] = tau
        res["doubled_head_frac"] = float(((sel >= 0).sum(-1) > w.k).float().mean())
        res["config"]["gap_threshold"] = tau
    # needle recall (semantic sanity of the synthetic retrieval task)
    from hierarchical_sparse_attention_hsa_amd.workloads import needle_chunks
    sh = sel.cpu().numpy()
    hit = tot = 0
    for b in range(w.B):
        nd = set(needle_chunks(w, b).tolist())
        for h in range(w.Hq):
            got = set(sh[b, h].tolist())
            hit += len(nd & got)
            tot += len(nd)
    res["needle_recall"] = hit / max(tot, 1)
    ties = cuts = 0
    for b in range(w.B):
        for g in range(w.Hkv):
            t, c = near_tie_rows(q[b, g * G:(g + 1) * G], L[b, g],
                                 torch.full((G,), Nc, dtype=torch.int64, device="cuda"), w.k)
            ties += t
            cuts += c
    res["near_tie_rows"] = {"rows": w.B * w.Hq, "with_cut": cuts, "near_tie": ties}
    log(f"[{wname}] {ms_step:.3f} ms/step, kernels {dict(zip(names, np.round(per, 4)))}, "
        f"{dom['kernel']} {dom['achieved']:.0f} GB/s, {other['kernel']} {other['achieved']:.0f} GB/s, "
        f"needle recall {res['needle_recall']:.4f}")
    if cpu_baseline:
        res["cpu_baseline"] = decode_cpu_baseline(w, q, k, v, tau=tau)
    del q, k, v, L, out, sel, sc, ws
    torch.cuda.empty_cache()
    return res


def bench_decode_varlen(wname, steps, warmup):
    """Incremental decoding: each step decodes one query per sequence over
    its current cache length (hsa_forward_decode_varlen) and appends one
    token (hsa_append_kv), so lengths advance by one per step."""
    import torch
    import hierarchical_sparse_attention_hsa_amd as hsa
    from hierarchical_sparse_attention_hsa_amd.workloads import WORKLOADS, cache_lengths, decode_inputs

    w = WORKLOADS[wname]
    G = w.Hq // w.Hkv
    esz = 2 if w.dtype == "bf16" else 4
    Nc = w.T // w.S
    t0 = time.perf_counter()
    q, k, v = decode_inputs(w, "cuda")
    L = torch.empty((w.B, w.Hkv, Nc, w.D), dtype=k.dtype, device="cuda")
    hsa.hsa_build_landmarks(k, L, w.S)
    lens0 = cache_lengths(w)
    lens = torch.tensor(lens0, dtype=torch.int64, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 6)
    k_new = torch.randn((w.B, w.Hkv, w.D), generator=gen, device="cuda").to(k.dtype)
    v_new = torch.randn((w.B, w.Hkv, w.D), generator=gen, device="cuda").to(k.dtype)
    torch.cuda.synchronize()
    log(f"[{wname}] generated inputs in {time.perf_counter() - t0:.1f} s; cache lengths "
        f"{int(lens0.min())} .. {int(lens0.max())}")
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.B, w.Hq, w.k), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, w.k), dtype=torch.float32, device="cuda")
    dims = hsa.make_dims(w.B, w.Hq, w.Hkv, w.D, w.S, w.k, w.T, hsa.HSA_ATTN_BF16 if esz == 2 else hsa.HSA_ATTN_FP32)
    ws = torch.empty(hsa.hsa_attn_workspace_size(dims, True), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step(ev):
        if ev is not None:
            hsa.hsa_attn_set_timing_events(ev[:8])
        hsa.hsa_forward_decode_varlen(q, k, v, L, lens, w.S, w.k, out=out, sel_idx=sel, sel_score=sc, workspace=ws)
        if ev is not None:
            hsa.hsa_attn_set_timing_events(ev[8:])
        hsa.hsa_append_kv(k_new, v_new, k, v, L, lens, w.S)

    secs, per, secs_ev = timed_steps(step, steps, warmup, 5, HipEvents())
    ms_step = 1e3 * secs / steps
    # landmark bytes the scan reads in the instrumented steps, the second to
    # last run of `steps` (lengths grow by one per step)
    ln = lens.cpu().numpy()
    mid = ln - steps - steps // 2
    lm_bytes = float(np.sum(mid // w.S)) * w.Hkv * w.D * esz
    names = ["decode_scan", "decode_merge", "decode_attn", "decode_fuse", "append_kv"]
    dom, other = decode_roofline(wname, per[0], lm_bytes, per[2], distinct_tile_bytes(sel, w))
    res = {
        "workload": wname, "value": w.B / (ms_step / 1e3), "unit": "queries/s", "ms_per_step": ms_step,
        "ms_per_step_timed_kernels": 1e3 * secs_ev / steps,
        "kernel_ms": {n: float(x) for n, x in zip(names, per)},
        "config": {"workload": wname, "batch_queries": w.B, "cache_capacity": w.T,
                   "cache_tokens": [int(lens0.min()), int(lens0.max())], "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "chunk": w.S, "top_k": w.k, "needles": w.needles},
        "dtype": w.dtype,
        "roofline": dom,
        "roofline_other": other,
    }
    log(f"[{wname}] {ms_step:.3f} ms/step, kernels {dict(zip(names, np.round(per, 4)))}, "
        f"{dom['kernel']} {dom['achieved']:.0f} GB/s, {other['kernel']} {other['achieved']:.0f} GB/s")
    del q, k, v, L, out, sel, sc, ws
    torch.cuda.empty_cache()
    return res


# attainable HBM read bandwidth measured in this run (attainable_read_gbps),
# reported beside the nominal peak in the HBM-bound rooflines
ATTAINABLE = {}


def attainable_read_gbps(gib=8, reps=5):
    """Best read bandwidth of the stream probe (measure/stream_read.hip, a
    library of its own) over a few launch shapes on a `gib` GiB buffer,
    timed with events on torch's current stream, where the probe launches."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "hierarchical_sparse_attention_hsa_amd", "libhsa_attn_stream.so"))
    lib.hsa_attn_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.hsa_attn_stream_read.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = (0.0, None)
    for blocks in (1024, 2048, 4096, 8192):
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
        for unroll in (4, 8):
            def run():
                rc = lib.hsa_attn_stream_read(buf.data_ptr(), nbytes, blocks, unroll, sink.data_ptr(), stream)
                if rc != 0:
                    raise RuntimeError(f"stream probe launch failed: HIP error {rc}")
            run()
            run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            gbs = reps * nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9
            if gbs > best[0]:
                best = (gbs, f"{blocks} workgroups x 256 threads, {unroll} 16-byte loads in flight per thread")
        del sink
    del buf
    torch.cuda.empty_cache()
    log(f"attainable HBM read bandwidth (stream probe, {gib} GiB): {best[0]:.0f} GB/s ({best[1]})")
    return best


def decode_roofline(wname, per_scan_ms, lm_bytes, per_attn_ms, attn_bytes):
    """Roofline of the dominant decode kernel (the longer of the landmark scan
    and the chunk attention, both HBM-bound) with the other one beside it.
    Algorithmic bytes: the landmarks the scan reads; the distinct selected
    K/V tiles the attention reads."""
    kern = {"decode_scan_kernel": (per_scan_ms, lm_bytes), "decode_attn_kernel": (per_attn_ms, attn_bytes)}
    out = {}
    for name, (ms, nbytes) in kern.items():
        gbs = nbytes / (ms / 1e3) / 1e9
        out[name] = {"kernel": name, "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": profiled_traffic(wname, name),
                     "alg_bytes_per_launch": nbytes, "ms": ms}
        if ATTAINABLE:
            out[name]["attainable"] = ATTAINABLE["GBps"]
            out[name]["frac_of_attainable"] = gbs / ATTAINABLE["GBps"]
    dom = max(kern, key=lambda n: kern[n][0])
    other = [n for n in kern if n != dom][0]
    return out[dom], out[other]


def distinct_tile_bytes(sel, w):
    """K and V bytes of the distinct (b, g, chunk) tiles the heads selected."""
    G = w.Hq // w.Hkv
    kk = sel.shape[-1]
    s = sel.view(w.B, w.Hkv, G * kk).cpu().numpy()
    distinct = sum(len(set(s[b, g][s[b, g] >= 0].tolist())) for b in range(w.B) for g in range(w.Hkv))
    return distinct * 2 * w.S * w.D * (2 if w.dtype == "bf16" else 4)


def decode_cpu_baseline(w, q, k, v, queries=(0, 37), min_seconds=10.0, tau=None):
    """The oracle on a bounded sample: the listed queries, all heads.  Host
    copies and the oracle's own landmark build are untimed (landmarks are
    precomputed in this workload); scoring, top-k, chunk attention and fusion
    are timed, repeated per KV group so that about min_seconds of work is
    measured."""
    from oracle import hsa_oracle as O
    G = w.Hq // w.Hkv
    queries = [b for b in queries if b < w.B]
    reps = None
    total = 0.0
    for b in queries:
        qb = q[b].float().cpu().double().numpy()
        for g in range(w.Hkv):
            Kg = k[b, g].float().cpu().double().numpy()
            Vg = v[b, g].float().cpu().double().numpy()
            Lg = O.landmarks(Kg, w.S, w.dtype)
            args = (qb[g * G:(g + 1) * G], np.full(G, w.T), Kg, Vg, Lg, w.S, w.k)
            fn = O.hsa_rows
            if tau is not None:  # near-tie adaptive budget
                args, fn = args + (tau,), O.hsa_rows_adaptive
            if reps is None:  # size the repetition count on the first group
                t0 = time.perf_counter()
                fn(*args)
                one = time.perf_counter() - t0
                reps = max(1, min(1000, int(min_seconds / (one * len(queries) * w.Hkv))))
            t0 = time.perf_counter()
            for _ in range(reps):
                fn(*args)
            total += time.perf_counter() - t0
            del Kg, Vg
    return {"value": len(queries) * reps / total, "unit": "queries/s", "cores": blas_threads(), "kind": "oracle",
            "host": host_info(),
            "sample": f"queries {list(queries)} of {w.B} (all {w.Hq} heads), each KV group's oracle call repeated "
                      f"{reps} times ({total:.1f} s timed); oracle landmark build and host copies untimed"}


# ---------------------------------------------------------------- prefill
def bench_prefill(wname, steps, warmup, cpu_baseline):
    import torch
    import hierarchical_sparse_attention_hsa_amd as hsa
    from hierarchical_sparse_attention_hsa_amd.workloads import WORKLOADS, prefill_inputs

    w = WORKLOADS[wname]
    esz = 2 if w.dtype == "bf16" else 4
    Nc = w.T // w.S
    off = int(w.extra.get("q_offset", 0))  # cached prefix (chunked prefill)
    Tq = w.T - off
    t0 = time.perf_counter()
    q, k, v = prefill_inputs(w, "cuda")
    if off:
        q = q[:, :, off:].contiguous()
    torch.cuda.synchronize()
    log(f"[{wname}] generated inputs in {time.perf_counter() - t0:.1f} s")
    L = torch.empty((w.B, w.Hkv, Nc, w.D), dtype=k.dtype, device="cuda")
    if off:  # the prefix's landmarks exist already
        hsa.hsa_build_landmarks(k, L, w.S, 0, off // w.S)
    tau = w.extra.get("gap_threshold")  # near-tie adaptive budget
    kk = w.k if tau is None else 2 * w.k  # selection slots per row
    out = torch.empty((w.B, w.Hq, Tq, w.D), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.B, w.Hq, Tq, kk), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, Tq, kk), dtype=torch.float32, device="cuda")
    events = HipEvents()
    # the default workspace (hsa_attn_workspace_size), allocated once; the
    # rows run in slabs as large as it holds
    dims = hsa.make_dims(w.B, w.Hq, w.Hkv, w.D, w.S, w.k, w.T, hsa.HSA_ATTN_BF16 if esz == 2 else hsa.HSA_ATTN_FP32)
    ws = torch.empty(hsa.hsa_attn_workspace_size(dims, 3 if tau is not None else 0), dtype=torch.uint8,
                     device="cuda")
    slab_rows = hsa.hsa_attn_prefill_slab_rows(dims, ws.numel(), tau is not None, True)
    nslab = -(-Tq // slab_rows)
    log(f"[{wname}] workspace {ws.numel() / 1e9:.2f} GB: {nslab} slab(s) of {slab_rows} query rows")

    def step(ev):
        if ev is not None:
            hsa.hsa_attn_set_timing_events(ev[:2])
        hsa.hsa_build_landmarks(k, L, w.S, off // w.S, Nc)  # the new tokens' chunks
        if ev is not None:
            hsa.hsa_attn_set_timing_events(ev[2:])
        if off:
            hsa.hsa_forward_prefill_cached(q, k, v, L, off, w.S, w.k, out=out, sel_idx=sel, sel_score=sc,
                                           workspace=ws)
        elif tau is not None:
            hsa.hsa_forward_prefill_adaptive(q, k, v, L, w.S, w.k, tau, out=out, sel_idx=sel, sel_score=sc,
                                             workspace=ws)
        else:
            hsa.hsa_forward_prefill(q, k, v, L, w.S, w.k, out=out, sel_idx=sel, sel_score=sc, workspace=ws)

    # launches: landmarks; the V transpose; per group of up to 64 slabs
    # zero, select, scan and scatter, then per slab remote and local.
    # Per-kernel times are summed over the slabs.
    names = ["landmarks", "prefill_zero", "prefill_select", "prefill_vt", "prefill_scan", "prefill_scatter",
             "prefill_remote", "prefill_local"]
    order = ["landmarks", "prefill_vt"]
    for s0 in range(0, nslab, 64):
        order += ["prefill_zero", "prefill_select", "prefill_scan", "prefill_scatter"]
        order += ["prefill_remote", "prefill_local"] * min(64, nslab - s0)
    secs, per_launch, secs_ev = timed_steps(step, steps, warmup, len(order), events)
    per = np.array([sum(t for n, t in zip(order, per_launch) if n == name) for name in names])
    ms_step = 1e3 * secs / steps
    # exact algorithmic work
    p = np.arange(off, w.T)
    n_p = np.minimum(p // w.S, Nc)
    score_flops = 2.0 * w.B * w.Hq * w.D * n_p.sum()
    n_pairs = int((sel >= 0).sum().item())  # kept (row, chunk) pairs: sum of min(n_p, k) without adaptivity
    attn_flops = 4.0 * w.S * w.D * n_pairs
    # split of the selected pairs into remote and local ones, counted from
    # this run's selection by the library's rule: remote = a chunk before
    # the query's 64-chunk window, or a window chunk selected by fewer than
    # LOCAL_MIN_ROWS rows of the query's 32-row block (same head)
    win0 = torch.div(torch.arange(off, w.T, device="cuda") // w.S, 64, rounding_mode="floor") * 64
    kept = sel >= 0
    in_win = kept & (sel >= win0[None, None, :, None])
    blk = (torch.arange(Tq, device="cuda") // 32)[None, None, :, None]
    bh = torch.arange(w.B * w.Hq, device="cuda").view(w.B, w.Hq, 1, 1)
    key = ((bh * ((Tq + 31) // 32) + blk) * 64 + (sel - win0[None, None, :, None]).clamp(0, 63)).expand_as(sel)
    cnt = torch.bincount(key[in_win].flatten(), minlength=w.B * w.Hq * ((Tq + 31) // 32) * 64)
    n_local = int((cnt[cnt >= LOCAL_MIN_ROWS]).sum().item())
    n_remote = int(kept.sum().item()) - n_local
    del in_win, key, cnt
    remote_flops = 4.0 * w.S * w.D * n_remote
    local_flops = 4.0 * w.S * w.D * (n_pairs - n_remote)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    attn_ms = float(per[3:].sum())
    sel_tf = score_flops / (per[2] / 1e3) / 1e12
    att_tf = attn_flops / (attn_ms / 1e3) / 1e12
    kern = {2: ("prefill_select_kernel", score_flops), 6: ("prefill_remote_kernel", remote_flops),
            7: ("prefill_local_kernel", local_flops)}
    dom = max(kern, key=lambda i: per[i])
    dom_name, dom_flops = kern[dom]
    dom_tf = dom_flops / (per[dom] / 1e3) / 1e12
    res = {
        "workload": wname, "value": w.B * Tq / (ms_step / 1e3), "unit": "tokens/s", "ms_per_step": ms_step,
        "ms_per_step_timed_kernels": 1e3 * secs_ev / steps,
        "kernel_ms": {n: float(x) for n, x in zip(names, per)},
        "scoring_tflops": sel_tf, "scoring_mfma_frac": sel_tf / peak,
        # rocprofv3 MFMA counters of the scoring and local kernels (profiles/), null once the library changed
        "scoring_mfma_counters": profiled_mfma(wname, "prefill_select_kernel"),
        "local_mfma_counters": profiled_mfma(wname, "prefill_local_kernel"),
        "attention_ms": attn_ms, "attention_tflops": att_tf, "attention_mfma_frac": att_tf / peak,
        "remote_pair_frac": n_remote / max(n_pairs, 1),
        "remote_tflops": remote_flops / (per[6] / 1e3) / 1e12,
        "local_tflops": local_flops / (per[7] / 1e3) / 1e12,
        "landmark_GBps": (w.B * w.Hkv * (Nc - off // w.S) * w.S * w.D * esz) / (per[0] / 1e3) / 1e9,
        "workspace_bytes": int(ws.numel()), "slabs": nslab, "slab_rows": slab_rows,
        "config": {"workload": wname, "batch": w.B, "seq_len": w.T, "query_tokens": Tq, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.D, "chunk": w.S, "top_k": w.k, "lowrank": w.lowrank},
        "dtype": w.dtype,
        "roofline": {"kernel": dom_name, "bound": "mfma", "achieved": dom_tf, "peak": peak, "unit": "TFLOP/s",
                     "frac": dom_tf / peak, "traffic": profiled_traffic(wname, dom_name),
                     "alg_flops_per_launch": dom_flops},
    }
    if tau is None:
        G = w.Hq // w.Hkv
        ties = cuts = 0
        n_all = torch.clamp(torch.arange(off, w.T, device="cuda") // w.S, max=Nc)
        blk = 16384
        for b in range(w.B):
            for h in range(w.Hq):
                for r0 in range(0, Tq, blk):
                    t, c = near_tie_rows(q[b, h, r0:r0 + blk], L[b, h // G], n_all[r0:r0 + blk], w.k)
                    ties += t
                    cuts += c
        res["near_tie_rows"] = {"rows": w.B * w.Hq * Tq, "with_cut": cuts, "near_tie": ties}
    log(f"[{wname}] {ms_step:.3f} ms/step, kernels {dict(zip(names, np.round(per, 4)))}, "
        f"scoring {sel_tf:.1f} TFLOP/s, attention {att_tf:.1f} TFLOP/s, remote pairs {n_remote / max(n_pairs, 1):.3f}")
    if tau is not None:
        res["gap_threshold"] = tau
        res["doubled_row_frac"] = float(((sel >= 0).sum(-1) > w.k).float().mean())
        res["config"]["gap_threshold"] = tau
    if cpu_baseline:
        res["cpu_baseline"] = prefill_cpu_baseline(w, q, k, v, tau=tau)
    del q, k, v, L, out, sel, sc, ws
    torch.cuda.empty_cache()
    return res


def prefill_cpu_baseline(w, q, k, v, chunks=tuple(range(250, 4001, 250)), tau=None):
    """The oracle on a bounded sample: all heads of the query chunks listed
    (64 tokens each).  Host copies and landmark building are untimed."""
    from oracle import hsa_oracle as O
    G = w.Hq // w.Hkv
    off = int(w.extra.get("q_offset", 0))  # q holds the rows from off on
    if off:  # 16 chunks spread over the new tokens
        chunks = sorted({int(c) for c in np.linspace(off // w.S, w.T // w.S - 1, 16)})
    chunks = [c for c in chunks if off <= c * w.S < w.T] or [w.T // w.S - 1]
    total = 0.0
    for g in range(w.Hkv):
        Kg = k[0, g].float().cpu().double().numpy()
        Vg = v[0, g].float().cpu().double().numpy()
        Lg = O.landmarks(Kg, w.S, w.dtype)
        for c in chunks:
            pos = np.arange(c * w.S, min(w.T, (c + 1) * w.S))
            qq = q[0, g * G:(g + 1) * G, c * w.S - off:(c + 1) * w.S - off].float().cpu().double().numpy()
            t0 = time.perf_counter()
            for hh in range(G):
                if tau is None:
                    O.hsa_rows(qq[hh], pos, Kg, Vg, Lg, w.S, w.k)
                else:  # near-tie adaptive budget
                    O.hsa_rows_adaptive(qq[hh], pos, Kg, Vg, Lg, w.S, w.k, tau)
            total += time.perf_counter() - t0
    tokens = len(chunks) * w.S
    return {"value": tokens / total, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "host": host_info(),
            "sample": f"query chunks {list(chunks)} ({tokens} tokens, all {w.Hq} heads; {total:.1f} s timed); "
                      f"host copies and oracle landmark build untimed"}


# ---------------------------------------------------------------- backward
def bench_backward(wname, steps, warmup, cpu_baseline):
    import torch
    import hierarchical_sparse_attention_hsa_amd as hsa
    from hierarchical_sparse_attention_hsa_amd.workloads import WORKLOADS, prefill_inputs

    w = WORKLOADS[wname]
    Nc = w.T // w.S
    t0 = time.perf_counter()
    q, k, v = prefill_inputs(w, "cuda")
    dout = torch.randn((w.B, w.Hq, w.T, w.D), dtype=torch.float32, device="cuda",
                       generator=torch.Generator("cuda").manual_seed(w.seed + 100))
    L = torch.empty((w.B, w.Hkv, Nc, w.D), dtype=k.dtype, device="cuda")
    hsa.hsa_build_landmarks(k, L, w.S)
    sel = torch.empty((w.B, w.Hq, w.T, w.k), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.B, w.Hq, w.T, w.k), dtype=torch.float32, device="cuda")
    out = hsa.hsa_forward_prefill(q, k, v, L, w.S, w.k, sel_idx=sel, sel_score=sc)  # the forward, untimed
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"[{wname}] inputs and forward in {time.perf_counter() - t0:.1f} s")
    dq = torch.empty_like(out)
    dk = torch.empty((w.B, w.Hkv, w.T, w.D), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    dims = hsa.make_dims(w.B, w.Hq, w.Hkv, w.D, w.S, w.k, w.T, hsa.HSA_ATTN_BF16)
    ws = torch.empty(hsa.hsa_attn_workspace_size(dims, 4), dtype=torch.uint8, device="cuda")

    def step(ev):
        if ev is not None:
            hsa.hsa_attn_set_timing_events(ev)
        hsa.hsa_backward_prefill(q, k, v, L, out, dout, sel, sc, w.S, dq=dq, dk=dk, dv=dv, workspace=ws)

    names = ["bwd_zero", "bwd_prep", "bwd_scan", "bwd_scatter", "bwd_kt", "bwd_chunk", "bwd_dq"]
    if w.T % w.S:
        names.append("bwd_tail")
    secs, per, secs_ev = timed_steps(step, steps, warmup, len(names), HipEvents())
    ms_step = 1e3 * secs / steps
    n_pairs = int((sel >= 0).sum().item())
    # per kept pair: S = K q, dA = V do, dq = K^T dlogit, dV += a do, dK += dlogit q
    flops = 10.0 * w.S * w.D * n_pairs
    ci = names.index("bwd_chunk")
    tf = flops / (per[ci] / 1e3) / 1e12
    res = {
        "workload": wname, "value": w.B * w.T / (ms_step / 1e3), "unit": "tokens/s", "ms_per_step": ms_step,
        "ms_per_step_timed_kernels": 1e3 * secs_ev / steps,
        "kernel_ms": {n: float(x) for n, x in zip(names, per)},
        "config": {"workload": wname, "batch": w.B, "seq_len": w.T, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "chunk": w.S, "top_k": w.k, "lowrank": w.lowrank},
        "dtype": w.dtype,
        "roofline": {"kernel": "bwd_chunk_kernel", "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                     "traffic": profiled_traffic(wname, "bwd_chunk_kernel"), "alg_flops_per_launch": flops},
    }
    log(f"[{wname}] {ms_step:.3f} ms/step, kernels {dict(zip(names, np.round(per, 4)))}, chunk kernel {tf:.1f} TFLOP/s")
    if cpu_baseline:
        res["cpu_baseline"] = backward_cpu_baseline(w, q, k, v, dout, sel)
    del q, k, v, L, out, sel, sc, dq, dk, dv, ws, dout
    torch.cuda.empty_cache()
    return res


def backward_cpu_baseline(w, q, k, v, dout, sel, chunks=(500, 1500, 2500, 3500)):
    """The oracle's backward on a bounded sample: all heads of the query chunks
    listed (64 tokens each), with the forward's selection; host copies and
    the oracle's landmark build untimed."""
    from oracle import hsa_oracle as O
    G = w.Hq // w.Hkv
    total = 0.0
    for g in range(w.Hkv):
        Kg = k[0, g].float().cpu().double().numpy()
        Vg = v[0, g].float().cpu().double().numpy()
        Lg = O.landmarks(Kg, w.S, w.dtype)
        for c in chunks:
            pos = np.arange(c * w.S, (c + 1) * w.S)
            for hh in range(g * G, (g + 1) * G):
                qq = q[0, hh, c * w.S:(c + 1) * w.S].float().cpu().double().numpy()
                gg = dout[0, hh, c * w.S:(c + 1) * w.S].double().cpu().numpy()
                ss = sel[0, hh, c * w.S:(c + 1) * w.S].cpu().numpy()
                t0 = time.perf_counter()
                O.hsa_rows_backward(qq, pos, Kg, Vg, Lg, w.S, ss, gg)
                total += time.perf_counter() - t0
    tokens = len(chunks) * w.S
    return {"value": tokens / total, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "host": host_info(),
            "sample": f"query chunks {list(chunks)} ({tokens} tokens, all {w.Hq} heads; {total:.1f} s timed); "
                      f"forward selection from the layer, host copies and oracle landmark build untimed"}


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one device copy of exactly 1 GiB (the reference kernel for HBM byte counters)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="write profiles/<workload>.md and .traffic.json from the rocprofv3 CSVs in DIR and exit")
    ap.add_argument("--profile-command", action="append", default=[],
                    help="with --summarize-profile: a command line to record in the summary")
    ap.add_argument("--profile-kernel", default="kernels",
                    help="with --summarize-profile: the kernel the summary is named for")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args.workload, args.summarize_profile, args.profile_command, args.profile_kernel)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this layer is measured on one GPU; its multi-GPU sharding is a design only, not "
              "built. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import hierarchical_sparse_attention_hsa_amd as hsa
    hsa.load_library()
    cpu = not args.no_cpu_baseline
    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        # evict the freshly written source from L2 and the 256 MiB MALL, so
        # that the copy reads all of it from HBM (a partly cached source made
        # the read scale drift from run to run)
        flush = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
        flush.fill_(1)
        torch.cuda.synchronize()
        del flush
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB read + 1 GiB written")
        del src, dst
    results = {}
    if args.workload == "all" or args.workload.startswith("decode"):
        gbs, how = attainable_read_gbps()
        ATTAINABLE.update({"GBps": gbs, "probe": how})
    if args.workload == "all":
        results["prefill"] = bench_prefill("prefill_256k_bf16", args.steps, args.warmup, cpu)
        main_res = bench_decode("decode_1m_bf16", args.steps, args.warmup, cpu)
        # the 16M-token decode rides along once the 1M caches are freed (its
        # oracle baseline would stream 32 GiB caches through the host: none)
        results["decode_16m"] = bench_decode("decode_16m_bf16", args.steps, args.warmup, False)
    elif "varlen" in args.workload:
        main_res = bench_decode_varlen(args.workload, args.steps, args.warmup)
    elif args.workload.startswith("backward"):
        main_res = bench_backward(args.workload, args.steps, args.warmup, cpu)
    elif args.workload.startswith("decode"):
        main_res = bench_decode(args.workload, args.steps, args.warmup, cpu)
    else:
        main_res = bench_prefill(args.workload, args.steps, args.warmup, cpu)
    line = {
        "metric": METRIC, "value": main_res["value"], "unit": main_res["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": main_res["dtype"],
        "data": "synthetic", "config": main_res["config"], "roofline": main_res["roofline"],
    }
    if "cpu_baseline" in main_res:
        line["cpu_baseline"] = main_res["cpu_baseline"]
    # the rest of the workload's record (kernel times, the other roofline,
    # MFMA counters, near-tie counts, ...)
    for key, val in main_res.items():
        if key not in line and key != "workload":
            line[key] = val
    for key in ("prefill", "decode_16m"):
        if key in results:
            line[key] = results[key]
    if ATTAINABLE:
        line["hbm_read_attainable"] = {"GBps": ATTAINABLE["GBps"], "frac_of_peak": ATTAINABLE["GBps"] / PEAK_HBM_GBS,
                                       "probe": ATTAINABLE["probe"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
