"""Host-side checks of the benchmark's accounting (no GPU)."""
import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_local_min_rows_matches_the_kernels():
    # the benchmark splits the algorithmic attention work between the local
    # and the chunk-major prefill kernels with the kernels' own threshold
    src = open(os.path.join(ROOT, "hierarchical_sparse_attention_hsa_amd", "csrc", "prefill_kernels.hpp")).read()
    m = re.search(r"#define HSA_LOCAL_MIN_ROWS (\d+)", src)
    assert m and int(m.group(1)) == bench.LOCAL_MIN_ROWS


def test_stream_probe_library_exports_and_validates():
    # the benchmark's read-bandwidth probe is a library of its own; bad
    # arguments are rejected before any HIP call
    import ctypes
    import pytest
    path = os.path.join(ROOT, "hierarchical_sparse_attention_hsa_amd", "libhsa_attn_stream.so")
    if not os.path.exists(path):
        pytest.skip("libhsa_attn_stream.so not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    f = lib.hsa_attn_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(None, 1 << 20, 64, 4, None, None) != 0
    assert f(16, 1 << 20, 64, 3, 16, None) != 0   # unroll must be 4 or 8
    assert f(16, 17, 64, 4, 16, None) != 0        # not a whole number of 16-byte words


def test_profile_bytes_follow_the_request_counters(tmp_path):
    # read bytes = 128 per read request, 32 per 32-byte one (counted among
    # them); write bytes = WRITE_SIZE KiB; the 1 GiB copy is the check
    import csv
    import json

    def write(name, header, rows):
        with open(tmp_path / name, "w", newline="") as fh:
            w = csv.writer(fh)
            w.writerow(header)
            w.writerows(rows)

    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    copy = "__amd_rocclr_copyBuffer"
    kern = "void hsa_attn::decode_scan_kernel<hsa_attn::BF16, 128, 4>(int)"
    gib = 1 << 30
    write("w_kernel_stats.csv", ["Name", "Calls", "AverageNs", "TotalDurationNs"], [[kern, 1, 1000.0, 1000.0]])
    write("w_RDREQ.csv", hdr, [[1, copy, "TCC_EA0_RDREQ_sum", gib // 128], [1, copy, "TCC_EA0_RDREQ_32B_sum", 0],
                               [2, kern, "TCC_EA0_RDREQ_sum", 1000], [2, kern, "TCC_EA0_RDREQ_32B_sum", 100]])
    write("w_WRITE_SIZE.csv", hdr, [[1, copy, "WRITE_SIZE", gib // 1024], [2, kern, "WRITE_SIZE", 3]])
    bench.summarize_profile("w", str(tmp_path), ["cmd"], "decode_scan_kernel", out_dir=str(tmp_path))
    rec = json.load(open(tmp_path / "w.traffic.json"))
    assert rec["check_copy_1GiB"] == {"copy_read_GiB": 1.0, "copy_written_GiB": 1.0}
    (name, b), = rec["traffic_bytes_per_launch"].items()
    assert "decode_scan_kernel" in name and b == 900 * 128 + 100 * 32 + 3 * 1024


def test_device_code_digest_hashes_the_fatbin_section():
    # committed counter records are matched to the built kernels by a digest
    # of the library's .hip_fatbin section; the section located by the
    # benchmark's own ELF reader must be the one readelf reports
    import hashlib
    import shutil
    import subprocess

    import pytest

    lib = os.path.join(ROOT, "hierarchical_sparse_attention_hsa_amd", "libhsa_attn.so")
    if not os.path.exists(lib) or shutil.which("readelf") is None:
        pytest.skip("library not built or readelf missing")
    out = subprocess.run(["readelf", "-S", "-W", lib], capture_output=True, text=True, check=True).stdout
    m = re.search(r"\.hip_fatbin\s+\S+\s+[0-9a-f]+\s+([0-9a-f]+)\s+([0-9a-f]+)", out)
    assert m, "no .hip_fatbin section"
    off, size = int(m.group(1), 16), int(m.group(2), 16)
    data = open(lib, "rb").read()[off:off + size]
    assert size > 0 and bench.device_code_digest() == hashlib.sha256(data).hexdigest()[:16]
