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
