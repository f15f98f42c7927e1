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
