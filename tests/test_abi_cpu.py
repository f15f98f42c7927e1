"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import hierarchical_sparse_attention_hsa_amd as hsa
from hierarchical_sparse_attention_hsa_amd import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsa_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hsa.library_path()),
                                reason="libhsa_attn.so not built (run __graft_entry__.build())")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const char\*|hsa_attn_status_t)\s+(\w+)\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(hsa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = hsa.load_library()
    for name in header_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {hsa.library_path()}").read()
    for name in header_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_struct_layout_matches_header():
    assert ctypes.sizeof(Dims) == 40
    assert Dims.seq_len.offset == 24 and Dims.dtype.offset == 32


def dims(**kw):
    base = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, chunk_size=64, top_k=16,
                seq_len=4096, dtype=hsa.HSA_ATTN_BF16, reserved=0)
    base.update(kw)
    return Dims(**base)


def status_of(d, call="prefill", ws=1 << 30, ptr=0x1000, **kw):
    lib = hsa.load_library()
    p = ctypes.c_void_p(ptr)
    if call == "prefill":
        return lib.hsa_forward_prefill(ctypes.byref(d), p, p, p, p, p, None, None, p, ws, None)
    if call == "decode":
        return lib.hsa_forward_decode(ctypes.byref(d), p, p, p, p, p, None, None, p, ws, None)
    if call == "landmarks":
        return lib.hsa_build_landmarks(ctypes.byref(d), p, p, kw.get("c0", 0), kw.get("c1", 1), None)
    raise ValueError(call)


@pytest.mark.parametrize("call", ["prefill", "decode", "landmarks"])
def test_invalid_arguments_are_rejected_on_the_host(call):
    assert status_of(dims(num_q_heads=6, num_kv_heads=4), call) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert status_of(dims(batch=0), call) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert status_of(dims(top_k=0), call) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert status_of(dims(seq_len=-1), call) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert status_of(dims(dtype=7), call) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert status_of(dims(reserved=1), call) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert status_of(dims(), call, ptr=0x1004) == hsa.HSA_ATTN_INVALID_ARGUMENT  # misaligned
    assert "aligned" in hsa.hsa_attn_last_error()
    assert status_of(dims(head_dim=96), call) == hsa.HSA_ATTN_UNSUPPORTED


def test_null_pointers_and_ranges():
    lib = hsa.load_library()
    d = dims()
    p = ctypes.c_void_p(0x1000)
    assert lib.hsa_forward_prefill(ctypes.byref(d), None, p, p, p, p, None, None, p, 1 << 30, None) == 1
    assert lib.hsa_forward_decode(None, p, p, p, p, p, None, None, p, 1 << 30, None) == 1
    assert lib.hsa_forward_prefill(ctypes.byref(d), p, p, p, p, p, p, None, p, 1 << 30, None) == 1  # one sel output
    assert status_of(dims(), "landmarks", c0=3, c1=2) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert status_of(dims(), "landmarks", c0=0, c1=65) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert status_of(dims(), "landmarks", c0=5, c1=5) == hsa.HSA_ATTN_OK  # empty range enqueues nothing
    lib = hsa.load_library()
    d = dims()
    assert lib.hsa_build_landmarks(ctypes.byref(d), None, None, 0, 0, None) == hsa.HSA_ATTN_OK
    assert lib.hsa_build_landmarks(ctypes.byref(d), None, p, 0, 1, None) == hsa.HSA_ATTN_INVALID_ARGUMENT


def test_supported_envelope():
    for call in ("prefill", "decode"):
        assert status_of(dims(chunk_size=32), call) == hsa.HSA_ATTN_UNSUPPORTED
        assert status_of(dims(num_q_heads=48, num_kv_heads=3), call) == hsa.HSA_ATTN_UNSUPPORTED  # G = 16
    assert status_of(dims(top_k=65), "prefill") == hsa.HSA_ATTN_UNSUPPORTED
    assert status_of(dims(top_k=65), "decode") == hsa.HSA_ATTN_UNSUPPORTED
    # more than 32 prefill slots: up to four query heads per KV head
    assert status_of(dims(top_k=33, num_q_heads=64), "prefill") == hsa.HSA_ATTN_UNSUPPORTED
    for kk, hq in ((33, 32), (64, 32), (64, 8), (32, 64)):
        assert status_of(dims(top_k=kk, num_q_heads=hq), "prefill") not in (
            hsa.HSA_ATTN_INVALID_ARGUMENT, hsa.HSA_ATTN_UNSUPPORTED, hsa.HSA_ATTN_WORKSPACE_TOO_SMALL), (kk, hq)
    # landmarks accept any chunk size and group size
    assert status_of(dims(chunk_size=1, num_q_heads=3, num_kv_heads=3), "landmarks", c0=0, c1=0) == 0


def test_decode_workspace_size_and_too_small_workspace():
    d = dims(batch=2, seq_len=64 * 100 + 7)
    n = hsa.hsa_attn_workspace_size(d, 1)
    assert n > 0 and n % 256 == 0
    assert status_of(d, "decode", ws=n - 1) == hsa.HSA_ATTN_WORKSPACE_TOO_SMALL
    assert "workspace" in hsa.hsa_attn_last_error()


def min_prefill_workspace(d, adaptive=False, given=False):
    lo, hi = 0, 1 << 50
    while lo < hi:
        mid = (lo + hi) // 2
        if hsa.hsa_attn_prefill_slab_rows(d, mid, adaptive, given) > 0:
            hi = mid
        else:
            lo = mid + 1
    return lo


def test_prefill_workspace_slabs():
    """The prefill runs its query rows in slabs as large as the workspace
    holds: the default size takes the whole call in one slab when its worst
    case stays within 16 GiB, a smaller workspace gives smaller slabs (whole
    64-row chunks, spread evenly), and below one 64-row slab the call is
    refused before anything is launched."""
    d = dims(batch=2, seq_len=64 * 100 + 7)
    n = hsa.hsa_attn_workspace_size(d, 0)
    assert n > 0 and n % 256 == 0
    assert n >= 2 * 32 * (64 * 100 + 7) * 16 * 4  # selection of every row
    assert hsa.hsa_attn_prefill_slab_rows(d, n) == 64 * 101
    m = min_prefill_workspace(d)
    assert hsa.hsa_attn_prefill_slab_rows(d, m) == 64
    assert status_of(d, "prefill", ws=m - 1) == hsa.HSA_ATTN_WORKSPACE_TOO_SMALL
    assert "workspace" in hsa.hsa_attn_last_error()
    # a slab of 64 rows holds every pair of its rows chunk-major: 4 + 4 D bytes each
    per_row = 2 * 32 * 16 * (4 + 4 * 128)
    m2 = min_prefill_workspace(d, given=True)
    assert m - m2 == 2 * 32 * (64 * 100 + 7) * 16 * 8 // 256 * 256 or abs(m - m2 - 2 * 32 * 6407 * 16 * 8) < 1024
    # slabs are equal numbers of whole chunks
    for ws in (m + per_row * 64 * 3, m + per_row * 64 * 50, m + per_row * 64 * 60):
        rows = hsa.hsa_attn_prefill_slab_rows(d, ws)
        assert rows % 64 == 0 and 64 <= rows
        nslab = -(-101 // (rows // 64))
        assert (rows // 64) == -(-101 // nslab)
        assert rows <= 64 + (ws - m) // per_row
    # the long prefill: the default workspace stays far below the one-slab worst case
    big = dims(seq_len=1 << 18)
    nb = hsa.hsa_attn_workspace_size(big, 0)
    worst_one_slab = 32 * (1 << 18) * 16 * (4 + 4 * 128)
    assert nb < 20e9 and nb < worst_one_slab / 3
    assert hsa.hsa_attn_prefill_slab_rows(big, nb) < (1 << 18)
    # a 1M-token prefill fits the 288 GB card with the default size
    huge = dims(seq_len=1 << 20)
    assert hsa.hsa_attn_workspace_size(huge, 0) < 40e9


def test_status_strings():
    assert hsa.hsa_attn_status_string(0) == "ok"
    assert hsa.hsa_attn_status_string(3) == "workspace too small"
    assert hsa.hsa_attn_status_string(99) == "unknown status"


def test_varlen_and_append_validation():
    lib = hsa.load_library()
    p = ctypes.c_void_p(0x1000)
    d = dims(seq_len=64 * 100)
    # cache_lens is required and must be 8-byte aligned
    assert lib.hsa_forward_decode_varlen(ctypes.byref(d), p, p, p, p, None, p, None, None, p, 1 << 30,
                                         None) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert "cache_lens" in hsa.hsa_attn_last_error()
    assert lib.hsa_forward_decode_varlen(ctypes.byref(d), p, p, p, p, ctypes.c_void_p(0x1004), p, None, None, p,
                                         1 << 30, None) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert lib.hsa_forward_decode_varlen(ctypes.byref(d), p, p, p, p, p, p, None, None, p, 16,
                                         None) == hsa.HSA_ATTN_WORKSPACE_TOO_SMALL
    assert lib.hsa_forward_decode_varlen(ctypes.byref(dims(chunk_size=32)), p, p, p, p, p, p, None, None, p,
                                         1 << 30, None) == hsa.HSA_ATTN_UNSUPPORTED
    # append: every buffer is required; any chunk size; D in {64, 128}
    assert lib.hsa_append_kv(ctypes.byref(d), p, p, p, p, p, None, None) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert lib.hsa_append_kv(ctypes.byref(d), None, p, p, p, p, p, None) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert lib.hsa_append_kv(ctypes.byref(d), p, p, p, p, p, ctypes.c_void_p(0x1004),
                             None) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert lib.hsa_append_kv(ctypes.byref(dims(head_dim=96)), p, p, p, p, p, p, None) == hsa.HSA_ATTN_UNSUPPORTED


def test_prefill_cached_offset_validation():
    lib = hsa.load_library()
    p = ctypes.c_void_p(0x1000)
    d = dims(seq_len=64 * 100)
    for off in (-64, 65, 64 * 101):
        assert lib.hsa_forward_prefill_cached(ctypes.byref(d), off, p, p, p, p, p, None, None, p, 1 << 40,
                                              None) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert "q_offset" in hsa.hsa_attn_last_error()
    # the whole sequence as prefix: nothing to compute
    assert lib.hsa_forward_prefill_cached(ctypes.byref(d), 64 * 100, p, p, p, p, p, None, None, p, 1 << 40,
                                          None) == hsa.HSA_ATTN_OK


def test_adaptive_decode_validation():
    lib = hsa.load_library()
    p = ctypes.c_void_p(0x1000)

    def call(d, tau, lens=None, ws=1 << 30):
        return lib.hsa_forward_decode_adaptive(ctypes.byref(d), tau, p, p, p, p, lens, p, None, None, p, ws, None)

    for bad in (float("nan"), -1e-6, float("-inf")):
        assert call(dims(), bad) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert call(dims(top_k=33), 0.1) == hsa.HSA_ATTN_UNSUPPORTED  # 2k must fit 64 list slots
    assert call(dims(), 0.1, lens=ctypes.c_void_p(0x1004)) == hsa.HSA_ATTN_INVALID_ARGUMENT  # misaligned
    assert call(dims(), 0.1, ws=16) == hsa.HSA_ATTN_WORKSPACE_TOO_SMALL
    # the adaptive workspace is the plain decode workspace of the doubled budget
    d = dims(top_k=16, seq_len=1 << 20)
    assert hsa.hsa_attn_workspace_size(d, 2) == hsa.hsa_attn_workspace_size(dims(top_k=32, seq_len=1 << 20), 1)
    assert hsa.hsa_attn_workspace_size(dims(top_k=32), 2) > hsa.hsa_attn_workspace_size(dims(top_k=32), 1)
    n = ctypes.c_size_t(0)
    assert lib.hsa_attn_workspace_size(ctypes.byref(d), 5, ctypes.byref(n)) == hsa.HSA_ATTN_INVALID_ARGUMENT


def test_adaptive_prefill_validation():
    lib = hsa.load_library()
    p = ctypes.c_void_p(0x1000)

    def call(d, tau, ws=1 << 40):
        return lib.hsa_forward_prefill_adaptive(ctypes.byref(d), tau, p, p, p, p, p, None, None, p, ws, None)

    for bad in (float("nan"), -0.5):
        assert call(dims(), bad) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert call(dims(top_k=33), 0.1) == hsa.HSA_ATTN_UNSUPPORTED  # 2k must stay <= 64
    assert call(dims(top_k=17, num_q_heads=64), 0.1) == hsa.HSA_ATTN_UNSUPPORTED  # 2k > 32 needs G <= 4
    assert call(dims(), 0.1, ws=16) == hsa.HSA_ATTN_WORKSPACE_TOO_SMALL
    d = dims(top_k=16, seq_len=1 << 15)
    assert hsa.hsa_attn_workspace_size(d, 3) == hsa.hsa_attn_workspace_size(dims(top_k=32, seq_len=1 << 15), 0)


def test_backward_validation():
    lib = hsa.load_library()
    p = ctypes.c_void_p(0x1000)

    def call(d, ws=1 << 40, **null):
        args = [p] * 11
        for i in null.get("null", []):
            args[i] = None
        return lib.hsa_backward_prefill(ctypes.byref(d), *args, p, ws, None)

    assert call(dims(dtype=hsa.HSA_ATTN_FP32)) == hsa.HSA_ATTN_UNSUPPORTED  # bf16 only
    assert call(dims(top_k=33)) == hsa.HSA_ATTN_UNSUPPORTED
    for i in range(11):  # q k v landmarks out dout sel_idx sel_score dq dk dv
        assert call(dims(), null=[i]) == hsa.HSA_ATTN_INVALID_ARGUMENT, i
    assert call(dims(), ws=16) == hsa.HSA_ATTN_WORKSPACE_TOO_SMALL
    assert lib.hsa_backward_prefill(ctypes.byref(dims()), *([ctypes.c_void_p(0x1008)] + [p] * 10), p, 1 << 40,
                                    None) == hsa.HSA_ATTN_INVALID_ARGUMENT  # misaligned
    # workspace: pairs * (4 D + 12) + rows * 4 + transposed K + bucket tables
    d = dims(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, top_k=16, seq_len=1 << 18)
    pairs = 32 * (1 << 18) * 16
    need = hsa.hsa_attn_workspace_size(d, 4)
    assert pairs * (4 * 128 + 12) < need < pairs * (4 * 128 + 12) + (1 << 30) + 8 * 4096 * 64 * 128 * 2


def test_binding_rejects_wrong_output_buffers_before_any_launch():
    """The binding checks every caller-supplied output (shape, dtype, device,
    contiguity) and the workspace before it calls the library: the C ABI
    cannot see buffer sizes, so a wrong buffer would be written out of
    bounds.  CPU tensors stand in for device ones: every check here fires
    before a pointer is taken."""
    import torch
    B, Hq, Hkv, T, D, S, k = 1, 4, 2, 256, 64, 64, 4
    q = torch.zeros((B, Hq, T, D), dtype=torch.bfloat16)
    kv = torch.zeros((B, Hkv, T, D), dtype=torch.bfloat16)
    L = torch.zeros((B, Hkv, T // S, D), dtype=torch.bfloat16)
    f32 = torch.float32
    good_out = torch.zeros((B, Hq, T, D), dtype=f32)
    cases = {
        "out dtype": dict(out=torch.zeros((B, Hq, T, D), dtype=torch.bfloat16)),
        "out shape": dict(out=torch.zeros((B, Hq, T, D + 1), dtype=f32)),
        "out strided": dict(out=torch.zeros((B, Hq, D, T), dtype=f32).transpose(2, 3)),
        "sel_idx int64": dict(out=good_out, sel_idx=torch.zeros((B, Hq, T, k), dtype=torch.int64),
                              sel_score=torch.zeros((B, Hq, T, k), dtype=f32)),
        "sel_idx slots": dict(out=good_out, sel_idx=torch.zeros((B, Hq, T, k + 1), dtype=torch.int32),
                              sel_score=torch.zeros((B, Hq, T, k + 1), dtype=f32)),
        "sel_score dtype": dict(out=good_out, sel_idx=torch.zeros((B, Hq, T, k), dtype=torch.int32),
                                sel_score=torch.zeros((B, Hq, T, k), dtype=torch.float64)),
        "only sel_idx": dict(out=good_out, sel_idx=torch.zeros((B, Hq, T, k), dtype=torch.int32)),
    }
    for name, kw in cases.items():
        with pytest.raises(ValueError):
            hsa.hsa_forward_prefill(q, kv, kv, L, S, k, **kw)
        with pytest.raises(ValueError):
            hsa.hsa_forward_prefill_cached(q[:, :, S:].contiguous(), kv, kv, L, S, S, k,
                                           **{n: (t[:, :, S:].contiguous() if t is not None else None)
                                              for n, t in kw.items()})
    # the adaptive calls write 2k slots per row
    with pytest.raises(ValueError):
        hsa.hsa_forward_prefill_adaptive(q, kv, kv, L, S, k, 0.1, out=good_out,
                                         sel_idx=torch.zeros((B, Hq, T, k), dtype=torch.int32),
                                         sel_score=torch.zeros((B, Hq, T, k), dtype=f32))
    qd = torch.zeros((B, Hq, D), dtype=torch.bfloat16)
    for kw in (dict(out=torch.zeros((B, Hq, D), dtype=torch.bfloat16)),
               dict(out=torch.zeros((B, Hq + 1, D), dtype=f32)),
               dict(sel_idx=torch.zeros((B, Hq, k), dtype=torch.int64), sel_score=torch.zeros((B, Hq, k)))):
        with pytest.raises(ValueError):
            hsa.hsa_forward_decode(qd, kv, kv, L, S, k, **kw)
    with pytest.raises(ValueError):
        hsa.hsa_forward_decode_adaptive(qd, kv, kv, L, S, k, 0.1, out=torch.zeros((B, Hq, D)),
                                        sel_idx=torch.zeros((B, Hq, k), dtype=torch.int32),
                                        sel_score=torch.zeros((B, Hq, k)))
    # backward gradients are float32 [B,Hq,T,D] / [B,Hkv,T,D]
    sel = torch.zeros((B, Hq, T, k), dtype=torch.int32)
    sc = torch.zeros((B, Hq, T, k), dtype=f32)
    for kw in (dict(dq=torch.zeros((B, Hq, T, D), dtype=torch.bfloat16)),
               dict(dk=torch.zeros((B, Hq, T, D), dtype=f32)),
               dict(dv=torch.zeros((B, Hkv, T, D - 1), dtype=f32))):
        with pytest.raises(ValueError):
            hsa.hsa_backward_prefill(q, kv, kv, L, good_out, good_out, sel, sc, S, **kw)


@pytest.mark.gpu
def test_binding_rejects_tensors_on_another_device():
    import torch
    B, Hq, Hkv, T, D, S, k = 1, 4, 2, 256, 64, 64, 4
    q = torch.zeros((B, Hq, T, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, Hkv, T, D), dtype=torch.bfloat16, device="cuda")
    L = torch.zeros((B, Hkv, T // S, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        hsa.hsa_forward_prefill(q, kv, kv, L, S, k, out=torch.zeros((B, Hq, T, D)))
    with pytest.raises(ValueError):
        hsa.hsa_forward_prefill(q, kv, kv, L, S, k, workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        hsa.hsa_forward_prefill(q, kv.cpu(), kv, L, S, k)


def test_noalloc_decode_rejects_oversized_shapes_on_the_host():
    """The no-allocation decode sizes its work before any HIP call: a shape
    whose scratch exceeds the library's fixed array is refused on the host
    (no GPU needed), as are the usual invalid dimensions."""
    lib = hsa.load_library()
    p = ctypes.c_void_p(0x1000)
    big = dims(batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, top_k=64, seq_len=1 << 22)
    st = lib.hsa_forward_decode_noalloc(ctypes.byref(big), p, p, p, p, p, None, None, None)
    assert st == hsa.HSA_ATTN_WORKSPACE_TOO_SMALL
    assert "scratch" in hsa.hsa_attn_last_error()
    bad = dims(num_q_heads=30)
    assert lib.hsa_forward_decode_noalloc(ctypes.byref(bad), p, p, p, p, p, None, None, None) == \
        hsa.HSA_ATTN_INVALID_ARGUMENT


DEBUG_LIB = os.path.join(ROOT, "hierarchical_sparse_attention_hsa_amd", "libhsa_attn_debug.so")


@pytest.mark.skipif(not os.path.exists(DEBUG_LIB), reason="libhsa_attn_debug.so not built")
def test_debug_library_exports_the_same_calls_and_reserves_its_flag_block():
    # the debug build (HSA_ATTN_DEBUG=1) exports every declared call; its
    # workspaces carry a 256-byte flag block in front of the release layout
    out = os.popen(f"nm -D --defined-only {DEBUG_LIB}").read()
    for name in header_functions():
        assert re.search(rf"\bT {name}\b", out), name
    shapes = [(dims(batch=2, seq_len=64 * 100 + 7), 1), (dims(seq_len=64 * 40), 0), (dims(seq_len=64 * 40), 4)]
    release = [hsa.hsa_attn_workspace_size(d, kind) for d, kind in shapes]
    with hsa.debug_library():
        assert hsa.library_path() == DEBUG_LIB
        debug = [hsa.hsa_attn_workspace_size(d, kind) for d, kind in shapes]
        # a NULL flags pointer is rejected before any HIP call
        st = hsa.load_library().hsa_attn_debug_flags(None, None)
        assert st == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert [x - y for x, y in zip(debug, release)] == [256] * len(shapes)
    assert hsa.library_path().endswith("libhsa_attn.so")


def test_release_library_has_no_debug_flags():
    flags = ctypes.c_uint32(7)
    st = hsa.load_library().hsa_attn_debug_flags(None, ctypes.byref(flags))
    assert st == hsa.HSA_ATTN_UNSUPPORTED and flags.value == 7
    assert "HSA_ATTN_DEBUG" in hsa.hsa_attn_last_error()


def test_debug_environment_variable_selects_the_debug_library():
    code = ("import hierarchical_sparse_attention_hsa_amd as h, ctypes; "
            "print(h.library_path()); "
            "print(h.load_library().hsa_attn_debug_flags(None, None))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root,
                       env=dict(os.environ, HSA_ATTN_DEBUG="1"), timeout=300)
    assert r.returncode == 0, r.stderr
    path, status = r.stdout.split()
    assert path.endswith("libhsa_attn_debug.so")
    assert int(status) == hsa.HSA_ATTN_INVALID_ARGUMENT  # the debug build's answer to a NULL flags pointer


def test_empty_calls_return_ok_without_looking_at_pointers():
    """No query rows means nothing to read or write: the call returns OK
    before any pointer check, so the NULL data pointers of empty tensors are
    accepted (no HIP call is made, so this runs without a GPU)."""
    lib = hsa.load_library()
    d0 = dims(seq_len=0)
    n11 = [None] * 11
    assert lib.hsa_forward_prefill(ctypes.byref(d0), None, None, None, None, None, None, None, None, 0,
                                   None) == hsa.HSA_ATTN_OK
    assert lib.hsa_forward_prefill_adaptive(ctypes.byref(d0), ctypes.c_float(0.5), None, None, None, None, None,
                                            None, None, None, 0, None) == hsa.HSA_ATTN_OK
    assert lib.hsa_backward_prefill(ctypes.byref(d0), *n11, None, 0, None) == hsa.HSA_ATTN_OK
    # a cached prefix covering the whole sequence: q and out are empty
    p = ctypes.c_void_p(0x1000)
    d = dims(seq_len=64 * 10)
    assert lib.hsa_forward_prefill_cached(ctypes.byref(d), 64 * 10, None, p, p, p, None, None, None, None, 0,
                                          None) == hsa.HSA_ATTN_OK
    # empty calls still reject malformed dims
    assert lib.hsa_forward_prefill(ctypes.byref(dims(seq_len=0, top_k=0)), None, None, None, None, None, None,
                                   None, None, 0, None) == hsa.HSA_ATTN_INVALID_ARGUMENT
    assert lib.hsa_backward_prefill(ctypes.byref(dims(seq_len=0, dtype=hsa.HSA_ATTN_FP32)), *n11, None, 0,
                                    None) == hsa.HSA_ATTN_UNSUPPORTED
    # a non-empty prefill still needs its pointers
    assert lib.hsa_forward_prefill(ctypes.byref(dims(seq_len=64)), None, p, p, p, p, None, None, p, 1 << 30,
                                   None) == hsa.HSA_ATTN_INVALID_ARGUMENT
