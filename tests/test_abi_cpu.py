"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

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
    assert status_of(dims(top_k=33), "prefill") == hsa.HSA_ATTN_UNSUPPORTED
    assert status_of(dims(top_k=65), "decode") == hsa.HSA_ATTN_UNSUPPORTED
    # landmarks accept any chunk size and group size
    assert status_of(dims(chunk_size=1, num_q_heads=3, num_kv_heads=3), "landmarks", c0=0, c1=0) == 0


@pytest.mark.parametrize("is_decode", [0, 1])
def test_workspace_size_and_too_small_workspace(is_decode):
    d = dims(batch=2, seq_len=64 * 100 + 7)
    n = hsa.hsa_attn_workspace_size(d, is_decode)
    assert n > 0 and n % 256 == 0
    call = "decode" if is_decode else "prefill"
    assert status_of(d, call, ws=n - 1) == hsa.HSA_ATTN_WORKSPACE_TOO_SMALL
    assert "workspace" in hsa.hsa_attn_last_error()
    if not is_decode:
        assert n >= 2 * 32 * (64 * 100 + 7) * 16 * 4  # selection of every row


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
    assert call(dims(top_k=17), 0.1) == hsa.HSA_ATTN_UNSUPPORTED  # 2k must stay <= 32
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
