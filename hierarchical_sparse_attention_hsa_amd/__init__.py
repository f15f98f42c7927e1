"""Hierarchical Sparse Attention (HSA) forward layer for AMD MI355X (gfx950).

Thin Python binding of the C ABI in ``include/hsa_attn.h`` (libhsa_attn.so,
built in-tree by ``hierarchical_sparse_attention_hsa_amd.build``).  The
binding only marshals arguments: torch tensors supply device pointers and the
current HIP stream, and every step of the layer runs in the library's HIP
kernels.  There is no fallback: if the library is missing or a call fails,
an exception is raised.

Functions carry the C names:

    hsa_build_landmarks(k, landmarks, chunk_size, chunk_begin=0, chunk_end=None)
    hsa_forward_prefill(q, k, v, landmarks, chunk_size, top_k, out=None, sel_idx=None, sel_score=None, workspace=None)
    hsa_forward_decode(q, k_cache, v_cache, landmarks, chunk_size, top_k, out=None, sel_idx=None, sel_score=None, workspace=None)
    hsa_forward_prefill_cached(q_new, k, v, landmarks, q_offset, chunk_size, top_k, ...)
    hsa_forward_decode_varlen(q, k_cache, v_cache, landmarks, cache_lens, chunk_size, top_k, ...)
    hsa_append_kv(k_new, v_new, k_cache, v_cache, landmarks, cache_lens, chunk_size)
    hsa_attn_workspace_size(...)
"""
from __future__ import annotations

import contextlib
import ctypes
import os

__all__ = [
    "library_path", "load_library", "Dims", "HSAError", "EXPORTED_SYMBOLS",
    "hsa_build_landmarks", "hsa_forward_prefill", "hsa_forward_prefill_cached", "hsa_forward_decode",
    "hsa_forward_decode_varlen", "hsa_forward_decode_adaptive", "hsa_forward_prefill_adaptive", "hsa_append_kv",
    "hsa_backward_prefill", "hsa_attn_set_timing_events", "hsa_attn_workspace_size",
    "hsa_attn_status_string", "hsa_attn_last_error", "landmarks_shape", "hsa_forward_decode_noalloc",
    "hsa_attn_prefill_slab_rows", "hsa_attn_debug_flags", "debug_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
EXPORTED_SYMBOLS = (
    "hsa_build_landmarks", "hsa_forward_prefill", "hsa_forward_prefill_cached", "hsa_forward_decode",
    "hsa_forward_decode_varlen", "hsa_forward_decode_adaptive", "hsa_forward_prefill_adaptive",
    "hsa_append_kv", "hsa_backward_prefill", "hsa_attn_set_timing_events", "hsa_attn_workspace_size",
    "hsa_attn_status_string",
    "hsa_attn_last_error", "hsa_forward_decode_noalloc", "hsa_attn_prefill_slab_rows", "hsa_attn_debug_flags",
)

HSA_ATTN_OK = 0
HSA_ATTN_INVALID_ARGUMENT = 1
HSA_ATTN_UNSUPPORTED = 2
HSA_ATTN_WORKSPACE_TOO_SMALL = 3
HSA_ATTN_HIP_ERROR = 4
HSA_ATTN_FP32 = 0
HSA_ATTN_BF16 = 1


class Dims(ctypes.Structure):
    """Mirror of hsa_attn_dims_t."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("seq_len", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class HSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libhsa_attn_debug.so" if _ACTIVE == "debug" else "libhsa_attn.so")


_LIB = None          # the library the calls go to
_LOADED = {}         # "release" / "debug" -> loaded library
# HSA_ATTN_DEBUG=1 in the environment sends every call of the process to the
# debug library
_ACTIVE = "debug" if os.environ.get("HSA_ATTN_DEBUG", "") == "1" else "release"


@contextlib.contextmanager
def debug_library():
    """Within the block, every call goes to libhsa_attn_debug.so: the same
    kernels built with HSA_ATTN_DEBUG=1, which poison each call's workspace
    and outputs before its kernels and check the indices the kernels read
    back from the workspace (hsa_attn_debug_flags reads the result).  Its
    workspaces are 256 bytes larger (hsa_attn_workspace_size inside the
    block gives the size)."""
    global _LIB, _ACTIVE
    prev_lib, prev_active = _LIB, _ACTIVE
    _ACTIVE, _LIB = "debug", _LOADED.get("debug")
    try:
        load_library()
        yield
    finally:
        _LIB, _ACTIVE = prev_lib, prev_active


def load_library():
    """Load libhsa_attn.so (built in-tree; libhsa_attn_debug.so inside
    debug_library()); raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if _ACTIVE in _LOADED:
        _LIB = _LOADED[_ACTIVE]
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m hierarchical_sparse_attention_hsa_amd.build`")
    lib = ctypes.CDLL(path)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    dims = ctypes.POINTER(Dims)
    lib.hsa_build_landmarks.argtypes = [dims, P, P, I64, I64, P]
    lib.hsa_forward_prefill.argtypes = [dims, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_forward_decode.argtypes = [dims, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_forward_decode_noalloc.argtypes = [dims, P, P, P, P, P, P, P, P]
    lib.hsa_forward_decode_varlen.argtypes = [dims, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_forward_prefill_cached.argtypes = [dims, I64, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_forward_decode_adaptive.argtypes = [dims, ctypes.c_float, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_forward_prefill_adaptive.argtypes = [dims, ctypes.c_float, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_backward_prefill.argtypes = [dims, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    lib.hsa_append_kv.argtypes = [dims, P, P, P, P, P, P, P]
    lib.hsa_attn_workspace_size.argtypes = [dims, ctypes.c_int, ctypes.POINTER(SZ)]
    lib.hsa_attn_prefill_slab_rows.argtypes = [dims, ctypes.c_int, ctypes.c_int, SZ, ctypes.POINTER(I64)]
    lib.hsa_attn_set_timing_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.hsa_attn_status_string.argtypes = [ctypes.c_int]
    lib.hsa_attn_status_string.restype = ctypes.c_char_p
    lib.hsa_attn_last_error.argtypes = []
    lib.hsa_attn_last_error.restype = ctypes.c_char_p
    lib.hsa_attn_debug_flags.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
    for f in ("hsa_build_landmarks", "hsa_forward_prefill", "hsa_forward_prefill_cached", "hsa_forward_decode",
              "hsa_forward_decode_noalloc",
              "hsa_forward_decode_varlen", "hsa_forward_decode_adaptive", "hsa_forward_prefill_adaptive",
              "hsa_append_kv", "hsa_backward_prefill", "hsa_attn_workspace_size", "hsa_attn_set_timing_events",
              "hsa_attn_prefill_slab_rows", "hsa_attn_debug_flags"):
        getattr(lib, f).restype = ctypes.c_int
    _LOADED[_ACTIVE] = lib
    _LIB = lib
    return lib


def hsa_attn_debug_flags(workspace=None) -> int:
    """Flag word of the last debug-library call that used `workspace` (a
    device tensor; None: the no-allocation decode's scratch): 0 when every
    check passed, else HSA_ATTN_DEBUG_* bits (include/hsa_attn.h).  Waits
    for the device.  The release library raises HSAError (unsupported)."""
    flags = ctypes.c_uint32(0)
    ptr = None if workspace is None else workspace.data_ptr()
    _check(load_library().hsa_attn_debug_flags(ptr, ctypes.byref(flags)), "hsa_attn_debug_flags")
    return int(flags.value)


def hsa_attn_status_string(status: int) -> str:
    return load_library().hsa_attn_status_string(status).decode()


def hsa_attn_last_error() -> str:
    return load_library().hsa_attn_last_error().decode()


def _check(status: int, what: str):
    if status != HSA_ATTN_OK:
        raise HSAError(status, f"{what}: {hsa_attn_status_string(status)}: {hsa_attn_last_error()}")


# ---------------------------------------------------------------- tensor marshalling

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return HSA_ATTN_BF16
    if t.dtype == torch.float32:
        return HSA_ATTN_FP32
    raise TypeError(f"unsupported storage dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_dims(batch, num_q_heads, num_kv_heads, head_dim, chunk_size, top_k, seq_len, dtype) -> Dims:
    return Dims(batch, num_q_heads, num_kv_heads, head_dim, chunk_size, top_k, seq_len, dtype, 0)


def _same_device(device, *tensors):
    """Every given tensor lives on `device` (the library reads and writes them
    with kernels launched there)."""
    for t in tensors:
        if t is not None and t.device != device:
            raise ValueError(f"all tensors must be on {device}, got one on {t.device}")


def _output(t, shape, dtype, device, name):
    """Validate a caller-supplied output buffer, or allocate one.  The C ABI
    cannot see buffer sizes, so a wrong shape or dtype here would become an
    out-of-bounds device write."""
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _selection(sel_idx, sel_score, shape, device):
    """Optional selection outputs: both or neither, int32 / float32 of shape
    [..., slots]."""
    torch = _torch()
    if (sel_idx is None) != (sel_score is None):
        raise ValueError("give both sel_idx and sel_score or neither")
    if sel_idx is None:
        return None, None
    return (_output(sel_idx, shape, torch.int32, device, "sel_idx"),
            _output(sel_score, shape, torch.float32, device, "sel_score"))


def _workspace(workspace, dims, kind, device):
    """The caller's workspace (any dtype, contiguous, on the device), or a
    new one of hsa_attn_workspace_size bytes."""
    torch = _torch()
    if workspace is None:
        need = hsa_attn_workspace_size(dims, kind)
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if workspace.device != device:
        raise ValueError(f"workspace must be on {device}, got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace


def landmarks_shape(k_shape, chunk_size):
    B, Hkv, T, D = k_shape
    return (B, Hkv, T // chunk_size, D)


def hsa_attn_set_timing_events(events) -> None:
    """Record caller-created hipEvent_t handles (ints) around each kernel
    launch of the following calls on this thread: events[2i] before and
    events[2i+1] after launch i.  Pass None or [] to switch off."""
    global _EVENT_ARRAY
    if not events:
        _EVENT_ARRAY = None
        _check(load_library().hsa_attn_set_timing_events(None, 0), "hsa_attn_set_timing_events")
        return
    if len(events) % 2:
        raise ValueError("events come in (before, after) pairs")
    arr = (ctypes.c_void_p * len(events))(*events)
    _EVENT_ARRAY = arr  # keep alive while the library holds the pointer
    _check(load_library().hsa_attn_set_timing_events(arr, len(events) // 2), "hsa_attn_set_timing_events")


_EVENT_ARRAY = None


def hsa_attn_workspace_size(dims: Dims, is_decode) -> int:
    """Workspace bytes; is_decode: False/0 prefill, True/1 decode, 2 adaptive-budget decode,
    3 adaptive-budget prefill, 4 prefill backward."""
    n = ctypes.c_size_t(0)
    _check(load_library().hsa_attn_workspace_size(ctypes.byref(dims), int(is_decode), ctypes.byref(n)),
           "hsa_attn_workspace_size")
    return n.value


def hsa_attn_prefill_slab_rows(dims: Dims, workspace_bytes: int, adaptive: bool = False,
                               selection_given: bool = False) -> int:
    """Query rows per slab a prefill call uses with a workspace of
    workspace_bytes (0: too small)."""
    n = ctypes.c_int64(0)
    _check(load_library().hsa_attn_prefill_slab_rows(ctypes.byref(dims), int(bool(adaptive)),
                                                     int(bool(selection_given)), int(workspace_bytes),
                                                     ctypes.byref(n)), "hsa_attn_prefill_slab_rows")
    return n.value


def hsa_build_landmarks(k, landmarks, chunk_size: int, chunk_begin: int = 0, chunk_end=None):
    """Mean-pool chunks [chunk_begin, chunk_end) of k [B, Hkv, T, D] into
    landmarks [B, Hkv, T // chunk_size, D] (same dtype), asynchronously."""
    B, Hkv, T, D = k.shape
    if tuple(landmarks.shape) != landmarks_shape(k.shape, chunk_size) or landmarks.dtype != k.dtype:
        raise ValueError("landmarks must be [B, Hkv, T // chunk_size, D] with the dtype of k")
    if chunk_end is None:
        chunk_end = T // chunk_size
    dims = make_dims(B, Hkv, Hkv, D, chunk_size, 1, T, _dtype_code(k))
    _same_device(k.device, landmarks)
    _check(load_library().hsa_build_landmarks(ctypes.byref(dims), _ptr(k), _ptr(landmarks), int(chunk_begin),
                                              int(chunk_end), _stream(k.device)), "hsa_build_landmarks")
    return landmarks


def _forward(is_decode, q, k, v, landmarks, chunk_size, top_k, out, sel_idx, sel_score, workspace, lens=None):
    torch = _torch()
    B, Hkv, T, D = k.shape
    Hq = q.shape[1]
    if v.shape != k.shape or v.dtype != k.dtype or q.dtype != k.dtype:
        raise ValueError("q, k and v must share dtype; v must match k's shape")
    expect_q = (B, Hq, D) if is_decode else (B, Hq, T, D)
    if tuple(q.shape) != expect_q:
        raise ValueError(f"q must be {expect_q}, got {tuple(q.shape)}")
    if tuple(landmarks.shape) != landmarks_shape(k.shape, chunk_size) or landmarks.dtype != k.dtype:
        raise ValueError("landmarks must be [B, Hkv, T // chunk_size, D] with the dtype of k")
    dims = make_dims(B, Hq, Hkv, D, chunk_size, top_k, T, _dtype_code(k))
    _same_device(q.device, k, v, landmarks, lens)
    out = _output(out, expect_q, torch.float32, q.device, "out")
    sel_idx, sel_score = _selection(sel_idx, sel_score, expect_q[:-1] + (top_k,), q.device)
    workspace = _workspace(workspace, dims, int(is_decode), q.device)
    lib = load_library()
    if lens is not None:
        if lens.dtype != torch.int64 or tuple(lens.shape) != (B,):
            raise ValueError("cache_lens must be an int64 tensor of shape [B]")
        st = lib.hsa_forward_decode_varlen(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(landmarks),
                                           _ptr(lens), _ptr(out), _ptr(sel_idx), _ptr(sel_score), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(q.device))
        _check(st, "hsa_forward_decode_varlen")
        return out
    fn = lib.hsa_forward_decode if is_decode else lib.hsa_forward_prefill
    st = fn(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(landmarks), _ptr(out), _ptr(sel_idx),
            _ptr(sel_score), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(st, "hsa_forward_decode" if is_decode else "hsa_forward_prefill")
    return out


def hsa_forward_prefill(q, k, v, landmarks, chunk_size: int, top_k: int, out=None, sel_idx=None, sel_score=None,
                        workspace=None):
    """Causal HSA over a sequence: q [B,Hq,T,D], k/v [B,Hkv,T,D] -> out [B,Hq,T,D] fp32."""
    return _forward(False, q, k, v, landmarks, chunk_size, top_k, out, sel_idx, sel_score, workspace)


def hsa_forward_decode(q, k_cache, v_cache, landmarks, chunk_size: int, top_k: int, out=None, sel_idx=None,
                       sel_score=None, workspace=None):
    """HSA for single-token queries q [B,Hq,D] after caches k/v [B,Hkv,T,D] -> out [B,Hq,D] fp32."""
    return _forward(True, q, k_cache, v_cache, landmarks, chunk_size, top_k, out, sel_idx, sel_score, workspace)


def hsa_forward_decode_noalloc(q, k_cache, v_cache, landmarks, chunk_size: int, top_k: int, out, sel_idx=None,
                               sel_score=None):
    """hsa_forward_decode without a workspace: the library uses its own
    fixed per-GPU scratch array and allocates nothing (the caller passes the
    output buffer too).  Calls that overlap on one GPU race."""
    torch = _torch()
    B, Hkv, T, D = k_cache.shape
    Hq = q.shape[1]
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q, k and v must share dtype; v must match k's shape")
    if tuple(q.shape) != (B, Hq, D):
        raise ValueError(f"q must be {(B, Hq, D)}, got {tuple(q.shape)}")
    if tuple(landmarks.shape) != landmarks_shape(k_cache.shape, chunk_size) or landmarks.dtype != k_cache.dtype:
        raise ValueError("landmarks must be [B, Hkv, T // chunk_size, D] with the dtype of k")
    if out is None:
        raise ValueError("out must be given: this entry point allocates nothing")
    _same_device(q.device, k_cache, v_cache, landmarks)
    out = _output(out, (B, Hq, D), torch.float32, q.device, "out")
    sel_idx, sel_score = _selection(sel_idx, sel_score, (B, Hq, top_k), q.device)
    dims = make_dims(B, Hq, Hkv, D, chunk_size, top_k, T, _dtype_code(k_cache))
    st = load_library().hsa_forward_decode_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                   _ptr(landmarks), _ptr(out), _ptr(sel_idx), _ptr(sel_score),
                                                   _stream(q.device))
    _check(st, "hsa_forward_decode_noalloc")
    return out


def hsa_forward_decode_varlen(q, k_cache, v_cache, landmarks, cache_lens, chunk_size: int, top_k: int, out=None,
                              sel_idx=None, sel_score=None, workspace=None):
    """HSA for single-token queries q [B,Hq,D] after caches k/v [B,Hkv,T_cap,D]
    holding cache_lens[b] tokens each (int64 [B] on the device) -> out [B,Hq,D] fp32."""
    return _forward(True, q, k_cache, v_cache, landmarks, chunk_size, top_k, out, sel_idx, sel_score, workspace,
                    lens=cache_lens)


def hsa_forward_decode_adaptive(q, k_cache, v_cache, landmarks, chunk_size: int, top_k: int, gap_threshold: float,
                                cache_lens=None, out=None, sel_idx=None, sel_score=None, workspace=None):
    """Decode with the near-tie adaptive budget: a query head keeps its best
    2*top_k chunks when its top_k-th and (top_k+1)-th scores differ by less
    than gap_threshold, else top_k.  q [B,Hq,D], caches [B,Hkv,T,D] (cache_lens
    optional, int64 [B] device) -> out [B,Hq,D] fp32; sel_idx/sel_score
    [B,Hq,2*top_k]."""
    torch = _torch()
    B, Hkv, T, D = k_cache.shape
    Hq = q.shape[1]
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype or q.dtype != k_cache.dtype:
        raise ValueError("q, k and v must share dtype; v must match k's shape")
    if tuple(q.shape) != (B, Hq, D):
        raise ValueError(f"q must be {(B, Hq, D)}, got {tuple(q.shape)}")
    if tuple(landmarks.shape) != landmarks_shape(k_cache.shape, chunk_size) or landmarks.dtype != k_cache.dtype:
        raise ValueError("landmarks must be [B, Hkv, T // chunk_size, D] with the dtype of k")
    if cache_lens is not None and (cache_lens.dtype != torch.int64 or tuple(cache_lens.shape) != (B,)):
        raise ValueError("cache_lens must be an int64 tensor of shape [B]")
    dims = make_dims(B, Hq, Hkv, D, chunk_size, top_k, T, _dtype_code(k_cache))
    _same_device(q.device, k_cache, v_cache, landmarks, cache_lens)
    out = _output(out, (B, Hq, D), torch.float32, q.device, "out")
    sel_idx, sel_score = _selection(sel_idx, sel_score, (B, Hq, 2 * top_k), q.device)
    workspace = _workspace(workspace, dims, 2, q.device)
    st = load_library().hsa_forward_decode_adaptive(
        ctypes.byref(dims), float(gap_threshold), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(landmarks),
        _ptr(cache_lens), _ptr(out), _ptr(sel_idx), _ptr(sel_score), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(st, "hsa_forward_decode_adaptive")
    return out


def hsa_forward_prefill_adaptive(q, k, v, landmarks, chunk_size: int, top_k: int, gap_threshold: float, out=None,
                                 sel_idx=None, sel_score=None, workspace=None):
    """Causal prefill with the near-tie adaptive budget: a query row keeps its
    best 2*top_k chunks when its top_k-th and (top_k+1)-th scores differ by
    less than gap_threshold, else top_k.  q [B,Hq,T,D], k/v [B,Hkv,T,D] ->
    out [B,Hq,T,D] fp32; sel_idx/sel_score [B,Hq,T,2*top_k]."""
    torch = _torch()
    B, Hkv, T, D = k.shape
    Hq = q.shape[1]
    if v.shape != k.shape or v.dtype != k.dtype or q.dtype != k.dtype:
        raise ValueError("q, k and v must share dtype; v must match k's shape")
    if tuple(q.shape) != (B, Hq, T, D):
        raise ValueError(f"q must be {(B, Hq, T, D)}, got {tuple(q.shape)}")
    if tuple(landmarks.shape) != landmarks_shape(k.shape, chunk_size) or landmarks.dtype != k.dtype:
        raise ValueError("landmarks must be [B, Hkv, T // chunk_size, D] with the dtype of k")
    dims = make_dims(B, Hq, Hkv, D, chunk_size, top_k, T, _dtype_code(k))
    _same_device(q.device, k, v, landmarks)
    out = _output(out, (B, Hq, T, D), torch.float32, q.device, "out")
    sel_idx, sel_score = _selection(sel_idx, sel_score, (B, Hq, T, 2 * top_k), q.device)
    workspace = _workspace(workspace, dims, 3, q.device)
    st = load_library().hsa_forward_prefill_adaptive(
        ctypes.byref(dims), float(gap_threshold), _ptr(q), _ptr(k), _ptr(v), _ptr(landmarks), _ptr(out),
        _ptr(sel_idx), _ptr(sel_score), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q.device))
    _check(st, "hsa_forward_prefill_adaptive")
    return out


def hsa_backward_prefill(q, k, v, landmarks, out, dout, sel_idx, sel_score, chunk_size: int, dq=None, dk=None,
                         dv=None, workspace=None):
    """Gradients of the causal prefill: q [B,Hq,T,D], k/v [B,Hkv,T,D] (bf16),
    the forward's out [B,Hq,T,D] fp32 and selection sel_idx/sel_score
    [B,Hq,T,k], and the upstream gradient dout [B,Hq,T,D] fp32 ->
    (dq [B,Hq,T,D], dk, dv [B,Hkv,T,D]) fp32."""
    torch = _torch()
    B, Hkv, T, D = k.shape
    Hq = q.shape[1]
    if v.shape != k.shape or v.dtype != k.dtype or q.dtype != k.dtype:
        raise ValueError("q, k and v must share dtype; v must match k's shape")
    if tuple(q.shape) != (B, Hq, T, D) or tuple(out.shape) != (B, Hq, T, D) or tuple(dout.shape) != (B, Hq, T, D):
        raise ValueError("q, out and dout must be [B, Hq, T, D]")
    if out.dtype != torch.float32 or dout.dtype != torch.float32:
        raise ValueError("out and dout must be float32")
    if tuple(landmarks.shape) != landmarks_shape(k.shape, chunk_size) or landmarks.dtype != k.dtype:
        raise ValueError("landmarks must be [B, Hkv, T // chunk_size, D] with the dtype of k")
    top_k = sel_idx.shape[-1]
    if tuple(sel_idx.shape) != (B, Hq, T, top_k) or sel_score.shape != sel_idx.shape:
        raise ValueError("sel_idx and sel_score must be [B, Hq, T, k]")
    if sel_idx.dtype != torch.int32 or sel_score.dtype != torch.float32:
        raise ValueError("sel_idx must be int32 and sel_score float32")
    dims = make_dims(B, Hq, Hkv, D, chunk_size, top_k, T, _dtype_code(k))
    _same_device(q.device, k, v, landmarks, out, dout, sel_idx, sel_score)
    dq = _output(dq, (B, Hq, T, D), torch.float32, q.device, "dq")
    dk = _output(dk, (B, Hkv, T, D), torch.float32, q.device, "dk")
    dv = _output(dv, (B, Hkv, T, D), torch.float32, q.device, "dv")
    workspace = _workspace(workspace, dims, 4, q.device)
    st = load_library().hsa_backward_prefill(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(landmarks), _ptr(out), _ptr(dout), _ptr(sel_idx),
        _ptr(sel_score), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q.device))
    _check(st, "hsa_backward_prefill")
    return dq, dk, dv


def hsa_append_kv(k_new, v_new, k_cache, v_cache, landmarks, cache_lens, chunk_size: int):
    """Append k_new/v_new [B,Hkv,D] at position cache_lens[b] of the caches
    [B,Hkv,T_cap,D], build the landmark of a chunk the token completes, and
    advance cache_lens (int64 [B], device), asynchronously."""
    torch = _torch()
    B, Hkv, T, D = k_cache.shape
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new and v_new must be [B, Hkv, D]")
    if v_cache.shape != k_cache.shape or len({t.dtype for t in (k_new, v_new, k_cache, v_cache, landmarks)}) != 1:
        raise ValueError("caches, new rows and landmarks must share dtype and cache shape")
    if tuple(landmarks.shape) != landmarks_shape(k_cache.shape, chunk_size):
        raise ValueError("landmarks must be [B, Hkv, T_cap // chunk_size, D]")
    if cache_lens.dtype != torch.int64 or tuple(cache_lens.shape) != (B,):
        raise ValueError("cache_lens must be an int64 tensor of shape [B]")
    dims = make_dims(B, Hkv, Hkv, D, chunk_size, 1, T, _dtype_code(k_cache))
    _same_device(k_cache.device, k_new, v_new, v_cache, landmarks, cache_lens)
    _check(load_library().hsa_append_kv(ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(landmarks), _ptr(cache_lens), _stream(k_cache.device)),
           "hsa_append_kv")


def hsa_forward_prefill_cached(q, k, v, landmarks, q_offset: int, chunk_size: int, top_k: int, out=None,
                               sel_idx=None, sel_score=None, workspace=None):
    """Causal HSA for the last Tq = T - q_offset positions of a sequence whose
    keys k/v [B,Hkv,T,D] (prefix and new tokens) and landmarks are given:
    q [B,Hq,Tq,D] -> out [B,Hq,Tq,D] fp32."""
    torch = _torch()
    B, Hkv, T, D = k.shape
    Hq = q.shape[1]
    Tq = T - q_offset
    if v.shape != k.shape or v.dtype != k.dtype or q.dtype != k.dtype:
        raise ValueError("q, k and v must share dtype; v must match k's shape")
    if tuple(q.shape) != (B, Hq, Tq, D):
        raise ValueError(f"q must be {(B, Hq, Tq, D)}, got {tuple(q.shape)}")
    if tuple(landmarks.shape) != landmarks_shape(k.shape, chunk_size) or landmarks.dtype != k.dtype:
        raise ValueError("landmarks must be [B, Hkv, T // chunk_size, D] with the dtype of k")
    dims = make_dims(B, Hq, Hkv, D, chunk_size, top_k, T, _dtype_code(k))
    _same_device(q.device, k, v, landmarks)
    out = _output(out, (B, Hq, Tq, D), torch.float32, q.device, "out")
    sel_idx, sel_score = _selection(sel_idx, sel_score, (B, Hq, Tq, top_k), q.device)
    workspace = _workspace(workspace, dims, 0, q.device)
    st = load_library().hsa_forward_prefill_cached(ctypes.byref(dims), int(q_offset), _ptr(q), _ptr(k), _ptr(v),
                                                   _ptr(landmarks), _ptr(out), _ptr(sel_idx), _ptr(sel_score),
                                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                                   _stream(q.device))
    _check(st, "hsa_forward_prefill_cached")
    return out
