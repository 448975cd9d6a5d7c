"""Thin ctypes binding of libpensieve (include/pensieve.h).

Argument marshalling only: every function takes torch tensors for device
buffers (PyTorch supplies device memory and streams), checks that they are
contiguous tensors of the expected dtype on the current GPU, and calls the C
entry point of the same name.  All arithmetic happens in the library's HIP
kernels; there is no fallback path.  A missing library raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpensieve.so")

PENSIEVE_OK = 0
PENSIEVE_ERR_INVALID_ARG = 1
PENSIEVE_ERR_UNSUPPORTED = 2
PENSIEVE_ERR_WORKSPACE_TOO_SMALL = 3
PENSIEVE_ERR_HIP = 4
PENSIEVE_F32, PENSIEVE_F16, PENSIEVE_BF16, PENSIEVE_FP8_E4M3 = 0, 1, 2, 3
PENSIEVE_FLAG_VECTOR_ONLY = 1
PENSIEVE_FLAG_NO_SPLIT = 2
PENSIEVE_FLAG_SINGLE_STREAM = 4

EXPORTED = (
    "pensieve_version", "pensieve_last_error", "pensieve_kv_append", "pensieve_attn_workspace_size",
    "pensieve_attn_fwd", "pensieve_attn_split_partial", "pensieve_attn_split_merge", "pensieve_debug_plan",
    "pensieve_trace_enable", "pensieve_trace_read", "pensieve_kv_swap_out", "pensieve_kv_swap_in",
    "pensieve_cache_plan_evictions", "pensieve_cache_build_batch", "pensieve_kv_append_fp8",
    "pensieve_attn_fwd_noalloc",
)
TRACE_KERNELS = {0: "kv_append", 1: "attn_vector", 2: "attn_mfma", 3: "split_merge", 4: "kv_swap"}


class PensieveError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pensieve status {status}: {message}")
        self.status = status


class BatchDesc(ctypes.Structure):
    """Mirror of pensieve_batch_desc; keeps its host length arrays alive."""

    _fields_ = [
        ("num_reqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("flags", ctypes.c_int32),
        ("context_lens_host", ctypes.POINTER(ctypes.c_int32)),
        ("cu_q_lens_host", ctypes.POINTER(ctypes.c_int32)),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("q_pos_host", ctypes.POINTER(ctypes.c_int32)),
    ]


class TraceRecord(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("items", ctypes.c_int32), ("ms", ctypes.c_float)]


# Mirror of pensieve_conversation (host planning calls).
CONVERSATION_DTYPE = np.dtype([("cached_tokens", "<i4"), ("dropped_blocks", "<i4"), ("new_tokens", "<i4"),
                               ("activity", "<f4")], align=True)

_lib = None


def load_library(path: Optional[str] = None):
    """Load libpensieve.so (built in-tree by paged_kv_token_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m paged_kv_token_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
    dp = ctypes.POINTER(BatchDesc)
    lib.pensieve_version.restype = ctypes.c_char_p
    lib.pensieve_last_error.restype = ctypes.c_char_p
    lib.pensieve_kv_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    f32 = ctypes.c_float
    lib.pensieve_kv_append_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, vp]
    lib.pensieve_kv_swap_out.argtypes = [vp, vp, i32, vp, vp, i32, i32p, i32p, i32, i32, i32, i32, vp]
    lib.pensieve_kv_swap_in.argtypes = [vp, vp, i32, vp, vp, i32, i32p, i32p, i32, i32, i32, i32, vp]
    lib.pensieve_attn_workspace_size.argtypes = [dp, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.pensieve_attn_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.pensieve_attn_fwd_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.pensieve_attn_split_partial.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                ctypes.c_size_t, vp]
    lib.pensieve_attn_split_merge.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.pensieve_debug_plan.argtypes = [dp, i32, i32p, i32, i32p]
    lib.pensieve_trace_enable.argtypes = [i32]
    lib.pensieve_trace_read.argtypes = [ctypes.POINTER(TraceRecord), i32, i32p]
    lib.pensieve_cache_plan_evictions.argtypes = [vp, i32, i32, i32p, i32p]
    lib.pensieve_cache_build_batch.argtypes = [vp, i32, i32p, i32, i32p, i32, i32, i32p, i32p, i32p,
                                               i32p, i32p, i32p, i32p, i32p, i32p]
    for name in EXPORTED[2:]:
        getattr(lib, name).restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != PENSIEVE_OK:
        raise PensieveError(status, load_library().pensieve_last_error().decode())


# ---- tensor marshalling ------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    """pensieve_dtype of a tensor; uint8 and float8_e4m3fn tensors are E4M3 pools."""
    torch = _torch()
    return {torch.float32: PENSIEVE_F32, torch.float16: PENSIEVE_F16, torch.bfloat16: PENSIEVE_BF16,
            torch.uint8: PENSIEVE_FP8_E4M3, torch.float8_e4m3fn: PENSIEVE_FP8_E4M3}[t.dtype]


def _pool_ptr(t, name: str, desc_or_code, q=None):
    """A pool tensor: the query dtype, or (E4M3 pools) uint8 / float8_e4m3fn."""
    code = desc_or_code.kv_dtype if isinstance(desc_or_code, BatchDesc) else int(desc_or_code)
    p = _ptr(t, name)
    if p is not None and dtype_code(t) != code:
        raise ValueError(f"{name} holds {t.dtype}, which does not match kv_dtype {code}")
    return p


def _ptr(t, name: str, dtype=None):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_desc(*, num_heads: int, num_kv_heads: int, head_dim: int, num_blocks: int, block_table_stride: int,
              dtype: int, softmax_scale: float, context_lens_host, cu_q_lens_host, block_size: int = 16,
              flags: int = 0, kv_dtype: Optional[int] = None, k_scale: float = 1.0,
              v_scale: float = 1.0, q_pos_host=None) -> BatchDesc:
    ctx = np.ascontiguousarray(context_lens_host, dtype=np.int32)
    cu = np.ascontiguousarray(cu_q_lens_host, dtype=np.int32)
    d = BatchDesc(len(ctx), num_heads, num_kv_heads, head_dim, block_size, num_blocks, block_table_stride, dtype,
                  float(softmax_scale), flags,
                  ctx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                  cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    d.kv_dtype = dtype if kv_dtype is None else int(kv_dtype)
    d.k_scale = float(k_scale)
    d.v_scale = float(v_scale)
    qp = None
    if q_pos_host is not None:
        qp = np.ascontiguousarray(q_pos_host, dtype=np.int32)
        if qp.shape != (int(cu[-1]) if len(cu) else 0,):
            raise ValueError("q_pos_host must hold one position per query row")
        d.q_pos_host = qp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    d._keep = (ctx, cu, qp)  # host arrays must outlive the descriptor
    return d


def _shape(t, name: str, shape):
    """Raise ValueError unless tensor t has exactly this shape (None entries match anything)."""
    if t is None:
        return
    got = tuple(t.shape)
    if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
        raise ValueError(f"{name} has shape {got}, expected {tuple('*' if w is None else w for w in shape)}")


def _pool_shapes(k_pool, v_pool, num_blocks=None, hkv=None, d=None):
    """K and V pools [NB][Hkv][16][d]; returns (NB, Hkv, d)."""
    if k_pool.dim() != 4 or k_pool.shape[2] != 16:
        raise ValueError(f"k_pool has shape {tuple(k_pool.shape)}, expected [num_blocks][Hkv][16][head_dim]")
    nb, hk, _, dd = k_pool.shape
    _shape(k_pool, "k_pool", (num_blocks, hkv, 16, d))
    _shape(v_pool, "v_pool", (nb, hk, 16, dd))
    return int(nb), int(hk), int(dd)


def _check_batch(desc: BatchDesc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos, o=None):
    """Tensor shapes against the descriptor, before any pointer reaches the library."""
    ctx, cu, _ = desc._keep
    R = int(desc.num_reqs)
    T = int(cu[-1]) if R > 0 else 0
    _shape(q, "q", (T, desc.num_heads, desc.head_dim))
    _shape(o, "o", (T, desc.num_heads, desc.head_dim))
    if o is not None and q is not None and o.dtype != q.dtype:
        raise ValueError(f"o holds {o.dtype}, q holds {q.dtype}")
    _pool_shapes(k_pool, v_pool, desc.num_blocks, desc.num_kv_heads, desc.head_dim)
    _shape(block_tables, "block_tables", (R, desc.block_table_stride))
    _shape(context_lens, "context_lens", (R,))
    _shape(cu_q_lens, "cu_q_lens", (R + 1,))
    _shape(q_pos, "q_pos", (T,))


def _check_append(k_new, v_new, k_pool, v_pool, slot_mapping):
    if k_new.dim() != 3:
        raise ValueError(f"k_new has shape {tuple(k_new.shape)}, expected [num_tokens][Hkv][head_dim]")
    n, hkv, d = k_new.shape
    _shape(v_new, "v_new", (n, hkv, d))
    _pool_shapes(k_pool, v_pool, None, hkv, d)
    _shape(slot_mapping, "slot_mapping", (n,))


# ---- entry points --------------------------------------------------------------------
def pensieve_version() -> str:
    return load_library().pensieve_version().decode()


def pensieve_kv_append(k_new, v_new, k_pool, v_pool, slot_mapping, stream=None):
    torch = _torch()
    lib = load_library()
    _check_append(k_new, v_new, k_pool, v_pool, slot_mapping)
    n, hkv, d = k_new.shape
    nb = k_pool.shape[0]
    _check(lib.pensieve_kv_append(_ptr(k_new, "k_new"), _ptr(v_new, "v_new", k_new.dtype),
                                  _ptr(k_pool, "k_pool", k_new.dtype), _ptr(v_pool, "v_pool", k_new.dtype),
                                  _ptr(slot_mapping, "slot_mapping", torch.int32), n, hkv, d, k_pool.shape[2], nb,
                                  dtype_code(k_new), _stream(stream)))


def pensieve_kv_append_fp8(k_new, v_new, k_pool, v_pool, slot_mapping, k_scale: float, v_scale: float,
                           stream=None):
    """Append f16 / bf16 rows into E4M3 pools (uint8 or float8_e4m3fn tensors): code = E4M3(x / scale)."""
    torch = _torch()
    lib = load_library()
    _check_append(k_new, v_new, k_pool, v_pool, slot_mapping)
    n, hkv, d = k_new.shape
    nb = k_pool.shape[0]
    _check(lib.pensieve_kv_append_fp8(_ptr(k_new, "k_new"), _ptr(v_new, "v_new", k_new.dtype),
                                      _pool_ptr(k_pool, "k_pool", PENSIEVE_FP8_E4M3),
                                      _pool_ptr(v_pool, "v_pool", PENSIEVE_FP8_E4M3),
                                      _ptr(slot_mapping, "slot_mapping", torch.int32), n, hkv, d, k_pool.shape[2], nb,
                                      dtype_code(k_new), float(k_scale), float(v_scale), _stream(stream)))


def _host_ptr(t, name: str, dtype):
    """A host tensor; the library itself checks that it is page-locked and mapped for the device."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.is_cuda:
        raise ValueError(f"{name} must be a pinned host tensor")
    if not t.is_contiguous() or t.dtype != dtype:
        raise ValueError(f"{name} must be contiguous {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _block_list(blocks):
    arr = np.ascontiguousarray(np.asarray(blocks, dtype=np.int32).reshape(-1))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _kv_swap(fn, k_pool, v_pool, k_host, v_host, first, second, stream):
    k_arr, k_p = _block_list(first)
    s_arr, s_p = _block_list(second)
    if len(k_arr) != len(s_arr):
        raise ValueError("block lists differ in length")
    _, hkv, d = _pool_shapes(k_pool, v_pool)
    _shape(k_host, "k_host", (None,) + tuple(k_pool.shape[1:]))
    _shape(v_host, "v_host", (k_host.shape[0],) + tuple(v_pool.shape[1:]))
    _check(fn(_ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool", k_pool.dtype), k_pool.shape[0],
              _host_ptr(k_host, "k_host", k_pool.dtype), _host_ptr(v_host, "v_host", k_pool.dtype), k_host.shape[0],
              k_p, s_p, len(k_arr), hkv, d, dtype_code(k_pool), _stream(stream)))


def pensieve_kv_swap_out(k_pool, v_pool, k_host, v_host, device_blocks, host_blocks, stream=None):
    """Copy device blocks device_blocks[i] of the pools to host blocks host_blocks[i] of the pinned host tier."""
    _kv_swap(load_library().pensieve_kv_swap_out, k_pool, v_pool, k_host, v_host, device_blocks, host_blocks, stream)


def pensieve_kv_swap_in(k_pool, v_pool, k_host, v_host, host_blocks, device_blocks, stream=None):
    """Copy host blocks host_blocks[i] of the pinned host tier to device blocks device_blocks[i] of the pools."""
    _kv_swap(load_library().pensieve_kv_swap_in, k_pool, v_pool, k_host, v_host, host_blocks, device_blocks, stream)


def pensieve_attn_workspace_size(desc: BatchDesc, num_partitions: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().pensieve_attn_workspace_size(ctypes.byref(desc), num_partitions, ctypes.byref(out)))
    return int(out.value)


def pensieve_attn_fwd(desc: BatchDesc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos, o,
                      workspace, stream=None):
    torch = _torch()
    _check_batch(desc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos, o)
    _check(load_library().pensieve_attn_fwd(
        ctypes.byref(desc), _ptr(q, "q"), _pool_ptr(k_pool, "k_pool", desc), _pool_ptr(v_pool, "v_pool", desc),
        _ptr(block_tables, "block_tables", torch.int32), _ptr(context_lens, "context_lens", torch.int32),
        _ptr(cu_q_lens, "cu_q_lens", torch.int32), _ptr(q_pos, "q_pos", torch.int32), _ptr(o, "o", q.dtype),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))


def pensieve_attn_fwd_noalloc(desc: BatchDesc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos, o,
                              stream=None):
    """pensieve_attn_fwd with the library's own device scratch instead of a workspace (allocates nothing)."""
    torch = _torch()
    _check_batch(desc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos, o)
    _check(load_library().pensieve_attn_fwd_noalloc(
        ctypes.byref(desc), _ptr(q, "q"), _pool_ptr(k_pool, "k_pool", desc), _pool_ptr(v_pool, "v_pool", desc),
        _ptr(block_tables, "block_tables", torch.int32), _ptr(context_lens, "context_lens", torch.int32),
        _ptr(cu_q_lens, "cu_q_lens", torch.int32), _ptr(q_pos, "q_pos", torch.int32), _ptr(o, "o", q.dtype),
        _stream(stream)))


def pensieve_attn_split_partial(desc: BatchDesc, num_partitions: int, q, k_pool, v_pool, block_tables,
                                context_lens, cu_q_lens, q_pos, part_o, part_m, part_l, workspace, stream=None):
    torch = _torch()
    _check_batch(desc, q, k_pool, v_pool, block_tables, context_lens, cu_q_lens, q_pos)
    T, P = int(q.shape[0]), int(num_partitions)
    _shape(part_o, "part_o", (T, desc.num_heads, P, desc.head_dim))
    _shape(part_m, "part_m", (T, desc.num_heads, P))
    _shape(part_l, "part_l", (T, desc.num_heads, P))
    _check(load_library().pensieve_attn_split_partial(
        ctypes.byref(desc), num_partitions, _ptr(q, "q"), _pool_ptr(k_pool, "k_pool", desc),
        _pool_ptr(v_pool, "v_pool", desc), _ptr(block_tables, "block_tables", torch.int32),
        _ptr(context_lens, "context_lens", torch.int32), _ptr(cu_q_lens, "cu_q_lens", torch.int32),
        _ptr(q_pos, "q_pos", torch.int32), _ptr(part_o, "part_o", torch.float32),
        _ptr(part_m, "part_m", torch.float32), _ptr(part_l, "part_l", torch.float32),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))


def pensieve_attn_split_merge(part_o, part_m, part_l, o, stream=None):
    torch = _torch()
    t, hq, p, d = part_o.shape
    _shape(part_m, "part_m", (t, hq, p))
    _shape(part_l, "part_l", (t, hq, p))
    _shape(o, "o", (t, hq, d))
    _check(load_library().pensieve_attn_split_merge(
        _ptr(part_o, "part_o", torch.float32), _ptr(part_m, "part_m", torch.float32),
        _ptr(part_l, "part_l", torch.float32), t, hq, d, p, dtype_code(o), _ptr(o, "o"), _stream(stream)))


def pensieve_debug_plan(desc: BatchDesc, num_partitions: int = 0) -> np.ndarray:
    """Work list the library would launch: int32 [n][10] (see pensieve.h)."""
    lib = load_library()
    n = ctypes.c_int32(0)
    _check(lib.pensieve_debug_plan(ctypes.byref(desc), num_partitions, None, 0, ctypes.byref(n)))
    out = np.zeros((max(n.value, 1), 10), dtype=np.int32)
    _check(lib.pensieve_debug_plan(ctypes.byref(desc), num_partitions,
                                   out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value, ctypes.byref(n)))
    return out[:n.value]


def pensieve_trace_enable(enable=True, every: int = 1) -> None:
    """Turn launch timing on (every `every`-th launch of each kernel kind) or off."""
    _check(load_library().pensieve_trace_enable(max(1, int(every)) if enable else 0))


def pensieve_trace_read(max_records: int = 1 << 16):
    """Per-launch records [(kernel name, work items, ms)] since the last read."""
    buf = (TraceRecord * max_records)()
    n = ctypes.c_int32(0)
    _check(load_library().pensieve_trace_read(buf, max_records, ctypes.byref(n)))
    return [(TRACE_KERNELS.get(buf[i].kernel, str(buf[i].kernel)), int(buf[i].items), float(buf[i].ms))
            for i in range(n.value)]


# ---- host cache planning -----------------------------------------------------
def conversations(cached_tokens, dropped_blocks, new_tokens, activity) -> np.ndarray:
    """Array of pensieve_conversation records from per-conversation sequences."""
    n = len(cached_tokens)
    out = np.zeros(n, dtype=CONVERSATION_DTYPE)
    out["cached_tokens"] = cached_tokens
    out["dropped_blocks"] = dropped_blocks
    out["new_tokens"] = new_tokens
    out["activity"] = activity
    return out


def _conv_arg(convs):
    if not isinstance(convs, np.ndarray) or convs.dtype != CONVERSATION_DTYPE or not convs.flags.c_contiguous:
        raise TypeError("conversations must be a contiguous array of CONVERSATION_DTYPE records")
    return ctypes.c_void_p(convs.ctypes.data if len(convs) else 0), len(convs)


def _i32_out(n: int) -> np.ndarray:
    return np.zeros(max(int(n), 0), dtype=np.int32)


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def pensieve_cache_plan_evictions(convs: np.ndarray, free_blocks: int):
    """Leading blocks each conversation drops so the step fits: (evict[n] int32, total)."""
    ptr, n = _conv_arg(convs)
    evict = _i32_out(n)
    freed = ctypes.c_int32(0)
    _check(load_library().pensieve_cache_plan_evictions(ptr, n, int(free_blocks), _i32p(evict),
                                                        ctypes.byref(freed)))
    return evict, int(freed.value)


def pensieve_cache_build_batch(convs: np.ndarray, block_tables: np.ndarray, free_list) -> dict:
    """Unified batch of the scheduled conversations; updates block_tables [n][stride] in place.

    Returns a dict of int32 arrays: request_conv, cu_q_lens, context_lens, q_pos,
    slot_mapping, req_block_tables, and the int blocks_used.
    """
    ptr, n = _conv_arg(convs)
    if (not isinstance(block_tables, np.ndarray) or block_tables.dtype != np.int32 or block_tables.ndim != 2
            or not block_tables.flags.c_contiguous or not block_tables.flags.writeable
            or block_tables.shape[0] != n):
        raise TypeError("block_tables must be a writeable C-contiguous int32 array [n][stride]")
    stride = int(block_tables.shape[1])
    free = np.ascontiguousarray(free_list, dtype=np.int32)
    lib = load_library()
    reqs, rows, used = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    none = ctypes.POINTER(ctypes.c_int32)()
    _check(lib.pensieve_cache_build_batch(ptr, n, _i32p(block_tables), stride, _i32p(free), len(free), -1,
                                          ctypes.byref(reqs), ctypes.byref(rows), ctypes.byref(used),
                                          none, none, none, none, none, none))
    R, T = int(reqs.value), int(rows.value)
    out = {"request_conv": _i32_out(R), "cu_q_lens": _i32_out(R + 1), "context_lens": _i32_out(R),
           "q_pos": _i32_out(T), "slot_mapping": _i32_out(T),
           "req_block_tables": np.zeros((R, stride), dtype=np.int32)}
    _check(lib.pensieve_cache_build_batch(ptr, n, _i32p(block_tables), stride, _i32p(free), len(free), T,
                                          ctypes.byref(reqs), ctypes.byref(rows), ctypes.byref(used),
                                          _i32p(out["request_conv"]), _i32p(out["cu_q_lens"]),
                                          _i32p(out["context_lens"]), _i32p(out["q_pos"]),
                                          _i32p(out["slot_mapping"]), _i32p(out["req_block_tables"])))
    out["blocks_used"] = int(used.value)
    return out
