"""Thin ctypes binding of ``libpa.so`` (the C ABI in ``include/pa.h``).

Same names as the C entry points.  Every function only marshals arguments:
device tensors become pointers, the stream defaults to PyTorch's current
stream, and a non-OK status raises :class:`PAError`.  All compute runs in the
HIP kernels; there is no fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
_lib = None

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_MISALIGNED = -3
PA_ERR_WORKSPACE = -4
PA_ERR_HIP = -5
PA_ERR_NO_SPACE = -6

PA_F32, PA_F16, PA_BF16, PA_K8_F16, PA_K8_BF16 = 0, 1, 2, 3, 4
TORCH_TO_PA = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
NAME_TO_PA = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16}
BLOCK_SIZE = 16

# every symbol include/pa.h declares
EXPORTS = ("pa_init_pool", "pa_write_kv", "pa_decode_workspace_bytes", "pa_decode",
           "pa_verify_decode", "pa_write_kv_k8", "pa_decode_k8", "pa_reduce", "pa_debug_slot_ids", "pa_copy_blocks", "pa_gather_blocks",
           "pa_scatter_blocks", "pa_status_string")


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {pa_status_string(status)} ({status})")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libpa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m paged_kv_cache_365_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64p, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    desc = ctypes.POINTER(PoolDesc)
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_init_pool.restype = ctypes.c_int
    lib.pa_init_pool.argtypes = [desc, vp, vp, i32, vp]
    lib.pa_write_kv.restype = ctypes.c_int
    lib.pa_write_kv.argtypes = [desc, vp, vp, vp, vp, i64p, i32, vp]
    lib.pa_decode_workspace_bytes.restype = sz
    lib.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode.argtypes = [desc, vp, vp, vp, vp, i32, vp, i32, i32, i32, ctypes.c_float, i32,
                              vp, sz, vp, vp]
    lib.pa_verify_decode.restype = ctypes.c_int
    lib.pa_verify_decode.argtypes = [desc, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                     ctypes.c_float, i32, vp, sz, vp, vp]
    lib.pa_write_kv_k8.restype = ctypes.c_int
    lib.pa_write_kv_k8.argtypes = [desc, vp, vp, vp, vp, vp, i64p, i32, vp]
    lib.pa_decode_k8.restype = ctypes.c_int
    lib.pa_decode_k8.argtypes = [desc, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32,
                                 ctypes.c_float, i32, vp, sz, vp, vp]
    lib.pa_reduce.restype = ctypes.c_int
    lib.pa_reduce.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.pa_debug_slot_ids.restype = ctypes.c_int
    lib.pa_debug_slot_ids.argtypes = [vp, i32, vp, i32, i32, i32, i32, vp, vp]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [desc, vp, vp, vp, i32, vp]
    lib.pa_gather_blocks.restype = ctypes.c_int
    lib.pa_gather_blocks.argtypes = [desc, vp, vp, vp, i32, vp, vp, vp]
    lib.pa_scatter_blocks.restype = ctypes.c_int
    lib.pa_scatter_blocks.argtypes = [desc, vp, vp, vp, i32, vp, vp, vp]
    if path is None:
        _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PAError(fn, status)


def pool_desc(k_pool: torch.Tensor, v_pool: torch.Tensor | None = None) -> PoolDesc:
    """Descriptor of a K pool tensor shaped [num_blocks][H_kv][d / x][16][x].  An
    int8 K pool (quantised keys) takes its value type from ``v_pool``."""
    nb, hkv, nchunk, bs, x = k_pool.shape
    if k_pool.dtype == torch.int8:
        vt = None if v_pool is None else v_pool.dtype
        dt = {torch.float16: PA_K8_F16, torch.bfloat16: PA_K8_BF16}.get(vt, -1)
    else:
        dt = TORCH_TO_PA.get(k_pool.dtype, -1)
    return PoolDesc(nb, bs, hkv, nchunk * x, dt)


def pa_status_string(status: int) -> str:
    return load().pa_status_string(status).decode()


def pa_init_pool(k_pool, v_pool, fill: int = 0, stream=None) -> None:
    desc = pool_desc(k_pool, v_pool)
    _check("pa_init_pool", load().pa_init_pool(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool),
                                               fill, _stream(stream)))


def pa_write_kv(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None) -> None:
    desc = pool_desc(k_pool, v_pool)
    n = int(slot_mapping.shape[0])
    _check("pa_write_kv", load().pa_write_kv(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool),
                                             _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), n,
                                             _stream(stream)))


def pa_decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int,
                              max_context_len: int, partition_size: int) -> int:
    return int(load().pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                                partition_size))


def pa_decode(q, k_pool, v_pool, block_tables, context_lens, max_context_len: int, scale: float,
              partition_size: int = 0, workspace=None, out=None, stream=None) -> None:
    desc = pool_desc(k_pool, v_pool)
    B, Hq, _ = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode", load().pa_decode(
        ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), B, Hq, int(max_context_len),
        float(scale), int(partition_size), _ptr(workspace), ws_bytes, _ptr(out), _stream(stream)))


def pa_verify_decode(q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                     scale: float, partition_size: int = 0, workspace=None, out=None,
                     stream=None) -> None:
    """q and out: [B][T][H_q][d] (T draft tokens per sequence)."""
    desc = pool_desc(k_pool, v_pool)
    B, T, Hq, _ = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_verify_decode", load().pa_verify_decode(
        ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), B, T, Hq, int(max_context_len),
        float(scale), int(partition_size), _ptr(workspace), ws_bytes, _ptr(out), _stream(stream)))


def pa_write_kv_k8(k_pool, v_pool, k_scale, k_new, v_new, slot_mapping, stream=None) -> None:
    """int8 key pool: k_new / v_new [T][H_kv][d] in the value type, k_scale float32 [H_kv][d]."""
    desc = pool_desc(k_pool, v_pool)
    n = int(slot_mapping.shape[0])
    _check("pa_write_kv_k8", load().pa_write_kv_k8(
        ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(k_new), _ptr(v_new),
        _ptr(slot_mapping), n, _stream(stream)))


def pa_decode_k8(q, k_pool, v_pool, k_scale, block_tables, context_lens, max_context_len: int,
                 scale: float, partition_size: int = 0, workspace=None, out=None,
                 stream=None) -> None:
    """q and out: [B][T][H_q][d] in the value type (T = 1: decode)."""
    desc = pool_desc(k_pool, v_pool)
    B, T, Hq, _ = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_k8", load().pa_decode_k8(
        ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), B, T, Hq, int(max_context_len),
        float(scale), int(partition_size), _ptr(workspace), ws_bytes, _ptr(out), _stream(stream)))


def pa_reduce(workspace, context_lens, num_seqs: int, num_q_heads: int, head_dim: int,
              max_context_len: int, partition_size: int, out, stream=None) -> None:
    _check("pa_reduce", load().pa_reduce(
        _ptr(workspace), _ptr(context_lens), num_seqs, num_q_heads, head_dim,
        int(max_context_len), int(partition_size), TORCH_TO_PA.get(out.dtype, -1), _ptr(out),
        _stream(stream)))


def pa_debug_slot_ids(block_tables, context_lens, max_context_len: int, num_blocks: int,
                      slot_ids, stream=None, block_size: int = BLOCK_SIZE) -> None:
    B = int(context_lens.shape[0])
    _check("pa_debug_slot_ids", load().pa_debug_slot_ids(
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), B,
        int(max_context_len), int(num_blocks), int(block_size), _ptr(slot_ids), _stream(stream)))


def pa_copy_blocks(k_pool, v_pool, src_dst, stream=None) -> None:
    """src_dst: int32 device tensor [n][2] of (source, destination) blocks."""
    desc = pool_desc(k_pool, v_pool)
    n = int(src_dst.shape[0]) if src_dst is not None else 0
    _check("pa_copy_blocks", load().pa_copy_blocks(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool),
                                                   _ptr(src_dst), n, _stream(stream)))


def pa_gather_blocks(k_pool, v_pool, block_ids, k_dst, v_dst, stream=None) -> None:
    desc = pool_desc(k_pool, v_pool)
    _check("pa_gather_blocks", load().pa_gather_blocks(
        ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool), _ptr(block_ids), int(block_ids.shape[0]),
        _ptr(k_dst), _ptr(v_dst), _stream(stream)))


def pa_scatter_blocks(k_pool, v_pool, block_ids, k_src, v_src, stream=None) -> None:
    desc = pool_desc(k_pool, v_pool)
    _check("pa_scatter_blocks", load().pa_scatter_blocks(
        ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool), _ptr(block_ids), int(block_ids.shape[0]),
        _ptr(k_src), _ptr(v_src), _stream(stream)))


# ---------------------------------------------------------------------------
# convenience: one decode step (decode, then reduce when split)
# ---------------------------------------------------------------------------
def workspace_for(q, k_pool, max_context_len: int, partition_size: int):
    """A float32 workspace tensor for pa_decode's partials (None when unsplit)."""
    if partition_size <= 0:
        return None
    n = pa_decode_workspace_bytes(q.shape[0], q.shape[1], q.shape[2], max_context_len,
                                  partition_size)
    return torch.empty(n // 4, dtype=torch.float32, device=q.device)


def paged_attention(q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                    scale: float, partition_size: int = 0, workspace=None, out=None, stream=None):
    """out = pa_decode (+ pa_reduce when partition_size > 0).  Returns out."""
    if out is None:
        out = torch.empty_like(q)
    if partition_size > 0:
        if workspace is None:
            workspace = workspace_for(q, k_pool, max_context_len, partition_size)
        pa_decode(q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale,
                  partition_size, workspace, None, stream)
        pa_reduce(workspace, context_lens, q.shape[0], q.shape[1], q.shape[2], max_context_len,
                  partition_size, out, stream)
    else:
        pa_decode(q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale, 0, None,
                  out, stream)
    return out


def verify_attention(q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                     scale: float, partition_size: int = 0, workspace=None, out=None, stream=None):
    """out = pa_verify_decode (+ pa_reduce over T * H_q rows when split).  q is
    [B][T][H_q][d]; returns out of the same shape."""
    if out is None:
        out = torch.empty_like(q)
    B, T, Hq, D = q.shape
    if partition_size > 0:
        if workspace is None:
            n = pa_decode_workspace_bytes(B, T * Hq, D, max_context_len, partition_size)
            workspace = torch.empty(n // 4, dtype=torch.float32, device=q.device)
        pa_verify_decode(q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale,
                         partition_size, workspace, None, stream)
        pa_reduce(workspace, context_lens, B, T * Hq, D, max_context_len, partition_size, out,
                  stream)
    else:
        pa_verify_decode(q, k_pool, v_pool, block_tables, context_lens, max_context_len, scale, 0,
                         None, out, stream)
    return out


def k8_attention(q, k_pool, v_pool, k_scale, block_tables, context_lens, max_context_len: int,
                 scale: float, partition_size: int = 0, workspace=None, out=None, stream=None):
    """out = pa_decode_k8 (+ pa_reduce over T * H_q rows when split).  q is
    [B][T][H_q][d]; returns out of the same shape."""
    if out is None:
        out = torch.empty_like(q)
    B, T, Hq, D = q.shape
    if partition_size > 0:
        if workspace is None:
            n = pa_decode_workspace_bytes(B, T * Hq, D, max_context_len, partition_size)
            workspace = torch.empty(n // 4, dtype=torch.float32, device=q.device)
        pa_decode_k8(q, k_pool, v_pool, k_scale, block_tables, context_lens, max_context_len, scale,
                     partition_size, workspace, None, stream)
        pa_reduce(workspace, context_lens, B, T * Hq, D, max_context_len, partition_size, out,
                  stream)
    else:
        pa_decode_k8(q, k_pool, v_pool, k_scale, block_tables, context_lens, max_context_len, scale,
                     0, None, out, stream)
    return out
