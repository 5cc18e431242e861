"""Paged KV-cache decode attention for AMD MI355X (gfx950).

A thin ctypes binding over ``libpa.so`` (the C ABI in ``include/pa.h``): the
functions below only turn torch tensors into pointers and sizes; every step
of the computation runs in libpa's HIP kernels.  PyTorch supplies device
memory and streams.  If ``libpa.so`` has not been built this module raises
ImportError -- there is no fallback implementation.

Pool layout (BS = block_size, D = head_dim, X = 16 / element size,
VS = min(BS, 8)):
    k_cache: [num_blocks, Hkv, D // X, BS, X]
    v_cache: [num_blocks, Hkv, BS // VS, D, VS]
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_F32, PA_F16, PA_BF16 = 0, 1, 2
_DTYPE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m paged_kv_cache_118_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    sig = {
        "pa_strerror": (ctypes.c_char_p, [i32]),
        "pa_decode": (i32, [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i64,
                            i32, i32, vp, sz, vp]),
        "pa_decode_write": (i32, [vp, vp, vp, vp, i64, vp, vp, vp, vp, f32, i32, i32, i32, i32,
                                  i32, i32, i32, i64, i32, i32, vp, sz, vp]),
        "pa_decode_noalloc": (i32, [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32,
                                    i32, i64, i32, i32, vp]),
        "pa_decode_noalloc_scratch_bytes": (sz, []),
        "pa_decode_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32, i32, i32]),
        "pa_decode_partition_size": (i32, [i32, i32, i32, i32, i32, i32, i32, i32]),
        "pa_prefill": (i32, [vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32,
                             i32, i64, i32, vp]),
        "pa_reshape_and_cache": (i32, [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i64,
                                       i32, vp]),
        "pa_copy_blocks": (i32, [vp, vp, vp, i32, i32, i32, i32, i64, i32, vp]),
        "pa_swap_blocks": (i32, [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, vp]),
        "pa_alloc_create": (vp, [i64, i32, ctypes.c_uint64]),
        "pa_alloc_destroy": (None, [vp]),
        "pa_alloc_add_seq": (i32, [vp, i64, i32]),
        "pa_alloc_fork": (i32, [vp, i64, i64]),
        "pa_alloc_append": (i32, [vp, i64, i32, vp, vp, vp]),
        "pa_alloc_append_batch": (i32, [vp, vp, vp, i32, vp, vp, vp, vp]),
        "pa_alloc_free_seq": (i32, [vp, i64]),
        "pa_alloc_discard_seq": (i32, [vp, i64]),
        "pa_alloc_share_groups": (i32, [vp, vp, i32, i32, vp, vp, vp]),
        "pa_decode_shared": (i32, [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32,
                                   i32, i64, i32, vp, vp, i32, vp, sz, vp]),
        "pa_decode_shared_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32, i32, i32]),
        "pa_bench_stream_read": (i32, [vp, sz, vp, i32, vp]),
        "pa_alloc_block_tables": (i32, [vp, vp, i32, i32, vp, vp]),
        "pa_alloc_num_free": (i64, [vp]),
        "pa_alloc_refcount": (i32, [vp, i64]),
        "pa_alloc_seq_len": (i32, [vp, i64]),
        "pa_alloc_seq_num_blocks": (i32, [vp, i64]),
        "pa_alloc_add_seq_tokens": (i32, [vp, i64, vp, i32, ctypes.c_uint64, vp]),
        "pa_alloc_append_tokens": (i32, [vp, i64, vp, i32, vp, vp, vp]),
        "pa_alloc_num_cached": (i64, [vp]),
        "pa_alloc_num_evictable": (i64, [vp]),
        "pa_alloc_reset_prefix_cache": (i32, [vp]),
        "pa_prefix_block_hash": (i32, [vp, ctypes.c_uint64, vp, i32, vp]),
    }
    # PA_ALLOC_LIB: the host allocator from another build of alloc.cpp (the
    # sanitizer build of build.py), for CPU test runs; everything else stays
    alloc_lib = ctypes.CDLL(os.environ["PA_ALLOC_LIB"]) if os.environ.get("PA_ALLOC_LIB") else lib
    for name, (res, args) in sig.items():
        src = alloc_lib if name.startswith(("pa_alloc_", "pa_prefix_block_hash")) else lib
        fn = getattr(src, name)
        fn.restype = res
        fn.argtypes = args
        if src is not lib:
            setattr(lib, name, fn)
    return lib


_lib = _load()

# every symbol include/pa.h declares (checked by the CPU test suite)
EXPORTED = ("pa_strerror", "pa_decode", "pa_decode_write", "pa_decode_noalloc",
            "pa_decode_noalloc_scratch_bytes", "pa_decode_workspace_bytes",
            "pa_decode_partition_size",
            "pa_prefill", "pa_swap_blocks",
            "pa_reshape_and_cache", "pa_copy_blocks", "pa_alloc_create", "pa_alloc_destroy",
            "pa_alloc_add_seq", "pa_alloc_fork", "pa_alloc_append", "pa_alloc_append_batch",
            "pa_alloc_free_seq", "pa_alloc_discard_seq", "pa_alloc_share_groups",
            "pa_decode_shared", "pa_decode_shared_workspace_bytes", "pa_bench_stream_read",
            "pa_alloc_block_tables", "pa_alloc_num_free", "pa_alloc_refcount",
            "pa_alloc_seq_len", "pa_alloc_seq_num_blocks", "pa_alloc_add_seq_tokens",
            "pa_alloc_append_tokens", "pa_alloc_num_cached", "pa_alloc_num_evictable",
            "pa_alloc_reset_prefix_cache", "pa_prefix_block_hash")


def lib():
    return _lib


class PAError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"libpa status {status}: {pa_strerror(status)}")


class OutOfBlocks(PAError):
    pass


def pa_strerror(status: int) -> str:
    return _lib.pa_strerror(status).decode()


def _check(rc: int) -> None:
    if rc == -3:
        raise OutOfBlocks(rc)
    if rc != 0:
        raise PAError(rc)


def _dev_ptr(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, device=None) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        if device is not None and stream.device != device:
            raise ValueError(f"stream is on {stream.device}, the tensors on {device}")
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _on_device(device, **tensors) -> None:
    """Every given tensor lives on ``device``: libpa's kernels run there (the
    call makes it current) and dereference these pointers there."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the call's tensors on {device}")


def _scratch(nbytes: int, device, stream) -> torch.Tensor:
    """A uint8 device buffer for one call's kernels on ``stream``: when that
    is not the current stream, the caching allocator is told the buffer is in
    use there until that stream's work is done."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None:
        ts = stream if isinstance(stream, torch.cuda.Stream) else \
            torch.cuda.ExternalStream(int(stream), device=device)
        if ts != torch.cuda.current_stream(device):
            buf.record_stream(ts)
    return buf


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def v_slab(block_size: int) -> int:
    return block_size if block_size < 8 else 8


def k_pool_shape(num_blocks, num_kv_heads, block_size, head_dim, dtype):
    """K pool shape [blocks][Hkv][D/X][BS][X], X = 16 / element size (pa.h)."""
    x = 16 // torch.empty((), dtype=dtype).element_size()
    return (num_blocks, num_kv_heads, head_dim // x, block_size, x)


def v_pool_shape(num_blocks, num_kv_heads, block_size, head_dim):
    """V pool shape [blocks][Hkv][BS/VS][D][VS], VS = min(BS, 8) (pa.h)."""
    vs = v_slab(block_size)
    return (num_blocks, num_kv_heads, block_size // vs, head_dim, vs)


def _check_pools(k_cache, v_cache, num_kv_heads, block_size, head_dim):
    nb = k_cache.shape[0]
    want_k = k_pool_shape(nb, num_kv_heads, block_size, head_dim, k_cache.dtype)
    want_v = v_pool_shape(nb, num_kv_heads, block_size, head_dim)
    if tuple(k_cache.shape) != want_k:
        raise ValueError(f"k_cache shape {tuple(k_cache.shape)} is not {want_k}")
    if tuple(v_cache.shape) != want_v:
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} is not {want_v}")
    if k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must have one dtype")
    return nb


# ---------------------------------------------------------------- decode --
def pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                              max_context_len, partition_size=0, dtype=torch.float16) -> int:
    return int(_lib.pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              block_size, max_context_len, partition_size,
                                              _DTYPE[dtype]))


def pa_decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_context_len, partition_size=0, dtype=torch.float16) -> int:
    return int(_lib.pa_decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             block_size, max_context_len, partition_size,
                                             _DTYPE[dtype]))


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
              num_kv_heads, max_context_len, partition_size=0, workspace=None, stream=None):
    """out[b, h] = softmax over the first context_lens[b] positions (see pa.h).

    ``max_context_len`` is a host int >= every context length.  ``workspace``
    is a uint8 device tensor of pa_decode_workspace_bytes(...) bytes (no
    initialisation needed, reusable across calls); one is allocated when
    omitted and needed."""
    B, hq, D = q.shape
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("pools must have q's dtype")
    nb = _check_pools(k_cache, v_cache, num_kv_heads, block_size, D)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    dt = _dtype_code(q)
    dev = q.device
    _on_device(dev, q=q, out=out, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
               context_lens=context_lens, workspace=workspace)
    ws_bytes = int(_lib.pa_decode_workspace_bytes(B, hq, num_kv_heads, D, block_size,
                                                  max_context_len, partition_size, dt))
    if ws_bytes and workspace is None:
        workspace = _scratch(ws_bytes, dev, stream)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(dev):
        _check(_lib.pa_decode(_dev_ptr(out, "out"), _dev_ptr(q, "q"),
                              _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                              _dev_ptr(block_tables, "block_tables"),
                              _dev_ptr(context_lens, "context_lens"), float(scale), block_size,
                              num_kv_heads, B, hq, D, block_tables.shape[1],
                              int(max_context_len), nb, dt, int(partition_size), ws_ptr, ws_len,
                              _stream(stream, dev)))
    return out


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                      num_kv_heads, max_context_len, partition_size=0, stream=None):
    """pa_decode with the split's scratch in libpa's static per-device array
    (nothing allocated; see pa.h).  Raises PAError with status -7 when the
    call would need more than pa_decode_noalloc_scratch_bytes()."""
    B, hq, D = q.shape
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("pools must have q's dtype")
    nb = _check_pools(k_cache, v_cache, num_kv_heads, block_size, D)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    dev = q.device
    _on_device(dev, q=q, out=out, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
               context_lens=context_lens)
    with torch.cuda.device(dev):
        _check(_lib.pa_decode_noalloc(_dev_ptr(out, "out"), _dev_ptr(q, "q"),
                                      _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                                      _dev_ptr(block_tables, "block_tables"),
                                      _dev_ptr(context_lens, "context_lens"), float(scale),
                                      block_size, num_kv_heads, B, hq, D, block_tables.shape[1],
                                      int(max_context_len), nb, _dtype_code(q),
                                      int(partition_size), _stream(stream, dev)))
    return out


def pa_decode_noalloc_scratch_bytes() -> int:
    return int(_lib.pa_decode_noalloc_scratch_bytes())


def pa_decode_shared_workspace_bytes(num_seqs, num_groups, num_q_heads, num_kv_heads, head_dim,
                                     block_size, max_context_len, dtype=torch.float16) -> int:
    return int(_lib.pa_decode_shared_workspace_bytes(num_seqs, num_groups, num_q_heads,
                                                     num_kv_heads, head_dim, block_size,
                                                     max_context_len, _DTYPE[dtype]))


def pa_decode_shared(out, q, k_cache, v_cache, block_tables, context_lens, group_start,
                     group_prefix_len, scale, block_size, num_kv_heads, max_context_len,
                     workspace=None, stream=None):
    """pa_decode for groups of consecutive sequences sharing their leading
    blocks (see pa.h): group_start int32 [G+1], group_prefix_len int32 [G]
    (device tensors, e.g. from BlockAllocator.share_groups)."""
    B, hq, D = q.shape
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("pools must have q's dtype")
    nb = _check_pools(k_cache, v_cache, num_kv_heads, block_size, D)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    G = group_prefix_len.shape[0]
    if group_start.dtype != torch.int32 or group_prefix_len.dtype != torch.int32 or \
            tuple(group_start.shape) != (G + 1,):
        raise ValueError("group_start must be int32 [G+1], group_prefix_len int32 [G]")
    dt = _dtype_code(q)
    dev = q.device
    _on_device(dev, q=q, out=out, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
               context_lens=context_lens, group_start=group_start,
               group_prefix_len=group_prefix_len, workspace=workspace)
    ws_bytes = int(_lib.pa_decode_shared_workspace_bytes(B, G, hq, num_kv_heads, D, block_size,
                                                         max_context_len, dt))
    if ws_bytes and workspace is None:
        workspace = _scratch(ws_bytes, dev, stream)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(dev):
        _check(_lib.pa_decode_shared(_dev_ptr(out, "out"), _dev_ptr(q, "q"),
                                     _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                                     _dev_ptr(block_tables, "block_tables"),
                                     _dev_ptr(context_lens, "context_lens"), float(scale),
                                     block_size, num_kv_heads, B, hq, D, block_tables.shape[1],
                                     int(max_context_len), nb, dt,
                                     _dev_ptr(group_start, "group_start"),
                                     _dev_ptr(group_prefix_len, "group_prefix_len"), G, ws_ptr,
                                     ws_len, _stream(stream, dev)))
    return out


def bench_stream_read(buf, sink, workgroups, stream=None):
    """Measurement helper (include/pa_bench.h): read every byte of the device
    tensor ``buf`` once with 16-byte non-temporal loads; ``sink`` a uint32
    device tensor of workgroups * 256 entries."""
    if sink.numel() < workgroups * 256 or sink.dtype != torch.int32 and sink.dtype != torch.uint32:
        raise ValueError("sink must hold workgroups * 256 32-bit entries")
    dev = buf.device
    _on_device(dev, buf=buf, sink=sink)
    with torch.cuda.device(dev):
        _check(_lib.pa_bench_stream_read(_dev_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                                         _dev_ptr(sink, "sink"), int(workgroups),
                                         _stream(stream, dev)))


def pa_decode_write(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale,
                    block_size, num_kv_heads, max_context_len, partition_size=0, workspace=None,
                    stream=None):
    """One decode iteration in one launch (see pa.h): sequence b's new token,
    rows k_new[b] / v_new[b] ([num_seqs, Hkv, D]; the sequence dim may be
    strided), is stored at position context_lens[b] - 1 of its table, and
    ``out`` is pa_decode's result over the context including it."""
    B, hq, D = q.shape
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("pools must have q's dtype")
    nb = _check_pools(k_cache, v_cache, num_kv_heads, block_size, D)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (B, num_kv_heads, D) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [num_seqs, num_kv_heads, head_dim] of q's dtype")
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{name} rows must be [Hkv, D] contiguous per sequence")
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be a device tensor on q's device")
    if k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must have one sequence stride")
    dt = _dtype_code(q)
    dev = q.device
    _on_device(dev, q=q, out=out, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
               context_lens=context_lens, workspace=workspace)
    ws_bytes = int(_lib.pa_decode_workspace_bytes(B, hq, num_kv_heads, D, block_size,
                                                  max_context_len, partition_size, dt))
    if ws_bytes and workspace is None:
        workspace = _scratch(ws_bytes, dev, stream)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(dev):
        _check(_lib.pa_decode_write(_dev_ptr(out, "out"), _dev_ptr(q, "q"),
                                    ctypes.c_void_p(k_new.data_ptr()),
                                    ctypes.c_void_p(v_new.data_ptr()), k_new.stride(0),
                                    _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                                    _dev_ptr(block_tables, "block_tables"),
                                    _dev_ptr(context_lens, "context_lens"), float(scale),
                                    block_size, num_kv_heads, B, hq, D, block_tables.shape[1],
                                    int(max_context_len), nb, dt, int(partition_size), ws_ptr,
                                    ws_len, _stream(stream, dev)))
    return out


def pa_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
               block_size, num_kv_heads, max_query_len, max_context_len, stream=None):
    """Chunked-prefill attention (see pa.h): q / out [num_tokens, Hq, D];
    sequence b's query rows are query_start[b] .. query_start[b+1]-1 (int32
    device tensor of num_seqs + 1), the last ones of its context."""
    T, hq, D = q.shape
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("pools must have q's dtype")
    nb = _check_pools(k_cache, v_cache, num_kv_heads, block_size, D)
    B = context_lens.shape[0]
    for name, t, shape in (("block_tables", block_tables, None), ("context_lens", context_lens,
                                                                   (B,)),
                           ("query_start", query_start, (B + 1,))):
        if t.dtype != torch.int32 or (shape is not None and tuple(t.shape) != shape):
            raise ValueError(f"{name} must be int32 of the right shape")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    dev = q.device
    _on_device(dev, q=q, out=out, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
               context_lens=context_lens, query_start=query_start)
    with torch.cuda.device(dev):
        _check(_lib.pa_prefill(_dev_ptr(out, "out"), _dev_ptr(q, "q"),
                               _dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                               _dev_ptr(block_tables, "block_tables"),
                               _dev_ptr(context_lens, "context_lens"),
                               _dev_ptr(query_start, "query_start"), float(scale), block_size,
                               num_kv_heads, B, hq, D, block_tables.shape[1],
                               int(max_query_len), int(max_context_len), nb, _dtype_code(q),
                               _stream(stream, dev)))
    return out


# ------------------------------------------------------------ cache ops --
def pa_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, block_size, stream=None):
    """Write token rows k, v ([T, Hkv, D]; the token dim may be strided) into
    their slots (int64 [T], negative = skip)."""
    T, hkv, D = k.shape
    if v.shape != k.shape or k.dtype != k_cache.dtype or v.dtype != k_cache.dtype:
        raise ValueError("k / v must match each other and the pools")
    for name, t in (("k", k), ("v", v)):
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{name} rows must be [Hkv, D] contiguous per token")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    for name, t in (("k", k), ("v", v)):
        if not t.is_cuda or t.device != k_cache.device:
            raise ValueError(f"{name} must be a device tensor on the pools' device")
    nb = _check_pools(k_cache, v_cache, hkv, block_size, D)
    dev = k_cache.device
    _on_device(dev, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping)
    with torch.cuda.device(dev):
        _check(_lib.pa_reshape_and_cache(ctypes.c_void_p(k.data_ptr()),
                                         ctypes.c_void_p(v.data_ptr()),
                                         _dev_ptr(k_cache, "k_cache"),
                                         _dev_ptr(v_cache, "v_cache"),
                                         _dev_ptr(slot_mapping, "slot_mapping"), T, k.stride(0),
                                         v.stride(0), hkv, D, block_size, nb,
                                         _dtype_code(k_cache), _stream(stream, dev)))


def pa_copy_blocks(k_cache, v_cache, src_dst_pairs, block_size, stream=None):
    """Copy whole blocks src -> dst in both pools; pairs int64 [P, 2]."""
    if src_dst_pairs.dtype != torch.int64 or src_dst_pairs.dim() != 2 or \
            src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be int64 [num_pairs, 2]")
    if v_cache.dim() != 5:
        raise ValueError("v_cache must be [blocks][Hkv][BS/VS][D][VS]")
    hkv, D = v_cache.shape[1], v_cache.shape[3]
    nb = _check_pools(k_cache, v_cache, hkv, block_size, D)
    dev = k_cache.device
    _on_device(dev, k_cache=k_cache, v_cache=v_cache, src_dst_pairs=src_dst_pairs)
    with torch.cuda.device(dev):
        _check(_lib.pa_copy_blocks(_dev_ptr(k_cache, "k_cache"), _dev_ptr(v_cache, "v_cache"),
                                   _dev_ptr(src_dst_pairs, "src_dst_pairs"),
                                   src_dst_pairs.shape[0], hkv, D, block_size, nb,
                                   _dtype_code(k_cache), _stream(stream, dev)))


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, src_dst_pairs, block_size, stream=None):
    """Copy whole blocks from (src_k, src_v) to (dst_k, dst_v), pools of one
    layout that may live on the device or in pinned host memory; pairs int64
    [P, 2] on the device or pinned.  Pageable host tensors are refused."""
    if src_dst_pairs.dtype != torch.int64 or src_dst_pairs.dim() != 2 or \
            src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be int64 [num_pairs, 2]")
    for name, t in (("src_k", src_k), ("src_v", src_v), ("dst_k", dst_k), ("dst_v", dst_v),
                    ("src_dst_pairs", src_dst_pairs)):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a device tensor or pinned host memory")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    hkv, D = src_v.shape[1], src_v.shape[3]
    ns = _check_pools(src_k, src_v, hkv, block_size, D)
    nd = _check_pools(dst_k, dst_v, hkv, block_size, D)
    if src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools must have one dtype")
    # the device tensors among them share one device, where the copy runs
    devs = {t.device for t in (src_k, src_v, dst_k, dst_v, src_dst_pairs) if t.is_cuda}
    if len(devs) > 1:
        raise ValueError("the device tensors must share one device")
    dev = devs.pop() if devs else torch.device("cuda", torch.cuda.current_device())
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    with torch.cuda.device(dev):
        _check(_lib.pa_swap_blocks(ptr(src_k), ptr(src_v), ptr(dst_k), ptr(dst_v),
                                   ptr(src_dst_pairs), src_dst_pairs.shape[0], ns, nd, hkv, D,
                                   block_size, _dtype_code(src_k), _stream(stream, dev)))


# ------------------------------------------------------------ allocator --
class BlockAllocator:
    """Host ref-counted block pool (pa_alloc_* in pa.h)."""

    def __init__(self, num_blocks: int, block_size: int, shuffle_seed: int = 0):
        self._h = _lib.pa_alloc_create(num_blocks, block_size, shuffle_seed)
        if not self._h:
            raise ValueError("pa_alloc_create failed")
        self._destroy = _lib.pa_alloc_destroy  # still reachable at interpreter exit
        self.block_size = block_size
        self.num_blocks = num_blocks

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._destroy(h)
            self._h = None

    def add_seq(self, seq_id: int, num_tokens: int) -> None:
        _check(_lib.pa_alloc_add_seq(self._h, seq_id, num_tokens))

    def fork(self, parent_id: int, child_id: int) -> None:
        _check(_lib.pa_alloc_fork(self._h, parent_id, child_id))

    def append(self, seq_id: int, n_tokens: int):
        """Returns (slots int64[n_tokens], cow_pair (src, dst) or None)."""
        slots = np.empty(max(n_tokens, 1), dtype=np.int64)
        pair = np.empty(2, dtype=np.int64)
        n = ctypes.c_int32(0)
        _check(_lib.pa_alloc_append(self._h, seq_id, n_tokens,
                                    slots.ctypes.data_as(ctypes.c_void_p),
                                    pair.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n)))
        return slots[:n_tokens], ((int(pair[0]), int(pair[1])) if n.value else None)

    def append_batch(self, seq_ids, n_tokens):
        """One step for many sequences in one call.  Returns (slots int64[sum
        n_tokens], cow pairs int64[k][2]); on failure raises PAError (OutOfBlocks
        for PA_ENOMEM) with .done = the number of sequences appended before
        the failing one."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        nt = np.ascontiguousarray(n_tokens, dtype=np.int32)
        if ids.shape != nt.shape or ids.ndim != 1:
            raise ValueError("seq_ids and n_tokens must be 1-D and of one length")
        slots = np.empty(max(int(nt.sum()), 1), dtype=np.int64)
        pairs = np.empty((max(len(ids), 1), 2), dtype=np.int64)
        ncow, done = ctypes.c_int32(0), ctypes.c_int32(0)
        st = _lib.pa_alloc_append_batch(self._h, ids.ctypes.data_as(ctypes.c_void_p),
                                        nt.ctypes.data_as(ctypes.c_void_p), len(ids),
                                        slots.ctypes.data_as(ctypes.c_void_p),
                                        pairs.ctypes.data_as(ctypes.c_void_p),
                                        ctypes.byref(ncow), ctypes.byref(done))
        if st != 0:
            err = OutOfBlocks(st) if st == -3 else PAError(st)
            err.done = done.value
            raise err
        return slots[:int(nt.sum())], pairs[:ncow.value]

    def free_seq(self, seq_id: int) -> None:
        _check(_lib.pa_alloc_free_seq(self._h, seq_id))

    def discard_seq(self, seq_id: int) -> None:
        """free_seq for a sequence whose slots were never written: the prefix
        table entries it created are dropped first (pa_alloc_discard_seq)."""
        _check(_lib.pa_alloc_discard_seq(self._h, seq_id))

    def share_groups(self, seq_ids, max_members: int = 16):
        """Groups for pa_decode_shared (pa_alloc_share_groups): returns
        (group_start int32[G+1], group_prefix_len int32[G])."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        gs = np.empty(len(ids) + 1, dtype=np.int32)
        gp = np.empty(max(len(ids), 1), dtype=np.int32)
        ng = ctypes.c_int32(0)
        _check(_lib.pa_alloc_share_groups(self._h, ids.ctypes.data_as(ctypes.c_void_p), len(ids),
                                          max_members, gs.ctypes.data_as(ctypes.c_void_p),
                                          gp.ctypes.data_as(ctypes.c_void_p), ctypes.byref(ng)))
        return gs[:ng.value + 1].copy(), gp[:ng.value].copy()

    def block_tables(self, seq_ids, max_blocks: int):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((len(ids), max_blocks), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        _check(_lib.pa_alloc_block_tables(self._h, ids.ctypes.data_as(ctypes.c_void_p), len(ids),
                                          max_blocks, tables.ctypes.data_as(ctypes.c_void_p),
                                          lens.ctypes.data_as(ctypes.c_void_p)))
        return tables, lens

    def num_free(self) -> int:
        return int(_lib.pa_alloc_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(_lib.pa_alloc_refcount(self._h, block))

    def seq_len(self, seq_id: int) -> int:
        return int(_lib.pa_alloc_seq_len(self._h, seq_id))

    def seq_num_blocks(self, seq_id: int) -> int:
        return int(_lib.pa_alloc_seq_num_blocks(self._h, seq_id))

    # ---- automatic prefix caching
    def add_seq_tokens(self, seq_id: int, tokens, salt: int = 0) -> int:
        """New sequence with prompt ``tokens``; returns how many leading
        tokens already have their K/V in reused blocks."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(_lib.pa_alloc_add_seq_tokens(self._h, seq_id, t.ctypes.data_as(ctypes.c_void_p),
                                            len(t), salt, ctypes.byref(n)))
        return n.value

    def append_tokens(self, seq_id: int, tokens):
        """As ``append`` for known tokens; blocks they fill become cached."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(max(len(t), 1), dtype=np.int64)
        pair = np.empty(2, dtype=np.int64)
        n = ctypes.c_int32(0)
        _check(_lib.pa_alloc_append_tokens(self._h, seq_id, t.ctypes.data_as(ctypes.c_void_p),
                                           len(t), slots.ctypes.data_as(ctypes.c_void_p),
                                           pair.ctypes.data_as(ctypes.c_void_p),
                                           ctypes.byref(n)))
        return slots[:len(t)], ((int(pair[0]), int(pair[1])) if n.value else None)

    def num_cached(self) -> int:
        return int(_lib.pa_alloc_num_cached(self._h))

    def num_evictable(self) -> int:
        return int(_lib.pa_alloc_num_evictable(self._h))

    def reset_prefix_cache(self) -> None:
        _check(_lib.pa_alloc_reset_prefix_cache(self._h))


def prefix_block_hash(parent, salt: int, tokens) -> bytes:
    """SHA-256 block identity of pa_prefix_block_hash (parent: 32 bytes or
    None)."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    out = (ctypes.c_uint8 * 32)()
    par = None if parent is None else (ctypes.c_uint8 * 32).from_buffer_copy(bytes(parent))
    _check(_lib.pa_prefix_block_hash(par, salt, t.ctypes.data_as(ctypes.c_void_p), len(t), out))
    return bytes(out)
