"""Python binding of libkvx (include/kvx.h): argument marshalling only.

Each kvx_* function here takes torch tensors, checks that they are device tensors of the
right dtype and contiguity, and passes their data pointers, sizes and the current HIP stream
to the C entry point of the same name. Every step of the path runs in libkvx's kernels; there
is no fallback. A non-zero status raises KvxError with the library's status string.

The library is located like the pages' NCCL loader (page "0. vllm 如何使用 nccl 传输 kv cache",
§2.1 and §2.2): an environment variable (KVX_SO_PATH) names it, else the in-tree build is
used; it is opened with ctypes.CDLL and every exported function gets a restype/argtypes
entry from one signature table.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(_HERE, "libkvx.so")

KVX_SUCCESS = 0
KVX_ERR_INVALID_ARGUMENT = 1
KVX_ERR_MISALIGNED = 2
KVX_ERR_CAPACITY = 3
KVX_ERR_HIP = 4

DEVERR_BLOCK_RANGE = 1
DEVERR_TABLE_RANGE = 2
DEVERR_SLOT_RANGE = 4
DEVERR_OFFSETS = 8
DEVERR_TIMEOUT = 16

MODE_PACK, MODE_UNPACK, MODE_DIRECT = 0, 1, 2
MAX_SOURCES = 8
ARRIVALS_BYTES = 4096  # workspace of one signalling copy (KVX_ARRIVALS_BYTES)
NOALLOC_SLOTS = 16  # arrivals workspaces the library keeps per GPU for kvx_pack_signal_noalloc
MAX_EXTENT_BYTES = 1 << 56  # largest byte extent one call may describe (KVX_MAX_EXTENT_BYTES)
XFER_BYTES = 32  # sizeof(kvx_xfer)

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

# name -> (restype, argtypes); mirrors include/kvx.h
SIGNATURES = {
    "kvx_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvx_abi_version": (_I32, []),
    "kvx_slot_mapping": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _I64, _I32, _P, _P, _P]),
    "kvx_reshape_and_cache": (ctypes.c_int, [_P, _I64, _P, _I64, _I64, _I64, _P, _P, _I64, _I32,
                                             _I64, _I64, _I64, _P, _P]),
    "kvx_build_xfer_list": (ctypes.c_int, [_P, _P, _P, _I32, _I64, _I32, _P, _I64, _P, _P, _P]),
    "kvx_pack": (ctypes.c_int, [_P, _I32, _I64, _I64, _P, _P, _I64, _P, _P, _P]),
    "kvx_unpack": (ctypes.c_int, [_P, _I32, _P, _I32, _I64, _I64, _I32, _P, _P, _I64, _P, _P]),
    "kvx_pack_split": (ctypes.c_int, [_P, _I32, _I64, _I64, _I32, _P, _P, _I64, _P, _I32, _P, _P]),
    "kvx_pack_kv_first": (ctypes.c_int, [_P, _I32, _I64, _I64, _I64, _P, _I32, _P, _P, _I64, _P, _P, _P]),
    "kvx_unpack_kv_first": (ctypes.c_int, [_P, _P, _I32, _I64, _I64, _I64, _P, _I32, _P, _P, _I64, _P, _P]),
    "kvx_copy_direct": (ctypes.c_int, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _I64, _P, _P]),
    "kvx_signal_add": (ctypes.c_int, [_P, ctypes.c_uint64, _P]),
    "kvx_signal_wait": (ctypes.c_int, [_P, ctypes.c_uint64, _I64, _P, _P]),
    "kvx_pack_signal": (ctypes.c_int, [_P, _I32, _I64, _I64, _P, _P, _I64, _P, _P, ctypes.c_uint64, _P, _P, _P]),
    "kvx_copy_direct_signal": (ctypes.c_int, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _I64, _P, ctypes.c_uint64,
                                              _P, _P, _P]),
    "kvx_pack_signal_noalloc": (ctypes.c_int, [_P, _I32, _I64, _I64, _P, _P, _I64, _P, _P, ctypes.c_uint64, _I32,
                                               _P, _P]),
}


class KvxError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {message} (status {status})")
        self.status = status


def library_path() -> str:
    return os.environ.get("KVX_SO_PATH") or DEFAULT_LIB


def _load():
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"libkvx not found at {path}: build it with `python -m block_table_contiguous_amd.build` "
            "(the KV transfer path has no fallback)")
    lib = ctypes.CDLL(path)
    funcs = {}
    for name, (restype, argtypes) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = restype
        f.argtypes = argtypes
        funcs[name] = f
    return lib, funcs


LIB, _F = _load()


def kvx_status_string(status: int) -> str:
    return _F["kvx_status_string"](int(status)).decode()


def kvx_abi_version() -> int:
    return int(_F["kvx_abi_version"]())


def _check(fn: str, status: int):
    if status != KVX_SUCCESS:
        raise KvxError(fn, status, kvx_status_string(status))


# ---------------------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("kvx: tensors must live on the GPU")
    return t.data_ptr()


_raw_stream = None  # torch's internal raw-handle query, once it has been seen to agree


def _public_stream() -> int:
    import torch

    return torch.cuda.current_stream().cuda_stream


def _current_stream() -> int:
    """The current device's current stream handle. torch.cuda.current_stream() builds a Stream
    object per call (a third of a small call's host time), so the binding uses torch's raw
    handle query instead, but only after checking once that it returns the same handle as the
    public API; if the query is missing or disagrees, every call uses the public API."""
    global _raw_stream
    if _raw_stream is None:
        import torch

        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        dev = getattr(torch._C, "_cuda_getDevice", None)
        fast = None
        if raw is not None and dev is not None:
            fast = lambda: raw(dev())  # noqa: E731
            try:
                if fast() != _public_stream():
                    fast = None
            except Exception:  # a changed signature: fall back to the public API
                fast = None
        _raw_stream = fast or _public_stream
    return _raw_stream()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _rows_contiguous(t) -> bool:
    """Every t[i] is densely packed (the dimensions after the first are contiguous)."""
    if t.is_contiguous():  # the common case, without walking the strides
        return True
    expect = 1
    for size, stride in zip(reversed(t.shape[1:]), reversed(t.stride()[1:])):
        if size != 1 and stride != expect:
            return False
        expect *= size
    return True


def _want(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"kvx: {name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"kvx: {name} must be contiguous")


def _want_runs(xfers, xfer_count, total_blocks: int):
    """A run list the copy kernels may read up to total_blocks records of."""
    import torch

    _want(xfers, torch.int64, "xfers")
    _want(xfer_count, torch.int64, "xfer_count")
    if xfers.numel() // 4 < total_blocks or xfer_count.numel() < 1:
        raise ValueError("kvx: the run list holds fewer than total_blocks records")


def layer_base_table(layers: Sequence, device=None):
    """Device int64 array of the layers' base addresses (the per-layer cache pointers the
    pack/unpack kernels index)."""
    import torch

    dev = device if device is not None else layers[0].device
    return torch.tensor([t.data_ptr() for t in layers], dtype=torch.int64, device=dev)


def flatten_tables(tables: Sequence[np.ndarray], device):
    """Per-request id lists -> (ids int32 [N], req_offsets int64 [R+1]) device tensors (CSR)."""
    import torch

    counts = np.array([len(t) for t in tables], dtype=np.int64)
    offsets = np.zeros(len(tables) + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    ids = np.concatenate([np.asarray(t, np.int32) for t in tables]) if len(tables) else np.zeros(0, np.int32)
    return (torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(device),
            torch.from_numpy(offsets).to(device))


def new_xfer_list(capacity: int, device):
    """Storage for `capacity` kvx_xfer records (int64 [capacity][4]) plus its count."""
    import torch

    return (torch.zeros((max(int(capacity), 1), 4), dtype=torch.int64, device=device),
            torch.zeros(1, dtype=torch.int64, device=device))


def decode_xfers(xfers, count) -> List[tuple]:
    """Host copy of a run list as (src_block, dst_block, buf_block, num_blocks, req) tuples."""
    n = int(count.item()) if hasattr(count, "item") else int(count)
    raw = xfers[:n].cpu().numpy()
    tail = raw[:, 3].copy().view(np.int32).reshape(n, 2)
    return [(int(a), int(b), int(c), int(t[0]), int(t[1])) for (a, b, c, _), t in zip(raw, tail)]


def cache_strides(kv_cache, layout: str = "blocks_tokens_kv"):
    """(num_blocks, block_size, block_stride, token_stride, kv_stride) in bytes for a 5-D cache
    tensor in one of three layouts:
      blocks_tokens_kv  [blocks][block_size][K,V][heads][head_dim]
      blocks_kv_tokens  [blocks][K,V][block_size][heads][head_dim]
      kv_blocks_tokens  [K,V][blocks][block_size][heads][head_dim]"""
    e = kv_cache.element_size()
    s = [x * e for x in kv_cache.stride()]
    sh = kv_cache.shape
    if layout == "blocks_tokens_kv":
        return sh[0], sh[1], s[0], s[1], s[2]
    if layout == "blocks_kv_tokens":
        return sh[0], sh[2], s[0], s[2], s[1]
    if layout == "kv_blocks_tokens":
        return sh[1], sh[2], s[1], s[2], s[0]
    raise ValueError(f"unknown layout {layout}")


# ---------------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------------

def kvx_slot_mapping(block_table, req_idx, positions, block_size: int, slot_mapping,
                     err_flag=None, max_blocks_per_req: Optional[int] = None, stream=None):
    """slot_mapping[i] = block_table[req_idx[i], positions[i] // bs] * bs + positions[i] % bs."""
    import torch

    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("kvx: block_table must be a row-major int32 [num_reqs][width] tensor")
    _want(req_idx, torch.int32, "req_idx")
    _want(positions, torch.int64, "positions")
    _want(slot_mapping, torch.int64, "slot_mapping")
    T = req_idx.numel()
    if positions.numel() != T or slot_mapping.numel() != T:
        raise ValueError("kvx: req_idx, positions and slot_mapping need the same length")
    width = block_table.shape[1] if max_blocks_per_req is None else int(max_blocks_per_req)
    if width > block_table.shape[1]:
        raise ValueError("kvx: max_blocks_per_req is wider than the block table")
    # a one-row table's row stride is never used (it can be 0 for a broadcast row)
    row_stride = block_table.stride(0) if block_table.shape[0] > 1 else max(block_table.shape[1], width)
    st = _F["kvx_slot_mapping"](_ptr(block_table), block_table.shape[0], width,
                                row_stride, _ptr(req_idx), _ptr(positions), T,
                                int(block_size), _ptr(slot_mapping), _ptr(err_flag), _stream(stream))
    _check("kvx_slot_mapping", st)


def kvx_reshape_and_cache(key, value, slot_mapping, kv_cache, num_blocks: int, block_size: int,
                          block_stride_bytes: int, token_stride_bytes: int, kv_stride_bytes: int,
                          err_flag=None, stream=None):
    """Write key[i] / value[i] rows into kv_cache at slot_mapping[i] (negative slot = skip)."""
    import torch

    _want(slot_mapping, torch.int64, "slot_mapping")
    T = slot_mapping.numel()
    if key.shape[0] != T or value.shape[0] != T or key.shape != value.shape:
        raise ValueError("kvx: key/value must be [num_tokens, ...] of the same shape")
    e = key.element_size()
    row = key.numel() // T * e if T else 0
    for name, t in (("key", key), ("value", value)):
        if not _rows_contiguous(t):
            raise ValueError(f"kvx: each {name} row must be contiguous")
    if T and num_blocks > 0:
        last = ((int(num_blocks) - 1) * int(block_stride_bytes) + (int(block_size) - 1) * int(token_stride_bytes)
                + int(kv_stride_bytes) + row)
        room = kv_cache.untyped_storage().nbytes() - kv_cache.storage_offset() * kv_cache.element_size()
        if last > room:
            raise ValueError("kvx: num_blocks, block_size and the strides address bytes past the end of kv_cache")
    st = _F["kvx_reshape_and_cache"](_ptr(key), key.stride(0) * e, _ptr(value), value.stride(0) * e,
                                     T, row, _ptr(slot_mapping), _ptr(kv_cache), int(num_blocks),
                                     int(block_size), int(block_stride_bytes), int(token_stride_bytes),
                                     int(kv_stride_bytes), _ptr(err_flag), _stream(stream))
    _check("kvx_reshape_and_cache", st)


def kvx_build_xfer_list(src_ids, dst_ids, req_offsets, mode: int, xfers, xfer_count,
                        err_flag=None, stream=None):
    """Cut the CSR block lists into maximal runs (see include/kvx.h)."""
    import torch

    _want(req_offsets, torch.int64, "req_offsets")
    for name, t in (("src_ids", src_ids), ("dst_ids", dst_ids)):
        if t is not None:
            _want(t, torch.int32, name)
    _want(xfers, torch.int64, "xfers")
    if req_offsets.numel() < 1:
        raise ValueError("kvx: req_offsets needs num_reqs + 1 entries")
    if src_ids is not None and dst_ids is not None and src_ids.numel() != dst_ids.numel():
        raise ValueError("kvx: src_ids and dst_ids must list the same number of blocks")
    ref = src_ids if src_ids is not None else dst_ids
    total = ref.numel() if ref is not None else 0
    capacity = xfers.numel() // 4
    st = _F["kvx_build_xfer_list"](_ptr(src_ids), _ptr(dst_ids), _ptr(req_offsets),
                                   req_offsets.numel() - 1, total, int(mode), _ptr(xfers), capacity,
                                   _ptr(xfer_count), _ptr(err_flag), _stream(stream))
    _check("kvx_build_xfer_list", st)


def kvx_pack(layer_bases, block_bytes: int, num_cache_blocks: int, xfers, xfer_count,
             total_blocks: int, send_buf, err_flag=None, stream=None):
    """Gather the listed blocks of every layer into send_buf [L][total_blocks][block_bytes]."""
    import torch

    _want(layer_bases, torch.int64, "layer_bases")
    _want_runs(xfers, xfer_count, total_blocks)
    L = layer_bases.numel()
    if send_buf.numel() * send_buf.element_size() < L * total_blocks * block_bytes:
        raise ValueError("kvx: send_buf smaller than num_layers * total_blocks * block_bytes")
    st = _F["kvx_pack"](_ptr(layer_bases), L, int(block_bytes), int(num_cache_blocks), _ptr(xfers),
                        _ptr(xfer_count), int(total_blocks), _ptr(send_buf), _ptr(err_flag),
                        _stream(stream))
    _check("kvx_pack", st)


def kvx_unpack(send_bufs: Sequence, layer_bases, block_bytes: int, num_cache_blocks: int,
               rows_per_block: int, xfers, xfer_count, total_blocks: int, err_flag=None,
               stream=None):
    """Scatter send buffer(s) into the listed destination blocks; with several sources each
    destination row is the concatenation of the sources' rows (head merge)."""
    import torch

    _want(layer_bases, torch.int64, "layer_bases")
    _want_runs(xfers, xfer_count, total_blocks)
    L = layer_bases.numel()
    S = len(send_bufs)
    if not 1 <= S <= MAX_SOURCES:
        raise ValueError(f"kvx: 1..{MAX_SOURCES} send buffers")
    for b in send_bufs:
        if b.numel() * b.element_size() < L * total_blocks * (block_bytes // S):
            raise ValueError("kvx: a send buffer is smaller than num_layers * total_blocks * block_bytes/num_src")
    arr = (ctypes.c_void_p * S)(*[_ptr(b) for b in send_bufs])
    st = _F["kvx_unpack"](arr, S, _ptr(layer_bases), L, int(block_bytes), int(num_cache_blocks),
                          int(rows_per_block), _ptr(xfers), _ptr(xfer_count), int(total_blocks),
                          _ptr(err_flag), _stream(stream))
    _check("kvx_unpack", st)


def kvx_copy_direct(src_layer_bases, dst_layer_bases, block_bytes: int, src_num_blocks: int,
                    dst_num_blocks: int, xfers, xfer_count, total_blocks: int, err_flag=None,
                    stream=None):
    """Copy the listed blocks of every layer from the source caches straight into the
    destination caches (no buffer); the runs come from kvx_build_xfer_list(MODE_DIRECT)."""
    import torch

    _want(src_layer_bases, torch.int64, "src_layer_bases")
    _want(dst_layer_bases, torch.int64, "dst_layer_bases")
    _want_runs(xfers, xfer_count, total_blocks)
    L = src_layer_bases.numel()
    if dst_layer_bases.numel() != L:
        raise ValueError("kvx: source and destination layer tables differ in length")
    st = _F["kvx_copy_direct"](_ptr(src_layer_bases), _ptr(dst_layer_bases), L, int(block_bytes),
                               int(src_num_blocks), int(dst_num_blocks), _ptr(xfers), _ptr(xfer_count),
                               int(total_blocks), _ptr(err_flag), _stream(stream))
    _check("kvx_copy_direct", st)


def kvx_pack_split(layer_bases, block_bytes: int, num_cache_blocks: int, rows_per_block: int,
                   xfers, xfer_count, total_blocks: int, send_bufs: Sequence, err_flag=None,
                   stream=None):
    """Pack for num_dst receivers that each own a head shard: send_bufs[d] gets piece d of
    every row of every listed block (the inverse of kvx_unpack's merge)."""
    import torch

    _want(layer_bases, torch.int64, "layer_bases")
    _want_runs(xfers, xfer_count, total_blocks)
    L = layer_bases.numel()
    D = len(send_bufs)
    if not 1 <= D <= MAX_SOURCES:
        raise ValueError(f"kvx: 1..{MAX_SOURCES} send buffers")
    for b in send_bufs:
        if b.numel() * b.element_size() < L * total_blocks * (block_bytes // D):
            raise ValueError("kvx: a send buffer is smaller than num_layers * total_blocks * block_bytes/num_dst")
    arr = (ctypes.c_void_p * D)(*[_ptr(b) for b in send_bufs])
    st = _F["kvx_pack_split"](_ptr(layer_bases), L, int(block_bytes), int(num_cache_blocks),
                              int(rows_per_block), _ptr(xfers), _ptr(xfer_count), int(total_blocks), arr, D,
                              _ptr(err_flag), _stream(stream))
    _check("kvx_pack_split", st)


def kvx_pack_kv_first(layer_bases, segment_bytes: int, plane_stride_bytes: int, num_cache_blocks: int,
                      req_offsets, xfers, xfer_count, total_blocks: int, send_buf, err_flag=None,
                      stream=None):
    """Pack from kv-first caches: per layer and request, the K segments then the V segments."""
    import torch

    _want(layer_bases, torch.int64, "layer_bases")
    _want_runs(xfers, xfer_count, total_blocks)
    _want(req_offsets, torch.int64, "req_offsets")
    L = layer_bases.numel()
    if send_buf.numel() * send_buf.element_size() < L * 2 * total_blocks * segment_bytes:
        raise ValueError("kvx: send_buf smaller than num_layers * 2 * total_blocks * segment_bytes")
    st = _F["kvx_pack_kv_first"](_ptr(layer_bases), L, int(segment_bytes), int(plane_stride_bytes),
                                 int(num_cache_blocks), _ptr(req_offsets), req_offsets.numel() - 1,
                                 _ptr(xfers), _ptr(xfer_count), int(total_blocks), _ptr(send_buf),
                                 _ptr(err_flag), _stream(stream))
    _check("kvx_pack_kv_first", st)


def kvx_unpack_kv_first(send_buf, layer_bases, segment_bytes: int, plane_stride_bytes: int,
                        num_cache_blocks: int, req_offsets, xfers, xfer_count, total_blocks: int,
                        err_flag=None, stream=None):
    """Scatter a kv-first buffer (per request: K segments, then V segments) into kv-first caches."""
    import torch

    _want(layer_bases, torch.int64, "layer_bases")
    _want_runs(xfers, xfer_count, total_blocks)
    _want(req_offsets, torch.int64, "req_offsets")
    L = layer_bases.numel()
    if send_buf.numel() * send_buf.element_size() < L * 2 * total_blocks * segment_bytes:
        raise ValueError("kvx: send_buf smaller than num_layers * 2 * total_blocks * segment_bytes")
    st = _F["kvx_unpack_kv_first"](_ptr(send_buf), _ptr(layer_bases), L, int(segment_bytes),
                                   int(plane_stride_bytes), int(num_cache_blocks), _ptr(req_offsets),
                                   req_offsets.numel() - 1, _ptr(xfers), _ptr(xfer_count), int(total_blocks),
                                   _ptr(err_flag), _stream(stream))
    _check("kvx_unpack_kv_first", st)


def new_arrivals(device):
    """A zeroed arrivals workspace for the signalling copies (one per concurrent stream)."""
    import torch

    return torch.zeros(ARRIVALS_BYTES // 4, dtype=torch.int32, device=device)


def _want_signal(counter, arrivals):
    import torch

    _want(counter, torch.int64, "counter")
    _want(arrivals, torch.int32, "arrivals")
    if counter.numel() < 1 or arrivals.numel() * 4 < ARRIVALS_BYTES:
        raise ValueError(f"kvx: counter needs one element and arrivals {ARRIVALS_BYTES} bytes")


def kvx_pack_signal(layer_bases, block_bytes: int, num_cache_blocks: int, xfers, xfer_count,
                    total_blocks: int, send_buf, counter, arrivals, delta: int = 1, err_flag=None,
                    stream=None):
    """kvx_pack whose launch also adds `delta` to `counter` (int64 device tensor, read as
    uint64) once every packed byte is visible device-wide. `arrivals` is an int32 device
    tensor of ARRIVALS_BYTES // 4 zeros (new_arrivals); each call leaves it all zero again
    (one per concurrent stream)."""
    import torch

    _want(layer_bases, torch.int64, "layer_bases")
    _want_runs(xfers, xfer_count, total_blocks)
    _want_signal(counter, arrivals)
    L = layer_bases.numel()
    if send_buf.numel() * send_buf.element_size() < L * total_blocks * block_bytes:
        raise ValueError("kvx: send_buf smaller than num_layers * total_blocks * block_bytes")
    st = _F["kvx_pack_signal"](_ptr(layer_bases), L, int(block_bytes), int(num_cache_blocks), _ptr(xfers),
                               _ptr(xfer_count), int(total_blocks), _ptr(send_buf), _ptr(counter), int(delta),
                               _ptr(arrivals), _ptr(err_flag), _stream(stream))
    _check("kvx_pack_signal", st)


def kvx_pack_signal_noalloc(layer_bases, block_bytes: int, num_cache_blocks: int, xfers, xfer_count,
                            total_blocks: int, send_buf, counter, slot: int = 0, delta: int = 1, err_flag=None,
                            stream=None):
    """kvx_pack_signal with the arrivals workspace taken from the library's own static array
    (workspace `slot` of NOALLOC_SLOTS): nothing is allocated, here or in the library. Calls
    that use the same slot must not overlap in time; the stream must belong to the current
    device."""
    import torch

    _want(layer_bases, torch.int64, "layer_bases")
    _want_runs(xfers, xfer_count, total_blocks)
    _want(counter, torch.int64, "counter")
    L = layer_bases.numel()
    if send_buf.numel() * send_buf.element_size() < L * total_blocks * block_bytes:
        raise ValueError("kvx: send_buf smaller than num_layers * total_blocks * block_bytes")
    st = _F["kvx_pack_signal_noalloc"](_ptr(layer_bases), L, int(block_bytes), int(num_cache_blocks), _ptr(xfers),
                                       _ptr(xfer_count), int(total_blocks), _ptr(send_buf), _ptr(counter),
                                       int(delta), int(slot), _ptr(err_flag), _stream(stream))
    _check("kvx_pack_signal_noalloc", st)


def kvx_copy_direct_signal(src_layer_bases, dst_layer_bases, block_bytes: int, src_num_blocks: int,
                           dst_num_blocks: int, xfers, xfer_count, total_blocks: int, counter, arrivals,
                           delta: int = 1, err_flag=None, stream=None):
    """kvx_copy_direct whose launch also adds `delta` to `counter` once every copied byte is
    visible device-wide (the one-sided write with its signal); `arrivals` as kvx_pack_signal."""
    import torch

    _want(src_layer_bases, torch.int64, "src_layer_bases")
    _want(dst_layer_bases, torch.int64, "dst_layer_bases")
    _want_runs(xfers, xfer_count, total_blocks)
    _want_signal(counter, arrivals)
    L = src_layer_bases.numel()
    if dst_layer_bases.numel() != L:
        raise ValueError("kvx: source and destination layer tables differ in length")
    st = _F["kvx_copy_direct_signal"](_ptr(src_layer_bases), _ptr(dst_layer_bases), L, int(block_bytes),
                                      int(src_num_blocks), int(dst_num_blocks), _ptr(xfers), _ptr(xfer_count),
                                      int(total_blocks), _ptr(counter), int(delta), _ptr(arrivals),
                                      _ptr(err_flag), _stream(stream))
    _check("kvx_copy_direct_signal", st)


def kvx_signal_add(counter, delta: int = 1, stream=None):
    """Once the work enqueued on `stream` so far has finished, add `delta` to the uint64
    counter (an int64 device tensor of one element, read as unsigned)."""
    _want(counter, _torch_int64(), "counter")
    _check("kvx_signal_add", _F["kvx_signal_add"](_ptr(counter), int(delta), _stream(stream)))


def kvx_signal_wait(counter, value: int, timeout_us: int = 10_000_000, err=None, stream=None):
    """Hold the work enqueued on `stream` after this call until counter >= value (polled on
    the GPU); after timeout_us the wait ends and sets DEVERR_TIMEOUT in `err`."""
    _want(counter, _torch_int64(), "counter")
    _check("kvx_signal_wait", _F["kvx_signal_wait"](_ptr(counter), int(value), int(timeout_us),
                                                    _ptr(err), _stream(stream)))


def _torch_int64():
    import torch

    return torch.int64
