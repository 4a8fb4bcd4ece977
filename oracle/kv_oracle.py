"""CPU oracle for the paged KV-cache transfer path (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may use this
module. It shares no code with the HIP library or its binding and imports neither.

Sources (the four pages this path is built from):
  [nccl]    "0. vllm 如何使用 nccl 传输 kv cache" — sections 2.3 (P2P NCCL engine) and
            2.4 (KV cache connector: extract_kv_from_layer / inject_kv_into_layer).
  [v1]      "vllm v1 调度逻辑 和 distributed 分布式原理" (Excalidraw diagram) — labels
            "batch tensor 组装" (slot formula), "Paged kv cache" (block B3, 16 slots),
            the all-layers KV-memory list (48 x 147456 blocks, one shared block_table),
            and the two "shape of layer i" layouts.
  [flagcx]  "5. flagcx connector design & dev & test" — §1.2 final design, _send_blocks
            (flatten to an xfer list: per layer x per contiguous group x per request).
  [pd]      "vLLM PD 分离" — §四 4.2 _build_transfer_params (per-layer, per-block source and
            destination addresses; TP heterogeneity) and §七 item 3 (destination address =
            per-layer base + block length x block id).

Readings where the pages are silent or garbled are stated at each function.

Every function works on raw bytes and returns new arrays (inputs are never modified).
Device-side error bits are mirrored so error cases can be compared too.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

# Error bits (same meaning as the library's device error flag; the values are restated
# here, not imported).
DEVERR_BLOCK_RANGE = 1  # a cache block id outside [0, num_cache_blocks)
DEVERR_TABLE_RANGE = 2  # slot mapping: request index / position outside the block table
DEVERR_SLOT_RANGE = 4   # new-token write: a slot beyond the cache
DEVERR_OFFSETS = 8      # run building: request offsets not a valid CSR over the blocks

# Which side(s) a run must be consecutive on.
MODE_PACK, MODE_UNPACK, MODE_DIRECT = 0, 1, 2


def _as_block_bytes(cache: np.ndarray) -> np.ndarray:
    """A cache whose first axis is the block id, viewed as [num_blocks][block_bytes] uint8."""
    c = np.ascontiguousarray(cache)
    return c.reshape(c.shape[0], -1).view(np.uint8)


def _reject_repeats(targets, what: str) -> None:
    """Raise ValueError if any target appears twice. Reading (the pages' receiver allocates
    fresh blocks for every request, [pd] §三 3.2): two entries that would write the same
    destination block or slot are invalid input, not a case with a defined winner, so the
    oracle refuses them instead of choosing one. Targets outside the cache are not writes
    (they are skipped and flagged) and are not passed here."""
    seen = set()
    for t in targets:
        if t in seen:
            raise ValueError(f"{what} {t} is written twice: destinations must be distinct")
        seen.add(t)


def buffer_order(tables: Sequence[np.ndarray]) -> List[Tuple[int, int, int]]:
    """The flat request-major order of all listed blocks: (request r, index j in r's table,
    position p). Position p = (blocks of requests before r) + j; this is where block j of
    request r sits inside one layer's slice of the send buffer. [flagcx] §1.2 (_send_blocks:
    the list is flattened over layers, contiguous groups and requests; reading: layer
    outermost, then request, then block-table order)."""
    order, p = [], 0
    for r, t in enumerate(tables):
        for j in range(len(t)):
            order.append((r, j, p))
            p += 1
    return order


# ---------------------------------------------------------------------------------------
# a1 — slot mapping
# ---------------------------------------------------------------------------------------

def slot_mapping(block_table: np.ndarray, req_idx: Sequence[int], positions: Sequence[int],
                 block_size: int) -> Tuple[np.ndarray, int]:
    """Slot of every flat token: the block the token's position falls in, looked up in its
    request's row of the block table, times the block size, plus the position's offset
    inside that block. [v1] label "batch tensor 组装".

    block_table: [num_reqs][width] ids (rows padded with negative ids).
    Returns (slots int64 [T], error bits). A token whose request index is outside the
    table, whose position is negative or beyond the row, or whose table entry is negative
    gets slot -1 and raises DEVERR_TABLE_RANGE (reading: the pages define only the
    in-range case).
    """
    bt = np.asarray(block_table)
    num_reqs, width = bt.shape
    T = len(req_idx)
    slots = np.empty(T, dtype=np.int64)
    err = 0
    for i in range(T):
        r = int(req_idx[i])
        pos = int(positions[i])
        if r < 0 or r >= num_reqs or pos < 0 or pos // block_size >= width:
            slots[i] = -1
            err |= DEVERR_TABLE_RANGE
            continue
        block = int(bt[r, pos // block_size])
        if block < 0:
            slots[i] = -1
            err |= DEVERR_TABLE_RANGE
            continue
        slots[i] = block * block_size + pos % block_size
    return slots, err


# ---------------------------------------------------------------------------------------
# a2 — new-token K/V write through the slot mapping
# ---------------------------------------------------------------------------------------

def reshape_and_cache(cache: np.ndarray, key_rows: np.ndarray, value_rows: np.ndarray,
                      slots: Sequence[int], num_blocks: int, block_size: int,
                      block_stride: int, token_stride: int, kv_stride: int
                      ) -> Tuple[np.ndarray, int]:
    """Write token i's K row and V row into the cache slot slots[i]: block slot//block_size,
    in-block offset slot%block_size. [v1] "Paged kv cache" (token t of a block occupies
    slot t) with the slot formula of "batch tensor 组装"; the write itself is the
    recomputed-token write of [pd] §五 5.2.

    cache: any array, taken as flat bytes. key_rows/value_rows: [T][row_bytes] (any dtype,
    taken as bytes per row). Strides are in bytes: byte address of (block, offset, kv) =
    block*block_stride + offset*token_stride + kv*kv_stride (kv 0 = K, 1 = V). For the
    [blocks][block_size][K,V][heads][head_dim] layout: token_stride = 2*row_bytes,
    kv_stride = row_bytes, block_stride = block_size*token_stride.

    Reading: a negative slot means "no slot" (a padding token) and is skipped; a slot in a
    block >= num_blocks is skipped and raises DEVERR_SLOT_RANGE. Two tokens with the same
    slot inside the cache are invalid input (ValueError), since each new token owns its slot.
    Returns (new cache bytes, flat uint8, error bits).
    """
    _reject_repeats([int(s) for s in slots if int(s) >= 0 and int(s) // block_size < num_blocks],
                    "slot")
    out = np.ascontiguousarray(cache).reshape(-1).view(np.uint8).copy()
    K = np.ascontiguousarray(key_rows).reshape(len(slots), -1).view(np.uint8)
    V = np.ascontiguousarray(value_rows).reshape(len(slots), -1).view(np.uint8)
    row = K.shape[1]
    err = 0
    for i in range(len(slots)):
        s = int(slots[i])
        if s < 0:
            continue
        block, offset = s // block_size, s % block_size
        if block >= num_blocks:
            err |= DEVERR_SLOT_RANGE
            continue
        at = block * block_stride + offset * token_stride
        out[at:at + row] = K[i]
        out[at + kv_stride:at + kv_stride + row] = V[i]
    return out, err


# ---------------------------------------------------------------------------------------
# a3 — transfer list: maximal contiguous runs
# ---------------------------------------------------------------------------------------

def xfer_list(src_tables: Sequence[np.ndarray], dst_tables: Sequence[np.ndarray],
              mode: int) -> List[Tuple[int, int, int, int, int]]:
    """The transfer list: every request's blocks cut into maximal contiguous groups, in
    request order and, inside a request, block-table order. [flagcx] §1.2 (_send_blocks
    flattens to an xfer list per layer x contiguous group x request); [pd] §四 4.2 (source
    and destination address per block); [pd] §七 item 3 (address = base + id x length).

    Reading of "contiguous group": consecutive block-table entries whose ids step by +1 on
    the side(s) the copy addresses — the cache side being read for MODE_PACK, the cache
    side being written for MODE_UNPACK, both for MODE_DIRECT. A group never spans two
    requests and has no length cap. The list is the same for every layer (one block
    table serves all layers: [v1] KV-memory list).

    Returns tuples (src_block, dst_block, buf_block, num_blocks, req) where buf_block is
    the group's first position in the flat request-major order; for MODE_PACK dst_block
    is that buffer position, for MODE_UNPACK src_block is.
    """
    uses_src = mode in (MODE_PACK, MODE_DIRECT)
    uses_dst = mode in (MODE_UNPACK, MODE_DIRECT)
    tables = src_tables if uses_src else dst_tables
    runs = []
    p = 0
    for r in range(len(tables)):
        n = len(tables[r])
        src = [int(x) for x in src_tables[r]] if uses_src else None
        dst = [int(x) for x in dst_tables[r]] if uses_dst else None
        j = 0
        while j < n:
            k = j + 1
            while k < n:
                if uses_src and src[k] != src[k - 1] + 1:
                    break
                if uses_dst and dst[k] != dst[k - 1] + 1:
                    break
                k += 1
            s = src[j] if uses_src else p + j
            d = dst[j] if uses_dst else p + j
            runs.append((s, d, p + j, k - j, r))
            j = k
        p += n
    return runs


# ---------------------------------------------------------------------------------------
# a4 — pack (gather into the contiguous send buffer)
# ---------------------------------------------------------------------------------------

def pack(layer_caches: Sequence[np.ndarray], src_tables: Sequence[np.ndarray],
         buf_init: np.ndarray = None) -> Tuple[np.ndarray, int]:
    """Gather every listed block of every layer into one buffer [L][N][block_bytes]: layer l,
    position p = (blocks of earlier requests) + j holds block src_tables[r][j] of layer l's
    cache, whole blocks, unfilled tail slots included. [nccl] §2.4 (extract_kv_from_layer
    gathers layer[block_ids] for each request and layer); [flagcx] §1.2 (buffer order:
    layer, then request, then block-table order); [v1] KV-memory list (per-layer caches,
    one block table for all layers).

    A block id outside [0, num_blocks) is not copied (that buffer block keeps buf_init's
    bytes, zeros by default) and raises DEVERR_BLOCK_RANGE.
    """
    caches = [_as_block_bytes(c) for c in layer_caches]
    L = len(caches)
    nb, bb = caches[0].shape
    order = buffer_order(src_tables)
    N = len(order)
    buf = np.zeros((L, N, bb), np.uint8) if buf_init is None else \
        np.ascontiguousarray(buf_init).reshape(L, N, bb).view(np.uint8).copy()
    err = 0
    for l in range(L):
        for r, j, p in order:
            b = int(src_tables[r][j])
            if b < 0 or b >= nb:
                err |= DEVERR_BLOCK_RANGE
                continue
            buf[l, p] = caches[l][b]
    return buf, err


# ---------------------------------------------------------------------------------------
# a5 / a6 — unpack (scatter), with the optional merge of head-split sources
# ---------------------------------------------------------------------------------------

def unpack_block(src_blocks: Sequence[np.ndarray], rows_per_block: int) -> np.ndarray:
    """One destination block from the matching block of each of S sources. Every source
    block is rows_per_block equal rows; destination row k is source 0's row k, then source
    1's row k, and so on. With S = 1 this is a plain copy. [pd] §四 4.2 (handles
    TP heterogeneity: mapping between different TP sizes). Reading: source s holds the
    contiguous head range [s*H/S, (s+1)*H/S), the usual head sharding, and a row is one
    (token, K/V) pair, so rows_per_block = block_size*2 for the [block][token][K,V][head]
    [dim] layout."""
    S = len(src_blocks)
    srcs = [np.ascontiguousarray(b).reshape(-1).view(np.uint8) for b in src_blocks]
    row_src = len(srcs[0]) // rows_per_block
    out = np.empty(S * len(srcs[0]), np.uint8)
    for k in range(rows_per_block):
        for s in range(S):
            at = (k * S + s) * row_src
            out[at:at + row_src] = srcs[s][k * row_src:(k + 1) * row_src]
    return out


def unpack(src_buffers: Sequence[np.ndarray], dst_caches: Sequence[np.ndarray],
           dst_tables: Sequence[np.ndarray], rows_per_block: int = 1
           ) -> Tuple[List[np.ndarray], int]:
    """Scatter the buffer into the receiver's own blocks: for layer l and position
    p = (blocks of earlier requests) + j, destination block dst_tables[r][j] of layer l gets
    the buffer's block (l, p); blocks not listed keep their bytes. With S > 1 sources (one
    per sender TP rank, each [L][N][block_bytes/S]) each destination block is merged row by
    row from the S sources (unpack_block). [nccl] §2.3 step 14 / §2.4 (inject the received
    tensor into kv_cache_layer[block_ids]); [pd] §七 item 3 (destination = layer base +
    block length x block id); [pd] §四 4.2 (TP heterogeneity).

    Reading: a destination id outside [0, num_blocks) is skipped and raises
    DEVERR_BLOCK_RANGE; a destination id inside the cache listed twice is invalid input
    (ValueError), since the receiver allocates fresh blocks.
    Returns (new destination caches as [num_blocks][block_bytes] uint8, error bits).
    """
    S = len(src_buffers)
    out = [_as_block_bytes(c).copy() for c in dst_caches]
    L = len(out)
    nb, bb = out[0].shape
    order = buffer_order(dst_tables)
    _reject_repeats([int(dst_tables[r][j]) for r, j, _ in order if 0 <= int(dst_tables[r][j]) < nb],
                    "destination block")
    N = len(order)
    bufs = [np.ascontiguousarray(b).reshape(-1).view(np.uint8).reshape(L, N, bb // S) for b in src_buffers]
    err = 0
    for l in range(L):
        for r, j, p in order:
            d = int(dst_tables[r][j])
            if d < 0 or d >= nb:
                err |= DEVERR_BLOCK_RANGE
                continue
            if S == 1:
                out[l][d] = bufs[0][l, p]
            else:
                out[l][d] = unpack_block([bufs[s][l, p] for s in range(S)], rows_per_block)
    return out, err


def copy_direct(src_caches: Sequence[np.ndarray], dst_caches: Sequence[np.ndarray],
                src_tables: Sequence[np.ndarray], dst_tables: Sequence[np.ndarray]
                ) -> Tuple[List[np.ndarray], int]:
    """Move every listed block straight from the sender's cache into the receiver's, with no
    send buffer in between: for every layer l and table entry (r, j), destination block
    dst_tables[r][j] of layer l gets source block src_tables[r][j] of layer l. [pd] §四 4.2
    (_build_transfer_params / batch_transfer_sync_write: one write per source address,
    destination address and length, from the prefill cache into the decode cache); [pd]
    §七 item 3 (address = layer base + block length x block id).

    Reading: an entry whose source or destination id is outside its cache is not copied
    and raises DEVERR_BLOCK_RANGE (pack's rule for sources, unpack's for destinations); a
    destination id inside the cache listed twice is invalid input (ValueError), as for unpack.
    Returns (new destination caches as [num_blocks][block_bytes] uint8, error bits).
    """
    srcs = [_as_block_bytes(c) for c in src_caches]
    out = [_as_block_bytes(c).copy() for c in dst_caches]
    nbs, nbd = srcs[0].shape[0], out[0].shape[0]
    _reject_repeats([int(d) for t in dst_tables for d in t if 0 <= int(d) < nbd], "destination block")
    err = 0
    for l in range(len(out)):
        for r in range(len(src_tables)):
            for j in range(len(src_tables[r])):
                s, d = int(src_tables[r][j]), int(dst_tables[r][j])
                if s < 0 or s >= nbs or d < 0 or d >= nbd:
                    err |= DEVERR_BLOCK_RANGE
                    continue
                out[l][d] = srcs[l][s]
    return out, err


# ---------------------------------------------------------------------------------------
# f1 — kv-first caches: (K/V plane, blocks, block_size, heads, head_dim)
# ---------------------------------------------------------------------------------------

def _planes(cache: np.ndarray) -> np.ndarray:
    """A kv-first layer cache viewed as [2][num_blocks][segment bytes] uint8."""
    c = np.ascontiguousarray(cache)
    return c.reshape(2, c.shape[1], -1).view(np.uint8)


def pack_kv_first(layer_caches: Sequence[np.ndarray], src_tables: Sequence[np.ndarray]
                  ) -> Tuple[np.ndarray, int]:
    """Gather from kv-first caches. For each layer and each request r, the buffer holds the
    request's blocks as the gather over the block axis returns them: every listed block's K
    segment in table order, then every listed block's V segment. [nccl] §2.4
    (extract_kv_from_layer indexes dimension 1 when the K/V dimension comes first); [v1] the
    two "shape of layer i" layouts (reading: kv-first = (2, blocks, ...)).

    Buffer layout: [L][sum over r of 2*n_r][segment bytes]; request r starts at segment
    2*(blocks of earlier requests). Out-of-range ids are skipped (zeros) and raise
    DEVERR_BLOCK_RANGE.
    """
    planes = [_planes(c) for c in layer_caches]
    L = len(planes)
    _, nb, seg = planes[0].shape
    N = sum(len(t) for t in src_tables)
    buf = np.zeros((L, 2 * N, seg), np.uint8)
    err = 0
    for l in range(L):
        at = 0
        for t in src_tables:
            for kv in range(2):
                for b in t:
                    b = int(b)
                    if 0 <= b < nb:
                        buf[l, at] = planes[l][kv, b]
                    else:
                        err |= DEVERR_BLOCK_RANGE
                    at += 1
    return buf, err


def unpack_kv_first(buf: np.ndarray, dst_caches: Sequence[np.ndarray],
                    dst_tables: Sequence[np.ndarray]) -> Tuple[List[np.ndarray], int]:
    """Inverse of pack_kv_first into the receiver's kv-first caches: request r's K segments
    go to plane 0 of its destination blocks in table order, then its V segments to plane 1.
    [nccl] §2.3 step 14 / §2.4 (inject_kv_into_layer). Unlisted blocks keep their bytes;
    out-of-range destination ids are skipped and raise DEVERR_BLOCK_RANGE; an in-range
    destination id listed twice is invalid input (ValueError), as for unpack."""
    out = [_planes(c).copy() for c in dst_caches]
    L = len(out)
    _, nb, seg = out[0].shape
    _reject_repeats([int(d) for t in dst_tables for d in t if 0 <= int(d) < nb], "destination block")
    N = sum(len(t) for t in dst_tables)
    src = np.ascontiguousarray(buf).reshape(-1).view(np.uint8).reshape(L, 2 * N, seg)
    err = 0
    for l in range(L):
        at = 0
        for t in dst_tables:
            for kv in range(2):
                for d in t:
                    d = int(d)
                    if 0 <= d < nb:
                        out[l][kv, d] = src[l, at]
                    else:
                        err |= DEVERR_BLOCK_RANGE
                    at += 1
    return out, err


# ---------------------------------------------------------------------------------------
# f2 — sender-side head split (the inverse of the receiver's head merge)
# ---------------------------------------------------------------------------------------

def split_block(block: np.ndarray, num_dst: int, rows_per_block: int) -> List[np.ndarray]:
    """Cut one full-head block into num_dst head shards: shard d's row k is the d-th of
    num_dst equal pieces of the block's row k. [pd] §四 4.2 (TP heterogeneity). Reading:
    receiver rank d owns heads [d*H/num_dst, (d+1)*H/num_dst)."""
    b = np.ascontiguousarray(block).reshape(-1).view(np.uint8)
    row = len(b) // rows_per_block
    piece = row // num_dst
    shards = [np.empty(rows_per_block * piece, np.uint8) for _ in range(num_dst)]
    for k in range(rows_per_block):
        for d in range(num_dst):
            shards[d][k * piece:(k + 1) * piece] = b[k * row + d * piece:k * row + (d + 1) * piece]
    return shards


def pack_split(layer_caches: Sequence[np.ndarray], src_tables: Sequence[np.ndarray],
               num_dst: int, rows_per_block: int) -> Tuple[List[np.ndarray], int]:
    """Pack for num_dst receiving ranks that each own a head shard: buffer d is
    [L][N][block_bytes/num_dst] in pack's order (layer, request, block-table order) and holds
    shard d of every listed block (split_block). Out-of-range ids are skipped (zeros) and
    raise DEVERR_BLOCK_RANGE."""
    caches = [_as_block_bytes(c) for c in layer_caches]
    L = len(caches)
    nb, bb = caches[0].shape
    order = buffer_order(src_tables)
    N = len(order)
    bufs = [np.zeros((L, N, bb // num_dst), np.uint8) for _ in range(num_dst)]
    err = 0
    for l in range(L):
        for r, j, p in order:
            b = int(src_tables[r][j])
            if b < 0 or b >= nb:
                err |= DEVERR_BLOCK_RANGE
                continue
            for d, shard in enumerate(split_block(caches[l][b], num_dst, rows_per_block)):
                bufs[d][l, p] = shard
    return bufs, err
