"""Seeded synthetic inputs for the paged KV-cache transfer path.

This module only *makes inputs*: cache geometry, per-request block tables,
destination block ids, token lengths and the byte contents of caches and new
K/V rows. It contains no step of the method itself (no slot arithmetic, no
gather, no scatter, no run coalescing), so both the CPU oracle and the HIP
path can take their inputs from here without sharing any of the method.

Shapes follow the pages' workload:
  * 16-token blocks, one block table shared by every layer, per-layer caches
    that are separate allocations ("vllm v1 调度逻辑 和 distributed 分布式原理",
    KV-memory diagram: 48 layer tensors of 147456 blocks, 1.125 GiB each);
  * 8 requests of 576 blocks (same diagram, scheduler-step label);
  * block ids handed out from a shuffled free pool (same diagram, prefix-cache
    toy with its free-block queue).

Random values the caches hold are drawn here from numpy's PCG64 (host) or from
a seeded torch generator on the device (large caches). The oracle never needs
the two to agree: it always reads the actual input bytes.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

# 0xFFFF is a NaN bit pattern in both fp16 and bf16; no finite draw produces it.
SENTINEL16 = 0xFFFF
# Byte used to pre-fill large destination caches (fast device fill).
FILL_BYTE = 0xA5


@dataclasses.dataclass(frozen=True)
class PagedSpec:
    """Geometry of one layer's paged cache in the [blocks][block_size][K,V][heads][head_dim]
    layout. All sizes are in elements except the *_bytes properties."""

    num_layers: int
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    elem_bytes: int = 2

    @property
    def row_bytes(self) -> int:
        """Bytes of one token's K (or V) row: heads x head_dim x element."""
        return self.num_kv_heads * self.head_dim * self.elem_bytes

    @property
    def block_bytes(self) -> int:
        return self.block_size * 2 * self.row_bytes

    @property
    def layer_bytes(self) -> int:
        return self.num_blocks * self.block_bytes

    @property
    def shape5(self):
        return (self.num_blocks, self.block_size, 2, self.num_kv_heads, self.head_dim)


@dataclasses.dataclass
class TransferCase:
    """Inputs of one pack -> unpack round trip.

    src_tables[r] are request r's block ids in the sender's cache, in block-table order;
    dst_tables[r] are the receiver's freshly allocated ids for the same blocks.
    src_caches / dst_caches are filled only for host-sized cases (None otherwise).
    """

    name: str
    src_spec: PagedSpec
    dst_spec: PagedSpec
    lengths: List[int]
    src_tables: List[np.ndarray]
    dst_tables: List[np.ndarray]
    seed: int
    num_src: int = 1
    rows_per_block: int = 1
    src_caches: Optional[List[np.ndarray]] = None
    dst_caches: Optional[List[np.ndarray]] = None
    # for head-split cases: the per-source packed buffers [L][N][block_bytes/num_src]
    src_buffers: Optional[List[np.ndarray]] = None

    @property
    def total_blocks(self) -> int:
        return int(sum(len(t) for t in self.src_tables)) if self.src_tables else \
            int(sum(len(t) for t in self.dst_tables))


# ----------------------------------------------------------------------------------------
# value generators
# ----------------------------------------------------------------------------------------

def fp16_uniform_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """uniform(-1, 1) float32 draws rounded to fp16 (numpy round-to-nearest-even), as uint16."""
    return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32).astype(np.float16).view(np.uint16)


def bf16_normal_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """normal(0, 1) float32 draws rounded to bf16 with round-to-nearest-even on the bit
    pattern, as uint16. (Finite draws only, so no NaN handling is needed.)"""
    f = rng.standard_normal(size=shape, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform random 16-bit words (any bit pattern, NaNs included)."""
    return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def fill_device_random_(tensor, seed: int):
    """Fill a device tensor (any dtype) with seeded uniform random 16-bit words, in place.
    Used for caches too large to generate on the host."""
    import torch

    flat = tensor.view(-1).view(torch.int16)
    g = torch.Generator(device=tensor.device)
    g.manual_seed(int(seed))
    chunk = 1 << 28  # 512 MiB of int16 per draw keeps the temporary small
    for s in range(0, flat.numel(), chunk):
        part = flat[s:s + chunk]
        part.random_(-32768, 32768, generator=g)
    return tensor


def fill_device_byte_(tensor, byte: int = FILL_BYTE):
    import torch

    tensor.view(-1).view(torch.uint8).fill_(byte)
    return tensor


# ----------------------------------------------------------------------------------------
# block-table generators
# ----------------------------------------------------------------------------------------

def blocks_for(length: int, block_size: int) -> int:
    """Number of blocks a request of `length` tokens occupies (whole blocks, last one
    partly filled)."""
    return (int(length) + block_size - 1) // block_size


def pop_tables(pool: np.ndarray, counts) -> List[np.ndarray]:
    """Hand out ids from a shuffled free pool, front first, `counts[r]` ids per request."""
    out, at = [], 0
    for c in counts:
        out.append(np.asarray(pool[at:at + c], dtype=np.int32).copy())
        at += c
    if at > len(pool):
        raise ValueError("free pool exhausted")
    return out


def contiguous_tables(rng: np.random.Generator, num_blocks: int, num_reqs: int,
                      blocks_per_req: int, run: int) -> List[np.ndarray]:
    """Block tables made of `blocks_per_req / run` runs of `run` consecutive ids; each run
    sits in its own run-aligned slot, slots drawn without replacement."""
    if blocks_per_req % run:
        raise ValueError("blocks_per_req must be a multiple of run")
    per_req = blocks_per_req // run
    slots = rng.permutation(num_blocks // run)[: num_reqs * per_req]
    tables = []
    for r in range(num_reqs):
        ids = [np.arange(s * run, (s + 1) * run) for s in slots[r * per_req:(r + 1) * per_req]]
        tables.append(np.concatenate(ids).astype(np.int32))
    return tables


def fragmented_tables(rng: np.random.Generator, num_blocks: int, num_reqs: int,
                      blocks_per_req, slot: int = 32, p: float = 0.5) -> List[np.ndarray]:
    """Block tables whose runs have geometric(p) lengths (support >= 1), capped at `slot`
    and truncated to the request's size. Each run lives in its own `slot`-block slot (slots
    drawn without replacement) at a random offset, so ids never repeat. `blocks_per_req` is
    one count for every request or a list of per-request counts."""
    counts = list(blocks_per_req) if np.ndim(blocks_per_req) else [int(blocks_per_req)] * num_reqs
    order = rng.permutation(num_blocks // slot)
    at = 0
    tables = []
    for left in counts:
        ids = []
        while left > 0:
            if at >= len(order):
                raise ValueError("not enough free slots for the requested runs")
            n = int(min(rng.geometric(p), slot, left))
            s = int(order[at])
            at += 1
            off = int(rng.integers(0, slot - n + 1))
            ids.append(np.arange(s * slot + off, s * slot + off + n))
            left -= n
        tables.append(np.concatenate(ids).astype(np.int32) if ids else np.zeros(0, np.int32))
    return tables


def pad_table(tables: List[np.ndarray], width: int, pad: int = -1) -> np.ndarray:
    """Per-request id lists as one [num_reqs][width] int32 table padded with `pad`."""
    t = np.full((len(tables), width), pad, dtype=np.int32)
    for r, ids in enumerate(tables):
        t[r, :len(ids)] = ids
    return t


# ----------------------------------------------------------------------------------------
# the five workloads (sizes overridable so host tests can run scaled-down copies)
# ----------------------------------------------------------------------------------------

TINY_SEED, DECODE_SEED, CONTIG_SEED, FRAG_SEED, ASYM_SEED = 1001, 1002, 1003, 1004, 1005


def tiny_roundtrip(seed: int = TINY_SEED) -> TransferCase:
    """2 layers of [64][16][K,V][2][16] fp16 uniform(-1,1); requests of 17, 40 and 5 tokens;
    source ids popped from one shuffled pool, destination ids from a second one."""
    spec = PagedSpec(num_layers=2, num_blocks=64, block_size=16, num_kv_heads=2, head_dim=16)
    rng = np.random.default_rng(seed)
    lengths = [17, 40, 5]
    counts = [blocks_for(n, spec.block_size) for n in lengths]
    src_tables = pop_tables(rng.permutation(spec.num_blocks), counts)
    dst_tables = pop_tables(rng.permutation(spec.num_blocks), counts)
    src_caches = [fp16_uniform_bits(rng, spec.shape5) for _ in range(spec.num_layers)]
    dst_caches = [np.full(spec.shape5, SENTINEL16, np.uint16) for _ in range(spec.num_layers)]
    return TransferCase("tiny", spec, spec, lengths, src_tables, dst_tables, seed,
                        src_caches=src_caches, dst_caches=dst_caches)


@dataclasses.dataclass
class DecodeWriteCase:
    """Inputs of slot_mapping + the new-token K/V write."""

    spec: PagedSpec
    lengths: List[int]
    tables: List[np.ndarray]
    block_table: np.ndarray      # [num_reqs][max_blocks] int32, padded with -1
    req_idx: np.ndarray          # [T] int32, request-major
    positions: np.ndarray        # [T] int64, 0..len_r-1 within each request
    key: Optional[np.ndarray]    # [T][H][D] uint16 bit patterns
    value: Optional[np.ndarray]
    seed: int


def decode_write(seed: int = DECODE_SEED, num_reqs: int = 32, max_len: int = 2048,
                 num_blocks: int = 4096, num_kv_heads: int = 8, head_dim: int = 128,
                 with_values: bool = True) -> DecodeWriteCase:
    """1 layer of [num_blocks][16][K,V][8][128] bf16 pre-filled with a sentinel; `num_reqs`
    requests with lengths uniform in [1, max_len]; tables popped from a shuffled pool; new
    K/V rows bf16 normal(0,1). Tokens are flat request-major with positions 0..len-1."""
    spec = PagedSpec(num_layers=1, num_blocks=num_blocks, block_size=16,
                     num_kv_heads=num_kv_heads, head_dim=head_dim)
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(1, max_len + 1, size=num_reqs)]
    counts = [blocks_for(n, spec.block_size) for n in lengths]
    if sum(counts) > num_blocks:
        raise ValueError("requests do not fit the cache")
    tables = pop_tables(rng.permutation(num_blocks), counts)
    width = blocks_for(max_len, spec.block_size)
    block_table = pad_table(tables, width)
    req_idx = np.concatenate([np.full(n, r, np.int32) for r, n in enumerate(lengths)])
    positions = np.concatenate([np.arange(n, dtype=np.int64) for n in lengths])
    key = value = None
    if with_values:
        T = len(req_idx)
        key = bf16_normal_bits(rng, (T, num_kv_heads, head_dim))
        value = bf16_normal_bits(rng, (T, num_kv_heads, head_dim))
    return DecodeWriteCase(spec, lengths, tables, block_table, req_idx, positions, key, value, seed)


def pages_contiguous(seed: int = CONTIG_SEED, num_layers: int = 48, num_blocks: int = 147456,
                     num_reqs: int = 8, blocks_per_req: int = 576, run: int = 64,
                     num_kv_heads: int = 1, head_dim: int = 128) -> TransferCase:
    """The pages' shape: 48 layers of [147456][16][K,V][128] bf16 (8 KiB blocks), 8 requests
    x 576 blocks in runs of 64; destination ids are the first N of a permutation of a second
    cache of the same shape. Cache contents are filled on the device."""
    spec = PagedSpec(num_layers, num_blocks, 16, num_kv_heads, head_dim)
    rng = np.random.default_rng(seed)
    src_tables = contiguous_tables(rng, num_blocks, num_reqs, blocks_per_req, run)
    dst_tables = pop_tables(rng.permutation(num_blocks), [blocks_per_req] * num_reqs)
    lengths = [blocks_per_req * spec.block_size] * num_reqs
    return TransferCase("contiguous", spec, spec, lengths, src_tables, dst_tables, seed)


def pages_fragmented(seed: int = FRAG_SEED, num_layers: int = 48, num_blocks: int = 147456,
                     num_reqs: int = 8, blocks_per_req: int = 576,
                     num_kv_heads: int = 1, head_dim: int = 128) -> TransferCase:
    """As pages_contiguous, but the source tables have geometric(0.5) run lengths (mean 2),
    mimicking churn after preemption and prefix-cache reuse."""
    spec = PagedSpec(num_layers, num_blocks, 16, num_kv_heads, head_dim)
    rng = np.random.default_rng(seed)
    src_tables = fragmented_tables(rng, num_blocks, num_reqs, blocks_per_req)
    dst_tables = pop_tables(rng.permutation(num_blocks), [blocks_per_req] * num_reqs)
    lengths = [blocks_per_req * spec.block_size] * num_reqs
    return TransferCase("fragmented", spec, spec, lengths, src_tables, dst_tables, seed)


def asym_tp(seed: int = ASYM_SEED, num_layers: int = 32, num_reqs: int = 16,
            blocks_per_req: int = 256, dst_blocks: int = 8192, num_kv_heads: int = 8,
            head_dim: int = 128, num_src: int = 2) -> TransferCase:
    """Receive side of a TP num_src -> 1 transfer: num_src packed send buffers, each holding
    num_kv_heads/num_src heads of every block ([L][N][16][K,V][H/num_src][D] bf16, random
    words, filled on the device), merged by head into a full-head destination cache at random
    destination ids (drawn from a pool twice the size needed)."""
    dst_spec = PagedSpec(num_layers, dst_blocks, 16, num_kv_heads, head_dim)
    src_spec = PagedSpec(num_layers, num_reqs * blocks_per_req, 16, num_kv_heads // num_src, head_dim)
    rng = np.random.default_rng(seed)
    dst_tables = pop_tables(rng.permutation(dst_blocks), [blocks_per_req] * num_reqs)
    lengths = [blocks_per_req * 16] * num_reqs
    return TransferCase("asym_tp", src_spec, dst_spec, lengths, [], dst_tables, seed,
                        num_src=num_src, rows_per_block=16 * 2)


def random_transfer(seed: int, num_layers: int, num_blocks: int, block_size: int,
                    num_kv_heads: int, head_dim: int, lengths, elem_bytes: int = 2,
                    run_p: float = 0.5, slot: Optional[int] = None,
                    with_caches: bool = True) -> TransferCase:
    """A host-sized random round trip: requests of the given token lengths (0 allowed), source
    tables with geometric(run_p) runs in random `slot`-block slots (by default the largest
    slot <= 8 that leaves one slot per block), destination ids from a permutation.
    Source caches random words; destination caches the sentinel."""
    spec = PagedSpec(num_layers, num_blocks, block_size, num_kv_heads, head_dim, elem_bytes)
    rng = np.random.default_rng(seed)
    counts = [blocks_for(n, block_size) for n in lengths]
    if sum(counts) > num_blocks:
        raise ValueError("requests do not fit the cache")
    if slot is None:
        slot = max(1, min(8, num_blocks // max(sum(counts), 1)))
    src_tables = fragmented_tables(rng, num_blocks, len(counts), counts, slot=slot, p=run_p)
    dst_tables = pop_tables(rng.permutation(num_blocks), counts)
    src_caches = dst_caches = None
    if with_caches:
        words = spec.block_bytes // 2
        src_caches = [random_words(rng, (num_blocks, words)) for _ in range(num_layers)]
        dst_caches = [np.full((num_blocks, words), SENTINEL16, np.uint16) for _ in range(num_layers)]
    return TransferCase(f"random{seed}", spec, spec, list(lengths), src_tables, dst_tables, seed,
                        src_caches=src_caches, dst_caches=dst_caches)
