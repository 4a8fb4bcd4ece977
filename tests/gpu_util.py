"""Device-side setup shared by the GPU parity tests.

Inputs come from `workloads`; expected values come only from `oracle` applied to host
copies of those inputs (or to the oracle's own earlier outputs), never from the HIP path.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as W

DEV = "cuda:0"


def log(msg: str):
    print(f"[kvx-test] {msg}", flush=True)
    sys.stdout.flush()


def kvx():
    from block_table_contiguous_amd import kvx as K
    return K


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_bytes(t: torch.Tensor) -> np.ndarray:
    """Flat uint8 host copy of a device tensor's bytes."""
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


class HostStage:
    """Reusable pinned host buffers for streaming large device tensors to the host one at a
    time (a 1.125 GiB layer at a time for the full-size checks). get() returns a numpy view
    of the slot's buffer; it stays valid until the next get() on the same slot."""

    def __init__(self):
        self._bufs = {}

    def get(self, t: torch.Tensor, slot: int = 0) -> np.ndarray:
        flat = t.detach().contiguous().view(-1).view(torch.uint8)
        n = flat.numel()
        b = self._bufs.get(slot)
        if b is None or b.numel() < n:
            self._bufs.pop(slot, None)
            b = torch.empty(max(n, 1), dtype=torch.uint8, pin_memory=True)
            self._bufs[slot] = b
        b[:n].copy_(flat, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        return b[:n].numpy()


def same_bytes(got: np.ndarray, want: np.ndarray) -> bool:
    """Byte-for-byte equality of two arrays of equal byte size, compared in 64-bit words and
    256 MiB pieces so a 1 GiB layer needs no 1 GiB temporary."""
    a = np.ascontiguousarray(got).reshape(-1).view(np.uint8)
    b = np.ascontiguousarray(want).reshape(-1).view(np.uint8)
    if a.size != b.size:
        return False
    if a.size % 8 == 0:
        a, b = a.view(np.uint64), b.view(np.uint64)
    step = 1 << 25
    return all(np.array_equal(a[i:i + step], b[i:i + step]) for i in range(0, a.size, step))


def reshape_and_cache_raw(K, key, value, slots, cache, num_blocks, block_size, block_stride,
                          token_stride, kv_stride, err):
    """The new-token write through the C entry point itself, skipping the binding's geometry
    check. For geometries whose blocks overlap on purpose (2^30-slot blocks 64 KiB apart, to
    reach slots past 2^31 without a 512 GiB cache): the binding bounds the addressed bytes by
    the geometry, while these tests keep every slot inside the allocation, which is what the
    C entry point asks of its caller."""
    T = slots.numel()
    row = key.numel() // T * key.element_size()
    st = K._F["kvx_reshape_and_cache"](key.data_ptr(), row, value.data_ptr(), row, T, row, slots.data_ptr(),
                                       cache.data_ptr(), int(num_blocks), int(block_size), int(block_stride),
                                       int(token_stride), int(kv_stride), err.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == K.KVX_SUCCESS, st


def layers_from_host(arrs, block_bytes):
    """Per-layer uint8 [num_blocks][block_bytes] device tensors (separate allocations)."""
    return [to_dev(np.ascontiguousarray(a).view(np.uint8).reshape(-1, block_bytes)) for a in arrs]


class Transfer:
    """A pack -> unpack round trip on the device for one TransferCase."""

    def __init__(self, case: W.TransferCase, src_layers, dst_layers):
        K = kvx()
        self.K = K
        self.case = case
        self.src = src_layers
        self.dst = dst_layers
        self.L = len(src_layers)
        self.BB = case.src_spec.block_bytes
        self.nb_src = case.src_spec.num_blocks
        self.nb_dst = case.dst_spec.num_blocks
        self.N = case.total_blocks
        self.src_bases = K.layer_base_table(src_layers)
        self.dst_bases = K.layer_base_table(dst_layers)
        self.src_ids, self.offsets = K.flatten_tables(case.src_tables, DEV)
        self.dst_ids, _ = K.flatten_tables(case.dst_tables, DEV)
        self.xp, self.cp = K.new_xfer_list(self.N, DEV)
        self.xu, self.cu = K.new_xfer_list(self.N, DEV)
        self.buf = torch.empty(max(self.L * self.N * self.BB, 16), dtype=torch.uint8, device=DEV)
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)

    def build(self):
        K = self.K
        K.kvx_build_xfer_list(self.src_ids, None, self.offsets, K.MODE_PACK, self.xp, self.cp, self.err)
        K.kvx_build_xfer_list(None, self.dst_ids, self.offsets, K.MODE_UNPACK, self.xu, self.cu, self.err)

    def pack(self):
        self.K.kvx_pack(self.src_bases, self.BB, self.nb_src, self.xp, self.cp, self.N, self.buf, self.err)

    def unpack(self):
        self.K.kvx_unpack([self.buf], self.dst_bases, self.BB, self.nb_dst, 1, self.xu, self.cu, self.N,
                          self.err)

    def run(self):
        self.build()
        self.pack()
        self.unpack()
        torch.cuda.synchronize()

    def err_bits(self) -> int:
        return int(self.err.item())


def check_runs_equal(K, xfers, count, expected):
    got = K.decode_xfers(xfers, count)
    assert len(got) == len(expected), (len(got), len(expected))
    for i, (g, e) in enumerate(zip(got, expected)):
        assert g == tuple(e), (i, g, e)
