"""The C ABI without a GPU: the library loads, exports every function include/kvx.h
declares, and rejects bad arguments on the host before anything is enqueued."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvx.h")


@pytest.fixture(scope="module")
def kvx():
    from block_table_contiguous_amd import kvx as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvx_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "kvx_abi_version", "kvx_build_xfer_list", "kvx_pack", "kvx_reshape_and_cache",
        "kvx_slot_mapping", "kvx_status_string", "kvx_unpack", "kvx_pack_split",
        "kvx_pack_kv_first", "kvx_unpack_kv_first", "kvx_signal_add", "kvx_signal_wait",
        "kvx_copy_direct", "kvx_pack_signal", "kvx_copy_direct_signal", "kvx_pack_signal_noalloc"])


def test_every_declared_symbol_is_exported(kvx):
    for name in declared_functions():
        assert hasattr(kvx.LIB, name), name
        assert name in kvx.SIGNATURES, name


def test_status_strings(kvx):
    for code in range(5):
        s = kvx.kvx_status_string(code)
        assert s.startswith("kvx: ")
    assert "unknown" in kvx.kvx_status_string(99)
    assert kvx.kvx_abi_version() == 5


def test_xfer_struct_size(kvx):
    class Xfer(ctypes.Structure):
        _fields_ = [("src_block", ctypes.c_int64), ("dst_block", ctypes.c_int64),
                    ("buf_block", ctypes.c_int64), ("num_blocks", ctypes.c_int32), ("req", ctypes.c_int32)]
    assert ctypes.sizeof(Xfer) == kvx.XFER_BYTES == 32


P = 0x10000  # a fake, 16-byte aligned, non-null device address: never dereferenced here


def call(kvx, name, *args):
    return kvx._F[name](*args)


def test_pack_validation(kvx):
    ok = dict(bases=P, L=2, bb=8192, nb=100, x=P, cnt=P, n=10, buf=P)

    def pack(**kw):
        a = {**ok, **kw}
        return call(kvx, "kvx_pack", a["bases"], a["L"], a["bb"], a["nb"], a["x"], a["cnt"], a["n"],
                    a["buf"], None, None)
    assert pack(L=-1) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(bb=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(n=-5) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(n=1 << 31) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(bases=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(x=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(bb=8200) == kvx.KVX_ERR_MISALIGNED
    assert pack(buf=P + 8) == kvx.KVX_ERR_MISALIGNED
    # empty work is a no-op that never reaches the device
    assert pack(n=0, bases=None) == kvx.KVX_SUCCESS
    assert pack(L=0) == kvx.KVX_SUCCESS


def test_unpack_validation(kvx):
    def unpack(S=1, srcs=(P,), bases=P, L=2, bb=8192, nb=100, rows=1, x=P, cnt=P, n=10):
        arr = (ctypes.c_void_p * max(len(srcs), 1))(*srcs) if srcs is not None else None
        return call(kvx, "kvx_unpack", arr, S, bases, L, bb, nb, rows, x, cnt, n, None, None)
    assert unpack(S=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert unpack(S=9, srcs=(P,) * 9) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert unpack(rows=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert unpack(S=2, srcs=(P, P), rows=3, bb=64) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert unpack(S=2, srcs=(P, None), rows=32) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert unpack(S=2, srcs=(P, P + 16 * 3 + 8), rows=32) == kvx.KVX_ERR_MISALIGNED
    assert unpack(bb=8200) == kvx.KVX_ERR_MISALIGNED
    assert unpack(srcs=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert unpack(n=0) == kvx.KVX_SUCCESS


def test_build_validation(kvx):
    def build(src=P, dst=P, ro=P, R=2, n=10, mode=0, x=P, cap=10, cnt=P):
        return call(kvx, "kvx_build_xfer_list", src, dst, ro, R, n, mode, x, cap, cnt, None, None)
    assert build(mode=3) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert build(mode=-1) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert build(cap=9) == kvx.KVX_ERR_CAPACITY
    assert build(R=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert build(src=None, mode=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert build(dst=None, mode=1) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert build(dst=None, mode=2) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert build(cnt=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert build(ro=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert build(x=P + 4) == kvx.KVX_ERR_MISALIGNED
    assert build(x=P + 8) == kvx.KVX_ERR_MISALIGNED  # records are written as 16-byte vectors
    assert build(n=-1) == kvx.KVX_ERR_INVALID_ARGUMENT


def test_slot_and_reshape_validation(kvx):
    def slots(bt=P, R=4, W=8, stride=8, rq=P, pos=P, T=10, bs=16, out=P):
        return call(kvx, "kvx_slot_mapping", bt, R, W, stride, rq, pos, T, bs, out, None, None)
    assert slots(bs=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert slots(T=-1) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert slots(W=9) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert slots(out=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert slots(T=0, out=None) == kvx.KVX_SUCCESS

    def rc(k=P, ks=4096, v=P, vs=4096, T=10, row=2048, sm=P, c=P, nb=64, bs=16,
           bst=65536, tst=4096, kst=2048):
        return call(kvx, "kvx_reshape_and_cache", k, ks, v, vs, T, row, sm, c, nb, bs, bst, tst, kst,
                    None, None)
    assert rc(row=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert rc(bs=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert rc(sm=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert rc(k=P + 2) == kvx.KVX_ERR_MISALIGNED
    assert rc(row=2040) == kvx.KVX_ERR_MISALIGNED
    assert rc(kst=2056) == kvx.KVX_ERR_MISALIGNED
    assert rc(T=0) == kvx.KVX_SUCCESS


def test_split_and_kv_first_validation(kvx):
    def split(D=2, bufs=(P, P), L=2, bb=65536, nb=100, rows=32, x=P, cnt=P, n=10):
        arr = (ctypes.c_void_p * max(len(bufs), 1))(*bufs) if bufs is not None else None
        return call(kvx, "kvx_pack_split", P, L, bb, nb, rows, x, cnt, n, arr, D, None, None)
    assert split(D=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert split(D=9, bufs=(P,) * 9) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert split(rows=3) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert split(bufs=(P, None)) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert split(bufs=(P, P + 8)) == kvx.KVX_ERR_MISALIGNED
    assert split(n=0) == kvx.KVX_SUCCESS

    def kvf(fn, seg=4096, plane=4096 * 100, nb=100, ro=P, R=2, x=P, cnt=P, n=10, buf=P):
        if fn == "kvx_pack_kv_first":
            return call(kvx, fn, P, 2, seg, plane, nb, ro, R, x, cnt, n, buf, None, None)
        return call(kvx, fn, buf, P, 2, seg, plane, nb, ro, R, x, cnt, n, None, None)
    for fn in ("kvx_pack_kv_first", "kvx_unpack_kv_first"):
        assert kvf(fn, seg=512) == kvx.KVX_ERR_MISALIGNED
        assert kvf(fn, plane=8) == kvx.KVX_ERR_MISALIGNED
        assert kvf(fn, plane=4096 * 99) == kvx.KVX_ERR_INVALID_ARGUMENT  # V plane would overlap K
        assert kvf(fn, seg=0) == kvx.KVX_ERR_INVALID_ARGUMENT
        assert kvf(fn, ro=None) == kvx.KVX_ERR_INVALID_ARGUMENT
        assert kvf(fn, R=0) == kvx.KVX_ERR_INVALID_ARGUMENT
        assert kvf(fn, buf=P + 16 + 8) == kvx.KVX_ERR_MISALIGNED
        assert kvf(fn, n=0) == kvx.KVX_SUCCESS


def test_signal_validation(kvx):
    assert call(kvx, "kvx_signal_add", None, 1, None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert call(kvx, "kvx_signal_add", P + 4, 1, None) == kvx.KVX_ERR_MISALIGNED

    def wait(counter=P, value=1, timeout=1000):
        return call(kvx, "kvx_signal_wait", counter, value, timeout, None, None)
    assert wait(counter=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert wait(timeout=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert wait(timeout=-3) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert wait(timeout=60_000_001) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert wait(counter=P + 12) == kvx.KVX_ERR_MISALIGNED


def test_binding_rejects_undersized_tensors(kvx):
    """The binding checks sizes the C ABI cannot see, before any pointer is taken."""
    import torch
    bases = torch.zeros(2, dtype=torch.int64)
    x, c = torch.zeros((9, 4), dtype=torch.int64), torch.zeros(1, dtype=torch.int64)
    buf = torch.zeros(2 * 10 * 64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="run list"):
        kvx.kvx_pack(bases, 64, 100, x, c, 10, buf)  # 9 records for 10 blocks
    with pytest.raises(ValueError, match="run list"):
        kvx.kvx_unpack([buf], bases, 64, 100, 1, x, c, 10)
    x10 = torch.zeros((10, 4), dtype=torch.int64)
    with pytest.raises(ValueError, match="send_buf smaller"):
        kvx.kvx_pack(bases, 64, 100, x10, c, 10, buf[:-16])
    with pytest.raises(ValueError, match="send buffer is smaller"):
        kvx.kvx_unpack([buf, buf[:100]], bases, 64, 100, 2, x10, c, 10)
    with pytest.raises(TypeError):
        kvx.kvx_pack(bases, 64, 100, x10.int(), c, 10, buf)
    # run building: both id lists must list the same blocks
    ro = torch.tensor([0, 10], dtype=torch.int64)
    ids10, ids9 = torch.zeros(10, dtype=torch.int32), torch.zeros(9, dtype=torch.int32)
    with pytest.raises(ValueError, match="same number of blocks"):
        kvx.kvx_build_xfer_list(ids10, ids9, ro, kvx.MODE_DIRECT, x10, c)
    with pytest.raises(ValueError, match="num_reqs \\+ 1"):
        kvx.kvx_build_xfer_list(ids10, None, torch.zeros(0, dtype=torch.int64), kvx.MODE_PACK, x10, c)
    # slot mapping: a width limit past the table's columns would read past each row
    table = torch.zeros((1, 6), dtype=torch.int32)
    req, pos = torch.zeros(4, dtype=torch.int32), torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError, match="wider than the block table"):
        kvx.kvx_slot_mapping(table, req, pos, 16, torch.zeros(4, dtype=torch.int64), max_blocks_per_req=7)
    # new-token write: the geometry must stay inside kv_cache's storage
    cache = torch.zeros((4, 16, 2, 1, 128), dtype=torch.int16)  # 4 blocks of 8 KiB
    key = torch.zeros((3, 1, 128), dtype=torch.int16)
    slots = torch.zeros(3, dtype=torch.int64)
    with pytest.raises(ValueError, match="past the end of kv_cache"):
        kvx.kvx_reshape_and_cache(key, key, slots, cache, 5, 16, 8192, 512, 256)
    with pytest.raises(ValueError, match="past the end of kv_cache"):
        kvx.kvx_reshape_and_cache(key, key, slots, cache[1:], 4, 16, 8192, 512, 256)
    with pytest.raises(ValueError, match="past the end of kv_cache"):
        kvx.kvx_reshape_and_cache(key, key, slots, cache, 4, 16, 8192, 528, 256)
    with pytest.raises(ValueError, match="on the GPU"):  # the exact fit passes the size check
        kvx.kvx_reshape_and_cache(key, key, slots, cache, 4, 16, 8192, 512, 256)


def test_copy_direct_validation(kvx):
    def direct(sb=P, db=P, L=2, bb=8192, nbs=100, nbd=100, x=P, cnt=P, n=10):
        return call(kvx, "kvx_copy_direct", sb, db, L, bb, nbs, nbd, x, cnt, n, None, None)
    assert direct(L=-1) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert direct(bb=0) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert direct(nbd=-1) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert direct(n=1 << 31) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert direct(sb=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert direct(db=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert direct(x=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert direct(nbs=0) == kvx.KVX_ERR_INVALID_ARGUMENT  # nothing to read from
    assert direct(bb=8200) == kvx.KVX_ERR_MISALIGNED
    assert direct(n=0, sb=None) == kvx.KVX_SUCCESS


def test_signalling_copy_validation(kvx):
    """The pack and direct copy that carry a completion signal check the counter and the
    arrivals word first, then everything the plain calls check."""
    cnt, arr = 0x1000, 0x2000  # fake, suitably aligned device addresses: never dereferenced here

    def pack(lb=P, L=2, bb=8192, nb=100, x=P, c=P, n=10, buf=P, counter=cnt, arrivals=arr):
        return call(kvx, "kvx_pack_signal", lb, L, bb, nb, x, c, n, buf, counter, 1, arrivals, None, None)

    def direct(sb=P, db=P, L=2, bb=8192, nbs=100, nbd=100, x=P, c=P, n=10, counter=cnt, arrivals=arr):
        return call(kvx, "kvx_copy_direct_signal", sb, db, L, bb, nbs, nbd, x, c, n, counter, 1, arrivals,
                    None, None)

    for fn in (pack, direct):
        assert fn(counter=None) == kvx.KVX_ERR_INVALID_ARGUMENT
        assert fn(arrivals=None) == kvx.KVX_ERR_INVALID_ARGUMENT
        assert fn(counter=cnt + 4) == kvx.KVX_ERR_MISALIGNED
        assert fn(arrivals=arr + 64) == kvx.KVX_ERR_MISALIGNED
        assert fn(L=-1) == kvx.KVX_ERR_INVALID_ARGUMENT
        assert fn(bb=0) == kvx.KVX_ERR_INVALID_ARGUMENT
        assert fn(n=1 << 31) == kvx.KVX_ERR_INVALID_ARGUMENT
        assert fn(x=None) == kvx.KVX_ERR_INVALID_ARGUMENT
        assert fn(bb=8200) == kvx.KVX_ERR_MISALIGNED
    assert pack(buf=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(buf=P + 8) == kvx.KVX_ERR_MISALIGNED
    assert direct(sb=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert direct(nbs=0) == kvx.KVX_ERR_INVALID_ARGUMENT


def test_allocation_free_pack_validation(kvx):
    """The allocation-free signalling pack refuses a slot outside the library's array before
    anything else, then checks what kvx_pack_signal checks; none of this touches HIP."""
    def pack(slot=0, counter=0x1000, L=2, bb=8192, n=10, buf=P, x=P):
        return call(kvx, "kvx_pack_signal_noalloc", P, L, bb, 100, x, P, n, buf, counter, 1, slot, None, None)

    assert kvx.NOALLOC_SLOTS == 16
    assert pack(slot=-1) == kvx.KVX_ERR_CAPACITY
    assert pack(slot=16) == kvx.KVX_ERR_CAPACITY
    assert pack(slot=16, counter=None) == kvx.KVX_ERR_CAPACITY
    assert pack(counter=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(counter=0x1004) == kvx.KVX_ERR_MISALIGNED
    assert pack(L=-1) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(x=None) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert pack(bb=8200) == kvx.KVX_ERR_MISALIGNED
    assert pack(buf=P + 8) == kvx.KVX_ERR_MISALIGNED
    assert "scratch" in kvx.kvx_status_string(kvx.KVX_ERR_CAPACITY)


def test_byte_extents_past_the_limit(kvx):
    """Sizes whose byte extent passes KVX_MAX_EXTENT_BYTES (2^56) describe no real allocation;
    every entry point refuses them before anything else could form an overflowing offset,
    including products that overflow 64 bits. An extent exactly at the limit passes that check
    and meets the next one (here a misaligned buffer)."""
    M = 1 << 56
    bb = 1 << 17
    big_nb = M // bb + 1           # one block more than a cache at the limit
    assert kvx.MAX_EXTENT_BYTES == M

    def pack(fn="kvx_pack", nb=100, L=2, n=10, b=bb, buf=P):
        if fn == "kvx_pack":
            return call(kvx, fn, P, L, b, nb, P, P, n, buf, None, None)
        if fn == "kvx_pack_signal":
            return call(kvx, fn, P, L, b, nb, P, P, n, buf, 0x1000, 1, 0x2000, None, None)
        return call(kvx, fn, P, L, b, nb, P, P, n, buf, 0x1000, 1, 0, None, None)
    for fn in ("kvx_pack", "kvx_pack_signal", "kvx_pack_signal_noalloc"):
        assert pack(fn, nb=big_nb) == kvx.KVX_ERR_INVALID_ARGUMENT, fn
        assert pack(fn, nb=1 << 62, b=1 << 10) == kvx.KVX_ERR_INVALID_ARGUMENT, fn  # overflows int64
        assert pack(fn, L=2, n=1 << 30, b=1 << 26) == kvx.KVX_ERR_INVALID_ARGUMENT, fn  # buffer: 2^57
        assert pack(fn, nb=M // bb, buf=P + 8) == kvx.KVX_ERR_MISALIGNED, fn  # exactly at the limit

    def unpack(nb=100, n=10, b=bb, S=1):
        arr = (ctypes.c_void_p * S)(*([P] * S))
        return call(kvx, "kvx_unpack", arr, S, P, 2, b, nb, 32, P, P, n, None, None)
    assert unpack(nb=big_nb) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert unpack(nb=big_nb, S=2) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert unpack(n=1 << 30, b=1 << 26) == kvx.KVX_ERR_INVALID_ARGUMENT

    def direct(fn, nbs=100, nbd=100):
        if fn == "kvx_copy_direct":
            return call(kvx, fn, P, P, 2, bb, nbs, nbd, P, P, 10, None, None)
        return call(kvx, fn, P, P, 2, bb, nbs, nbd, P, P, 10, 0x1000, 1, 0x2000, None, None)
    for fn in ("kvx_copy_direct", "kvx_copy_direct_signal"):
        assert direct(fn, nbs=big_nb) == kvx.KVX_ERR_INVALID_ARGUMENT, fn
        assert direct(fn, nbd=big_nb) == kvx.KVX_ERR_INVALID_ARGUMENT, fn

    arr = (ctypes.c_void_p * 2)(P, P)
    assert call(kvx, "kvx_pack_split", P, 2, bb, big_nb, 32, P, P, 10, arr, 2, None, None) == \
        kvx.KVX_ERR_INVALID_ARGUMENT

    for fn in ("kvx_pack_kv_first", "kvx_unpack_kv_first"):
        def kvf(seg=4096, plane=4096 * 100, n=10):
            if fn == "kvx_pack_kv_first":
                return call(kvx, fn, P, 2, seg, plane, 100, P, 2, P, P, n, P, None, None)
            return call(kvx, fn, P, P, 2, seg, plane, 100, P, 2, P, P, n, None, None)
        assert kvf(plane=M) == kvx.KVX_ERR_INVALID_ARGUMENT, fn      # the V plane ends past 2^56
        assert kvf(n=1 << 30, seg=1 << 25, plane=(1 << 25) * 100) == kvx.KVX_ERR_INVALID_ARGUMENT, fn

    assert call(kvx, "kvx_slot_mapping", P, 4, 8, 1 << 55, P, P, 10, 16, P, None, None) == \
        kvx.KVX_ERR_INVALID_ARGUMENT

    def rc(T=10, nb=64, bst=65536, ks=4096):
        return call(kvx, "kvx_reshape_and_cache", P, ks, P, 4096, T, 2048, P, P, nb, 16, bst, 4096, 2048,
                    None, None)
    assert rc(nb=1 << 41) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert rc(nb=1 << 60, bst=1 << 20) == kvx.KVX_ERR_INVALID_ARGUMENT
    assert rc(T=1 << 50, ks=1 << 10) == kvx.KVX_ERR_INVALID_ARGUMENT


def _run_python(code, env_extra=None):
    import subprocess
    import sys

    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=120)


def test_binding_fails_loudly_without_the_library():
    """No fallback: without the built library the binding refuses to import."""
    r = _run_python("import block_table_contiguous_amd.kvx", {"KVX_SO_PATH": "/nonexistent/libkvx.so"})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "no fallback" in r.stderr


def test_product_path_never_imports_the_oracle():
    """The package and its binding load without touching the oracle or the input generators."""
    r = _run_python("import sys, block_table_contiguous_amd, block_table_contiguous_amd.kvx, "
                    "block_table_contiguous_amd.build; "
                    "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.') or m == 'workloads']; "
                    "print(bad); sys.exit(1 if bad else 0)")
    assert r.returncode == 0, r.stdout + r.stderr
