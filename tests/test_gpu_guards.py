"""Guard bands: every buffer a kernel reads or writes is placed inside a larger allocation whose
margins before and after hold a known byte, and the margins must be unchanged afterwards. The
cases aim at the edges: ids just outside the caches (-1, num_blocks), run lists filled to their
last record, record counts at the builder's tile and workgroup-cap boundaries, offsets that are
not a CSR, and slots just past the cache. The interiors are compared with the oracle as in the
other parity tests."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, check_runs_equal, host_bytes, kvx, log, to_dev

pytestmark = pytest.mark.gpu

GUARD = 4096
MARK = 0x5A


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"start {request.node.name}")
    yield
    torch.cuda.synchronize()
    log(f"end {request.node.name}")


class Guarded:
    """nbytes of device memory between two GUARD-byte margins of MARK."""

    def __init__(self, nbytes, init=None):
        self.n = int(nbytes)
        self.full = torch.full((self.n + 2 * GUARD,), MARK, dtype=torch.uint8, device=DEV)
        self.inner = self.full[GUARD:GUARD + self.n]
        if init is not None:
            self.inner.copy_(torch.from_numpy(np.ascontiguousarray(init).view(np.uint8).reshape(-1)).to(DEV))

    def check(self, what):
        h = self.full.cpu().numpy()
        assert np.all(h[:GUARD] == MARK), f"{what}: bytes written before the buffer"
        assert np.all(h[GUARD + self.n:] == MARK), f"{what}: bytes written after the buffer"

    def host(self):
        return host_bytes(self.inner)


def _layers(arrs, block_bytes):
    g = [Guarded(a.nbytes, a) for a in arrs]
    return g, kvx().layer_base_table([x.inner for x in g])


def _runs(N):
    g = Guarded(max(N, 1) * 32)
    return g, g.inner.view(torch.int64).view(max(N, 1), 4)


@pytest.mark.parametrize("N", [1, 2047, 2048, 2049, 6151, 2048 * 256 + 5])
@pytest.mark.parametrize("mode", ["pack", "unpack", "direct"])
def test_run_list_fills_exactly_its_array(N, mode):
    """Every position its own run (random ids, several requests), so the list uses all N
    records; N at one tile, the tile boundary, several tiles, and past the 256-workgroup cap."""
    K = kvx()
    rng = np.random.default_rng(N)
    ids = rng.permutation(4 * N).astype(np.int32)[:N]
    ids2 = rng.permutation(4 * N).astype(np.int32)[:N]
    cuts = np.sort(rng.choice(np.arange(1, N), size=min(5, N - 1), replace=False)) if N > 1 else []
    src_tables = np.split(ids, cuts)
    dst_tables = np.split(ids2, cuts)
    sid, ro = K.flatten_tables(src_tables, DEV)
    did, _ = K.flatten_tables(dst_tables, DEV)
    g, x = _runs(N)
    cnt = Guarded(8)
    c = cnt.inner.view(torch.int64)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    m = {"pack": K.MODE_PACK, "unpack": K.MODE_UNPACK, "direct": K.MODE_DIRECT}[mode]
    K.kvx_build_xfer_list(sid if m != K.MODE_UNPACK else None, did if m != K.MODE_PACK else None, ro, m, x, c, err)
    torch.cuda.synchronize()
    g.check("run list")
    cnt.check("run count")
    assert int(err.item()) == 0
    om = {"pack": O.MODE_PACK, "unpack": O.MODE_UNPACK, "direct": O.MODE_DIRECT}[mode]
    if N <= 6151:
        check_runs_equal(K, x, c, O.xfer_list(src_tables, dst_tables, om))
    else:
        assert int(c.item()) == len(O.xfer_list(src_tables, dst_tables, om))


def test_run_list_with_offsets_that_are_not_a_csr():
    """Offsets that decrease and overshoot: the offsets bit is raised and no record is written
    outside the array."""
    K = kvx()
    N = 3000
    ids = torch.from_numpy(np.random.default_rng(1).permutation(N).astype(np.int32)).to(DEV)
    for ro_h in ([0, 2500, 100, 2999, 3000], [0, 10, 20, 5000, 3000], [7, 1000, 2000, 2000, 3001]):
        ro = torch.tensor(ro_h, dtype=torch.int64, device=DEV)
        g, x = _runs(N)
        cnt = Guarded(8)
        c = cnt.inner.view(torch.int64)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        K.kvx_build_xfer_list(ids, None, ro, K.MODE_PACK, x, c, err)
        torch.cuda.synchronize()
        g.check(f"run list, offsets {ro_h}")
        cnt.check("run count")
        assert int(err.item()) & K.DEVERR_OFFSETS
        assert int(c.item()) >= 1  # the count itself is unspecified for such offsets


@pytest.mark.parametrize("block_bytes", [1024 * 8, 7680, 16 * 3])
def test_copies_stay_inside_their_buffers(block_bytes):
    """Pack, unpack and the direct copy with ids -1, num_blocks and num_blocks + 5 on either
    side: guards around every layer cache, the send buffer and the run arrays."""
    K = kvx()
    rng = np.random.default_rng(block_bytes)
    L, nb = 2, 40
    src_tables = [np.array([nb - 1, nb, 0, 1, -1, 7], np.int32), np.array([nb + 5, 3], np.int32)]
    dst_tables = [np.array([0, nb - 1, -1, nb, 12, 13], np.int32), np.array([nb + 5, 20], np.int32)]
    N = 8
    src_h = [W.random_words(rng, (nb, block_bytes // 2)) for _ in range(L)]
    dst_h = [W.random_words(rng, (nb, block_bytes // 2)) for _ in range(L)]
    src, sbase = _layers(src_h, block_bytes)
    dst, dbase = _layers(dst_h, block_bytes)
    dst2, dbase2 = _layers(dst_h, block_bytes)
    sid, ro = K.flatten_tables(src_tables, DEV)
    did, _ = K.flatten_tables(dst_tables, DEV)
    lists = {}
    for name, m in (("pack", K.MODE_PACK), ("unpack", K.MODE_UNPACK), ("direct", K.MODE_DIRECT)):
        g, x = _runs(N)
        c = torch.zeros(1, dtype=torch.int64, device=DEV)
        K.kvx_build_xfer_list(sid if m != K.MODE_UNPACK else None, did if m != K.MODE_PACK else None, ro, m, x, c)
        lists[name] = (g, x, c)
    buf = Guarded(L * N * block_bytes, np.zeros(L * N * block_bytes, np.uint8))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_pack(sbase, block_bytes, nb, lists["pack"][1], lists["pack"][2], N, buf.inner, err)
    K.kvx_unpack([buf.inner], dbase, block_bytes, nb, 1, lists["unpack"][1], lists["unpack"][2], N, err)
    K.kvx_copy_direct(sbase, dbase2, block_bytes, nb, nb, lists["direct"][1], lists["direct"][2], N, err)
    torch.cuda.synchronize()
    for name, (g, _, _) in lists.items():
        g.check(f"{name} runs")
    buf.check("send buffer")
    for l in range(L):
        src[l].check(f"source layer {l}")
        dst[l].check(f"destination layer {l}")
        dst2[l].check(f"direct destination layer {l}")
    exp_buf, e1 = O.pack(src_h, src_tables)
    exp_dst, e2 = O.unpack([exp_buf], dst_h, dst_tables)
    exp_dir, e3 = O.copy_direct(src_h, dst_h, src_tables, dst_tables)
    assert np.array_equal(buf.host(), exp_buf.reshape(-1))
    for l in range(L):
        assert np.array_equal(dst[l].host().reshape(nb, block_bytes), exp_dst[l])
        assert np.array_equal(dst2[l].host().reshape(nb, block_bytes), exp_dir[l])
    assert int(err.item()) == (e1 | e2 | e3) == O.DEVERR_BLOCK_RANGE


def test_kv_first_stays_inside_its_planes():
    K = kvx()
    rng = np.random.default_rng(5)
    L, nb, seg = 2, 30, 2048
    src_tables = [np.array([0, nb - 1, nb, -1, 4], np.int32), np.array([9], np.int32)]
    dst_tables = [np.array([nb - 1, 0, -1, nb, 6], np.int32), np.array([11], np.int32)]
    N = 6
    src_h = [W.random_words(rng, (2, nb, seg // 2)) for _ in range(L)]
    dst_h = [W.random_words(rng, (2, nb, seg // 2)) for _ in range(L)]
    src, sbase = _layers(src_h, seg)
    dst, dbase = _layers(dst_h, seg)
    sid, ro = K.flatten_tables(src_tables, DEV)
    did, _ = K.flatten_tables(dst_tables, DEV)
    xp, cp = K.new_xfer_list(N, DEV)
    xu, cu = K.new_xfer_list(N, DEV)
    K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp)
    K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu)
    buf = Guarded(L * 2 * N * seg, np.zeros(L * 2 * N * seg, np.uint8))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_pack_kv_first(sbase, seg, nb * seg, nb, ro, xp, cp, N, buf.inner, err)
    K.kvx_unpack_kv_first(buf.inner, dbase, seg, nb * seg, nb, ro, xu, cu, N, err)
    torch.cuda.synchronize()
    buf.check("kv-first buffer")
    for l in range(L):
        src[l].check(f"source planes {l}")
        dst[l].check(f"destination planes {l}")
    exp_buf, e1 = O.pack_kv_first(src_h, src_tables)
    exp_dst, e2 = O.unpack_kv_first(exp_buf, dst_h, dst_tables)
    assert np.array_equal(buf.host(), exp_buf.reshape(-1))
    for l in range(L):
        assert np.array_equal(dst[l].host().reshape(2, nb, seg), exp_dst[l])
    assert int(err.item()) == (e1 | e2) == O.DEVERR_BLOCK_RANGE


@pytest.mark.parametrize("H,D", [(8, 128), (4, 16)])
def test_split_and_merge_stay_inside_their_buffers(H, D):
    """Sender split and receiver merge (2 and 4 shards), ids just outside the caches."""
    K = kvx()
    rng = np.random.default_rng(H * D)
    L, nb, bs = 2, 24, 16
    BB = bs * 2 * H * D * 2
    tables = [np.array([0, nb - 1, nb, -1, 5], np.int32), np.array([nb + 2, 9, 10], np.int32)]
    N = 8
    src_h = [W.random_words(rng, (nb, BB // 2)) for _ in range(L)]
    dst_h = [W.random_words(rng, (nb, BB // 2)) for _ in range(L)]
    for S in (2, 4):
        src, sbase = _layers(src_h, BB)
        dst, dbase = _layers(dst_h, BB)
        ids, ro = K.flatten_tables(tables, DEV)
        xp, cp = K.new_xfer_list(N, DEV)
        xu, cu = K.new_xfer_list(N, DEV)
        K.kvx_build_xfer_list(ids, None, ro, K.MODE_PACK, xp, cp)
        K.kvx_build_xfer_list(None, ids, ro, K.MODE_UNPACK, xu, cu)
        shards = [Guarded(L * N * BB // S, np.zeros(L * N * BB // S, np.uint8)) for _ in range(S)]
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        K.kvx_pack_split(sbase, BB, nb, bs * 2, xp, cp, N, [s.inner for s in shards], err)
        K.kvx_unpack([s.inner for s in shards], dbase, BB, nb, bs * 2, xu, cu, N, err)
        torch.cuda.synchronize()
        for d, s in enumerate(shards):
            s.check(f"shard {d} of {S}")
        for l in range(L):
            src[l].check(f"source layer {l}")
            dst[l].check(f"destination layer {l}")
        exp_s, e1 = O.pack_split(src_h, tables, S, rows_per_block=bs * 2)
        exp_m, e2 = O.unpack(list(exp_s), dst_h, tables, rows_per_block=bs * 2)
        for d in range(S):
            assert np.array_equal(shards[d].host(), exp_s[d].reshape(-1))
        for l in range(L):
            assert np.array_equal(dst[l].host().reshape(nb, BB), exp_m[l])
        assert int(err.item()) == (e1 | e2) == O.DEVERR_BLOCK_RANGE


@pytest.mark.parametrize("row,T", [(256, 40), (256, 4200), (2048, 40), (4112, 30)])
def test_slots_and_write_stay_inside_their_buffers(row, T):
    """Slot mapping into a guarded output, then the new-token write (each of its three kernels)
    into a guarded cache, with slots -1, the last slot, and just past the cache."""
    K = kvx()
    rng = np.random.default_rng(row + T)
    bs = 16
    nb = -(-T // bs) + 2
    table = rng.permutation(nb).astype(np.int32)[None, :]
    pos = rng.permutation(nb * bs - 1)[:T].astype(np.int64)  # distinct, below the last slot
    pos[0] = nb * bs + 3       # past the table's width: slot -1
    pos[1] = nb * bs - 1       # the table's last slot
    req = np.zeros(T, np.int32)
    out = Guarded(T * 8)
    slots = out.inner.view(torch.int64)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_slot_mapping(to_dev(table), to_dev(req), to_dev(pos), bs, slots, err)
    torch.cuda.synchronize()
    out.check("slot mapping output")
    exp_slots, e1 = O.slot_mapping(table, req, pos, bs)
    assert np.array_equal(slots.cpu().numpy(), exp_slots) and int(err.item()) == e1
    s = exp_slots.copy()
    s[2] = nb * bs              # just past the cache
    key = W.random_words(rng, (T, row // 2))
    val = W.random_words(rng, (T, row // 2))
    cache_h = W.random_words(rng, (nb, bs, 2, row // 2))
    cache = Guarded(cache_h.nbytes, cache_h)
    err.zero_()
    K.kvx_reshape_and_cache(to_dev(key), to_dev(val), to_dev(s), cache.inner, nb, bs, bs * 2 * row, 2 * row, row, err)
    torch.cuda.synchronize()
    cache.check("cache")
    exp, e2 = O.reshape_and_cache(cache_h, key, val, s, nb, bs, bs * 2 * row, 2 * row, row)
    assert np.array_equal(cache.host(), exp)
    assert int(err.item()) == e2 == O.DEVERR_SLOT_RANGE
