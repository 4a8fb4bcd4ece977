"""GPU parity for the direct cache-to-cache transfer: run lists built in KVX_MODE_DIRECT, then
every listed block of every layer copied from the source caches into the destination caches,
byte for byte against the oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, check_runs_equal, host_bytes, kvx, layers_from_host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"start {request.node.name}")
    yield
    torch.cuda.synchronize()
    log(f"end {request.node.name}")


def _direct_case(src_tables, dst_tables, src_caches, dst_caches, block_bytes):
    K = kvx()
    L = len(src_caches)
    src = layers_from_host(src_caches, block_bytes)
    dst = layers_from_host(dst_caches, block_bytes)
    nbs, nbd = src[0].shape[0], dst[0].shape[0]
    sid, ro = K.flatten_tables(src_tables, DEV)
    did, _ = K.flatten_tables(dst_tables, DEV)
    N = int(sum(len(t) for t in src_tables))
    x, c = K.new_xfer_list(N, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(sid, did, ro, K.MODE_DIRECT, x, c, err)
    K.kvx_copy_direct(K.layer_base_table(src), K.layer_base_table(dst), block_bytes, nbs, nbd, x, c, N, err)
    torch.cuda.synchronize()
    check_runs_equal(K, x, c, O.xfer_list(src_tables, dst_tables, O.MODE_DIRECT))
    exp, e = O.copy_direct(src_caches, dst_caches, src_tables, dst_tables)
    for l in range(L):
        assert np.array_equal(host_bytes(dst[l]).reshape(nbd, block_bytes), exp[l]), f"layer {l}"
    assert int(err.item()) == e
    return e


GEOMS = [  # (block_size, heads, head_dim, elem_bytes)
    (16, 2, 16, 2),    # 2 KiB
    (4, 1, 8, 2),      # 128 B
    (1, 1, 8, 1),      # 16 B
    (16, 8, 128, 2),   # 64 KiB
    (16, 1, 128, 2),   # 8 KiB
    (16, 3, 40, 2),    # 7680 B, not whole KiB
]


@pytest.mark.parametrize("geom", GEOMS, ids=[f"bs{g[0]}h{g[1]}d{g[2]}e{g[3]}" for g in GEOMS])
def test_direct_geometries(geom):
    bs, H, D, e = geom
    spec = W.PagedSpec(3, 1, bs, H, D, e)
    nb = max(64, min(5000, (32 << 20) // spec.block_bytes))
    rng = np.random.default_rng(sum(geom) * 7 + 1)
    lengths = [int(x) for x in rng.integers(0, bs * 40, size=19)]
    lengths[2] = 0
    while sum(W.blocks_for(n, bs) for n in lengths) * 3 > nb:
        lengths = lengths[:-1]
    c = W.random_transfer(int(rng.integers(1 << 30)), 3, nb, bs, H, D, lengths, elem_bytes=e)
    assert _direct_case(c.src_tables, c.dst_tables, c.src_caches, c.dst_caches, spec.block_bytes) == 0


def test_direct_contiguous_both_sides_and_unequal_caches():
    """Long runs consecutive on both sides (each request's blocks sit in order in both caches)
    between caches of different sizes."""
    rng = np.random.default_rng(12)
    L, bb, nbs, nbd = 2, 8192, 900, 1300
    counts = [130, 0, 77, 200, 1]
    src_tables, dst_tables, a, b = [], [], 10, 400
    for n in counts:
        src_tables.append(np.arange(a, a + n, dtype=np.int32))
        dst_tables.append(np.arange(b, b + n, dtype=np.int32))
        a += n + 3
        b += n + 11
    src = [W.random_words(rng, (nbs, bb // 2)) for _ in range(L)]
    dst = [np.full((nbd, bb // 2), W.SENTINEL16, np.uint16) for _ in range(L)]
    assert _direct_case(src_tables, dst_tables, src, dst, bb) == 0


def test_direct_shared_prefix_and_out_of_range():
    """Requests sharing source blocks, and ids out of range on either side (skipped, flagged)."""
    rng = np.random.default_rng(13)
    L, bb, nb = 2, 2048, 300
    shared = np.arange(40, 52, dtype=np.int32)
    src_tables = [np.concatenate([shared, np.array(x, np.int32)]) for x in ([100, 101, 7], [200], [5, 6, 9])]
    perm = rng.permutation(nb).astype(np.int32)
    dst_tables, k = [], 0
    for t in src_tables:
        dst_tables.append(perm[k:k + len(t)].copy())
        k += len(t)
    src_tables[1][3] = nb + 5      # source out of range
    dst_tables[2][0] = -3          # destination out of range
    dst_tables[0][-1] = nb         # destination out of range
    src = [W.random_words(rng, (nb, bb // 2)) for _ in range(L)]
    dst = [np.full((nb, bb // 2), W.SENTINEL16, np.uint16) for _ in range(L)]
    assert _direct_case(src_tables, dst_tables, src, dst, bb) == O.DEVERR_BLOCK_RANGE


def test_direct_within_one_cache():
    """Source and destination are the same caches (a copy between blocks of one cache, as when
    a shared prefix is forked), with disjoint source and destination blocks."""
    K = kvx()
    rng = np.random.default_rng(14)
    L, bb, nb = 2, 4096, 800
    ids = rng.permutation(nb).astype(np.int32)
    src_ids, dst_ids = ids[:250], ids[250:500]
    src_tables = [src_ids[:100], src_ids[100:100], src_ids[100:250]]
    dst_tables = [dst_ids[:100], dst_ids[100:100], dst_ids[100:250]]
    caches_h = [W.random_words(rng, (nb, bb // 2)) for _ in range(L)]
    caches = layers_from_host(caches_h, bb)
    bases = K.layer_base_table(caches)
    sid, ro = K.flatten_tables(src_tables, DEV)
    did, _ = K.flatten_tables(dst_tables, DEV)
    x, c = K.new_xfer_list(250, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(sid, did, ro, K.MODE_DIRECT, x, c, err)
    K.kvx_copy_direct(bases, bases, bb, nb, nb, x, c, 250, err)
    torch.cuda.synchronize()
    exp, e = O.copy_direct(caches_h, caches_h, src_tables, dst_tables)
    assert e == 0 and int(err.item()) == 0
    for l in range(L):
        assert np.array_equal(host_bytes(caches[l]).reshape(nb, bb), exp[l]), f"layer {l}"
