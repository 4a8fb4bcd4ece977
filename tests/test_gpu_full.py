"""GPU parity at the full workload sizes, in the launch configuration the benchmark times:
48 layers of [147456][16][K,V][128] bf16 (1.125 GiB each, separate allocations), 8 requests x
576 blocks, contiguous (runs of 64) and fragmented (geometric run lengths) block tables,
unpacked into a second 48-layer cache at random ids. Three layers are checked in full against
the oracle; every layer is checked on sampled blocks the oracle places one by one."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, Transfer, check_runs_equal, host_bytes, kvx, log

pytestmark = [pytest.mark.gpu, pytest.mark.big]

FULL_LAYERS = (0, 23, 47)
SAMPLES = 384


@pytest.fixture(scope="module")
def pages_caches():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec = W.pages_contiguous().src_spec
    log(f"allocating 2 x {spec.num_layers} layers of {spec.layer_bytes} B")
    src = [torch.empty((spec.num_blocks, spec.block_bytes), dtype=torch.uint8, device=DEV)
           for _ in range(spec.num_layers)]
    dst = [torch.empty_like(src[0]) for _ in range(spec.num_layers)]
    for l, t in enumerate(src):
        W.fill_device_random_(t, W.CONTIG_SEED * 1000 + l)
    torch.cuda.synchronize()
    log("source caches filled")
    yield spec, src, dst
    del src, dst
    torch.cuda.empty_cache()


def _check_transfer(case, src, dst):
    spec = case.src_spec
    for t in dst:
        W.fill_device_byte_(t)
    tr = Transfer(case, src, dst)
    tr.run()
    log(f"{case.name}: transfer done, checking")
    assert tr.err_bits() == 0
    check_runs_equal(tr.K, tr.xp, tr.cp, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_PACK))
    check_runs_equal(tr.K, tr.xu, tr.cu, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_UNPACK))
    N, BB = tr.N, tr.BB
    buf = tr.buf.view(spec.num_layers, N, BB)
    for l in FULL_LAYERS:
        src_l = host_bytes(src[l]).reshape(spec.num_blocks, BB)
        exp_buf, e1 = O.pack([src_l], case.src_tables)
        assert np.array_equal(host_bytes(buf[l]).reshape(N, BB), exp_buf[0]), f"pack layer {l}"
        before = np.full((spec.num_blocks, BB), W.FILL_BYTE, np.uint8)
        exp_dst, e2 = O.unpack([exp_buf], [before], case.dst_tables)
        assert np.array_equal(host_bytes(dst[l]).reshape(spec.num_blocks, BB), exp_dst[0]), f"unpack layer {l}"
        assert e1 == e2 == 0
        log(f"{case.name}: layer {l} identical")
    order = O.buffer_order(case.src_tables)
    rng = np.random.default_rng(case.seed)
    listed = set(int(x) for x in np.concatenate(case.dst_tables))
    for _ in range(SAMPLES):
        l = int(rng.integers(spec.num_layers))
        r, j, p = order[int(rng.integers(N))]
        s_id, d_id = int(case.src_tables[r][j]), int(case.dst_tables[r][j])
        want = host_bytes(src[l][s_id])
        assert np.array_equal(host_bytes(buf[l, p]), want), (l, p)
        assert np.array_equal(host_bytes(dst[l][d_id]), want), (l, d_id)
        free = int(rng.integers(spec.num_blocks))
        if free not in listed:
            assert np.all(host_bytes(dst[l][free]) == W.FILL_BYTE), (l, free)
    log(f"{case.name}: {SAMPLES} sampled blocks identical")


def test_pages_contiguous_full(pages_caches):
    spec, src, dst = pages_caches
    _check_transfer(W.pages_contiguous(), src, dst)


def test_pages_fragmented_full(pages_caches):
    spec, src, dst = pages_caches
    _check_transfer(W.pages_fragmented(), src, dst)


def test_pages_contiguous_kv_first_full(pages_caches):
    """The same 48 allocations viewed as kv-first caches (K plane, V plane) of 147456 blocks
    with 4 KiB segments: pack and unpack through the kv-first entry points."""
    spec, src, dst = pages_caches
    case = W.pages_contiguous()
    K = kvx()
    nb, seg, L = spec.num_blocks, spec.block_bytes // 2, spec.num_layers
    for t in dst:
        W.fill_device_byte_(t)
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    did, _ = K.flatten_tables(case.dst_tables, DEV)
    N = case.total_blocks
    xp, cp = K.new_xfer_list(N, DEV)
    xu, cu = K.new_xfer_list(N, DEV)
    buf = torch.empty(L * 2 * N * seg, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp, err)
    K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu, err)
    K.kvx_pack_kv_first(K.layer_base_table(src), seg, nb * seg, nb, ro, xp, cp, N, buf, err)
    K.kvx_unpack_kv_first(buf, K.layer_base_table(dst), seg, nb * seg, nb, ro, xu, cu, N, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    bufv = buf.view(L, 2 * N, seg)
    for l in FULL_LAYERS:
        src_l = host_bytes(src[l]).reshape(2, nb, seg)
        exp_buf, e1 = O.pack_kv_first([src_l], case.src_tables)
        assert np.array_equal(host_bytes(bufv[l]).reshape(2 * N, seg), exp_buf[0]), f"kv-first pack layer {l}"
        before = np.full((2, nb, seg), W.FILL_BYTE, np.uint8)
        exp_dst, e2 = O.unpack_kv_first(exp_buf, [before], case.dst_tables)
        assert np.array_equal(host_bytes(dst[l]).reshape(2, nb, seg), exp_dst[0]), f"kv-first unpack layer {l}"
        assert e1 == e2 == 0
        log(f"kv-first: layer {l} identical")
    # where each (plane, source block) lands in a layer's buffer, as the oracle places it:
    # pack a tag cache whose segment (kv, b) holds the number kv*nb + b
    tags = (np.arange(2 * nb, dtype=np.int64).reshape(2, nb, 1)).view(np.uint8)
    tag_buf, _ = O.pack_kv_first([tags], case.src_tables)
    where = tag_buf[0].copy().view(np.int64).reshape(-1)  # segment g -> kv*nb + source id
    pos_of_src = {int(v): g for g, v in enumerate(where)}
    src_to_dst = {int(s): int(d) for s, d in zip(np.concatenate(case.src_tables), np.concatenate(case.dst_tables))}
    rng = np.random.default_rng(7)
    for _ in range(SAMPLES):
        l = int(rng.integers(L))
        g = int(rng.integers(2 * N))
        kv, s_id = divmod(int(where[g]), nb)
        d_id = src_to_dst[s_id]
        want = host_bytes(src[l].view(2, nb, seg)[kv, s_id])
        assert pos_of_src[kv * nb + s_id] == g
        assert np.array_equal(host_bytes(bufv[l, g]), want), (l, g)
        assert np.array_equal(host_bytes(dst[l].view(2, nb, seg)[kv, d_id]), want), (l, g, d_id)
    log(f"kv-first: {SAMPLES} sampled segments identical")
