"""GPU parity for the widened layouts: kv-first caches (pack/unpack) and the sender-side
head split, byte for byte against the oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, host_bytes, kvx, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"start {request.node.name}")
    yield
    torch.cuda.synchronize()
    log(f"end {request.node.name}")


def _lists(K, src_tables, dst_tables):
    sid, ro = K.flatten_tables(src_tables, DEV)
    did, _ = K.flatten_tables(dst_tables, DEV)
    N = int(sum(len(t) for t in src_tables))
    xp, cp = K.new_xfer_list(N, DEV)
    xu, cu = K.new_xfer_list(N, DEV)
    K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp)
    K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu)
    return ro, xp, cp, xu, cu, N


def _kv_first_roundtrip(seed, L, nb, seg, lengths, bs=16, gap=0, corrupt=False):
    K = kvx()
    case = W.random_transfer(seed, L, nb, bs, 1, 8, lengths, with_caches=False)
    src_tables, dst_tables = case.src_tables, case.dst_tables
    if corrupt:
        src_tables = [t.copy() for t in src_tables]
        dst_tables = [t.copy() for t in dst_tables]
        src_tables[1][0] = nb + 3
        dst_tables[-1][-1] = -2
    rng = np.random.default_rng(seed)
    words = seg // 2
    # planes are (2, nb + gap, seg): plane stride (nb + gap) * seg, only nb blocks addressable
    src_h = [W.random_words(rng, (2, nb + gap, words)) for _ in range(L)]
    dst_h = [np.full((2, nb + gap, words), W.SENTINEL16, np.uint16) for _ in range(L)]
    src = [to_dev(a) for a in src_h]
    dst = [to_dev(a) for a in dst_h]
    ro, xp, cp, xu, cu, N = _lists(K, src_tables, dst_tables)
    buf = torch.zeros(L * 2 * N * seg, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    plane = (nb + gap) * seg
    K.kvx_pack_kv_first(K.layer_base_table(src), seg, plane, nb, ro, xp, cp, N, buf, err)
    K.kvx_unpack_kv_first(buf, K.layer_base_table(dst), seg, plane, nb, ro, xu, cu, N, err)
    torch.cuda.synchronize()
    # oracle: the addressable part of each plane is blocks [0, nb)
    exp_buf, e1 = O.pack_kv_first([a[:, :nb] for a in src_h], src_tables)
    exp_dst, e2 = O.unpack_kv_first(exp_buf, [a[:, :nb] for a in dst_h], dst_tables)
    assert np.array_equal(host_bytes(buf), exp_buf.reshape(-1)), "kv-first pack != oracle"
    for l in range(L):
        got = host_bytes(dst[l]).reshape(2, nb + gap, seg)
        assert np.array_equal(got[:, :nb], exp_dst[l]), f"kv-first unpack layer {l}"
        assert np.all(got[:, nb:].view(np.uint16) == W.SENTINEL16)  # the gap is untouched
    assert int(err.item()) == (e1 | e2)


@pytest.mark.parametrize("seg", [1024, 4096, 8192, 65536])
def test_kv_first_roundtrip_segments(seg):
    rng = np.random.default_rng(seg)
    lengths = [int(x) for x in rng.integers(0, 400, size=13)]
    lengths[2] = 0
    lengths[5] = 17
    nb = max(256, min(4000, (64 << 20) // (2 * seg)))
    while sum(W.blocks_for(n, 16) for n in lengths) * 3 > nb:
        lengths = lengths[:-1]
    _kv_first_roundtrip(seg, 3, nb, seg, lengths)


def test_kv_first_plane_gap_and_many_requests():
    rng = np.random.default_rng(5)
    lengths = [int(x) for x in rng.integers(0, 90, size=300)]
    _kv_first_roundtrip(6, 2, 9000, 2048, lengths, gap=37)


def test_kv_first_out_of_range():
    _kv_first_roundtrip(7, 2, 500, 4096, [40, 70, 0, 33], corrupt=True)


def _split_case(seed, S, H, D, bs=16, L=3, nb=300):
    K = kvx()
    rng = np.random.default_rng(seed)
    spec = W.PagedSpec(L, nb, bs, H, D)
    counts = [int(x) for x in rng.integers(0, 25, size=9)]
    src_tables = W.pop_tables(rng.permutation(nb), counts)
    dst_tables = W.pop_tables(rng.permutation(nb), counts)
    BB = spec.block_bytes
    src_h = [W.random_words(rng, (nb, BB // 2)) for _ in range(L)]
    src = [to_dev(a) for a in src_h]
    ro, xp, cp, xu, cu, N = _lists(K, src_tables, dst_tables)
    bufs = [torch.zeros(L * N * BB // S, dtype=torch.uint8, device=DEV) for _ in range(S)]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_pack_split(K.layer_base_table(src), BB, nb, bs * 2, xp, cp, N, bufs, err)
    torch.cuda.synchronize()
    exp, e = O.pack_split(src_h, src_tables, S, rows_per_block=bs * 2)
    for d in range(S):
        assert np.array_equal(host_bytes(bufs[d]), exp[d].reshape(-1)), f"shard {d}"
    assert int(err.item()) == e == 0
    # merging the shards on the receiver gives what a plain pack + unpack gives
    dst_h = np.full((nb, BB // 2), W.SENTINEL16, np.uint16)
    dst = [to_dev(dst_h) for _ in range(L)]
    K.kvx_unpack(bufs, K.layer_base_table(dst), BB, nb, bs * 2, xu, cu, N, err)
    torch.cuda.synchronize()
    plain, _ = O.unpack(list(exp), [dst_h] * L, dst_tables, rows_per_block=bs * 2)
    for l in range(L):
        assert np.array_equal(host_bytes(dst[l]).reshape(nb, BB), plain[l]), f"merge layer {l}"
    assert int(err.item()) == 0


@pytest.mark.parametrize("S,H,D", [(2, 8, 128), (4, 8, 128), (2, 4, 32), (3, 6, 64), (8, 8, 128)])
def test_split_then_merge(S, H, D):
    """Row pieces of 1 KiB and more take the one-batch kernels; 256 B and 128 B pieces the
    general path."""
    _split_case(S * 1000 + H * 10 + D, S, H, D)
