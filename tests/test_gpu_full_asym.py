"""GPU parity at the full asymmetric-TP receive size: two send buffers, each holding 4 of 8
KV heads of 32 layers x (16 requests x 256 blocks) bf16 16-token blocks, merged by head into
32 full-head [8192][16][K,V][8][128] caches at random destination ids. Two layers are checked
in full against the oracle, all layers on sampled blocks."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, check_runs_equal, host_bytes, kvx, log

pytestmark = [pytest.mark.gpu, pytest.mark.big]


def test_asym_tp_full():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K = kvx()
    case = W.asym_tp()
    L, N, S = case.dst_spec.num_layers, case.total_blocks, case.num_src
    BB, nb = case.dst_spec.block_bytes, case.dst_spec.num_blocks
    BBs = BB // S
    log(f"asym: {S} sources of {L * N * BBs} B, {L} dst layers of {nb * BB} B")
    srcs = [torch.empty((L, N, BBs), dtype=torch.uint8, device=DEV) for _ in range(S)]
    for s, t in enumerate(srcs):
        W.fill_device_random_(t, W.ASYM_SEED * 10 + s)
    dst = [torch.empty((nb, BB), dtype=torch.uint8, device=DEV) for _ in range(L)]
    for t in dst:
        W.fill_device_byte_(t)
    ids, ro = K.flatten_tables(case.dst_tables, DEV)
    x, c = K.new_xfer_list(N, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(None, ids, ro, K.MODE_UNPACK, x, c, err)
    K.kvx_unpack(srcs, K.layer_base_table(dst), BB, nb, case.rows_per_block, x, c, N, err)
    torch.cuda.synchronize()
    log("asym: unpack done, checking")
    assert int(err.item()) == 0
    check_runs_equal(K, x, c, O.xfer_list([], case.dst_tables, O.MODE_UNPACK))
    for l in (0, L - 1):
        src_l = [host_bytes(t[l]).reshape(1, N, BBs) for t in srcs]
        before = np.full((nb, BB), W.FILL_BYTE, np.uint8)
        exp, e = O.unpack(src_l, [before], case.dst_tables, rows_per_block=case.rows_per_block)
        assert e == 0
        assert np.array_equal(host_bytes(dst[l]).reshape(nb, BB), exp[0]), f"layer {l}"
        log(f"asym: layer {l} identical")
    order = O.buffer_order(case.dst_tables)
    rng = np.random.default_rng(case.seed)
    for _ in range(384):
        l = int(rng.integers(L))
        r, j, p = order[int(rng.integers(N))]
        d_id = int(case.dst_tables[r][j])
        want = O.unpack_block([host_bytes(t[l, p]) for t in srcs], case.rows_per_block)
        assert np.array_equal(host_bytes(dst[l][d_id]), want), (l, p, d_id)
    log("asym: sampled blocks identical")


def test_asym_tp_split_full():
    """The sender side of the same transfer with the roles reversed: 32 full-head
    [8192][16][K,V][8][128] caches split into 2 head shards of 16 x 256 listed blocks."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K = kvx()
    case = W.asym_tp()
    L, N, S = case.dst_spec.num_layers, case.total_blocks, case.num_src
    BB, nb = case.dst_spec.block_bytes, case.dst_spec.num_blocks
    BBs = BB // S
    full = [W.fill_device_random_(torch.empty((nb, BB), dtype=torch.uint8, device=DEV), 900 + l)
            for l in range(L)]
    shards = [torch.zeros((L, N, BBs), dtype=torch.uint8, device=DEV) for _ in range(S)]
    ids, ro = K.flatten_tables(case.dst_tables, DEV)
    x, c = K.new_xfer_list(N, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(ids, None, ro, K.MODE_PACK, x, c, err)
    K.kvx_pack_split(K.layer_base_table(full), BB, nb, case.rows_per_block, x, c, N, shards, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for l in (0, L - 1):
        exp, e = O.pack_split([host_bytes(full[l]).reshape(nb, BB)], case.dst_tables, S, case.rows_per_block)
        assert e == 0
        for d in range(S):
            assert np.array_equal(host_bytes(shards[d][l]).reshape(N, BBs), exp[d][0]), f"layer {l} shard {d}"
        log(f"split: layer {l} identical")
    order = O.buffer_order(case.dst_tables)
    rng = np.random.default_rng(11)
    for _ in range(384):
        l = int(rng.integers(L))
        r, j, p = order[int(rng.integers(N))]
        blk = int(case.dst_tables[r][j])
        want = O.split_block(host_bytes(full[l][blk]), S, case.rows_per_block)
        for d in range(S):
            assert np.array_equal(host_bytes(shards[d][l, p]), want[d]), (l, p, d)
    log("split: sampled blocks identical")
