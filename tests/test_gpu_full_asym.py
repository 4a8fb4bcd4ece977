"""GPU parity at the full asymmetric-TP receive size: two send buffers, each holding 4 of 8
KV heads of 32 layers x (16 requests x 256 blocks) bf16 16-token blocks, merged by head into
32 full-head [8192][16][K,V][8][128] caches at random destination ids; and the sender side,
32 full-head caches split into 2 head shards. Every layer is streamed to the host and
compared whole, byte for byte, with the oracle's merge (or split) of that layer."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, HostStage, check_runs_equal, kvx, log, same_bytes

pytestmark = [pytest.mark.gpu, pytest.mark.big]


def _progress(what, l, L):
    if l % 8 == 7 or l == L - 1:
        log(f"{what}: layers 0..{l} identical")


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
    stage = HostStage()
    before = np.full((nb, BB), W.FILL_BYTE, np.uint8)
    for l in range(L):
        src_l = [stage.get(t[l], 10 + s).reshape(1, N, BBs) for s, t in enumerate(srcs)]
        exp, e = O.unpack(src_l, [before], case.dst_tables, rows_per_block=case.rows_per_block)
        assert e == 0
        assert same_bytes(stage.get(dst[l], 0), exp[0]), f"layer {l}"
        _progress("asym merge", l, L)


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
    check_runs_equal(K, x, c, O.xfer_list(case.dst_tables, [], O.MODE_PACK))
    stage = HostStage()
    for l in range(L):
        exp, e = O.pack_split([stage.get(full[l], 0).reshape(nb, BB)], case.dst_tables, S, case.rows_per_block)
        assert e == 0
        for d in range(S):
            assert same_bytes(stage.get(shards[d][l], 10 + d), exp[d][0]), f"layer {l} shard {d}"
        _progress("asym split", l, L)
