"""HIP graph replays against the oracle. The whole step captured once and replayed (run lists,
pack, unpack, slot mapping and the per-layer new-token writes), with the program's own eager
work refilling the send buffer and the receive caches between replays; and the per-layer writes
alone, replayed while the eager slot mapping moves the tokens between replays."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, host_bytes, kvx, layers_from_host, log, to_dev

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_oracle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K = kvx()
    rng = np.random.default_rng(41)
    lengths = [int(x) for x in rng.integers(1, 900, size=6)]
    L, nb = 4, 700
    case = W.random_transfer(41, L, nb, 16, 1, 128, lengths)  # 8 KiB blocks
    spec, N = case.src_spec, case.total_blocks
    BB, bs, row = spec.block_bytes, spec.block_size, spec.row_bytes
    R = len(lengths)
    src = layers_from_host(case.src_caches, BB)
    dst = layers_from_host(case.dst_caches, BB)
    sb, db = K.layer_base_table(src), K.layer_base_table(dst)
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    did, _ = K.flatten_tables(case.dst_tables, DEV)
    xp, cp = K.new_xfer_list(N, DEV)
    xu, cu = K.new_xfer_list(N, DEV)
    buf = torch.zeros(L * N * BB, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    table_h = W.pad_table(case.dst_tables, max(len(t) for t in case.dst_tables))
    req_h = np.arange(R, dtype=np.int32)
    pos_h = np.array([n - 1 for n in lengths], dtype=np.int64)
    table, req, pos = to_dev(table_h), to_dev(req_h), to_dev(pos_h)
    slots = torch.empty(R, dtype=torch.int64, device=DEV)
    new_k = W.bf16_normal_bits(rng, (L, R, row // 2))
    new_v = W.bf16_normal_bits(rng, (L, R, row // 2))
    kd, vd = to_dev(new_k), to_dev(new_v)
    view = dst[0].view(torch.int16).view(nb, bs, 2, spec.num_kv_heads, spec.head_dim)
    cnb, cbs, bst, tst, kst = K.cache_strides(view)

    def step():
        K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp, err)
        K.kvx_pack(sb, BB, nb, xp, cp, N, buf, err)
        K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu, err)
        K.kvx_unpack([buf], db, BB, nb, 1, xu, cu, N, err)
        K.kvx_slot_mapping(table, req, pos, bs, slots, err)
        for l in range(L):
            K.kvx_reshape_and_cache(kd[l], vd[l], slots, dst[l], cnb, cbs, bst, tst, kst, err)

    # expected: the oracle's pack, unpack into the sentinel caches, then the writes
    exp_buf, e1 = O.pack(case.src_caches, case.src_tables)
    exp_dst, e2 = O.unpack([exp_buf], case.dst_caches, case.dst_tables)
    exp_slots, e3 = O.slot_mapping(table_h, req_h, pos_h, bs)
    expected = []
    for l in range(L):
        out, e4 = O.reshape_and_cache(exp_dst[l], new_k[l], new_v[l], exp_slots, nb, bs, bst, tst, kst)
        assert e4 == 0
        expected.append(out)
    assert e1 == e2 == e3 == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        # eager work between replays: wipe what the step writes
        buf.fill_(0)
        xp.fill_(-1)
        xu.fill_(-1)
        slots.fill_(-7)
        for l in range(L):
            dst[l].copy_(to_dev(case.dst_caches[l].view(np.uint8).reshape(nb, BB)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert np.array_equal(slots.cpu().numpy(), exp_slots), f"replay {rep}: slots"
        assert np.array_equal(host_bytes(buf), exp_buf.reshape(-1)), f"replay {rep}: send buffer"
        for l in range(L):
            assert np.array_equal(host_bytes(dst[l]), expected[l]), f"replay {rep}: layer {l}"
        log(f"graph replay {rep} identical to the oracle")


def test_layer_writes_graph_replays_read_the_slots_of_the_moment():
    """The per-layer new-token writes alone captured once, as a decode loop replays a captured
    forward: between replays the program's eager slot mapping moves every request's token to
    another position, and the caches are refilled. Each replay must write at the slots computed
    just before it, in every layer, as the oracle does."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K = kvx()
    rng = np.random.default_rng(43)
    lengths = [int(x) for x in rng.integers(40, 600, size=5)]
    L, nb, bs = 4, 300, 16
    case = W.random_transfer(43, L, nb, bs, 1, 128, lengths)  # 8 KiB blocks, 256 B rows
    spec = case.dst_spec
    BB, row, R = spec.block_bytes, spec.row_bytes, len(lengths)
    dst = layers_from_host(case.dst_caches, BB)
    table_h = W.pad_table(case.dst_tables, max(len(t) for t in case.dst_tables))
    req_h = np.arange(R, dtype=np.int32)
    table, req = to_dev(table_h), to_dev(req_h)
    pos = torch.zeros(R, dtype=torch.int64, device=DEV)
    slots = torch.empty(R, dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    new_k = W.bf16_normal_bits(rng, (L, R, row // 2))
    new_v = W.bf16_normal_bits(rng, (L, R, row // 2))
    kd, vd = to_dev(new_k), to_dev(new_v)
    view = dst[0].view(torch.int16).view(nb, bs, 2, spec.num_kv_heads, spec.head_dim)
    cnb, cbs, bst, tst, kst = K.cache_strides(view)

    def writes():
        for l in range(L):
            K.kvx_reshape_and_cache(kd[l], vd[l], slots, dst[l], cnb, cbs, bst, tst, kst, err)

    K.kvx_slot_mapping(table, req, pos, bs, slots, err)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        writes()  # warm outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        writes()
    for rep in range(4):
        positions = np.array([int(rng.integers(0, n)) for n in lengths], dtype=np.int64)
        for l in range(L):
            dst[l].copy_(to_dev(case.dst_caches[l].view(np.uint8).reshape(nb, BB)))
        pos.copy_(to_dev(positions))
        K.kvx_slot_mapping(table, req, pos, bs, slots, err)
        g.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        exp_slots, e = O.slot_mapping(table_h, req_h, positions, bs)
        assert e == 0 and np.array_equal(slots.cpu().numpy(), exp_slots), f"replay {rep}: slots"
        for l in range(L):
            exp, e = O.reshape_and_cache(case.dst_caches[l].view(np.uint8).reshape(nb, BB), new_k[l], new_v[l],
                                         exp_slots, nb, bs, bst, tst, kst)
            assert e == 0
            assert np.array_equal(host_bytes(dst[l]), exp), f"replay {rep}: layer {l}"
        log(f"write graph replay {rep} at positions {positions.tolist()} identical to the oracle")
