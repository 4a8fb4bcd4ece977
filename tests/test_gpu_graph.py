"""HIP graph replays against the oracle. The whole step captured once and replayed (run lists,
pack, unpack, slot mapping and the per-layer new-token writes), with the program's own eager
work refilling the send buffer and the receive caches between replays; the per-layer writes
alone, replayed while the eager slot mapping moves the tokens between replays; and every other
copy (kv-first, direct, split and merge, both signalling packs) replayed the same way."""
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


def test_other_entry_points_graph_replays():
    """Every other copy captured once in a HIP graph and replayed, as a caller that captures its
    transfer would: the three run lists, the kv-first pack and unpack of the same caches viewed as
    (K/V plane, blocks, segment), the direct copy, the head split into 2 shards and their merge,
    the signalling pack and the allocation-free signalling pack. Between replays the program's
    eager work wipes every output and resets the counters; after each replay every output is
    compared with the oracle, each counter must have been added to exactly once, and the
    caller's arrivals workspace must be back to zero."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    K = kvx()
    rng = np.random.default_rng(47)
    lengths = [int(x) for x in rng.integers(1, 500, size=6)]
    L, nb, bs, H, D, S = 3, 240, 16, 8, 128, 2
    case = W.random_transfer(47, L, nb, bs, H, D, lengths)  # 64 KiB blocks, 2 KiB rows
    BB, N = case.src_spec.block_bytes, case.total_blocks
    seg, rows = BB // 2, bs * 2
    src_h = [np.ascontiguousarray(c).view(np.uint8).reshape(nb, BB) for c in case.src_caches]
    dst_h = [np.ascontiguousarray(c).view(np.uint8).reshape(nb, BB) for c in case.dst_caches]
    src = layers_from_host(src_h, BB)
    kvf_dst, dir_dst, mrg_dst = (layers_from_host(dst_h, BB) for _ in range(3))
    sb = K.layer_base_table(src)
    kvf_b, dir_b, mrg_b = K.layer_base_table(kvf_dst), K.layer_base_table(dir_dst), K.layer_base_table(mrg_dst)
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    did, _ = K.flatten_tables(case.dst_tables, DEV)
    (xp, cp), (xu, cu), (xd, cd) = (K.new_xfer_list(N, DEV) for _ in range(3))
    kbuf = torch.zeros(L * N * BB, dtype=torch.uint8, device=DEV)
    shards = [torch.zeros(L * N * BB // S, dtype=torch.uint8, device=DEV) for _ in range(S)]
    sbuf = torch.zeros(L * N * BB, dtype=torch.uint8, device=DEV)
    nbuf = torch.zeros(L * N * BB, dtype=torch.uint8, device=DEV)
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    ncounter = torch.zeros(1, dtype=torch.int64, device=DEV)
    arrivals = K.new_arrivals(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)

    def transfer():
        K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp, err)
        K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu, err)
        K.kvx_build_xfer_list(sid, did, ro, K.MODE_DIRECT, xd, cd, err)
        K.kvx_pack_kv_first(sb, seg, nb * seg, nb, ro, xp, cp, N, kbuf, err)
        K.kvx_unpack_kv_first(kbuf, kvf_b, seg, nb * seg, nb, ro, xu, cu, N, err)
        K.kvx_copy_direct(sb, dir_b, BB, nb, nb, xd, cd, N, err)
        K.kvx_pack_split(sb, BB, nb, rows, xp, cp, N, shards, err)
        K.kvx_unpack(shards, mrg_b, BB, nb, rows, xu, cu, N, err)
        K.kvx_pack_signal(sb, BB, nb, xp, cp, N, sbuf, counter, arrivals, 1, err)
        K.kvx_pack_signal_noalloc(sb, BB, nb, xp, cp, N, nbuf, ncounter, 3, 1, err)

    planes = lambda arrs: [a.reshape(2, nb, seg) for a in arrs]  # noqa: E731
    exp_buf, e1 = O.pack(src_h, case.src_tables)
    exp_k, e2 = O.pack_kv_first(planes(src_h), case.src_tables)
    exp_kvf, e3 = O.unpack_kv_first(exp_k, planes(dst_h), case.dst_tables)
    exp_dir, e4 = O.copy_direct(src_h, dst_h, case.src_tables, case.dst_tables)
    exp_sh, e5 = O.pack_split(src_h, case.src_tables, S, rows_per_block=rows)
    exp_mrg, e6 = O.unpack(list(exp_sh), dst_h, case.dst_tables, rows_per_block=rows)
    assert e1 == e2 == e3 == e4 == e5 == e6 == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        transfer()  # warm outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        transfer()
    for rep in range(3):
        for t in (kbuf, sbuf, nbuf, *shards):
            t.fill_(0)
        for t in (xp, xu, xd):
            t.fill_(-1)
        counter.zero_()
        ncounter.zero_()
        for layers in (kvf_dst, dir_dst, mrg_dst):
            for l in range(L):
                layers[l].copy_(to_dev(dst_h[l]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert int(counter.item()) == 1 and int(ncounter.item()) == 1, f"replay {rep}: signal counters"
        assert int(arrivals.abs().sum().item()) == 0, f"replay {rep}: arrivals left non-zero"
        assert np.array_equal(host_bytes(kbuf), exp_k.reshape(-1)), f"replay {rep}: kv-first buffer"
        assert np.array_equal(host_bytes(sbuf), exp_buf.reshape(-1)), f"replay {rep}: signalling pack"
        assert np.array_equal(host_bytes(nbuf), exp_buf.reshape(-1)), f"replay {rep}: allocation-free pack"
        for d in range(S):
            assert np.array_equal(host_bytes(shards[d]), exp_sh[d].reshape(-1)), f"replay {rep}: shard {d}"
        for l in range(L):
            assert np.array_equal(host_bytes(kvf_dst[l]), exp_kvf[l].reshape(-1)), f"replay {rep}: kv-first layer {l}"
            assert np.array_equal(host_bytes(dir_dst[l]), exp_dir[l].reshape(-1)), f"replay {rep}: direct layer {l}"
            assert np.array_equal(host_bytes(mrg_dst[l]), exp_mrg[l].reshape(-1)), f"replay {rep}: merge layer {l}"
        log(f"graph replay {rep} of the other entry points identical to the oracle")
