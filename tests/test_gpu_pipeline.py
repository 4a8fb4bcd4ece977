"""GPU tests of the device-side completion signal and of a layer-pipelined transfer.

The signal counter is checked against its definition (a monotone sum of the deltas; a wait
lets the stream go on exactly when the counter reaches the expected value, or when its
time runs out). The pipelined transfer — per layer: producer stream packs the layer and adds
1 to the counter, consumer stream waits for that count and unpacks the layer — must give
byte for byte what the oracle's pack and unpack give. A bf16 matrix product on the producer
stream before each layer stands in for that layer's forward pass, so the consumer would run
ahead of the data if the wait did not hold it.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, host_bytes, kvx, layers_from_host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"start {request.node.name}")
    yield
    torch.cuda.synchronize()
    log(f"end {request.node.name}")


def _busy(n: int, size: int = 4096):
    """About n bf16 [size x size] products: device work that takes a while, nothing else."""
    a = torch.ones((size, size), dtype=torch.bfloat16, device=DEV)
    b = torch.ones((size, size), dtype=torch.bfloat16, device=DEV)
    c = torch.empty_like(a)
    for _ in range(n):
        torch.mm(a, b, out=c)
    return c


def test_signal_add_sums_deltas():
    K = kvx()
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    for d in (1, 2, 3, 4, 5):
        K.kvx_signal_add(counter, d)
    torch.cuda.synchronize()
    assert int(counter.item()) == 15
    # the full 64-bit range: a carry out of the low word
    counter.fill_((1 << 40) - 1)
    K.kvx_signal_add(counter, 2)
    K.kvx_signal_add(counter, (1 << 33))
    torch.cuda.synchronize()
    assert int(counter.item()) == (1 << 40) + 1 + (1 << 33)


def test_wait_holds_the_stream_until_signalled():
    K = kvx()
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    marker = torch.zeros(1, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(prod):
        _busy(150)
        K.kvx_signal_add(counter, 1)  # enqueued before the wait that expects it
    with torch.cuda.stream(cons):
        K.kvx_signal_wait(counter, 1, 20_000_000, err)
        marker.fill_(7)
    prod_done, cons_done = prod.query(), cons.query()
    log(f"right after enqueue: producer done {prod_done}, consumer done {cons_done}")
    if not prod_done:
        assert not cons_done, "the consumer finished before the producer's signal"
    torch.cuda.synchronize()
    assert int(marker.item()) == 7
    assert int(err.item()) == 0
    assert int(counter.item()) == 1


def test_wait_on_a_reached_count_passes_at_once():
    K = kvx()
    counter = torch.full((1,), 9, dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for v in (0, 1, 9):
            K.kvx_signal_wait(counter, v, 1_000_000, err)
        b.record()
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert a.elapsed_time(b) < 100.0  # ms: nowhere near the 1 s limit


def test_wait_times_out_and_lets_the_stream_go_on():
    """The wait's own time limit, set tiny from the host: the counter never reaches 1."""
    K = kvx()
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    marker = torch.zeros(1, dtype=torch.int32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        K.kvx_signal_wait(counter, 1, 3000, err)
        b.record()
        marker.fill_(5)
    torch.cuda.synchronize()
    assert int(err.item()) == K.DEVERR_TIMEOUT
    assert int(marker.item()) == 5
    ms = a.elapsed_time(b)
    log(f"timed-out wait took {ms:.3f} ms (limit 3 ms)")
    assert 2.5 <= ms < 200.0


def _pipelined_roundtrip(seed, L, nb, H, D, lengths, forward_products, fused=False):
    K = kvx()
    case = W.random_transfer(seed, L, nb, 16, H, D, lengths)
    BB, N = case.src_spec.block_bytes, case.total_blocks
    src = layers_from_host(case.src_caches, BB)
    dst = layers_from_host(case.dst_caches, BB)
    sb, db = K.layer_base_table(src), K.layer_base_table(dst)
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    did, _ = K.flatten_tables(case.dst_tables, DEV)
    xp, cp = K.new_xfer_list(N, DEV)
    xu, cu = K.new_xfer_list(N, DEV)
    buf = torch.full((L, max(N, 1), BB), 0x5A, dtype=torch.uint8, device=DEV)
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    arrivals = K.new_arrivals(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    werr = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp, err)
    K.kvx_build_xfer_list(None, did, ro, K.MODE_UNPACK, xu, cu, err)
    torch.cuda.synchronize()
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    for l in range(L):
        with torch.cuda.stream(prod):
            if forward_products:
                _busy(forward_products, 2048)
            if fused:  # the pack's own launch carries the signal
                K.kvx_pack_signal(sb[l:l + 1], BB, nb, xp, cp, N, buf[l], counter, arrivals, 1, err)
            else:
                K.kvx_pack(sb[l:l + 1], BB, nb, xp, cp, N, buf[l], err)
                K.kvx_signal_add(counter, 1)
        with torch.cuda.stream(cons):
            K.kvx_signal_wait(counter, l + 1, 20_000_000, werr)
            K.kvx_unpack([buf[l]], db[l:l + 1], BB, nb, 1, xu, cu, N, err)
    torch.cuda.synchronize()
    assert int(werr.item()) == 0
    assert int(counter.item()) == L
    assert not bool(arrivals.any())
    exp_buf, e1 = O.pack(case.src_caches, case.src_tables)
    exp_dst, e2 = O.unpack([exp_buf], case.dst_caches, case.dst_tables)
    assert int(err.item()) == e1 | e2 == 0
    if N:
        assert np.array_equal(host_bytes(buf).reshape(L, N, BB), exp_buf.reshape(L, N, BB))
    for l in range(L):
        assert np.array_equal(host_bytes(dst[l]).reshape(nb, BB),
                              exp_dst[l].view(np.uint8).reshape(nb, BB)), f"layer {l}"


@pytest.mark.parametrize("fused", [False, True], ids=["signal-kernel", "signal-in-pack"])
@pytest.mark.parametrize("forward_products", [0, 3])
def test_layer_pipelined_transfer_matches_oracle(forward_products, fused):
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 700, size=7)]
    _pipelined_roundtrip(31, 6, 600, 1, 40, lengths, forward_products, fused)  # 2560 B blocks


@pytest.mark.parametrize("fused", [False, True], ids=["signal-kernel", "signal-in-pack"])
def test_layer_pipelined_transfer_whole_kib_blocks(fused):
    """8 KiB blocks (one head of 128 at 16 tokens): the one-batch copy kernels."""
    rng = np.random.default_rng(32)
    lengths = [int(x) for x in rng.integers(100, 1500, size=5)]
    _pipelined_roundtrip(32, 8, 800, 1, 128, lengths, 2, fused)


@pytest.mark.parametrize("bb_heads_dim", [(1, 128), (1, 40), (8, 128)], ids=["8KiB", "2560B", "64KiB"])
def test_signalling_copies_match_the_plain_ones(bb_heads_dim):
    """kvx_pack_signal and kvx_copy_direct_signal against the oracle's pack and direct copy,
    twice in a row on one arrivals workspace: each call adds its delta exactly once, leaves the
    arrivals workspace at 0, and moves the same bytes the plain call defines. An empty transfer
    still adds its delta."""
    K = kvx()
    H, D = bb_heads_dim
    rng = np.random.default_rng(40 + H + D)
    lengths = [int(x) for x in rng.integers(1, 900, size=6)]
    L, nb = 3, 400
    case = W.random_transfer(41 + D, L, nb, 16, H, D, lengths)
    BB, N = case.src_spec.block_bytes, case.total_blocks
    src = layers_from_host(case.src_caches, BB)
    dst = layers_from_host(case.dst_caches, BB)
    sb, db = K.layer_base_table(src), K.layer_base_table(dst)
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    did, _ = K.flatten_tables(case.dst_tables, DEV)
    xp, cp = K.new_xfer_list(N, DEV)
    xd, cd = K.new_xfer_list(N, DEV)
    buf = torch.full((L, N, BB), 0x5A, dtype=torch.uint8, device=DEV)
    counter = torch.full((1,), 100, dtype=torch.int64, device=DEV)
    arrivals = K.new_arrivals(DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp, err)
    K.kvx_build_xfer_list(sid, did, ro, K.MODE_DIRECT, xd, cd, err)
    K.kvx_pack_signal(sb, BB, nb, xp, cp, N, buf, counter, arrivals, 3, err)
    K.kvx_pack_signal(sb, BB, nb, xp, cp, N, buf, counter, arrivals, 5, err)
    K.kvx_copy_direct_signal(sb, db, BB, nb, nb, xd, cd, N, counter, arrivals, 7, err)
    K.kvx_pack_signal(sb, BB, nb, xp, cp, 0, buf, counter, arrivals, 11, err)  # nothing to copy
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert int(counter.item()) == 100 + 3 + 5 + 7 + 11
    assert not bool(arrivals.any())
    exp_buf, e1 = O.pack(case.src_caches, case.src_tables)
    exp_dst, e2 = O.copy_direct(case.src_caches, case.dst_caches, case.src_tables, case.dst_tables)
    assert e1 == e2 == 0
    assert np.array_equal(host_bytes(buf).reshape(L, N, BB), exp_buf.reshape(L, N, BB))
    for l in range(L):
        assert np.array_equal(host_bytes(dst[l]).reshape(nb, BB), exp_dst[l]), f"layer {l}"


@pytest.mark.parametrize("blocks", [1, 3, 40, 700])
def test_signalling_pack_small_launches(blocks):
    """One layer, 1 to 700 blocks of 8 KiB: launches of 1, 2, 20 and 350 workgroups, fewer and
    more than the 16 group counters the arrivals workspace holds. Each call adds its delta once
    and leaves the workspace zero; the buffer matches the oracle."""
    K = kvx()
    rng = np.random.default_rng(60 + blocks)
    nb = 2048
    src_h = W.random_words(rng, (nb, 4096))
    table = [rng.permutation(nb)[:blocks].astype(np.int32)]
    src = layers_from_host([src_h], 8192)
    sid, ro = K.flatten_tables(table, DEV)
    xp, cp = K.new_xfer_list(blocks, DEV)
    K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp)
    buf = torch.zeros((blocks, 8192), dtype=torch.uint8, device=DEV)
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    arrivals = K.new_arrivals(DEV)
    for delta in (1, 2, 4):
        K.kvx_pack_signal(K.layer_base_table(src), 8192, nb, xp, cp, blocks, buf, counter, arrivals, delta)
    torch.cuda.synchronize()
    assert int(counter.item()) == 7 and not bool(arrivals.any())
    exp, e = O.pack([src_h], table)
    assert e == 0 and np.array_equal(host_bytes(buf).reshape(blocks, 8192), exp[0])


def test_signalling_packs_on_two_streams_with_their_own_words():
    """Two senders, each on its own stream with its own counter and arrivals workspace, pack
    different transfers at the same time, layer by layer; both counters reach their layer
    counts and both buffers match the oracle."""
    K = kvx()
    runs = []
    for seed, (H, D) in ((50, (1, 128)), (51, (1, 40))):
        rng = np.random.default_rng(seed)
        lengths = [int(x) for x in rng.integers(1, 800, size=5)]
        case = W.random_transfer(seed, 4, 500, 16, H, D, lengths)
        BB, N = case.src_spec.block_bytes, case.total_blocks
        src = layers_from_host(case.src_caches, BB)
        sid, ro = K.flatten_tables(case.src_tables, DEV)
        xp, cp = K.new_xfer_list(N, DEV)
        K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp)
        runs.append(dict(case=case, BB=BB, N=N, src=src, sb=K.layer_base_table(src), xp=xp, cp=cp,
                         buf=torch.zeros((4, N, BB), dtype=torch.uint8, device=DEV),
                         counter=torch.zeros(1, dtype=torch.int64, device=DEV),
                         arrivals=K.new_arrivals(DEV),
                         stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    for l in range(4):
        for r in runs:
            with torch.cuda.stream(r["stream"]):
                K.kvx_pack_signal(r["sb"][l:l + 1], r["BB"], 500, r["xp"], r["cp"], r["N"], r["buf"][l],
                                  r["counter"], r["arrivals"], 1)
    torch.cuda.synchronize()
    for r in runs:
        assert int(r["counter"].item()) == 4 and not bool(r["arrivals"].any())
        exp, e = O.pack(r["case"].src_caches, r["case"].src_tables)
        assert e == 0
        assert np.array_equal(host_bytes(r["buf"]).reshape(exp.shape), exp)


@pytest.mark.parametrize("fused", [False, True], ids=["signal-kernel", "signal-in-copy"])
def test_layer_pipelined_direct_copy_then_consumer_reads(fused):
    """Per layer: the producer copies the layer's blocks cache to cache (no buffer) and adds 1;
    the consumer waits for that count, then copies the destination layer out with a kernel
    of its own (a torch copy). What the consumer read must be the oracle's direct copy: the
    wait ordered its reads after the producer's writes."""
    K = kvx()
    rng = np.random.default_rng(33)
    lengths = [int(x) for x in rng.integers(100, 1200, size=5)]
    L, nb = 6, 700
    case = W.random_transfer(33, L, nb, 16, 1, 128, lengths)
    BB, N = case.src_spec.block_bytes, case.total_blocks
    src = layers_from_host(case.src_caches, BB)
    dst = layers_from_host(case.dst_caches, BB)
    seen = [torch.empty_like(t) for t in dst]
    sb, db = K.layer_base_table(src), K.layer_base_table(dst)
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    did, _ = K.flatten_tables(case.dst_tables, DEV)
    x, c = K.new_xfer_list(N, DEV)
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    werr = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(sid, did, ro, K.MODE_DIRECT, x, c, err)
    torch.cuda.synchronize()
    arrivals = K.new_arrivals(DEV)
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    for l in range(L):
        with torch.cuda.stream(prod):
            _busy(2, 2048)
            if fused:  # the one-sided write carries its own signal
                K.kvx_copy_direct_signal(sb[l:l + 1], db[l:l + 1], BB, nb, nb, x, c, N, counter, arrivals, 1, err)
            else:
                K.kvx_copy_direct(sb[l:l + 1], db[l:l + 1], BB, nb, nb, x, c, N, err)
                K.kvx_signal_add(counter, 1)
        with torch.cuda.stream(cons):
            K.kvx_signal_wait(counter, l + 1, 20_000_000, werr)
            seen[l].copy_(dst[l])
    torch.cuda.synchronize()
    assert int(werr.item()) == 0 and int(err.item()) == 0 and int(counter.item()) == L
    exp, e = O.copy_direct(case.src_caches, case.dst_caches, case.src_tables, case.dst_tables)
    assert e == 0
    for l in range(L):
        assert np.array_equal(host_bytes(seen[l]).reshape(nb, BB), exp[l]), f"layer {l}"
