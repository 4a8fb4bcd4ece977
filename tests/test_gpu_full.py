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
from gpu_util import DEV, Transfer, check_runs_equal, host_bytes, kvx, log, to_dev

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
    for t in dst:
        W.fill_device_byte_(t)
    tr = Transfer(case, src, dst)
    tr.run()
    log(f"{case.name}: transfer done, checking")
    _verify(case, tr)


def _verify(case, tr):
    """The run lists, the send buffer and the destination caches against the oracle: three
    layers in full, every layer on sampled blocks, and untouched blocks still the fill byte."""
    spec, src, dst = case.src_spec, tr.src, tr.dst
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


def test_step_new_token_write_full(pages_caches):
    """The rest of the benchmark's step at full size: after the contiguous transfer, the
    receiver's slot mapping for each request's last prompt token (recomputed locally) and the
    per-layer new-token write of its 256-byte K and V rows into all 48 destination layers, one
    launch per layer as in the step. Every block that receives a new row is compared with the
    oracle: the block as the transfer left it (the source block), then the oracle's write."""
    spec, src, dst = pages_caches
    case = W.pages_contiguous()
    for t in dst:
        W.fill_device_byte_(t)
    tr = Transfer(case, src, dst)
    tr.run()
    K = tr.K
    L, nb, bs, row = spec.num_layers, spec.num_blocks, spec.block_size, spec.row_bytes
    R = len(case.dst_tables)
    table_h = W.pad_table(case.dst_tables, max(len(t) for t in case.dst_tables))
    req_h = np.arange(R, dtype=np.int32)
    pos_h = np.array([n - 1 for n in case.lengths], dtype=np.int64)
    rng = np.random.default_rng(case.seed + 7)
    new_k = W.bf16_normal_bits(rng, (L, R, row // 2))
    new_v = W.bf16_normal_bits(rng, (L, R, row // 2))
    slots = torch.empty(R, dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_slot_mapping(to_dev(table_h), to_dev(req_h), to_dev(pos_h), bs, slots, err)
    kd, vd = to_dev(new_k), to_dev(new_v)
    view = dst[0].view(torch.int16).view(nb, bs, 2, spec.num_kv_heads, spec.head_dim)
    cnb, cbs, bst, tst, kst = K.cache_strides(view)
    for l in range(L):
        K.kvx_reshape_and_cache(kd[l], vd[l], slots, dst[l], cnb, cbs, bst, tst, kst, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and tr.err_bits() == 0
    exp_slots, e = O.slot_mapping(table_h, req_h, pos_h, bs)
    assert e == 0 and np.array_equal(slots.cpu().numpy(), exp_slots)
    # the written blocks, gathered into a small cache: block i of it is destination block blocks[i]
    blocks = sorted(set(int(s) // bs for s in exp_slots))
    where = {b: i for i, b in enumerate(blocks)}
    mini_slots = np.array([where[int(s) // bs] * bs + int(s) % bs for s in exp_slots], np.int64)
    dst_to_src = {int(d): int(s_) for s_, d in zip(np.concatenate(case.src_tables), np.concatenate(case.dst_tables))}
    for l in range(L):
        before = np.stack([host_bytes(src[l][dst_to_src[b]]) for b in blocks])
        exp, e = O.reshape_and_cache(before, new_k[l], new_v[l], mini_slots, len(blocks), bs, bst, tst, kst)
        assert e == 0
        got = np.stack([host_bytes(dst[l][b]) for b in blocks]).reshape(-1)
        assert np.array_equal(got, exp), f"layer {l}"
    log(f"new-token write: {R} tokens x {L} layers identical")


def test_layer_pipelined_transfer_full(pages_caches):
    """The contiguous transfer layer by layer at full size: per layer, a bf16 product on a
    forward stream, then on a copy stream that layer's pack and a signal add, and on a
    consumer stream the signal wait and that layer's unpack. Checked like the one-launch
    transfer."""
    spec, src, dst = pages_caches
    case = W.pages_contiguous()
    for t in dst:
        W.fill_device_byte_(t)
    tr = Transfer(case, src, dst)
    tr.build()
    K, L, N, BB, nb = tr.K, spec.num_layers, tr.N, tr.BB, spec.num_blocks
    tr.buf.fill_(0x5A)
    bufv = tr.buf.view(L, N, BB)
    a = torch.full((2048, 2048), 0.5, dtype=torch.bfloat16, device=DEV)
    c = torch.empty_like(a)
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    werr = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    fwd, cpy, cons = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    evs = [torch.cuda.Event() for _ in range(L)]
    for l in range(L):
        with torch.cuda.stream(fwd):
            torch.mm(a, a, out=c)
            evs[l].record(fwd)
        cpy.wait_event(evs[l])
        K.kvx_pack(tr.src_bases[l:l + 1], BB, nb, tr.xp, tr.cp, N, bufv[l], tr.err, stream=cpy)
        K.kvx_signal_add(counter, 1, stream=cpy)
        K.kvx_signal_wait(counter, l + 1, 20_000_000, werr, stream=cons)
        K.kvx_unpack([bufv[l]], tr.dst_bases[l:l + 1], BB, nb, 1, tr.xu, tr.cu, N, tr.err, stream=cons)
    torch.cuda.synchronize()
    assert int(werr.item()) == 0 and int(counter.item()) == L
    log("layer-pipelined transfer done, checking")
    _verify(case, tr)


def test_pages_contiguous_direct_full(pages_caches):
    """The contiguous transfer at full size with no send buffer: runs built in direct mode,
    every listed block of the 48 layers copied from the source caches into the destination
    caches. Three layers checked in full against the oracle, all layers on sampled blocks."""
    spec, src, dst = pages_caches
    case = W.pages_contiguous()
    K = kvx()
    L, nb, BB, N = spec.num_layers, spec.num_blocks, spec.block_bytes, case.total_blocks
    for t in dst:
        W.fill_device_byte_(t)
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    did, _ = K.flatten_tables(case.dst_tables, DEV)
    x, c = K.new_xfer_list(N, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(sid, did, ro, K.MODE_DIRECT, x, c, err)
    K.kvx_copy_direct(K.layer_base_table(src), K.layer_base_table(dst), BB, nb, nb, x, c, N, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    check_runs_equal(K, x, c, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_DIRECT))
    for l in FULL_LAYERS:
        before = np.full((nb, BB), W.FILL_BYTE, np.uint8)
        exp, e = O.copy_direct([host_bytes(src[l]).reshape(nb, BB)], [before], case.src_tables,
                               case.dst_tables)
        assert e == 0
        assert np.array_equal(host_bytes(dst[l]).reshape(nb, BB), exp[0]), f"direct layer {l}"
        log(f"direct: layer {l} identical")
    rng = np.random.default_rng(case.seed + 1)
    flat_s, flat_d = np.concatenate(case.src_tables), np.concatenate(case.dst_tables)
    for _ in range(SAMPLES):
        l = int(rng.integers(L))
        i = int(rng.integers(N))
        assert np.array_equal(host_bytes(dst[l][int(flat_d[i])]), host_bytes(src[l][int(flat_s[i])])), (l, i)
    log(f"direct: {SAMPLES} sampled blocks identical")


def test_run_lists_past_the_workgroup_cap():
    """1.18M blocks of 16 bytes in 300 requests: more tiles than the run builder's workgroups,
    so each workgroup walks several sub-tiles. Run lists in both modes and the transfer's
    bytes against the oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rng = np.random.default_rng(90)
    lengths = [int(x) for x in rng.integers(0, 8000, size=300)]
    case = W.random_transfer(91, 1, 3_000_000, 1, 1, 8, lengths, elem_bytes=1)
    BB = case.src_spec.block_bytes
    assert case.total_blocks > 256 * 2048
    src = [torch.from_numpy(case.src_caches[0].view(np.uint8).reshape(-1, BB)).to(DEV)]
    dst = [torch.from_numpy(case.dst_caches[0].view(np.uint8).reshape(-1, BB)).to(DEV)]
    tr = Transfer(case, src, dst)
    tr.run()
    log("1.18M-block transfer done, checking")
    assert tr.err_bits() == 0
    check_runs_equal(tr.K, tr.xp, tr.cp, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_PACK))
    check_runs_equal(tr.K, tr.xu, tr.cu, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_UNPACK))
    exp_buf, e1 = O.pack(case.src_caches, case.src_tables)
    exp_dst, e2 = O.unpack([exp_buf], case.dst_caches, case.dst_tables)
    assert e1 == e2 == 0
    assert np.array_equal(host_bytes(tr.buf)[: exp_buf.nbytes], exp_buf.reshape(-1))
    assert np.array_equal(host_bytes(dst[0]), exp_dst[0].reshape(-1))
