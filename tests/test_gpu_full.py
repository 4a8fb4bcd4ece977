"""GPU parity at the full workload sizes, in the launch configuration the benchmark times:
48 layers of [147456][16][K,V][128] bf16 (1.125 GiB each, separate allocations), 8 requests x
576 blocks, contiguous (runs of 64) and fragmented (geometric run lengths) block tables,
unpacked into a second 48-layer cache at random ids. Every layer is streamed to the host and
compared whole, byte for byte, with the oracle's output for that layer: the send buffer's
slice and the entire destination cache (listed blocks and the untouched rest)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, HostStage, Transfer, check_runs_equal, kvx, log, same_bytes, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.big]


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


@pytest.fixture(scope="module")
def stage():
    st = HostStage()
    yield st
    st._bufs.clear()


def _progress(what, l, L):
    if l % 8 == 7 or l == L - 1:
        log(f"{what}: layers 0..{l} identical")


def _check_transfer(case, src, dst, stage):
    for t in dst:
        W.fill_device_byte_(t)
    tr = Transfer(case, src, dst)
    tr.run()
    log(f"{case.name}: transfer done, checking")
    _verify(case, tr, stage)


def _verify(case, tr, stage):
    """The run lists, then every layer: its slice of the send buffer against the oracle's pack
    of the host copy of that layer, and the whole destination layer against the oracle's
    unpack of that buffer into a cache holding the fill byte (as the device cache did)."""
    spec, src, dst = case.src_spec, tr.src, tr.dst
    assert tr.err_bits() == 0
    check_runs_equal(tr.K, tr.xp, tr.cp, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_PACK))
    check_runs_equal(tr.K, tr.xu, tr.cu, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_UNPACK))
    L, N, BB, nb = spec.num_layers, tr.N, tr.BB, spec.num_blocks
    buf = tr.buf.view(L, N, BB)
    before = np.full((nb, BB), W.FILL_BYTE, np.uint8)
    for l in range(L):
        exp_buf, e1 = O.pack([stage.get(src[l], 0).reshape(nb, BB)], case.src_tables)
        assert same_bytes(stage.get(buf[l], 1), exp_buf), f"pack layer {l}"
        exp_dst, e2 = O.unpack([exp_buf], [before], case.dst_tables)
        assert same_bytes(stage.get(dst[l], 2), exp_dst[0]), f"unpack layer {l}"
        assert e1 == e2 == 0
        _progress(case.name, l, L)


def test_pages_contiguous_full(pages_caches, stage):
    spec, src, dst = pages_caches
    _check_transfer(W.pages_contiguous(), src, dst, stage)


def test_pages_fragmented_full(pages_caches, stage):
    spec, src, dst = pages_caches
    _check_transfer(W.pages_fragmented(), src, dst, stage)


def test_pages_contiguous_kv_first_full(pages_caches, stage):
    """The same 48 allocations viewed as kv-first caches (K plane, V plane) of 147456 blocks
    with 4 KiB segments: pack and unpack through the kv-first entry points, every layer
    compared whole with the oracle's kv-first pack and unpack."""
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
    before = np.full((2, nb, seg), W.FILL_BYTE, np.uint8)
    for l in range(L):
        exp_buf, e1 = O.pack_kv_first([stage.get(src[l], 0).reshape(2, nb, seg)], case.src_tables)
        assert same_bytes(stage.get(bufv[l], 1), exp_buf), f"kv-first pack layer {l}"
        exp_dst, e2 = O.unpack_kv_first(exp_buf, [before], case.dst_tables)
        assert same_bytes(stage.get(dst[l], 2), exp_dst[0]), f"kv-first unpack layer {l}"
        assert e1 == e2 == 0
        _progress("kv-first", l, L)


def test_step_new_token_write_full(pages_caches, stage):
    """The benchmark's whole step at full size: the contiguous transfer, then the receiver's
    slot mapping for each request's last prompt token (recomputed locally) and the per-layer
    new-token write of its 256-byte K and V rows into all 48 destination layers, one launch
    per layer as in the step. Every destination layer is compared whole with the oracle's
    pack, unpack and new-token write of that layer."""
    spec, src, dst = pages_caches
    case = W.pages_contiguous()
    for t in dst:
        W.fill_device_byte_(t)
    tr = Transfer(case, src, dst)
    tr.run()
    K = tr.K
    L, nb, bs, row, BB = spec.num_layers, spec.num_blocks, spec.block_size, spec.row_bytes, spec.block_bytes
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
    before = np.full((nb, BB), W.FILL_BYTE, np.uint8)
    for l in range(L):
        exp_buf, e1 = O.pack([stage.get(src[l], 0).reshape(nb, BB)], case.src_tables)
        moved, e2 = O.unpack([exp_buf], [before], case.dst_tables)
        exp, e3 = O.reshape_and_cache(moved[0], new_k[l], new_v[l], exp_slots, nb, bs, bst, tst, kst)
        assert e1 == e2 == e3 == 0
        assert same_bytes(stage.get(dst[l], 2), exp), f"layer {l}"
        _progress("step with new-token writes", l, L)


@pytest.mark.parametrize("fused", [False, True], ids=["signal-kernel", "signal-in-pack"])
def test_layer_pipelined_transfer_full(pages_caches, stage, fused):
    """The contiguous transfer layer by layer at full size: per layer, a bf16 product on a
    forward stream, then on a copy stream that layer's pack and a signal add (a separate
    launch, or carried by the pack's own launch), and on a consumer stream the signal wait
    and that layer's unpack. Checked like the one-launch transfer, every layer whole."""
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
    arrivals = K.new_arrivals(DEV)
    werr = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    fwd, cpy, cons = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    evs = [torch.cuda.Event() for _ in range(L)]
    for l in range(L):
        with torch.cuda.stream(fwd):
            torch.mm(a, a, out=c)
            evs[l].record(fwd)
        cpy.wait_event(evs[l])
        if fused:
            K.kvx_pack_signal(tr.src_bases[l:l + 1], BB, nb, tr.xp, tr.cp, N, bufv[l], counter, arrivals, 1,
                              tr.err, stream=cpy)
        else:
            K.kvx_pack(tr.src_bases[l:l + 1], BB, nb, tr.xp, tr.cp, N, bufv[l], tr.err, stream=cpy)
            K.kvx_signal_add(counter, 1, stream=cpy)
        K.kvx_signal_wait(counter, l + 1, 20_000_000, werr, stream=cons)
        K.kvx_unpack([bufv[l]], tr.dst_bases[l:l + 1], BB, nb, 1, tr.xu, tr.cu, N, tr.err, stream=cons)
    torch.cuda.synchronize()
    assert int(werr.item()) == 0 and int(counter.item()) == L and not bool(arrivals.any())
    log("layer-pipelined transfer done, checking")
    _verify(case, tr, stage)


def test_pages_contiguous_direct_full(pages_caches, stage):
    """The contiguous transfer at full size with no send buffer: runs built in direct mode,
    every listed block of the 48 layers copied from the source caches into the destination
    caches. Every destination layer compared whole with the oracle's direct copy."""
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
    before = np.full((nb, BB), W.FILL_BYTE, np.uint8)
    for l in range(L):
        exp, e = O.copy_direct([stage.get(src[l], 0).reshape(nb, BB)], [before], case.src_tables,
                               case.dst_tables)
        assert e == 0
        assert same_bytes(stage.get(dst[l], 2), exp[0]), f"direct layer {l}"
        _progress("direct", l, L)


def test_run_lists_past_the_workgroup_cap(stage):
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
    assert same_bytes(stage.get(tr.buf, 1)[: exp_buf.nbytes], exp_buf)
    assert same_bytes(stage.get(dst[0], 2), exp_dst[0])
