"""GPU parity at oracle-sized inputs: every kernel through the C ABI, compared byte for byte
with the CPU oracle on the same seeded inputs (several tiles, ragged tails, edge cases)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import (DEV, Transfer, check_runs_equal, host_bytes, kvx, layers_from_host, log,
                      reshape_and_cache_raw, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"start {request.node.name}")
    yield
    torch.cuda.synchronize()
    log(f"end {request.node.name}")


def host_roundtrip(case):
    """Oracle pack then oracle unpack of the host caches."""
    buf, e1 = O.pack(case.src_caches, case.src_tables)
    out, e2 = O.unpack([buf], case.dst_caches, case.dst_tables)
    return buf, out, e1 | e2


def run_case(case):
    t = Transfer(case, layers_from_host(case.src_caches, case.src_spec.block_bytes),
                 layers_from_host(case.dst_caches, case.dst_spec.block_bytes))
    t.run()
    buf, out, err = host_roundtrip(case)
    check_runs_equal(t.K, t.xp, t.cp, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_PACK))
    check_runs_equal(t.K, t.xu, t.cu, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_UNPACK))
    got = host_bytes(t.buf)[: buf.nbytes]
    assert np.array_equal(got, buf.reshape(-1)), "pack differs from the oracle"
    for l in range(t.L):
        assert np.array_equal(host_bytes(t.dst[l]).reshape(out[l].shape), out[l]), f"unpack layer {l}"
    assert t.err_bits() == err
    return t


def test_tiny_roundtrip():
    """2 layers of [64][16][K,V][2][16] fp16, requests of 17/40/5 tokens."""
    run_case(W.tiny_roundtrip())


GEOMS = [  # (block_size, heads, head_dim, elem_bytes) -> block bytes
    (16, 2, 16, 2),    # 2 KiB
    (4, 1, 8, 2),      # 128 B
    (1, 1, 8, 1),      # 16 B: one vector per block
    (16, 8, 128, 2),   # 64 KiB: several batches per block
    (16, 1, 128, 2),   # 8 KiB: the pages' block
    (16, 3, 40, 2),    # 7680 B: not a multiple of 1 KiB (ragged lanes)
]


@pytest.mark.parametrize("geom", GEOMS, ids=[f"bs{g[0]}h{g[1]}d{g[2]}e{g[3]}" for g in GEOMS])
def test_random_roundtrip_geometries(geom):
    bs, H, D, e = geom
    spec = W.PagedSpec(3, 1, bs, H, D, e)
    nb = max(64, min(6000, (48 << 20) // spec.block_bytes))
    rng = np.random.default_rng(hash(geom) & 0xffff)
    lengths = [int(x) for x in rng.integers(0, bs * 40, size=23)]
    lengths[3] = 0
    lengths[7] = 1
    while sum(W.blocks_for(n, bs) for n in lengths) * 3 > nb:
        lengths = lengths[:-1]
    run_case(W.random_transfer(int(rng.integers(1 << 30)), 3, nb, bs, H, D, lengths, elem_bytes=e))


@pytest.mark.parametrize("latent,elem", [(576, 2), (656, 1)], ids=["latent576-bf16", "latent656-u8"])
def test_mla_latent_cache_roundtrip(latent, elem):
    """MLA caches are (blocks, block_size, latent): one latent row per token, no K/V split (the
    nccl page §2.4 gathers them whole, like blocks-first caches). A block is then 16 * latent *
    elem bytes: 18 KiB for a 576-wide bf16 latent (whole KiB: the one-batch kernels) and
    10,496 B for a 656-byte row (not whole KiB: the general kernels). The generator's K/V
    doubling is folded into the row width, which gives the same block bytes."""
    bs = 16
    spec = W.PagedSpec(2, 1, bs, 1, latent // 2, elem)
    assert spec.block_bytes == bs * latent * elem
    nb = 1500
    rng = np.random.default_rng(latent)
    lengths = [int(x) for x in rng.integers(0, 900, size=11)]
    lengths[4] = 0
    run_case(W.random_transfer(latent, 2, nb, bs, 1, latent // 2, lengths, elem_bytes=elem))


@pytest.mark.parametrize("bs,H,D,contiguous", [(16, 1, 128, True), (16, 3, 40, False)],
                         ids=["8KiB-shared-run", "7680B-shared-scattered"])
def test_shared_prefix_transfer(bs, H, D, contiguous):
    """Prefix sharing (the v1 diagram's prefix-cache toy at scale): 9 requests whose tables all
    start with the same 37 cached blocks, then blocks of their own. The shared blocks are read
    once per request; every request gets fresh receiver blocks."""
    rng = np.random.default_rng(bs * 1000 + D)
    L, nb = 3, 2000
    spec = W.PagedSpec(L, nb, bs, H, D)
    if contiguous:
        shared = np.arange(500, 537)
        pool = rng.permutation(np.setdiff1d(np.arange(nb), shared))
    else:
        perm = rng.permutation(nb)
        shared, pool = perm[:37], perm[37:]
    counts = [int(x) for x in rng.integers(0, 60, size=9)]
    counts[2] = 0
    src_tables, k = [], 0
    for c in counts:
        src_tables.append(np.concatenate([shared, pool[k:k + c]]).astype(np.int32))
        k += c
    dst_pool = rng.permutation(nb)
    dst_tables, k = [], 0
    for t in src_tables:
        dst_tables.append(dst_pool[k:k + len(t)].astype(np.int32))
        k += len(t)
    words = spec.block_bytes // 2
    case = W.TransferCase("shared-prefix", spec, spec, [len(t) * bs for t in src_tables], src_tables,
                          dst_tables, 0,
                          src_caches=[W.random_words(rng, (nb, words)) for _ in range(L)],
                          dst_caches=[np.full((nb, words), W.SENTINEL16, np.uint16) for _ in range(L)])
    run_case(case)


def test_many_blocks_several_scan_tiles():
    """> 4 tiles of the run-list scan (8192 positions per tile), many requests, empty ones,
    small blocks so every wavefront spans many runs."""
    rng = np.random.default_rng(77)
    lengths = [int(x) for x in rng.integers(0, 320, size=1000)]
    for i in range(0, 1000, 37):
        lengths[i] = 0
    case = W.random_transfer(78, 2, 120000, 4, 1, 8, lengths, run_p=0.3)
    assert case.total_blocks > 4 * 8192
    run_case(case)


def test_offsets_beyond_the_lds_stage():
    """5000 requests: past the 4096 request offsets the run builder stages in LDS, so it reads
    them from global memory; a third of the requests are empty."""
    rng = np.random.default_rng(79)
    lengths = [int(x) for x in rng.integers(0, 40, size=5000)]
    for i in range(0, 5000, 3):
        lengths[i] = 0
    case = W.random_transfer(80, 1, 40000, 4, 1, 8, lengths, run_p=0.4)
    assert len(case.src_tables) >= 4096
    run_case(case)


@pytest.mark.parametrize("num_reqs,max_len,seed", [(8, 6000, 93), (200, 7000, 94), (255, 7000, 95),
                                                   (256, 7000, 96)])
def test_run_lists_few_requests_many_positions(num_reqs, max_len, seed):
    """Run lists in every mode from a few hundred requests or fewer over many positions of
    16-byte blocks: the builder's prefix pass takes several rounds, and past 524,288 positions
    each workgroup walks several sub-tiles. Up to 255 requests each builder thread handles one
    request start; 256 take the general path. Every fifth request is empty."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(1, max_len, size=num_reqs)]
    for i in range(0, num_reqs, 5):
        lengths[i] = 0
    case = W.random_transfer(seed, 1, 2_000_000, 1, 1, 8, lengths, elem_bytes=1, with_caches=False)
    if num_reqs > 8:
        assert case.total_blocks > 256 * 2048
    else:
        assert case.total_blocks > 4 * 4096
    K = kvx()
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    did, _ = K.flatten_tables(case.dst_tables, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    for mode, omode, a, b in ((K.MODE_PACK, O.MODE_PACK, sid, None),
                              (K.MODE_UNPACK, O.MODE_UNPACK, None, did),
                              (K.MODE_DIRECT, O.MODE_DIRECT, sid, did)):
        x, c = K.new_xfer_list(case.total_blocks, DEV)
        K.kvx_build_xfer_list(a, b, ro, mode, x, c, err)
        check_runs_equal(K, x, c, O.xfer_list(case.src_tables, case.dst_tables, omode))
    assert int(err.item()) == 0


def test_single_request_single_block():
    run_case(W.random_transfer(5, 1, 16, 16, 1, 8, [3]))


def test_all_blocks_one_run():
    """Source ids 0..N-1 in order and destination ids likewise: one run each way."""
    spec = W.PagedSpec(2, 512, 16, 1, 8)
    rng = np.random.default_rng(9)
    src = [W.random_words(rng, (512, spec.block_bytes // 2)) for _ in range(2)]
    dst = [np.full((512, spec.block_bytes // 2), W.SENTINEL16, np.uint16) for _ in range(2)]
    tables = [np.arange(0, 300, dtype=np.int32)]
    case = W.TransferCase("one-run", spec, spec, [300 * 16], tables, [np.arange(100, 400, dtype=np.int32)], 9,
                          src_caches=src, dst_caches=dst)
    t = run_case(case)
    assert int(t.cp.item()) == 1 and int(t.cu.item()) == 1


def test_empty_transfer():
    K = kvx()
    x, c = K.new_xfer_list(0, DEV)
    c.fill_(-1)
    ids = torch.zeros(0, dtype=torch.int32, device=DEV)
    ro = torch.zeros(3, dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(ids, None, ro, K.MODE_PACK, x, c, err)
    torch.cuda.synchronize()
    assert int(c.item()) == 0 and int(err.item()) == 0
    # packing zero blocks enqueues nothing and succeeds
    bases = torch.zeros(2, dtype=torch.int64, device=DEV)
    K.kvx_pack(bases, 2048, 10, x, c, 0, torch.empty(16, dtype=torch.uint8, device=DEV), err)


def test_direct_mode_runs():
    case = W.random_transfer(31, 1, 3000, 16, 1, 8, [900, 0, 450, 33], run_p=0.2, with_caches=False)
    K = kvx()
    src, ro = K.flatten_tables(case.src_tables, DEV)
    dst, _ = K.flatten_tables(case.dst_tables, DEV)
    x, c = K.new_xfer_list(case.total_blocks, DEV)
    K.kvx_build_xfer_list(src, dst, ro, K.MODE_DIRECT, x, c)
    torch.cuda.synchronize()
    check_runs_equal(K, x, c, O.xfer_list(case.src_tables, case.dst_tables, O.MODE_DIRECT))


def test_bad_offsets_flagged():
    K = kvx()
    ids = torch.arange(10, dtype=torch.int32, device=DEV)
    ro = torch.tensor([0, 6, 4, 10], dtype=torch.int64, device=DEV)  # decreasing
    x, c = K.new_xfer_list(10, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(ids, None, ro, K.MODE_PACK, x, c, err)
    torch.cuda.synchronize()
    assert int(err.item()) & K.DEVERR_OFFSETS
    assert 1 <= int(c.item()) <= 10


def test_out_of_range_ids_skipped_and_flagged():
    """Source id past the cache (pack) and destination ids past the cache or negative (unpack):
    skipped, flagged, everything else as the oracle says."""
    spec = W.PagedSpec(2, 40, 4, 1, 8)
    rng = np.random.default_rng(4)
    src = [W.random_words(rng, (40, spec.block_bytes // 2)) for _ in range(2)]
    dst = [np.full((40, spec.block_bytes // 2), W.SENTINEL16, np.uint16) for _ in range(2)]
    src_tables = [np.array([38, 39, 40, 41, 3], np.int32), np.array([7, 8], np.int32)]
    dst_tables = [np.array([0, 1, 2, 45, -1], np.int32), np.array([20, 21], np.int32)]
    case = W.TransferCase("oob", spec, spec, [20, 8], src_tables, dst_tables, 4, src_caches=src, dst_caches=dst)
    t = Transfer(case, layers_from_host(src, spec.block_bytes), layers_from_host(dst, spec.block_bytes))
    t.buf.zero_()
    t.run()
    buf, e1 = O.pack(src, src_tables)  # zeros where skipped, like the zeroed device buffer
    out, e2 = O.unpack([buf], dst, dst_tables)
    assert np.array_equal(host_bytes(t.buf)[: buf.nbytes], buf.reshape(-1))
    for l in range(2):
        assert np.array_equal(host_bytes(t.dst[l]).reshape(out[l].shape), out[l])
    assert t.err_bits() == (e1 | e2) == O.DEVERR_BLOCK_RANGE


# ------------------------------------------------------------------------- slot mapping

def test_slot_mapping_golden_and_errors():
    import json
    import os
    K = kvx()
    path = os.path.join(os.path.dirname(__file__), "golden", "slot_mapping_cases.json")
    for case in json.load(open(path))["cases"]:
        bt = to_dev(np.array(case["block_table"], np.int32))
        rq = to_dev(np.array(case["req_idx"], np.int32))
        pos = to_dev(np.array(case["positions"], np.int64))
        out = torch.empty(len(case["req_idx"]), dtype=torch.int64, device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        K.kvx_slot_mapping(bt, rq, pos, case["block_size"], out, err)
        torch.cuda.synchronize()
        exp, eerr = O.slot_mapping(np.array(case["block_table"]), case["req_idx"], case["positions"],
                                   case["block_size"])
        assert out.cpu().numpy().tolist() == exp.tolist(), case["name"]
        assert int(err.item()) == eerr, case["name"]


def test_slot_mapping_positions_past_32_bits():
    """Positions and slots beyond 2^31 take the kernels' 64-bit division: blocks of 2^30
    slots, positions up to 3 * 2^30 - 1."""
    K = kvx()
    bs = 1 << 30
    table = np.array([[7, 9, 11], [4, -1, 2]], np.int32)
    req = np.array([0, 0, 0, 1, 1, 1, 0], np.int32)
    pos = np.array([(1 << 31) + 5, 3 * bs - 1, 0, bs + 1, 2 * bs + 17, (1 << 31) - 1, 3 * bs], np.int64)
    slots = torch.empty(len(req), dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_slot_mapping(to_dev(table), to_dev(req), to_dev(pos), bs, slots, err)
    torch.cuda.synchronize()
    exp, e = O.slot_mapping(table, req, pos, bs)
    assert np.array_equal(slots.cpu().numpy(), exp)
    assert int(err.item()) == e == O.DEVERR_TABLE_RANGE


@pytest.mark.parametrize("row", [256, 1024], ids=["general", "whole-KiB"])
def test_reshape_and_cache_slots_past_32_bits(row):
    """Slots beyond 2^31 (blocks of 2^30 slots, only the first few used) in both write kernels."""
    K = kvx()
    bs, nb, bst, tst, kst = 1 << 30, 3, 64 << 10, 2 * row, row
    slots_h = np.array([2 * bs + 5, 3, bs + 7, -1, 3 * bs + 1, 2 * bs + 6], np.int64)
    T = len(slots_h)
    rng = np.random.default_rng(row)
    key = W.random_words(rng, (T, row // 2))
    val = W.random_words(rng, (T, row // 2))
    cache_h = np.full(nb * bst // 2, W.SENTINEL16, np.uint16)
    cache = to_dev(cache_h)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    reshape_and_cache_raw(K, to_dev(key), to_dev(val), to_dev(slots_h), cache, nb, bs, bst, tst, kst, err)
    torch.cuda.synchronize()
    exp, e = O.reshape_and_cache(cache_h, key, val, slots_h, nb, bs, bst, tst, kst)
    assert np.array_equal(host_bytes(cache), exp)
    assert int(err.item()) == e == O.DEVERR_SLOT_RANGE


def test_slot_mapping_decode_workload():
    """32 requests of 1..2048 tokens over a 4096-block table, all T tokens."""
    K = kvx()
    d = W.decode_write(with_values=False)
    out = torch.empty(len(d.req_idx), dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_slot_mapping(to_dev(d.block_table), to_dev(d.req_idx), to_dev(d.positions), 16, out, err)
    torch.cuda.synchronize()
    exp, eerr = O.slot_mapping(d.block_table, d.req_idx, d.positions, 16)
    assert np.array_equal(out.cpu().numpy(), exp) and int(err.item()) == eerr == 0


def test_slot_mapping_row_stride_and_width():
    """A block-table view with a row stride larger than its width, and a width limit."""
    K = kvx()
    full = np.arange(4 * 10, dtype=np.int32).reshape(4, 10)
    bt = to_dev(full)[:, :6]
    rq = np.array([0, 1, 2, 3, 3, 3], np.int32)
    pos = np.array([0, 17, 40, 63, 64, 95], np.int64)
    out = torch.empty(6, dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_slot_mapping(bt, to_dev(rq), to_dev(pos), 16, out, err, max_blocks_per_req=5)
    torch.cuda.synchronize()
    exp, eerr = O.slot_mapping(full[:, :5], rq, pos, 16)
    assert out.cpu().numpy().tolist() == exp.tolist() and int(err.item()) == eerr


# ------------------------------------------------------------------------- new-token write

def _reshape_check(d, layout, slots_np):
    K = kvx()
    s = d.spec
    nb, bs, H, D = s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim
    shape = {"blocks_tokens_kv": (nb, bs, 2, H, D), "blocks_kv_tokens": (nb, 2, bs, H, D),
             "kv_blocks_tokens": (2, nb, bs, H, D)}[layout]
    cache_h = np.full(shape, W.SENTINEL16, np.uint16)
    cache = to_dev(cache_h)
    _, _, bst, tst, kst = K.cache_strides(cache, layout)
    key, val = to_dev(d.key), to_dev(d.value)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_reshape_and_cache(key, val, to_dev(slots_np), cache, nb, bs, bst, tst, kst, err)
    torch.cuda.synchronize()
    exp, eerr = O.reshape_and_cache(cache_h, d.key, d.value, slots_np, nb, bs, bst, tst, kst)
    assert np.array_equal(host_bytes(cache), exp)
    assert int(err.item()) == eerr
    return exp


def test_reshape_and_cache_decode_workload():
    """1 layer [4096][16][K,V][8][128] bf16 sentinel-filled, 32 requests, every prompt token
    written through the slots computed by the GPU slot mapping."""
    K = kvx()
    d = W.decode_write()
    slots = torch.empty(len(d.req_idx), dtype=torch.int64, device=DEV)
    K.kvx_slot_mapping(to_dev(d.block_table), to_dev(d.req_idx), to_dev(d.positions), 16, slots)
    exp_slots, _ = O.slot_mapping(d.block_table, d.req_idx, d.positions, 16)
    assert np.array_equal(slots.cpu().numpy(), exp_slots)
    exp = _reshape_check(d, "blocks_tokens_kv", exp_slots)
    # sentinel everywhere outside the 2T written rows (tail slots of last blocks included)
    v = exp.view(np.uint16).reshape(d.spec.shape5)
    written = np.zeros(d.spec.shape5[:2], bool)
    written.reshape(-1)[exp_slots] = True
    assert np.all(v[~written] == W.SENTINEL16)


@pytest.mark.parametrize("layout", ["blocks_kv_tokens", "kv_blocks_tokens"])
def test_reshape_and_cache_other_layouts(layout):
    d = W.decode_write(seed=8, num_reqs=9, max_len=300, num_blocks=256, num_kv_heads=2, head_dim=64)
    slots, _ = O.slot_mapping(d.block_table, d.req_idx, d.positions, 16)
    _reshape_check(d, layout, slots)


def test_reshape_and_cache_padding_and_range():
    d = W.decode_write(seed=10, num_reqs=4, max_len=100, num_blocks=32, num_kv_heads=1, head_dim=8)
    slots, _ = O.slot_mapping(d.block_table, d.req_idx, d.positions, 16)
    slots = slots.copy()
    slots[::7] = -1
    slots[3] = 32 * 16 + 5  # block 32: past the cache
    _reshape_check(d, "blocks_tokens_kv", slots)


# ------------------------------------------------------------------------- head merge

@pytest.mark.parametrize("S,H,D,rows_tok", [(2, 8, 128, 2), (4, 8, 64, 2), (2, 2, 8, 2), (3, 6, 16, 2)])
def test_head_merge_small(S, H, D, rows_tok):
    """S head-split sources merged into full-head blocks at random destination ids."""
    K = kvx()
    bs, L = 16, 3
    dspec = W.PagedSpec(L, 300, bs, H, D)
    rng = np.random.default_rng(S * 100 + H)
    counts = [int(x) for x in rng.integers(0, 30, size=7)]
    dst_tables = W.pop_tables(rng.permutation(300), counts)
    N = sum(counts)
    BB = dspec.block_bytes
    srcs = [W.random_words(rng, (L, N, BB // S // 2)) for _ in range(S)]
    dst_h = [np.full((300, BB // 2), W.SENTINEL16, np.uint16) for _ in range(L)]
    dst = layers_from_host(dst_h, BB)
    ids, ro = K.flatten_tables(dst_tables, DEV)
    x, c = K.new_xfer_list(N, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_build_xfer_list(None, ids, ro, K.MODE_UNPACK, x, c, err)
    K.kvx_unpack([to_dev(s) for s in srcs], K.layer_base_table(dst), BB, 300, bs * rows_tok, x, c, N, err)
    torch.cuda.synchronize()
    exp, eerr = O.unpack(srcs, dst_h, dst_tables, rows_per_block=bs * rows_tok)
    for l in range(L):
        assert np.array_equal(host_bytes(dst[l]).reshape(exp[l].shape), exp[l]), l
    assert int(err.item()) == eerr == 0


@pytest.mark.parametrize("H,D", [(4, 128), (8, 128), (16, 128), (32, 128), (2, 256)])
@pytest.mark.parametrize("layout", ["blocks_tokens_kv", "blocks_kv_tokens", "kv_blocks_tokens"])
def test_reshape_and_cache_whole_kib_rows(H, D, layout):
    """Rows of 1, 2, 4 and 8 KiB take the one-batch write kernel (8 KiB rows spread one token
    over two wavefronts); padding tokens and a slot past the cache included."""
    d = W.decode_write(seed=H * 1000 + D, num_reqs=7, max_len=150, num_blocks=96, num_kv_heads=H, head_dim=D)
    slots, _ = O.slot_mapping(d.block_table, d.req_idx, d.positions, 16)
    slots = slots.copy()
    slots[5::11] = -1
    slots[2] = 96 * 16 + 3
    _reshape_check(d, layout, slots)


def test_reshape_and_cache_strided_rows():
    """K and V as views into one fused [T][3][H][D] tensor (row stride 3 rows)."""
    K = kvx()
    d = W.decode_write(seed=77, num_reqs=5, max_len=90, num_blocks=64, num_kv_heads=8, head_dim=128)
    T = len(d.req_idx)
    s = d.spec
    slots, _ = O.slot_mapping(d.block_table, d.req_idx, d.positions, 16)
    fused = np.zeros((T, 3, 8, 128), np.uint16)
    fused[:, 1] = d.key
    fused[:, 2] = d.value
    fused_d = to_dev(fused)
    cache_h = np.full(s.shape5, W.SENTINEL16, np.uint16)
    cache = to_dev(cache_h)
    nb, bs, bst, tst, kst = K.cache_strides(cache)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_reshape_and_cache(fused_d[:, 1], fused_d[:, 2], to_dev(slots), cache, nb, bs, bst, tst, kst, err)
    torch.cuda.synchronize()
    exp, e = O.reshape_and_cache(cache_h, d.key, d.value, slots, nb, bs, bst, tst, kst)
    assert np.array_equal(host_bytes(cache), exp) and int(err.item()) == e == 0
