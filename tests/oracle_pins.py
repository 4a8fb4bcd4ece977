"""Checks that pin the CPU oracle to something other than itself.

Each check takes the oracle module as an argument so the same checks can be run against
deliberately broken copies of it (see test_oracle_mutants.py). A check raises
AssertionError when the oracle disagrees with:
  * values worked by hand from the pages (tests/golden/*.json, each with its citation),
  * numpy library routines the step reduces to (fancy-index gather, index-put scatter),
  * brute-force element loops over the semantic 5-D layout (no byte-offset arithmetic),
  * invariants that hold for any input (run expansion, maximality, round trip).
"""
from __future__ import annotations

import json
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tagged_caches(num_layers, num_blocks, block_bytes):
    """Every byte of block b in layer l holds 10*l + b."""
    return [np.repeat((10 * l + np.arange(num_blocks)).astype(np.uint8)[:, None], block_bytes, 1)
            for l in range(num_layers)]


# --------------------------------------------------------------------------- slot mapping

def pin_slot_golden(o):
    for case in _golden("slot_mapping_cases.json")["cases"]:
        bt = np.array(case["block_table"], np.int32)
        slots, err = o.slot_mapping(bt, case["req_idx"], case["positions"], case["block_size"])
        assert slots.tolist() == case["expected"], case["name"]
        assert err == case.get("expected_err", 0), case["name"]


def pin_slot_outside_the_table(o):
    """Tokens the slot rule cannot place (the pages define only the in-range case; the reading
    taken is slot -1 and the table-range bit), on a table with no padding, so that an index
    taken from the wrong end of a row would land on a real block: a request index past the
    table or negative, a position negative or past its row. The in-range tokens beside them
    keep their slots by the slot rule."""
    bt = np.array([[5, 7], [2, 9]], np.int32)
    bs = 4
    req = [0, 0, 1, 2, -1, 0, 1]
    pos = [3, -1, 5, 0, 0, 8, 7]
    slots, err = o.slot_mapping(bt, req, pos, bs)
    assert slots.tolist() == [5 * 4 + 3, -1, 9 * 4 + 1, -1, -1, -1, 9 * 4 + 3]
    assert err == o.DEVERR_TABLE_RANGE


def pin_slot_owner_brute_force(o):
    """Walk every slot of every listed block and record which (request, position) owns it;
    each token's slot must be owned by that token."""
    d = W.decode_write(seed=5, num_reqs=6, max_len=70, num_blocks=64, num_kv_heads=1,
                       head_dim=8, with_values=False)
    bs = d.spec.block_size
    owner = {}
    for r, ids in enumerate(d.tables):
        pos = 0
        for b in ids:
            for t in range(bs):
                owner[int(b) * bs + t] = (r, pos)
                pos += 1
    slots, err = o.slot_mapping(d.block_table, d.req_idx, d.positions, bs)
    assert err == 0
    for i in range(len(slots)):
        assert owner[int(slots[i])] == (int(d.req_idx[i]), int(d.positions[i]))
    assert len(set(slots.tolist())) == len(slots)  # disjoint tables -> unique slots


# --------------------------------------------------------------------------- new-token write

def _decode_case(seed, H, D, num_blocks=48, num_reqs=5, max_len=60):
    d = W.decode_write(seed=seed, num_reqs=num_reqs, max_len=max_len, num_blocks=num_blocks,
                       num_kv_heads=H, head_dim=D)
    return d


def pin_reshape_readback_blocks_first(o):
    """[blocks][tokens][K,V][H][D]: read every token back through the 5-D view."""
    d = _decode_case(11, H=2, D=8)
    s = d.spec
    slots, _ = o.slot_mapping(d.block_table, d.req_idx, d.positions, s.block_size)
    cache = np.full(s.shape5, W.SENTINEL16, np.uint16)
    row = s.row_bytes
    out, err = o.reshape_and_cache(cache, d.key, d.value, slots, s.num_blocks, s.block_size,
                                   s.block_size * 2 * row, 2 * row, row)
    assert err == 0
    v5 = out.view(np.uint16).reshape(s.shape5)
    touched = np.zeros(s.shape5[:3], bool)
    for i, sl in enumerate(slots):
        b, t = divmod(int(sl), s.block_size)
        assert np.array_equal(v5[b, t, 0], d.key[i]) and np.array_equal(v5[b, t, 1], d.value[i])
        touched[b, t, :] = True
    assert np.all(v5[~touched] == W.SENTINEL16)
    assert touched.sum() == 2 * len(slots)


def pin_reshape_element_loop_kv_inner_layout(o):
    """(blocks, K/V, tokens, H, D) layout, element by element."""
    d = _decode_case(12, H=2, D=4, num_blocks=40, num_reqs=4, max_len=50)
    s = d.spec
    nb, bs, H, D = s.num_blocks, s.block_size, s.num_kv_heads, s.head_dim
    slots, _ = o.slot_mapping(d.block_table, d.req_idx, d.positions, bs)
    cache = np.full((nb, 2, bs, H, D), W.SENTINEL16, np.uint16)
    row = H * D * 2
    out, err = o.reshape_and_cache(cache, d.key, d.value, slots, nb, bs, 2 * bs * row, row, bs * row)
    v = out.view(np.uint16).reshape(nb, 2, bs, H, D)
    expect = np.full_like(v, W.SENTINEL16)
    for i, sl in enumerate(slots):
        b, t = int(sl) // bs, int(sl) % bs
        for h in range(H):
            for e in range(D):
                expect[b, 0, t, h, e] = d.key[i, h, e]
                expect[b, 1, t, h, e] = d.value[i, h, e]
    assert err == 0 and np.array_equal(v, expect)


def pin_reshape_kv_first_layout(o):
    """(K/V, blocks, tokens, H, D): the K and V planes are a whole cache apart."""
    d = _decode_case(13, H=1, D=8, num_blocks=40, num_reqs=4, max_len=50)
    s = d.spec
    nb, bs = s.num_blocks, s.block_size
    slots, _ = o.slot_mapping(d.block_table, d.req_idx, d.positions, bs)
    cache = np.full((2, nb, bs, 1, 8), W.SENTINEL16, np.uint16)
    row = 16
    out, err = o.reshape_and_cache(cache, d.key, d.value, slots, nb, bs, bs * row, row, nb * bs * row)
    v = out.view(np.uint16).reshape(2, nb, bs, 1, 8)
    for i, sl in enumerate(slots):
        b, t = divmod(int(sl), bs)
        assert np.array_equal(v[0, b, t], d.key[i]) and np.array_equal(v[1, b, t], d.value[i])
    assert err == 0


def pin_reshape_padding_and_range(o):
    """Negative slots are skipped silently (also when repeated); slots past the cache are
    skipped and flagged (also when repeated); every other token lands in its own slot."""
    cache = np.zeros((4, 2, 2, 1, 8), np.uint16)  # 4 blocks of 2 tokens, row = 16 B
    key = np.arange(5 * 8, dtype=np.uint16).reshape(5, 1, 8) + 1
    val = key + 100
    slots = [-1, 8, 3, 8, -1]
    out, err = o.reshape_and_cache(cache, key, val, slots, 4, 2, 64, 32, 16)
    v = out.view(np.uint16).reshape(4, 2, 2, 1, 8)
    assert err == o.DEVERR_SLOT_RANGE
    assert np.array_equal(v[1, 1, 0], key[2]) and np.array_equal(v[1, 1, 1], val[2])
    v[1, 1] = 0
    assert not v.any()


def _raises_value_error(fn):
    try:
        fn()
    except ValueError:
        return True
    return False


def pin_repeated_destinations_rejected(o):
    """Two entries that would write the same destination block (or slot) inside the cache
    are invalid input and every writing step refuses them, because a receiver allocates a
    fresh block for every listed block ("vLLM PD 分离" §三 3.2): no step picks a winner.
    Ids outside the cache are not writes, so repeating them is still allowed."""
    cache = np.zeros((4, 2, 2, 1, 8), np.uint16)
    key = np.ones((2, 1, 8), np.uint16)
    assert _raises_value_error(lambda: o.reshape_and_cache(cache, key, key, [3, 3], 4, 2, 64, 32, 16))
    assert _raises_value_error(lambda: o.reshape_and_cache(cache, key, key, [7, 7], 4, 2, 64, 32, 16))
    _, err = o.reshape_and_cache(cache, key, key, [8, 8], 4, 2, 64, 32, 16)
    assert err == o.DEVERR_SLOT_RANGE
    buf = np.arange(3 * 16, dtype=np.uint8).reshape(1, 3, 16)
    recv = [np.zeros((4, 16), np.uint8)]
    same_req = [np.array([2, 0, 2])]
    two_reqs = [np.array([1, 2]), np.array([2])]
    for tables in (same_req, two_reqs):
        assert _raises_value_error(lambda: o.unpack([buf], recv, tables))
        halves = [buf[:, :, :8], buf[:, :, 8:]]
        assert _raises_value_error(lambda: o.unpack(halves, recv, tables, rows_per_block=1))
        src_tables = [np.arange(len(t)) for t in tables]
        assert _raises_value_error(lambda: o.copy_direct([np.zeros((4, 16), np.uint8)], recv, src_tables, tables))
        kvf_buf = np.zeros((1, 6, 1024), np.uint8)
        kvf_recv = [np.zeros((2, 4, 1024), np.uint8)]
        assert _raises_value_error(lambda: o.unpack_kv_first(kvf_buf, kvf_recv, tables))
    out, err = o.unpack([buf], recv, [np.array([-1, 4, -1])])
    assert err == o.DEVERR_BLOCK_RANGE and not out[0].any()
    out, err = o.copy_direct([np.ones((4, 16), np.uint8)], recv, [np.array([0, 1, 2])], [np.array([4, 1, 4])])
    assert err == o.DEVERR_BLOCK_RANGE and out[0][1].all() and not out[0][[0, 2, 3]].any()
    out, err = o.unpack_kv_first(np.ones((1, 6, 1024), np.uint8), [np.zeros((2, 4, 1024), np.uint8)],
                                 [np.array([-1, 0, -1])])
    assert err == o.DEVERR_BLOCK_RANGE and out[0][:, 0].all() and not out[0][:, 1:].any()


# --------------------------------------------------------------------------- runs

def pin_xfer_golden(o):
    g = _golden("transfer_hw4.json")
    src = [np.array(t) for t in g["src_tables"]]
    dst = [np.array(t) for t in g["dst_tables"]]
    for mode, key in ((o.MODE_PACK, "runs_pack"), (o.MODE_UNPACK, "runs_unpack"),
                      (o.MODE_DIRECT, "runs_direct")):
        got = [list(x) for x in o.xfer_list(src, dst, mode)]
        assert got == g[key], key


def check_runs(runs, src_tables, dst_tables, mode):
    """Invariants any correct run list satisfies."""
    uses_src = mode in (0, 2)
    uses_dst = mode in (1, 2)
    flat_src = np.concatenate(src_tables) if uses_src else None
    flat_dst = np.concatenate(dst_tables) if uses_dst else None
    req_of = np.concatenate([np.full(len(t), r) for r, t in enumerate(src_tables if uses_src else dst_tables)])
    N = len(req_of)
    assert sum(n for *_, n, _ in runs) == N
    assert len(runs) <= N
    covered = 0
    for (s, d, b, n, r) in runs:
        assert b == covered and n >= 1
        assert np.all(req_of[b:b + n] == r)
        if uses_src:
            assert np.array_equal(flat_src[b:b + n], s + np.arange(n))
        else:
            assert s == b
        if uses_dst:
            assert np.array_equal(flat_dst[b:b + n], d + np.arange(n))
        else:
            assert d == b
        covered += n
    # maximal: the block after a run is in another request or breaks the +1 step
    for (s, d, b, n, r) in runs:
        e = b + n
        if e < N and req_of[e] == r:
            breaks = (uses_src and flat_src[e] != flat_src[e - 1] + 1) or \
                     (uses_dst and flat_dst[e] != flat_dst[e - 1] + 1)
            assert breaks


def pin_xfer_invariants(o):
    for seed in range(4):
        c = W.random_transfer(seed, 1, 600, 4, 1, 2, [5, 0, 61, 17, 1, 230], with_caches=False)
        for mode in (o.MODE_PACK, o.MODE_UNPACK, o.MODE_DIRECT):
            check_runs(o.xfer_list(c.src_tables, c.dst_tables, mode), c.src_tables, c.dst_tables, mode)


def pin_xfer_pages_contiguous_count(o):
    """Runs of 64 in their own slots: at most 9 runs per 576-block request (72 in all)."""
    c = W.pages_contiguous(num_layers=1)
    runs = o.xfer_list(c.src_tables, c.dst_tables, o.MODE_PACK)
    check_runs(runs, c.src_tables, c.dst_tables, o.MODE_PACK)
    assert len(runs) <= 72
    assert all(n % 64 == 0 for *_, n, _ in runs)


# --------------------------------------------------------------------------- pack

def pin_pack_golden(o):
    g = _golden("transfer_hw4.json")
    caches = _tagged_caches(g["num_layers"], g["num_blocks"], 16)
    buf, err = o.pack(caches, [np.array(t) for t in g["src_tables"]])
    assert err == 0
    assert buf.shape == (2, 6, 16)
    assert buf[:, :, 0].tolist() == g["buffer_tags"]
    assert np.all(buf == buf[:, :, :1])


def pin_pack_tiny_byte_offsets(o):
    g = _golden("byte_counts.json")["tiny_config"]
    c = W.tiny_roundtrip()
    bb = c.src_spec.block_bytes
    assert bb == g["block_bytes"]
    assert [len(t) for t in c.src_tables] == g["blocks_per_request"]
    buf, err = o.pack(c.src_caches, c.src_tables)
    flat = buf.reshape(-1)
    assert flat.nbytes == g["buffer_bytes"]
    for l in range(2):
        layer = c.src_caches[l].reshape(64, -1).view(np.uint8)
        for r, off in enumerate(g["request_offsets"]):
            at = l * g["layer1_offset"] + off
            assert np.array_equal(flat[at:at + bb], layer[c.src_tables[r][0]])


def pin_pack_pages_volume(o):
    """One layer of the pages' geometry (fewer blocks in the pool): 8 x 576 blocks of 8 KiB
    give the stated per-(request, layer) and per-layer volumes."""
    g = _golden("byte_counts.json")["pages_kv_memory"]
    c = W.pages_contiguous(num_layers=1, num_blocks=9216, run=64)
    spec = c.src_spec
    assert spec.block_bytes == g["block_bytes"]
    assert W.PagedSpec(48, 147456, 16, 1, 128).layer_bytes == g["layer_bytes"]
    layer = np.zeros((spec.num_blocks, spec.block_bytes), np.uint8)
    layer[:, :8] = np.arange(spec.num_blocks, dtype=np.uint64)[:, None].view(np.uint8)
    buf, _ = o.pack([layer], c.src_tables)
    assert buf.nbytes == g["layer_slice_bytes"]
    assert g["request_layer_bytes"] * g["requests"] == buf.nbytes
    ids = buf[0, :, :8].copy().view(np.uint64).reshape(-1)
    per = g["request_layer_bytes"] // g["block_bytes"]
    for r in range(g["requests"]):
        assert np.array_equal(ids[r * per:(r + 1) * per], c.src_tables[r])


def pin_pack_equals_fancy_index(o):
    c = W.random_transfer(21, 3, 300, 4, 2, 4, [9, 40, 0, 77, 3])
    buf, err = o.pack(c.src_caches, c.src_tables)
    for l in range(3):
        ref = np.concatenate([c.src_caches[l][t] for t in c.src_tables])
        assert np.array_equal(buf[l].view(np.uint16), ref)


def pin_pack_element_loop(o):
    spec = W.PagedSpec(2, 12, 2, 2, 2)
    rng = np.random.default_rng(3)
    caches = [W.random_words(rng, spec.shape5) for _ in range(2)]
    tables = [np.array([3, 4, 9]), np.array([0]), np.array([11, 5])]
    buf, err = o.pack(caches, tables)
    b5 = buf.view(np.uint16).reshape(2, 6, 2, 2, 2, 2)
    p = 0
    for r, t in enumerate(tables):
        for j, blk in enumerate(t):
            for l in range(2):
                for tok in range(2):
                    for kv in range(2):
                        for h in range(2):
                            for e in range(2):
                                assert b5[l, p, tok, kv, h, e] == caches[l][blk, tok, kv, h, e]
            p += 1


def pin_pack_out_of_range(o):
    caches = _tagged_caches(1, 4, 16)
    buf, err = o.pack(caches, [np.array([1, 4]), np.array([-1, 2])])
    assert err == o.DEVERR_BLOCK_RANGE
    assert buf[0, :, 0].tolist() == [1, 0, 0, 2]


# --------------------------------------------------------------------------- unpack

def pin_unpack_golden(o):
    g = _golden("transfer_hw4.json")
    caches = _tagged_caches(2, 8, 16)
    src = [np.array(t) for t in g["src_tables"]]
    dst = [np.array(t) for t in g["dst_tables"]]
    buf, _ = o.pack(caches, src)
    sentinel = [np.full((8, 16), 0xEE, np.uint8) for _ in range(2)]
    out, err = o.unpack([buf], sentinel, dst)
    assert err == 0
    for l in range(2):
        got = [None if np.all(out[l][b] == 0xEE) else int(out[l][b][0]) for b in range(8)]
        assert got == g["dst_tags_after_unpack"][l]


def pin_shared_prefix_golden(o):
    """Two requests sharing prefix blocks: runs in all three modes, the buffer (shared blocks
    appear once per request) and the receiver's blocks, all worked by hand."""
    g = _golden("prefix_sharing_hw8.json")
    src = [np.array(t) for t in g["src_tables"]]
    dst = [np.array(t) for t in g["dst_tables"]]
    for mode, key in ((o.MODE_PACK, "runs_pack"), (o.MODE_UNPACK, "runs_unpack"),
                      (o.MODE_DIRECT, "runs_direct")):
        assert [list(x) for x in o.xfer_list(src, dst, mode)] == g[key], key
    nb = g["num_blocks"]
    buf, err = o.pack(_tagged_caches(2, nb, 16), src)
    assert err == 0 and buf[:, :, 0].tolist() == g["buffer_tags"]
    assert np.all(buf == buf[:, :, :1])
    out, err = o.unpack([buf], [np.full((nb, 16), 0xEE, np.uint8) for _ in range(2)], dst)
    assert err == 0
    for l in range(2):
        got = [None if np.all(out[l][b] == 0xEE) else int(out[l][b][0]) for b in range(nb)]
        assert got == g["dst_tags_after_unpack"][l]


def pin_direct_golden(o):
    """A direct cache-to-cache transfer leaves the receiver's blocks exactly as pack then
    unpack does, for both hand-worked cases (HW4 and the shared-prefix HW8)."""
    for name in ("transfer_hw4.json", "prefix_sharing_hw8.json"):
        g = _golden(name)
        nb = g["num_blocks"]
        src = [np.array(t) for t in g["src_tables"]]
        dst = [np.array(t) for t in g["dst_tables"]]
        out, err = o.copy_direct(_tagged_caches(2, nb, 16), [np.full((nb, 16), 0xEE, np.uint8)] * 2,
                                 src, dst)
        assert err == 0
        for l in range(2):
            got = [None if np.all(out[l][b] == 0xEE) else int(out[l][b][0]) for b in range(nb)]
            assert got == g["dst_tags_after_unpack"][l], name


def pin_direct_equals_pack_then_unpack(o):
    for seed in range(3):
        c = W.random_transfer(300 + seed, 2, 300, 4, 1, 8, [37, 0, 90, 5, 211])
        buf, e1 = o.pack(c.src_caches, c.src_tables)
        want, e2 = o.unpack([buf], c.dst_caches, c.dst_tables)
        got, e3 = o.copy_direct(c.src_caches, c.dst_caches, c.src_tables, c.dst_tables)
        assert e1 == e2 == e3 == 0
        for l in range(2):
            assert np.array_equal(got[l], want[l])


def pin_direct_out_of_range(o):
    """An entry with either id out of range moves nothing; every other entry moves."""
    caches = _tagged_caches(1, 8, 16)
    before = [np.full((6, 16), 0xEE, np.uint8)]
    out, err = o.copy_direct(caches, before, [np.array([1, 9, 3]), np.array([-1, 4, 2])],
                             [np.array([0, 1, 7]), np.array([2, 5, -1])])
    assert err == o.DEVERR_BLOCK_RANGE
    got = [None if np.all(out[0][b] == 0xEE) else int(out[0][b][0]) for b in range(6)]
    assert got == [1, None, None, None, None, 4]


def pin_unpack_equals_index_put(o):
    c = W.random_transfer(22, 2, 200, 4, 2, 4, [13, 0, 50, 7])
    buf, _ = o.pack(c.src_caches, c.src_tables)
    out, err = o.unpack([buf], c.dst_caches, c.dst_tables)
    for l in range(2):
        ref = c.dst_caches[l].copy()
        ref[np.concatenate(c.dst_tables)] = buf[l].view(np.uint16)
        assert np.array_equal(out[l].view(np.uint16), ref)


def pin_roundtrip(o):
    c = W.tiny_roundtrip()
    buf, _ = o.pack(c.src_caches, c.src_tables)
    out, err = o.unpack([buf], c.dst_caches, c.dst_tables)
    assert err == 0
    listed = np.concatenate(c.dst_tables)
    for l in range(2):
        src = c.src_caches[l].reshape(64, -1)
        got = out[l].view(np.uint16)
        assert np.array_equal(got[listed], src[np.concatenate(c.src_tables)])
        rest = np.setdiff1d(np.arange(64), listed)
        assert np.all(got[rest] == W.SENTINEL16)
    # packing with the receiver's ids and unpacking with the same ids reproduces them
    buf2, _ = o.pack(out, c.dst_tables)
    assert np.array_equal(buf2, buf)


def pin_unpack_out_of_range(o):
    """Ids past the cache and negative ids are both skipped (a negative id must not wrap
    around to the last block)."""
    buf = np.arange(4 * 16, dtype=np.uint8).reshape(1, 4, 16)
    out, err = o.unpack([buf], [np.zeros((4, 16), np.uint8)], [np.array([3, 7]), np.array([0, -1])])
    assert err == o.DEVERR_BLOCK_RANGE
    assert np.array_equal(out[0][3], buf[0, 0]) and np.array_equal(out[0][0], buf[0, 2])
    assert not out[0][1].any() and not out[0][2].any()


def pin_head_merge_golden(o):
    g = _golden("head_merge_hw6.json")
    s0 = np.array(g["src0"], np.uint16)
    s1 = np.array(g["src1"], np.uint16)
    got = o.unpack_block([s0, s1], g["rows_per_block"]).view(np.uint16).reshape(2, 4)
    assert got.tolist() == g["expected"]


def pin_head_merge_element_loop(o):
    """Each destination element (token, K/V, head h, dim) comes from sender h // (H/S), local
    head h % (H/S), at the same buffer position."""
    for S in (2, 4):
        H, D, bs, L = 4, 2, 2, 2
        dspec = W.PagedSpec(L, 10, bs, H, D)
        rng = np.random.default_rng(S)
        tables = [np.array([7, 2, 3]), np.array([9])]
        N = 4
        bufs = [W.random_words(rng, (L, N, bs, 2, H // S, D)) for _ in range(S)]
        dst = [np.full(dspec.shape5, W.SENTINEL16, np.uint16) for _ in range(L)]
        out, err = o.unpack(bufs, dst, tables, rows_per_block=bs * 2)
        p = 0
        for r, t in enumerate(tables):
            for j, blk in enumerate(t):
                for l in range(L):
                    got = out[l].view(np.uint16).reshape(dspec.shape5)
                    for tok in range(bs):
                        for kv in range(2):
                            for h in range(H):
                                for e in range(D):
                                    s, hl = h // (H // S), h % (H // S)
                                    assert got[blk, tok, kv, h, e] == bufs[s][l, p, tok, kv, hl, e]
                p += 1


def pin_head_merge_one_source_is_plain(o):
    c = W.random_transfer(23, 1, 50, 2, 2, 4, [9, 4])
    buf, _ = o.pack(c.src_caches, c.src_tables)
    a, _ = o.unpack([buf], c.dst_caches, c.dst_tables, rows_per_block=4)
    b, _ = o.unpack([buf], c.dst_caches, c.dst_tables, rows_per_block=1)
    assert np.array_equal(a[0], b[0])




# --------------------------------------------------------------------------- kv-first (f1)

def _kv_first_tagged(num_blocks, seg):
    c = np.zeros((2, num_blocks, seg), np.uint8)
    for b in range(num_blocks):
        c[0, b] = 10 + b
        c[1, b] = 20 + b
    return c


def pin_kv_first_golden(o):
    g = _golden("kv_first_hw7.json")
    cache = _kv_first_tagged(g["num_blocks"], 16)
    src = [np.array(t) for t in g["src_tables"]]
    dst = [np.array(t) for t in g["dst_tables"]]
    buf, err = o.pack_kv_first([cache], src)
    assert err == 0 and buf.shape == (1, 6, 16)
    assert buf[0, :, 0].tolist() == g["buffer_tags"] and np.all(buf == buf[:, :, :1])
    out, err = o.unpack_kv_first(buf, [np.zeros_like(cache)], dst)
    got = [[None if not out[0][kv, b].any() else int(out[0][kv, b][0]) for b in range(4)] for kv in range(2)]
    assert err == 0 and got == g["dst_plane_tags_after_unpack"]


def pin_kv_first_equals_block_axis_gather(o):
    """Each request's slice equals numpy's gather along the block axis, layer[:, ids]."""
    rng = np.random.default_rng(31)
    caches = [W.random_words(rng, (2, 40, 4, 2, 8)) for _ in range(2)]
    tables = [np.array([5, 6, 7, 1]), np.array([], dtype=np.int64), np.array([39, 0, 2])]
    buf, err = o.pack_kv_first(caches, tables)
    for l in range(2):
        ref = np.concatenate([caches[l][:, t].reshape(-1) for t in tables]).view(np.uint8)
        assert np.array_equal(buf[l].reshape(-1), ref)


def pin_kv_first_element_loop(o):
    rng = np.random.default_rng(32)
    nb, bs, H, D = 9, 2, 2, 2
    cache = W.random_words(rng, (2, nb, bs, H, D))
    tables = [np.array([4, 1]), np.array([8])]
    buf, _ = o.pack_kv_first([cache], tables)
    b5 = buf.view(np.uint16).reshape(1, 6, bs, H, D)
    seg_at = 0
    for t in tables:
        for kv in range(2):
            for blk in t:
                for tok in range(bs):
                    for h in range(H):
                        for e in range(D):
                            assert b5[0, seg_at, tok, h, e] == cache[kv, blk, tok, h, e]
                seg_at += 1


def pin_kv_first_roundtrip(o):
    rng = np.random.default_rng(33)
    src = [W.random_words(rng, (2, 50, 64)) for _ in range(3)]
    s_tab = [np.array([3, 4, 5, 9]), np.array([0]), np.array([], dtype=np.int64), np.array([49, 48])]
    d_tab = [np.array([10, 11, 30, 31]), np.array([2]), np.array([], dtype=np.int64), np.array([0, 1])]
    buf, _ = o.pack_kv_first(src, s_tab)
    dst = [np.full((2, 50, 64), W.SENTINEL16, np.uint16) for _ in range(3)]
    out, err = o.unpack_kv_first(buf, dst, d_tab)
    listed = np.concatenate(d_tab).astype(int)
    for l in range(3):
        got = out[l].view(np.uint16).reshape(2, 50, 64)
        assert np.array_equal(got[:, listed], src[l][:, np.concatenate(s_tab).astype(int)])
        rest = np.setdiff1d(np.arange(50), listed)
        assert np.all(got[:, rest] == W.SENTINEL16)


def pin_kv_first_out_of_range(o):
    cache = _kv_first_tagged(4, 16)
    buf, err = o.pack_kv_first([cache], [np.array([1, 4]), np.array([-1])])
    assert err == o.DEVERR_BLOCK_RANGE
    assert buf[0, :, 0].tolist() == [11, 0, 21, 0, 0, 0]
    out, err = o.unpack_kv_first(buf, [np.zeros_like(cache)], [np.array([2, -1]), np.array([7])])
    assert err == o.DEVERR_BLOCK_RANGE
    assert out[0][0, 2, 0] == 11 and out[0][1, 2, 0] == 21
    assert out[0][:, [0, 1, 3]].sum() == 0


# --------------------------------------------------------------------------- head split (f2)

def pin_split_golden(o):
    """HW6 read backwards: splitting the merged rows gives back the two senders' rows."""
    g = _golden("head_merge_hw6.json")
    full = np.array(g["expected"], np.uint16)
    s0, s1 = o.split_block(full, 2, g["rows_per_block"])
    assert s0.view(np.uint16).reshape(2, 2).tolist() == g["src0"]
    assert s1.view(np.uint16).reshape(2, 2).tolist() == g["src1"]


def pin_split_element_loop(o):
    """Shard d holds heads [d*H/S, (d+1)*H/S) of every (token, K/V) row."""
    for S in (2, 4):
        rng = np.random.default_rng(40 + S)
        nb, bs, H, D = 12, 2, 4, 2
        caches = [W.random_words(rng, (nb, bs, 2, H, D)) for _ in range(2)]
        tables = [np.array([3, 9, 10]), np.array([0])]
        bufs, err = o.pack_split(caches, tables, S, rows_per_block=bs * 2)
        assert err == 0
        for d in range(S):
            v = bufs[d].view(np.uint16).reshape(2, 4, bs, 2, H // S, D)
            p = 0
            for t in tables:
                for blk in t:
                    for l in range(2):
                        for tok in range(bs):
                            for kv in range(2):
                                for h in range(H // S):
                                    for e in range(D):
                                        assert v[l, p, tok, kv, h, e] == caches[l][blk, tok, kv, d * (H // S) + h, e]
                    p += 1


def pin_split_then_merge_is_pack(o):
    c = W.random_transfer(44, 2, 80, 4, 4, 8, [20, 0, 35, 6])
    for S in (2, 4):
        bufs, e1 = o.pack_split(c.src_caches, c.src_tables, S, rows_per_block=8)
        merged, e2 = o.unpack(bufs, c.dst_caches, c.dst_tables, rows_per_block=8)
        buf, _ = o.pack(c.src_caches, c.src_tables)
        plain, _ = o.unpack([buf], c.dst_caches, c.dst_tables)
        assert e1 == e2 == 0
        for l in range(2):
            assert np.array_equal(merged[l], plain[l])


def pin_empty_transfer(o):
    """No listed block (no requests, or only empty ones): no runs, an empty buffer, and every
    receiving cache keeps its bytes, in every copy form."""
    rng = np.random.default_rng(41)
    src = [W.random_words(rng, (12, 64)) for _ in range(2)]
    dst = [W.random_words(rng, (12, 64)) for _ in range(2)]
    for tables in ([], [np.zeros(0, np.int32), np.zeros(0, np.int32)]):
        for mode in (o.MODE_PACK, o.MODE_UNPACK, o.MODE_DIRECT):
            assert o.xfer_list(tables, tables, mode) == []
        buf, err = o.pack(src, tables)
        assert err == 0 and buf.shape == (2, 0, 128)
        out, err = o.unpack([buf], dst, tables)
        assert err == 0 and all(np.array_equal(a, b.view(np.uint8)) for a, b in zip(out, dst))
        out, err = o.copy_direct(src, dst, tables, tables)
        assert err == 0 and all(np.array_equal(a, b.view(np.uint8)) for a, b in zip(out, dst))
        kplanes = [c.reshape(2, 12, 32) for c in src]
        dplanes = [c.reshape(2, 12, 32) for c in dst]
        kbuf, err = o.pack_kv_first(kplanes, tables)
        assert err == 0 and kbuf.shape == (2, 0, 64)
        out, err = o.unpack_kv_first(kbuf, dplanes, tables)
        assert err == 0 and all(np.array_equal(a, b.view(np.uint8)) for a, b in zip(out, dplanes))
        shards, err = o.pack_split(src, tables, 2, rows_per_block=4)
        assert err == 0 and [s.shape for s in shards] == [(2, 0, 64)] * 2
        out, err = o.unpack(shards, dst, tables, rows_per_block=4)
        assert err == 0 and all(np.array_equal(a, b.view(np.uint8)) for a, b in zip(out, dst))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
