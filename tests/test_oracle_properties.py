"""The CPU oracle against brute-force element loops on hypothesis-drawn tiny shapes (no GPU).

Each property draws a geometry (block size, heads, head width, layers, cache size) and tables
(empty requests, shared source blocks, ids outside the cache on either side), runs one oracle
function and checks every element of its output through the semantic 5-D layout
[block][token][K,V][head][dim] with plain index loops: no byte offsets, no slicing of blocks.
The pages fix what each element must hold: the gather and scatter of whole blocks by id (nccl
page §2.4), the transfer-list runs of consecutive ids (flagcx page §1.2), the slot rule of the
v1 diagram's batch-tensor label, and the head mapping of asymmetric TP (pd page §四 4.2, with
the contiguous head-range reading)."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O
import workloads as W

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def transfers(draw, even_heads=False):
    bs = draw(st.integers(1, 4))
    H = draw(st.sampled_from([2, 4])) if even_heads else draw(st.integers(1, 3))
    D = draw(st.sampled_from([4, 8]))  # 2-byte elements: rows of 8 or 16 bytes per head
    L = draw(st.integers(1, 2))
    nb = draw(st.integers(1, 10))
    R = draw(st.integers(0, 4))
    counts = [draw(st.integers(0, 4)) for _ in range(R)]
    pool = draw(st.permutations(list(range(-2, nb + 2))))  # distinct destination ids
    total = 0
    for r in range(R):
        counts[r] = min(counts[r], len(pool) - total)
        total += counts[r]
    src = [np.array(draw(st.lists(st.integers(-1, nb), min_size=c, max_size=c)), np.int64) for c in counts]
    dst, at = [], 0
    for c in counts:
        dst.append(np.array(pool[at:at + c], np.int64))
        at += c
    seed = draw(st.integers(0, 2 ** 31))
    return bs, H, D, L, nb, src, dst, seed


def _order(tables):
    """(request, index, buffer position) in buffer order."""
    out, p = [], 0
    for r, t in enumerate(tables):
        for j in range(len(t)):
            out.append((r, j, p))
            p += 1
    return out


@SETTINGS
@given(transfers())
def test_pack_unpack_direct_element_loops(case):
    bs, H, D, L, nb, src, dst, seed = case
    rng = np.random.default_rng(seed)
    shape = (nb, bs, 2, H, D)
    caches = [W.random_words(rng, shape) for _ in range(L)]
    recv = [W.random_words(rng, shape) for _ in range(L)]
    order = _order(src)
    N = len(order)

    buf, e_pack = O.pack(caches, src)
    b5 = buf.view(np.uint16).reshape((L, N) + shape[1:])
    bad_src = any(not 0 <= int(src[r][j]) < nb for r, j, _ in order)
    assert e_pack == (O.DEVERR_BLOCK_RANGE if bad_src else 0)
    for l in range(L):
        for r, j, p in order:
            b = int(src[r][j])
            for t in range(bs):
                for kv in range(2):
                    for h in range(H):
                        for e in range(D):
                            want = caches[l][b, t, kv, h, e] if 0 <= b < nb else 0
                            assert b5[l, p, t, kv, h, e] == want

    out, e_unpack = O.unpack([buf], recv, dst)
    bad_dst = any(not 0 <= int(dst[r][j]) < nb for r, j, _ in order)
    assert e_unpack == (O.DEVERR_BLOCK_RANGE if bad_dst else 0)
    owner = {int(dst[r][j]): p for r, j, p in order if 0 <= int(dst[r][j]) < nb}
    for l in range(L):
        o5 = out[l].view(np.uint16).reshape(shape)
        for d in range(nb):
            for t in range(bs):
                for kv in range(2):
                    for h in range(H):
                        for e in range(D):
                            want = b5[l, owner[d], t, kv, h, e] if d in owner else recv[l][d, t, kv, h, e]
                            assert o5[d, t, kv, h, e] == want

    direct, e_direct = O.copy_direct(caches, recv, src, dst)
    pairs = {}
    for r, j, _ in order:
        s, d = int(src[r][j]), int(dst[r][j])
        if 0 <= s < nb and 0 <= d < nb:
            pairs[d] = s
    assert e_direct == (O.DEVERR_BLOCK_RANGE if (bad_src or bad_dst) else 0)
    for l in range(L):
        o5 = direct[l].view(np.uint16).reshape(shape)
        for d in range(nb):
            for t in range(bs):
                for kv in range(2):
                    for h in range(H):
                        for e in range(D):
                            want = caches[l][pairs[d], t, kv, h, e] if d in pairs else recv[l][d, t, kv, h, e]
                            assert o5[d, t, kv, h, e] == want


@SETTINGS
@given(transfers())
def test_runs_expand_to_the_tables_and_are_maximal(case):
    _, _, _, _, _, src, dst, _ = case
    for mode in (O.MODE_PACK, O.MODE_UNPACK, O.MODE_DIRECT):
        runs = O.xfer_list(src, dst, mode)
        # expanding every run position by position gives back the tables in buffer order
        got = []
        for s, d, b, n, r in runs:
            assert n >= 1
            for i in range(n):
                got.append((r, (s + i) if mode != O.MODE_UNPACK else None,
                            (d + i) if mode != O.MODE_PACK else None, b + i))
        want = [(r, int(src[r][j]) if mode != O.MODE_UNPACK else None,
                 int(dst[r][j]) if mode != O.MODE_PACK else None, p) for r, j, p in _order(src)]
        assert got == want
        # maximal: two neighbouring runs of one request could not have been one run
        for (s0, d0, b0, n0, r0), (s1, d1, b1, n1, r1) in zip(runs, runs[1:]):
            if r0 == r1:
                joins_src = mode == O.MODE_UNPACK or s1 == s0 + n0
                joins_dst = mode == O.MODE_PACK or d1 == d0 + n0
                assert not (joins_src and joins_dst)


@SETTINGS
@given(transfers(even_heads=True), st.sampled_from([2]))
def test_head_merge_and_split_element_loops(case, S):
    bs, H, D, L, nb, _, dst, seed = case
    rng = np.random.default_rng(seed)
    shape = (nb, bs, 2, H, D)
    order = _order(dst)
    N = len(order)
    Hs = H // S
    shards = [W.random_words(rng, (L, N, bs, 2, Hs, D)) for _ in range(S)]
    recv = [W.random_words(rng, shape) for _ in range(L)]
    out, err = O.unpack(shards, recv, dst, rows_per_block=bs * 2)
    owner = {int(dst[r][j]): p for r, j, p in order if 0 <= int(dst[r][j]) < nb}
    for l in range(L):
        o5 = out[l].view(np.uint16).reshape(shape)
        for d in range(nb):
            for t in range(bs):
                for kv in range(2):
                    for h in range(H):
                        for e in range(D):
                            if d in owner:
                                want = shards[h // Hs][l, owner[d], t, kv, h % Hs, e]
                            else:
                                want = recv[l][d, t, kv, h, e]
                            assert o5[d, t, kv, h, e] == want
    # the split of a full-head cache puts head h of every listed block in shard h // Hs
    caches = [W.random_words(rng, shape) for _ in range(L)]
    split, e_split = O.pack_split(caches, dst, S, rows_per_block=bs * 2)
    for s in range(S):
        s5 = split[s].view(np.uint16).reshape(L, N, bs, 2, Hs, D)
        for l in range(L):
            for r, j, p in order:
                b = int(dst[r][j])
                for t in range(bs):
                    for kv in range(2):
                        for h in range(Hs):
                            for e in range(D):
                                want = caches[l][b, t, kv, s * Hs + h, e] if 0 <= b < nb else 0
                                assert s5[l, p, t, kv, h, e] == want


@SETTINGS
@given(transfers())
def test_kv_first_element_loops(case):
    bs, H, D, L, nb, src, dst, seed = case
    rng = np.random.default_rng(seed)
    shape = (2, nb, bs, H, D)
    caches = [W.random_words(rng, shape) for _ in range(L)]
    recv = [W.random_words(rng, shape) for _ in range(L)]
    buf, _ = O.pack_kv_first(caches, src)
    N = sum(len(t) for t in src)
    b6 = buf.view(np.uint16).reshape(L, 2 * N, bs, H, D)
    for l in range(L):
        at = 0
        for t_ in src:
            for kv in range(2):
                for b in t_:
                    b = int(b)
                    for t in range(bs):
                        for h in range(H):
                            for e in range(D):
                                want = caches[l][kv, b, t, h, e] if 0 <= b < nb else 0
                                assert b6[l, at, t, h, e] == want
                    at += 1
    out, _ = O.unpack_kv_first(buf, recv, dst)
    for l in range(L):
        o5 = out[l].view(np.uint16).reshape(shape)
        written = {}
        at = 0
        for t_ in dst:
            for kv in range(2):
                for d in t_:
                    if 0 <= int(d) < nb:
                        written[(kv, int(d))] = at
                    at += 1
        for kv in range(2):
            for d in range(nb):
                for t in range(bs):
                    for h in range(H):
                        for e in range(D):
                            if (kv, d) in written:
                                want = b6[l, written[(kv, d)], t, h, e]
                            else:
                                want = recv[l][kv, d, t, h, e]
                            assert o5[kv, d, t, h, e] == want


@SETTINGS
@given(st.integers(1, 4), st.integers(1, 3), st.sampled_from([4, 8]), st.integers(2, 8),
       st.sampled_from(["blocks_tokens_kv", "blocks_kv_tokens", "kv_blocks_tokens"]),
       st.integers(0, 2 ** 31))
def test_slot_rule_and_write_element_loops(bs, H, D, nb, layout, seed):
    """Slots from the slot rule written element by element into one of three layouts."""
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 4))
    width = nb // R
    ids = rng.permutation(nb)
    bt = np.full((R, width), -1, np.int32)
    for r in range(R):
        bt[r] = ids[r * width:(r + 1) * width]
    req = rng.integers(0, R, size=12).astype(np.int32)
    pos = rng.integers(0, width * bs + 2, size=12).astype(np.int64)  # some past the table
    slots, err = O.slot_mapping(bt, req, pos, bs)
    for i in range(12):
        c = int(pos[i]) // bs
        want = int(bt[req[i], c]) * bs + int(pos[i]) % bs if c < width else -1
        assert int(slots[i]) == want
    assert err == (O.DEVERR_TABLE_RANGE if (slots < 0).any() else 0)
    # keep the first writer of each slot (the write assumes distinct slots)
    seen, keep = set(), []
    for i, s in enumerate(slots.tolist()):
        if s < 0 or s not in seen:
            keep.append(i)
            seen.add(s)
    slots = slots[keep]
    T = len(slots)
    key = W.random_words(rng, (T, H, D))
    val = W.random_words(rng, (T, H, D))
    dims = {"blocks_tokens_kv": (nb, bs, 2, H, D), "blocks_kv_tokens": (nb, 2, bs, H, D),
            "kv_blocks_tokens": (2, nb, bs, H, D)}[layout]
    cache = W.random_words(rng, dims)
    row = H * D * 2
    bst, tst, kst = {"blocks_tokens_kv": (bs * 2 * row, 2 * row, row),
                     "blocks_kv_tokens": (2 * bs * row, row, bs * row),
                     "kv_blocks_tokens": (bs * row, row, nb * bs * row)}[layout]
    out, e = O.reshape_and_cache(cache, key, val, slots, nb, bs, bst, tst, kst)
    assert e == 0
    o5 = out.view(np.uint16).reshape(dims)

    def at(blk, t, kv, h, d):
        return {"blocks_tokens_kv": (blk, t, kv, h, d), "blocks_kv_tokens": (blk, kv, t, h, d),
                "kv_blocks_tokens": (kv, blk, t, h, d)}[layout]

    written = {}
    for i, s in enumerate(slots.tolist()):
        if s >= 0:
            written[(s // bs, s % bs)] = i
    for blk in range(nb):
        for t in range(bs):
            for kv in range(2):
                for h in range(H):
                    for d in range(D):
                        i = written.get((blk, t))
                        if i is None:
                            want = cache[at(blk, t, kv, h, d)]
                        else:
                            want = (key if kv == 0 else val)[i, h, d]
                        assert o5[at(blk, t, kv, h, d)] == want
