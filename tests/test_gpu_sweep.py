"""GPU parity over a seeded sweep of random small cases. Each case draws a geometry (block
size, heads, head width, element size, layer count), a request mix (empty requests, single
blocks, long and short runs) and, in some cases, ids outside the caches; every entry point
the geometry admits then runs through the C ABI and is compared byte for byte with the
oracle on the same inputs: the run lists in all three modes, pack, unpack, the direct copy,
the kv-first view of the same caches, the head split and merge, and the slot mapping with
the new-token write in a random cache layout."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, check_runs_equal, host_bytes, kvx, layers_from_host, log, to_dev

pytestmark = pytest.mark.gpu

NUM_CASES = 256


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"start {request.node.name}")
    yield
    torch.cuda.synchronize()
    log(f"end {request.node.name}")


def _draw(seed):
    """A random transfer case; returns (case, geometry tuple, corrupted)."""
    rng = np.random.default_rng(90_000 + seed)
    bs = int(rng.choice([1, 2, 4, 8, 16, 32]))
    H = int(rng.choice([1, 2, 3, 4, 8]))
    D = int(rng.choice([8, 16, 40, 64, 128]))
    e = int(rng.choice([1, 2]))
    L = int(rng.integers(1, 4))
    BB = W.PagedSpec(L, 1, bs, H, D, e).block_bytes
    nb = int(max(16, min(2500, (6 << 20) // BB)))
    R = int(rng.integers(0, 13))
    cap = max(1, nb // (3 * max(R, 1)))
    counts = [int(rng.integers(0, cap + 1)) for _ in range(R)]
    if R and rng.random() < 0.3:
        counts[int(rng.integers(0, R))] = 1
    lengths = [c * bs - int(rng.integers(0, bs)) if c else 0 for c in counts]
    p = float(rng.choice([0.15, 0.5, 0.9]))
    case = W.random_transfer(int(rng.integers(1 << 30)), L, nb, bs, H, D, lengths, elem_bytes=e, run_p=p)
    corrupted = False
    N = case.total_blocks
    if N and rng.random() < 0.3:
        corrupted = True
        src_tables = [t.copy() for t in case.src_tables]
        dst_tables = [t.copy() for t in case.dst_tables]
        flat = [(r, j) for r, t in enumerate(src_tables) for j in range(len(t))]
        r, j = flat[int(rng.integers(0, N))]
        src_tables[r][j] = int(rng.choice([nb, nb + 7, -1]))
        r, j = flat[int(rng.integers(0, N))]
        dst_tables[r][j] = int(rng.choice([nb, -3]))
        case.src_tables, case.dst_tables = src_tables, dst_tables
    return case, (bs, H, D, e), corrupted


@pytest.mark.parametrize("seed", range(NUM_CASES))
def test_random_case_all_copies(seed):
    K = kvx()
    case, (bs, H, D, e), corrupted = _draw(seed)
    spec = case.src_spec
    L, nb, BB, N = spec.num_layers, spec.num_blocks, spec.block_bytes, case.total_blocks
    log(f"seed {seed}: L={L} nb={nb} block_bytes={BB} requests={len(case.src_tables)} N={N} "
        f"corrupted={corrupted}")
    src = layers_from_host(case.src_caches, BB)
    sbase = K.layer_base_table(src)
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    did, _ = K.flatten_tables(case.dst_tables, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)

    # run lists, all three modes
    lists = {}
    for mode, name in ((K.MODE_PACK, "pack"), (K.MODE_UNPACK, "unpack"), (K.MODE_DIRECT, "direct")):
        x, c = K.new_xfer_list(N, DEV)
        K.kvx_build_xfer_list(sid if mode != K.MODE_UNPACK else None,
                              did if mode != K.MODE_PACK else None, ro, mode, x, c, err)
        lists[name] = (x, c)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for name, mode in (("pack", O.MODE_PACK), ("unpack", O.MODE_UNPACK), ("direct", O.MODE_DIRECT)):
        check_runs_equal(K, *lists[name], O.xfer_list(case.src_tables, case.dst_tables, mode))
    xp, cp = lists["pack"]
    xu, cu = lists["unpack"]

    # pack -> unpack
    buf = torch.zeros(max(L * N * BB, 16), dtype=torch.uint8, device=DEV)
    dst = layers_from_host(case.dst_caches, BB)
    K.kvx_pack(sbase, BB, nb, xp, cp, N, buf, err)
    K.kvx_unpack([buf], K.layer_base_table(dst), BB, nb, 1, xu, cu, N, err)
    torch.cuda.synchronize()
    exp_buf, e1 = O.pack(case.src_caches, case.src_tables)
    exp_dst, e2 = O.unpack([exp_buf], case.dst_caches, case.dst_tables)
    assert np.array_equal(host_bytes(buf)[: exp_buf.nbytes], exp_buf.reshape(-1)), "pack"
    for l in range(L):
        assert np.array_equal(host_bytes(dst[l]).reshape(nb, BB), exp_dst[l]), f"unpack layer {l}"
    assert int(err.item()) == e1 | e2
    err.zero_()

    # direct copy
    dst2 = layers_from_host(case.dst_caches, BB)
    K.kvx_copy_direct(sbase, K.layer_base_table(dst2), BB, nb, nb, *lists["direct"], N, err)
    torch.cuda.synchronize()
    exp_direct, e3 = O.copy_direct(case.src_caches, case.dst_caches, case.src_tables, case.dst_tables)
    for l in range(L):
        assert np.array_equal(host_bytes(dst2[l]).reshape(nb, BB), exp_direct[l]), f"direct layer {l}"
    assert int(err.item()) == e3
    err.zero_()

    # the same memory viewed as kv-first caches (2, nb, BB/2), when a segment is whole KiB
    seg = BB // 2
    if seg % 1024 == 0:
        kbuf = torch.zeros(max(L * 2 * N * seg, 16), dtype=torch.uint8, device=DEV)
        dst3 = layers_from_host(case.dst_caches, BB)
        K.kvx_pack_kv_first(sbase, seg, nb * seg, nb, ro, xp, cp, N, kbuf, err)
        K.kvx_unpack_kv_first(kbuf, K.layer_base_table(dst3), seg, nb * seg, nb, ro, xu, cu, N, err)
        torch.cuda.synchronize()
        planes = [np.ascontiguousarray(a).view(np.uint8).reshape(2, nb, seg) for a in case.src_caches]
        dplanes = [np.ascontiguousarray(a).view(np.uint8).reshape(2, nb, seg) for a in case.dst_caches]
        exp_k, e4 = O.pack_kv_first(planes, case.src_tables)
        exp_kd, e5 = O.unpack_kv_first(exp_k, dplanes, case.dst_tables)
        assert np.array_equal(host_bytes(kbuf)[: exp_k.nbytes], exp_k.reshape(-1)), "kv-first pack"
        for l in range(L):
            assert np.array_equal(host_bytes(dst3[l]).reshape(2, nb, seg), exp_kd[l]), f"kv-first layer {l}"
        assert int(err.item()) == e4 | e5
        err.zero_()

    # head split on the sender and merge on the receiver, where the heads divide evenly
    rows = bs * 2
    for S in (2, 4):
        if (H * D * e) % (S * 16):
            continue
        shards = [torch.zeros(max(L * N * BB // S, 16), dtype=torch.uint8, device=DEV) for _ in range(S)]
        dst4 = layers_from_host(case.dst_caches, BB)
        K.kvx_pack_split(sbase, BB, nb, rows, xp, cp, N, shards, err)
        K.kvx_unpack(shards, K.layer_base_table(dst4), BB, nb, rows, xu, cu, N, err)
        torch.cuda.synchronize()
        exp_s, e6 = O.pack_split(case.src_caches, case.src_tables, S, rows_per_block=rows)
        exp_m, e7 = O.unpack(list(exp_s), case.dst_caches, case.dst_tables, rows_per_block=rows)
        for d in range(S):
            assert np.array_equal(host_bytes(shards[d])[: exp_s[d].nbytes], exp_s[d].reshape(-1)), f"shard {d}/{S}"
        for l in range(L):
            assert np.array_equal(host_bytes(dst4[l]).reshape(nb, BB), exp_m[l]), f"merge {S} layer {l}"
        assert int(err.item()) == e6 | e7
        err.zero_()


LAYOUTS = ["blocks_tokens_kv", "blocks_kv_tokens", "kv_blocks_tokens"]


@pytest.mark.parametrize("seed", range(NUM_CASES // 2))
def test_random_case_slots_and_write(seed):
    """Random requests, token subsets in random order, padding tokens, a slot past the cache,
    one of three cache layouts: slot mapping then the new-token write."""
    K = kvx()
    rng = np.random.default_rng(70_000 + seed)
    H = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([8, 64, 128, 256]))
    R = int(rng.integers(1, 10))
    nb = int(rng.integers(R * 12, R * 24 + 1))
    d = W.decode_write(seed=int(rng.integers(1 << 30)), num_reqs=R, max_len=160, num_blocks=nb,
                       num_kv_heads=H, head_dim=D)
    layout = LAYOUTS[int(rng.integers(0, 3))]
    log(f"seed {seed}: H={H} D={D} requests={R} nb={nb} tokens={len(d.req_idx)} layout={layout}")
    T = len(d.req_idx)
    pick = rng.permutation(T)[: int(rng.integers(1, T + 1))]
    req, pos = d.req_idx[pick].copy(), d.positions[pick].copy()
    if len(pos) > 2:
        pos[1] = 10_000  # past the table's width
    slots = torch.empty(len(pick), dtype=torch.int64, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_slot_mapping(to_dev(d.block_table), to_dev(req), to_dev(pos), 16, slots, err)
    torch.cuda.synchronize()
    exp_slots, es = O.slot_mapping(d.block_table, req, pos, 16)
    assert np.array_equal(slots.cpu().numpy(), exp_slots)
    assert int(err.item()) == es
    s = exp_slots.copy()
    if len(s) > 3:
        s[2] = nb * 16 + 1  # a slot past the cache
    shape = {"blocks_tokens_kv": (nb, 16, 2, H, D), "blocks_kv_tokens": (nb, 2, 16, H, D),
             "kv_blocks_tokens": (2, nb, 16, H, D)}[layout]
    cache_h = np.full(shape, W.SENTINEL16, np.uint16)
    cache = to_dev(cache_h)
    _, _, bst, tst, kst = K.cache_strides(cache, layout)
    key, val = d.key[pick], d.value[pick]
    err.zero_()
    K.kvx_reshape_and_cache(to_dev(key), to_dev(val), to_dev(s), cache, nb, 16, bst, tst, kst, err)
    torch.cuda.synchronize()
    exp, ew = O.reshape_and_cache(cache_h, key, val, s, nb, 16, bst, tst, kst)
    assert np.array_equal(host_bytes(cache), exp)
    assert int(err.item()) == ew
