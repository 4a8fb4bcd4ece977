"""The allocation-free signalling pack (kvx_pack_signal_noalloc) against the entry point it is a
variant of (kvx_pack_signal): two calls in a row on one slot, the second with a smaller input,
must give the same bytes and the same counter increments; and two slots used from two streams at
once must not interfere. The arrivals workspaces live in the library's static array."""
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


def _transfer(K, seed, L, nb, H, D, lengths):
    case = W.random_transfer(seed, L, nb, 16, H, D, lengths)
    BB, N = case.src_spec.block_bytes, case.total_blocks
    src = layers_from_host(case.src_caches, BB)
    sid, ro = K.flatten_tables(case.src_tables, DEV)
    xp, cp = K.new_xfer_list(N, DEV)
    K.kvx_build_xfer_list(sid, None, ro, K.MODE_PACK, xp, cp)
    return case, BB, N, src, K.layer_base_table(src), xp, cp


@pytest.mark.parametrize("H,D", [(1, 128), (1, 40)], ids=["8KiB", "2560B"])
def test_noalloc_pack_signal_matches_pack_signal(H, D):
    K = kvx()
    rng = np.random.default_rng(70 + D)
    big = [int(x) for x in rng.integers(200, 1500, size=8)]
    small = big[:3]
    for i, lengths in enumerate((big, small)):  # the second call moves less than the first
        case, BB, N, src, sb, xp, cp = _transfer(K, 71 + i, 3, 1200, H, D, lengths)
        nb = case.src_spec.num_blocks
        ref = torch.full((3, N, BB), 0x11, dtype=torch.uint8, device=DEV)
        got = torch.full((3, N, BB), 0x22, dtype=torch.uint8, device=DEV)
        c_ref = torch.full((1,), 1000, dtype=torch.int64, device=DEV)
        c_got = torch.full((1,), 1000, dtype=torch.int64, device=DEV)
        arrivals = K.new_arrivals(DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        torch.cuda.synchronize()
        for delta in (1, 5):
            K.kvx_pack_signal(sb, BB, nb, xp, cp, N, ref, c_ref, arrivals, delta, err)
            K.kvx_pack_signal_noalloc(sb, BB, nb, xp, cp, N, got, c_got, slot=3, delta=delta, err_flag=err)
        torch.cuda.synchronize()
        log(f"call {i}: {N} blocks of {BB} B x 3 layers")
        assert int(err.item()) == 0
        assert int(c_got.item()) == int(c_ref.item()) == 1006
        assert np.array_equal(host_bytes(got), host_bytes(ref))
        exp, e = O.pack(case.src_caches, case.src_tables)
        assert e == 0 and np.array_equal(host_bytes(got).reshape(exp.shape), exp)


def test_noalloc_slots_on_two_streams():
    """Two senders on two streams, slots 0 and 15 (the first and the last), packing layer by
    layer at the same time; both counters reach their layer counts and both buffers match the
    oracle."""
    K = kvx()
    runs = []
    for slot, (seed, D) in zip((0, K.NOALLOC_SLOTS - 1), ((80, 128), (81, 40))):
        rng = np.random.default_rng(seed)
        lengths = [int(x) for x in rng.integers(1, 900, size=5)]
        case, BB, N, src, sb, xp, cp = _transfer(K, seed, 4, 600, 1, D, lengths)
        runs.append(dict(case=case, BB=BB, N=N, sb=sb, xp=xp, cp=cp, slot=slot, stream=torch.cuda.Stream(),
                         buf=torch.zeros((4, N, BB), dtype=torch.uint8, device=DEV),
                         counter=torch.zeros(1, dtype=torch.int64, device=DEV)))
    torch.cuda.synchronize()
    for l in range(4):
        for r in runs:
            with torch.cuda.stream(r["stream"]):
                K.kvx_pack_signal_noalloc(r["sb"][l:l + 1], r["BB"], 600, r["xp"], r["cp"], r["N"], r["buf"][l],
                                          r["counter"], slot=r["slot"])
    torch.cuda.synchronize()
    for r in runs:
        assert int(r["counter"].item()) == 4
        exp, e = O.pack(r["case"].src_caches, r["case"].src_tables)
        assert e == 0 and np.array_equal(host_bytes(r["buf"]).reshape(exp.shape), exp)


def test_noalloc_rejects_a_slot_past_the_array():
    K = kvx()
    case, BB, N, src, sb, xp, cp = _transfer(K, 90, 1, 64, 1, 128, [40])
    buf = torch.zeros((N, BB), dtype=torch.uint8, device=DEV)
    counter = torch.zeros(1, dtype=torch.int64, device=DEV)
    for slot in (-1, K.NOALLOC_SLOTS):
        with pytest.raises(K.KvxError) as ei:
            K.kvx_pack_signal_noalloc(sb, BB, 64, xp, cp, N, buf, counter, slot=slot)
        assert ei.value.status == K.KVX_ERR_CAPACITY
    torch.cuda.synchronize()
    assert int(counter.item()) == 0
