"""GPU parity of the new-token write for rows that are not whole KiB, against the oracle.
Launches of 4096 tokens and more take the vector-sliced kernel (several tokens per
wavefront, rows up to 2 KiB); smaller launches and longer rows take the one-wavefront-per-token
kernel. Cases cover both, rows from 16 B to past 4 KiB, three cache layouts, power-of-two and
other block sizes, padding tokens, slots past the cache and slots past 2^31."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import DEV, host_bytes, kvx, log, reshape_and_cache_raw, to_dev

pytestmark = pytest.mark.gpu

VECTOR_MIN_TOKENS = 4096  # the library's default switch between the two kernels


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"start {request.node.name}")
    yield
    torch.cuda.synchronize()
    log(f"end {request.node.name}")


SHAPES = {"blocks_tokens_kv": lambda nb, bs, w: (nb, bs, 2, w),
          "blocks_kv_tokens": lambda nb, bs, w: (nb, 2, bs, w),
          "kv_blocks_tokens": lambda nb, bs, w: (2, nb, bs, w)}


def _strides(layout, nb, bs, row):
    """(block_stride, token_stride, kv_stride) in bytes of a dense cache in `layout`."""
    if layout == "blocks_tokens_kv":
        return bs * 2 * row, 2 * row, row
    if layout == "blocks_kv_tokens":
        return 2 * bs * row, row, bs * row
    return bs * row, row, nb * bs * row


def _write_case(seed, T, row, bs, nb, layout, pad_every=0, past_cache=()):
    K = kvx()
    rng = np.random.default_rng(seed)
    w = row // 2
    key = W.random_words(rng, (T, w))
    val = W.random_words(rng, (T, w))
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    if pad_every:
        slots[::pad_every] = -1
    for i in past_cache:
        slots[i] = nb * bs + int(rng.integers(0, bs))
    cache_h = np.full(SHAPES[layout](nb, bs, w), W.SENTINEL16, np.uint16)
    cache = to_dev(cache_h)
    bst, tst, kst = _strides(layout, nb, bs, row)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    K.kvx_reshape_and_cache(to_dev(key), to_dev(val), to_dev(slots), cache, nb, bs, bst, tst, kst, err)
    torch.cuda.synchronize()
    exp, e = O.reshape_and_cache(cache_h, key, val, slots, nb, bs, bst, tst, kst)
    assert np.array_equal(host_bytes(cache), exp)
    assert int(err.item()) == e
    return e


@pytest.mark.parametrize("row", [16, 48, 128, 256, 400, 1040, 2064, 4080])
@pytest.mark.parametrize("layout", list(SHAPES))
def test_vector_kernel_rows(row, layout):
    """5000 tokens: rows from one vector to 255 vectors. Up to 2 KiB the vector kernel takes them
    (tokens per wavefront 128 down to 1); 2064 and 4080 B rows go to the per-token kernel."""
    T, bs = 5000, 16
    nb = -(-T // bs) + 37
    e = _write_case(row * 7 + len(layout), T, row, bs, nb, layout, pad_every=13, past_cache=(5, 4321))
    assert e == O.DEVERR_SLOT_RANGE


@pytest.mark.parametrize("bs", [1, 3, 12, 16, 20, 64])
def test_vector_kernel_block_sizes(bs):
    """Power-of-two block sizes take a shift, others a division."""
    T = VECTOR_MIN_TOKENS + 11
    nb = -(-T // bs) + 5
    assert _write_case(bs, T, 256, bs, nb, "blocks_tokens_kv", pad_every=29) == 0


@pytest.mark.parametrize("bs", [1 << 28, 3 << 28])
def test_vector_kernel_slots_past_32_bits(bs):
    """Slots past 2^31 in the vector kernel: blocks of 2^28 or 3 * 2^28 slots (only a few
    slots of each used), most tokens padding so the launch still takes the vector kernel."""
    K = kvx()
    T, row, nb = VECTOR_MIN_TOKENS + 3, 256, 12
    rng = np.random.default_rng(bs % 1000)
    key = W.random_words(rng, (T, row // 2))
    val = W.random_words(rng, (T, row // 2))
    slots = np.full(T, -1, np.int64)
    picks = [0, 1, 2, 5, 7, 9, 11]
    at = rng.permutation(T)[: len(picks) + 1]
    for i, b in zip(at, picks):
        slots[i] = b * bs + int(rng.integers(0, 4))  # first few slots of block b
    slots[at[-1]] = nb * bs + 1                      # past the cache
    # a block holds 128 tokens' rows (64 KiB of 512 B); only offsets 0..3 are used
    bst, tst, kst = 64 << 10, 2 * row, row
    cache_h = np.full(nb * bst // 2, W.SENTINEL16, np.uint16)
    cache = to_dev(cache_h)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    reshape_and_cache_raw(K, to_dev(key), to_dev(val), to_dev(slots), cache, nb, bs, bst, tst, kst, err)
    torch.cuda.synchronize()
    exp, e = O.reshape_and_cache(cache_h, key, val, slots, nb, bs, bst, tst, kst)
    assert np.array_equal(host_bytes(cache), exp)
    assert int(err.item()) == e == O.DEVERR_SLOT_RANGE


@pytest.mark.parametrize("T,row", [(1, 256), (300, 256), (VECTOR_MIN_TOKENS - 1, 400), (600, 4112), (5000, 8208)])
def test_per_token_kernel(T, row):
    """Below the vector kernel's token count, and rows past 4 KiB that are not whole KiB."""
    bs = 16
    nb = -(-T // bs) + 3
    _write_case(T * 3 + row, T, row, bs, nb, "blocks_tokens_kv", pad_every=17 if T > 1 else 0,
                past_cache=(1,) if T > 2 else ())
