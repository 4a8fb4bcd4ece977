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
from gpu_util import DEV, Transfer, check_runs_equal, host_bytes, log

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
    spec = case.src_spec
    for t in dst:
        W.fill_device_byte_(t)
    tr = Transfer(case, src, dst)
    tr.run()
    log(f"{case.name}: transfer done, checking")
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
