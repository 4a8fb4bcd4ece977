"""The entry points keep no state between calls: independent transfers enqueued on separate
streams, and from separate host threads, each match the oracle. Default-priority streams only."""
import threading

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


class Job:
    """One round trip (run lists, pack, unpack) with its own caches, buffer and stream."""

    def __init__(self, seed, bs, H, D):
        K = kvx()
        self.K = K
        rng = np.random.default_rng(seed)
        lengths = [int(x) for x in rng.integers(0, bs * 30, size=9)]
        self.case = W.random_transfer(seed, 2, 800, bs, H, D, lengths)
        spec = self.case.src_spec
        self.BB, self.nb, self.N = spec.block_bytes, spec.num_blocks, self.case.total_blocks
        self.src = layers_from_host(self.case.src_caches, self.BB)
        self.dst = layers_from_host(self.case.dst_caches, self.BB)
        self.sid, self.ro = K.flatten_tables(self.case.src_tables, DEV)
        self.did, _ = K.flatten_tables(self.case.dst_tables, DEV)
        self.xp, self.cp = K.new_xfer_list(self.N, DEV)
        self.xu, self.cu = K.new_xfer_list(self.N, DEV)
        self.buf = torch.zeros(max(2 * self.N * self.BB, 16), dtype=torch.uint8, device=DEV)
        self.err = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.sb, self.db = K.layer_base_table(self.src), K.layer_base_table(self.dst)
        self.stream = torch.cuda.Stream()

    def enqueue(self, reps=1):
        K = self.K
        with torch.cuda.stream(self.stream):
            for _ in range(reps):
                K.kvx_build_xfer_list(self.sid, None, self.ro, K.MODE_PACK, self.xp, self.cp, self.err)
                K.kvx_pack(self.sb, self.BB, self.nb, self.xp, self.cp, self.N, self.buf, self.err)
                K.kvx_build_xfer_list(None, self.did, self.ro, K.MODE_UNPACK, self.xu, self.cu, self.err)
                K.kvx_unpack([self.buf], self.db, self.BB, self.nb, 1, self.xu, self.cu, self.N, self.err)

    def check(self):
        self.stream.synchronize()
        buf, e1 = O.pack(self.case.src_caches, self.case.src_tables)
        out, e2 = O.unpack([buf], self.case.dst_caches, self.case.dst_tables)
        assert np.array_equal(host_bytes(self.buf)[: buf.nbytes], buf.reshape(-1))
        for l in range(2):
            assert np.array_equal(host_bytes(self.dst[l]).reshape(self.nb, self.BB), out[l])
        assert int(self.err.item()) == e1 | e2 == 0


GEOMS = [(16, 1, 128), (16, 3, 40), (4, 1, 8), (16, 8, 128)]  # 8 KiB, 7680 B, 64 B, 64 KiB blocks


def test_interleaved_streams():
    jobs = [Job(100 + i, *g) for i, g in enumerate(GEOMS)]
    torch.cuda.synchronize()
    for _ in range(3):
        for j in jobs:
            j.enqueue()
    for j in jobs:
        j.check()


def test_host_threads():
    jobs = [Job(200 + i, *g) for i, g in enumerate(GEOMS)]
    torch.cuda.synchronize()
    errors = []

    def work(j):
        try:
            torch.cuda.set_device(0)
            j.enqueue(reps=5)
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for j in jobs:
        j.check()
