"""The C ABI used from plain C, with no Python or PyTorch in the path: tests/c_abi/roundtrip.c
(compiled with gcc against include/kvx.h by the build step) runs the three run lists, pack,
unpack and the direct copy on a HIP stream of its own, and checks host-side status codes. Its
outputs are compared here byte for byte with the oracle."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import log

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "roundtrip")
MAGIC = 0x4B5658


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"start {request.node.name}")
    yield
    log(f"end {request.node.name}")


@pytest.mark.parametrize("bs,H,D", [(16, 1, 64), (16, 3, 40), (4, 1, 8)], ids=["2KiB", "7680B", "64B"])
def test_plain_c_roundtrip(bs, H, D, tmp_path):
    assert os.path.exists(EXE), "tests/c_abi/roundtrip is built by __graft_entry__.build()"
    rng = np.random.default_rng(bs * 100 + H * 10 + D)
    lengths = [int(x) for x in rng.integers(0, bs * 12, size=7)]
    lengths[1] = max(lengths[1], bs)
    lengths[2] = max(lengths[2], bs)
    case = W.random_transfer(int(rng.integers(1 << 30)), 2, 300, bs, H, D, lengths)
    spec = case.src_spec
    L, nb, BB, N = spec.num_layers, spec.num_blocks, spec.block_bytes, case.total_blocks
    src_tables = [t.copy() for t in case.src_tables]
    dst_tables = [t.copy() for t in case.dst_tables]
    src_tables[1][0] = nb + 2   # outside the source cache
    dst_tables[2][-1] = -1      # outside the destination cache
    offsets = np.zeros(len(src_tables) + 1, np.int64)
    np.cumsum([len(t) for t in src_tables], out=offsets[1:])
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([MAGIC, L, nb, BB, len(src_tables), N], np.int64).tobytes())
        f.write(offsets.tobytes())
        f.write(np.concatenate(src_tables).astype(np.int32).tobytes())
        f.write(np.concatenate(dst_tables).astype(np.int32).tobytes())
        for c in case.src_caches:
            f.write(np.ascontiguousarray(c).tobytes())
        for c in case.dst_caches:
            f.write(np.ascontiguousarray(c).tobytes())
    log(f"running {EXE}: L={L} nb={nb} block_bytes={BB} N={N}")
    r = subprocess.run([EXE, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip())
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(out, np.uint8)
    hdr = raw[:40].view(np.int64)
    at = 40
    buf = raw[at:at + L * N * BB]
    at += L * N * BB
    dst = raw[at:at + L * nb * BB].reshape(L, nb, BB)
    at += L * nb * BB
    dst2 = raw[at:at + L * nb * BB].reshape(L, nb, BB)

    exp_buf, e1 = O.pack(case.src_caches, src_tables)
    exp_dst, e2 = O.unpack([exp_buf], case.dst_caches, dst_tables)
    exp_dir, e3 = O.copy_direct(case.src_caches, case.dst_caches, src_tables, dst_tables)
    assert int(hdr[0]) == len(O.xfer_list(src_tables, dst_tables, O.MODE_PACK))
    assert int(hdr[1]) == len(O.xfer_list(src_tables, dst_tables, O.MODE_UNPACK))
    assert int(hdr[2]) == len(O.xfer_list(src_tables, dst_tables, O.MODE_DIRECT))
    assert int(hdr[3]) == (e1 | e2 | e3) == O.DEVERR_BLOCK_RANGE
    assert int(hdr[4]) == 4, "host-side status checks"
    assert np.array_equal(buf, exp_buf.reshape(-1))
    for l in range(L):
        assert np.array_equal(dst[l], exp_dst[l]), f"unpack layer {l}"
        assert np.array_equal(dst2[l], exp_dir[l]), f"direct layer {l}"
