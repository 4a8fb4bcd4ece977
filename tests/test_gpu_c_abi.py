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
from gpu_util import kvx, log

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


REST = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "rest")
REST_MAGIC = 0x4B565852


def test_plain_c_rest_of_the_abi(tmp_path):
    """tests/c_abi/rest.c: the slot mapping and new-token write, the kv-first pack and unpack,
    the head split and the two-source merge, the signal add and wait, the signalling pack and
    the signalling direct copy each feeding a consumer stream layer by layer, the
    allocation-free signalling pack likewise, and the ABI version, all from plain C; every
    output against the oracle, and ten host-side status codes."""
    assert os.path.exists(REST), "tests/c_abi/rest is built by __graft_entry__.build()"
    rng = np.random.default_rng(77)
    bs, H, D, L, nb = 16, 1, 64, 2, 200
    lengths = [int(x) for x in rng.integers(1, 500, size=6)]
    case = W.random_transfer(78, L, nb, bs, H, D, lengths)
    row = H * D * 2
    BB, N, R = case.src_spec.block_bytes, case.total_blocks, len(lengths)
    seg = BB // 2
    offsets = np.zeros(R + 1, np.int64)
    np.cumsum([len(t) for t in case.src_tables], out=offsets[1:])
    width = max(len(t) for t in case.dst_tables)
    table = W.pad_table(case.dst_tables, width)
    pairs = [(r, p) for r in range(R) for p in range(lengths[r])]
    pick = rng.permutation(len(pairs))[:300]
    req = np.array([pairs[i][0] for i in pick], np.int32)
    pos = np.array([pairs[i][1] for i in pick], np.int64)
    T = len(req)
    key = W.random_words(rng, (T, row // 2))
    val = W.random_words(rng, (T, row // 2))
    src = [np.ascontiguousarray(c).view(np.uint8).reshape(nb, BB) for c in case.src_caches]
    dst = [np.ascontiguousarray(c).view(np.uint8).reshape(nb, BB) for c in case.dst_caches]
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([REST_MAGIC, L, nb, bs, row, R, N, T, width], np.int64).tobytes())
        f.write(offsets.tobytes())
        f.write(np.concatenate(case.src_tables).astype(np.int32).tobytes())
        f.write(np.concatenate(case.dst_tables).astype(np.int32).tobytes())
        f.write(table.astype(np.int32).tobytes())
        f.write(req.tobytes())
        f.write(pos.tobytes())
        f.write(key.tobytes())
        f.write(val.tobytes())
        for c in src:
            f.write(c.tobytes())
        for c in dst:
            f.write(c.tobytes())
    log(f"running {REST}: L={L} nb={nb} block_bytes={BB} N={N} T={T}")
    r = subprocess.run([REST, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip())
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(out, np.uint8)
    hdr = raw[:64].view(np.int64)
    at = 64

    def take(n):
        nonlocal at
        part = raw[at:at + n]
        at += n
        return part

    slots = take(T * 8).view(np.int64)
    written = take(nb * BB)
    kbuf = take(L * 2 * N * seg)
    kvf = take(L * nb * BB).reshape(L, nb, BB)
    sh0, sh1 = take(L * N * BB // 2), take(L * N * BB // 2)
    merged = take(L * nb * BB).reshape(L, nb, BB)
    signalled = take(L * nb * BB).reshape(L, nb, BB)
    seen = take(L * nb * BB).reshape(L, nb, BB)
    nbuf = take(L * N * BB)
    nsignalled = take(L * nb * BB).reshape(L, nb, BB)
    assert at == raw.size

    assert int(hdr[0]) == 0 and int(hdr[1]) == 0, "error flags"
    assert int(hdr[2]) == L and int(hdr[3]) == 42, "signal counters"
    assert int(hdr[4]) == 10, "host-side status checks"
    assert int(hdr[5]) == kvx().kvx_abi_version(), "ABI version"
    assert int(hdr[6]) == L and int(hdr[7]) == L, "direct-copy and allocation-free signal counters"
    exp_slots, e = O.slot_mapping(table, req, pos, bs)
    assert e == 0 and np.array_equal(slots, exp_slots)
    exp_w, e = O.reshape_and_cache(dst[0], key, val, exp_slots, nb, bs, bs * 2 * row, 2 * row, row)
    assert e == 0 and np.array_equal(written, exp_w)
    exp_k, e1 = O.pack_kv_first([c.reshape(2, nb, seg) for c in src], case.src_tables)
    exp_kvf, e2 = O.unpack_kv_first(exp_k, [c.reshape(2, nb, seg) for c in dst], case.dst_tables)
    assert e1 == e2 == 0 and np.array_equal(kbuf, exp_k.reshape(-1))
    exp_sh, e1 = O.pack_split(src, case.src_tables, 2, bs * 2)
    exp_m, e2 = O.unpack(exp_sh, dst, case.dst_tables, rows_per_block=bs * 2)
    assert e1 == e2 == 0
    assert np.array_equal(sh0, exp_sh[0].reshape(-1)) and np.array_equal(sh1, exp_sh[1].reshape(-1))
    exp_buf, e1 = O.pack(src, case.src_tables)
    exp_s, e2 = O.unpack([exp_buf], dst, case.dst_tables)
    assert e1 == e2 == 0
    exp_d, e = O.copy_direct(src, dst, case.src_tables, case.dst_tables)
    assert e == 0
    assert np.array_equal(nbuf, exp_buf.reshape(-1)), "allocation-free signalled pack"
    for l in range(L):
        assert np.array_equal(kvf[l], exp_kvf[l].reshape(nb, BB)), f"kv-first layer {l}"
        assert np.array_equal(merged[l], exp_m[l]), f"merge layer {l}"
        assert np.array_equal(signalled[l], exp_s[l]), f"signalled transfer layer {l}"
        assert np.array_equal(seen[l], exp_d[l]), f"direct layer {l} as seen after its signal"
        assert np.array_equal(nsignalled[l], exp_s[l]), f"allocation-free signalled transfer layer {l}"
