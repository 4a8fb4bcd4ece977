"""The pins are strong enough: each plausible mistake planted in a copy of the oracle (a
dropped term, a wrong index or sign, a transposed operand, a wrong order) makes at least
one pin fail. Mistakes are planted in the oracle's source text on the CPU only."""
import importlib.util
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kv_oracle.py")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("slot_drop_offset", "block * block_size + pos % block_size", "block * block_size"),
    ("slot_drop_scale", "block * block_size + pos % block_size", "block + pos % block_size"),
    ("slot_index_by_offset", "bt[r, pos // block_size]", "bt[r, pos % block_size]"),
    ("slot_no_row_check", "pos // block_size >= width", "pos // block_size > width"),
    ("slot_padding_kept", "        if block < 0:\n            slots[i] = -1", "        if block < -1:\n            slots[i] = -1"),
    ("reshape_swap_kv", "out[at:at + row] = K[i]", "out[at:at + row] = V[i]"),
    ("reshape_token_stride_swapped", "offset * token_stride", "offset * kv_stride"),
    ("reshape_skip_zero_slot", "if s < 0:", "if s <= 0:"),
    ("reshape_no_range_check", "if block >= num_blocks:", "if block > num_blocks:"),
    ("runs_no_step", "src[k] != src[k - 1] + 1", "src[k] != src[k - 1]"),
    ("runs_dst_wrong_side", "dst[k] != dst[k - 1] + 1", "src[k] != src[k - 1] + 1 if uses_src else dst[k] != dst[k - 1]"),
    ("runs_buf_not_global", "runs.append((s, d, p + j, k - j, r))", "runs.append((s, d, j, k - j, r))"),
    ("runs_len_off_by_one", "runs.append((s, d, p + j, k - j, r))", "runs.append((s, d, p + j, k - j + 1, r))"),
    ("runs_cross_requests", "        p += n\n    return runs", "        p += n\n    return _merge(runs)\n\ndef _merge(runs):\n    out = []\n    for x in runs:\n        if out and out[-1][0] + out[-1][3] == x[0] and out[-1][1] + out[-1][3] == x[1]:\n            a = out.pop(); out.append((a[0], a[1], a[2], a[3] + x[3], a[4])); continue\n        out.append(x)\n    return out"),
    ("order_local_position", "            order.append((r, j, p))", "            order.append((r, j, j))"),
    ("order_requests_reversed", "    for r, t in enumerate(tables):\n        for j in range(len(t)):\n            order.append((r, j, p))",
     "    for r, t in reversed(list(enumerate(tables))):\n        for j in range(len(t)):\n            order.append((r, j, p))"),
    ("pack_layer0_only", "buf[l, p] = caches[l][b]", "buf[l, p] = caches[0][b]"),
    ("pack_dedups_shared_blocks", "            buf[l, p] = caches[l][b]\n    return buf, err",
     "            if any(int(src_tables[rr][jj]) == b for rr, jj, pp in order if pp < p):\n                continue\n"
     "            buf[l, p] = caches[l][b]\n    return buf, err"),
    ("direct_reads_dst_id", "out[l][d] = srcs[l][s]", "out[l][d] = srcs[l][d % nbs]"),
    ("direct_layer0_only", "out[l][d] = srcs[l][s]", "out[l][d] = srcs[0][s]"),
    ("direct_no_dst_range_check", "if s < 0 or s >= nbs or d < 0 or d >= nbd:", "if s < 0 or s >= nbs or d >= nbd:"),
    ("runs_direct_ignores_dst", "                if uses_dst and dst[k] != dst[k - 1] + 1:",
     "                if uses_dst and not uses_src and dst[k] != dst[k - 1] + 1:"),
    ("pack_no_range_check", "if b < 0 or b >= nb:", "if b >= nb:"),
    ("unpack_to_position", "out[l][d] = bufs[0][l, p]", "out[l][p % nb] = bufs[0][l, p]"),
    ("unpack_layer_swap", "out[l][d] = bufs[0][l, p]", "out[l][d] = bufs[0][L - 1 - l, p]"),
    ("merge_transposed", "at = (k * S + s) * row_src", "at = (s * rows_per_block + k) * row_src"),
    ("merge_sources_swapped", "srcs[s][k * row_src:(k + 1) * row_src]", "srcs[S - 1 - s][k * row_src:(k + 1) * row_src]"),
    ("unpack_no_range_check", "if d < 0 or d >= nb:", "if d >= nb:"),
    ("kv_first_interleaved", "            for kv in range(2):\n                for b in t:", "            for b in t:\n                for kv in range(2):"),
    ("kv_first_planes_swapped", "buf[l, at] = planes[l][kv, b]", "buf[l, at] = planes[l][1 - kv, b]"),
    ("kv_first_unpack_one_plane", "out[l][kv, d] = src[l, at]", "out[l][0, d] = src[l, at]"),
    ("kv_first_no_range_check", "                    if 0 <= b < nb:\n                        buf[l, at]", "                    if b < nb:\n                        buf[l, at]"),
    ("split_pieces_reversed", "b[k * row + d * piece:k * row + (d + 1) * piece]",
     "b[k * row + (num_dst - 1 - d) * piece:k * row + (num_dst - d) * piece]"),
    ("split_rows_transposed", "b[k * row + d * piece:k * row + (d + 1) * piece]",
     "b[(d * rows_per_block + k) * piece:(d * rows_per_block + k + 1) * piece]"),
    ("split_shards_misrouted", "                bufs[d][l, p] = shard", "                bufs[num_dst - 1 - d][l, p] = shard"),
    ("repeats_accepted", "        if t in seen:\n            raise", "        if t in seen and False:\n            raise"),
    ("reshape_repeats_accepted", "    _reject_repeats([int(s) for s in slots", "    ([int(s) for s in slots"),
    ("unpack_repeats_accepted", "    _reject_repeats([int(dst_tables[r][j]) for r, j, _ in order",
     "    ([int(dst_tables[r][j]) for r, j, _ in order"),
    ("direct_repeats_accepted", "    _reject_repeats([int(d) for t in dst_tables for d in t if 0 <= int(d) < nbd]",
     "    ([int(d) for t in dst_tables for d in t if 0 <= int(d) < nbd]"),
    ("kv_first_repeats_accepted", "    _reject_repeats([int(d) for t in dst_tables for d in t if 0 <= int(d) < nb]",
     "    ([int(d) for t in dst_tables for d in t if 0 <= int(d) < nb]"),
    ("reshape_repeats_out_of_cache_rejected", "if int(s) >= 0 and int(s) // block_size < num_blocks]", "if int(s) >= 0]"),
    ("unpack_repeats_out_of_cache_rejected", "order if 0 <= int(dst_tables[r][j]) < nb]", "order]"),
    ("direct_repeats_out_of_cache_rejected", "for d in t if 0 <= int(d) < nbd]", "for d in t]"),
    ("kv_first_repeats_out_of_cache_rejected", "for d in t if 0 <= int(d) < nb]", "for d in t]"),
    ("slot_request_past_table", "if r < 0 or r >= num_reqs or pos < 0", "if r < 0 or pos < 0"),
    ("slot_negative_position", "if r < 0 or r >= num_reqs or pos < 0 or", "if r < 0 or r >= num_reqs or"),
    ("reshape_value_over_key", "out[at + kv_stride:at + kv_stride + row] = V[i]", "out[at:at + row] = V[i]"),
    ("reshape_block_stride_as_token", "at = block * block_stride + offset * token_stride",
     "at = block * token_stride + offset * token_stride"),
    ("direct_no_src_lower_check", "if s < 0 or s >= nbs or d < 0 or d >= nbd:", "if s >= nbs or d < 0 or d >= nbd:"),
]


def _mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, old
    text = text.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _failing_pins(mod):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:  # AssertionError, or a crash the mistake causes
            failed.append(pin.__name__)
    return failed


def test_unmutated_copy_passes():
    text = open(SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(text, "oracle_copy", "exec"), mod.__dict__)
    assert _failing_pins(mod) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    assert _failing_pins(_mutant(old, new)), f"no pin catches mutant {name}"
