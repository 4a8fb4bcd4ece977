"""MI355X-native KV-cache transfer path: pack, unpack, run-list building, slot mapping and
the new-token K/V write, as hand-written HIP kernels for gfx950 behind a C ABI
(include/kvx.h, built into libkvx.so by `python -m block_table_contiguous_amd.build`).

Import `block_table_contiguous_amd.kvx` for the Python binding; importing it loads libkvx
and fails loudly if the library has not been built.
"""
