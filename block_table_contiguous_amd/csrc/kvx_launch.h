// Internal interface between the C-ABI entry points (kvx_api.hip) and the gfx950 kernels
// (kvx_kernels.hip). Arguments are already validated when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvx.h"

namespace kvx {

// Launch-shape knobs. Defaults are compiled in; each can be overridden once per process
// through the environment (read on first use) so sweeps need no rebuild.
// Per copy kernel: bytes of buffer one wavefront owns, the cache policy (bit 0:
// non-temporal loads, bit 1: non-temporal stores) and the batch of the one-batch kernels.
struct CopyTuning {
  int64_t wave_bytes;  // general path (KVX_WAVE_BYTES_{PACK,UNPACK,MERGE,SPLIT,DIRECT})
  int nt_mode;         // KVX_NT_{PACK,UNPACK,MERGE,SPLIT,DIRECT,KVF_PACK,KVF_UNPACK}
  int batch;           // one-batch path: KiB per wavefront, 4 or 8 (KVX_BATCH_{...})
};
struct Tuning {
  CopyTuning pack, unpack, merge, split, kvf_pack, kvf_unpack, direct;
  int xcd_remap;  // 1: give each XCD a contiguous slice of the work (KVX_XCD_REMAP)
  int xcd_remap_split;  // the same for the head split (KVX_XCD_REMAP_SPLIT)
  int one_batch;  // 1: one-batch-per-wavefront kernels where blocks allow (KVX_ONE_BATCH)
  int write_nt;   // cache policy of the new-token write, bits as nt_mode (KVX_NT_WRITE)
  int64_t write_vec_min;  // fewest tokens for the vector-sliced write of sub-KiB rows (KVX_WRITE_VEC_MIN)
};
const Tuning& tuning();

hipError_t launch_slot_mapping(const int32_t* block_table, int64_t num_reqs, int64_t max_cols,
                               int64_t row_stride, const int32_t* req_idx,
                               const int64_t* positions, int64_t num_tokens, int32_t block_size,
                               int64_t* slots, int32_t* err, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, int64_t key_stride, const void* value,
                                    int64_t value_stride, int64_t num_tokens, int64_t row_bytes,
                                    const int64_t* slots, void* cache, int64_t num_blocks,
                                    int32_t block_size, int64_t block_stride,
                                    int64_t token_stride, int64_t kv_stride, int32_t* err,
                                    hipStream_t stream);

hipError_t launch_build_xfer_list(const int32_t* src_ids, const int32_t* dst_ids,
                                  const int64_t* req_offsets, int32_t num_reqs,
                                  int64_t total_blocks, int32_t mode, kvx_xfer* xfers,
                                  int64_t* xfer_count, int32_t* err, hipStream_t stream);

// A completion signal carried by a copy launch: once every byte of the launch is written and
// visible device-wide, `delta` is added to *counter. `arrivals` is KVX_ARRIVALS_BYTES of
// counters that are 0 before the launch; the launch counts its finished workgroups there and
// leaves them 0 again.
struct SignalSpec {
  uint64_t* counter;
  uint64_t delta;
  uint32_t* arrivals;
};

// Run copies: pack (layer_bases -> buffer), single-source unpack (buffer -> layer_bases) or
// direct (layer_bases -> dst_layer_bases, no buffer). Pack and direct may carry a signal.
enum { kDirToBuffer = 0, kDirFromBuffer = 1, kDirDirect = 2 };
hipError_t launch_copy_runs(int dir, void* const* layer_bases, void* const* dst_layer_bases,
                            int32_t num_layers, int64_t block_bytes, int64_t num_cache_blocks,
                            int64_t dst_num_cache_blocks, const kvx_xfer* xfers,
                            const int64_t* xfer_count, int64_t total_blocks, void* buffer,
                            int32_t* err, hipStream_t stream, const SignalSpec* signal = nullptr);

// One-wavefront signal add (kvx_signal.hip): used when a signalling copy has nothing to copy.
hipError_t launch_signal_add(uint64_t* counter, uint64_t delta, hipStream_t stream);

// head shards: split (to_buffer: cache -> num_shards buffers) or merge (buffers -> cache)
hipError_t launch_shards(bool to_buffer, void* const* shards, int32_t num_shards,
                         void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                         int64_t num_cache_blocks, int32_t rows_per_block, const kvx_xfer* xfers,
                         const int64_t* xfer_count, int64_t total_blocks, int32_t* err,
                         hipStream_t stream);

// kv-first caches (K plane, V plane at + plane_stride); segment_bytes a multiple of 1 KiB
hipError_t launch_kv_first(bool to_buffer, void* const* layer_bases, int32_t num_layers,
                           int64_t segment_bytes, int64_t plane_stride, int64_t num_cache_blocks,
                           const int64_t* req_offsets, int32_t num_reqs, const kvx_xfer* xfers,
                           const int64_t* xfer_count, int64_t total_blocks, void* buffer,
                           int32_t* err, hipStream_t stream);

}  // namespace kvx
