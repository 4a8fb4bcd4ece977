// C-ABI entry points of libkvx: argument validation, then one asynchronous launch each.
// Validation runs entirely on the host and touches no HIP API, so a bad call returns its
// status before anything is enqueued (and can be tested without a GPU).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstring>
#include <mutex>

#include "kvx.h"
#include "kvx_launch.h"

// The allocation-free signalling pack keeps its arrivals workspaces here: KVX_NOALLOC_SLOTS
// workspaces of KVX_ARRIVALS_BYTES per GPU (64 KiB), zero when the library is loaded and left
// zero by every call that completes. In host code `scratch` only names the variable; its
// device address on each GPU comes from hipGetSymbolAddress (scratch_words below) and is the
// only form of it passed to kernels.
static __device__ __align__(256) uint32_t scratch[KVX_NOALLOC_SLOTS * (KVX_ARRIVALS_BYTES / 4)];

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool mult16(int64_t v) { return (v & 15) == 0; }

inline kvx_status from_hip(hipError_t e) { return e == hipSuccess ? KVX_SUCCESS : KVX_ERR_HIP; }

constexpr int64_t kMaxBlocks = 0x7fffffff;  // block ids and run lengths are int32

// count x bytes stays within KVX_MAX_EXTENT_BYTES (both non-negative): the kernels form 64-bit
// byte offsets from such products, and nothing larger can be a real allocation.
inline bool extent_ok(int64_t count, int64_t bytes) {
  return count >= 0 && bytes >= 0 && (count == 0 || bytes <= KVX_MAX_EXTENT_BYTES / count);
}

// A copy's extents: one layer's cache (blocks x block bytes) and the whole buffer or transfer
// (layers x blocks x block bytes; layers and blocks are both below 2^31, so their product fits).
inline bool copy_extents_ok(int32_t num_layers, int64_t total_blocks, int64_t cache_blocks,
                            int64_t block_bytes) {
  return extent_ok(cache_blocks, block_bytes) &&
         extent_ok((int64_t)num_layers * total_blocks, block_bytes);
}

// Device address of `scratch` on the GPU that owns `stream`, looked up once per device (with
// that device current: the call requires it) and kept. No allocation is involved.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch[kMaxDevices] = {};

kvx_status scratch_words(hipStream_t stream, uint32_t** out) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &dev) != hipSuccess)
    return KVX_ERR_HIP;
  if (dev != cur || dev < 0 || dev >= kMaxDevices) return KVX_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVX_ERR_HIP;
    g_scratch[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch[dev];
  return KVX_SUCCESS;
}

}  // namespace

extern "C" {

const char* kvx_status_string(kvx_status status) {
  // A C caller may pass any int here. Read the argument's bytes as an int: in C++ a value of
  // the enum type outside its enumerators has no defined meaning.
  int32_t code;
  static_assert(sizeof(code) == sizeof(status), "kvx_status is passed as a 32-bit int");
  memcpy(&code, &status, sizeof(code));
  switch (code) {
    case KVX_SUCCESS: return "kvx: success";
    case KVX_ERR_INVALID_ARGUMENT: return "kvx: invalid argument (null pointer, negative size or bad mode)";
    case KVX_ERR_MISALIGNED: return "kvx: pointer, size or stride not a multiple of 16 bytes";
    case KVX_ERR_CAPACITY: return "kvx: output array smaller than the worst case, or request beyond the library's fixed scratch";
    case KVX_ERR_HIP: return "kvx: HIP kernel launch failed";
  }
  return "kvx: unknown status";
}

int32_t kvx_abi_version(void) { return 5; }

kvx_status kvx_slot_mapping(const int32_t* block_table, int64_t num_reqs,
                            int64_t max_blocks_per_req, int64_t bt_row_stride,
                            const int32_t* req_idx, const int64_t* positions,
                            int64_t num_tokens, int32_t block_size, int64_t* slot_mapping,
                            int32_t* err_flag, hipStream_t stream) {
  if (num_tokens < 0 || num_reqs < 0 || block_size < 1 || max_blocks_per_req < 0 ||
      bt_row_stride < max_blocks_per_req || !extent_ok(num_reqs, bt_row_stride) ||
      !extent_ok(num_tokens, 8))
    return KVX_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return KVX_SUCCESS;
  if (!req_idx || !positions || !slot_mapping || (num_reqs > 0 && !block_table))
    return KVX_ERR_INVALID_ARGUMENT;
  return from_hip(kvx::launch_slot_mapping(block_table, num_reqs, max_blocks_per_req,
                                           bt_row_stride, req_idx, positions, num_tokens,
                                           block_size, slot_mapping, err_flag, stream));
}

kvx_status kvx_reshape_and_cache(const void* key, int64_t key_stride_bytes, const void* value,
                                 int64_t value_stride_bytes, int64_t num_tokens,
                                 int64_t row_bytes, const int64_t* slot_mapping,
                                 void* kv_cache, int64_t num_blocks, int32_t block_size,
                                 int64_t block_stride_bytes, int64_t token_stride_bytes,
                                 int64_t kv_stride_bytes, int32_t* err_flag,
                                 hipStream_t stream) {
  if (num_tokens < 0 || row_bytes <= 0 || num_blocks < 0 || block_size < 1 ||
      key_stride_bytes < 0 || value_stride_bytes < 0 || block_stride_bytes < 0 ||
      token_stride_bytes < 0 || kv_stride_bytes < 0)
    return KVX_ERR_INVALID_ARGUMENT;
  if (!extent_ok(num_blocks, block_stride_bytes) || !extent_ok(block_size, token_stride_bytes) ||
      !extent_ok(num_tokens, key_stride_bytes) || !extent_ok(num_tokens, value_stride_bytes) ||
      !extent_ok(1, kv_stride_bytes) || !extent_ok(num_tokens, row_bytes))
    return KVX_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return KVX_SUCCESS;
  if (!key || !value || !slot_mapping || !kv_cache) return KVX_ERR_INVALID_ARGUMENT;
  if (!aligned16(key) || !aligned16(value) || !aligned16(kv_cache) || !mult16(row_bytes) ||
      !mult16(key_stride_bytes) || !mult16(value_stride_bytes) || !mult16(block_stride_bytes) ||
      !mult16(token_stride_bytes) || !mult16(kv_stride_bytes))
    return KVX_ERR_MISALIGNED;
  return from_hip(kvx::launch_reshape_and_cache(
      key, key_stride_bytes, value, value_stride_bytes, num_tokens, row_bytes, slot_mapping,
      kv_cache, num_blocks, block_size, block_stride_bytes, token_stride_bytes, kv_stride_bytes,
      err_flag, stream));
}

kvx_status kvx_build_xfer_list(const int32_t* src_ids, const int32_t* dst_ids,
                               const int64_t* req_offsets, int32_t num_reqs,
                               int64_t total_blocks, int32_t mode, kvx_xfer* xfers,
                               int64_t capacity, int64_t* xfer_count, int32_t* err_flag,
                               hipStream_t stream) {
  if (mode != KVX_MODE_PACK && mode != KVX_MODE_UNPACK && mode != KVX_MODE_DIRECT)
    return KVX_ERR_INVALID_ARGUMENT;
  if (num_reqs < 0 || total_blocks < 0 || total_blocks > kMaxBlocks || capacity < 0)
    return KVX_ERR_INVALID_ARGUMENT;
  if (!xfer_count || !req_offsets) return KVX_ERR_INVALID_ARGUMENT;
  if (total_blocks > 0 && num_reqs == 0) return KVX_ERR_INVALID_ARGUMENT;
  if (total_blocks > 0) {
    const bool need_src = mode != KVX_MODE_UNPACK, need_dst = mode != KVX_MODE_PACK;
    if ((need_src && !src_ids) || (need_dst && !dst_ids) || !xfers) return KVX_ERR_INVALID_ARGUMENT;
  }
  if (!aligned16(xfers)) return KVX_ERR_MISALIGNED;
  if (capacity < total_blocks) return KVX_ERR_CAPACITY;
  return from_hip(kvx::launch_build_xfer_list(src_ids, dst_ids, req_offsets, num_reqs,
                                              total_blocks, mode, xfers, xfer_count, err_flag,
                                              stream));
}

kvx_status kvx_pack(void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                    int64_t num_cache_blocks, const kvx_xfer* xfers,
                    const int64_t* xfer_count, int64_t total_blocks, void* send_buf,
                    int32_t* err_flag, hipStream_t stream) {
  if (num_layers < 0 || block_bytes <= 0 || num_cache_blocks < 0 || total_blocks < 0 ||
      total_blocks > kMaxBlocks ||
      !copy_extents_ok(num_layers, total_blocks, num_cache_blocks, block_bytes))
    return KVX_ERR_INVALID_ARGUMENT;
  if (num_layers == 0 || total_blocks == 0) return KVX_SUCCESS;
  if (!layer_bases || !xfers || !xfer_count || !send_buf) return KVX_ERR_INVALID_ARGUMENT;
  if (!mult16(block_bytes) || !aligned16(send_buf)) return KVX_ERR_MISALIGNED;
  return from_hip(kvx::launch_copy_runs(kvx::kDirToBuffer, layer_bases, nullptr, num_layers,
                                        block_bytes, num_cache_blocks, 0, xfers, xfer_count,
                                        total_blocks, send_buf, err_flag, stream));
}

kvx_status kvx_unpack(const void* const* send_bufs, int32_t num_src, void* const* layer_bases,
                      int32_t num_layers, int64_t block_bytes, int64_t num_cache_blocks,
                      int32_t rows_per_block, const kvx_xfer* xfers,
                      const int64_t* xfer_count, int64_t total_blocks, int32_t* err_flag,
                      hipStream_t stream) {
  if (num_src < 1 || num_src > KVX_MAX_SOURCES || num_layers < 0 || block_bytes <= 0 ||
      num_cache_blocks < 0 || total_blocks < 0 || total_blocks > kMaxBlocks ||
      rows_per_block < 1 ||
      !copy_extents_ok(num_layers, total_blocks, num_cache_blocks, block_bytes))
    return KVX_ERR_INVALID_ARGUMENT;
  if (!mult16(block_bytes)) return KVX_ERR_MISALIGNED;
  if (num_src > 1 && block_bytes % ((int64_t)rows_per_block * num_src * 16) != 0)
    return KVX_ERR_INVALID_ARGUMENT;
  if (num_layers == 0 || total_blocks == 0) return KVX_SUCCESS;
  if (!send_bufs || !layer_bases || !xfers || !xfer_count) return KVX_ERR_INVALID_ARGUMENT;
  for (int32_t s = 0; s < num_src; ++s) {
    if (!send_bufs[s]) return KVX_ERR_INVALID_ARGUMENT;
    if (!aligned16(send_bufs[s])) return KVX_ERR_MISALIGNED;
  }
  if (num_src == 1)
    return from_hip(kvx::launch_copy_runs(kvx::kDirFromBuffer, layer_bases, nullptr, num_layers,
                                          block_bytes, num_cache_blocks, 0, xfers, xfer_count,
                                          total_blocks, const_cast<void*>(send_bufs[0]), err_flag,
                                          stream));
  return from_hip(kvx::launch_shards(false, const_cast<void* const*>(send_bufs), num_src, layer_bases,
                                     num_layers, block_bytes, num_cache_blocks, rows_per_block,
                                     xfers, xfer_count, total_blocks, err_flag, stream));
}

kvx_status kvx_copy_direct(void* const* src_layer_bases, void* const* dst_layer_bases,
                           int32_t num_layers, int64_t block_bytes, int64_t src_num_blocks,
                           int64_t dst_num_blocks, const kvx_xfer* xfers,
                           const int64_t* xfer_count, int64_t total_blocks, int32_t* err_flag,
                           hipStream_t stream) {
  if (num_layers < 0 || block_bytes <= 0 || src_num_blocks < 0 || dst_num_blocks < 0 ||
      total_blocks < 0 || total_blocks > kMaxBlocks ||
      !copy_extents_ok(num_layers, total_blocks, src_num_blocks, block_bytes) ||
      !extent_ok(dst_num_blocks, block_bytes))
    return KVX_ERR_INVALID_ARGUMENT;
  if (num_layers == 0 || total_blocks == 0) return KVX_SUCCESS;
  if (!src_layer_bases || !dst_layer_bases || !xfers || !xfer_count || src_num_blocks == 0)
    return KVX_ERR_INVALID_ARGUMENT;
  if (!mult16(block_bytes)) return KVX_ERR_MISALIGNED;
  return from_hip(kvx::launch_copy_runs(kvx::kDirDirect, src_layer_bases, dst_layer_bases,
                                        num_layers, block_bytes, src_num_blocks, dst_num_blocks,
                                        xfers, xfer_count, total_blocks, nullptr, err_flag,
                                        stream));
}

kvx_status kvx_pack_split(void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                          int64_t num_cache_blocks, int32_t rows_per_block, const kvx_xfer* xfers,
                          const int64_t* xfer_count, int64_t total_blocks, void* const* send_bufs,
                          int32_t num_dst, int32_t* err_flag, hipStream_t stream) {
  if (num_dst < 1 || num_dst > KVX_MAX_SOURCES || num_layers < 0 || block_bytes <= 0 ||
      num_cache_blocks < 0 || total_blocks < 0 || total_blocks > kMaxBlocks || rows_per_block < 1 ||
      !copy_extents_ok(num_layers, total_blocks, num_cache_blocks, block_bytes))
    return KVX_ERR_INVALID_ARGUMENT;
  if (!mult16(block_bytes)) return KVX_ERR_MISALIGNED;
  if (block_bytes % ((int64_t)rows_per_block * num_dst * 16) != 0) return KVX_ERR_INVALID_ARGUMENT;
  if (num_layers == 0 || total_blocks == 0) return KVX_SUCCESS;
  if (!send_bufs || !layer_bases || !xfers || !xfer_count) return KVX_ERR_INVALID_ARGUMENT;
  for (int32_t d = 0; d < num_dst; ++d) {
    if (!send_bufs[d]) return KVX_ERR_INVALID_ARGUMENT;
    if (!aligned16(send_bufs[d])) return KVX_ERR_MISALIGNED;
  }
  return from_hip(kvx::launch_shards(true, send_bufs, num_dst, layer_bases, num_layers, block_bytes,
                                     num_cache_blocks, rows_per_block, xfers, xfer_count,
                                     total_blocks, err_flag, stream));
}

static kvx_status signal_checks(uint64_t* counter, uint32_t* arrivals) {
  if (!counter || !arrivals) return KVX_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)counter & 7u) != 0 || ((uintptr_t)arrivals & 127u) != 0) return KVX_ERR_MISALIGNED;
  return KVX_SUCCESS;
}

kvx_status kvx_pack_signal(void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                           int64_t num_cache_blocks, const kvx_xfer* xfers,
                           const int64_t* xfer_count, int64_t total_blocks, void* send_buf,
                           uint64_t* counter, uint64_t delta, uint32_t* arrivals,
                           int32_t* err_flag, hipStream_t stream) {
  const kvx_status sc = signal_checks(counter, arrivals);
  if (sc != KVX_SUCCESS) return sc;
  if (num_layers < 0 || block_bytes <= 0 || num_cache_blocks < 0 || total_blocks < 0 ||
      total_blocks > kMaxBlocks ||
      !copy_extents_ok(num_layers, total_blocks, num_cache_blocks, block_bytes))
    return KVX_ERR_INVALID_ARGUMENT;
  if (num_layers == 0 || total_blocks == 0)  // nothing to copy: the signal still goes out
    return from_hip(kvx::launch_signal_add(counter, delta, stream));
  if (!layer_bases || !xfers || !xfer_count || !send_buf) return KVX_ERR_INVALID_ARGUMENT;
  if (!mult16(block_bytes) || !aligned16(send_buf)) return KVX_ERR_MISALIGNED;
  const kvx::SignalSpec sig = {counter, delta, arrivals};
  return from_hip(kvx::launch_copy_runs(kvx::kDirToBuffer, layer_bases, nullptr, num_layers,
                                        block_bytes, num_cache_blocks, 0, xfers, xfer_count,
                                        total_blocks, send_buf, err_flag, stream, &sig));
}

kvx_status kvx_copy_direct_signal(void* const* src_layer_bases, void* const* dst_layer_bases,
                                  int32_t num_layers, int64_t block_bytes, int64_t src_num_blocks,
                                  int64_t dst_num_blocks, const kvx_xfer* xfers,
                                  const int64_t* xfer_count, int64_t total_blocks,
                                  uint64_t* counter, uint64_t delta, uint32_t* arrivals,
                                  int32_t* err_flag, hipStream_t stream) {
  const kvx_status sc = signal_checks(counter, arrivals);
  if (sc != KVX_SUCCESS) return sc;
  if (num_layers < 0 || block_bytes <= 0 || src_num_blocks < 0 || dst_num_blocks < 0 ||
      total_blocks < 0 || total_blocks > kMaxBlocks ||
      !copy_extents_ok(num_layers, total_blocks, src_num_blocks, block_bytes) ||
      !extent_ok(dst_num_blocks, block_bytes))
    return KVX_ERR_INVALID_ARGUMENT;
  if (num_layers == 0 || total_blocks == 0)
    return from_hip(kvx::launch_signal_add(counter, delta, stream));
  if (!src_layer_bases || !dst_layer_bases || !xfers || !xfer_count || src_num_blocks == 0)
    return KVX_ERR_INVALID_ARGUMENT;
  if (!mult16(block_bytes)) return KVX_ERR_MISALIGNED;
  const kvx::SignalSpec sig = {counter, delta, arrivals};
  return from_hip(kvx::launch_copy_runs(kvx::kDirDirect, src_layer_bases, dst_layer_bases,
                                        num_layers, block_bytes, src_num_blocks, dst_num_blocks,
                                        xfers, xfer_count, total_blocks, nullptr, err_flag, stream,
                                        &sig));
}

kvx_status kvx_pack_signal_noalloc(void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                                   int64_t num_cache_blocks, const kvx_xfer* xfers,
                                   const int64_t* xfer_count, int64_t total_blocks, void* send_buf,
                                   uint64_t* counter, uint64_t delta, int32_t slot,
                                   int32_t* err_flag, hipStream_t stream) {
  if (slot < 0 || slot >= KVX_NOALLOC_SLOTS) return KVX_ERR_CAPACITY;
  if (!counter) return KVX_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)counter & 7u) != 0) return KVX_ERR_MISALIGNED;
  if (num_layers < 0 || block_bytes <= 0 || num_cache_blocks < 0 || total_blocks < 0 ||
      total_blocks > kMaxBlocks ||
      !copy_extents_ok(num_layers, total_blocks, num_cache_blocks, block_bytes))
    return KVX_ERR_INVALID_ARGUMENT;
  if (num_layers == 0 || total_blocks == 0)
    return from_hip(kvx::launch_signal_add(counter, delta, stream));
  if (!layer_bases || !xfers || !xfer_count || !send_buf) return KVX_ERR_INVALID_ARGUMENT;
  if (!mult16(block_bytes) || !aligned16(send_buf)) return KVX_ERR_MISALIGNED;
  uint32_t* words = nullptr;
  const kvx_status st = scratch_words(stream, &words);
  if (st != KVX_SUCCESS) return st;
  const kvx::SignalSpec sig = {counter, delta, words + (int64_t)slot * (KVX_ARRIVALS_BYTES / 4)};
  return from_hip(kvx::launch_copy_runs(kvx::kDirToBuffer, layer_bases, nullptr, num_layers,
                                        block_bytes, num_cache_blocks, 0, xfers, xfer_count,
                                        total_blocks, send_buf, err_flag, stream, &sig));
}

static kvx_status kv_first_checks(void* const* layer_bases, int32_t num_layers,
                                  int64_t segment_bytes, int64_t plane_stride_bytes,
                                  int64_t num_cache_blocks, const int64_t* req_offsets,
                                  int32_t num_reqs, const kvx_xfer* xfers,
                                  const int64_t* xfer_count, int64_t total_blocks,
                                  const void* buffer) {
  if (num_layers < 0 || segment_bytes <= 0 || plane_stride_bytes < 0 || num_cache_blocks < 0 ||
      total_blocks < 0 || total_blocks > kMaxBlocks || num_reqs < 0 ||
      !extent_ok(2, plane_stride_bytes) || !extent_ok(2, segment_bytes) ||
      !extent_ok((int64_t)num_layers * total_blocks, 2 * segment_bytes))
    return KVX_ERR_INVALID_ARGUMENT;
  if (segment_bytes % 1024 != 0 || !mult16(plane_stride_bytes)) return KVX_ERR_MISALIGNED;
  // the V plane starts after the K plane's blocks (planes never overlap)
  if (num_cache_blocks > plane_stride_bytes / segment_bytes) return KVX_ERR_INVALID_ARGUMENT;
  if (num_layers == 0 || total_blocks == 0) return KVX_SUCCESS;
  if (num_reqs == 0 || !layer_bases || !req_offsets || !xfers || !xfer_count || !buffer)
    return KVX_ERR_INVALID_ARGUMENT;
  if (!aligned16(buffer)) return KVX_ERR_MISALIGNED;
  return KVX_SUCCESS;
}

kvx_status kvx_pack_kv_first(void* const* layer_bases, int32_t num_layers, int64_t segment_bytes,
                             int64_t plane_stride_bytes, int64_t num_cache_blocks,
                             const int64_t* req_offsets, int32_t num_reqs, const kvx_xfer* xfers,
                             const int64_t* xfer_count, int64_t total_blocks, void* send_buf,
                             int32_t* err_flag, hipStream_t stream) {
  const kvx_status st = kv_first_checks(layer_bases, num_layers, segment_bytes, plane_stride_bytes,
                                        num_cache_blocks, req_offsets, num_reqs, xfers, xfer_count,
                                        total_blocks, send_buf);
  if (st != KVX_SUCCESS || num_layers == 0 || total_blocks == 0) return st;
  return from_hip(kvx::launch_kv_first(true, layer_bases, num_layers, segment_bytes,
                                       plane_stride_bytes, num_cache_blocks, req_offsets, num_reqs,
                                       xfers, xfer_count, total_blocks, send_buf, err_flag, stream));
}

kvx_status kvx_unpack_kv_first(const void* send_buf, void* const* layer_bases, int32_t num_layers,
                               int64_t segment_bytes, int64_t plane_stride_bytes,
                               int64_t num_cache_blocks, const int64_t* req_offsets,
                               int32_t num_reqs, const kvx_xfer* xfers, const int64_t* xfer_count,
                               int64_t total_blocks, int32_t* err_flag, hipStream_t stream) {
  const kvx_status st = kv_first_checks(layer_bases, num_layers, segment_bytes, plane_stride_bytes,
                                        num_cache_blocks, req_offsets, num_reqs, xfers, xfer_count,
                                        total_blocks, send_buf);
  if (st != KVX_SUCCESS || num_layers == 0 || total_blocks == 0) return st;
  return from_hip(kvx::launch_kv_first(false, layer_bases, num_layers, segment_bytes,
                                       plane_stride_bytes, num_cache_blocks, req_offsets, num_reqs,
                                       xfers, xfer_count, total_blocks, const_cast<void*>(send_buf),
                                       err_flag, stream));
}

}  // extern "C"
