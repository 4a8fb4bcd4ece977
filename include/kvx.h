/*
 * kvx.h — C ABI of libkvx: the data-parallel hot path of prefill/decode-disaggregated
 * KV-cache transfer on one AMD Instinct MI355X (gfx950).
 *
 * Sources (the pages this interface is built from):
 *   "0. vllm 如何使用 nccl 传输 kv cache", §2.4 KV cache connector: the sender gathers
 *       layer[block_ids] for each request and layer; the receiver writes the received tensor
 *       into kv_cache_layer[block_ids].
 *   "vllm v1 调度逻辑 和 distributed 分布式原理" (diagram): the slot rule of the
 *       batch-tensor label; 16-slot paged blocks; one block table serving all layers whose
 *       per-layer caches are separate allocations.
 *   "5. flagcx connector design & dev & test", §1.2 final design, _send_blocks: the
 *       transfer list is flattened per layer x contiguous group x request.
 *   "vLLM PD 分离", §四 4.2 (_build_transfer_params: per-layer, per-block source and
 *       destination addresses; TP heterogeneity) and §七 item 3 (a block's address is the
 *       layer's base address plus block length times block id).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked [host]. Every device pointer, and every
 *     byte size or byte stride, must be a multiple of 16 (the kernels move 16-byte vectors),
 *     except the int32/int64 index arrays, which need only their natural alignment.
 *   - The call validates its arguments on the host, then enqueues its kernel(s) on `stream`
 *     and returns. It never synchronises, never allocates or frees memory, and keeps no
 *     state between calls (safe to call from several threads); the one exception is the
 *     arrivals workspace of the signalling copies, which the caller owns (or, for
 *     kvx_pack_signal_noalloc, the library's static array). The caller owns all memory
 *     and must keep it alive until the stream work completes.
 *   - Return value: KVX_SUCCESS, or an error detected before anything was enqueued
 *     (KVX_ERR_INVALID_ARGUMENT, KVX_ERR_MISALIGNED, KVX_ERR_CAPACITY), or KVX_ERR_HIP when
 *     the launch itself failed.
 *   - Data-dependent errors (an id outside its range) are found on the device: the
 *     offending element is skipped and the matching KVX_DEVERR_* bit is OR-ed into
 *     `*err_flag` (if err_flag is not NULL). The caller clears the flag before the call and
 *     reads it after synchronising.
 *   - Results are bit-exact: all data is moved as raw bytes (no floating-point ops).
 *   - Block ids are int32; positions, slots, offsets and counts are int64; byte offsets are
 *     computed in 64-bit. Sizes that describe a byte extent past KVX_MAX_EXTENT_BYTES (a
 *     cache's blocks x block bytes, a buffer's layers x blocks x block bytes, a count times
 *     its stride) cannot be a real allocation and return KVX_ERR_INVALID_ARGUMENT, so that no
 *     offset a kernel forms can overflow.
 */
#ifndef KVX_H
#define KVX_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvx_status {
  KVX_SUCCESS = 0,
  KVX_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, negative size, bad mode, ... */
  KVX_ERR_MISALIGNED = 2,       /* a pointer, size or stride is not a multiple of 16    */
  KVX_ERR_CAPACITY = 3,         /* an output array is smaller than the worst case, or a
                                   request goes past the library's fixed scratch          */
  KVX_ERR_HIP = 4               /* the HIP launch failed                                */
} kvx_status;

/* Largest byte extent one call may describe (2^56 bytes, 64 PiB). */
#define KVX_MAX_EXTENT_BYTES (1LL << 56)

/* Device error bits OR-ed into *err_flag. */
#define KVX_DEVERR_BLOCK_RANGE 1 /* a cache block id outside [0, num_cache_blocks)        */
#define KVX_DEVERR_TABLE_RANGE 2 /* slot mapping: request index or position off the table */
#define KVX_DEVERR_SLOT_RANGE 4  /* new-token write: slot in a block >= num_blocks         */
#define KVX_DEVERR_OFFSETS 8     /* run building: req_offsets is not a CSR over the blocks */
#define KVX_DEVERR_TIMEOUT 16    /* signal wait: the counter did not reach its value in time */

/* Which side(s) of a transfer a run must be +1-consecutive on. */
#define KVX_MODE_PACK 0   /* cache -> buffer: runs consecutive in the source ids        */
#define KVX_MODE_UNPACK 1 /* buffer -> cache: runs consecutive in the destination ids   */
#define KVX_MODE_DIRECT 2 /* cache -> cache: consecutive in both (one descriptor = one
                             (src, dst, length) triple of the pages' RDMA transfer)     */

/* Most sources one kvx_unpack call can merge. */
#define KVX_MAX_SOURCES 8

/* Bytes of the arrivals workspace of one signalling copy (kvx_pack_signal,
 * kvx_copy_direct_signal). */
#define KVX_ARRIVALS_BYTES 4096

/* Arrivals workspaces the library keeps per GPU for kvx_pack_signal_noalloc. */
#define KVX_NOALLOC_SLOTS 16

/* One run (a "contiguous group" of the flagcx page §1.2): num_blocks blocks of one request
 * that are consecutive on the addressed side(s).
 *   src_block  first id read     (cache id for PACK/DIRECT; buffer position for UNPACK)
 *   dst_block  first id written  (buffer position for PACK; cache id for UNPACK/DIRECT)
 *   buf_block  position of the run's first block in the flat request-major order of all
 *              listed blocks: (blocks of earlier requests) + index in its block table.
 *              That is where the run sits inside one layer's slice of the send buffer.
 *   num_blocks run length (>= 1); req: the request index. 32 bytes; arrays of them are
 *   16-byte aligned. */
typedef struct kvx_xfer {
  int64_t src_block;
  int64_t dst_block;
  int64_t buf_block;
  int32_t num_blocks;
  int32_t req;
} kvx_xfer;

/* Static description of a status code (never NULL). [host] */
const char* kvx_status_string(kvx_status status);

/* Library ABI version (increases when a signature or struct changes). [host] */
int32_t kvx_abi_version(void);

/*
 * kvx_slot_mapping — slot of every flat token (page "vllm v1 调度逻辑 和 distributed
 * 分布式原理", batch-tensor label):
 *     slot_mapping[i] = block_table[req_idx[i]][positions[i] / block_size] * block_size
 *                       + positions[i] % block_size
 *   block_table      int32 [num_reqs][bt_row_stride]; row r's first max_blocks_per_req
 *                    entries are valid columns (unused columns may hold negative ids).
 *   req_idx          int32 [num_tokens];  positions  int64 [num_tokens].
 *   slot_mapping     int64 [num_tokens] (output).
 * A token whose request index is outside [0, num_reqs), whose position is negative or
 * maps past column max_blocks_per_req-1, or whose table entry is negative, gets slot -1
 * and raises KVX_DEVERR_TABLE_RANGE. num_tokens == 0 enqueues nothing.
 * Errors: INVALID_ARGUMENT for NULL arrays (when num_tokens > 0), num_tokens < 0,
 * num_reqs < 0, block_size < 1, max_blocks_per_req < 0 or > bt_row_stride.
 */
kvx_status kvx_slot_mapping(const int32_t* block_table, int64_t num_reqs,
                            int64_t max_blocks_per_req, int64_t bt_row_stride,
                            const int32_t* req_idx, const int64_t* positions,
                            int64_t num_tokens, int32_t block_size, int64_t* slot_mapping,
                            int32_t* err_flag, hipStream_t stream);

/*
 * kvx_reshape_and_cache — write each new token's K row and V row into its cache slot
 * (slot rule of the batch-tensor label; 16-slot block of the "Paged kv cache" label; the
 * recomputed last prompt token of "vLLM PD 分离" §五 5.2 is written this way):
 *     block = slot / block_size, offset = slot % block_size
 *     cache[block*block_stride + offset*token_stride + 0*kv_stride + (0..row_bytes)] = key[i]
 *     cache[block*block_stride + offset*token_stride + 1*kv_stride + (0..row_bytes)] = value[i]
 *   key, value     token i's row starts at key + i*key_stride_bytes (resp. value); each row is
 *                  row_bytes = num_kv_heads*head_dim*element bytes, a multiple of 16.
 *   slot_mapping   int64 [num_tokens]; slot < 0 means "no slot" (padding) and is skipped.
 *   kv_cache       num_blocks blocks. Strides in bytes; for the [blocks][block_size][K,V][heads]
 *                  [head_dim] layout: kv_stride = row_bytes, token_stride = 2*row_bytes,
 *                  block_stride = block_size*token_stride. (blocks, K/V, tokens, ...) and
 *                  (K/V, blocks, tokens, ...) layouts are expressed with other strides.
 * A slot in a block >= num_blocks is skipped and raises KVX_DEVERR_SLOT_RANGE. Two tokens
 * with the same slot race (the pages never produce that). The caller guarantees every
 * addressed byte lies inside the kv_cache allocation.
 */
kvx_status kvx_reshape_and_cache(const void* key, int64_t key_stride_bytes, const void* value,
                                 int64_t value_stride_bytes, int64_t num_tokens,
                                 int64_t row_bytes, const int64_t* slot_mapping,
                                 void* kv_cache, int64_t num_blocks, int32_t block_size,
                                 int64_t block_stride_bytes, int64_t token_stride_bytes,
                                 int64_t kv_stride_bytes, int32_t* err_flag,
                                 hipStream_t stream);

/*
 * kvx_build_xfer_list — cut every request's block list into maximal runs (flagcx page §1.2,
 * _send_blocks; "vLLM PD 分离" §四 4.2 and §七 item 3).
 *   Requests are given in CSR form: request r owns flat positions
 *   [req_offsets[r], req_offsets[r+1]) of src_ids / dst_ids (int32 block ids);
 *   req_offsets is int64 [num_reqs+1] with req_offsets[0] = 0, non-decreasing, and
 *   req_offsets[num_reqs] = total_blocks.
 *   src_ids is required for PACK and DIRECT, dst_ids for UNPACK and DIRECT (the other may
 *   be NULL). A run breaks at every request start and wherever an addressed side does not
 *   step by +1. Runs are written in request order, then block-table order, to
 *   xfers[0 .. *xfer_count), with buf_block = flat position of the run's first block.
 *   xfers       kvx_xfer [capacity] (output), 16-byte aligned (else KVX_ERR_MISALIGNED:
 *               records are written as 16-byte vectors); capacity >= total_blocks is
 *               required (the worst case is one run per block), else KVX_ERR_CAPACITY.
 *   xfer_count  int64 [1] (output, device): number of runs written.
 * The list is the same for every layer (one block table serves all layers), so one list
 * drives kvx_pack / kvx_unpack for all layers. An invalid req_offsets raises
 * KVX_DEVERR_OFFSETS (runs are then cut where the offsets say, clamped to the blocks).
 * total_blocks == 0 writes *xfer_count = 0.
 */
kvx_status kvx_build_xfer_list(const int32_t* src_ids, const int32_t* dst_ids,
                               const int64_t* req_offsets, int32_t num_reqs,
                               int64_t total_blocks, int32_t mode, kvx_xfer* xfers,
                               int64_t capacity, int64_t* xfer_count, int32_t* err_flag,
                               hipStream_t stream);

/*
 * kvx_pack — gather all listed blocks of all layers into one contiguous send buffer
 * ("0. vllm 如何使用 nccl 传输 kv cache" §2.4, extract_kv_from_layer; flagcx page §1.2 for
 * the order layer -> request -> block-table order):
 *     send_buf[l][p] = block xfer.src_block + (p - xfer.buf_block) of layer l's cache,
 *     for every run xfer and p in [xfer.buf_block, xfer.buf_block + xfer.num_blocks)
 *   layer_bases   DEVICE array [num_layers] of device pointers, one per layer's cache
 *                 (separate allocations). A layer's cache is num_cache_blocks blocks of
 *                 block_bytes contiguous bytes each: block b starts at base + b*block_bytes.
 *   xfers, xfer_count  a list from kvx_build_xfer_list in KVX_MODE_PACK or KVX_MODE_DIRECT
 *                 (read on the device; no host synchronisation is needed). Counts larger
 *                 than total_blocks are clamped.
 *   send_buf      [num_layers][total_blocks][block_bytes] bytes (output).
 * Whole blocks are copied, including unfilled tail slots. A run (part) whose source ids
 * fall outside [0, num_cache_blocks), or whose buffer positions fall outside
 * [0, total_blocks), is skipped and raises KVX_DEVERR_BLOCK_RANGE.
 * total_blocks == 0 or num_layers == 0 enqueues nothing.
 */
kvx_status kvx_pack(void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                    int64_t num_cache_blocks, const kvx_xfer* xfers,
                    const int64_t* xfer_count, int64_t total_blocks, void* send_buf,
                    int32_t* err_flag, hipStream_t stream);

/*
 * kvx_unpack — scatter send buffer(s) into the receiver's own blocks
 * ("0. vllm 如何使用 nccl 传输 kv cache" §2.3 step 14 and §2.4, inject_kv_into_layer;
 * "vLLM PD 分离" §七 item 3 for the addressing and §四 4.2 for TP heterogeneity):
 *     block xfer.dst_block + (p - xfer.buf_block) of layer l's cache  <-  buffer block (l, p)
 *   send_bufs     [host] array [num_src] of device pointers, 1 <= num_src <= KVX_MAX_SOURCES.
 *                 Source s is [num_layers][total_blocks][block_bytes/num_src] bytes.
 *   num_src == 1: plain copy of whole blocks.
 *   num_src  > 1: head merge for a TP num_src -> 1 receive. Every block is rows_per_block
 *                 rows (rows_per_block = block_size*2 for the [tokens][K,V][heads][head_dim]
 *                 block: one row per (token, K/V)); destination row k is the concatenation
 *                 of row k of source 0, source 1, ... (source s holds heads
 *                 [s*H/num_src, (s+1)*H/num_src)). block_bytes must be a multiple of
 *                 rows_per_block*num_src*16.
 *   layer_bases   DEVICE array [num_layers] of the destination caches (num_cache_blocks
 *                 blocks of block_bytes each).
 *   xfers, xfer_count  a list from kvx_build_xfer_list in KVX_MODE_UNPACK or
 *                 KVX_MODE_DIRECT.
 * Blocks not listed keep their bytes. Destination ids must be unique (a receiver allocates
 * fresh blocks); duplicates race. Out-of-range destination ids or buffer positions are
 * skipped and raise KVX_DEVERR_BLOCK_RANGE.
 */
kvx_status kvx_unpack(const void* const* send_bufs, int32_t num_src, void* const* layer_bases,
                      int32_t num_layers, int64_t block_bytes, int64_t num_cache_blocks,
                      int32_t rows_per_block, const kvx_xfer* xfers,
                      const int64_t* xfer_count, int64_t total_blocks, int32_t* err_flag,
                      hipStream_t stream);

/*
 * kvx_copy_direct — move the listed blocks of every layer straight from the sender's caches
 * into the receiver's, with no send buffer ("vLLM PD 分离" §四 4.2: one write per source
 * address, destination address and length, from the prefill cache into the decode cache;
 * §七 item 3: address = layer base + block length x id). For layer l and every run, blocks
 * src_block .. src_block + num_blocks - 1 of src layer l go to dst_block .. of dst layer l.
 * It is the one-pass form of pack + unpack: 2 x block_bytes of HBM traffic per (layer, block)
 * instead of 4, and the data-parallel part of a one-sided transfer whose destination is a
 * peer's cache.
 *   src_layer_bases / dst_layer_bases  device arrays [num_layers] of layer base pointers.
 *   src_num_blocks / dst_num_blocks    blocks per layer on each side (src_num_blocks >= 1).
 *   xfers, xfer_count, total_blocks    a run list built with KVX_MODE_DIRECT (runs
 *                                      consecutive on both sides).
 * The two sides may be the same caches (a copy between blocks of one cache), but no
 * destination block may also be a source block of the same call, and destination ids must
 * be unique: blocks move concurrently, in no particular order.
 * An entry whose source or destination id is outside its cache is skipped and raises
 * KVX_DEVERR_BLOCK_RANGE. Errors: INVALID_ARGUMENT for NULL pointers (when there is work),
 * negative sizes or src_num_blocks == 0; MISALIGNED for block_bytes not a multiple of 16.
 */
kvx_status kvx_copy_direct(void* const* src_layer_bases, void* const* dst_layer_bases,
                           int32_t num_layers, int64_t block_bytes, int64_t src_num_blocks,
                           int64_t dst_num_blocks, const kvx_xfer* xfers,
                           const int64_t* xfer_count, int64_t total_blocks, int32_t* err_flag,
                           hipStream_t stream);

/*
 * kvx_pack_split — sender-side head split for an asymmetric TP transfer where the receiver
 * runs num_dst ranks ("vLLM PD 分离" §四 4.2, TP heterogeneity): the inverse of kvx_unpack's
 * merge. Every full-head cache block is rows_per_block rows (block_size*2 for the
 * [tokens][K,V][heads][head_dim] block); receiver d owns heads [d*H/num_dst, (d+1)*H/num_dst),
 * i.e. piece d of each row. Buffer d is [num_layers][total_blocks][block_bytes/num_dst] in
 * pack's order and holds piece d of every row of every listed block:
 *     send_bufs[d][l][p] row k = bytes [d*piece, (d+1)*piece) of row k of the block that
 *     kvx_pack would put at (l, p).
 *   send_bufs     [host] array [num_dst] of device pointers, 1 <= num_dst <= KVX_MAX_SOURCES.
 *   block_bytes must be a multiple of rows_per_block*num_dst*16. Runs: KVX_MODE_PACK or
 *   KVX_MODE_DIRECT. Errors and range handling as kvx_pack.
 */
kvx_status kvx_pack_split(void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                          int64_t num_cache_blocks, int32_t rows_per_block, const kvx_xfer* xfers,
                          const int64_t* xfer_count, int64_t total_blocks, void* const* send_bufs,
                          int32_t num_dst, int32_t* err_flag, hipStream_t stream);

/*
 * kvx_pack_kv_first / kvx_unpack_kv_first — the same transfer for kv-first caches, whose
 * layer tensor is (K/V plane, blocks, block_size, heads, head_dim) ("vllm v1 调度逻辑 和
 * distributed 分布式原理", "shape of layer i"; "0. vllm 如何使用 nccl 传输 kv cache" §2.4,
 * which gathers along dimension 1 when the K/V dimension comes first).
 *   A block is one segment_bytes segment in each plane: block b's K segment starts at
 *   base + b*segment_bytes and its V segment at base + plane_stride_bytes + b*segment_bytes
 *   (plane_stride_bytes = num_cache_blocks*segment_bytes for a contiguous tensor).
 *   Buffer layout: [num_layers][2*total_blocks][segment_bytes]; in each layer, request r's
 *   part starts at segment 2*req_offsets[r] and is its K segments in block-table order, then
 *   its V segments — exactly what gathering the layer tensor along the block axis with the
 *   request's block ids returns, one contiguous tensor per (request, layer).
 *   req_offsets   int64 [num_reqs+1], the CSR the run list was built from.
 *   plane_stride_bytes >= num_cache_blocks*segment_bytes (the planes do not overlap), else
 *   KVX_ERR_INVALID_ARGUMENT.
 *   segment_bytes must be a multiple of 1024 (KVX_ERR_MISALIGNED otherwise): true for any
 *   16-token block with heads*head_dim a multiple of 32 at 2 bytes per element.
 *   Runs: pack needs KVX_MODE_PACK or KVX_MODE_DIRECT; unpack KVX_MODE_UNPACK or
 *   KVX_MODE_DIRECT. Out-of-range ids are skipped and raise KVX_DEVERR_BLOCK_RANGE.
 */
kvx_status kvx_pack_kv_first(void* const* layer_bases, int32_t num_layers, int64_t segment_bytes,
                             int64_t plane_stride_bytes, int64_t num_cache_blocks,
                             const int64_t* req_offsets, int32_t num_reqs, const kvx_xfer* xfers,
                             const int64_t* xfer_count, int64_t total_blocks, void* send_buf,
                             int32_t* err_flag, hipStream_t stream);

kvx_status kvx_unpack_kv_first(const void* send_buf, void* const* layer_bases, int32_t num_layers,
                               int64_t segment_bytes, int64_t plane_stride_bytes,
                               int64_t num_cache_blocks, const int64_t* req_offsets,
                               int32_t num_reqs, const kvx_xfer* xfers, const int64_t* xfer_count,
                               int64_t total_blocks, int32_t* err_flag, hipStream_t stream);

/*
 * kvx_signal_add / kvx_signal_wait — device-side completion signalling between two streams
 * ("5. flagcx connector design & dev & test", §1.2, the send path and wait_for_layer_load:
 * the last transfer of a batch adds to the receiver's signal counter, and the receiver's
 * stream waits on the GPU until the counter is at least the value it was told to expect).
 * Used to pipeline a transfer layer by layer: the producer stream packs layer l and then
 * adds 1; the consumer stream waits for l+1 and then moves layer l on.
 *   counter     one uint64 in device memory, 8-byte aligned, owned by the caller; it only
 *               ever grows, so waiting for the largest expected value covers smaller ones.
 *   kvx_signal_add: once every piece of work enqueued on `stream` before this call has
 *               finished, atomically adds `delta` to *counter (a device-coherent atomic).
 *               The kernel boundary in front of it has already made that earlier work's
 *               writes visible to the whole device, so whoever sees the new count on this
 *               GPU also sees those writes.
 *   kvx_signal_wait: work enqueued on `stream` after this call starts only once
 *               *counter >= value; that work acquires at its own kernel boundary, so it
 *               reads what the producer wrote before the add. The wait is one wavefront polling the
 *               counter on the GPU; the host is never blocked. After timeout_us microseconds
 *               of wall-clock time it gives up, ORs KVX_DEVERR_TIMEOUT into *err_flag (if
 *               not NULL) and lets the stream go on, so a missing signal cannot keep the
 *               device busy for ever. timeout_us must be in [1, 60000000].
 *   Enqueue every add before the wait that expects it (host program order): the two
 *   streams may then share a hardware queue without waiting on each other in a circle.
 * Errors: INVALID_ARGUMENT for a NULL counter or a timeout out of range, MISALIGNED for a
 * counter not 8-byte aligned, KVX_ERR_HIP when the launch (or the wall-clock rate query)
 * fails.
 */
kvx_status kvx_signal_add(uint64_t* counter, uint64_t delta, hipStream_t stream);

kvx_status kvx_signal_wait(const uint64_t* counter, uint64_t value, int64_t timeout_us,
                           int32_t* err_flag, hipStream_t stream);

/*
 * kvx_pack_signal / kvx_copy_direct_signal — kvx_pack and kvx_copy_direct whose launch also
 * carries the completion signal ("5. flagcx connector design & dev & test", §1.2: the last
 * transfer of a batch adds to the receiver's signal counter, putSignal; the receiver's
 * wait_for_layer_load waits for the count). Same copy, same arguments and errors as the
 * plain call, plus:
 *   counter    the uint64 signal counter (device memory, 8-byte aligned), as kvx_signal_add.
 *              Once every byte this call writes is visible to the whole device, the call
 *              adds `delta` to it, exactly once. A kvx_signal_wait for the new count (or work
 *              that reads the counter) therefore sees all of this call's bytes.
 *   arrivals   KVX_ARRIVALS_BYTES of device memory (128-byte aligned), owned by the caller,
 *              all zero before the first call; each call counts its finished workgroups
 *              there (16 group counters and a total, each on its own 128-byte line) and
 *              leaves it all zero again when it ends. Calls that share an arrivals workspace
 *              must not run at the same time (enqueue them on one stream); give concurrent
 *              streams one each. A call that has nothing to copy (num_layers == 0 or
 *              total_blocks == 0) still adds `delta`.
 * Used for the per-layer sender pipeline: kvx_pack_signal of layer l with delta 1 replaces
 * kvx_pack + kvx_signal_add, and saves the separate signal launch.
 * Errors: as kvx_pack / kvx_copy_direct, plus INVALID_ARGUMENT for a NULL counter or
 * arrivals, MISALIGNED for a counter not 8-byte or arrivals not 128-byte aligned.
 */
kvx_status kvx_pack_signal(void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                           int64_t num_cache_blocks, const kvx_xfer* xfers,
                           const int64_t* xfer_count, int64_t total_blocks, void* send_buf,
                           uint64_t* counter, uint64_t delta, uint32_t* arrivals,
                           int32_t* err_flag, hipStream_t stream);

kvx_status kvx_copy_direct_signal(void* const* src_layer_bases, void* const* dst_layer_bases,
                                  int32_t num_layers, int64_t block_bytes, int64_t src_num_blocks,
                                  int64_t dst_num_blocks, const kvx_xfer* xfers,
                                  const int64_t* xfer_count, int64_t total_blocks,
                                  uint64_t* counter, uint64_t delta, uint32_t* arrivals,
                                  int32_t* err_flag, hipStream_t stream);

/*
 * kvx_pack_signal_noalloc — kvx_pack_signal for callers that cannot allocate, not even the
 * arrivals workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same copy, signal, arguments and errors as kvx_pack_signal, except that the
 * arrivals workspace is workspace `slot` of the library's own static array of
 * KVX_NOALLOC_SLOTS workspaces of KVX_ARRIVALS_BYTES per GPU (64 KiB, held by each GPU the
 * library runs on until the process ends).
 *   slot       0 <= slot < KVX_NOALLOC_SLOTS, else KVX_ERR_CAPACITY before anything else.
 *              Every call on one GPU that uses the same slot shares that workspace: such
 *              calls must not overlap in time (enqueue them on one stream) or they race.
 *              Calls on different slots may run concurrently, e.g. one slot per sender
 *              stream. The workspaces are zero when the library is loaded and every completed
 *              call leaves its workspace zero, as kvx_pack_signal leaves its own.
 *   stream     must belong to the current device (KVX_ERR_INVALID_ARGUMENT otherwise): the
 *              first call on each device looks up the array's address on that device once,
 *              with hipGetSymbolAddress, and keeps it.
 * Allocates nothing, frees nothing, and never synchronises.
 */
kvx_status kvx_pack_signal_noalloc(void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                                   int64_t num_cache_blocks, const kvx_xfer* xfers,
                                   const int64_t* xfer_count, int64_t total_blocks, void* send_buf,
                                   uint64_t* counter, uint64_t delta, int32_t slot,
                                   int32_t* err_flag, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVX_H */
