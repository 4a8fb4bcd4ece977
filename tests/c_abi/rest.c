/* A plain C consumer of the libkvx entry points that roundtrip.c does not cover (no Python,
 * no PyTorch): the slot mapping and the new-token write, the kv-first pack and unpack, the
 * head split and the two-source head merge, the signal add and wait, the signalling pack and
 * the signalling direct copy each feeding a consumer stream layer by layer, the allocation-free
 * signalling pack likewise, and the ABI version. It reads one case from a file, runs everything
 * on HIP streams of its own and writes every output to a file for the test to compare with the
 * oracle. It also checks host-side status codes of these entry points.
 *
 *   rest IN OUT
 *   IN:  int64 {magic, L, nb, bs, row, R, N, T, width},
 *        int64 req_offsets[R+1], int32 src_ids[N], int32 dst_ids[N],
 *        int32 block_table[R][width], int32 req_idx[T], int64 positions[T],
 *        uint8 key[T][row], uint8 value[T][row],
 *        uint8 src caches [L][nb][BB], uint8 dst caches [L][nb][BB]   (BB = bs * 2 * row)
 *   OUT: int64 {error flag, wait error flag, signal counter, add counter, status checks passed,
 *              ABI version, direct-copy signal counter, allocation-free signal counter},
 *        int64 slots[T], uint8 layer 0 of the dst caches after the new-token write [nb][BB],
 *        uint8 kv-first buffer [L][2N][BB/2], dst caches after the kv-first unpack,
 *        uint8 shard 0 [L][N][BB/2], shard 1 [L][N][BB/2], dst caches after the merge,
 *        dst caches after the layer-by-layer signalled transfer,
 *        each dst layer as the consumer copied it once the signalled direct copy's count for it
 *        arrived, the allocation-free pack's buffer [L][N][BB], and the dst caches it was
 *        unpacked into layer by layer
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvx.h"

#define MAGIC 0x4B565852LL

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));       \
      exit(2);                                                                \
    }                                                                         \
  } while (0)

#define KVX_OK(call)                                                          \
  do {                                                                        \
    kvx_status s_ = (call);                                                   \
    if (s_ != KVX_SUCCESS) {                                                  \
      fprintf(stderr, "%s failed: %s\n", #call, kvx_status_string(s_));       \
      exit(3);                                                                \
    }                                                                         \
  } while (0)

static void* read_exact(FILE* f, size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p || fread(p, 1, n, f) != n) {
    fprintf(stderr, "short input\n");
    exit(4);
  }
  return p;
}

static void* device_copy(const void* host, size_t n) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, n ? n : 16));
  if (n) HIP_OK(hipMemcpy(d, host, n, hipMemcpyHostToDevice));
  return d;
}

static void* device_zeros(size_t n) {
  void* d = NULL;
  HIP_OK(hipMalloc(&d, n ? n : 16));
  HIP_OK(hipMemset(d, 0, n ? n : 16));
  return d;
}

/* L per-layer caches, each its own allocation, filled from host; returns the device array of
 * their base pointers and keeps the host-side pointers in *layers. */
static void* make_layers(const uint8_t* host, int64_t L, size_t layer, void*** layers) {
  *layers = (void**)malloc((size_t)L * sizeof(void*));
  for (int64_t l = 0; l < L; ++l) (*layers)[l] = device_copy(host + l * layer, layer);
  return device_copy(*layers, (size_t)L * sizeof(void*));
}

static void write_layers(FILE* out, void** layers, int64_t L, size_t layer, uint8_t* scratch_h) {
  for (int64_t l = 0; l < L; ++l) {
    HIP_OK(hipMemcpy(scratch_h, layers[l], layer, hipMemcpyDeviceToHost));
    fwrite(scratch_h, 1, layer, out);
  }
}

static void write_device(FILE* out, const void* d, size_t n) {
  uint8_t* h = (uint8_t*)malloc(n ? n : 1);
  if (n) HIP_OK(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
  fwrite(h, 1, n, out);
  free(h);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: rest IN OUT\n");
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 4;
  int64_t* hdr = (int64_t*)read_exact(in, 9 * sizeof(int64_t));
  if (hdr[0] != MAGIC) return 4;
  const int64_t L = hdr[1], nb = hdr[2], bs = hdr[3], row = hdr[4], R = hdr[5], N = hdr[6];
  const int64_t T = hdr[7], width = hdr[8];
  const int64_t BB = bs * 2 * row, seg = BB / 2;
  int64_t* ro = (int64_t*)read_exact(in, (size_t)(R + 1) * sizeof(int64_t));
  int32_t* sid = (int32_t*)read_exact(in, (size_t)N * sizeof(int32_t));
  int32_t* did = (int32_t*)read_exact(in, (size_t)N * sizeof(int32_t));
  int32_t* table = (int32_t*)read_exact(in, (size_t)(R * width) * sizeof(int32_t));
  int32_t* req = (int32_t*)read_exact(in, (size_t)T * sizeof(int32_t));
  int64_t* pos = (int64_t*)read_exact(in, (size_t)T * sizeof(int64_t));
  uint8_t* key = (uint8_t*)read_exact(in, (size_t)(T * row));
  uint8_t* val = (uint8_t*)read_exact(in, (size_t)(T * row));
  const size_t layer = (size_t)(nb * BB);
  uint8_t* src_h = (uint8_t*)read_exact(in, (size_t)L * layer);
  uint8_t* dst_h = (uint8_t*)read_exact(in, (size_t)L * layer);
  fclose(in);

  void **src_l, **kvf_l, **mrg_l, **sig_l, **wr_l, **dir_l, **seen_l, **nsig_l;
  void* src_bases = make_layers(src_h, L, layer, &src_l);
  void* kvf_bases = make_layers(dst_h, L, layer, &kvf_l);
  void* mrg_bases = make_layers(dst_h, L, layer, &mrg_l);
  void* sig_bases = make_layers(dst_h, L, layer, &sig_l);
  void* wr_bases = make_layers(dst_h, 1, layer, &wr_l);
  (void)wr_bases;
  void* dir_bases = make_layers(dst_h, L, layer, &dir_l);
  void* seen_bases = make_layers(dst_h, L, layer, &seen_l);
  (void)seen_bases;
  void* nsig_bases = make_layers(dst_h, L, layer, &nsig_l);
  int64_t* ro_d = (int64_t*)device_copy(ro, (size_t)(R + 1) * sizeof(int64_t));
  int32_t* sid_d = (int32_t*)device_copy(sid, (size_t)N * sizeof(int32_t));
  int32_t* did_d = (int32_t*)device_copy(did, (size_t)N * sizeof(int32_t));
  int32_t* table_d = (int32_t*)device_copy(table, (size_t)(R * width) * sizeof(int32_t));
  int32_t* req_d = (int32_t*)device_copy(req, (size_t)T * sizeof(int32_t));
  int64_t* pos_d = (int64_t*)device_copy(pos, (size_t)T * sizeof(int64_t));
  void* key_d = device_copy(key, (size_t)(T * row));
  void* val_d = device_copy(val, (size_t)(T * row));
  const int64_t cap = N > 0 ? N : 1;
  kvx_xfer* xp = (kvx_xfer*)device_zeros((size_t)cap * sizeof(kvx_xfer));
  kvx_xfer* xu = (kvx_xfer*)device_zeros((size_t)cap * sizeof(kvx_xfer));
  kvx_xfer* xd = (kvx_xfer*)device_zeros((size_t)cap * sizeof(kvx_xfer));
  int64_t* counts = (int64_t*)device_zeros(3 * sizeof(int64_t));
  int64_t* slots = (int64_t*)device_zeros((size_t)T * sizeof(int64_t));
  int32_t* err = (int32_t*)device_zeros(sizeof(int32_t));
  int32_t* werr = (int32_t*)device_zeros(sizeof(int32_t));
  uint64_t* counter = (uint64_t*)device_zeros(sizeof(uint64_t));
  uint64_t* add_counter = (uint64_t*)device_zeros(sizeof(uint64_t));
  uint32_t* arrivals = (uint32_t*)device_zeros(KVX_ARRIVALS_BYTES);
  uint64_t* dcounter = (uint64_t*)device_zeros(sizeof(uint64_t));
  uint32_t* darrivals = (uint32_t*)device_zeros(KVX_ARRIVALS_BYTES);
  uint64_t* ncounter = (uint64_t*)device_zeros(sizeof(uint64_t));
  const size_t buf_bytes = (size_t)(L * N * BB);
  void* kbuf = device_zeros(buf_bytes);
  void* shard[2] = {device_zeros(buf_bytes / 2), device_zeros(buf_bytes / 2)};
  uint8_t* sbuf = (uint8_t*)device_zeros(buf_bytes);
  uint8_t* nbuf = (uint8_t*)device_zeros(buf_bytes);

  hipStream_t s, prod, cons;
  HIP_OK(hipStreamCreate(&s));
  HIP_OK(hipStreamCreate(&prod));
  HIP_OK(hipStreamCreate(&cons));

  /* host-side status codes: nothing is enqueued for these */
  int64_t checks = 0;
  checks += kvx_slot_mapping(table_d, R, width, width, req_d, pos_d, T, 0, slots, err, s) ==
            KVX_ERR_INVALID_ARGUMENT;
  checks += kvx_reshape_and_cache(key_d, row, val_d, row, T, 8, slots, wr_l[0], nb, (int32_t)bs,
                                  bs * 2 * row, 2 * row, row, err, s) == KVX_ERR_MISALIGNED;
  checks += kvx_pack_kv_first(src_bases, (int32_t)L, 1000, nb * 1000, nb, ro_d, (int32_t)R, xp, counts,
                              N, kbuf, err, s) == KVX_ERR_MISALIGNED;
  checks += kvx_pack_split(src_bases, (int32_t)L, BB, nb, (int32_t)(bs * 2), xp, counts, N, shard,
                           KVX_MAX_SOURCES + 1, err, s) == KVX_ERR_INVALID_ARGUMENT;
  checks += kvx_signal_wait(counter, 1, 0, werr, s) == KVX_ERR_INVALID_ARGUMENT;
  checks += kvx_signal_add((uint64_t*)((char*)counter + 4), 1, s) == KVX_ERR_MISALIGNED;
  checks += kvx_pack_signal(src_bases, (int32_t)L, BB, nb, xp, counts, N, sbuf, counter, 1, NULL, err, s) ==
            KVX_ERR_INVALID_ARGUMENT;
  checks += kvx_pack_signal(src_bases, (int32_t)L, BB, nb, xp, counts, N, sbuf, counter, 1,
                            (uint32_t*)((char*)arrivals + 64), err, s) == KVX_ERR_MISALIGNED;
  checks += kvx_copy_direct_signal(src_bases, dir_bases, (int32_t)L, BB, nb, nb, xd, counts + 2, N,
                                   dcounter, 1, NULL, err, s) == KVX_ERR_INVALID_ARGUMENT;
  checks += kvx_pack_signal_noalloc(src_bases, (int32_t)L, BB, nb, xp, counts, N, nbuf, ncounter, 1,
                                    KVX_NOALLOC_SLOTS, err, s) == KVX_ERR_CAPACITY;

  /* slot mapping, then the new-token write into (a copy of) destination layer 0 */
  KVX_OK(kvx_slot_mapping(table_d, R, width, width, req_d, pos_d, T, (int32_t)bs, slots, err, s));
  KVX_OK(kvx_reshape_and_cache(key_d, row, val_d, row, T, row, slots, wr_l[0], nb, (int32_t)bs,
                               bs * 2 * row, 2 * row, row, err, s));
  /* run lists */
  KVX_OK(kvx_build_xfer_list(sid_d, NULL, ro_d, (int32_t)R, N, KVX_MODE_PACK, xp, cap, counts, err, s));
  KVX_OK(kvx_build_xfer_list(NULL, did_d, ro_d, (int32_t)R, N, KVX_MODE_UNPACK, xu, cap, counts + 1, err, s));
  /* the same caches viewed as kv-first: K plane then V plane of nb segments each */
  KVX_OK(kvx_pack_kv_first(src_bases, (int32_t)L, seg, nb * seg, nb, ro_d, (int32_t)R, xp, counts, N,
                           kbuf, err, s));
  KVX_OK(kvx_unpack_kv_first(kbuf, kvf_bases, (int32_t)L, seg, nb * seg, nb, ro_d, (int32_t)R, xu,
                             counts + 1, N, err, s));
  /* head split into 2 shards, then the two-source merge */
  KVX_OK(kvx_pack_split(src_bases, (int32_t)L, BB, nb, (int32_t)(bs * 2), xp, counts, N, shard, 2, err, s));
  const void* shards[2] = {shard[0], shard[1]};
  KVX_OK(kvx_unpack(shards, 2, mrg_bases, (int32_t)L, BB, nb, (int32_t)(bs * 2), xu, counts + 1, N, err, s));
  /* a plain signal add */
  KVX_OK(kvx_signal_add(add_counter, 5, s));
  KVX_OK(kvx_signal_add(add_counter, 37, s));
  HIP_OK(hipStreamSynchronize(s));

  /* layer by layer: the producer's pack carries the signal; the consumer waits for it and
   * unpacks that layer */
  for (int64_t l = 0; l < L; ++l) {
    void* const* src_one = (void* const*)((char*)src_bases + l * sizeof(void*));
    void* const* dst_one = (void* const*)((char*)sig_bases + l * sizeof(void*));
    uint8_t* slice = sbuf + l * N * BB;
    KVX_OK(kvx_pack_signal(src_one, 1, BB, nb, xp, counts, N, slice, counter, 1, arrivals, err, prod));
    KVX_OK(kvx_signal_wait(counter, (uint64_t)(l + 1), 20000000, werr, cons));
    const void* one[1] = {slice};
    KVX_OK(kvx_unpack(one, 1, dst_one, 1, BB, nb, 1, xu, counts + 1, N, err, cons));
  }
  HIP_OK(hipStreamSynchronize(prod));
  HIP_OK(hipStreamSynchronize(cons));

  /* the direct copy, layer by layer with the signal in its launch: once a layer's count has
   * arrived the consumer copies that destination layer (what a reader sees at that moment) */
  KVX_OK(kvx_build_xfer_list(sid_d, did_d, ro_d, (int32_t)R, N, KVX_MODE_DIRECT, xd, cap, counts + 2, err, s));
  HIP_OK(hipStreamSynchronize(s));
  for (int64_t l = 0; l < L; ++l) {
    void* const* src_one = (void* const*)((char*)src_bases + l * sizeof(void*));
    void* const* dst_one = (void* const*)((char*)dir_bases + l * sizeof(void*));
    KVX_OK(kvx_copy_direct_signal(src_one, dst_one, 1, BB, nb, nb, xd, counts + 2, N, dcounter, 1,
                                  darrivals, err, prod));
    KVX_OK(kvx_signal_wait(dcounter, (uint64_t)(l + 1), 20000000, werr, cons));
    HIP_OK(hipMemcpyAsync(seen_l[l], dir_l[l], layer, hipMemcpyDeviceToDevice, cons));
  }
  /* the allocation-free signalling pack (library workspace 0), as the pipeline above */
  for (int64_t l = 0; l < L; ++l) {
    void* const* src_one = (void* const*)((char*)src_bases + l * sizeof(void*));
    void* const* dst_one = (void* const*)((char*)nsig_bases + l * sizeof(void*));
    uint8_t* slice = nbuf + l * N * BB;
    KVX_OK(kvx_pack_signal_noalloc(src_one, 1, BB, nb, xp, counts, N, slice, ncounter, 1, 0, err, prod));
    KVX_OK(kvx_signal_wait(ncounter, (uint64_t)(l + 1), 20000000, werr, cons));
    const void* one[1] = {slice};
    KVX_OK(kvx_unpack(one, 1, dst_one, 1, BB, nb, 1, xu, counts + 1, N, err, cons));
  }
  HIP_OK(hipStreamSynchronize(prod));
  HIP_OK(hipStreamSynchronize(cons));

  int64_t out_hdr[8];
  int32_t e = 0, we = 0;
  uint64_t c = 0, ac = 0, dc = 0, nc = 0;
  HIP_OK(hipMemcpy(&e, err, sizeof(e), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&we, werr, sizeof(we), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&c, counter, sizeof(c), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&ac, add_counter, sizeof(ac), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&dc, dcounter, sizeof(dc), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&nc, ncounter, sizeof(nc), hipMemcpyDeviceToHost));
  out_hdr[0] = e;
  out_hdr[1] = we;
  out_hdr[2] = (int64_t)c;
  out_hdr[3] = (int64_t)ac;
  out_hdr[4] = checks;
  out_hdr[5] = kvx_abi_version();
  out_hdr[6] = (int64_t)dc;
  out_hdr[7] = (int64_t)nc;
  FILE* out = fopen(argv[2], "wb");
  if (!out) return 5;
  uint8_t* scratch_h = (uint8_t*)malloc(layer);
  fwrite(out_hdr, sizeof(int64_t), 8, out);
  write_device(out, slots, (size_t)T * sizeof(int64_t));
  write_layers(out, wr_l, 1, layer, scratch_h);
  write_device(out, kbuf, buf_bytes);
  write_layers(out, kvf_l, L, layer, scratch_h);
  write_device(out, shard[0], buf_bytes / 2);
  write_device(out, shard[1], buf_bytes / 2);
  write_layers(out, mrg_l, L, layer, scratch_h);
  write_layers(out, sig_l, L, layer, scratch_h);
  write_layers(out, seen_l, L, layer, scratch_h);
  write_device(out, nbuf, buf_bytes);
  write_layers(out, nsig_l, L, layer, scratch_h);
  fclose(out);
  HIP_OK(hipStreamDestroy(s));
  HIP_OK(hipStreamDestroy(prod));
  HIP_OK(hipStreamDestroy(cons));
  printf("rest: error flag %d, wait flag %d, signals %llu / %llu / %llu, add %llu, %lld of 10 status "
         "checks, ABI %d\n", e, we, (unsigned long long)c, (unsigned long long)dc, (unsigned long long)nc,
         (unsigned long long)ac, (long long)checks, (int)out_hdr[5]);
  return 0;
}
