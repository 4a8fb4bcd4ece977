/* Host-side argument validation of every libkvx entry point, driven from plain C. Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer against a host-only build of the library
 * (no device code, no GPU): every call here must return its status before any HIP call, and
 * the sanitizers check the host code on the way. Pointers are real host memory so that a
 * stray dereference would be caught instead of faulting; the library must not dereference
 * them at all. Exit 0 when every status matches. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvx.h"

static unsigned char arena[1 << 16] __attribute__((aligned(256)));
#define P ((void*)(arena + 4096))
#define AT(o) ((void*)(arena + 4096 + (o)))
#define NUL ((void*)0)

static int calls = 0, failures = 0;

static void expect(const char* what, kvx_status got, kvx_status want) {
  ++calls;
  if (got != want) {
    ++failures;
    printf("MISMATCH %s: got %d (%s), want %d\n", what, (int)got, kvx_status_string(got), (int)want);
  }
}

static kvx_status pack(void* bases, int32_t L, int64_t bb, int64_t nb, void* x, void* cnt, int64_t n,
                       void* buf) {
  return kvx_pack((void* const*)bases, L, bb, nb, (const kvx_xfer*)x, (const int64_t*)cnt, n, buf, NUL, NUL);
}

static kvx_status unpack(const void* const* srcs, int32_t S, int64_t bb, int32_t rows, int64_t n) {
  return kvx_unpack(srcs, S, (void* const*)P, 2, bb, 100, rows, (const kvx_xfer*)P, (const int64_t*)P, n,
                    NUL, NUL);
}

static kvx_status build(void* src, void* dst, void* ro, int32_t R, int64_t n, int32_t mode, void* x,
                        int64_t cap, void* cnt) {
  return kvx_build_xfer_list((const int32_t*)src, (const int32_t*)dst, (const int64_t*)ro, R, n, mode,
                             (kvx_xfer*)x, cap, (int64_t*)cnt, NUL, NUL);
}

static kvx_status slots(int64_t W, int64_t stride, int64_t T, int32_t bs, void* out) {
  return kvx_slot_mapping((const int32_t*)P, 4, W, stride, (const int32_t*)P, (const int64_t*)P, T, bs,
                          (int64_t*)out, NUL, NUL);
}

static kvx_status write_rows(void* k, int64_t T, int64_t row, void* sm, int32_t bs, int64_t kst) {
  return kvx_reshape_and_cache(k, 4096, P, 4096, T, row, (const int64_t*)sm, P, 64, bs, 65536, 4096, kst,
                               NUL, NUL);
}

static kvx_status split(void* const* bufs, int32_t D, int32_t rows, int64_t n) {
  return kvx_pack_split((void* const*)P, 2, 65536, 100, rows, (const kvx_xfer*)P, (const int64_t*)P, n, bufs,
                        D, NUL, NUL);
}

static kvx_status kvf(int pack_side, int64_t seg, int64_t plane, void* ro, int32_t R, int64_t n, void* buf) {
  if (pack_side)
    return kvx_pack_kv_first((void* const*)P, 2, seg, plane, 100, (const int64_t*)ro, R, (const kvx_xfer*)P,
                             (const int64_t*)P, n, buf, NUL, NUL);
  return kvx_unpack_kv_first(buf, (void* const*)P, 2, seg, plane, 100, (const int64_t*)ro, R,
                             (const kvx_xfer*)P, (const int64_t*)P, n, NUL, NUL);
}

static kvx_status direct(void* sb, void* db, int32_t L, int64_t bb, int64_t nbs, int64_t nbd, void* x,
                         int64_t n) {
  return kvx_copy_direct((void* const*)sb, (void* const*)db, L, bb, nbs, nbd, (const kvx_xfer*)x,
                         (const int64_t*)P, n, NUL, NUL);
}

static kvx_status pack_signal(void* counter, void* arrivals, int32_t L, int64_t bb, void* x, int64_t n,
                              void* buf) {
  return kvx_pack_signal((void* const*)P, L, bb, 100, (const kvx_xfer*)x, (const int64_t*)P, n, buf,
                         (uint64_t*)counter, 1, (uint32_t*)arrivals, NUL, NUL);
}

static kvx_status direct_signal(void* counter, void* arrivals, int32_t L, int64_t bb, int64_t nbs, void* sb,
                                void* x, int64_t n) {
  return kvx_copy_direct_signal((void* const*)sb, (void* const*)P, L, bb, nbs, 100, (const kvx_xfer*)x,
                                (const int64_t*)P, n, (uint64_t*)counter, 1, (uint32_t*)arrivals, NUL, NUL);
}

static kvx_status noalloc(int32_t slot, void* counter, int32_t L, int64_t bb, void* x, void* buf) {
  return kvx_pack_signal_noalloc((void* const*)P, L, bb, 100, (const kvx_xfer*)x, (const int64_t*)P, 10, buf,
                                 (uint64_t*)counter, 1, slot, NUL, NUL);
}

int main(void) {
  const int64_t big = (int64_t)1 << 31;
  for (int s = 0; s <= 5; ++s) {
    const char* m = kvx_status_string((kvx_status)s);
    ++calls;
    if (!m || !*m) { ++failures; printf("MISMATCH empty status string %d\n", s); }
  }
  {
    const char* m = kvx_status_string((kvx_status)99);
    ++calls;
    if (!m || !*m) { ++failures; printf("MISMATCH empty string for an unknown status\n"); }
  }
  ++calls;
  if (kvx_abi_version() < 1) { ++failures; printf("MISMATCH abi version %d\n", kvx_abi_version()); }

  /* pack */
  expect("pack L<0", pack(P, -1, 8192, 100, P, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("pack bb=0", pack(P, 2, 0, 100, P, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("pack n<0", pack(P, 2, 8192, 100, P, P, -5, P), KVX_ERR_INVALID_ARGUMENT);
  expect("pack n=2^31", pack(P, 2, 8192, 100, P, P, big, P), KVX_ERR_INVALID_ARGUMENT);
  expect("pack bases null", pack(NUL, 2, 8192, 100, P, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("pack xfers null", pack(P, 2, 8192, 100, NUL, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("pack bb not 16", pack(P, 2, 8200, 100, P, P, 10, P), KVX_ERR_MISALIGNED);
  expect("pack buf misaligned", pack(P, 2, 8192, 100, P, P, 10, AT(8)), KVX_ERR_MISALIGNED);
  expect("pack empty", pack(NUL, 2, 8192, 100, P, P, 0, P), KVX_SUCCESS);
  expect("pack no layers", pack(P, 0, 8192, 100, P, P, 10, P), KVX_SUCCESS);

  /* unpack */
  {
    const void* one[1] = {P};
    const void* nine[9] = {P, P, P, P, P, P, P, P, P};
    const void* two[2] = {P, P};
    const void* two_null[2] = {P, NUL};
    const void* two_mis[2] = {P, AT(16 * 3 + 8)};
    expect("unpack S=0", unpack(one, 0, 8192, 1, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("unpack S=9", unpack(nine, 9, 8192, 1, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("unpack rows=0", unpack(one, 1, 8192, 0, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("unpack rows do not divide", unpack(two, 2, 64, 3, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("unpack null source", unpack(two_null, 2, 8192, 32, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("unpack misaligned source", unpack(two_mis, 2, 8192, 32, 10), KVX_ERR_MISALIGNED);
    expect("unpack bb not 16", unpack(one, 1, 8200, 1, 10), KVX_ERR_MISALIGNED);
    expect("unpack sources null", unpack(NUL, 1, 8192, 1, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("unpack empty", unpack(one, 1, 8192, 1, 0), KVX_SUCCESS);
  }

  /* run lists */
  expect("build mode 3", build(P, P, P, 2, 10, 3, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("build mode -1", build(P, P, P, 2, 10, -1, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("build capacity", build(P, P, P, 2, 10, 0, P, 9, P), KVX_ERR_CAPACITY);
  expect("build R=0", build(P, P, P, 0, 10, 0, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("build pack without src", build(NUL, P, P, 2, 10, 0, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("build unpack without dst", build(P, NUL, P, 2, 10, 1, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("build direct without dst", build(P, NUL, P, 2, 10, 2, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("build count null", build(P, P, P, 2, 10, 0, P, 10, NUL), KVX_ERR_INVALID_ARGUMENT);
  expect("build offsets null", build(P, P, NUL, 2, 10, 0, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
  expect("build records +4", build(P, P, P, 2, 10, 0, AT(4), 10, P), KVX_ERR_MISALIGNED);
  expect("build records +8", build(P, P, P, 2, 10, 0, AT(8), 10, P), KVX_ERR_MISALIGNED);
  expect("build n<0", build(P, P, P, 2, -1, 0, P, 10, P), KVX_ERR_INVALID_ARGUMENT);

  /* slot mapping and new-token write */
  expect("slots bs=0", slots(8, 8, 10, 0, P), KVX_ERR_INVALID_ARGUMENT);
  expect("slots T<0", slots(8, 8, -1, 16, P), KVX_ERR_INVALID_ARGUMENT);
  expect("slots width past stride", slots(9, 8, 10, 16, P), KVX_ERR_INVALID_ARGUMENT);
  expect("slots out null", slots(8, 8, 10, 16, NUL), KVX_ERR_INVALID_ARGUMENT);
  expect("slots empty", slots(8, 8, 0, 16, NUL), KVX_SUCCESS);
  expect("write row=0", write_rows(P, 10, 0, P, 16, 2048), KVX_ERR_INVALID_ARGUMENT);
  expect("write bs=0", write_rows(P, 10, 2048, P, 0, 2048), KVX_ERR_INVALID_ARGUMENT);
  expect("write slots null", write_rows(P, 10, 2048, NUL, 16, 2048), KVX_ERR_INVALID_ARGUMENT);
  expect("write key +2", write_rows(AT(2), 10, 2048, P, 16, 2048), KVX_ERR_MISALIGNED);
  expect("write row not 16", write_rows(P, 10, 2040, P, 16, 2048), KVX_ERR_MISALIGNED);
  expect("write kv stride not 16", write_rows(P, 10, 2048, P, 16, 2056), KVX_ERR_MISALIGNED);
  expect("write empty", write_rows(P, 0, 2048, P, 16, 2048), KVX_SUCCESS);

  /* head split */
  {
    void* two[2] = {P, P};
    void* nine[9] = {P, P, P, P, P, P, P, P, P};
    void* two_null[2] = {P, NUL};
    void* two_mis[2] = {P, AT(8)};
    expect("split D=0", split(two, 0, 32, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("split D=9", split(nine, 9, 32, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("split rows do not divide", split(two, 2, 3, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("split null shard", split(two_null, 2, 32, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("split misaligned shard", split(two_mis, 2, 32, 10), KVX_ERR_MISALIGNED);
    expect("split empty", split(two, 2, 32, 0), KVX_SUCCESS);
  }

  /* kv-first views, both directions */
  for (int side = 0; side < 2; ++side) {
    expect("kv-first segment 512", kvf(side, 512, 409600, P, 2, 10, P), KVX_ERR_MISALIGNED);
    expect("kv-first plane 8", kvf(side, 4096, 8, P, 2, 10, P), KVX_ERR_MISALIGNED);
    expect("kv-first planes overlap", kvf(side, 4096, 4096 * 99, P, 2, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("kv-first segment 0", kvf(side, 0, 409600, P, 2, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("kv-first offsets null", kvf(side, 4096, 409600, NUL, 2, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("kv-first R=0", kvf(side, 4096, 409600, P, 0, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("kv-first buffer +24", kvf(side, 4096, 409600, P, 2, 10, AT(24)), KVX_ERR_MISALIGNED);
    expect("kv-first empty", kvf(side, 4096, 409600, P, 2, 0, P), KVX_SUCCESS);
  }

  /* direct copy */
  expect("direct L<0", direct(P, P, -1, 8192, 100, 100, P, 10), KVX_ERR_INVALID_ARGUMENT);
  expect("direct bb=0", direct(P, P, 2, 0, 100, 100, P, 10), KVX_ERR_INVALID_ARGUMENT);
  expect("direct dst blocks<0", direct(P, P, 2, 8192, 100, -1, P, 10), KVX_ERR_INVALID_ARGUMENT);
  expect("direct n=2^31", direct(P, P, 2, 8192, 100, 100, P, big), KVX_ERR_INVALID_ARGUMENT);
  expect("direct src null", direct(NUL, P, 2, 8192, 100, 100, P, 10), KVX_ERR_INVALID_ARGUMENT);
  expect("direct dst null", direct(P, NUL, 2, 8192, 100, 100, P, 10), KVX_ERR_INVALID_ARGUMENT);
  expect("direct xfers null", direct(P, P, 2, 8192, 100, 100, NUL, 10), KVX_ERR_INVALID_ARGUMENT);
  expect("direct empty source cache", direct(P, P, 2, 8192, 0, 100, P, 10), KVX_ERR_INVALID_ARGUMENT);
  expect("direct bb not 16", direct(P, P, 2, 8200, 100, 100, P, 10), KVX_ERR_MISALIGNED);
  expect("direct empty", direct(NUL, P, 2, 8192, 100, 100, P, 0), KVX_SUCCESS);

  /* completion signal */
  expect("signal add null", kvx_signal_add(NUL, 1, NUL), KVX_ERR_INVALID_ARGUMENT);
  expect("signal add +4", kvx_signal_add((uint64_t*)AT(4), 1, NUL), KVX_ERR_MISALIGNED);
  expect("signal wait null", kvx_signal_wait(NUL, 1, 1000, NUL, NUL), KVX_ERR_INVALID_ARGUMENT);
  expect("signal wait timeout 0", kvx_signal_wait((const uint64_t*)P, 1, 0, NUL, NUL), KVX_ERR_INVALID_ARGUMENT);
  expect("signal wait timeout<0", kvx_signal_wait((const uint64_t*)P, 1, -3, NUL, NUL), KVX_ERR_INVALID_ARGUMENT);
  expect("signal wait timeout past limit", kvx_signal_wait((const uint64_t*)P, 1, 60000001, NUL, NUL),
         KVX_ERR_INVALID_ARGUMENT);
  expect("signal wait +12", kvx_signal_wait((const uint64_t*)AT(12), 1, 1000, NUL, NUL), KVX_ERR_MISALIGNED);

  /* signalling copies */
  {
    void* cnt = AT(1024);
    void* arr = AT(2048);
    expect("pack_signal counter null", pack_signal(NUL, arr, 2, 8192, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("pack_signal arrivals null", pack_signal(cnt, NUL, 2, 8192, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("pack_signal counter +4", pack_signal(AT(1028), arr, 2, 8192, P, 10, P), KVX_ERR_MISALIGNED);
    expect("pack_signal arrivals +64", pack_signal(cnt, AT(2048 + 64), 2, 8192, P, 10, P), KVX_ERR_MISALIGNED);
    expect("pack_signal L<0", pack_signal(cnt, arr, -1, 8192, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("pack_signal bb=0", pack_signal(cnt, arr, 2, 0, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("pack_signal n=2^31", pack_signal(cnt, arr, 2, 8192, P, big, P), KVX_ERR_INVALID_ARGUMENT);
    expect("pack_signal xfers null", pack_signal(cnt, arr, 2, 8192, NUL, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("pack_signal bb not 16", pack_signal(cnt, arr, 2, 8200, P, 10, P), KVX_ERR_MISALIGNED);
    expect("pack_signal buf null", pack_signal(cnt, arr, 2, 8192, P, 10, NUL), KVX_ERR_INVALID_ARGUMENT);
    expect("pack_signal buf +8", pack_signal(cnt, arr, 2, 8192, P, 10, AT(8)), KVX_ERR_MISALIGNED);
    expect("direct_signal counter null", direct_signal(NUL, arr, 2, 8192, 100, P, P, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("direct_signal arrivals null", direct_signal(cnt, NUL, 2, 8192, 100, P, P, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("direct_signal counter +4", direct_signal(AT(1028), arr, 2, 8192, 100, P, P, 10), KVX_ERR_MISALIGNED);
    expect("direct_signal arrivals +64", direct_signal(cnt, AT(2048 + 64), 2, 8192, 100, P, P, 10),
           KVX_ERR_MISALIGNED);
    expect("direct_signal L<0", direct_signal(cnt, arr, -1, 8192, 100, P, P, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("direct_signal xfers null", direct_signal(cnt, arr, 2, 8192, 100, P, NUL, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("direct_signal src null", direct_signal(cnt, arr, 2, 8192, 100, NUL, P, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("direct_signal empty source cache", direct_signal(cnt, arr, 2, 8192, 0, P, P, 10),
           KVX_ERR_INVALID_ARGUMENT);
    expect("direct_signal bb not 16", direct_signal(cnt, arr, 2, 8200, 100, P, P, 10), KVX_ERR_MISALIGNED);
  }

  /* allocation-free signalling pack: the slot is checked first */
  {
    void* cnt = AT(1024);
    expect("noalloc slot -1", noalloc(-1, cnt, 2, 8192, P, P), KVX_ERR_CAPACITY);
    expect("noalloc slot past the array", noalloc(KVX_NOALLOC_SLOTS, cnt, 2, 8192, P, P), KVX_ERR_CAPACITY);
    expect("noalloc slot past the array, counter null", noalloc(KVX_NOALLOC_SLOTS, NUL, 2, 8192, P, P),
           KVX_ERR_CAPACITY);
    expect("noalloc counter null", noalloc(0, NUL, 2, 8192, P, P), KVX_ERR_INVALID_ARGUMENT);
    expect("noalloc counter +4", noalloc(0, AT(1028), 2, 8192, P, P), KVX_ERR_MISALIGNED);
    expect("noalloc L<0", noalloc(0, cnt, -1, 8192, P, P), KVX_ERR_INVALID_ARGUMENT);
    expect("noalloc xfers null", noalloc(0, cnt, 2, 8192, NUL, P), KVX_ERR_INVALID_ARGUMENT);
    expect("noalloc bb not 16", noalloc(0, cnt, 2, 8200, P, P), KVX_ERR_MISALIGNED);
    expect("noalloc buf +8", noalloc(0, cnt, 2, 8192, P, AT(8)), KVX_ERR_MISALIGNED);
  }

  /* byte extents past KVX_MAX_EXTENT_BYTES, including products that overflow 64 bits; an extent
   * exactly at the limit passes that check and meets the next one */
  {
    const int64_t M = KVX_MAX_EXTENT_BYTES, bb = (int64_t)1 << 17, lim = M / bb;
    const void* two[2] = {P, P};
    void* twob[2] = {P, P};
    expect("pack cache extent past the limit", pack(P, 2, bb, lim + 1, P, P, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("pack cache extent overflowing", pack(P, 2, 1024, (int64_t)1 << 62, P, P, 10, P),
           KVX_ERR_INVALID_ARGUMENT);
    expect("pack buffer extent past the limit", pack(P, 2, (int64_t)1 << 26, 100, P, P, (int64_t)1 << 30, P),
           KVX_ERR_INVALID_ARGUMENT);
    expect("pack cache extent at the limit", pack(P, 2, bb, lim, P, P, 10, AT(8)), KVX_ERR_MISALIGNED);
    expect("unpack buffer extent past the limit",
           kvx_unpack(two, 2, (void* const*)P, 2, (int64_t)1 << 26, 100, 32, (const kvx_xfer*)P,
                      (const int64_t*)P, (int64_t)1 << 30, NUL, NUL),
           KVX_ERR_INVALID_ARGUMENT);
    expect("direct destination extent past the limit", direct(P, P, 2, bb, 100, lim + 1, P, 10),
           KVX_ERR_INVALID_ARGUMENT);
    expect("direct_signal source extent past the limit",
           direct_signal(AT(1024), AT(2048), 2, bb, lim + 1, P, P, 10), KVX_ERR_INVALID_ARGUMENT);
    expect("split cache extent past the limit",
           kvx_pack_split((void* const*)P, 2, bb, lim + 1, 32, (const kvx_xfer*)P, (const int64_t*)P, 10, twob, 2,
                          NUL, NUL),
           KVX_ERR_INVALID_ARGUMENT);
    expect("pack_signal cache extent overflowing",
           kvx_pack_signal((void* const*)P, 2, 1024, (int64_t)1 << 62, (const kvx_xfer*)P, (const int64_t*)P, 10, P,
                           (uint64_t*)AT(1024), 1, (uint32_t*)AT(2048), NUL, NUL),
           KVX_ERR_INVALID_ARGUMENT);
    expect("noalloc cache extent overflowing",
           kvx_pack_signal_noalloc((void* const*)P, 2, 1024, (int64_t)1 << 62, (const kvx_xfer*)P, (const int64_t*)P,
                                   10, P, (uint64_t*)AT(1024), 1, 0, NUL, NUL),
           KVX_ERR_INVALID_ARGUMENT);
    expect("kv-first plane past the limit", kvf(1, 4096, M, P, 2, 10, P), KVX_ERR_INVALID_ARGUMENT);
    expect("kv-first buffer extent past the limit",
           kvf(0, (int64_t)1 << 25, ((int64_t)1 << 25) * 100, P, 2, (int64_t)1 << 30, P), KVX_ERR_INVALID_ARGUMENT);
    expect("slot mapping table extent past the limit", slots(8, (int64_t)1 << 55, 10, 16, P),
           KVX_ERR_INVALID_ARGUMENT);
    expect("write cache extent overflowing",
           kvx_reshape_and_cache(P, 4096, P, 4096, 10, 2048, (const int64_t*)P, P, (int64_t)1 << 60, 16,
                                 (int64_t)1 << 20, 4096, 2048, NUL, NUL),
           KVX_ERR_INVALID_ARGUMENT);
    expect("write row extent overflowing", write_rows(P, (int64_t)1 << 50, 2048, P, 16, 2048),
           KVX_ERR_INVALID_ARGUMENT);
  }

  printf("validated %d calls, %d mismatches\n", calls, failures);
  return failures ? 1 : 0;
}
