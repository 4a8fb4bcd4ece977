/* A plain C consumer of libkvx (no Python, no PyTorch): reads one transfer's inputs from a
 * file, runs the run lists, pack, unpack and the direct copy through the C ABI on a HIP
 * stream, and writes every output back to a file for the test to compare with the oracle.
 * It also checks a few host-side status codes.
 *
 *   roundtrip IN OUT
 *   IN:  int64 {magic, L, nb, BB, R, N}, int64 req_offsets[R+1], int32 src_ids[N],
 *        int32 dst_ids[N], uint8 src caches [L][nb][BB], uint8 dst caches [L][nb][BB]
 *   OUT: int64 {pack runs, unpack runs, direct runs, error flag, status checks passed},
 *        uint8 buffer [L][N][BB], dst caches after unpack, dst caches after the direct copy
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvx.h"

#define MAGIC 0x4B5658LL

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

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: roundtrip IN OUT\n");
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 4;
  int64_t* hdr = (int64_t*)read_exact(in, 6 * sizeof(int64_t));
  if (hdr[0] != MAGIC) return 4;
  const int64_t L = hdr[1], nb = hdr[2], BB = hdr[3], R = hdr[4], N = hdr[5];
  int64_t* ro = (int64_t*)read_exact(in, (size_t)(R + 1) * sizeof(int64_t));
  int32_t* sid = (int32_t*)read_exact(in, (size_t)N * sizeof(int32_t));
  int32_t* did = (int32_t*)read_exact(in, (size_t)N * sizeof(int32_t));
  const size_t layer = (size_t)(nb * BB);
  uint8_t* src_h = (uint8_t*)read_exact(in, (size_t)L * layer);
  uint8_t* dst_h = (uint8_t*)read_exact(in, (size_t)L * layer);
  fclose(in);

  /* device copies: one allocation per layer cache, as a serving framework holds them */
  void** src_l = (void**)malloc(L * sizeof(void*));
  void** dst_l = (void**)malloc(L * sizeof(void*));
  void** dst2_l = (void**)malloc(L * sizeof(void*));
  for (int64_t l = 0; l < L; ++l) {
    src_l[l] = device_copy(src_h + l * layer, layer);
    dst_l[l] = device_copy(dst_h + l * layer, layer);
    dst2_l[l] = device_copy(dst_h + l * layer, layer);
  }
  void* src_bases = device_copy(src_l, L * sizeof(void*));
  void* dst_bases = device_copy(dst_l, L * sizeof(void*));
  void* dst2_bases = device_copy(dst2_l, L * sizeof(void*));
  int64_t* ro_d = (int64_t*)device_copy(ro, (size_t)(R + 1) * sizeof(int64_t));
  int32_t* sid_d = (int32_t*)device_copy(sid, (size_t)N * sizeof(int32_t));
  int32_t* did_d = (int32_t*)device_copy(did, (size_t)N * sizeof(int32_t));
  const int64_t cap = N > 0 ? N : 1;
  kvx_xfer *xp, *xu, *xd;
  int64_t* counts;
  int32_t* err;
  void* buf;
  HIP_OK(hipMalloc((void**)&xp, cap * sizeof(kvx_xfer)));
  HIP_OK(hipMalloc((void**)&xu, cap * sizeof(kvx_xfer)));
  HIP_OK(hipMalloc((void**)&xd, cap * sizeof(kvx_xfer)));
  HIP_OK(hipMalloc((void**)&counts, 3 * sizeof(int64_t)));
  HIP_OK(hipMalloc((void**)&err, sizeof(int32_t)));
  const size_t buf_bytes = (size_t)(L * N * BB);
  HIP_OK(hipMalloc(&buf, buf_bytes > 0 ? buf_bytes : 16));
  HIP_OK(hipMemset(err, 0, sizeof(int32_t)));
  HIP_OK(hipMemset(buf, 0, buf_bytes > 0 ? buf_bytes : 16));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  /* host-side status codes: nothing is enqueued for these */
  int64_t checks = 0;
  checks += kvx_pack(src_bases, (int32_t)L, 8, nb, xp, counts, N, buf, err, stream) == KVX_ERR_MISALIGNED;
  checks += kvx_build_xfer_list(sid_d, NULL, ro_d, (int32_t)R, N, KVX_MODE_PACK, xp, N - 1, counts,
                                err, stream) == (N > 0 ? KVX_ERR_CAPACITY : KVX_ERR_INVALID_ARGUMENT);
  checks += kvx_unpack(NULL, 1, dst_bases, (int32_t)L, BB, nb, 1, xu, counts + 1, N, err, stream) ==
            (N > 0 ? KVX_ERR_INVALID_ARGUMENT : KVX_SUCCESS);
  checks += kvx_build_xfer_list(sid_d, did_d, ro_d, (int32_t)R, N, 7, xd, cap, counts, err, stream) ==
            KVX_ERR_INVALID_ARGUMENT;

  KVX_OK(kvx_build_xfer_list(sid_d, NULL, ro_d, (int32_t)R, N, KVX_MODE_PACK, xp, cap, counts, err, stream));
  KVX_OK(kvx_build_xfer_list(NULL, did_d, ro_d, (int32_t)R, N, KVX_MODE_UNPACK, xu, cap, counts + 1, err, stream));
  KVX_OK(kvx_build_xfer_list(sid_d, did_d, ro_d, (int32_t)R, N, KVX_MODE_DIRECT, xd, cap, counts + 2, err, stream));
  KVX_OK(kvx_pack(src_bases, (int32_t)L, BB, nb, xp, counts, N, buf, err, stream));
  const void* srcs[1] = {buf};
  KVX_OK(kvx_unpack(srcs, 1, dst_bases, (int32_t)L, BB, nb, 1, xu, counts + 1, N, err, stream));
  KVX_OK(kvx_copy_direct(src_bases, dst2_bases, (int32_t)L, BB, nb, nb, xd, counts + 2, N, err, stream));
  HIP_OK(hipStreamSynchronize(stream));

  int64_t out_hdr[5];
  HIP_OK(hipMemcpy(out_hdr, counts, 3 * sizeof(int64_t), hipMemcpyDeviceToHost));
  int32_t e = 0;
  HIP_OK(hipMemcpy(&e, err, sizeof(int32_t), hipMemcpyDeviceToHost));
  out_hdr[3] = e;
  out_hdr[4] = checks;
  uint8_t* out_buf = (uint8_t*)malloc(buf_bytes + 1);
  if (buf_bytes > 0) HIP_OK(hipMemcpy(out_buf, buf, buf_bytes, hipMemcpyDeviceToHost));
  FILE* out = fopen(argv[2], "wb");
  if (!out) return 5;
  fwrite(out_hdr, sizeof(int64_t), 5, out);
  fwrite(out_buf, 1, buf_bytes, out);
  for (int pass = 0; pass < 2; ++pass) {
    for (int64_t l = 0; l < L; ++l) {
      HIP_OK(hipMemcpy(dst_h + l * layer, pass == 0 ? dst_l[l] : dst2_l[l], layer, hipMemcpyDeviceToHost));
      fwrite(dst_h + l * layer, 1, layer, out);
    }
  }
  fclose(out);
  HIP_OK(hipStreamDestroy(stream));
  printf("roundtrip: %lld/%lld/%lld runs, error flag %d, %lld of 4 status checks\n", (long long)out_hdr[0],
         (long long)out_hdr[1], (long long)out_hdr[2], e, (long long)checks);
  return 0;
}
