// Device-side completion signalling between streams: a monotone 64-bit counter that a
// producer stream adds to once its earlier work has finished, and a wait that holds a
// consumer stream until the counter reaches an expected value.
//
// Page "5. flagcx connector design & dev & test", §1.2 (send path and
// wait_for_layer_load): the sender adds to the receiver's signal counter with the last
// transfer of a batch, the receiver learns the count to expect, and its stream polls the
// counter on the GPU until it is at least that count before the forward goes on. Because
// the counter only grows, waiting for the largest expected value covers all smaller ones.
//
// Both calls launch one wavefront. Ordering comes from the kernel boundaries around them:
// a kernel starts only after the kernels before it in its stream have finished and their
// writes have been released to the whole device, and it starts with an acquire of its own.
// So the add needs no release of its own (it runs after the producer's kernels are done and
// visible) and the wait needs no acquire (the consumer's next kernel acquires when it
// starts). Both touch the counter with relaxed atomics at system scope, which reach the
// coherent copy without flushing or invalidating the caches: a release or acquire here
// would write back or drop the whole L2 of the XCD, on every poll, under whatever else is
// running. The wait sleeps between polls and is bounded by wall-clock time, so a signal
// that never arrives ends in an error bit instead of a stream that never drains.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvx.h"
#include "kvx_launch.h"

namespace kvx {

__global__ __launch_bounds__(64) void signal_add_kernel(uint64_t* counter, uint64_t delta) {
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(counter, delta, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__global__ __launch_bounds__(64) void signal_wait_kernel(const uint64_t* counter, uint64_t value,
                                                         uint64_t max_ticks, int32_t* err) {
  if (threadIdx.x != 0) return;
  uint64_t* c = const_cast<uint64_t*>(counter);
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) < value) {
    if (wall_clock64() - t0 > max_ticks) {
      if (err) __hip_atomic_fetch_or(err, KVX_DEVERR_TIMEOUT, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(32);  // about 2k cycles between polls
  }
}

hipError_t launch_signal_add(uint64_t* counter, uint64_t delta, hipStream_t stream) {
  signal_add_kernel<<<1, 64, 0, stream>>>(counter, delta);
  return hipGetLastError();
}

}  // namespace kvx

namespace {

constexpr int64_t kMaxTimeoutUs = 60ll * 1000 * 1000;

inline bool aligned8(const void* p) { return ((uintptr_t)p & 7u) == 0; }

}  // namespace

extern "C" {

kvx_status kvx_signal_add(uint64_t* counter, uint64_t delta, hipStream_t stream) {
  if (!counter) return KVX_ERR_INVALID_ARGUMENT;
  if (!aligned8(counter)) return KVX_ERR_MISALIGNED;
  return kvx::launch_signal_add(counter, delta, stream) == hipSuccess ? KVX_SUCCESS : KVX_ERR_HIP;
}

kvx_status kvx_signal_wait(const uint64_t* counter, uint64_t value, int64_t timeout_us,
                           int32_t* err_flag, hipStream_t stream) {
  if (!counter || timeout_us < 1 || timeout_us > kMaxTimeoutUs) return KVX_ERR_INVALID_ARGUMENT;
  if (!aligned8(counter)) return KVX_ERR_MISALIGNED;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    return KVX_ERR_HIP;
  const uint64_t max_ticks = (uint64_t)timeout_us * (uint64_t)khz / 1000u;
  kvx::signal_wait_kernel<<<1, 64, 0, stream>>>(counter, value, max_ticks, err_flag);
  return hipGetLastError() == hipSuccess ? KVX_SUCCESS : KVX_ERR_HIP;
}

}  // extern "C"
