// gfx950 (CDNA4) kernels for the paged KV-cache transfer path.
//
// Everything here is pure data movement: no floating-point arithmetic, no MFMA. Bytes move
// as 16-byte vectors through VGPRs (global_load_dwordx4 / global_store_dwordx4); a
// wavefront's 64 lanes cover 1 KiB of consecutive bytes per instruction, so every access is
// fully coalesced, and each lane keeps several loads in flight before it stores.
//
// Sources: slot rule of the batch-tensor label and the 16-slot block of the "Paged kv cache"
// label ("vllm v1 调度逻辑 和 distributed 分布式原理"); transfer-list flattening of
// "5. flagcx connector design & dev & test" §1.2 (_send_blocks); per-layer base + block
// length x id addressing of "vLLM PD 分离" §七 item 3; TP heterogeneity of §四 4.2.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "kvx.h"
#include "kvx_launch.h"

namespace kvx {

// --------------------------------------------------------------------------------------
// tuning knobs
// --------------------------------------------------------------------------------------

static int64_t env_i64(const char* name, int64_t dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  char* end = nullptr;
  long long v = strtoll(s, &end, 0);
  return (end && *end == '\0') ? (int64_t)v : dflt;
}

const Tuning& tuning() {
  static const Tuning t = {
      {env_i64("KVX_WAVE_BYTES_PACK", 8 * 1024), (int)env_i64("KVX_NT_PACK", 3),
       (int)env_i64("KVX_BATCH_PACK", 4)},
      {env_i64("KVX_WAVE_BYTES_UNPACK", 8 * 1024), (int)env_i64("KVX_NT_UNPACK", 3),
       (int)env_i64("KVX_BATCH_UNPACK", 8)},
      {env_i64("KVX_WAVE_BYTES_MERGE", 64 * 1024), (int)env_i64("KVX_NT_MERGE", 3),
       (int)env_i64("KVX_BATCH_MERGE", 8)},
      {env_i64("KVX_WAVE_BYTES_SPLIT", 64 * 1024), (int)env_i64("KVX_NT_SPLIT", 3),
       (int)env_i64("KVX_BATCH_SPLIT", 8)},
      {0, (int)env_i64("KVX_NT_KVF_PACK", 3), (int)env_i64("KVX_BATCH_KVF_PACK", 8)},
      {0, (int)env_i64("KVX_NT_KVF_UNPACK", 3), (int)env_i64("KVX_BATCH_KVF_UNPACK", 8)},
      {env_i64("KVX_WAVE_BYTES_DIRECT", 8 * 1024), (int)env_i64("KVX_NT_DIRECT", 3),
       (int)env_i64("KVX_BATCH_DIRECT", 8)},
      (int)env_i64("KVX_XCD_REMAP", 1),
      (int)env_i64("KVX_XCD_REMAP_SPLIT", 0),
      (int)env_i64("KVX_ONE_BATCH", 1),
      (int)env_i64("KVX_NT_WRITE", 0),
      env_i64("KVX_WRITE_VEC_MIN", 4096),
  };
  return t;
}

// --------------------------------------------------------------------------------------
// device helpers
// --------------------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int64_t i64x2 __attribute__((ext_vector_type(2)));
#define KVX_GLOBAL __attribute__((address_space(1)))
// Read-only view of memory no kernel writes while it runs (run list, layer bases, counts):
// uniform loads through it become scalar loads, which wait on lgkmcnt and so never stall
// behind the vector loads of the data being copied.
#define KVX_CONST __attribute__((address_space(4)))

template <class T>
__device__ __forceinline__ const KVX_CONST T* readonly(const T* p) {
  return (const KVX_CONST T*)p;
}

// One run, read field by field through the read-only view.
struct Run {
  int64_t src, dst, buf, n;
};
__device__ __forceinline__ Run load_run(const KVX_CONST kvx_xfer* xf, int64_t k) {
  Run r;
  r.src = xf[k].src_block;
  r.dst = xf[k].dst_block;
  r.buf = xf[k].buf_block;
  r.n = xf[k].num_blocks;
  return r;
}

constexpr int kWave = 64;
constexpr int kVec = 16;                 // bytes per lane access
constexpr int kWaveBytes = kWave * kVec; // bytes per wavefront instruction
constexpr int kNumXcd = 8;               // MI355X: 8 XCDs, workgroups dealt round-robin

#ifndef KVX_COPY_THREADS
#define KVX_COPY_THREADS 256
#endif
constexpr int kCopyThreads = KVX_COPY_THREADS;
constexpr int kCopyWavesPerWg = kCopyThreads / kWave;
#ifndef KVX_COPY_BATCH
#define KVX_COPY_BATCH 8
#endif
// 1 KiB wavefront loads a lane issues before its stores (8 -> 8 KiB in flight per wavefront)
constexpr int kCopyBatch = KVX_COPY_BATCH;
#ifndef KVX_WRITE_SLOTS
#define KVX_WRITE_SLOTS 4
#endif
// 1 KiB slots per wavefront in the new-token write. 4 against 8: as fast or faster at every
// row size and token count tried (a shorter chain per wavefront, twice the wavefronts); 2 was
// within a few percent of 4 either way, 16 slower.
constexpr int kWriteSlots = KVX_WRITE_SLOTS;

template <bool NT>
__device__ __forceinline__ u32x4 load16(const char* p) {
  const KVX_GLOBAL u32x4* g = (const KVX_GLOBAL u32x4*)p;
  if constexpr (NT) return __builtin_nontemporal_load(g);
  else return *g;
}

template <bool NT>
__device__ __forceinline__ void store16(char* p, u32x4 v) {
  KVX_GLOBAL u32x4* g = (KVX_GLOBAL u32x4*)p;
  if constexpr (NT) __builtin_nontemporal_store(v, g);
  else *g = v;
}

// Cache-policy bits of buffer instructions on gfx950: sc1 makes a store device-coherent
// (written through to the device's coherence point rather than held dirty in one XCD's L2),
// nt marks it non-temporal. Word 3 of a raw buffer resource.
constexpr int kCpolNt = 2, kCpolSc1 = 16;
constexpr int kRsrcWord3 = 0x00020000;

// A wavefront's 16-byte store at base + lane_off, base uniform across the wavefront. With
// DEVICE the store is device-coherent: once it is acknowledged (vmcnt) every XCD can read it,
// with no L2 write-back. Otherwise a plain global store with the NT policy.
template <bool NT, bool DEVICE>
__device__ __forceinline__ void store16_at(char* base, int64_t lane_off, u32x4 v) {
  if constexpr (DEVICE) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, kWaveBytes, kRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)lane_off, 0, NT ? (kCpolSc1 | kCpolNt) : kCpolSc1);
  } else {
    store16<NT>(base + lane_off, v);
  }
}

__device__ __forceinline__ int64_t uniform(int64_t v) {
  const int32_t lo = __builtin_amdgcn_readfirstlane((int32_t)(v & 0xffffffff));
  const int32_t hi = __builtin_amdgcn_readfirstlane((int32_t)(v >> 32));
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ void raise_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// Workgroup b runs on XCD b % 8. Renumber so that XCD x owns one contiguous slice of the
// workgroup index space: each XCD's L2 and address-translation caches then see 1/8 of the
// layers instead of all of them.
__device__ __forceinline__ int64_t xcd_slice_order(int64_t b, int64_t n) {
  const int64_t xcd = b % kNumXcd, idx = b / kNumXcd;
  const int64_t per = n / kNumXcd, rem = n % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// One wavefront copies nbytes (a multiple of 16) from src to dst. Batch j of K covers
// bytes [base + j KiB, base + (j+1) KiB): each instruction is one coalesced 1 KiB access,
// and a lane issues all K loads of a batch before its K stores.
template <int K, bool NTL, bool NTS, bool DEVICE = false>
__device__ __forceinline__ void wave_copy(const char* __restrict__ src, char* __restrict__ dst,
                                          int64_t nbytes, int lane) {
  constexpr int64_t kBatch = (int64_t)K * kWaveBytes;
  const int64_t lo = (int64_t)lane * kVec;
  int64_t base = 0;
  for (; base + kBatch <= nbytes; base += kBatch) {
    u32x4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = load16<NTL>(src + base + j * kWaveBytes + lo);
#pragma unroll
    for (int j = 0; j < K; ++j) store16_at<NTS, DEVICE>(dst + base + j * kWaveBytes, lo, v[j]);
  }
  if (base < nbytes) {
    u32x4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t o = base + j * kWaveBytes + lo;
      if (o < nbytes) v[j] = load16<NTL>(src + o);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t o = base + j * kWaveBytes + lo;
      if (o < nbytes) store16_at<NTS, DEVICE>(dst + base + j * kWaveBytes, lo, v[j]);
    }
  }
}

// Index of the last run whose buf_block <= p (runs sorted by buf_block), or -1. A 64-way
// search: every lane probes one pivot, a ballot picks the bracket; <= 3 rounds for 2^18 runs.
__device__ __forceinline__ int64_t find_run(const kvx_xfer* __restrict__ xfers, int64_t count,
                                            int64_t p, int lane) {
  int64_t lo = 0, hi = count;  // answer in [lo - 1, hi)
  while (hi - lo > 1) {
    const int64_t step = (hi - lo + kWave - 1) / kWave;
    const int64_t idx = lo + (int64_t)lane * step;
    const bool pred = idx < hi && xfers[idx].buf_block <= p;
    const uint64_t m = __ballot(pred);
    if (m == 0) return lo - 1;
    const int64_t j = 63 - __builtin_clzll(m);
    lo = lo + j * step;
    hi = (lo + step < hi) ? lo + step : hi;
  }
  if (hi - lo == 1 && xfers[lo].buf_block > p) return lo - 1;
  return lo;
}

// --------------------------------------------------------------------------------------
// a1 — slot mapping: one thread per token
// --------------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    const int32_t* __restrict__ block_table, int64_t num_reqs, int64_t max_cols,
    int64_t row_stride, const int32_t* __restrict__ req_idx,
    const int64_t* __restrict__ positions, int64_t num_tokens, int32_t block_size,
    int64_t* __restrict__ slots, int32_t* err) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < num_tokens; i += stride) {
    const int64_t r = req_idx[i];
    const int64_t pos = positions[i];
    int64_t slot = -1;
    if (r >= 0 && r < num_reqs && pos >= 0) {
      int64_t col, off;
      if (pos <= 0x7fffffff) {  // 32-bit division for every realistic position
        col = (uint32_t)pos / (uint32_t)block_size;
        off = (uint32_t)pos - (uint32_t)col * (uint32_t)block_size;
      } else {
        col = pos / block_size;
        off = pos - col * block_size;
      }
      if (col < max_cols) {
        const int32_t b = block_table[r * row_stride + col];
        if (b >= 0) slot = (int64_t)b * block_size + off;
      }
    }
    slots[i] = slot;
    if (slot < 0) raise_error(err, KVX_DEVERR_TABLE_RANGE);
  }
}

// --------------------------------------------------------------------------------------
// a2 — new-token K/V write: K row and V row of each token into its slot
// --------------------------------------------------------------------------------------

// New-token write, one wavefront per token (K row and V row in one pass): the shortest
// dependency chain per token, for launches too small to fill the chip. Rows need only be a
// multiple of 16 bytes.
template <int K>
__global__ __launch_bounds__(256) void write_tokens_kernel(
    const char* __restrict__ key, int64_t key_stride, const char* __restrict__ value,
    int64_t value_stride, int64_t num_tokens, int64_t row_bytes,
    const int64_t* __restrict__ slots, char* __restrict__ cache, int64_t num_blocks,
    int32_t block_size, int64_t block_stride, int64_t token_stride, int64_t kv_stride,
    int32_t* err) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves_per_wg = blockDim.x / kWave;
  const int64_t wave = uniform((int64_t)blockIdx.x * waves_per_wg + (threadIdx.x / kWave));
  const int64_t num_waves = (int64_t)gridDim.x * waves_per_wg;
  const int64_t nvec = row_bytes / kVec;  // vectors in one row
  const int64_t nv2 = 2 * nvec;           // vector q < nvec is in the K row, else in the V row
  const KVX_CONST int64_t* sl = readonly(slots);
  for (int64_t t = wave; t < num_tokens; t += num_waves) {
    const char* krow = key + t * key_stride;
    const char* vrow = value + t * value_stride;
    // The rows do not depend on the slot: their first batch is in flight before the slot
    // arrives. Lanes past the rows re-read vector 0 so every load is unconditional.
    u32x4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      int64_t q = (int64_t)j * kWave + lane;
      q = q < nv2 ? q : 0;
      v[j] = load16<false>(q < nvec ? krow + q * kVec : vrow + (q - nvec) * kVec);
    }
    const int64_t s = sl[t];
    if (s < 0) continue;  // padding token
    int64_t blk, off;
    if (s <= 0x7fffffff) {
      blk = (uint32_t)s / (uint32_t)block_size;
      off = (uint32_t)s - (uint32_t)blk * (uint32_t)block_size;
    } else {
      blk = s / block_size;
      off = s - blk * block_size;
    }
    if (blk >= num_blocks) {
      if (lane == 0) raise_error(err, KVX_DEVERR_SLOT_RANGE);
      continue;
    }
    char* kdst = cache + blk * block_stride + off * token_stride;
    char* vdst = kdst + kv_stride;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int64_t q = (int64_t)j * kWave + lane;
      if (q < nv2) store16<false>(q < nvec ? kdst + q * kVec : vdst + (q - nvec) * kVec, v[j]);
    }
    // rows longer than one batch (over K*64 vectors for K and V together)
    for (int64_t q0 = (int64_t)K * kWave; q0 < nv2; q0 += (int64_t)K * kWave) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        int64_t q = q0 + j * kWave + lane;
        q = q < nv2 ? q : 0;
        v[j] = load16<false>(q < nvec ? krow + q * kVec : vrow + (q - nvec) * kVec);
      }
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int64_t q = q0 + j * kWave + lane;
        if (q < nv2) store16<false>(q < nvec ? kdst + q * kVec : vdst + (q - nvec) * kVec, v[j]);
      }
    }
  }
}

struct WriteArgs {
  const char* key;
  const char* value;
  const int64_t* slots;
  char* cache;
  int32_t* err;
  int64_t key_stride, value_stride;
  int64_t num_tokens, row_bytes, num_blocks;
  int64_t block_stride, token_stride, kv_stride;
  int64_t total_slots;      // whole-KiB kernel: num_tokens * 2 * row KiB
  int32_t block_size;
  int32_t block_shift;      // vector kernel: log2(block_size) if a power of two, else -1
  int32_t tokens_per_wave;  // vector kernel: whole tokens per wavefront
};

// New-token write when a row is a multiple of 1 KiB. The (token, K/V, KiB of row) sequence
// is cut into 1 KiB slots and wavefront w owns slots [4w, 4w + 4): a 2 KiB row puts one
// token's K and V in one wavefront, an 8 KiB row spreads a token over four. The row loads do not
// depend on the slot mapping, so all of them are in flight before the (scalar) slot loads;
// then each slot's destination is formed and the stores go out, one batch per wavefront.
template <bool NTL, bool NTS>
__global__ __launch_bounds__(256) void write_slots_kernel(WriteArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = uniform((int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave));
  const int64_t s0 = w * kWriteSlots;
  if (s0 >= a.total_slots) return;
  const int64_t row_kib = a.row_bytes / kWaveBytes;
  const int64_t per_tok = 2 * row_kib;
  int64_t t = s0 / per_tok;
  const int64_t within = s0 - t * per_tok;
  int64_t kv = within / row_kib;
  int64_t piece = within - kv * row_kib;
  const KVX_CONST int64_t* sl = readonly(a.slots);

  const char* sp[kWriteSlots];
  int64_t tok[kWriteSlots], dof[kWriteSlots];
  bool live[kWriteSlots];
#pragma unroll
  for (int j = 0; j < kWriteSlots; ++j) {
    live[j] = s0 + j < a.total_slots;
    tok[j] = t;
    dof[j] = kv * a.kv_stride + piece * kWaveBytes;  // offset inside the token's slot
    sp[j] = live[j] ? (kv ? a.value + t * a.value_stride : a.key + t * a.key_stride) + piece * kWaveBytes
                    : a.key;  // idle slots re-read the first KiB of row 0
    if (++piece == row_kib) {
      piece = 0;
      if (++kv == 2) { kv = 0; ++t; }
    }
  }
  u32x4 v[kWriteSlots];
#pragma unroll
  for (int j = 0; j < kWriteSlots; ++j) v[j] = load16<NTL>(sp[j] + lane * kVec);

  char* dp[kWriteSlots];
  bool on[kWriteSlots];
  bool bad = false;
  int64_t cur = -1;
  char* base = nullptr;
  bool ok = false;
#pragma unroll
  for (int j = 0; j < kWriteSlots; ++j) {
    if (live[j] && tok[j] != cur) {
      cur = tok[j];
      const int64_t s = sl[cur];
      ok = false;
      if (s >= 0) {
        int64_t blk, off;
        if (s <= 0x7fffffff) {
          blk = (uint32_t)s / (uint32_t)a.block_size;
          off = (uint32_t)s - (uint32_t)blk * (uint32_t)a.block_size;
        } else {
          blk = s / a.block_size;
          off = s - blk * a.block_size;
        }
        if (blk < a.num_blocks) {
          base = a.cache + blk * a.block_stride + off * a.token_stride;
          ok = true;
        } else {
          bad = true;
        }
      }
    }
    on[j] = live[j] && ok;
    dp[j] = base + dof[j];
  }
#pragma unroll
  for (int j = 0; j < kWriteSlots; ++j)
    if (on[j]) store16<NTS>(dp[j] + lane * kVec, v[j]);
  if (bad && lane == 0) raise_error(a.err, KVX_DEVERR_SLOT_RANGE);
}

// New-token write for rows of up to 2 KiB that are not whole KiB (any multiple of 16 bytes).
// A wavefront takes tokens_per_wave whole tokens (as many as fit in kWriteSlots * 64 vectors:
// 8 tokens of 256-byte rows); lane l of instruction j takes vector 64 j + l of that run of
// (token, K/V, 16-byte vector) triples. Each lane's row loads and slot loads are all in flight
// before its stores. Indexing is by additions from one small division per lane, so a launch
// of a few tokens costs little more than its memory latency.
template <bool NTL, bool NTS>
__global__ __launch_bounds__(256) void write_vectors_kernel(WriteArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t w = uniform((int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave));
  const int64_t t0 = w * a.tokens_per_wave;
  if (t0 >= a.num_tokens) return;
  const int64_t t_end = t0 + a.tokens_per_wave < a.num_tokens ? t0 + a.tokens_per_wave : a.num_tokens;
  const uint32_t nvec = (uint32_t)(a.row_bytes / kVec);  // vectors per row
  const uint32_t tv = 2 * nvec;  // vectors per token (K row, then V row), at most 512
  // lane's vector as (token t, index r inside the token); each instruction moves on by 64
  // vectors = step_t tokens + step_r vectors
  const uint32_t step_t = kWave / tv, step_r = kWave - step_t * tv;
  const uint32_t tl = (uint32_t)lane / tv;
  uint32_t r = (uint32_t)lane - tl * tv;
  int64_t t = t0 + tl;
  const char* kp = a.key + t * a.key_stride;
  const char* vp = a.value + t * a.value_stride;
  const int64_t* slot_p = a.slots + t;
  const int64_t dk = (int64_t)step_t * a.key_stride, dv = (int64_t)step_t * a.value_stride;

  const char* sp[kWriteSlots];
  const int64_t* slp[kWriteSlots];
  int64_t dof[kWriteSlots];
  bool live[kWriteSlots];
#pragma unroll
  for (int j = 0; j < kWriteSlots; ++j) {
    live[j] = t < t_end;
    const bool is_v = r >= nvec;
    const uint32_t q = is_v ? r - nvec : r;
    dof[j] = (is_v ? a.kv_stride : 0) + (int64_t)q * kVec;  // offset inside the token's slot
    // idle lanes re-read the first vector of row 0 and slot 0
    sp[j] = live[j] ? (is_v ? vp : kp) + (int64_t)q * kVec : a.key;
    slp[j] = live[j] ? slot_p : a.slots;
    t += step_t;
    kp += dk;
    vp += dv;
    slot_p += step_t;
    r += step_r;
    if (r >= tv) {
      r -= tv;
      ++t;
      kp += a.key_stride;
      vp += a.value_stride;
      ++slot_p;
    }
  }
  u32x4 v[kWriteSlots];
#pragma unroll
  for (int j = 0; j < kWriteSlots; ++j) v[j] = load16<NTL>(sp[j]);
  int64_t sv[kWriteSlots];
#pragma unroll
  for (int j = 0; j < kWriteSlots; ++j) sv[j] = *slp[j];

  char* dp[kWriteSlots];
  bool on[kWriteSlots];
  bool bad = false;
  const int32_t shift = a.block_shift;
#pragma unroll
  for (int j = 0; j < kWriteSlots; ++j) {
    const int64_t s = sv[j];
    on[j] = false;
    dp[j] = a.cache;
    if (live[j] && s >= 0) {
      int64_t blk, off;
      if (shift >= 0) {
        blk = s >> shift;
        off = s & (((int64_t)1 << shift) - 1);
      } else if (s <= 0x7fffffff) {
        blk = (uint32_t)s / (uint32_t)a.block_size;
        off = (uint32_t)s - (uint32_t)blk * (uint32_t)a.block_size;
      } else {
        blk = s / a.block_size;
        off = s - blk * a.block_size;
      }
      if (blk < a.num_blocks) {
        dp[j] = a.cache + blk * a.block_stride + off * a.token_stride + dof[j];
        on[j] = true;
      } else {
        bad = true;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kWriteSlots; ++j)
    if (on[j]) store16<NTS>(dp[j], v[j]);
  if (__ballot(bad) != 0 && lane == 0) raise_error(a.err, KVX_DEVERR_SLOT_RANGE);
}

// --------------------------------------------------------------------------------------
// a3 — transfer list: run-start flags -> prefix scan -> compaction, tiles over up to 256 workgroups
// --------------------------------------------------------------------------------------

constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;                          // positions per thread in the own tile
constexpr int kScanTile = kScanThreads * kScanItems;   // 2048 positions per workgroup
constexpr int kScanWaves = kScanThreads / kWave;
#ifndef KVX_PREFIX_GROUPS
#define KVX_PREFIX_GROUPS 4
#endif
constexpr int kPrefixGroups = KVX_PREFIX_GROUPS;       // 1024-position groups per prefix round
constexpr int kLdsOffsets = 4096;  // request offsets staged in LDS when num_reqs < this
#ifndef KVX_BUILD_MAX_WGS
#define KVX_BUILD_MAX_WGS 256
#endif
constexpr int64_t kBuildMaxWgs = KVX_BUILD_MAX_WGS;  // one per CU

// Largest r in [0, R) with ro[r] <= p (0 if none).
template <class P>
__device__ __forceinline__ int32_t find_request(P ro, int32_t R, int64_t p) {
  int32_t lo = 0, hi = R - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (ro[mid] <= p) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Ids at positions p0 - 1 .. p0 + ITEMS, loaded unconditionally (indices clamped into
// [0, N), N > 0) so that all the loads of a round are in flight together.
template <int ITEMS>
__device__ __forceinline__ void chunk_ids(const int32_t* __restrict__ src,
                                          const int32_t* __restrict__ dst, int64_t N,
                                          bool use_src, bool use_dst, int64_t p0,
                                          int32_t (&sv)[ITEMS + 2], int32_t (&dv)[ITEMS + 2]) {
#pragma unroll
  for (int i = 0; i < ITEMS + 2; ++i) {
    int64_t p = p0 - 1 + i;
    p = p < 0 ? 0 : (p < N ? p : N - 1);
    sv[i] = use_src ? src[p] : 0;
    dv[i] = use_dst ? dst[p] : 0;
  }
}

// Run-start flags of positions p0 .. p0 + ITEMS (one past the chunk, for run ends) and the
// request of each of the first ITEMS, from the ids chunk_ids loaded. Position p starts a run
// if it is the first position, the first of its request, or an addressed side does not step
// by +1 from p - 1. Positions at or past N are not starts.
template <int ITEMS, class P>
__device__ __forceinline__ void chunk_flags(P ro, int32_t R, int64_t N, bool use_src,
                                            bool use_dst, int64_t p0,
                                            const int32_t (&sv)[ITEMS + 2],
                                            const int32_t (&dv)[ITEMS + 2],
                                            bool (&st)[ITEMS + 1], int32_t (&rq)[ITEMS]) {
  // r is the request holding p; cur and nxt are the starts of r and of r + 1 (past the last
  // request, never reached), kept in registers so that LDS is read again only where a request
  // boundary falls among the chunk's positions
  constexpr int64_t kNever = INT64_MAX;
  int32_t r = (p0 < N) ? find_request(ro, R, p0) : 0;
  int64_t cur = ro[r];
  int64_t nxt = r + 1 < R ? ro[r + 1] : kNever;
#pragma unroll
  for (int i = 0; i <= ITEMS; ++i) {
    const int64_t p = p0 + i;
    bool f = false;
    if (p < N) {
      while (nxt <= p) {
        ++r;
        cur = nxt;
        nxt = r + 1 < R ? ro[r + 1] : kNever;
      }
      f = (p == 0) || (p == cur) ||
          (use_src && (int64_t)sv[i + 1] != (int64_t)sv[i] + 1) ||
          (use_dst && (int64_t)dv[i + 1] != (int64_t)dv[i] + 1);
    }
    st[i] = f;
    if (i < ITEMS) rq[i] = r;
  }
}

// Wave-wide inclusive scans of 32-bit values with DPP moves: row shifts by 1, 2, 4 and 8
// inside each row of 16 lanes, then the broadcasts of lane 15 into rows 1 and 3 and of lane 31
// into rows 2 and 3. A lane whose source lies outside its row, or whose row the mask leaves
// out, takes the identity. Each step is a register move between lanes, where a shuffle would
// be a round trip through the LDS crossbar.
constexpr int kDppRowShr = 0x110, kDppWaveShr1 = 0x138, kDppRowBcast15 = 0x142,
              kDppRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ int32_t dpp_move(int32_t identity, int32_t v) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROWS, 0xf, false);
}

__device__ __forceinline__ int32_t wave_scan_sum(int32_t v) {
  v += dpp_move<kDppRowShr + 1, 0xf>(0, v);
  v += dpp_move<kDppRowShr + 2, 0xf>(0, v);
  v += dpp_move<kDppRowShr + 4, 0xf>(0, v);
  v += dpp_move<kDppRowShr + 8, 0xf>(0, v);
  v += dpp_move<kDppRowBcast15, 0xa>(0, v);
  v += dpp_move<kDppRowBcast31, 0xc>(0, v);
  return v;
}

__device__ __forceinline__ int32_t wave_scan_max(int32_t v) {
  v = max(v, dpp_move<kDppRowShr + 1, 0xf>(INT32_MIN, v));
  v = max(v, dpp_move<kDppRowShr + 2, 0xf>(INT32_MIN, v));
  v = max(v, dpp_move<kDppRowShr + 4, 0xf>(INT32_MIN, v));
  v = max(v, dpp_move<kDppRowShr + 8, 0xf>(INT32_MIN, v));
  v = max(v, dpp_move<kDppRowBcast15, 0xa>(INT32_MIN, v));
  v = max(v, dpp_move<kDppRowBcast31, 0xc>(INT32_MIN, v));
  return v;
}

// v of the lane before across the whole wave; `first` in lane 0
__device__ __forceinline__ int32_t wave_shift_up(int32_t v, int32_t first) {
  return dpp_move<kDppWaveShr1, 0xf>(first, v);
}

// Ids of one prefix round: kPrefixGroups groups of kScanThreads * 4 positions from `base`,
// 4 consecutive positions per lane (plus the one before and the one after).
struct PrefixRound {
  int32_t s[kPrefixGroups][6];
  int32_t d[kPrefixGroups][6];
};
constexpr int64_t kPrefixRound = (int64_t)kScanThreads * 4 * kPrefixGroups;

__device__ __forceinline__ void prefix_load(const int32_t* __restrict__ src,
                                            const int32_t* __restrict__ dst, int64_t N,
                                            bool use_src, bool use_dst, int64_t base,
                                            PrefixRound& r) {
#pragma unroll
  for (int g = 0; g < kPrefixGroups; ++g)
    chunk_ids<4>(src, dst, N, use_src, use_dst, base + ((int64_t)g * kScanThreads + threadIdx.x) * 4,
                 r.s[g], r.d[g]);
}

// Id breaks among the round's positions that lie in [1, begin): count and latest position.
__device__ __forceinline__ void prefix_count(const PrefixRound& r, int64_t base, int64_t begin,
                                             bool use_src, bool use_dst, int64_t& pc, int64_t& pl) {
#pragma unroll
  for (int g = 0; g < kPrefixGroups; ++g) {
    const int64_t q0 = base + ((int64_t)g * kScanThreads + threadIdx.x) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t p = q0 + i;
      const bool brk = (use_src && (int64_t)r.s[g][i + 1] != (int64_t)r.s[g][i] + 1) ||
                       (use_dst && (int64_t)r.d[g][i + 1] != (int64_t)r.d[g][i] + 1);
      if (p >= 1 && p < begin && brk) { ++pc; pl = p; }
    }
  }
}

// Workgroup b owns positions [b * span, (b + 1) * span), span a multiple of kScanTile. It
// first counts the run starts before its range and finds the latest of them (a pass over
// every earlier id and over the request offsets, no writes). Then, one kScanTile sub-tile
// at a time, it flags its positions (8 per thread), turns them into run indices and
// latest-start positions with a wave scan plus a 4-entry LDS pass, and writes the runs each
// thread starts and the lengths of the runs it ends, carrying the count and the latest start
// to the next sub-tile. No thread reads another's output, and no workgroup waits for another.
//
// The kernel is a chain of dependent memory round trips, so every load that depends on
// nothing is issued at the start, before the request offsets are staged in LDS: the ids of
// the first sub-tile, the first prefix round and, with fewer than kScanThreads requests, one
// offset per thread. The ids at the request starts (which need the offsets) are loaded before
// the prefix pass's arithmetic, and each later sub-tile's or round's ids before the current
// one is scanned.
template <class P>
__device__ __forceinline__ void build_tile(const int32_t* __restrict__ src,
                                           const int32_t* __restrict__ dst, P ro, int32_t R,
                                           int64_t N, bool use_src, bool use_dst,
                                           kvx_xfer* __restrict__ out, int64_t* __restrict__ count,
                                           int64_t span, int64_t* s_cnt, int64_t* s_last,
                                           int32_t (&sv)[kScanItems + 2], int32_t (&dv)[kScanItems + 2],
                                           PrefixRound& cur) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int64_t begin = (int64_t)blockIdx.x * span;
  const int64_t end = begin + span < N ? begin + span : N;

  // 1. run starts before the range: count and latest position. With a valid CSR a position
  //    p in [1, begin) starts a run iff its ids break the +1 step from p - 1 or a request
  //    starts at p, so the count is: position 0, plus the id breaks, plus the request starts
  //    that are not id breaks. (b) finds the request starts in [1, begin) (the first request
  //    at each) and loads the ids on both sides of each; (a) streams the ids in rounds.
  int64_t pc = 0, pl = -1;
  const bool one_each = R < kScanThreads;
  if (begin > 0) {
    // with fewer than kScanThreads requests, thread t takes request 1 + t: its start and the
    // ids on both sides of it are loaded before (a) runs
    const int32_t r1 = 1 + tid;
    int64_t q = 0;
    bool qs = false;
    int32_t a0 = 0, a1 = 0, b0 = 0, b1 = 0;
    if (one_each && r1 < R) {
      q = ro[r1];
      qs = q >= 1 && q < begin && q != ro[r1 - 1];  // the first request starting at q
      if (qs) {
        if (use_src) { a0 = src[q - 1]; a1 = src[q]; }
        if (use_dst) { b0 = dst[q - 1]; b1 = dst[q]; }
      }
    }
    for (int64_t base = 0; base < begin; base += kPrefixRound) {
      const bool more = base + kPrefixRound < begin;
      PrefixRound nxt;
      if (more) prefix_load(src, dst, N, use_src, use_dst, base + kPrefixRound, nxt);
      prefix_count(cur, base, begin, use_src, use_dst, pc, pl);
      if (more) cur = nxt;
    }
    if (one_each) {
      if (qs) {
        pl = q > pl ? q : pl;
        const bool brk = (use_src && (int64_t)a1 != (int64_t)a0 + 1) ||
                         (use_dst && (int64_t)b1 != (int64_t)b0 + 1);
        if (!brk) ++pc;
      }
    } else {
      for (int32_t r = 1 + tid; r < R; r += kScanThreads) {
        const int64_t qr = ro[r];
        if (qr >= 1 && qr < begin && qr != ro[r - 1]) {  // the first request starting at qr
          pl = qr > pl ? qr : pl;
          const bool brk = (use_src && (int64_t)src[qr] != (int64_t)src[qr - 1] + 1) ||
                           (use_dst && (int64_t)dst[qr] != (int64_t)dst[qr - 1] + 1);
          if (!brk) ++pc;
        }
      }
    }
    if (tid == 0) {  // position 0
      ++pc;
      pl = pl > 0 ? pl : 0;
    }
  }
  if (N <= INT32_MAX) {  // counts and positions fit 32 bits: DPP scans, totals in the last lane
    const int32_t c = wave_scan_sum((int32_t)pc);
    const int32_t l = wave_scan_max((int32_t)pl);
    if (lane == kWave - 1) { s_cnt[wid] = c; s_last[wid] = l; }
  } else {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      pc += __shfl_xor(pc, d, kWave);
      const int64_t o = __shfl_xor(pl, d, kWave);
      pl = o > pl ? o : pl;
    }
    if (lane == 0) { s_cnt[wid] = pc; s_last[wid] = pl; }
  }
  __syncthreads();
  int64_t carry_cnt = 0, carry_last = -1;
#pragma unroll
  for (int w = 0; w < kScanWaves; ++w) {
    carry_cnt += s_cnt[w];
    carry_last = s_last[w] > carry_last ? s_last[w] : carry_last;
  }
  __syncthreads();

  // 2. the own range, one sub-tile at a time (sv / dv hold the current sub-tile's ids)
  for (int64_t tile = begin; tile < end; tile += kScanTile) {
    const int64_t p0 = tile + (int64_t)tid * kScanItems;
    const bool more = tile + kScanTile < end;
    int32_t nsv[kScanItems + 2], ndv[kScanItems + 2];
    if (more) chunk_ids<kScanItems>(src, dst, N, use_src, use_dst, p0 + kScanTile, nsv, ndv);
    bool st[kScanItems + 1];
    int32_t rq[kScanItems];
    chunk_flags<kScanItems>(ro, R, N, use_src, use_dst, p0, sv, dv, st, rq);
    int64_t cnt = 0, last = -1;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i)
      if (st[i]) { ++cnt; last = p0 + i; }

    // workgroup scan of (cnt: sum, last: max): wave scans in 32 bits with the latest start
    // relative to the sub-tile, then a 4-entry LDS pass
    const int32_t ci32 = wave_scan_sum((int32_t)cnt);
    const int32_t li32 = wave_scan_max(last < 0 ? -1 : (int32_t)(last - tile));
    const int32_t lx32 = wave_shift_up(li32, -1);  // li of the lane before, -1 in lane 0
    const int64_t ci = ci32;
    const int64_t li = li32 < 0 ? -1 : tile + li32;
    const int64_t li_excl = lx32 < 0 ? -1 : tile + lx32;
    if (lane == kWave - 1) { s_cnt[wid] = ci; s_last[wid] = li; }
    __syncthreads();
    int64_t c_before = 0, l_before = -1, c_tile = 0, l_tile = -1;
#pragma unroll
    for (int w = 0; w < kScanWaves; ++w) {
      const int64_t c = s_cnt[w], l = s_last[w];
      if (w < wid) { c_before += c; l_before = l > l_before ? l : l_before; }
      c_tile += c;
      l_tile = l > l_tile ? l : l_tile;
    }

    int64_t k = carry_cnt + c_before + (ci - cnt);
    int64_t cur_start = carry_last;
    if (l_before > cur_start) cur_start = l_before;
    if (li_excl > cur_start) cur_start = li_excl;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int64_t p = p0 + i;
      if (p < N) {
        const bool ends = p == N - 1 || st[i + 1];
        if (k >= N) break;  // only with offsets that are not a CSR (flagged by workgroup 0)
        if (st[i]) {
          // a run that starts here: 16-byte stores of (src, dst) and, when it also ends here,
          // of (buf, num_blocks = 1 | req << 32); the xfer array is 16-byte aligned
          KVX_GLOBAL i64x2* x = (KVX_GLOBAL i64x2*)(out + k);
          i64x2 head;
          head.x = use_src ? (int64_t)sv[i + 1] : p;
          head.y = use_dst ? (int64_t)dv[i + 1] : p;
          x[0] = head;
          if (ends) {
            i64x2 tail;
            tail.x = p;
            tail.y = (int64_t)(((uint64_t)(uint32_t)rq[i] << 32) | 1u);
            x[1] = tail;
          } else {
            out[k].buf_block = p;
            out[k].req = rq[i];
          }
          cur_start = p;
          ++k;
        } else if (ends && k > 0) {  // k > 0 always: position 0 starts a run
          out[k - 1].num_blocks = (int32_t)(p - cur_start + 1);
        }
      }
    }
    carry_cnt += c_tile;
    if (l_tile > carry_last) carry_last = l_tile;
    if (more) {
#pragma unroll
      for (int i = 0; i < kScanItems + 2; ++i) { sv[i] = nsv[i]; dv[i] = ndv[i]; }
    }
    __syncthreads();  // the next sub-tile reuses s_cnt / s_last
  }
  if (blockIdx.x == gridDim.x - 1 && tid == 0) *count = carry_cnt;
}

__global__ __launch_bounds__(kScanThreads) void build_xfer_kernel(
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
    const int64_t* __restrict__ ro, int32_t R, int64_t N, int32_t mode,
    kvx_xfer* __restrict__ out, int64_t* __restrict__ count, int32_t* err, int64_t span) {
  __shared__ int64_t s_cnt[kScanWaves];
  __shared__ int64_t s_last[kScanWaves];
  __shared__ int64_t s_ro[kLdsOffsets + 1];
  const int tid = threadIdx.x;
  const bool use_src = mode != KVX_MODE_UNPACK;
  const bool use_dst = mode != KVX_MODE_PACK;
  const bool in_lds = R < kLdsOffsets;
  const bool one_each = R < kScanThreads;  // at most one offset per thread
  const bool check = blockIdx.x == 0;      // one workgroup checks the CSR
  const int64_t begin = (int64_t)blockIdx.x * span;

  // loads that depend on nothing, in flight together
  int64_t my_ro = 0;
  if (one_each && tid <= R) my_ro = ro[tid];
  int32_t sv[kScanItems + 2], dv[kScanItems + 2];
  if (N > 0) chunk_ids<kScanItems>(src, dst, N, use_src, use_dst, begin + (int64_t)tid * kScanItems, sv, dv);
  PrefixRound cur;
  if (begin > 0) prefix_load(src, dst, N, use_src, use_dst, 0, cur);

  // stage the offsets in LDS; CSR sanity: ro[0] == 0, non-decreasing, ro[R] == N
  if (one_each) {
    if (tid <= R) s_ro[tid] = my_ro;
  } else if (in_lds || check) {
    for (int32_t i = tid; i <= R; i += kScanThreads) {
      const int64_t v = ro[i];
      if (in_lds) s_ro[i] = v;
      if (check && i < R && ro[i + 1] < v) raise_error(err, KVX_DEVERR_OFFSETS);
    }
  }
  __syncthreads();
  if (check) {
    if (one_each) {
      if (tid < R && s_ro[tid + 1] < s_ro[tid]) raise_error(err, KVX_DEVERR_OFFSETS);
      if (tid == 0 && (s_ro[0] != 0 || s_ro[R] != N)) raise_error(err, KVX_DEVERR_OFFSETS);
    } else if (tid == 0 && (ro[0] != 0 || ro[R] != N)) {
      raise_error(err, KVX_DEVERR_OFFSETS);
    }
  }
  if (in_lds)
    build_tile<const int64_t*>(src, dst, s_ro, R, N, use_src, use_dst, out, count, span, s_cnt, s_last, sv, dv, cur);
  else
    build_tile<const int64_t*>(src, dst, ro, R, N, use_src, use_dst, out, count, span, s_cnt, s_last, sv, dv, cur);
}

// --------------------------------------------------------------------------------------
// a4 / a5 — pack and single-source unpack over the run list
// --------------------------------------------------------------------------------------

// Direction of a run copy: cache -> buffer (pack), buffer -> cache (unpack), or cache ->
// cache with no buffer (direct: every run's source and destination blocks are consecutive).
constexpr int kToBuffer = kDirToBuffer, kFromBuffer = kDirFromBuffer, kDirect = kDirDirect;

struct RunCopyArgs {
  const char* const* layer_bases;      // the cache read (pack, direct) or written (unpack)
  const char* const* dst_layer_bases;  // direct only: the cache written
  char* buffer;                        // pack and unpack only
  const kvx_xfer* xfers;
  const int64_t* xfer_count;
  int32_t* err;
  int64_t block_bytes;
  int64_t num_cache_blocks;
  int64_t dst_num_cache_blocks;        // direct only
  int64_t total_blocks;
  int64_t blocks_per_wave;
  int64_t waves_per_layer;
  int64_t total_waves;
  int64_t num_wgs;
  int32_t num_layers;
  int32_t xcd_remap;
  // completion signal folded into the launch (pack and direct only; null otherwise)
  uint64_t* signal;
  uint64_t signal_delta;
  uint32_t* arrivals;  // workgroups of the launch that have finished; every launch leaves it 0
};

// The completion signal inside a copy launch ("5. flagcx connector design & dev & test",
// §1.2: the sender's last write of a batch carries the signal that the receiver counts).
// In a signalling launch every data store is device-coherent (store16_at<., true>), so a
// store that has been acknowledged is at the device's coherence point and no XCD holds it
// dirty in its L2. Each wavefront waits for its acknowledgements and the workgroup meets at a
// barrier; then one thread counts the workgroup. Counting goes through kArrivalGroups group
// counters (workgroup b counts in group b % kArrivalGroups), each on its own 128-byte line,
// and one top counter: the last workgroup of a group resets its group counter and counts the
// group at the top; the last group resets the top counter and adds `delta` to the signal
// counter. Every workgroup's bytes were acknowledged before it counted itself, so whoever
// reads the new signal count reads every byte of the launch, and all counters are back at 0
// for the next launch. Spreading the counts over 16 lines keeps a 2304-workgroup launch from
// queueing on one address; no workgroup writes back or invalidates an L2 (an agent-scope
// release per workgroup writes the XCD's whole L2 back each time). The counter words are
// touched only by vector atomics and stores from one lane, never through the scalar cache.
constexpr uint32_t kArrivalGroups = 16;
constexpr uint32_t kArrivalStride = 32;  // 32-bit words between counters: one 128-byte line

__device__ __forceinline__ void arrive_and_signal(uint32_t* arrivals, uint64_t* counter, uint64_t delta) {
  __builtin_amdgcn_s_waitcnt(0);  // this wavefront's stores are acknowledged
  __syncthreads();                // and so are those of the other wavefronts
  if (threadIdx.x == 0) {
    const uint32_t G = gridDim.x, b = blockIdx.x;
    const uint32_t groups = G < kArrivalGroups ? G : kArrivalGroups;
    const uint32_t g = b % kArrivalGroups;
    const uint32_t members = (G - g + kArrivalGroups - 1) / kArrivalGroups;
    uint32_t* gc = arrivals + (1 + g) * kArrivalStride;
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == members) {
      __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == groups) {
        __hip_atomic_store(arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(counter, delta, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  }
}


// Work split: wavefront w owns layer l = w / waves_per_layer and buffer positions
// [c*B, min((c+1)*B, N)) of that layer (B = blocks_per_wave), so every wavefront moves the
// same number of bytes whatever the run lengths. It finds the run holding its first
// position, then walks the runs overlapping its range; each overlap is one contiguous copy
// on both sides (run blocks are consecutive in the cache and in the buffer).
template <int DIR, bool NTL, bool NTS, bool DEVICE>
__device__ __forceinline__ void copy_runs_body(const RunCopyArgs& a) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t wg = blockIdx.x;
  if (a.xcd_remap) wg = xcd_slice_order(wg, a.num_wgs);
  const int64_t w = uniform(wg * kCopyWavesPerWg + (threadIdx.x / kWave));
  if (w >= a.total_waves) return;
  const int64_t l = w / a.waves_per_layer;
  const int64_t c = w - l * a.waves_per_layer;
  const int64_t N = a.total_blocks;
  const int64_t p0 = c * a.blocks_per_wave;
  const int64_t p1 = (p0 + a.blocks_per_wave < N) ? p0 + a.blocks_per_wave : N;
  const int64_t BB = a.block_bytes;
  int64_t count = *a.xfer_count;
  if (count > N) count = N;
  if (count <= 0) return;
  char* cache = const_cast<char*>(a.layer_bases[l]);
  char* dcache = DIR == kDirect ? const_cast<char*>(a.dst_layer_bases[l]) : nullptr;
  char* buf = DIR == kDirect ? nullptr : a.buffer + l * N * BB;

  int64_t k = uniform(find_run(a.xfers, count, p0, lane));
  if (k < 0) k = 0;
  bool bad = false;
  for (; k < count; ++k) {
    const kvx_xfer x = a.xfers[k];
    const int64_t rb = x.buf_block;
    if (rb >= p1) break;
    int64_t lo = rb > p0 ? rb : p0;
    const int64_t re = rb + (int64_t)x.num_blocks;
    int64_t hi = re < p1 ? re : p1;
    if (lo >= hi) continue;
    // positions [lo, hi) of the run; trim the ends whose ids fall outside their cache
    const int64_t sid = (DIR == kFromBuffer ? x.dst_block : x.src_block) + (lo - rb);
    int64_t nlo = lo, nhi = hi;
    if (sid < 0) nlo = lo - sid;
    if (sid + (hi - lo) > a.num_cache_blocks) nhi = lo + (a.num_cache_blocks - sid);
    int64_t did = 0;
    if (DIR == kDirect) {
      did = x.dst_block + (lo - rb);
      if (lo - did > nlo) nlo = lo - did;
      if (lo + (a.dst_num_cache_blocks - did) < nhi) nhi = lo + (a.dst_num_cache_blocks - did);
    }
    if (nlo != lo || nhi != hi) bad = true;
    if (nlo >= nhi) continue;
    const int64_t bytes = (nhi - nlo) * BB;
    char* cptr = cache + (sid + (nlo - lo)) * BB;
    if (DIR == kToBuffer) wave_copy<kCopyBatch, NTL, NTS, DEVICE>(cptr, buf + nlo * BB, bytes, lane);
    else if (DIR == kFromBuffer) wave_copy<kCopyBatch, NTL, NTS, DEVICE>(buf + nlo * BB, cptr, bytes, lane);
    else wave_copy<kCopyBatch, NTL, NTS, DEVICE>(cptr, dcache + (did + (nlo - lo)) * BB, bytes, lane);
  }
  if (bad && lane == 0) raise_error(a.err, KVX_DEVERR_BLOCK_RANGE);
}

template <int DIR, bool NTL, bool NTS, bool SIGNAL>
__global__ __launch_bounds__(kCopyThreads) void copy_runs_kernel(RunCopyArgs a) {
  copy_runs_body<DIR, NTL, NTS, SIGNAL>(a);
  if constexpr (SIGNAL) arrive_and_signal(a.arrivals, a.signal, a.signal_delta);
}

// --------------------------------------------------------------------------------------
// a6 — head shards: merge (unpack from num_shards senders) and split (pack for num_shards
// receivers). A full-head cache block is rows_per_block rows; shard d holds piece d of
// every row, contiguously, in pack order.
// --------------------------------------------------------------------------------------

struct ShardArgs {
  char* shard[KVX_MAX_SOURCES];  // [L][N][block_bytes/num_shards] each
  const char* const* layer_bases;
  const kvx_xfer* xfers;
  const int64_t* xfer_count;
  int32_t* err;
  int64_t block_bytes;  // full-head cache block
  int64_t num_cache_blocks;
  int64_t total_blocks;
  int64_t row_piece;    // bytes of one shard's piece of a row
  int64_t blocks_per_wave;
  int64_t waves_per_layer;
  int64_t total_waves;
  int64_t num_wgs;
  int32_t num_shards;
  int32_t rows_per_block;
  int32_t num_layers;
  int32_t xcd_remap;
};

// Same work split as copy_runs_kernel. For each overlap of n blocks the cache side is
// n*rows_per_block rows of num_shards*row_piece bytes, and shard d's side is its own
// contiguous n*rows_per_block*row_piece bytes. Per shard the wavefront streams that shard's
// rows in order and meets the cache at the full row stride. TO_BUFFER = split (cache ->
// shards, ids from the run's source side); otherwise merge (shards -> cache).
template <bool TO_BUFFER, bool NTL, bool NTS>
__global__ __launch_bounds__(kCopyThreads) void shard_runs_kernel(ShardArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t wg = blockIdx.x;
  if (a.xcd_remap) wg = xcd_slice_order(wg, a.num_wgs);
  const int64_t w = uniform(wg * kCopyWavesPerWg + (threadIdx.x / kWave));
  if (w >= a.total_waves) return;
  const int64_t l = w / a.waves_per_layer;
  const int64_t c = w - l * a.waves_per_layer;
  const int64_t N = a.total_blocks;
  const int64_t p0 = c * a.blocks_per_wave;
  const int64_t p1 = (p0 + a.blocks_per_wave < N) ? p0 + a.blocks_per_wave : N;
  const int64_t S = a.num_shards;
  const int64_t BB = a.block_bytes;
  const int64_t BBs = BB / S;
  const int64_t piece = a.row_piece;
  const int64_t row_full = piece * S;
  const int64_t vs = piece / kVec;                    // vectors per piece
  const int64_t M = (vs + kWave - 1) / kWave;         // instructions per piece
  int64_t count = *a.xfer_count;
  if (count > N) count = N;
  if (count <= 0) return;
  char* cache = const_cast<char*>(a.layer_bases[l]);

  int64_t k = uniform(find_run(a.xfers, count, p0, lane));
  if (k < 0) k = 0;
  bool bad = false;
  for (; k < count; ++k) {
    const kvx_xfer x = a.xfers[k];
    const int64_t rb = x.buf_block;
    if (rb >= p1) break;
    const int64_t lo = rb > p0 ? rb : p0;
    const int64_t re = rb + (int64_t)x.num_blocks;
    const int64_t hi = re < p1 ? re : p1;
    if (lo >= hi) continue;
    const int64_t id0 = (TO_BUFFER ? x.src_block : x.dst_block) + (lo - rb);
    const int64_t id1 = id0 + (hi - lo);
    const int64_t v0 = id0 > 0 ? id0 : 0;
    const int64_t v1 = id1 < a.num_cache_blocks ? id1 : a.num_cache_blocks;
    if (v0 != id0 || v1 != id1) bad = true;
    if (v0 >= v1) continue;
    const int64_t bpos = lo + (v0 - id0);
    char* cblk = cache + v0 * BB;
    const int64_t rows = (v1 - v0) * a.rows_per_block;
    const int64_t steps = rows * M;
    for (int64_t d = 0; d < S; ++d) {
      char* sblk = a.shard[d] + (l * N + bpos) * BBs;
      char* ccol = cblk + d * piece;
      int64_t row = 0, m = 0;
      for (int64_t t0 = 0; t0 < steps; t0 += kCopyBatch) {
        const char* sp[kCopyBatch];
        char* dp[kCopyBatch];
        bool act[kCopyBatch];
#pragma unroll
        for (int j = 0; j < kCopyBatch; ++j) {
          const int64_t xv = m * kWave + lane;
          act[j] = (t0 + j < steps) && (xv < vs);
          char* sh = sblk + row * piece + xv * kVec;
          char* ca = ccol + row * row_full + xv * kVec;
          sp[j] = TO_BUFFER ? ca : sh;
          dp[j] = TO_BUFFER ? sh : ca;
          if (++m == M) { m = 0; ++row; }
        }
        u32x4 v[kCopyBatch];
#pragma unroll
        for (int j = 0; j < kCopyBatch; ++j)
          if (act[j]) v[j] = load16<NTL>(sp[j]);
#pragma unroll
        for (int j = 0; j < kCopyBatch; ++j)
          if (act[j]) store16<NTS>(dp[j], v[j]);
      }
    }
  }
  if (bad && lane == 0) raise_error(a.err, KVX_DEVERR_BLOCK_RANGE);
}

// --------------------------------------------------------------------------------------
// one-batch fast paths (block rows in whole KiB)
// --------------------------------------------------------------------------------------

// In the fast paths a wavefront moves one batch of K 1 KiB instructions (K KiB); K is chosen
// per kernel at launch (4 or 8).

// Pack / single-source unpack when block_bytes is a multiple of 1 KiB (a 16-token block of
// K,V x heads x head_dim x 2 B always is). Wavefront w owns K KiB of one layer's buffer
// slice; each of its K instruction slots lies inside one block. The slot addresses
// are worked out on the scalar unit (walking the runs from the one holding the first block),
// then the wavefront issues all its loads, then all its stores, and exits. On this
// architecture stores count in vmcnt, so a wavefront with a second batch would wait for its
// first batch's store acknowledgements; one batch per wavefront never does.
template <int DIR, bool NTL, bool NTS, int K, bool DEVICE>
__device__ __forceinline__ void copy_slots_body(const RunCopyArgs& a) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t wg = blockIdx.x;
  if (a.xcd_remap) wg = xcd_slice_order(wg, a.num_wgs);
  const int64_t w = uniform(wg * kCopyWavesPerWg + (threadIdx.x / kWave));
  if (w >= a.total_waves) return;
  const int64_t l = w / a.waves_per_layer;
  const int64_t u = w - l * a.waves_per_layer;
  const int64_t N = a.total_blocks;
  const int64_t BB = a.block_bytes;
  const int64_t layer_bytes = N * BB;
  const KVX_CONST kvx_xfer* xf = readonly(a.xfers);
  int64_t count = *readonly(a.xfer_count);
  if (count > N) count = N;
  if (count <= 0) return;
  char* cache = const_cast<char*>(*readonly(a.layer_bases + l));
  char* dcache = DIR == kDirect ? const_cast<char*>(*readonly(a.dst_layer_bases + l)) : nullptr;
  char* buf = DIR == kDirect ? nullptr : a.buffer + l * layer_bytes;

  const int64_t o0 = u * ((int64_t)K * kWaveBytes);
  int64_t q = o0 / BB;       // buffer position of the first slot
  int64_t off = o0 - q * BB; // byte offset inside that block (a multiple of 1 KiB)
  int64_t k = uniform(find_run(a.xfers, count, q, lane));
  if (k < 0) k = 0;
  Run x = load_run(xf, k);
  // Slots with nothing to move load from `idle` so every load is unconditional; only
  // stores are skipped. It is 1 KiB inside an allocation this launch owns: this wavefront's
  // own buffer range, or for a direct copy the first KiB of the source layer (whose cache
  // has at least one block).
  const char* idle = DIR == kDirect ? cache : buf + o0;
  const char* sp[K];
  char* dp[K];
  bool on[K];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t o = o0 + (int64_t)j * kWaveBytes;
    on[j] = false;
    sp[j] = idle;
    dp[j] = nullptr;
    if (o < layer_bytes) {
      while (x.buf + x.n <= q && k + 1 < count) x = load_run(xf, ++k);
      if (q >= x.buf && q < x.buf + x.n) {
        const int64_t id = (DIR == kFromBuffer ? x.dst : x.src) + (q - x.buf);
        const int64_t did = DIR == kDirect ? x.dst + (q - x.buf) : 0;
        const bool ok = id >= 0 && id < a.num_cache_blocks &&
                        (DIR != kDirect || (did >= 0 && did < a.dst_num_cache_blocks));
        if (ok) {
          char* c = cache + id * BB + off;
          if (DIR == kToBuffer) { sp[j] = c; dp[j] = buf + o; }
          else if (DIR == kFromBuffer) { sp[j] = buf + o; dp[j] = c; }
          else { sp[j] = c; dp[j] = dcache + did * BB + off; }
          on[j] = true;
        } else {
          bad = true;
        }
      }
    }
    off += kWaveBytes;
    if (off == BB) { off = 0; ++q; }
  }
  u32x4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = load16<NTL>(sp[j] + lane * kVec);
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (on[j]) store16_at<NTS, DEVICE>(dp[j], lane * kVec, v[j]);
  if (bad && lane == 0) raise_error(a.err, KVX_DEVERR_BLOCK_RANGE);
}

template <int DIR, bool NTL, bool NTS, int K, bool SIGNAL>
__global__ __launch_bounds__(kCopyThreads) void copy_slots_kernel(RunCopyArgs a) {
  copy_slots_body<DIR, NTL, NTS, K, SIGNAL>(a);
  if constexpr (SIGNAL) arrive_and_signal(a.arrivals, a.signal, a.signal_delta);
}

// Head shards when a row piece is a multiple of 1 KiB. TO_BUFFER = split (cache -> shards),
// otherwise merge (shards -> cache). Wavefront w owns K KiB of one layer's bytes taken in the
// shards' order (position q, then shard d, then row, then byte), so it moves one contiguous
// range of one shard and every S-th row piece of the cache block; slot j is bytes
// [xo, xo + 1 KiB) of row `row` of shard d, and the counters step without divisions. In
// interleaved A/B runs this order beat walking the cache block in its own order by 4.4% for
// the merge and 1.1% for the split.
template <bool TO_BUFFER, bool NTL, bool NTS, int K>
__global__ __launch_bounds__(kCopyThreads) void shard_slots_kernel(ShardArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t wg = blockIdx.x;
  if (a.xcd_remap) wg = xcd_slice_order(wg, a.num_wgs);
  const int64_t w = uniform(wg * kCopyWavesPerWg + (threadIdx.x / kWave));
  if (w >= a.total_waves) return;
  const int64_t l = w / a.waves_per_layer;
  const int64_t u = w - l * a.waves_per_layer;
  const int64_t N = a.total_blocks;
  const int64_t S = a.num_shards;
  const int64_t BB = a.block_bytes;
  const int64_t BBs = BB / S;
  const int64_t piece = a.row_piece;
  const int64_t row_full = piece * S;
  const int64_t layer_bytes = N * BB;
  const KVX_CONST kvx_xfer* xf = readonly(a.xfers);
  int64_t count = *readonly(a.xfer_count);
  if (count > N) count = N;
  if (count <= 0) return;
  char* cache = const_cast<char*>(*readonly(a.layer_bases + l));

  const int64_t rows = BBs / piece;
  const int64_t o0 = u * ((int64_t)K * kWaveBytes);
  int64_t q = o0 / BB;
  int64_t w_in = o0 - q * BB;
  int64_t d = w_in / BBs;
  int64_t row = (w_in - d * BBs) / piece;
  int64_t xo = w_in - d * BBs - row * piece;
  int64_t k = uniform(find_run(a.xfers, count, q, lane));
  if (k < 0) k = 0;
  Run x = load_run(xf, k);
  // Idle slots load the first KiB of shard 0's layer slice (always in bounds).
  const char* idle = a.shard[0] + l * N * BBs;
  const char* sp[K];
  char* dp[K];
  bool on[K];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t o = o0 + (int64_t)j * kWaveBytes;
    on[j] = false;
    sp[j] = idle;
    dp[j] = nullptr;
    if (o < layer_bytes) {
      while (x.buf + x.n <= q && k + 1 < count) x = load_run(xf, ++k);
      if (q >= x.buf && q < x.buf + x.n) {
        const int64_t id = (TO_BUFFER ? x.src : x.dst) + (q - x.buf);
        if (id >= 0 && id < a.num_cache_blocks) {
          char* sh = a.shard[d] + (l * N + q) * BBs + row * piece + xo;
          char* ca = cache + id * BB + row * row_full + d * piece + xo;
          sp[j] = TO_BUFFER ? ca : sh;
          dp[j] = TO_BUFFER ? sh : ca;
          on[j] = true;
        } else {
          bad = true;
        }
      }
    }
    xo += kWaveBytes;
    w_in += kWaveBytes;
    if (xo == piece) {
      xo = 0;
      if (++row == rows) { row = 0; ++d; }
    }
    if (w_in == BB) { w_in = 0; row = 0; d = 0; xo = 0; ++q; }
  }
  u32x4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = load16<NTL>(sp[j] + lane * kVec);
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (on[j]) store16<NTS>(dp[j] + lane * kVec, v[j]);
  if (bad && lane == 0) raise_error(a.err, KVX_DEVERR_BLOCK_RANGE);
}

// --------------------------------------------------------------------------------------
// f1 — kv-first caches (K plane, then V plane): one-batch kernel
// --------------------------------------------------------------------------------------

struct KvFirstArgs {
  const char* const* layer_bases;  // K plane base per layer; V plane at + plane_stride
  char* buffer;                    // [L][2N][segment]
  const kvx_xfer* xfers;
  const int64_t* xfer_count;
  const int64_t* req_offsets;      // [R+1]
  int32_t* err;
  int64_t segment_bytes;           // one block in one plane (a multiple of 1 KiB)
  int64_t plane_stride;
  int64_t num_cache_blocks;
  int64_t total_blocks;
  int64_t waves_per_layer;
  int64_t total_waves;
  int64_t num_wgs;
  int32_t num_reqs;
  int32_t num_layers;
  int32_t xcd_remap;
};

// Largest r in [0, R) with 2*ro[r] <= g: the request owning buffer segment g (empty
// requests are skipped because the largest such r is taken). 64-way search as find_run.
__device__ __forceinline__ int64_t find_segment_request(const int64_t* __restrict__ ro, int64_t R,
                                                        int64_t g, int lane) {
  int64_t lo = 0, hi = R;
  while (hi - lo > 1) {
    const int64_t step = (hi - lo + kWave - 1) / kWave;
    const int64_t idx = lo + (int64_t)lane * step;
    const bool pred = idx < hi && 2 * ro[idx] <= g;
    const uint64_t m = __ballot(pred);
    if (m == 0) return lo;
    const int64_t j = 63 - __builtin_clzll(m);
    lo = lo + j * step;
    hi = (lo + step < hi) ? lo + step : hi;
  }
  return lo;
}

// The buffer slice of layer l is, per request r, its K segments in table order, then its V
// segments (what a gather along the block axis of a (2, blocks, ...) tensor returns).
// Wavefront w owns K KiB of that slice: slot j is 1 KiB of segment g, which belongs to
// request r, plane `plane` and table index jj, i.e. position p = cum_r + jj. Runs never
// span requests, so p walks the runs of request r once per plane; the wavefront keeps the
// index of the request's first run to restart the walk for the V plane.
template <bool TO_BUFFER, bool NTL, bool NTS, int K>
__global__ __launch_bounds__(kCopyThreads) void kv_first_kernel(KvFirstArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  int64_t wg = blockIdx.x;
  if (a.xcd_remap) wg = xcd_slice_order(wg, a.num_wgs);
  const int64_t w = uniform(wg * kCopyWavesPerWg + (threadIdx.x / kWave));
  if (w >= a.total_waves) return;
  const int64_t l = w / a.waves_per_layer;
  const int64_t u = w - l * a.waves_per_layer;
  const int64_t N = a.total_blocks;
  const int64_t R = a.num_reqs;
  const int64_t SEG = a.segment_bytes;
  const int64_t layer_bytes = 2 * N * SEG;
  const KVX_CONST kvx_xfer* xf = readonly(a.xfers);
  const KVX_CONST int64_t* ro = readonly(a.req_offsets);
  int64_t count = *readonly(a.xfer_count);
  if (count > N) count = N;
  if (count <= 0) return;
  char* cache = const_cast<char*>(*readonly(a.layer_bases + l));
  char* buf = a.buffer + l * layer_bytes;

  const int64_t o0 = u * ((int64_t)K * kWaveBytes);
  int64_t g = o0 / SEG;
  int64_t in_seg = o0 - g * SEG;
  int64_t r = uniform(find_segment_request(a.req_offsets, R, g, lane));
  int64_t cum = ro[r];
  int64_t n_r = ro[r + 1] - cum;
  int64_t local = g - 2 * cum;
  int64_t plane = local >= n_r ? 1 : 0;
  int64_t jj = local - plane * n_r;
  int64_t p = cum + jj;
  int64_t k_first = uniform(find_run(a.xfers, count, cum, lane));
  if (k_first < 0) k_first = 0;
  int64_t k = uniform(find_run(a.xfers, count, p, lane));
  if (k < 0) k = 0;
  Run x = load_run(xf, k);
  const char* idle = buf + o0;
  const char* sp[K];
  char* dp[K];
  bool on[K];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int64_t o = o0 + (int64_t)j * kWaveBytes;
    on[j] = false;
    sp[j] = idle;
    dp[j] = nullptr;
    if (o < layer_bytes && jj < n_r) {
      while (x.buf + x.n <= p && k + 1 < count) x = load_run(xf, ++k);
      if (p >= x.buf && p < x.buf + x.n) {
        const int64_t id = (TO_BUFFER ? x.src : x.dst) + (p - x.buf);
        if (id >= 0 && id < a.num_cache_blocks) {
          char* c = cache + plane * a.plane_stride + id * SEG + in_seg;
          char* b = buf + o;
          sp[j] = TO_BUFFER ? c : b;
          dp[j] = TO_BUFFER ? b : c;
          on[j] = true;
        } else {
          bad = true;
        }
      }
    }
    in_seg += kWaveBytes;
    if (in_seg == SEG) {
      in_seg = 0;
      ++jj;
      ++p;
      if (jj == n_r) {
        if (plane == 0) {  // V plane of the same request: restart its runs
          plane = 1;
          jj = 0;
          p = cum;
          k = k_first;
          x = load_run(xf, k);
        } else {           // next non-empty request: its first run follows this one
          while (r + 1 < R && ro[r + 2] == ro[r + 1]) ++r;
          if (r + 1 < R) {
            ++r;
            cum = ro[r];
            n_r = ro[r + 1] - cum;
            plane = 0;
            jj = 0;
            p = cum;
            if (k + 1 < count) ++k;
            k_first = k;
            x = load_run(xf, k);
          }
        }
      }
    }
  }
  u32x4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = load16<NTL>(sp[j] + lane * kVec);
#pragma unroll
  for (int j = 0; j < K; ++j)
    if (on[j]) store16<NTS>(dp[j] + lane * kVec, v[j]);
  if (bad && lane == 0) raise_error(a.err, KVX_DEVERR_BLOCK_RANGE);
}

// --------------------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------------------

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

hipError_t launch_slot_mapping(const int32_t* block_table, int64_t num_reqs, int64_t max_cols,
                               int64_t row_stride, const int32_t* req_idx,
                               const int64_t* positions, int64_t num_tokens, int32_t block_size,
                               int64_t* slots, int32_t* err, hipStream_t stream) {
  const int64_t wgs = ceil_div(num_tokens, 256);
  const unsigned grid = (unsigned)(wgs < (1 << 20) ? wgs : (1 << 20));
  slot_mapping_kernel<<<grid, 256, 0, stream>>>(block_table, num_reqs, max_cols, row_stride,
                                                req_idx, positions, num_tokens, block_size,
                                                slots, err);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, int64_t key_stride, const void* value,
                                    int64_t value_stride, int64_t num_tokens, int64_t row_bytes,
                                    const int64_t* slots, void* cache, int64_t num_blocks,
                                    int32_t block_size, int64_t block_stride,
                                    int64_t token_stride, int64_t kv_stride, int32_t* err,
                                    hipStream_t stream) {
  const int64_t total_slots = num_tokens * 2 * (row_bytes / kWaveBytes);
  if (row_bytes % kWaveBytes == 0 && tuning().one_batch &&
      ceil_div(ceil_div(total_slots, kWriteSlots), 4) < ((int64_t)1 << 31)) {
    WriteArgs a;
    a.key = (const char*)key;
    a.value = (const char*)value;
    a.slots = slots;
    a.cache = (char*)cache;
    a.err = err;
    a.key_stride = key_stride;
    a.value_stride = value_stride;
    a.num_tokens = num_tokens;
    a.row_bytes = row_bytes;
    a.num_blocks = num_blocks;
    a.block_stride = block_stride;
    a.token_stride = token_stride;
    a.kv_stride = kv_stride;
    a.total_slots = total_slots;
    a.block_size = block_size;
    const unsigned grid = (unsigned)ceil_div(ceil_div(total_slots, kWriteSlots), 4);
    switch (tuning().write_nt & 3) {
      case 0: write_slots_kernel<false, false><<<grid, 256, 0, stream>>>(a); break;
      case 1: write_slots_kernel<true, false><<<grid, 256, 0, stream>>>(a); break;
      case 2: write_slots_kernel<false, true><<<grid, 256, 0, stream>>>(a); break;
      default: write_slots_kernel<true, true><<<grid, 256, 0, stream>>>(a); break;
    }
    return hipGetLastError();
  }
  const int64_t vec_per_token = 2 * (row_bytes / kVec);
  if (num_tokens < tuning().write_vec_min || vec_per_token > (int64_t)kWriteSlots * kWave) {
    const int64_t wgs = ceil_div(num_tokens, 4);
    const unsigned grid = (unsigned)(wgs < (1 << 20) ? wgs : (1 << 20));
    write_tokens_kernel<4><<<grid, 256, 0, stream>>>(
        (const char*)key, key_stride, (const char*)value, value_stride, num_tokens, row_bytes,
        slots, (char*)cache, num_blocks, block_size, block_stride, token_stride, kv_stride, err);
    return hipGetLastError();
  }
  WriteArgs a;
  a.key = (const char*)key;
  a.value = (const char*)value;
  a.slots = slots;
  a.cache = (char*)cache;
  a.err = err;
  a.key_stride = key_stride;
  a.value_stride = value_stride;
  a.num_tokens = num_tokens;
  a.row_bytes = row_bytes;
  a.num_blocks = num_blocks;
  a.block_stride = block_stride;
  a.token_stride = token_stride;
  a.kv_stride = kv_stride;
  a.block_size = block_size;
  a.total_slots = 0;
  a.block_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  a.tokens_per_wave = (int32_t)(((int64_t)kWriteSlots * kWave) / vec_per_token);
  const int64_t wgs = ceil_div(ceil_div(num_tokens, (int64_t)a.tokens_per_wave), 4);
  if (wgs >= ((int64_t)1 << 31)) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)wgs;
  switch (tuning().write_nt & 3) {
    case 0: write_vectors_kernel<false, false><<<grid, 256, 0, stream>>>(a); break;
    case 1: write_vectors_kernel<true, false><<<grid, 256, 0, stream>>>(a); break;
    case 2: write_vectors_kernel<false, true><<<grid, 256, 0, stream>>>(a); break;
    default: write_vectors_kernel<true, true><<<grid, 256, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_build_xfer_list(const int32_t* src_ids, const int32_t* dst_ids,
                                  const int64_t* req_offsets, int32_t num_reqs,
                                  int64_t total_blocks, int32_t mode, kvx_xfer* xfers,
                                  int64_t* xfer_count, int32_t* err, hipStream_t stream) {
  // One workgroup per kScanTile positions up to kBuildMaxWgs workgroups; past that each
  // workgroup takes several sub-tiles, which keeps the prefix passes' total work within
  // kBuildMaxWgs / 2 reads per position.
  const int64_t tiles = total_blocks > 0 ? ceil_div(total_blocks, kScanTile) : 1;
  const int64_t wgs = tiles < kBuildMaxWgs ? tiles : kBuildMaxWgs;
  const int64_t span = ceil_div(tiles, wgs) * kScanTile;
  const int64_t grid = total_blocks > 0 ? ceil_div(total_blocks, span) : 1;
  build_xfer_kernel<<<(unsigned)grid, kScanThreads, 0, stream>>>(
      src_ids, dst_ids, req_offsets, num_reqs, total_blocks, mode, xfers, xfer_count, err, span);
  return hipGetLastError();
}

// Blocks per wavefront: about wave_bytes of buffer each, and few enough wavefronts that the
// grid stays well inside 32-bit workgroup counts.
static int64_t blocks_per_wave_for(int64_t wave_bytes, int64_t block_bytes, int64_t num_layers,
                                   int64_t N) {
  int64_t bpw = wave_bytes / block_bytes;
  if (bpw < 1) bpw = 1;
  const int64_t max_waves = (int64_t)1 << 30;
  const int64_t min_bpw = ceil_div(num_layers * N, max_waves);
  return bpw > min_bpw ? bpw : min_bpw;
}

// Runtime (cache policy, batch) -> template instance. LAUNCH(NTL, NTS, K) launches one.
#ifndef KVX_SMALL_BATCH
#define KVX_SMALL_BATCH 4
#endif
#define KVX_POLICY_SWITCH(NT, K, LAUNCH)                       \
  switch (((NT) & 3) * 2 + ((K) <= KVX_SMALL_BATCH ? 0 : 1)) { \
    case 0: LAUNCH(false, false, KVX_SMALL_BATCH) break;       \
    case 1: LAUNCH(false, false, 8) break;                     \
    case 2: LAUNCH(true, false, KVX_SMALL_BATCH) break;        \
    case 3: LAUNCH(true, false, 8) break;                      \
    case 4: LAUNCH(false, true, KVX_SMALL_BATCH) break;        \
    case 5: LAUNCH(false, true, 8) break;                      \
    case 6: LAUNCH(true, true, KVX_SMALL_BATCH) break;         \
    default: LAUNCH(true, true, 8) break;                      \
  }

// Batch of the one-batch kernels: 4 or 8 KiB per wavefront.
static int batch_of(const CopyTuning& ct) { return ct.batch <= KVX_SMALL_BATCH ? KVX_SMALL_BATCH : 8; }

// The one-batch fast path needs whole-KiB rows and a grid that fits 32-bit workgroup ids.
static bool use_slots(bool whole_kib, int64_t num_layers, int64_t layer_bytes, int64_t unit) {
  if (!whole_kib || !tuning().one_batch) return false;
  const int64_t waves = num_layers * ceil_div(layer_bytes, unit);
  return ceil_div(waves, kCopyWavesPerWg) < ((int64_t)1 << 31);
}

hipError_t launch_copy_runs(int dir, void* const* layer_bases, void* const* dst_layer_bases,
                            int32_t num_layers, int64_t block_bytes, int64_t num_cache_blocks,
                            int64_t dst_num_cache_blocks, const kvx_xfer* xfers,
                            const int64_t* xfer_count, int64_t total_blocks, void* buffer,
                            int32_t* err, hipStream_t stream, const SignalSpec* signal) {
  RunCopyArgs a;
  a.signal = signal ? signal->counter : nullptr;
  a.signal_delta = signal ? signal->delta : 0;
  a.arrivals = signal ? signal->arrivals : nullptr;
  a.layer_bases = (const char* const*)layer_bases;
  a.dst_layer_bases = (const char* const*)dst_layer_bases;
  a.buffer = (char*)buffer;
  a.xfers = xfers;
  a.xfer_count = xfer_count;
  a.err = err;
  a.block_bytes = block_bytes;
  a.num_cache_blocks = num_cache_blocks;
  a.dst_num_cache_blocks = dst_num_cache_blocks;
  a.total_blocks = total_blocks;
  const CopyTuning& ct = dir == kToBuffer ? tuning().pack
                         : dir == kFromBuffer ? tuning().unpack : tuning().direct;
  const int K = batch_of(ct);
  const int64_t unit = (int64_t)K * kWaveBytes;
  const bool slots = use_slots(block_bytes % kWaveBytes == 0, num_layers, total_blocks * block_bytes, unit);
  if (slots) {  // one K KiB batch per wavefront
    a.blocks_per_wave = 0;
    a.waves_per_layer = ceil_div(total_blocks * block_bytes, unit);
  } else {      // general path: whole blocks, about wave_bytes per wavefront
    a.blocks_per_wave = blocks_per_wave_for(ct.wave_bytes, block_bytes, num_layers, total_blocks);
    a.waves_per_layer = ceil_div(total_blocks, a.blocks_per_wave);
  }
  a.total_waves = a.waves_per_layer * num_layers;
  a.num_wgs = ceil_div(a.total_waves, kCopyWavesPerWg);
  a.num_layers = num_layers;
  a.xcd_remap = tuning().xcd_remap;
  if (signal && (dir == kFromBuffer || a.num_wgs > 0xffffffffll)) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)a.num_wgs;
#define KVX_COPY_DIR(D, SIG, NTL, NTS, KB)                                                        \
  if (slots) copy_slots_kernel<D, NTL, NTS, KB, SIG><<<grid, kCopyThreads, 0, stream>>>(a); \
  else copy_runs_kernel<D, NTL, NTS, SIG><<<grid, kCopyThreads, 0, stream>>>(a);
#define KVX_COPY_T(NTL, NTS, KB)                                 \
  if (signal) { KVX_COPY_DIR(kToBuffer, true, NTL, NTS, KB) }    \
  else { KVX_COPY_DIR(kToBuffer, false, NTL, NTS, KB) }
#define KVX_COPY_F(NTL, NTS, KB) KVX_COPY_DIR(kFromBuffer, false, NTL, NTS, KB)
#define KVX_COPY_X(NTL, NTS, KB)                                 \
  if (signal) { KVX_COPY_DIR(kDirect, true, NTL, NTS, KB) }      \
  else { KVX_COPY_DIR(kDirect, false, NTL, NTS, KB) }
  if (dir == kToBuffer) { KVX_POLICY_SWITCH(ct.nt_mode, K, KVX_COPY_T) }
  else if (dir == kFromBuffer) { KVX_POLICY_SWITCH(ct.nt_mode, K, KVX_COPY_F) }
  else { KVX_POLICY_SWITCH(ct.nt_mode, K, KVX_COPY_X) }
#undef KVX_COPY_DIR
#undef KVX_COPY_T
#undef KVX_COPY_F
#undef KVX_COPY_X
  return hipGetLastError();
}

hipError_t launch_shards(bool to_buffer, void* const* shards, int32_t num_shards,
                         void* const* layer_bases, int32_t num_layers, int64_t block_bytes,
                         int64_t num_cache_blocks, int32_t rows_per_block, const kvx_xfer* xfers,
                         const int64_t* xfer_count, int64_t total_blocks, int32_t* err,
                         hipStream_t stream) {
  ShardArgs a;
  for (int i = 0; i < KVX_MAX_SOURCES; ++i) a.shard[i] = i < num_shards ? (char*)shards[i] : nullptr;
  a.layer_bases = (const char* const*)layer_bases;
  a.xfers = xfers;
  a.xfer_count = xfer_count;
  a.err = err;
  a.block_bytes = block_bytes;
  a.num_cache_blocks = num_cache_blocks;
  a.total_blocks = total_blocks;
  a.row_piece = block_bytes / ((int64_t)rows_per_block * num_shards);
  const CopyTuning& ct = to_buffer ? tuning().split : tuning().merge;
  const int K = batch_of(ct);
  const int64_t unit = (int64_t)K * kWaveBytes;
  const bool slots = use_slots(a.row_piece % kWaveBytes == 0, num_layers, total_blocks * block_bytes, unit);
  if (slots) {
    a.blocks_per_wave = 0;
    a.waves_per_layer = ceil_div(total_blocks * block_bytes, unit);
  } else {
    a.blocks_per_wave = blocks_per_wave_for(ct.wave_bytes, block_bytes, num_layers, total_blocks);
    a.waves_per_layer = ceil_div(total_blocks, a.blocks_per_wave);
  }
  a.total_waves = a.waves_per_layer * num_layers;
  a.num_wgs = ceil_div(a.total_waves, kCopyWavesPerWg);
  a.num_shards = num_shards;
  a.rows_per_block = rows_per_block;
  a.num_layers = num_layers;
  // the split writes its shards faster without the renumbering (2.3-2.5% in A/B runs)
  a.xcd_remap = to_buffer ? tuning().xcd_remap_split : tuning().xcd_remap;
  const unsigned grid = (unsigned)a.num_wgs;
#define KVX_SHARD_T(NTL, NTS, KB)                                                           \
  if (slots) shard_slots_kernel<true, NTL, NTS, KB><<<grid, kCopyThreads, 0, stream>>>(a); \
  else shard_runs_kernel<true, NTL, NTS><<<grid, kCopyThreads, 0, stream>>>(a);
#define KVX_SHARD_F(NTL, NTS, KB)                                                            \
  if (slots) shard_slots_kernel<false, NTL, NTS, KB><<<grid, kCopyThreads, 0, stream>>>(a); \
  else shard_runs_kernel<false, NTL, NTS><<<grid, kCopyThreads, 0, stream>>>(a);
  if (to_buffer) { KVX_POLICY_SWITCH(ct.nt_mode, K, KVX_SHARD_T) }
  else { KVX_POLICY_SWITCH(ct.nt_mode, K, KVX_SHARD_F) }
#undef KVX_SHARD_T
#undef KVX_SHARD_F
  return hipGetLastError();
}

hipError_t launch_kv_first(bool to_buffer, void* const* layer_bases, int32_t num_layers,
                           int64_t segment_bytes, int64_t plane_stride, int64_t num_cache_blocks,
                           const int64_t* req_offsets, int32_t num_reqs, const kvx_xfer* xfers,
                           const int64_t* xfer_count, int64_t total_blocks, void* buffer,
                           int32_t* err, hipStream_t stream) {
  KvFirstArgs a;
  a.layer_bases = (const char* const*)layer_bases;
  a.buffer = (char*)buffer;
  a.xfers = xfers;
  a.xfer_count = xfer_count;
  a.req_offsets = req_offsets;
  a.err = err;
  a.segment_bytes = segment_bytes;
  a.plane_stride = plane_stride;
  a.num_cache_blocks = num_cache_blocks;
  a.total_blocks = total_blocks;
  const CopyTuning& ct = to_buffer ? tuning().kvf_pack : tuning().kvf_unpack;
  const int K = batch_of(ct);
  a.waves_per_layer = ceil_div(2 * total_blocks * segment_bytes, (int64_t)K * kWaveBytes);
  a.total_waves = a.waves_per_layer * num_layers;
  a.num_wgs = ceil_div(a.total_waves, kCopyWavesPerWg);
  if (a.num_wgs >= ((int64_t)1 << 31)) return hipErrorInvalidConfiguration;
  a.num_reqs = num_reqs;
  a.num_layers = num_layers;
  a.xcd_remap = tuning().xcd_remap;
  const unsigned grid = (unsigned)a.num_wgs;
#define KVX_KVF_T(NTL, NTS, KB) kv_first_kernel<true, NTL, NTS, KB><<<grid, kCopyThreads, 0, stream>>>(a);
#define KVX_KVF_F(NTL, NTS, KB) kv_first_kernel<false, NTL, NTS, KB><<<grid, kCopyThreads, 0, stream>>>(a);
  if (to_buffer) { KVX_POLICY_SWITCH(ct.nt_mode, K, KVX_KVF_T) }
  else { KVX_POLICY_SWITCH(ct.nt_mode, K, KVX_KVF_F) }
#undef KVX_KVF_T
#undef KVX_KVF_F
  return hipGetLastError();
}

#undef KVX_POLICY_SWITCH

}  // namespace kvx
