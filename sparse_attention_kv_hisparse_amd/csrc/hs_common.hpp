// Shared pieces of the gfx950 HiSparse kernels: the copy engine's 16-byte /
// 4-byte chunk movers, exact division by a run-time constant, and host-side
// status/error helpers. Everything here is integer or opaque bytes.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "hisparse.h"

namespace hs {

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------------------
// Exact unsigned division by a run-time divisor d for numerators n < 2^31:
// q = (n * m) >> s with s = 31 + ceil(log2 d) and m = ceil(2^s / d).
// m < 2^33 so n*m < 2^64, and the rounding error n*(m*d - 2^s)/(d*2^s) stays
// below 1/d, so the quotient is exact (round-up reciprocal method).
// ---------------------------------------------------------------------------
struct FastDiv {
  uint32_t d;
  uint32_t s;
  uint64_t m;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint32_t s = 31 + l;
  const uint64_t m = ((1ull << s) + d - 1) / d;
  return FastDiv{d, s, m};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> f.s);
}

// ---------------------------------------------------------------------------
// Copy engine: rows are moved as independent 16-byte (or 4-byte) chunks, one
// per lane, with consecutive lanes on consecutive chunks of a row so a wave's
// accesses coalesce. Loads are nontemporal: pool rows are read once, and on
// gfx950 with cold caches nontemporal loads beat cached ones by ~30% on
// scattered 656-byte rows (cached loads allocate lines that then have to be
// evicted). Stores are ordinary write-back stores: a row that ends inside a
// 128-byte line leaves a partial line, which in L2 can merge with the
// neighbouring row's write (or be written back as one unit) instead of
// reaching HBM as a partial write. Measured against nontemporal stores on the
// device-pool decode step: 33.5 -> 29.5 us per copy launch, with every other
// copy (host pool, all-layer, scatter) the same or faster.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

template <int W>
struct Chunk;

template <>
struct Chunk<16> {
  typedef u32x4 T;
  static __device__ __forceinline__ T load(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  static __device__ __forceinline__ void store(char* p, T v) { *reinterpret_cast<u32x4*>(p) = v; }
};

template <>
struct Chunk<4> {
  typedef uint32_t T;
  static __device__ __forceinline__ T load(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
  static __device__ __forceinline__ void store(char* p, T v) { *reinterpret_cast<uint32_t*>(p) = v; }
};

// s_waitcnt immediate for vmcnt(0) alone: vmcnt bits [3:0] and [15:14] zero,
// expcnt [6:4] and lgkmcnt [11:8] at their no-wait maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

// Lanes with nothing to store in a branch-free round write a private 16-byte
// slot here instead. One slot per lane of a workgroup of up to 1024; the
// slots hold garbage and are never read.
namespace {
__device__ __align__(16) u32x4 g_store_sink[1024];
}
__device__ __forceinline__ char* store_sink() { return reinterpret_cast<char*>(&g_store_sink[threadIdx.x]); }

// Chunks a row of `row_bytes` splits into at width W.
inline int64_t chunks_per_row(int64_t row_bytes, int W) { return row_bytes / W; }

// ---------------------------------------------------------------------------
// Host helpers.
// ---------------------------------------------------------------------------
int set_error(int status, const char* fmt, ...);

// Largest dynamic LDS (bytes) one workgroup may use on the current device, and
// the compute-unit count; cached per device.
struct DeviceInfo {
  int device;
  int max_lds;
  int num_cus;
};
int device_info(DeviceInfo* out);

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace hs
