// Copy half of the swap-in: moves the rows a resolve published as a compact
// miss list (count[b], then (pool row, hot row) pairs in miss order) from the
// pool to the hot buffer. SGLang hisparse.cuh copies inside the resolving
// block and vLLM hisparse_kernels.cu runs hisparse_gather_compact_kernel over
// the same kind of list; here the list is copied by many 256-lane workgroups
// per request as one flat stream of W-byte chunks.
#pragma once

#include <hip/hip_runtime.h>

#include "hs_common.hpp"

namespace hs {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 8;  // chunks in flight per copy lane

// One miss list and the two row spaces it indexes.
struct MissList {
  const int32_t* count;  // [B] misses of request b
  const int64_t* src;    // [B, K] pool row of miss m
  const int32_t* dst;    // [B, K] hot row of miss m (outside [0, hot_nrows) = skip)
  const char* pool;      // device-visible address of the pool
  char* hot;
  int64_t hot_nrows;
  int64_t row_bytes;
  int32_t B, K;
  FastDiv cdiv;          // chunks per row
};

// Workgroup g serves request g % B, part g / B of `parts`. Consecutive lanes
// take consecutive chunks of a row, so each wave's accesses coalesce, and
// every lane keeps kCopyUnroll independent loads in flight.
template <int W>
__global__ __launch_bounds__(kCopyThreads) void swap_copy_kernel(MissList a, int32_t parts) {
  typedef Chunk<W> C;
  const int b = blockIdx.x % a.B;
  const int part = blockIdx.x / a.B;
  const int M = a.count[b];
  const uint32_t total = static_cast<uint32_t>(M) * a.cdiv.d;
  const int64_t* src = a.src + static_cast<int64_t>(b) * a.K;
  const int32_t* dst = a.dst + static_cast<int64_t>(b) * a.K;
  const uint32_t stride = static_cast<uint32_t>(parts) * kCopyThreads;
  for (uint32_t j0 = static_cast<uint32_t>(part) * kCopyThreads + threadIdx.x; j0 < total;
       j0 += stride * kCopyUnroll) {
    typename C::T v[kCopyUnroll];
    char* d[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint32_t j = j0 + u * stride;
      d[u] = nullptr;
      if (j < total) {
        const uint32_t m = fdiv(j, a.cdiv);
        const uint32_t c = j - m * a.cdiv.d;
        const int32_t hr = dst[m];
        if (hr >= 0 && hr < a.hot_nrows) {
          const int64_t off = static_cast<int64_t>(c) * W;
          v[u] = C::load(a.pool + src[m] * a.row_bytes + off);
          d[u] = a.hot + static_cast<int64_t>(hr) * a.row_bytes + off;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (d[u]) C::store(d[u], v[u]);
  }
}

// Grid: enough workgroups per request to cover its worst case (all K ids
// missing) at kCopyUnroll chunks per lane, capped at 8 per CU overall.
// W is 16 when pool, hot and row_bytes are 16-byte aligned, else 4.
inline int launch_swap_copy(const MissList& a, int W, int num_cus, hipStream_t stream) {
  const int64_t max_items = static_cast<int64_t>(a.K) * a.cdiv.d;
  int64_t parts = (max_items + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll);
  const int64_t cap = (8LL * num_cus + a.B - 1) / a.B;
  if (parts > cap) parts = cap;
  if (parts < 1) parts = 1;
  const dim3 grid(static_cast<unsigned>(a.B * parts));
  if (W == 16)
    hipLaunchKernelGGL(swap_copy_kernel<16>, grid, dim3(kCopyThreads), 0, stream, a,
                       static_cast<int32_t>(parts));
  else
    hipLaunchKernelGGL(swap_copy_kernel<4>, grid, dim3(kCopyThreads), 0, stream, a,
                       static_cast<int32_t>(parts));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(HS_ELAUNCH, "copy launch: %s", hipGetErrorString(e));
  return HS_OK;
}

}  // namespace
}  // namespace hs
