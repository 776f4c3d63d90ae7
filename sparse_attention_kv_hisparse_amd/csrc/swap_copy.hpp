// Copy half of the swap-in: moves the rows a resolve published as a compact
// miss list (count[b], then (pool row, hot row) pairs in miss order) from the
// pool to the hot buffer, on one (pool, hot) pair or replayed on several
// layers that share the plan. SGLang hisparse.cuh copies inside the resolving
// block; vLLM hisparse_kernels.cu runs hisparse_gather_compact_kernel over the
// same kind of list and hisparse_gather_plan_kernel for index-sharing layers.
// Here the list is copied by many 256-lane workgroups per request as one flat
// stream of W-byte chunks.
//
// Per entry (vLLM hisparse_gather_compact_kernel): the count is clamped to
// [0, K]; an entry with a negative pool row or a hot row outside the hot
// buffer is skipped; a pool row at or past the end of the pool zeroes the hot
// row instead of leaving stale bytes.
#pragma once

#include <hip/hip_runtime.h>

#include "hs_common.hpp"

namespace hs {
namespace {

constexpr int kCopyThreads = 256;       // lanes per copy workgroup: host pools, plan replay
constexpr int kCopyThreadsHbm = 1024;   // ... single pair from an HBM pool
constexpr int kCopyUnroll = 8;        // chunks per copy lane per round
constexpr int kMaxStagedPairs = 256;  // layer pointer pairs staged in LDS

// One miss list and the row spaces it indexes.
struct MissList {
  const int32_t* count;  // [B] misses of request b
  const int64_t* src;    // [B, K] pool row of miss m
  const int32_t* dst;    // [B, K] hot row of miss m
  const char* pool;      // device-visible address of the pool (single pair)
  char* hot;             // (single pair)
  const char* pool_v;    // non-MLA caches: the V pool and V hot buffer (same
  char* hot_v;           // geometry), or null; each miss then moves two rows
  const uint64_t* pool_layers;  // [layers] pool bases (layered replay)
  const uint64_t* hot_layers;   // [layers] hot bases (layered replay)
  int64_t pool_nrows;
  int64_t hot_nrows;
  int64_t row_bytes;
  int32_t B, K;
  int32_t layers;        // 1 for a single pair
  FastDiv cdiv;          // chunks per row
  FastDiv ldiv;          // layers
};

// Workgroup g serves request g % B, part g / B of `parts`. Items are
// (miss, layer, chunk) -- or (miss, K/V, chunk) for a single non-MLA pair --
// with the chunk fastest: consecutive lanes take consecutive chunks of one
// row, so each wave's accesses coalesce. A lane takes kCopyUnroll chunks per
// round; the generated code reads them one after another (it waits for each
// list entry, and so for every earlier access), and the waves of a full chip
// keep HBM busy. Rewrites with every read of a round in flight measured
// slower here, in HBM and over the host link alike.
template <int W, bool kLayers, int kT>
__global__ __launch_bounds__(kT) void swap_copy_kernel(MissList a, int32_t parts) {
  typedef Chunk<W> C;
  __shared__ uint64_t s_pool[kLayers ? kMaxStagedPairs : 1];
  __shared__ uint64_t s_hot[kLayers ? kMaxStagedPairs : 1];
  const bool staged = kLayers && a.layers <= kMaxStagedPairs;
  if (staged) {
    for (int l = threadIdx.x; l < a.layers; l += kT) {
      s_pool[l] = a.pool_layers[l];
      s_hot[l] = a.hot_layers[l];
    }
    __syncthreads();
  }
  const int b = blockIdx.x % a.B;
  const int part = blockIdx.x / a.B;
  int M = a.count[b];
  M = M < 0 ? 0 : (M > a.K ? a.K : M);
  const bool kv = !kLayers && a.pool_v != nullptr;   // uniform
  const uint32_t per_miss = (kLayers ? static_cast<uint32_t>(a.layers) : (kv ? 2u : 1u)) * a.cdiv.d;
  const uint32_t total = static_cast<uint32_t>(M) * per_miss;
  const int64_t* src = a.src + static_cast<int64_t>(b) * a.K;
  const int32_t* dst = a.dst + static_cast<int64_t>(b) * a.K;
  const uint32_t stride = static_cast<uint32_t>(parts) * kT;
  for (uint32_t j0 = static_cast<uint32_t>(part) * kT + threadIdx.x; j0 < total;
       j0 += stride * kCopyUnroll) {
    typename C::T v[kCopyUnroll];
    char* d[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const uint32_t j = j0 + u * stride;
      d[u] = nullptr;
      if (j < total) {
        const uint32_t q = fdiv(j, a.cdiv);          // (miss, layer) row
        const uint32_t c = j - q * a.cdiv.d;        // chunk in the row
        uint32_t m = q, l = 0;
        if (kLayers) {
          m = fdiv(q, a.ldiv);
          l = q - m * a.ldiv.d;
        } else if (kv) {
          m = q >> 1;
          l = q & 1;
        }
        const int64_t s = src[m];
        const int32_t hr = dst[m];
        if (s >= 0 && hr >= 0 && hr < a.hot_nrows) {
          const char* pbase = l ? a.pool_v : a.pool;
          char* hbase = l ? a.hot_v : a.hot;
          if (kLayers) {
            pbase = reinterpret_cast<const char*>(staged ? s_pool[l] : a.pool_layers[l]);
            hbase = reinterpret_cast<char*>(staged ? s_hot[l] : a.hot_layers[l]);
          }
          const int64_t off = static_cast<int64_t>(c) * W;
          char* to = hbase + static_cast<int64_t>(hr) * a.row_bytes + off;
          const char* from = pbase + s * a.row_bytes + off;
          const bool has = s < a.pool_nrows;
          if (W == 16 && kLayers &&
              ((reinterpret_cast<uintptr_t>(pbase) | reinterpret_cast<uintptr_t>(hbase)) & 15)) {
            // A layer base that is only 4-byte aligned: move this chunk as dwords.
#pragma unroll
            for (int k = 0; k < W; k += 4) Chunk<4>::store(to + k, has ? Chunk<4>::load(from + k) : 0u);
          } else {
            v[u] = has ? C::load(from) : typename C::T{};
            d[u] = to;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (d[u]) C::store(d[u], v[u]);
  }
}

// Lanes per CU at most: HBM wants many loads in flight; the host link does
// better with fewer requesters (a pinned-host pool copied with one 256-lane
// workgroup per CU takes ~11% less time than with eight, measured on the
// DeepSeek-V3.2-like decode step). From an HBM pool the same 2048 lanes per CU
// run as two 1024-lane workgroups: ~1.5% faster than eight of 256.
constexpr int kCopyLanesPerCu = 2048;
constexpr int kHostCopyLanesPerCu = 256;

// Grid: enough workgroups per request to cover its worst case (all K ids
// missing, every layer) at kCopyUnroll chunks per lane, capped per CU
// overall. W is 16 when the bases and row_bytes are 16-byte aligned, else 4.
inline int launch_swap_copy(const MissList& a, int W, int num_cus, hipStream_t stream,
                            bool host_pool = false) {
  const bool layered = a.pool_layers != nullptr;
  const bool wide = !layered && !host_pool;   // 1024-lane workgroups
  const int64_t T = wide ? kCopyThreadsHbm : kCopyThreads;
  const int64_t streams = layered ? a.layers : (a.pool_v ? 2 : 1);
  const int64_t max_items = static_cast<int64_t>(a.K) * streams * a.cdiv.d;
  int64_t parts = (max_items + T * kCopyUnroll - 1) / (T * kCopyUnroll);
  const int64_t per_cu = (host_pool ? kHostCopyLanesPerCu : kCopyLanesPerCu) / T;
  const int64_t cap = (per_cu * num_cus + a.B - 1) / a.B;
  if (parts > cap) parts = cap;
  if (parts < 1) parts = 1;
  const dim3 grid(static_cast<unsigned>(a.B * parts));
  const int32_t p = static_cast<int32_t>(parts);
  const dim3 block(static_cast<unsigned>(T));
  if (W == 16) {
    if (layered)
      hipLaunchKernelGGL((swap_copy_kernel<16, true, kCopyThreads>), grid, block, 0, stream, a, p);
    else if (wide)
      hipLaunchKernelGGL((swap_copy_kernel<16, false, kCopyThreadsHbm>), grid, block, 0, stream, a, p);
    else
      hipLaunchKernelGGL((swap_copy_kernel<16, false, kCopyThreads>), grid, block, 0, stream, a, p);
  } else {
    if (layered)
      hipLaunchKernelGGL((swap_copy_kernel<4, true, kCopyThreads>), grid, block, 0, stream, a, p);
    else if (wide)
      hipLaunchKernelGGL((swap_copy_kernel<4, false, kCopyThreadsHbm>), grid, block, 0, stream, a, p);
    else
      hipLaunchKernelGGL((swap_copy_kernel<4, false, kCopyThreads>), grid, block, 0, stream, a, p);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(HS_ELAUNCH, "copy launch: %s", hipGetErrorString(e));
  return HS_OK;
}

}  // namespace
}  // namespace hs
