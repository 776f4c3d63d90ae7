// Indexed row copies that share the swap-in's copy engine:
//   transfer_rows_all_layer -- tokenspeed kvcache/triton.py,
//     _kv_transfer_all_layer_mla_kernel; SGLang hisparse.cuh,
//     transfer_cache_dsv4_mla_kernel (generic row layout);
//   transfer_kv_all_layer -- tokenspeed, _kv_transfer_all_layer_kernel (K and
//     V caches of every layer);
//   store_kv_scatter / store_kv_cache -- tokenspeed, _store_kv_cache_kernel
//     (K half / both halves);
//   hisparse_state_reset -- initial per-request state.
//
// Work is one flat stream of (pair, layer, chunk) items rather than one warp
// per item looping over layers: every lane moves one 16-byte chunk, lanes of a
// wave cover consecutive chunks of consecutive rows, and a grid-stride loop
// takes several chunks per lane per round. In the transfer the generated code
// waits for each read before the next, so the waves in flight, not the
// unroll, keep bytes outstanding; that form measured best on the host link
// and in HBM. The scatter, with too few rows to fill the chip, issues all of
// a round's reads before its stores.
#include <hip/hip_runtime.h>

#include "hs_common.hpp"

namespace hs {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;          // chunks per lane per round, HBM-sized launches
constexpr int kHostLinkUnroll = 8;  // ... and with HS_TRANSFER_HOST_LINK
constexpr int kMaxStagedLayers = 256;

// Layer bases: streams [0, lk) come from the K arrays, [lk, num_layers) from
// the V arrays (null for MLA, where num_layers == lk).
struct LayerPtrs {
  const uint64_t* src_k;
  const uint64_t* dst_k;
  const uint64_t* src_v;
  const uint64_t* dst_v;
  int32_t lk;
};

template <int W, int U>
__global__ __launch_bounds__(kThreads) void transfer_kernel(
    LayerPtrs lp, const int64_t* __restrict__ src_idx, const int64_t* __restrict__ dst_idx,
    uint32_t total, int32_t num_layers, int64_t row_bytes, int64_t src_nrows, int64_t dst_nrows,
    FastDiv cdiv, FastDiv ldiv) {
  typedef Chunk<W> C;
  __shared__ uint64_t s_src[kMaxStagedLayers];
  __shared__ uint64_t s_dst[kMaxStagedLayers];
  const bool staged = num_layers <= kMaxStagedLayers;
  auto src_base = [&](int l) { return l < lp.lk ? lp.src_k[l] : lp.src_v[l - lp.lk]; };
  auto dst_base = [&](int l) { return l < lp.lk ? lp.dst_k[l] : lp.dst_v[l - lp.lk]; };
  if (staged) {
    for (int l = threadIdx.x; l < num_layers; l += kThreads) {
      s_src[l] = src_base(l);
      s_dst[l] = dst_base(l);
    }
    __syncthreads();
  }
  const uint32_t step = gridDim.x * kThreads * U;
  for (uint32_t j0 = blockIdx.x * kThreads * U + threadIdx.x; j0 < total; j0 += step) {
    typename C::T v[U];
    char* d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t j = j0 + u * kThreads;
      d[u] = nullptr;
      if (j < total) {
        const uint32_t row = fdiv(j, cdiv);          // (pair, layer) row
        const uint32_t c = j - row * cdiv.d;        // chunk in the row
        const uint32_t i = fdiv(row, ldiv);          // pair
        const uint32_t l = row - i * ldiv.d;        // layer
        const int64_t si = src_idx[i], di = dst_idx[i];
        if (si >= 0 && si < src_nrows && di >= 0 && di < dst_nrows) {
          const uint64_t sb = staged ? s_src[l] : src_base(static_cast<int>(l));
          const uint64_t db = staged ? s_dst[l] : dst_base(static_cast<int>(l));
          const int64_t off = static_cast<int64_t>(c) * W;
          const char* sp = reinterpret_cast<const char*>(sb) + si * row_bytes + off;
          char* dp = reinterpret_cast<char*>(db) + di * row_bytes + off;
          if (W == 4 || ((sb | db) & 15) == 0) {
            v[u] = C::load(sp);
            d[u] = dp;
          } else {
            // A layer base that is only 4-byte aligned: move this chunk as dwords.
#pragma unroll
            for (int k = 0; k < W; k += 4) Chunk<4>::store(dp + k, Chunk<4>::load(sp + k));
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (d[u]) C::store(d[u], v[u]);
  }
}

// One scatter stream: rows of a source (leading-axis stride in bytes) go to
// the destination rows loc[j].
struct ScatterSide {
  const char* src;
  int64_t src_stride;
  char* dst;
  int64_t dst_stride;
};

// Items are (entry, stream, chunk) with the chunk fastest; with a V side each
// entry has two streams, K then V (tokenspeed _store_kv_cache_kernel moves
// both halves in one launch).
template <int W>
__global__ __launch_bounds__(kThreads) void scatter_kernel(ScatterSide k, ScatterSide v, bool kv,
                                                           int64_t dst_nrows,
                                                           const int64_t* __restrict__ loc,
                                                           uint32_t total, FastDiv cdiv) {
  typedef Chunk<W> C;
  const uint32_t step = gridDim.x * kThreads * kUnroll;
  for (uint32_t j0 = blockIdx.x * kThreads * kUnroll + threadIdx.x; j0 < total; j0 += step) {
    // A round: every load of the round in flight at once, then the stores,
    // with no branch in front of them (a lane with nothing to store writes its
    // sink slot). The wait on entry tells the compiler the previous round is
    // done; without it, and with the stores behind branches, it waits for
    // every earlier access before each load and store, one row at a time.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    typename C::T val[kUnroll];
    int64_t to[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t j = j0 + u * kThreads;
      const uint32_t jj = j < total ? j : j0;
      const uint32_t q = fdiv(jj, cdiv);
      const uint32_t c = jj - q * cdiv.d;
      const uint32_t row = kv ? q >> 1 : q;
      // Field by field: a per-lane choice of a whole argument struct would be
      // read from the argument segment with vector loads.
      const bool isv = kv && (q & 1);
      const char* sbase = isv ? v.src : k.src;
      const int64_t sstride = isv ? v.src_stride : k.src_stride;
      // The source row is always in range (row < n): its load does not wait
      // for loc, so the two loads are in flight together.
      val[u] = C::load(sbase + static_cast<int64_t>(row) * sstride + static_cast<int64_t>(c) * W);
      to[u] = loc[row];
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before any use
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t j = j0 + u * kThreads;
      const uint32_t jj = j < total ? j : j0;
      const uint32_t q = fdiv(jj, cdiv);
      const uint32_t c = jj - q * cdiv.d;
      const bool isv = kv && (q & 1);
      char* dbase = isv ? v.dst : k.dst;
      const int64_t dstride = isv ? v.dst_stride : k.dst_stride;
      const bool ok = j < total && to[u] >= 0 && to[u] < dst_nrows;
      C::store(ok ? dbase + to[u] * dstride + static_cast<int64_t>(c) * W : store_sink(), val[u]);
    }
  }
}

__global__ __launch_bounds__(kThreads) void state_reset_kernel(int32_t* slot_tokens, int16_t* lru,
                                                               const int64_t* rows, int32_t H,
                                                               int64_t S_r, int64_t R) {
  const int64_t r = rows[blockIdx.x];
  if (r < 0 || r >= R) return;
  for (int64_t s = threadIdx.x; s < S_r; s += kThreads) slot_tokens[r * S_r + s] = -1;
  for (int32_t p = threadIdx.x; p < H; p += kThreads) lru[r * H + p] = static_cast<int16_t>(p);
}

// Write invalidation (vLLM hisparse_invalidate_written_slots_kernel): the
// workgroup of written entry j clears every slot of state row rows[j] whose
// key is the rewritten global row written[j]. Different keys never share a
// slot, so concurrent entries touch disjoint words.
__global__ __launch_bounds__(kThreads) void invalidate_kernel(int32_t* keys, int64_t R, int64_t S_r,
                                                              const int64_t* rows,
                                                              const int64_t* written, int64_t n) {
  for (int64_t j = blockIdx.x; j < n; j += gridDim.x) {
    const int64_t r = rows[j], g = written[j];
    if (r < 0 || r >= R || g < 0) continue;
    int32_t* row = keys + r * S_r;
    for (int64_t s = threadIdx.x; s < S_r; s += kThreads)
      if (static_cast<int64_t>(row[s]) == g) row[s] = -1;
  }
}

// Workgroups for a grid-stride copy of `items` chunks: enough to fill every
// CU several times over, never more than the work needs.
inline unsigned copy_grid(uint64_t items, int num_cus) {
  const uint64_t need = (items + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  const uint64_t cap = 16ull * static_cast<uint64_t>(num_cus > 0 ? num_cus : 256);
  return static_cast<unsigned>(need < cap ? (need > 0 ? need : 1) : cap);
}

}  // namespace
}  // namespace hs

using namespace hs;

namespace {

// Shared host side of both all-layer transfers: lp.lk layers of K, and as many
// of V when lp.src_v is set.
int launch_transfer(const LayerPtrs& lp, const int64_t* src_idx, const int64_t* dst_idx, int64_t n,
                    int32_t num_layers, int64_t row_bytes, int64_t src_nrows, int64_t dst_nrows,
                    uint32_t flags, hipStream_t stream) {
  if (flags & ~HS_TRANSFER_HOST_LINK) return set_error(HS_EINVAL, "unknown flags 0x%x", flags);
  if (n < 0 || num_layers < 0) return set_error(HS_EINVAL, "n and num_layers must be >= 0");
  if (n == 0 || num_layers == 0) return HS_OK;
  if (!lp.src_k || !lp.dst_k || !src_idx || !dst_idx || (lp.src_v && !lp.dst_v))
    return set_error(HS_EINVAL, "a required pointer is NULL");
  if (row_bytes <= 0 || (row_bytes & 3) != 0)
    return set_error(HS_EINVAL, "row_bytes=%lld must be a positive multiple of 4", (long long)row_bytes);
  if (row_bytes > (1ll << 20)) return set_error(HS_ERANGE, "row_bytes above 1 MiB");
  if (src_nrows < 0 || dst_nrows < 0) return set_error(HS_EINVAL, "row counts must be >= 0");
  if (num_layers > (1 << 24)) return set_error(HS_ERANGE, "too many layers");
  const int32_t streams = lp.src_v ? 2 * num_layers : num_layers;
  const bool host_link = (flags & HS_TRANSFER_HOST_LINK) != 0;
  // Layer base addresses live on the device; rows are 16-byte chunks when
  // row_bytes allows (a base that is only 4-byte aligned is moved as dwords
  // by the kernel).
  const int W = (row_bytes & 15) == 0 ? 16 : 4;
  const int64_t C = row_bytes / W;
  DeviceInfo di;
  int rc = device_info(&di);
  if (rc != HS_OK) return rc;
  const FastDiv cdiv = make_fastdiv(static_cast<uint32_t>(C));
  const FastDiv ldiv = make_fastdiv(static_cast<uint32_t>(streams));
  // Items must stay below 2^31 per launch: split the pairs into batches.
  const int64_t per_pair = C * streams;
  const int64_t max_pairs = ((1ll << 30) / per_pair) > 0 ? ((1ll << 30) / per_pair) : 0;
  if (max_pairs == 0) return set_error(HS_ERANGE, "one pair spans more than 2^30 chunks");
  for (int64_t p0 = 0; p0 < n; p0 += max_pairs) {
    const int64_t np = (n - p0) < max_pairs ? (n - p0) : max_pairs;
    const uint32_t total = static_cast<uint32_t>(np * per_pair);
    if (host_link) {
      // The host link is full with far fewer requesters than HBM needs:
      // one workgroup per two CUs, 8 chunks per lane per round (all-layer
      // load of 656-byte rows: 44.7 -> 47.7 GB/s against the HBM-sized
      // launch; offload 51.9 -> 51.7).
      const uint64_t need = (total + kThreads * kHostLinkUnroll - 1) / (kThreads * kHostLinkUnroll);
      const uint64_t cap = di.num_cus > 1 ? static_cast<uint64_t>(di.num_cus) / 2 : 1;
      const unsigned grid = static_cast<unsigned>(need < cap ? (need > 0 ? need : 1) : cap);
      if (W == 16)
        hipLaunchKernelGGL((transfer_kernel<16, kHostLinkUnroll>), dim3(grid), dim3(kThreads), 0,
                           stream, lp, src_idx + p0, dst_idx + p0, total, streams, row_bytes,
                           src_nrows, dst_nrows, cdiv, ldiv);
      else
        hipLaunchKernelGGL((transfer_kernel<4, kHostLinkUnroll>), dim3(grid), dim3(kThreads), 0,
                           stream, lp, src_idx + p0, dst_idx + p0, total, streams, row_bytes,
                           src_nrows, dst_nrows, cdiv, ldiv);
    } else {
      const unsigned grid = copy_grid(total, di.num_cus);
      if (W == 16)
        hipLaunchKernelGGL((transfer_kernel<16, kUnroll>), dim3(grid), dim3(kThreads), 0, stream,
                           lp, src_idx + p0, dst_idx + p0, total, streams, row_bytes, src_nrows,
                           dst_nrows, cdiv, ldiv);
      else
        hipLaunchKernelGGL((transfer_kernel<4, kUnroll>), dim3(grid), dim3(kThreads), 0, stream,
                           lp, src_idx + p0, dst_idx + p0, total, streams, row_bytes, src_nrows,
                           dst_nrows, cdiv, ldiv);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(HS_ELAUNCH, "transfer launch: %s", hipGetErrorString(e));
  }
  return HS_OK;
}

bool side_ok(const ScatterSide& sd, int64_t row_bytes) {
  return sd.src_stride >= row_bytes && sd.dst_stride >= row_bytes && (sd.src_stride & 3) == 0 &&
         (sd.dst_stride & 3) == 0 && aligned(sd.src, 4) && aligned(sd.dst, 4);
}

bool side_w16(const ScatterSide& sd) {
  return aligned(sd.src, 16) && aligned(sd.dst, 16) && (sd.src_stride & 15) == 0 &&
         (sd.dst_stride & 15) == 0;
}

int launch_scatter(const ScatterSide& k, const ScatterSide* v, int64_t dst_nrows, const int64_t* loc,
                   int64_t n, int64_t row_bytes, hipStream_t stream) {
  if (n < 0) return set_error(HS_EINVAL, "n must be >= 0");
  if (n == 0) return HS_OK;
  if (!k.src || !k.dst || !loc || (v && (!v->src || !v->dst)))
    return set_error(HS_EINVAL, "a required pointer is NULL");
  if (row_bytes <= 0 || (row_bytes & 3) != 0)
    return set_error(HS_EINVAL, "row_bytes=%lld must be a positive multiple of 4", (long long)row_bytes);
  if (row_bytes > (1ll << 20)) return set_error(HS_ERANGE, "row_bytes above 1 MiB");
  if (!side_ok(k, row_bytes) || (v && !side_ok(*v, row_bytes)))
    return set_error(HS_EINVAL,
                     "row strides must be >= row_bytes and multiples of 4, bases 4-byte aligned");
  if (dst_nrows < 0) return set_error(HS_EINVAL, "dst_nrows must be >= 0");
  const bool w16 = (row_bytes & 15) == 0 && side_w16(k) && (!v || side_w16(*v));
  const int W = w16 ? 16 : 4;
  const int64_t C = row_bytes / W;
  const int64_t streams = v ? 2 : 1;
  if (n * C * streams >= (1ll << 31)) return set_error(HS_ERANGE, "n * chunks per entry exceeds 2^31");
  DeviceInfo di;
  int rc = device_info(&di);
  if (rc != HS_OK) return rc;
  const uint32_t total = static_cast<uint32_t>(n * C * streams);
  const FastDiv cdiv = make_fastdiv(static_cast<uint32_t>(C));
  const unsigned grid = copy_grid(total, di.num_cus);
  const ScatterSide vv = v ? *v : k;
  if (W == 16)
    hipLaunchKernelGGL(scatter_kernel<16>, dim3(grid), dim3(kThreads), 0, stream, k, vv, v != nullptr,
                       dst_nrows, loc, total, cdiv);
  else
    hipLaunchKernelGGL(scatter_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, k, vv, v != nullptr,
                       dst_nrows, loc, total, cdiv);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(HS_ELAUNCH, "scatter launch: %s", hipGetErrorString(e));
  return HS_OK;
}

}  // namespace

extern "C" int transfer_rows_all_layer(const uint64_t* src_layer_ptrs, const uint64_t* dst_layer_ptrs,
                                       const int64_t* src_idx, const int64_t* dst_idx, int64_t n,
                                       int32_t num_layers, int64_t row_bytes, int64_t src_nrows,
                                       int64_t dst_nrows, uint32_t flags, hipStream_t stream) {
  const LayerPtrs lp{src_layer_ptrs, dst_layer_ptrs, nullptr, nullptr, num_layers};
  return launch_transfer(lp, src_idx, dst_idx, n, num_layers, row_bytes, src_nrows, dst_nrows,
                         flags, stream);
}

extern "C" int transfer_kv_all_layer(const uint64_t* k_src_layer_ptrs,
                                     const uint64_t* v_src_layer_ptrs,
                                     const uint64_t* k_dst_layer_ptrs,
                                     const uint64_t* v_dst_layer_ptrs, const int64_t* src_idx,
                                     const int64_t* dst_idx, int64_t n, int32_t num_layers,
                                     int64_t row_bytes, int64_t src_nrows, int64_t dst_nrows,
                                     uint32_t flags, hipStream_t stream) {
  if (flags & ~HS_TRANSFER_HOST_LINK) return set_error(HS_EINVAL, "unknown flags 0x%x", flags);
  if (!v_src_layer_ptrs || !v_dst_layer_ptrs) {
    if (n == 0 || num_layers == 0) return HS_OK;
    return set_error(HS_EINVAL, "a required pointer is NULL");
  }
  const LayerPtrs lp{k_src_layer_ptrs, k_dst_layer_ptrs, v_src_layer_ptrs, v_dst_layer_ptrs,
                     num_layers};
  return launch_transfer(lp, src_idx, dst_idx, n, num_layers, row_bytes, src_nrows, dst_nrows,
                         flags, stream);
}

extern "C" int hs_transfer_flags_for(const void* src_layer, const void* dst_layer, uint32_t* flags) {
  if (!src_layer || !dst_layer || !flags) return set_error(HS_EINVAL, "a required pointer is NULL");
  bool host = false;
  for (const void* p : {src_layer, dst_layer}) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(HS_EMEMKIND, "a layer base is not a HIP allocation (device or pinned host)");
    }
    if (attr.type == hipMemoryTypeHost) host = true;
    else if (attr.type != hipMemoryTypeDevice)
      return set_error(HS_EMEMKIND, "a layer base must be device memory or pinned host memory");
  }
  *flags = host ? HS_TRANSFER_HOST_LINK : 0u;
  return HS_OK;
}

extern "C" int store_kv_scatter(const void* src, int64_t src_row_stride_bytes, void* dst,
                                int64_t dst_row_stride_bytes, int64_t dst_nrows, const int64_t* loc,
                                int64_t n, int64_t row_bytes, hipStream_t stream) {
  const ScatterSide k{static_cast<const char*>(src), src_row_stride_bytes, static_cast<char*>(dst),
                      dst_row_stride_bytes};
  return launch_scatter(k, nullptr, dst_nrows, loc, n, row_bytes, stream);
}

extern "C" int store_kv_cache(const void* k_src, int64_t k_src_row_stride_bytes, const void* v_src,
                              int64_t v_src_row_stride_bytes, void* k_dst,
                              int64_t k_dst_row_stride_bytes, void* v_dst,
                              int64_t v_dst_row_stride_bytes, int64_t dst_nrows, const int64_t* loc,
                              int64_t n, int64_t row_bytes, hipStream_t stream) {
  const ScatterSide k{static_cast<const char*>(k_src), k_src_row_stride_bytes,
                      static_cast<char*>(k_dst), k_dst_row_stride_bytes};
  const ScatterSide v{static_cast<const char*>(v_src), v_src_row_stride_bytes,
                      static_cast<char*>(v_dst), v_dst_row_stride_bytes};
  return launch_scatter(k, &v, dst_nrows, loc, n, row_bytes, stream);
}

extern "C" int hisparse_state_reset(int32_t* slot_tokens, int16_t* lru, const int64_t* rows,
                                    int64_t n_rows, int32_t H, int64_t S_r, int64_t R,
                                    hipStream_t stream) {
  if (n_rows < 0 || H < 0 || R < 0) return set_error(HS_EINVAL, "sizes must be >= 0");
  if (n_rows == 0) return HS_OK;
  if (!slot_tokens || !lru || !rows) return set_error(HS_EINVAL, "a required pointer is NULL");
  if (H > 32768) return set_error(HS_ERANGE, "H exceeds 32768 (int16 slots)");
  if (S_r < static_cast<int64_t>(H) + 1) return set_error(HS_EINVAL, "S_r must be >= H+1");
  if (n_rows > 0x7fffffffll) return set_error(HS_ERANGE, "too many rows for one launch");
  hipLaunchKernelGGL(state_reset_kernel, dim3(static_cast<unsigned>(n_rows)), dim3(kThreads), 0,
                     stream, slot_tokens, lru, rows, H, S_r, R);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(HS_ELAUNCH, "reset launch: %s", hipGetErrorString(e));
  return HS_OK;
}

extern "C" int hisparse_invalidate_written(int32_t* slot_keys, int64_t R, int64_t S_r,
                                           const int64_t* rows, const int64_t* written, int64_t n,
                                           hipStream_t stream) {
  if (n < 0 || R < 0 || S_r < 0) return set_error(HS_EINVAL, "sizes must be >= 0");
  if (n == 0 || R == 0 || S_r == 0) return HS_OK;
  if (!slot_keys || !rows || !written) return set_error(HS_EINVAL, "a required pointer is NULL");
  DeviceInfo di;
  const int rc = device_info(&di);
  if (rc != HS_OK) return rc;
  const int64_t cap = 16ll * (di.num_cus > 0 ? di.num_cus : 256);
  const unsigned grid = static_cast<unsigned>(n < cap ? n : cap);
  hipLaunchKernelGGL(invalidate_kernel, dim3(grid), dim3(kThreads), 0, stream, slot_keys, R, S_r,
                     rows, written, n);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(HS_ELAUNCH, "invalidate launch: %s", hipGetErrorString(e));
  return HS_OK;
}
