// HiSparse decode-step swap-in for gfx950.
//
// What is computed follows SGLang hisparse.cuh (load_cache_to_device_buffer_kernel)
// and vLLM hisparse_kernels.cu (hisparse_resolve_residency_kernel +
// hisparse_gather_compact_kernel): classify the top-k ids, find which are
// resident in the request's LRU slots, hand the misses the oldest non-hit
// slots in top-k order, rewrite the LRU order, copy the missed rows in.
//
// How it is laid out here (MI355X-first, not a translation):
//  * resolve_kernel: one 1024-lane workgroup (16 wave64) per batch row. All
//    per-request scratch lives in LDS: a packed 64-bit (token, index) open
//    addressing table, the staged LRU row, the victim list, hit/pending bit
//    sets. Compaction never walks the LRU in wave-sized chunks with a running
//    scan (the pages' structure, whose wave64 window needs special care);
//    instead each position's rank is popcount(hit bits below it) plus one
//    block-wide exclusive scan over 64-bit words, so every position is placed
//    independently and the global loads of a phase are all issued up front.
//  * swap_copy_kernel: the misses, published as a compact (pool row, hot row)
//    list in a caller-provided workspace, are copied by many 256-lane
//    workgroups per request as a flat stream of 16-byte chunks.
#include <hip/hip_runtime.h>

#include "hs_common.hpp"

namespace hs {
namespace {

constexpr int kResolveThreads = 1024;
constexpr int kResolveWaves = kResolveThreads / kWave;
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr uint64_t kEmpty = ~0ull;  // (token -1, index 0xFFFFFFFF): never a live entry

// Knuth's multiplicative hashing (TAOCP vol. 3, 6.4): multiply by
// floor(2^32 / golden ratio) = 2654435761 and keep the TOP log2(T) bits of the
// 32-bit product. Both pages use this multiplier but keep the low bits
// (product mod size), which for power-of-two sizes only permutes id mod size;
// the high bits spread ids that share low bits. Only speed depends on this.
__device__ __forceinline__ uint32_t hash_home(int32_t key, uint32_t shift) {
  return (static_cast<uint32_t>(key) * 2654435761u) >> shift;
}

struct ResolveArgs {
  const int32_t* topk;
  int64_t topk_stride;
  const int64_t* req_rows;
  const int64_t* seq_lens;
  const int32_t* num_real;
  int32_t* slot_tokens;
  int16_t* lru;
  const int32_t* slot_rows;
  const int64_t* pool_rows;
  int64_t ctx_stride;
  int64_t pool_nrows;
  int32_t* out_rows;
  int32_t* miss_counts;
  int32_t* ws_count;  // [B]
  int64_t* ws_src;    // [B, K] pool row of miss m
  int32_t* ws_dst;    // [B, K] hot row of miss m (-1 = skip)
  int32_t B, K, H;
  int64_t S_r, R;
  uint32_t T;        // hash table entries (power of two, >= 2K)
  uint32_t shift;    // 32 - log2(T)
};

struct LdsLayout {
  // byte offsets
  uint32_t hash, pend, hit, hitpos, topk, scan, wtot, lru, victim, total;
};

__host__ __device__ inline uint32_t align_up(uint32_t x, uint32_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline LdsLayout lds_layout(int32_t K, int32_t H, uint32_t T) {
  const uint32_t kw = (static_cast<uint32_t>(K) + 63) / 64;
  const uint32_t hw = (static_cast<uint32_t>(H) + 63) / 64;
  const uint32_t mw = kw > hw ? kw : hw;
  LdsLayout l;
  uint32_t o = 0;
  l.hash = o;   o += 8 * T;
  l.pend = o;   o += 8 * kw;
  l.hit = o;    o += 8 * kw;
  l.hitpos = o; o += 8 * hw;
  l.topk = o;   o += 4 * static_cast<uint32_t>(K);
  l.scan = o;   o += 4 * mw;
  l.wtot = o;   o += 4 * 32;
  l.lru = o;    o += 2 * static_cast<uint32_t>(H);
  l.victim = o; o += 2 * static_cast<uint32_t>(K);
  l.total = align_up(o, 16);
  return l;
}

// Exclusive block-wide scan of popcount(word(w)) over w < nw (nw <= 1024).
// Writes the prefix of word w to scan[w] and returns the grand total to every
// thread. Two barriers; safe to call back to back.
template <class WordFn>
__device__ __forceinline__ int block_popc_scan(WordFn word, int nw, int32_t* scan, int32_t* wtot) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int own = tid < nw ? __popcll(word(tid)) : 0;
  int v = own;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int n = __shfl_up(v, off, kWave);
    if (lane >= off) v += n;
  }
  if (lane == kWave - 1) wtot[wave] = v;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kResolveWaves; ++w) {
    const int t = wtot[w];
    before += (w < wave) ? t : 0;
    total += t;
  }
  if (tid < nw) scan[tid] = before + v - own;
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(ResolveArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int b = blockIdx.x;
  const int32_t K = a.K, H = a.H;
  int32_t* out = a.out_rows + static_cast<int64_t>(b) * K;

  const int64_t r = a.req_rows[b];
  const int32_t nreal = a.num_real ? *a.num_real : a.B;
  if (b >= nreal || r < 0 || r >= a.R) {
    // Padding row (vLLM page's V2 convention): -1 everywhere, no misses.
    for (int i = tid; i < K; i += kResolveThreads) out[i] = -1;
    if (tid == 0) {
      a.ws_count[b] = 0;
      if (a.miss_counts) a.miss_counts[b] = 0;
    }
    return;
  }
  const int64_t L = a.seq_lens[b];
  const int32_t* ids = a.topk + static_cast<int64_t>(b) * a.topk_stride;
  int32_t* tokens = a.slot_tokens + r * a.S_r;
  int16_t* lru = a.lru + r * H;
  const int32_t* srows = a.slot_rows ? a.slot_rows + r * a.S_r : nullptr;
  const int64_t* prow = a.pool_rows ? a.pool_rows + r * a.ctx_stride : nullptr;
  const int64_t hot_base = r * a.S_r;

  const LdsLayout lay = lds_layout(K, H, a.T);
  uint64_t* hash = reinterpret_cast<uint64_t*>(lds + lay.hash);
  uint64_t* pend = reinterpret_cast<uint64_t*>(lds + lay.pend);
  uint64_t* hitb = reinterpret_cast<uint64_t*>(lds + lay.hit);
  uint64_t* hitpos = reinterpret_cast<uint64_t*>(lds + lay.hitpos);
  int32_t* s_topk = reinterpret_cast<int32_t*>(lds + lay.topk);
  int32_t* scan = reinterpret_cast<int32_t*>(lds + lay.scan);
  int32_t* wtot = reinterpret_cast<int32_t*>(lds + lay.wtot);
  int16_t* s_lru = reinterpret_cast<int16_t*>(lds + lay.lru);
  int16_t* victim = reinterpret_cast<int16_t*>(lds + lay.victim);
  const uint32_t tmask = a.T - 1;
  const int kw = (K + 63) / 64, hw = (H + 63) / 64;

  auto row_of = [&](int32_t s) -> int32_t {
    return srows ? srows[s] : static_cast<int32_t>(hot_base + s);
  };
  auto pool_of = [&](int64_t t) -> int64_t { return prow ? prow[t] : r * a.ctx_stride + t; };

  // ---- init ---------------------------------------------------------------
  for (uint32_t i = tid; i < a.T; i += kResolveThreads) hash[i] = kEmpty;
  for (int i = tid; i < kw; i += kResolveThreads) hitb[i] = 0;
  if (tid == 0) wtot[kResolveWaves] = 0;  // pending-id counter
  __syncthreads();

  // ---- 1. classify ids; bind the newest token; insert pending ids ----------
  // SGLang page: newest token -> newest_slot (= H), everything else hashed.
  // vLLM page: ids outside the pool resolve to -1 and are not misses.
  for (int base = 0; base < K; base += kResolveThreads) {
    const int i = base + tid;
    bool pending = false;
    if (i < K) {
      const int32_t t = ids[i];
      s_topk[i] = t;
      bool valid = t >= 0 && static_cast<int64_t>(t) < L && static_cast<int64_t>(t) < a.ctx_stride;
      if (valid) {
        const int64_t pr = pool_of(t);
        valid = pr >= 0 && pr < a.pool_nrows;
      }
      if (!valid) {
        out[i] = -1;
      } else if (static_cast<int64_t>(t) == L - 1) {
        out[i] = row_of(H);
      } else {
        pending = true;
        const uint64_t entry = (static_cast<uint64_t>(static_cast<uint32_t>(i)) << 32) |
                               static_cast<uint32_t>(t);
        uint32_t h = hash_home(t, a.shift);
        // At most K <= T/2 entries, so an empty cell is always found.
        while (atomicCAS(reinterpret_cast<unsigned long long*>(&hash[h]),
                         static_cast<unsigned long long>(kEmpty),
                         static_cast<unsigned long long>(entry)) != kEmpty) {
          h = (h + 1) & tmask;
        }
      }
    }
    const uint64_t m = __ballot(pending);
    if (lane == 0 && i < K) {
      pend[i >> 6] = m;
      if (m) atomicAdd(&wtot[kResolveWaves], static_cast<int>(__popcll(m)));
    }
  }
  __syncthreads();
  const int pending_n = wtot[kResolveWaves];

  // ---- 2a. LRU scan: stage the order, probe each slot's token --------------
  // A slot whose token is pending is a hit and serves that top-k entry.
  for (int base = 0; base < H; base += kResolveThreads * 4) {
    int32_t s[4];
    int32_t tok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = base + u * kResolveThreads + tid;
      s[u] = p < H ? static_cast<int32_t>(lru[p]) : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = base + u * kResolveThreads + tid;
      if (p < H) s_lru[p] = static_cast<int16_t>(s[u]);
      tok[u] = (s[u] >= 0 && s[u] < H) ? tokens[s[u]] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = base + u * kResolveThreads + tid;
      bool hit = false;
      if (tok[u] >= 0) {
        uint32_t h = hash_home(tok[u], a.shift);
        int idx = -1;
        while (true) {
          const uint64_t e = hash[h];
          if (e == kEmpty) break;
          if (static_cast<int32_t>(static_cast<uint32_t>(e)) == tok[u]) {
            idx = static_cast<int>(e >> 32);
            break;
          }
          h = (h + 1) & tmask;
        }
        if (idx >= 0) {
          // First claimant wins; a second slot with the same token (corrupt
          // state) is treated as evictable instead of double-serving the entry.
          const unsigned long long bit = 1ull << (idx & 63);
          const unsigned long long old =
              atomicOr(reinterpret_cast<unsigned long long*>(&hitb[idx >> 6]), bit);
          if (!(old & bit)) {
            hit = true;
            out[idx] = row_of(s[u]);
          }
        }
      }
      const uint64_t m = __ballot(hit);
      if (lane == 0 && p < H) hitpos[p >> 6] = m;
    }
  }
  __syncthreads();

  // ---- 2b. ranks of hits among LRU positions -------------------------------
  const int hits = block_popc_scan([&](int w) { return hitpos[w]; }, hw, scan, wtot);
  const int E = H - hits;            // evictable slots
  const int M = pending_n - hits;    // misses (<= E because K <= H)

  // ---- 2c. victims and the new LRU order -----------------------------------
  // New order: stale evictables, then the M victims (they receive the misses,
  // in miss order), then the hits -- every group in its old order.
  for (int base = 0; base < H; base += kResolveThreads) {
    const int p = base + tid;
    if (p < H) {
      const uint64_t wd = hitpos[p >> 6];
      const int bp = p & 63;
      const int hr = scan[p >> 6] + __popcll(wd & ((1ull << bp) - 1ull));
      const int16_t s = s_lru[p];
      int np;
      if ((wd >> bp) & 1ull) {
        np = E + hr;
      } else {
        const int e = p - hr;
        if (e < M) {
          victim[e] = s;
          np = E - M + e;
        } else {
          np = e - M;
        }
      }
      lru[np] = s;
    }
  }
  __syncthreads();

  // ---- 3. misses in top-k order take victims; publish the copy list --------
  auto miss_word = [&](int w) { return pend[w] & ~hitb[w]; };
  const int m_total = block_popc_scan(miss_word, kw, scan, wtot);
  int64_t* ws_src = a.ws_src + static_cast<int64_t>(b) * K;
  int32_t* ws_dst = a.ws_dst + static_cast<int64_t>(b) * K;
  for (int base = 0; base < K; base += kResolveThreads) {
    const int i = base + tid;
    if (i < K) {
      const uint64_t wd = miss_word(i >> 6);
      const int bp = i & 63;
      if ((wd >> bp) & 1ull) {
        const int m = scan[i >> 6] + __popcll(wd & ((1ull << bp) - 1ull));
        const int32_t t = s_topk[i];
        const int32_t v = m < M ? victim[m] : -1;
        if (v >= 0 && v < H) {
          const int32_t row = row_of(v);
          out[i] = row;
          tokens[v] = t;
          ws_src[m] = pool_of(t);
          ws_dst[m] = row;
        } else {
          out[i] = -1;
          ws_src[m] = 0;
          ws_dst[m] = -1;
        }
      }
    }
  }
  if (tid == 0) {
    a.ws_count[b] = m_total;
    if (a.miss_counts) a.miss_counts[b] = m_total;
  }
}

// Copy the published misses: workgroup g serves request g % B, part g / B.
template <int W>
__global__ __launch_bounds__(kCopyThreads) void swap_copy_kernel(
    const char* __restrict__ pool, char* __restrict__ hot, int64_t row_bytes, int64_t hot_nrows,
    const int32_t* __restrict__ ws_count, const int64_t* __restrict__ ws_src,
    const int32_t* __restrict__ ws_dst, int32_t B, int32_t K, int32_t parts, FastDiv cdiv) {
  typedef Chunk<W> C;
  const int b = blockIdx.x % B;
  const int part = blockIdx.x / B;
  const int M = ws_count[b];
  const uint32_t total = static_cast<uint32_t>(M) * cdiv.d;
  const int64_t* src = ws_src + static_cast<int64_t>(b) * K;
  const int32_t* dst = ws_dst + static_cast<int64_t>(b) * K;
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
        const uint32_t m = fdiv(j, cdiv);
        const uint32_t c = j - m * cdiv.d;
        const int32_t hr = dst[m];
        if (hr >= 0 && hr < hot_nrows) {
          v[u] = C::load(pool + src[m] * row_bytes + static_cast<int64_t>(c) * W);
          d[u] = hot + static_cast<int64_t>(hr) * row_bytes + static_cast<int64_t>(c) * W;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (d[u]) C::store(d[u], v[u]);
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WsLayout {
  size_t count, src, dst, total;
};

inline WsLayout ws_layout(int64_t B, int64_t K) {
  WsLayout w;
  w.count = 0;
  w.src = align256(4 * static_cast<size_t>(B));
  w.dst = w.src + align256(8 * static_cast<size_t>(B) * static_cast<size_t>(K));
  w.total = w.dst + align256(4 * static_cast<size_t>(B) * static_cast<size_t>(K));
  return w;
}

inline uint32_t pow2_at_least(uint32_t x) {
  uint32_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace
}  // namespace hs

using namespace hs;

extern "C" size_t hs_swap_in_workspace_bytes(int32_t B, int32_t K) {
  if (B <= 0 || K <= 0) return 0;
  return ws_layout(B, K).total;
}

extern "C" int hisparse_swap_in(const hs_swap_in_args* a, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (!a) return set_error(HS_EINVAL, "args is NULL");
  if (a->B < 0 || a->K < 0) return set_error(HS_EINVAL, "B and K must be >= 0");
  if (a->B == 0 || a->K == 0) return HS_OK;
  if (!a->topk_ids || !a->req_rows || !a->seq_lens || !a->slot_tokens || !a->lru || !a->pool ||
      !a->hot || !a->out_rows)
    return set_error(HS_EINVAL, "a required pointer is NULL");
  if (a->H < a->K) return set_error(HS_EINVAL, "hot_size H=%d must be >= top_k K=%d", a->H, a->K);
  if (a->H > 32768) return set_error(HS_ERANGE, "hot_size H=%d exceeds 32768 (int16 slots)", a->H);
  if (a->S_r < static_cast<int64_t>(a->H) + 1)
    return set_error(HS_EINVAL, "region_stride S_r=%lld must be >= H+1", (long long)a->S_r);
  if (a->R <= 0) return set_error(HS_EINVAL, "R must be > 0");
  if (a->topk_stride < a->K) return set_error(HS_EINVAL, "topk_stride must be >= K");
  if (a->ctx_stride <= 0) return set_error(HS_EINVAL, "ctx_stride must be > 0");
  if (a->pool_nrows < 0 || a->hot_nrows <= 0) return set_error(HS_EINVAL, "bad pool/hot row counts");
  if (a->row_bytes <= 0 || (a->row_bytes & 3) != 0)
    return set_error(HS_EINVAL, "row_bytes=%lld must be a positive multiple of 4", (long long)a->row_bytes);
  if (a->row_bytes > (1ll << 20)) return set_error(HS_ERANGE, "row_bytes above 1 MiB");
  if (!aligned(a->pool, 4) || !aligned(a->hot, 4))
    return set_error(HS_EINVAL, "pool and hot must be 4-byte aligned");
  if (!a->slot_rows) {
    if (a->R * a->S_r > 0x7fffffffll)
      return set_error(HS_ERANGE, "R*S_r exceeds int32 hot-row indices");
    if (a->hot_nrows < a->R * a->S_r)
      return set_error(HS_EINVAL, "hot_nrows < R*S_r with flat regions");
  }
  const int W = (aligned(a->pool, 16) && aligned(a->hot, 16) && (a->row_bytes & 15) == 0) ? 16 : 4;
  const int64_t C = a->row_bytes / W;
  if (static_cast<int64_t>(a->K) * C >= (1ll << 31))
    return set_error(HS_ERANGE, "top_k * chunks per row exceeds 2^31");
  const WsLayout wl = ws_layout(a->B, a->K);
  if (!workspace || workspace_bytes < wl.total || !aligned(workspace, 256))
    return set_error(HS_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned", wl.total);

  DeviceInfo di;
  int rc = device_info(&di);
  if (rc != HS_OK) return rc;
  const uint32_t T = pow2_at_least(static_cast<uint32_t>(2 * a->K) < 64 ? 64u : static_cast<uint32_t>(2 * a->K));
  uint32_t log2T = 0;
  while ((1u << log2T) < T) ++log2T;
  const LdsLayout lay = lds_layout(a->K, a->H, T);
  if (static_cast<int>(lay.total) > di.max_lds)
    return set_error(HS_ERANGE, "K=%d, H=%d need %u bytes of LDS; the device allows %d", a->K,
                     a->H, lay.total, di.max_lds);

  if (lay.total > 65536) {
    // Opt in to more than 64 KB of dynamic LDS (gfx950 has 160 KB per CU).
    const hipError_t fe = hipFuncSetAttribute(reinterpret_cast<const void*>(&resolve_kernel),
                                              hipFuncAttributeMaxDynamicSharedMemorySize,
                                              static_cast<int>(lay.total));
    if (fe != hipSuccess) {
      (void)hipGetLastError();
      return set_error(HS_ERANGE, "cannot raise dynamic LDS to %u bytes: %s", lay.total,
                       hipGetErrorString(fe));
    }
  }

  // Pool: device memory, or pinned host memory read directly by the kernels
  // (vLLM page's is_pinned_cpu_tensor check).
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, a->pool) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(HS_EMEMKIND, "pool is not a HIP allocation (device or pinned host)");
  }
  const char* pool_dev = nullptr;
  if (attr.type == hipMemoryTypeDevice) {
    pool_dev = static_cast<const char*>(a->pool);
  } else if (attr.type == hipMemoryTypeHost) {
    pool_dev = static_cast<const char*>(attr.devicePointer ? attr.devicePointer : a->pool);
  } else {
    return set_error(HS_EMEMKIND, "pool must be device memory or pinned host memory");
  }

  char* ws = static_cast<char*>(workspace);
  ResolveArgs ra;
  ra.topk = a->topk_ids;
  ra.topk_stride = a->topk_stride;
  ra.req_rows = a->req_rows;
  ra.seq_lens = a->seq_lens;
  ra.num_real = a->num_real;
  ra.slot_tokens = a->slot_tokens;
  ra.lru = a->lru;
  ra.slot_rows = a->slot_rows;
  ra.pool_rows = a->pool_rows;
  ra.ctx_stride = a->ctx_stride;
  ra.pool_nrows = a->pool_nrows;
  ra.out_rows = a->out_rows;
  ra.miss_counts = a->miss_counts;
  ra.ws_count = reinterpret_cast<int32_t*>(ws + wl.count);
  ra.ws_src = reinterpret_cast<int64_t*>(ws + wl.src);
  ra.ws_dst = reinterpret_cast<int32_t*>(ws + wl.dst);
  ra.B = a->B;
  ra.K = a->K;
  ra.H = a->H;
  ra.S_r = a->S_r;
  ra.R = a->R;
  ra.T = T;
  ra.shift = 32 - log2T;

  hipLaunchKernelGGL(resolve_kernel, dim3(a->B), dim3(kResolveThreads), lay.total, stream, ra);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(HS_ELAUNCH, "resolve launch: %s", hipGetErrorString(e));

  // Copy grid: enough workgroups per request to cover its worst case (all K
  // missing) at kCopyUnroll chunks per lane, capped so the whole launch is a
  // few thousand workgroups.
  const int64_t max_items = static_cast<int64_t>(a->K) * C;
  int64_t parts = (max_items + kCopyThreads * kCopyUnroll - 1) / (kCopyThreads * kCopyUnroll);
  const int64_t cap = (8LL * di.num_cus + a->B - 1) / a->B;
  if (parts > cap) parts = cap;
  if (parts < 1) parts = 1;
  const FastDiv cdiv = make_fastdiv(static_cast<uint32_t>(C));
  const dim3 grid(static_cast<unsigned>(a->B * parts));
  if (W == 16)
    hipLaunchKernelGGL(swap_copy_kernel<16>, grid, dim3(kCopyThreads), 0, stream, pool_dev,
                       static_cast<char*>(a->hot), a->row_bytes, a->hot_nrows, ra.ws_count,
                       ra.ws_src, ra.ws_dst, a->B, a->K, static_cast<int32_t>(parts), cdiv);
  else
    hipLaunchKernelGGL(swap_copy_kernel<4>, grid, dim3(kCopyThreads), 0, stream, pool_dev,
                       static_cast<char*>(a->hot), a->row_bytes, a->hot_nrows, ra.ws_count,
                       ra.ws_src, ra.ws_dst, a->B, a->K, static_cast<int32_t>(parts), cdiv);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(HS_ELAUNCH, "copy launch: %s", hipGetErrorString(e));
  return HS_OK;
}
