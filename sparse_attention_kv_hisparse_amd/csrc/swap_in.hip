// HiSparse decode-step swap-in for gfx950.
//
// What is computed follows SGLang hisparse.cuh (load_cache_to_device_buffer_kernel)
// and vLLM hisparse_kernels.cu (hisparse_resolve_residency_kernel +
// hisparse_gather_compact_kernel): classify the top-k ids, find which are
// resident in the request's LRU slots, give the misses the oldest non-hit
// slots in top-k order, rewrite the LRU order, copy the missed rows in.
//
// How it is laid out here (MI355X-first, not a translation):
//  * resolve_kernel: one 1024-lane workgroup (16 wave64) per batch row. A
//    request's resolution runs entirely out of LDS: the top-k ids, the LRU
//    row and the slot-token row are staged with coalesced loads in one round
//    trip, outputs are built in LDS and written once at the end, so no global
//    store ever sits in front of a dependent load.
//  * Compaction is stable and wave-local: each wave owns a contiguous,
//    64-aligned segment of LRU positions (and of top-k indices), ranks come
//    from ballot + mbcnt plus a running count, and only the 16 per-wave
//    totals cross waves, so there is no block-wide scan and no wave64 scan
//    window to get wrong (the pages' per-warp chunk scan needs one).
//  * Membership (which top-k ids some slot holds) goes through an LDS table
//    built per call. When the layout is flat and the table fits, it is a
//    direct-address table over positions naming the slot that holds each
//    one, and every id is looked up once. With paged addressing the slots'
//    keys go into a bucketed hash (Knuth's multiplicative hash, rebuilt with
//    a salted hash when a chain runs long) and every id is looked up once
//    there. Otherwise the pending ids go into that hash and every slot's
//    token is probed. No result depends on which one runs.
//  * swap_copy_kernel: the misses, published as a compact (pool row, hot row)
//    list in the caller's workspace, are copied by many workgroups per
//    request (1024-lane ones, two per CU, from an HBM pool; 256-lane ones
//    otherwise) as a flat stream of 16-byte chunks. The kernel boundary is
//    the only hand-off between the two, so no workgroup ever waits on another.
//  * With a pinned-host pool the resolve kernel copies its own request's rows
//    as well (phase 5): the host link is full with one workgroup per request.
//    Each lane issues its first chunk's read as soon as the misses are known,
//    before the victims and outputs are worked out.
#include <hip/hip_runtime.h>

#include <climits>
#include <type_traits>
#include <mutex>

#include "hs_common.hpp"
#include "swap_copy.hpp"

namespace hs {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kFuseUnroll = 12;  // chunks per lane per round, fused copy
constexpr int kEarlyChunks = 1;  // fused copy: chunks per lane loaded before the victims
// Entries per lane per pass: top-k phases take two (K = 2048 fills a pass of
// 1024 lanes exactly), LRU phases four (H = 4096). A lane slot past the end of
// a pass still costs issue cycles, so the unroll follows the common sizes.
constexpr int kKU = 2;
constexpr int kHU = 4;
constexpr int32_t kPending = INT32_MIN;    // s_out value of an id still unresolved
// Loop trips (bucket steps) an insert or a lookup may take under Knuth's hash
// before the workgroup switches to the salted one. Dense and uniform top-k
// sets take at most 3 or 4 at a quarter-full table.
constexpr int kTripLimit = 8;

// Home bucket of a key: Knuth's multiplicative hashing (TAOCP vol. 3, 6.4).
// Multiply by floor(2^32 / golden ratio) = 2654435761 and keep the TOP bits
// of the 32-bit product -- the top log2(buckets) bits pick the bucket. Both
// pages use this multiplier but keep the low bits (product mod size), which
// for power-of-two sizes only permutes id mod size. The top bits spread a run
// of consecutive ids evenly (three-distance theorem), and top-k ids are dense
// runs of recent positions. Only speed depends on the hash, never a result.
__device__ __forceinline__ uint32_t bucket_knuth(int32_t key, uint32_t bshift) {
  return (static_cast<uint32_t>(key) * 2654435761u) >> bshift;
}

// The fallback when Knuth's hash clusters. Any fixed hash lets whoever picks
// the ids pick ones that share home buckets (a 65,536-token context holds
// ~4,000 ids in any 1/16 of the buckets; such a set made the probe phase ~40x
// slower). When an insert or a lookup runs past kTripLimit buckets, the
// workgroup rebuilds its table with this hash: the key XOR a 32-bit salt
// drawn per workgroup and call (a splitmix64 mix of the shader clock and the
// batch row), through MurmurHash3's 32-bit finalizer (a bijection in which
// every input bit flips each output bit with probability close to 1/2); its
// top bits pick the bucket. A random multiplier alone was tried as the only
// hash and dropped: some draws spread dense position runs badly, and the
// slowest of B workgroups sets the kernel's time.
__device__ __forceinline__ uint32_t bucket_salted(int32_t key, uint32_t salt, uint32_t bshift) {
  uint32_t h = static_cast<uint32_t>(key) ^ salt;
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h >> bshift;
}

// splitmix64's output function (Steele, Lea and Flood, 2014).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct SwapArgs {
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
  const char* pool;
  int64_t pool_nrows;
  char* hot;
  int64_t hot_nrows;
  int64_t row_bytes;
  int32_t* out_rows;
  int32_t* miss_counts;
  int32_t* miss_mask; // [B, K] or null: 1 where the entry missed and got a slot
  unsigned long long* stats;  // [2] or null: hits and misses, accumulated
  const char* pool_v; // non-MLA caches: V pool / V hot buffer, or null
  char* hot_v;
  // vLLM-style paged addressing (kPaged instantiations only): hot block
  // table, source block table, resident block table, attention indices.
  const int32_t* hbt;
  int64_t hbt_stride;
  int32_t hbs;
  const int32_t* sbt;
  int64_t sbt_stride;
  int32_t sbt_nblocks, sbs;
  const int32_t* rbt;
  int64_t rbt_stride;
  int32_t rbt_nblocks, rbs, r_null;
  int32_t* att;
  int64_t att_stride, att_block_stride;
  int32_t* count;     // [B] misses of request b
  int64_t* src;       // [B, K] pool row of miss m
  int32_t* dst;       // [B, K] hot row of miss m (-1 = skip)
  int32_t B, K, H;
  int64_t S_r, R;
  uint32_t T;         // hash entries, power of two >= 2K, or >= 2H for the slots' keys (0 with a direct table)
  uint32_t dtab;      // direct-address table entries (ctx_stride), or 0 for the hash
  uint32_t shift;     // 32 - log2(T)
  int32_t stage_tokens;
  int32_t hbt_n;      // paged: hot block table entries staged in LDS (0 = read from HBM)
  int32_t sbt_n;      // paged: source block table entries staged in LDS (0 = read from HBM)
  FastDiv cdiv;       // chunks per row
  FastDiv hbs_div, sbs_div, rbs_div;   // paged: the three block sizes
};

struct LdsLayout {
  uint32_t hash, hidx, bcnt, out, topk, lru, nlru, tok, victim, hitpos, missw, wtot, seed, dummy,
      hbt, sbt, total;
};

__host__ __device__ inline uint32_t align_up(uint32_t x, uint32_t a) { return (x + a - 1) / a * a; }

// Wave w owns positions [w*seg, (w+1)*seg) of an n-long array; seg is a
// multiple of 64 so every 64-position chunk is one ballot word.
__host__ __device__ inline uint32_t wave_segment(int32_t n) {
  return align_up((static_cast<uint32_t>(n) + kWaves - 1) / kWaves, 64);
}

// dtab != 0: the direct-address table of dtab int16 entries replaces the hash
// (keys, indices and counts); the region still holds the fused copy's miss
// list (12 bytes per miss) after the lookup.
__host__ __device__ inline LdsLayout lds_layout(int32_t K, int32_t H, uint32_t T, bool stage_tokens,
                                                uint32_t hbt_n, uint32_t sbt_n, uint32_t dtab) {
  const uint32_t hwords = kWaves * wave_segment(H) / 64;
  const uint32_t kwords = kWaves * wave_segment(K) / 64;
  LdsLayout l;
  // every region starts on a 16-byte boundary
  uint32_t o = 0;
  if (dtab) {
    const uint32_t list = 12 * static_cast<uint32_t>(K);
    l.hash = o; o = align_up(o + (2 * dtab > list ? 2 * dtab : list), 16);   // table; later: miss list
    l.hidx = o;
    l.bcnt = o;
  } else {
    l.hash = o;   o = align_up(o + 4 * T, 16);                // keys; later: miss list
    l.hidx = o;   o = align_up(o + 2 * T, 16);                // top-k index of each key
    l.bcnt = o;   o = align_up(o + T, 16);                    // one count per 4-key bucket
  }
  l.out = o;    o = align_up(o + 4 * static_cast<uint32_t>(K), 16);
  l.topk = o;   o = align_up(o + 4 * static_cast<uint32_t>(K), 16);
  l.tok = o;    o = align_up(o + (stage_tokens ? 4 * static_cast<uint32_t>(H) : 0), 16);
  l.hitpos = o; o = align_up(o + 8 * hwords, 16);
  l.missw = o;  o = align_up(o + 8 * kwords, 16);
  l.wtot = o;   o = align_up(o + 4 * (2 * (kWaves + 1) + 2), 16);
  l.seed = o;   o = align_up(o + 16, 16);                     // the salted hash's salt
  l.dummy = o;  o = align_up(o + 8 * kThreads, 16);            // per-lane CAS sink
  l.lru = o;    o = align_up(o + 2 * static_cast<uint32_t>(H), 16);
  l.nlru = o;   o = align_up(o + 2 * static_cast<uint32_t>(H), 16);   // new LRU order; before it, pos_of
  l.victim = o; o = align_up(o + 2 * static_cast<uint32_t>(K), 16);
  l.hbt = o;    o = align_up(o + 4 * hbt_n, 16);                 // paged: hot block table row
  l.sbt = o;    o = align_up(o + 4 * sbt_n, 16);                 // paged: source block table row
  l.total = o;
  return l;
}

template <int N>
__device__ __forceinline__ bool any_of(const bool (&v)[N]) {
  bool r = false;
#pragma unroll
  for (int i = 0; i < N; ++i) r |= v[i];
  return r;
}

// A read of LDS through an address-space-3 pointer. Where one branch reads a
// table staged in LDS and the other the same table in HBM, plain (generic)
// loads let the compiler merge the two into one flat load through a selected
// address: a vector-memory round trip for the LDS side as well, waited for
// with the global loads. Typed LDS loads keep the two branches apart.
template <class T>
__device__ __forceinline__ T lds_read(const T* p) {
  return *(const __attribute__((address_space(3))) T*)p;
}

// popcount of the bits of a 64-bit wave mask held by lanes below this one.
__device__ __forceinline__ int rank_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// Sum of v over the 64 lanes of a wave, in every lane: an inclusive scan by
// DPP row shifts (within rows of 16) and row broadcasts (across rows), then
// lane 63. Called with all lanes active.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// Resolve request b (one workgroup): outputs, state updates and the miss list
// go to global memory; with kCopyW != 0 the workgroup then copies its own
// missed rows from a copy of the list kept in LDS (phase 5).
// kSlotRows / kPoolRows: whether the slot-row and pool-row tables are given.
// Without them no global load follows the first global store, so no wait on
// outstanding stores (vmcnt counts both) ever stalls a phase.
//
// LDS latency is ~230 cycles on gfx950, so every phase issues all of its
// independent LDS reads first and then works from registers. The hash is
// bucketed: four int32 keys per 16-byte bucket, a parallel int16 array with
// each key's top-k index and a per-bucket count, at most a quarter full, so
// an insert is almost always one atomicAdd and a lookup one 16-byte read.
// kPaged: vLLM-style addressing -- ids translate through the source block
// table to global ids, which are the slot keys and the pool rows; resident
// ids are served from the device cache as they are; slots live where the hot
// block table says; there is no newest-token slot.
template <bool kSlotRows, bool kPoolRows, int kCopyW, bool kPaged, bool kExact, bool kDirect>
__device__ void resolve(const SwapArgs& a, int b, unsigned char* lds, const LdsLayout& lay) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // Wave-uniform, and held in a scalar register so that every segment bound
  // derived from it compiles to scalar branches instead of exec masking.
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int32_t K = a.K, H = a.H;
  int32_t* out = a.out_rows + static_cast<int64_t>(b) * K;

  int32_t* hkey = reinterpret_cast<int32_t*>(lds + lay.hash);
  // Direct-address table (kDirect): entry t holds the slot of resident
  // position t. Never cleared: a lookup checks the token of the slot it reads,
  // so stale contents never match.
  int16_t* dtab = reinterpret_cast<int16_t*>(lds + lay.hash);
  int16_t* hidx = reinterpret_cast<int16_t*>(lds + lay.hidx);
  uint32_t* bcnt = reinterpret_cast<uint32_t*>(lds + lay.bcnt);
  int16_t* nlru = reinterpret_cast<int16_t*>(lds + lay.nlru);
  int32_t* s_out = reinterpret_cast<int32_t*>(lds + lay.out);
  int32_t* s_topk = reinterpret_cast<int32_t*>(lds + lay.topk);
  int32_t* s_tok = reinterpret_cast<int32_t*>(lds + lay.tok);
  uint64_t* hitpos = reinterpret_cast<uint64_t*>(lds + lay.hitpos);
  uint64_t* missw = reinterpret_cast<uint64_t*>(lds + lay.missw);
  // Cross-wave counts: pre_hit[w] / pre_miss[w] collect the totals of the
  // waves before w, entry kWaves the grand total; s_pending the pending ids
  // (hashed plans) and s_retry the hash fallback flag.
  int32_t* wtot = reinterpret_cast<int32_t*>(lds + lay.wtot);
  int32_t* pre_hit = wtot;
  int32_t* pre_miss = wtot + kWaves + 1;
  int32_t* s_pending = wtot + 2 * (kWaves + 1);
  int32_t* s_retry = s_pending + 1;   // set when Knuth's hash clusters
  int16_t* s_lru = reinterpret_cast<int16_t*>(lds + lay.lru);
  int16_t* victim = reinterpret_cast<int16_t*>(lds + lay.victim);
  // Inactive lanes aim their CAS at a private word, so the CAS of every
  // query can be issued unconditionally and all are in flight together.
  unsigned long long* sink64 = reinterpret_cast<unsigned long long*>(lds + lay.dummy) + tid;
  int32_t* sink32 = reinterpret_cast<int32_t*>(sink64);
  uint32_t* sinku = reinterpret_cast<uint32_t*>(sink64);
  const uint32_t bmask = a.T / 4 - 1;       // buckets - 1
  const uint32_t bshift = a.shift + 2;      // top log2(buckets) bits
  uint32_t* s_salt = reinterpret_cast<uint32_t*>(lds + lay.seed);
  const int32_t* ids = a.topk + static_cast<int64_t>(b) * a.topk_stride;

  const int64_t r = a.req_rows[b];
  const int32_t nreal = a.num_real ? *a.num_real : a.B;
  const int64_t L = kPaged ? 0 : a.seq_lens[b];
  if (b >= nreal || r < 0 || r >= a.R) {
    // Padding row (vLLM page's V2 convention): -1 everywhere, no misses.
    for (int i = tid; i < K; i += kThreads) out[i] = -1;
    if (kPaged && a.att)
      for (int i = tid; i < K; i += kThreads) a.att[static_cast<int64_t>(b) * a.att_stride + i] = -1;
    if (a.miss_mask)
      for (int i = tid; i < K; i += kThreads) a.miss_mask[static_cast<int64_t>(b) * K + i] = 0;
    if (tid == 0) {
      a.count[b] = 0;
      if (a.miss_counts) a.miss_counts[b] = 0;
    }
    return;
  }
  int32_t* tokens = a.slot_tokens + r * a.S_r;
  int16_t* lru = a.lru + r * H;
  const int32_t* srows = kSlotRows ? a.slot_rows + r * a.S_r : nullptr;
  const int64_t* prow = kPoolRows ? a.pool_rows + r * a.ctx_stride : nullptr;
  const int64_t hot_base = r * a.S_r;
  const int32_t* s_hbt = reinterpret_cast<const int32_t*>(lds + lay.hbt);
  auto row_of = [&](int32_t s) -> int32_t {
    if constexpr (kPaged) {
      const int32_t q = static_cast<int32_t>(fdiv(static_cast<uint32_t>(s), a.hbs_div));
      const int32_t blk = a.hbt_n ? lds_read(&s_hbt[q]) : a.hbt[r * a.hbt_stride + q];
      // In 64 bits: a table entry too large for an int32 row gives no row.
      const int64_t row = static_cast<int64_t>(blk) * a.hbs + (s - q * a.hbs);
      return (row < 0 || row > INT32_MAX) ? -1 : static_cast<int32_t>(row);
    }
    if constexpr (kSlotRows) return srows[s];
    return static_cast<int32_t>(hot_base + s);
  };
  auto pool_of = [&](int64_t t) -> int64_t {
    if constexpr (kPaged) return t;            // the key is the global id
    if constexpr (kPoolRows) return prow[t];
    return r * a.ctx_stride + t;
  };

  // ---- stage: ids, the LRU row and the slot-token row -----------------------
  // The first kKU * 1024 ids, the first 256 LRU positions of this wave's
  // segment (kept in registers for the probe or the lookup and the victim
  // step, which work on the same positions) and kHU * 1024 slot tokens land
  // with all loads in flight at once; a hash table is cleared while they are
  // outstanding. Longer rows follow in batches of four per lane.
  const int segH = static_cast<int>(wave_segment(H));
  const int segK = static_cast<int>(wave_segment(K));
  const int h0 = wave * segH;
  const int k0 = wave * segK;
  // Tile guards. With kExact (K a multiple of kKU * 1024 and H of kHU * 1024,
  // which the host checks) every top-k entry a pass or a wave segment names
  // is below K, every LRU position a segment chunk names is below H, and
  // every chunk offset lies inside its segment, so these fold to true and
  // the guarded loads and stores need no exec-mask branches.
  auto in_k = [&](int i) { return kExact || i < K; };
  auto in_h = [&](int p) { return kExact || p < H; };
  auto in_seg_h = [&](int off) { return kExact || off < segH; };
  auto in_seg_k = [&](int off) { return kExact || off < segK; };
  int32_t vi[kKU];
  int16_t vl[4];   // LRU entries at h0 + u*64 + lane

  // ---- 1. classify ids; bind the newest token; insert pending ids ----------
  // SGLang page: the newest token goes to newest_slot (= H), every other id is
  // hashed. vLLM page: ids outside the pool resolve to -1 and are not misses.
  // Without a pool-row table an id is valid iff 0 <= t < lim, one unsigned
  // compare: lim folds the sequence length, the row stride and the pool end.
  uint32_t lim = 0;
  int32_t newest_t = -1;   // never matches a valid id unless L-1 is one
  int32_t row_newest = 0;
  if constexpr (!kPaged) {
    int64_t l64 = L < a.ctx_stride ? L : a.ctx_stride;
    if constexpr (!kPoolRows) {
      const int64_t room = a.pool_nrows - r * a.ctx_stride;
      l64 = room < l64 ? room : l64;
    }
    l64 = l64 < 0 ? 0 : (l64 > INT32_MAX ? INT32_MAX : l64);
    lim = static_cast<uint32_t>(l64);
    if (L >= 1 && L - 1 < l64) newest_t = static_cast<int32_t>(L - 1);
    row_newest = row_of(H);
  }
  // vLLM page, first phase (paged addressing): position tt -> global id g
  // through the source block table (a physical block of 0 or below has no
  // row, nor has a global id past the pool), and the resident row res when
  // the resident table serves the position; -1 for none. Block and offset by
  // multiply-shift division (a negative tt lands past every table).
  [[maybe_unused]] auto translate = [&](int32_t tt, int64_t& g, int64_t& res) {
    g = tt;
    res = -1;
    if (a.sbt) {
      g = -1;
      const int32_t sq = static_cast<int32_t>(fdiv(static_cast<uint32_t>(tt), a.sbs_div));
      if (tt >= 0 && sq < a.sbt_nblocks) {
        const int32_t pb = a.sbt_n ? lds_read(reinterpret_cast<const int32_t*>(lds + lay.sbt) + sq)
                                   : a.sbt[r * a.sbt_stride + sq];
        if (pb > 0) g = static_cast<int64_t>(pb) * a.sbs + (tt - sq * a.sbs);
      }
    }
    if (g >= a.pool_nrows) g = -1;
    if (a.rbt) {
      const int32_t rq = static_cast<int32_t>(fdiv(static_cast<uint32_t>(tt), a.rbs_div));
      if (tt >= 0 && rq < a.rbt_nblocks) {
        const int32_t pb = a.rbt[r * a.rbt_stride + rq];
        if (pb != a.r_null && pb >= 0) {
          res = static_cast<int64_t>(pb) * a.rbs + (tt - rq * a.rbs);
          if (res > INT32_MAX) res = -1;
        }
      }
    }
  };
  // Classification + inserts (1) and the LRU scan (2), written once and run
  // with Knuth's hash. If an insert or a lookup runs past kTripLimit buckets,
  // the workgroup clears the table and its counts and runs both again with
  // the salted hash, reading the ids from global memory again. Nothing the
  // first run writes outside LDS survives into the second.
  auto classify_insert = [&](auto salted_tag, uint32_t salt) {
    constexpr bool kSalted = decltype(salted_tag)::value;
    for (int base = 0; base < K; base += kKU * kThreads) {
      int32_t t[kKU], o[kKU];
      uint32_t bk[kKU];
      bool ins[kKU];
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        const int i = base + u * kThreads + tid;
        t[u] = kSalted ? (in_k(i) ? ids[i] : 0) : (base == 0 ? vi[u] : (in_k(i) ? s_topk[i] : 0));
      }
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        const int i = base + u * kThreads + tid;
        if constexpr (kPaged) {
          // vLLM page, first phase: position -> global id through the source
          // block table (a physical block of 0 or below has no row), and a
          // resident row when the resident table holds the position.
          int64_t g = -1, res = -1;
          if (in_k(i)) translate(t[u], g, res);
          ins[u] = in_k(i) && res < 0 && g >= 0;
          o[u] = res >= 0 ? static_cast<int32_t>(res) : (g >= 0 ? kPending : -1);
          t[u] = static_cast<int32_t>(g);            // the key from here on
          if (ins[u]) s_topk[i] = t[u];
        } else {
          bool valid = in_k(i) && static_cast<uint32_t>(t[u]) < lim;
          if constexpr (kPoolRows) {
            if (valid) {
              const int64_t pr = prow[t[u]];
              valid = pr >= 0 && pr < a.pool_nrows;
            }
          }
          const bool newest = valid && t[u] == newest_t;
          ins[u] = valid && !newest;
          o[u] = !valid ? -1 : (newest ? row_newest : kPending);
        }
      }
      int npend = 0;
#pragma unroll
      for (int u = 0; u < kKU; ++u) npend += __popcll(__ballot(ins[u]));
#pragma unroll
      for (int u = 0; u < kKU; ++u)
        bk[u] = kSalted ? bucket_salted(t[u], salt, bshift) : bucket_knuth(t[u], bshift);
      // Each pending id takes the next entry of its home bucket with one LDS
      // atomicAdd on the bucket's count; a full bucket passes it on to the next
      // bucket (linear probing over buckets). A lookup stops at the first bucket
      // that is not full, which this order guarantees to be past the key; the
      // table is at most half full, so insertion terminates.
      const int nu = (K - base + kThreads - 1) / kThreads;   // live u, uniform
      int trips = 0;
      while (__ballot(any_of(ins)) != 0) {
        if (!kSalted && ++trips > kTripLimit) {   // clustered: fall back (uniform per wave)
          if (lane == 0) *s_retry = 1;
          break;
        }
        uint32_t p[kKU];
#pragma unroll
        for (int u = 0; u < kKU; ++u) p[u] = u < nu ? atomicAdd(ins[u] ? &bcnt[bk[u]] : sinku, 1u) : 4u;
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          if (ins[u] && p[u] < 4) {
            hkey[4 * bk[u] + p[u]] = t[u];
            hidx[4 * bk[u] + p[u]] = static_cast<int16_t>(base + u * kThreads + tid);
          }
          const bool full = ins[u] && p[u] >= 4;
          bk[u] = full ? ((bk[u] + 1) & bmask) : bk[u];
          ins[u] = full;
        }
      }
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        const int i = base + u * kThreads + tid;
        if (in_k(i)) s_out[i] = o[u];
      }
      if (lane == 0 && npend) atomicAdd(s_pending, npend);
    }
  };

  // ---- 2. LRU scan (hashed plans): probe each slot's token ----------------
  // Wave w walks its own 64-aligned segment of LRU positions. A slot whose
  // token is pending is a hit and serves that top-k entry; the first claimant
  // wins (a second slot with the same token -- corrupt state -- stays
  // evictable instead of serving the entry twice).
  // Returns the wave's hits.
  auto probe = [&](auto salted_tag, uint32_t salt) -> int {
    constexpr bool kSalted = decltype(salted_tag)::value;
    int run = 0;
    for (int c0 = 0; c0 < segH; c0 += 4 * kWave) {
      int32_t sl[4], key[4], idx[4];
      uint32_t bk[4];
      bool act[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = h0 + c0 + u * kWave + lane;
        sl[u] = c0 == 0 ? vl[u] : ((in_seg_h(c0 + u * kWave) && in_h(p)) ? s_lru[p] : -1);
      }
      // Each slot's hot row, worked out beside the token read (with paged
      // addressing it is an LDS table read of its own, kept off the CAS's path).
      int32_t rw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) rw[u] = row_of((sl[u] >= 0 && sl[u] < H) ? sl[u] : 0);
      // The staging choice is uniform: branching once keeps all four token
      // reads of a lane in flight together.
      // Reads at a clamped index and a select afterwards, rather than reads
      // under a lane mask: no exec-mask bookkeeping between the four reads.
      bool okl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) okl[u] = sl[u] >= 0 && sl[u] < H;
      if (a.stage_tokens) {
#pragma unroll
        for (int u = 0; u < 4; ++u) key[u] = lds_read(&s_tok[okl[u] ? sl[u] : 0]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) key[u] = tokens[okl[u] ? sl[u] : 0];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) key[u] = okl[u] ? key[u] : -1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        act[u] = key[u] >= 0;
        idx[u] = -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        bk[u] = kSalted ? bucket_salted(key[u], salt, bshift) : bucket_knuth(key[u], bshift);
      // Branch-free lookup step over one bucket (four keys, 16 bytes) per
      // query. Buckets fill in entry order, so a bucket whose last key is empty
      // is not full and ends a miss. Ends when no lane of the wave is still
      // searching; the top-k index of each found key is read once afterwards.
      // The bucket's four top-k indices (8 bytes) are read beside its keys, so
      // a found key's index needs no further LDS round trip.
      int trips = 0;
      while (__ballot(act[0] | act[1] | act[2] | act[3]) != 0) {
        if (!kSalted && ++trips > kTripLimit) {   // clustered: fall back (uniform per wave)
          if (lane == 0) *s_retry = 1;
          break;
        }
        u32x4 kv[4];
        uint64_t iv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kv[u] = reinterpret_cast<const u32x4*>(hkey)[bk[u]];
          iv[u] = reinterpret_cast<const uint64_t*>(hidx)[bk[u]];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int32_t kk = key[u];
          const bool m0 = static_cast<int32_t>(kv[u].x) == kk;
          const bool m1 = static_cast<int32_t>(kv[u].y) == kk;
          const bool m2 = static_cast<int32_t>(kv[u].z) == kk;
          const bool m3 = static_cast<int32_t>(kv[u].w) == kk;
          const bool found = m0 | m1 | m2 | m3;
          const uint32_t j = m0 ? 0u : (m1 ? 1u : (m2 ? 2u : 3u));
          const bool open = static_cast<int32_t>(kv[u].w) == -1;
          const int ii = static_cast<int16_t>(static_cast<uint32_t>(iv[u] >> (16 * j)) & 0xffffu);
          const int take = -static_cast<int>(act[u] && found);   // all ones or zero
          idx[u] = (ii & take) | (idx[u] & ~take);
          act[u] = act[u] && !found && !open;
          bk[u] = act[u] ? ((bk[u] + 1) & bmask) : bk[u];
        }
      }
      int32_t prev[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        prev[u] = atomicCAS(idx[u] >= 0 ? &s_out[idx[u]] : sink32, kPending, idx[u] >= 0 ? rw[u] : 0);
      // The chunk's hit words (one per 64 positions) leave in one store from
      // lanes 0-3; words past the row or the segment are not written.
      uint64_t mw = 0;
      int nw = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool hit = idx[u] >= 0 && prev[u] == kPending;
        const uint64_t m = __ballot(hit);
        const int p0 = h0 + c0 + u * kWave;
        if (in_seg_h(c0 + u * kWave) && in_h(p0)) {   // uniform, and true for a prefix of u
          mw = lane == u ? m : mw;
          run += __popcll(m);
          ++nw;
        }
      }
      if (lane < nw) hitpos[((h0 + c0) >> 6) + lane] = mw;
    }
    return run;
  };

  // Either plan below yields the hits among the LRU positions before this
  // wave's segment and in all, and M, the misses (pending ids that take a slot).
  int hits = 0, hits_before = 0, M = 0;
  // Direct plans keep the wave's first top-k chunks in registers from the
  // lookup to the write-out: the ids (vi), their outputs and miss words.
  [[maybe_unused]] int32_t vo[kKU];
  [[maybe_unused]] uint64_t vmw[kKU];
  if constexpr (kDirect) {
    // ---- 1-2, lookup plans: a table of the resident slots, one lookup per id --
    // Flat layout (the direct table): while the rows land, every slot 0..H-1
    // writes its index into the table entry of the position it holds. A
    // pending id is then a hit when its entry names a slot that holds it: two
    // dependent LDS reads (entry, then the slot's token and LRU position side
    // by side) per id, K lookups instead of H probes. The table is never
    // cleared; the token check rejects stale entries.
    // Paged addressing (keys are global ids, which span the whole pool): the
    // slots' keys go into the bucketed hash instead (key -> slot), and each
    // pending id's global id is looked up there. A chain past kTripLimit
    // buckets, in an insert or a lookup, rebuilds the hash with the salted
    // hash, as the hashed plans do.
    // Either way every LRU position writes its index into the entry of the
    // slot it names (pos_of), and a hit sets its LRU position's bit in the hit
    // words, so the victim step finds hits in LRU order without another pass.
    int16_t* pos_of = nlru;   // free until the new order is built
    int16_t* sink16 = reinterpret_cast<int16_t*>(sink64);
    int32_t vt[kHU];
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int i = k0 + u * kWave + lane;
      vi[u] = (in_seg_k(u * kWave) && in_k(i)) ? ids[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = h0 + u * kWave + lane;
      vl[u] = (in_seg_h(u * kWave) && in_h(p)) ? lru[p] : static_cast<int16_t>(-1);
    }
#pragma unroll
    for (int u = 0; u < kHU; ++u) {
      const int x = u * kThreads + tid;
      vt[u] = in_h(x) ? tokens[x] : -1;
    }
    const int nwh = (H + kWave - 1) / kWave;    // hit words
    for (int i = tid; i < nwh; i += kThreads) hitpos[i] = 0;
    if (tid < 2 * (kWaves + 1) + 2) wtot[tid] = 0;
    if constexpr (kPaged) {
      // The request's hot and source block table rows (every slot -> row and
      // position -> global id translation then stays in LDS), and the
      // bucket counts of the key hash, cleared before the first insert.
      int32_t* hb = reinterpret_cast<int32_t*>(lds + lay.hbt);
      for (int i = tid; i < a.hbt_n; i += kThreads) hb[i] = a.hbt[r * a.hbt_stride + i];
      int32_t* sb = reinterpret_cast<int32_t*>(lds + lay.sbt);
      for (int i = tid; i < a.sbt_n; i += kThreads) sb[i] = a.sbt[r * a.sbt_stride + i];
      u32x4* c4 = reinterpret_cast<u32x4*>(bcnt);
      for (uint32_t i = tid; i < a.T / 16; i += kThreads) c4[i] = u32x4{0u, 0u, 0u, 0u};
    }
    for (int c0 = kKU * kWave; c0 < segK; c0 += kKU * kWave) {   // K > 2048
      int32_t w[kKU];
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        const int i = k0 + c0 + u * kWave + lane;
        w[u] = (in_seg_k(c0 + u * kWave) && in_k(i)) ? ids[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        const int i = k0 + c0 + u * kWave + lane;
        if (in_seg_k(c0 + u * kWave) && in_k(i)) s_topk[i] = w[u];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = h0 + u * kWave + lane;
      if (in_seg_h(u * kWave) && in_h(p))
        *((static_cast<uint16_t>(vl[u]) < static_cast<uint32_t>(H)) ? &pos_of[vl[u]] : sink16) =
            static_cast<int16_t>(p);
    }
    if constexpr (!kPaged) {
#pragma unroll
      for (int u = 0; u < kHU; ++u) {
        const int x = u * kThreads + tid;
        if (in_h(x)) {
          if (a.stage_tokens) s_tok[x] = vt[u];
          *((static_cast<uint32_t>(vt[u]) < a.dtab) ? &dtab[vt[u]] : sink16) = static_cast<int16_t>(x);
        }
      }
    }
    for (int c0 = 4 * kWave; c0 < segH; c0 += 4 * kWave) {    // H > 4096
      int16_t wl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = h0 + c0 + u * kWave + lane;
        wl[u] = (in_seg_h(c0 + u * kWave) && in_h(p)) ? lru[p] : static_cast<int16_t>(-1);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = h0 + c0 + u * kWave + lane;
        if (in_seg_h(c0 + u * kWave) && in_h(p)) {
          s_lru[p] = wl[u];
          *((static_cast<uint16_t>(wl[u]) < static_cast<uint32_t>(H)) ? &pos_of[wl[u]] : sink16) =
              static_cast<int16_t>(p);
        }
      }
    }
    if constexpr (!kPaged) {
      for (int base = kHU * kThreads; base < H; base += 4 * kThreads) {
        int32_t wt[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int x = base + u * kThreads + tid;
          wt[u] = in_h(x) ? tokens[x] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int x = base + u * kThreads + tid;
          if (in_h(x)) {
            if (a.stage_tokens) s_tok[x] = wt[u];
            *((static_cast<uint32_t>(wt[u]) < a.dtab) ? &dtab[wt[u]] : sink16) = static_cast<int16_t>(x);
          }
        }
      }
    }
    __syncthreads();

    // Paged: every slot's key into the hash. A slot takes the next entry of
    // its key's home bucket with one LDS atomicAdd on the bucket's count; a
    // full bucket passes the key on to the next bucket.
    [[maybe_unused]] auto insert_keys = [&](auto salted_tag, uint32_t salt) {
      constexpr bool kSalted = decltype(salted_tag)::value;
      for (int base = 0; base < H; base += kHU * kThreads) {
        int32_t key[kHU];
        uint32_t bk[kHU];
        bool ins[kHU];
#pragma unroll
        for (int u = 0; u < kHU; ++u) {
          const int x = base + u * kThreads + tid;
          key[u] = (!kSalted && base == 0) ? vt[u] : (in_h(x) ? tokens[x] : -1);
          ins[u] = in_h(x) && key[u] >= 0;
          bk[u] = kSalted ? bucket_salted(key[u], salt, bshift) : bucket_knuth(key[u], bshift);
        }
        int trips = 0;
        while (__ballot(any_of(ins)) != 0) {
          if (!kSalted && ++trips > kTripLimit) {   // clustered: fall back (uniform per wave)
            if (lane == 0) *s_retry = 1;
            break;
          }
          uint32_t pq[kHU];
#pragma unroll
          for (int u = 0; u < kHU; ++u) pq[u] = atomicAdd(ins[u] ? &bcnt[bk[u]] : sinku, 1u);
#pragma unroll
          for (int u = 0; u < kHU; ++u) {
            if (ins[u] && pq[u] < 4) {
              hkey[4 * bk[u] + pq[u]] = key[u];
              hidx[4 * bk[u] + pq[u]] = static_cast<int16_t>(base + u * kThreads + tid);
            }
            const bool full = ins[u] && pq[u] >= 4;
            bk[u] = full ? ((bk[u] + 1) & bmask) : bk[u];
            ins[u] = full;
          }
        }
      }
    };

    // Lookup: each wave classifies and looks up its own segment of top-k
    // entries, records its miss words and adds its miss total to the later
    // waves' prefixes. Paged: the ids come from global memory again on the
    // salted pass, and the key (global id) replaces the id in vi / s_topk
    // for the write-out.
    auto lookup = [&](auto salted_tag, uint32_t salt) {
      constexpr bool kSalted = decltype(salted_tag)::value;
      int mrun = 0;
      for (int c0 = 0; c0 < segK && in_k(k0 + c0); c0 += kKU * kWave) {
        int32_t t[kKU], key[kKU], o[kKU], sl[kKU], tk[kKU], pp[kKU];
        bool inr[kKU], pend[kKU], ok[kKU], hit[kKU];
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          const int i = k0 + c0 + u * kWave + lane;
          inr[u] = in_seg_k(c0 + u * kWave) && in_k(i);
          t[u] = kSalted ? (inr[u] ? ids[i] : 0) : (c0 == 0 ? vi[u] : (inr[u] ? s_topk[i] : 0));
        }
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          if constexpr (kPaged) {
            int64_t g = -1, res = -1;
            if (inr[u]) translate(t[u], g, res);
            pend[u] = inr[u] && res < 0 && g >= 0;
            o[u] = res >= 0 ? static_cast<int32_t>(res) : (g >= 0 ? kPending : -1);
            key[u] = static_cast<int32_t>(g);
          } else {
            const bool valid = inr[u] && static_cast<uint32_t>(t[u]) < lim;
            const bool newest = valid && t[u] == newest_t;
            pend[u] = valid && !newest;
            o[u] = !valid ? -1 : (newest ? row_newest : kPending);
            key[u] = t[u];
          }
        }
        if constexpr (kPaged) {
          // Branch-free steps over one bucket per query: its four keys, its
          // count (entries past the count are not this call's) and its four
          // slot indices, read side by side. Ends when no lane of the wave is
          // still searching.
          bool act[kKU];
          uint32_t bk[kKU];
#pragma unroll
          for (int u = 0; u < kKU; ++u) {
            act[u] = pend[u];
            sl[u] = -1;
            bk[u] = kSalted ? bucket_salted(key[u], salt, bshift) : bucket_knuth(key[u], bshift);
          }
          int trips = 0;
          while (__ballot(any_of(act)) != 0) {
            if (!kSalted && ++trips > kTripLimit) {   // clustered: fall back (uniform per wave)
              if (lane == 0) *s_retry = 1;
              break;
            }
            u32x4 kv[kKU];
            uint64_t iv[kKU];
            uint32_t cn[kKU];
#pragma unroll
            for (int u = 0; u < kKU; ++u) {
              kv[u] = reinterpret_cast<const u32x4*>(hkey)[bk[u]];
              iv[u] = reinterpret_cast<const uint64_t*>(hidx)[bk[u]];
              cn[u] = bcnt[bk[u]];
            }
#pragma unroll
            for (int u = 0; u < kKU; ++u) {
              const int32_t kk = key[u];
              const bool m0 = cn[u] > 0 && static_cast<int32_t>(kv[u].x) == kk;
              const bool m1 = cn[u] > 1 && static_cast<int32_t>(kv[u].y) == kk;
              const bool m2 = cn[u] > 2 && static_cast<int32_t>(kv[u].z) == kk;
              const bool m3 = cn[u] > 3 && static_cast<int32_t>(kv[u].w) == kk;
              const bool found = m0 | m1 | m2 | m3;
              const uint32_t j = m0 ? 0u : (m1 ? 1u : (m2 ? 2u : 3u));
              const int ii = static_cast<int16_t>(static_cast<uint32_t>(iv[u] >> (16 * j)) & 0xffffu);
              sl[u] = (act[u] && found) ? ii : sl[u];
              act[u] = act[u] && !found && cn[u] >= 4;
              bk[u] = act[u] ? ((bk[u] + 1) & bmask) : bk[u];
            }
          }
#pragma unroll
          for (int u = 0; u < kKU; ++u) {
            ok[u] = pend[u] && static_cast<uint32_t>(sl[u]) < static_cast<uint32_t>(H);
            tk[u] = key[u];   // the hash holds exact keys: no token check
          }
        } else {
#pragma unroll
          for (int u = 0; u < kKU; ++u) sl[u] = dtab[pend[u] ? t[u] : 0];
#pragma unroll
          for (int u = 0; u < kKU; ++u) ok[u] = pend[u] && static_cast<uint32_t>(sl[u]) < static_cast<uint32_t>(H);
          if (a.stage_tokens) {
#pragma unroll
            for (int u = 0; u < kKU; ++u) tk[u] = lds_read(&s_tok[ok[u] ? sl[u] : 0]);
          } else {
#pragma unroll
            for (int u = 0; u < kKU; ++u) tk[u] = tokens[ok[u] ? sl[u] : 0];
          }
        }
#pragma unroll
        for (int u = 0; u < kKU; ++u) pp[u] = pos_of[ok[u] ? sl[u] : 0];
#pragma unroll
        for (int u = 0; u < kKU; ++u)
          hit[u] = ok[u] && tk[u] == key[u] && static_cast<uint32_t>(pp[u]) < static_cast<uint32_t>(H);
#pragma unroll
        for (int u = 0; u < kKU; ++u)
          atomicOr(hit[u] ? reinterpret_cast<unsigned long long*>(&hitpos[pp[u] >> 6]) : sink64,
                   hit[u] ? 1ull << (pp[u] & 63) : 0ull);
#pragma unroll
        for (int u = 0; u < kKU; ++u) o[u] = hit[u] ? row_of(sl[u]) : o[u];
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          const uint64_t mm = __ballot(pend[u] && !hit[u]);
          const int q = k0 + c0 + u * kWave;
          if (in_seg_k(c0 + u * kWave) && in_k(q)) {   // uniform
            if (lane == 0) missw[q >> 6] = mm;
            mrun += __popcll(mm);
          }
          if (c0 == 0) {
            vo[u] = o[u];
            vmw[u] = mm;
            if constexpr (kPaged) vi[u] = key[u];
          } else if (inr[u]) {
            s_out[q + lane] = o[u];
            if constexpr (kPaged) s_topk[q + lane] = key[u];
          }
        }
      }
      if (lane > wave && lane <= kWaves && mrun) atomicAdd(&pre_miss[lane], mrun);
    };

    if constexpr (kPaged) {
      insert_keys(std::false_type{}, 0u);
      __syncthreads();
      if (*s_retry == 0) lookup(std::false_type{}, 0u);
      __syncthreads();
      if (*s_retry != 0) {   // uniform: nothing writes the flag before the barrier below
        // Fallback: once every lane has read the flag, clear the counts, the
        // hit words and the cross-wave counters (the flag with them), then
        // insert and look up again with the salted hash.
        __syncthreads();
        u32x4* c4 = reinterpret_cast<u32x4*>(bcnt);
        for (uint32_t i = tid; i < a.T / 16; i += kThreads) c4[i] = u32x4{0u, 0u, 0u, 0u};
        for (int i = tid; i < nwh; i += kThreads) hitpos[i] = 0;
        if (tid < 2 * (kWaves + 1) + 2) wtot[tid] = 0;
        if (tid == 0) {   // the salt, fresh per workgroup and call
          const uint64_t z = static_cast<uint64_t>(clock64()) ^ (static_cast<uint64_t>(b) << 40);
          *s_salt = static_cast<uint32_t>(mix64(z + 0x9E3779B97F4A7C15ull));
        }
        __syncthreads();
        const uint32_t salt = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(*s_salt));
        insert_keys(std::true_type{}, salt);
        __syncthreads();
        lookup(std::true_type{}, salt);
        __syncthreads();
      }
    } else {
      lookup(std::false_type{}, 0u);
      __syncthreads();
    }
    // Hits before this wave's LRU segment, and in all, from the hit words:
    // both counts packed in one word (each at most H <= 32768) and summed
    // over the wave.
    uint32_t acc = 0;
    const int wbeg = h0 >> 6;
    for (int w = lane; w < nwh; w += kWave) {
      const uint32_t c = static_cast<uint32_t>(__popcll(hitpos[w]));
      acc += (c << 16) + (w < wbeg ? c : 0u);
    }
    acc = wave_sum(acc);
    hits = static_cast<int>(acc >> 16);
    hits_before = static_cast<int>(acc & 0xffffu);
    M = pre_miss[kWaves];
  } else {
  // ---- stage (hashed plans) ----------------------------------------------------
  {
    int32_t vt[kHU];
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int x = u * kThreads + tid;
      vi[u] = in_k(x) ? ids[x] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = h0 + u * kWave + lane;
      vl[u] = (in_seg_h(u * kWave) && in_h(p)) ? lru[p] : static_cast<int16_t>(-1);
    }
#pragma unroll
    for (int u = 0; u < kHU; ++u) {
      const int x = u * kThreads + tid;
      vt[u] = (a.stage_tokens && in_h(x)) ? tokens[x] : 0;
    }
    {
      // Keys start empty (-1, never a token id) and bucket counts at 0.
      u32x4* k4 = reinterpret_cast<u32x4*>(hkey);
      for (uint32_t i = tid; i < a.T / 4; i += kThreads) k4[i] = u32x4{~0u, ~0u, ~0u, ~0u};
      u32x4* c4 = reinterpret_cast<u32x4*>(bcnt);
      for (uint32_t i = tid; i < a.T / 16; i += kThreads) c4[i] = u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < 2 * (kWaves + 1) + 2) wtot[tid] = 0;   // prefixes and the retry flag
    if constexpr (kPaged) {
      // The request's hot block table row: every slot -> row translation in
      // the probe and the assign step then stays in LDS.
      int32_t* hb = reinterpret_cast<int32_t*>(lds + lay.hbt);
      for (int i = tid; i < a.hbt_n; i += kThreads) hb[i] = a.hbt[r * a.hbt_stride + i];
      // ... and the source block table row, so classifying an id needs no
      // dependent HBM read.
      int32_t* sb = reinterpret_cast<int32_t*>(lds + lay.sbt);
      for (int i = tid; i < a.sbt_n; i += kThreads) sb[i] = a.sbt[r * a.sbt_stride + i];
    }
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int x = u * kThreads + tid;
      if (in_k(x)) s_topk[x] = vi[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = h0 + u * kWave + lane;
      if (in_seg_h(u * kWave) && in_h(p)) s_lru[p] = vl[u];
    }
    if (a.stage_tokens) {
#pragma unroll
      for (int u = 0; u < kHU; ++u) {
        const int x = u * kThreads + tid;
        if (in_h(x)) s_tok[x] = vt[u];
      }
    }
  }
  for (int base = kKU * kThreads; base < K; base += 4 * kThreads) {
    int32_t wi[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = base + u * kThreads + tid;
      wi[u] = x < K ? ids[x] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = base + u * kThreads + tid;
      if (x < K) s_topk[x] = wi[u];
    }
  }
  for (int c0 = 4 * kWave; c0 < segH; c0 += 4 * kWave) {    // H > 4096
    int16_t wl[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = h0 + c0 + u * kWave + lane;
      wl[u] = (in_seg_h(c0 + u * kWave) && in_h(p)) ? lru[p] : static_cast<int16_t>(0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = h0 + c0 + u * kWave + lane;
      if (in_seg_h(c0 + u * kWave) && in_h(p)) s_lru[p] = wl[u];
    }
  }
  if (a.stage_tokens) {
    for (int base = kHU * kThreads; base < H; base += 4 * kThreads) {
      int32_t wt[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int x = base + u * kThreads + tid;
        wt[u] = in_h(x) ? tokens[x] : 0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int x = base + u * kThreads + tid;
        if (in_h(x)) s_tok[x] = wt[u];
      }
    }
  }
  __syncthreads();
  classify_insert(std::false_type{}, 0u);
  __syncthreads();
  int pending_n = *s_pending;
  int run = *s_retry == 0 ? probe(std::false_type{}, 0u) : 0;
  // Wave w adds its total to the prefix of every later wave and to the grand
  // total: one LDS atomic per lane, no scan after the barrier.
  if (lane > wave && lane <= kWaves && run) atomicAdd(&pre_hit[lane], run);
  __syncthreads();
  hits = pre_hit[kWaves];
  hits_before = pre_hit[wave];
  if (*s_retry != 0) {   // uniform: nothing writes the flag before the barrier below
    // Fallback: once every lane has read the flag, clear the table, its
    // counts and the cross-wave counters (the flag with them), then run
    // classification and the scan again with the salted hash.
    __syncthreads();
    u32x4* k4 = reinterpret_cast<u32x4*>(hkey);
    for (uint32_t i = tid; i < a.T / 4; i += kThreads) k4[i] = u32x4{~0u, ~0u, ~0u, ~0u};
    u32x4* c4 = reinterpret_cast<u32x4*>(bcnt);
    for (uint32_t i = tid; i < a.T / 16; i += kThreads) c4[i] = u32x4{0u, 0u, 0u, 0u};
    if (tid < 2 * (kWaves + 1) + 2) wtot[tid] = 0;
    if (tid == 0) {   // the salt, fresh per workgroup and call
      const uint64_t z = static_cast<uint64_t>(clock64()) ^ (static_cast<uint64_t>(b) << 40);
      *s_salt = static_cast<uint32_t>(mix64(z + 0x9E3779B97F4A7C15ull));
    }
    __syncthreads();
    // The same for the whole workgroup (a scalar register).
    const uint32_t salt = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(*s_salt));
    classify_insert(std::true_type{}, salt);
    __syncthreads();
    pending_n = *s_pending;
    run = probe(std::true_type{}, salt);
    if (lane > wave && lane <= kWaves && run) atomicAdd(&pre_hit[lane], run);
    __syncthreads();
    hits = pre_hit[kWaves];
    hits_before = pre_hit[wave];
  }
  M = pending_n - hits;    // misses (<= E because K <= H)
  }  // hashed plans

  // ---- 3. miss words, (host pools) early row loads, victims, new LRU order ---
  // New order: stale evictables, then the M victims (they receive the misses,
  // in miss order), then the hits -- every group in its old order. A
  // position's rank among hits is the hits of earlier waves, plus this wave's
  // earlier chunks, plus the hit lanes below it.
  const int E = H - hits;            // evictable slots
  // The fused copy's list (pool row, hot row) in miss order, kept in the table
  // region, which is free once the probe or the lookup is done (the layout
  // gives it at least 12K bytes).
  int64_t* l_src = reinterpret_cast<int64_t*>(lds + lay.hash);
  int32_t* l_dst = reinterpret_cast<int32_t*>(lds + lay.hash + 8u * static_cast<uint32_t>(K));
  // Hashed plans: an id still pending after the probe is a miss. Each wave
  // records its segment's miss words and adds its miss total to the later
  // waves' prefixes (the direct plans' lookup has done so already).
  auto miss_words = [&]() {
    int mrun = 0;
    for (int c0 = 0; c0 < segK && in_k(k0 + c0); c0 += kKU * kWave) {
      int32_t so[kKU];
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        const int i = k0 + c0 + u * kWave + lane;
        so[u] = (in_seg_k(c0 + u * kWave) && in_k(i)) ? s_out[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < kKU; ++u) {
        const int q = k0 + c0 + u * kWave;
        const uint64_t mm = __ballot(so[u] == kPending);
        if (in_seg_k(c0 + u * kWave) && in_k(q)) {
          if (lane == 0) missw[q >> 6] = mm;
          mrun += __popcll(mm);
        }
      }
    }
    if (lane > wave && lane <= kWaves && mrun) atomicAdd(&pre_miss[lane], mrun);
  };
  // Host pools: the pool row of every miss is known now; only its hot row
  // waits for the victims. The first kEarlyChunks chunks of every lane are
  // loaded here, in the fused copy's order, so the host link gets this
  // request's first reads before the victims and outputs are worked out. The
  // workgroup pauses until they are back: the generated code waits for each
  // load at once (under its branch the loaded value and the no-load path
  // share a register), and with no branch phase 4's global stores queue
  // behind the outstanding host reads instead. One per lane: with a whole
  // round (kFuseUnroll per lane) outstanding the link moved less and the
  // call got no faster; one per lane saves ~2% on the DeepSeek-V3.2-like step.
  constexpr bool kEarlyCopy = kEarlyChunks > 0 && kCopyW != 0 && !kSlotRows && !kPoolRows;
  const bool early = kEarlyCopy && (!kPaged || a.hbt_n != 0);   // uniform
  typedef Chunk<kCopyW == 0 ? 4 : kCopyW> CE;
  [[maybe_unused]] typename CE::T ev[kEarlyChunks > 0 ? kEarlyChunks : 1];
  if constexpr (kEarlyCopy) {
    if (early) {
      if constexpr (!kDirect) {
        miss_words();
        __syncthreads();
      }
      int mrun = pre_miss[wave];
      for (int c0 = 0; c0 < segK && in_k(k0 + c0); c0 += kKU * kWave) {
        uint64_t wd[kKU];
        int32_t t[kKU];
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          const int q = k0 + c0 + u * kWave;
          const int i = q + lane;
          const bool in = in_seg_k(c0 + u * kWave) && in_k(q);
          wd[u] = in ? ((kDirect && c0 == 0) ? vmw[u] : missw[q >> 6]) : 0;
          t[u] = (in && in_k(i)) ? ((kDirect && c0 == 0) ? vi[u] : s_topk[i]) : 0;
        }
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
          if ((wd[u] >> lane) & 1ull) l_src[mrun + rank_below(wd[u])] = pool_of(t[u]);
          mrun += __popcll(wd[u]);
        }
      }
      __syncthreads();
      // Every earlier global load returned long ago; saying so keeps the
      // compiler from waiting for them later, which (the counter retires in
      // order) would mean waiting for these loads as well.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      const uint32_t C = a.cdiv.d;
      const bool kv = a.pool_v != nullptr;
      const uint32_t total = static_cast<uint32_t>(pre_miss[kWaves]) * (kv ? 2u : 1u) * C;
#pragma unroll
      for (int u = 0; u < kEarlyChunks; ++u) {
        const uint32_t j = tid + u * kThreads;
        ev[u] = typename CE::T{};
        if (j < total) {
          const uint32_t q = fdiv(j, a.cdiv);     // (miss, K/V) row
          const uint32_t c = j - q * C;
          const int64_t sr = l_src[kv ? q >> 1 : q];
          if (sr >= 0 && sr < a.pool_nrows)
            ev[u] = CE::load(((kv && (q & 1)) ? a.pool_v : a.pool) + sr * a.row_bytes +
                             static_cast<int64_t>(c) * kCopyW);
        }
      }
    }
  }
  int run = hits_before;
  int16_t* sink16 = reinterpret_cast<int16_t*>(sink64);
  for (int c0 = 0; c0 < segH && in_h(h0 + c0); c0 += 4 * kWave) {
    // The chunk's four hit words arrive in one LDS read (lanes 0-3) and are
    // broadcast with readlane, so no read waits on the one before it.
    int16_t sp[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = h0 + c0 + u * kWave;     // chunk start
      const bool in = in_seg_h(c0 + u * kWave) && in_h(q);
      sp[u] = c0 == 0 ? vl[u] : ((in && in_h(q + lane)) ? s_lru[q + lane] : static_cast<int16_t>(0));
    }
    const uint64_t wl = (lane < 4 && in_seg_h(c0 + lane * kWave)) ? hitpos[((h0 + c0) >> 6) + lane] : 0;
    uint64_t wd[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = h0 + c0 + u * kWave;
      const bool in = in_seg_h(c0 + u * kWave) && in_h(q);
      const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(wl), u);
      const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(wl >> 32), u);
      wd[u] = in ? (static_cast<uint64_t>(hi) << 32 | lo) : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = h0 + c0 + u * kWave + lane;
      if (in_seg_h(c0 + u * kWave)) {       // uniform
        const bool h = (wd[u] >> lane) & 1ull;
        const int hr = run + rank_below(wd[u]);
        const int e = p - hr;              // rank among evictables
        const bool vic = !h && e < M;
        // hit: E + hr; victim: E - M + e; other evictable: e - M
        const int hm = -static_cast<int>(h);
        const int np = (hm & (E + hr)) | (~hm & (e - M + (vic ? E : 0)));
        if (in_h(p)) {
          // Lanes that are not victims write their private sink instead,
          // which keeps this step free of branches.
          *(vic ? &victim[e] : sink16) = sp[u];
          nlru[np] = sp[u];
        }
      }
      run += __popcll(wd[u]);
    }
  }
  if (!kDirect && !early) miss_words();
  __syncthreads();

  // ---- 4. misses in top-k order take victims; outputs; copy list -----------
  // Each wave finishes its own segment of top-k entries: the entries it does
  // not fill were final before the last barrier.
  const int m_total = pre_miss[kWaves];
  const int miss_before = pre_miss[wave];
  int64_t* ws_src = a.src + static_cast<int64_t>(b) * K;
  int32_t* ws_dst = a.dst + static_cast<int64_t>(b) * K;
  int32_t* mask = a.miss_mask ? a.miss_mask + static_cast<int64_t>(b) * K : nullptr;
  run = miss_before;
  for (int c0 = 0; c0 < segK && in_k(k0 + c0); c0 += kKU * kWave) {
    uint64_t wd[kKU];
    int32_t so[kKU], t[kKU];
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int q = k0 + c0 + u * kWave;
      const int i = q + lane;
      const bool in = in_seg_k(c0 + u * kWave) && in_k(q);
      wd[u] = in ? ((kDirect && c0 == 0) ? vmw[u] : missw[q >> 6]) : 0;
      so[u] = (in && in_k(i)) ? ((kDirect && c0 == 0) ? vo[u] : s_out[i]) : 0;
      t[u] = (in && in_k(i)) ? ((kDirect && c0 == 0) ? vi[u] : s_topk[i]) : 0;
    }
    int m[kKU], v[kKU];
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      m[u] = run + rank_below(wd[u]);
      run += __popcll(wd[u]);
      v[u] = (((wd[u] >> lane) & 1ull) && m[u] < M) ? victim[m[u]] : -1;
    }
#pragma unroll
    for (int u = 0; u < kKU; ++u) {
      const int i = k0 + c0 + u * kWave + lane;
      if (!in_seg_k(c0 + u * kWave) || !in_k(i)) continue;
      int32_t o = so[u];
      const bool missed = ((wd[u] >> lane) & 1ull) && v[u] >= 0 && v[u] < H;
      if (mask) mask[i] = missed ? 1 : 0;
      if ((wd[u] >> lane) & 1ull) {
        int64_t pr = 0;
        if (v[u] >= 0 && v[u] < H) {
          o = row_of(v[u]);
          tokens[v[u]] = t[u];
          pr = pool_of(t[u]);
        } else {
          o = -1;
        }
        ws_src[m[u]] = pr;
        ws_dst[m[u]] = o;
        if constexpr (kCopyW != 0) {
          if (!early) l_src[m[u]] = pr;
          l_dst[m[u]] = o;
        }
      }
      out[i] = o;
      if (kPaged && a.att) {  // vLLM page, store_hot_index
        const int32_t ob = static_cast<int32_t>(fdiv(static_cast<uint32_t>(o < 0 ? 0 : o), a.hbs_div));
        a.att[static_cast<int64_t>(b) * a.att_stride + i] =
            o < 0 ? -1 : static_cast<int32_t>(ob * a.att_block_stride + (o - ob * a.hbs));
      }
    }
  }
  // The new LRU order, built in LDS by phase 3, goes out in one coalesced pass.
  if ((H & 3) == 0 && (reinterpret_cast<uintptr_t>(lru) & 7) == 0) {
    // four slots per 8-byte store
    const uint64_t* n8 = reinterpret_cast<const uint64_t*>(nlru);
    uint64_t* l8 = reinterpret_cast<uint64_t*>(lru);
    for (int q = tid; q < H / 4; q += kThreads) l8[q] = n8[q];
  } else {
    for (int p = tid; p < H; p += kThreads) lru[p] = nlru[p];
  }
  if (tid == 0) {
    a.count[b] = m_total;
    if (a.miss_counts) a.miss_counts[b] = m_total;
    if (a.stats) {   // vLLM hisparse_kernels.cu, stats: hits, misses
      atomicAdd(&a.stats[0], static_cast<unsigned long long>(hits));
      atomicAdd(&a.stats[1], static_cast<unsigned long long>(m_total));
    }
  }

  // ---- 5. (host pools) the request's own row copies -------------------------
  // The workgroup copies its misses straight from the LDS list, as soon as its
  // own resolution is done, in rounds of kFuseUnroll chunks per lane. This
  // saves a second launch and its start-up and drain. The generated code
  // waits for each read before issuing the next, so a lane keeps about one
  // read in flight. A few dozen workgroups of 1024 lanes fill the host link
  // that way, and rewrites with every read of a round in flight moved less
  // over the link, so the loop stays in this plain form.
  if constexpr (kCopyW != 0) {
    typedef Chunk<kCopyW> CW;
    __syncthreads();
    const uint32_t C = a.cdiv.d;
    const bool kv = a.pool_v != nullptr;    // uniform: a V row per miss too
    const uint32_t total = static_cast<uint32_t>(m_total) * (kv ? 2u : 1u) * C;
    uint32_t j_first = tid;
    if constexpr (kEarlyCopy) {
      if (early) {   // the chunks loaded in phase 3 go to their hot rows now
#pragma unroll
        for (int u = 0; u < kEarlyChunks; ++u) {
          const uint32_t j = tid + u * kThreads;
          if (j < total) {
            const uint32_t q = fdiv(j, a.cdiv);
            const uint32_t c = j - q * C;
            const uint32_t mm = kv ? q >> 1 : q;
            const int64_t sr = l_src[mm];
            const int32_t hr = l_dst[mm];
            if (sr >= 0 && sr < a.pool_nrows && hr >= 0 && hr < a.hot_nrows)
              CW::store(((kv && (q & 1)) ? a.hot_v : a.hot) + static_cast<int64_t>(hr) * a.row_bytes +
                            static_cast<int64_t>(c) * kCopyW,
                        ev[u]);
          }
        }
        j_first += kEarlyChunks * kThreads;
      }
    }
    for (uint32_t j0 = j_first; j0 < total; j0 += kThreads * kFuseUnroll) {
      typename CW::T cv[kFuseUnroll];
      char* cd[kFuseUnroll];
#pragma unroll
      for (int u = 0; u < kFuseUnroll; ++u) {
        const uint32_t j = j0 + u * kThreads;
        cd[u] = nullptr;
        if (j < total) {
          const uint32_t q = fdiv(j, a.cdiv);     // (miss, K/V) row
          const uint32_t c = j - q * C;
          const uint32_t mm = kv ? q >> 1 : q;
          const bool isv = kv && (q & 1);
          const int64_t sr = l_src[mm];
          const int32_t hr = l_dst[mm];
          if (sr >= 0 && sr < a.pool_nrows && hr >= 0 && hr < a.hot_nrows) {
            const int64_t off = static_cast<int64_t>(c) * kCopyW;
            cv[u] = CW::load((isv ? a.pool_v : a.pool) + sr * a.row_bytes + off);
            cd[u] = (isv ? a.hot_v : a.hot) + static_cast<int64_t>(hr) * a.row_bytes + off;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kFuseUnroll; ++u)
        if (cd[u]) CW::store(cd[u], cv[u]);
    }
  }
}

// Resolve: one 1024-lane workgroup per batch row. Publishes the miss list
// (pool row, hot row) and its length to the workspace for the copy kernel;
// with kCopyW != 0 also copies the rows itself (W-byte chunks).
template <bool kSlotRows, bool kPoolRows, int kCopyW, bool kPaged, bool kExact, bool kDirect>
__global__ __launch_bounds__(kThreads) void resolve_kernel(SwapArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const LdsLayout lay = lds_layout(a.K, a.H, a.T, a.stage_tokens != 0, static_cast<uint32_t>(a.hbt_n),
                                   static_cast<uint32_t>(a.sbt_n), a.dtab);
  resolve<kSlotRows, kPoolRows, kCopyW, kPaged, kExact, kDirect>(a, blockIdx.x, lds, lay);
}

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct WsLayout {
  size_t count, src, dst, total;
};

inline WsLayout ws_layout(int64_t B, int64_t K) {
  WsLayout w;
  w.count = 0;
  w.src = w.count + align256(4 * static_cast<size_t>(B));
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

namespace {

constexpr int kEmptyCall = 1;  // internal: nothing to launch

// Opt a resolve kernel in to more than 64 KB of dynamic LDS (gfx950 has
// 160 KB per CU), once per device, kernel and size.
int allow_lds(int device, const void* fn, uint32_t bytes) {
  static std::mutex mu;
  struct Entry { int device; const void* fn; uint32_t bytes; };
  static Entry done[64];
  static int n = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n; ++i)
    if (done[i].device == device && done[i].fn == fn && done[i].bytes >= bytes) return HS_OK;
  const hipError_t fe = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                            static_cast<int>(bytes));
  if (fe != hipSuccess) {
    (void)hipGetLastError();
    return set_error(HS_ERANGE, "cannot raise dynamic LDS to %u bytes: %s", bytes,
                     hipGetErrorString(fe));
  }
  if (n < 64) done[n++] = Entry{device, fn, bytes};
  return HS_OK;
}

// The resolve kernel for the given tables and fused copy width (0 = none).
// `exact` (K a multiple of kKU * 1024, H of kHU * 1024) selects the
// instantiation without tile guards, for the flat and the paged layouts;
// `direct` a lookup per id instead of a probe per slot: the direct-address
// table for the flat layout, the hash of the slots' keys for paged addressing.
template <int kW>
const void* pick_resolve(bool slot_rows, bool pool_rows, bool paged, bool exact, bool direct) {
  if (paged && direct)   // the paged key hash, looked up once per id
    return exact ? reinterpret_cast<const void*>(&resolve_kernel<false, false, kW, true, true, true>)
                 : reinterpret_cast<const void*>(&resolve_kernel<false, false, kW, true, false, true>);
  if (paged)
    return exact ? reinterpret_cast<const void*>(&resolve_kernel<false, false, kW, true, true, false>)
                 : reinterpret_cast<const void*>(&resolve_kernel<false, false, kW, true, false, false>);
  if (slot_rows)
    return pool_rows ? reinterpret_cast<const void*>(&resolve_kernel<true, true, kW, false, false, false>)
                     : reinterpret_cast<const void*>(&resolve_kernel<true, false, kW, false, false, false>);
  if (pool_rows) return reinterpret_cast<const void*>(&resolve_kernel<false, true, kW, false, false, false>);
  if (direct)
    return exact ? reinterpret_cast<const void*>(&resolve_kernel<false, false, kW, false, true, true>)
                 : reinterpret_cast<const void*>(&resolve_kernel<false, false, kW, false, false, true>);
  return exact ? reinterpret_cast<const void*>(&resolve_kernel<false, false, kW, false, true, false>)
               : reinterpret_cast<const void*>(&resolve_kernel<false, false, kW, false, false, false>);
}

// Everything a launch needs, validated once per call.
struct Plan {
  SwapArgs s;
  const void* resolve_fn;   // resolution only
  const void* fused_fn;     // resolution + the request's own copies, or null
  LdsLayout lay;
  bool host_pool;           // the pool is pinned host memory
  int W;
  int64_t C;
  int num_cus;
};

// Point the plan's miss list (count, pool rows, hot rows) into a workspace of
// at least ws_layout(B, K).total bytes, 256-byte aligned.
void bind_workspace(Plan* pl, void* workspace) {
  const WsLayout wl = ws_layout(pl->s.B, pl->s.K);
  char* ws = static_cast<char*>(workspace);
  pl->s.count = reinterpret_cast<int32_t*>(ws + wl.count);
  pl->s.src = reinterpret_cast<int64_t*>(ws + wl.src);
  pl->s.dst = reinterpret_cast<int32_t*>(ws + wl.dst);
}

// Validates the call and fills the plan; the workspace must hold the list.
// With bind_later (the allocation-free entry point only) the workspace
// arguments are ignored and the caller binds its own array afterwards
// (bind_workspace), having checked its size itself.
int prepare(const hs_swap_in_args* a, void* workspace, size_t workspace_bytes, Plan* pl,
            bool bind_later = false) {
  if (!a) return set_error(HS_EINVAL, "args is NULL");
  if (a->B < 0 || a->K < 0) return set_error(HS_EINVAL, "B and K must be >= 0");
  if (a->B == 0 || a->K == 0) return kEmptyCall;
  const hs_paged_addressing* pa = a->paged;
  const bool pg = pa != nullptr;
  if (!a->topk_ids || !a->req_rows || (!a->seq_lens && !pg) || !a->slot_tokens || !a->lru ||
      !a->pool || !a->hot || !a->out_rows)
    return set_error(HS_EINVAL, "a required pointer is NULL");
  if (a->H < a->K) return set_error(HS_EINVAL, "hot_size H=%d must be >= top_k K=%d", a->H, a->K);
  if (a->H > 32768) return set_error(HS_ERANGE, "hot_size H=%d exceeds 32768 (int16 slots)", a->H);
  if (a->S_r < static_cast<int64_t>(a->H) + 1)
    return set_error(HS_EINVAL, "region_stride S_r=%lld must be >= H+1", (long long)a->S_r);
  if (a->R <= 0) return set_error(HS_EINVAL, "R must be > 0");
  if (a->topk_stride < a->K) return set_error(HS_EINVAL, "topk_stride must be >= K");
  if (a->ctx_stride <= 0 && !pg) return set_error(HS_EINVAL, "ctx_stride must be > 0");
  if (pg) {
    // vLLM-style addressing: the tables replace slot_rows / pool_rows /
    // ctx_stride, keys are int32 global ids and rows int32.
    if (a->slot_rows || a->pool_rows)
      return set_error(HS_EINVAL, "slot_rows / pool_rows are not used with paged addressing");
    if (!pa->hot_block_table || pa->hot_block_size <= 0)
      return set_error(HS_EINVAL, "paged addressing needs a hot block table and block size");
    if (pa->hot_table_stride < (static_cast<int64_t>(a->H) + pa->hot_block_size - 1) / pa->hot_block_size)
      return set_error(HS_EINVAL, "the hot block table does not cover H slots");
    if (pa->src_block_table &&
        (pa->src_block_size <= 0 || pa->src_num_blocks < 0 || pa->src_table_stride < pa->src_num_blocks))
      return set_error(HS_EINVAL, "bad source block table geometry");
    if (pa->resident_block_table &&
        (pa->resident_block_size <= 0 || pa->resident_num_blocks < 0 ||
         pa->resident_table_stride < pa->resident_num_blocks))
      return set_error(HS_EINVAL, "bad resident block table geometry");
    // vLLM page, host checks of hisparse_resolve_residency.
    if (pa->resident_block_table && !pa->src_block_table)
      return set_error(HS_EINVAL, "a resident block table needs a source block table");
    if (pa->resident_block_table && pa->resident_block_size != pa->hot_block_size)
      return set_error(HS_EINVAL, "resident and hot block sizes must match");
    if (pa->resident_block_table && pa->resident_null_block < 0)
      return set_error(HS_EINVAL, "the resident null block must be non-negative");
    if (pa->attention_indices && pa->attention_row_stride < a->K)
      return set_error(HS_EINVAL, "attention_row_stride must be >= K");
    if (a->pool_nrows > 0x7fffffffll || a->hot_nrows > 0x7fffffffll)
      return set_error(HS_ERANGE, "paged addressing keeps global ids and rows in int32");
  }
  if (a->pool_nrows < 0 || a->hot_nrows <= 0) return set_error(HS_EINVAL, "bad pool/hot row counts");
  if (a->row_bytes <= 0 || (a->row_bytes & 3) != 0)
    return set_error(HS_EINVAL, "row_bytes=%lld must be a positive multiple of 4", (long long)a->row_bytes);
  if (a->row_bytes > (1ll << 20)) return set_error(HS_ERANGE, "row_bytes above 1 MiB");
  if (!aligned(a->pool, 4) || !aligned(a->hot, 4))
    return set_error(HS_EINVAL, "pool and hot must be 4-byte aligned");
  if (!a->slot_rows && !pg) {
    if (a->R > 0x7fffffffll / a->S_r)   // S_r >= H + 1 >= 2
      return set_error(HS_ERANGE, "R*S_r exceeds int32 hot-row indices");
    if (a->hot_nrows < a->R * a->S_r)
      return set_error(HS_EINVAL, "hot_nrows < R*S_r with flat regions");
  }
  if ((a->pool_v == nullptr) != (a->hot_v == nullptr))
    return set_error(HS_EINVAL, "pool_v and hot_v are given together or not at all");
  if (a->pool_v && (!aligned(a->pool_v, 4) || !aligned(a->hot_v, 4)))
    return set_error(HS_EINVAL, "pool_v and hot_v must be 4-byte aligned");
  if (a->stats && !aligned(a->stats, 8)) return set_error(HS_EINVAL, "stats must be 8-byte aligned");
  const bool kv = a->pool_v != nullptr;
  const int W = (aligned(a->pool, 16) && aligned(a->hot, 16) && (a->row_bytes & 15) == 0 &&
                 (!kv || (aligned(a->pool_v, 16) && aligned(a->hot_v, 16))))
                    ? 16
                    : 4;
  const int64_t C = a->row_bytes / W;
  if (static_cast<int64_t>(a->K) * (kv ? 2 : 1) * C >= (1ll << 31))
    return set_error(HS_ERANGE, "top_k * streams * chunks per row exceeds 2^31");
  const WsLayout wl = ws_layout(a->B, a->K);
  if (!bind_later && (!workspace || workspace_bytes < wl.total || !aligned(workspace, 256)))
    return set_error(HS_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned", wl.total);

  DeviceInfo di;
  int rc = device_info(&di);
  if (rc != HS_OK) return rc;
  // LDS plan, best first. Flat layout with positions below ctx_stride as
  // keys: a direct-address table of ctx_stride int16 entries when it fits,
  // with the slot-token row staged, then without. Paged addressing: a hash
  // of the slots' keys, a quarter full, then half full (both looked up once
  // per id). Otherwise a quarter-full hash of the pending ids with the
  // slot-token row staged; a half-full one with the row staged; then the same
  // without staging (tokens gathered from HBM), each probed with every slot.
  // Shorter chains matter most: a wave's loop runs as long as its longest
  // chain.
  const uint32_t k2 = 2u * static_cast<uint32_t>(a->K) < 64u ? 64u : 2u * static_cast<uint32_t>(a->K);
  const uint32_t h2 = 2u * static_cast<uint32_t>(a->H) < 64u ? 64u : 2u * static_cast<uint32_t>(a->H);
  // Paged: the request's hot block table row (one entry per block of slots)
  // and source block table row go to LDS when they are small; larger rows
  // are read from HBM.
  uint32_t hbt_n = 0, sbt_n = 0;
  if (pg) {
    const int64_t nb = (static_cast<int64_t>(a->H) + pa->hot_block_size - 1) / pa->hot_block_size;
    if (nb <= 2048) hbt_n = static_cast<uint32_t>(nb);
    if (pa->src_block_table && pa->src_num_blocks <= 2048) sbt_n = static_cast<uint32_t>(pa->src_num_blocks);
  }
  const bool flat = !pg && !a->slot_rows && !a->pool_rows;
  const uint32_t dtab_n = (flat && a->ctx_stride <= (1 << 16)) ? static_cast<uint32_t>(a->ctx_stride) : 0u;
  constexpr int kPlans = 8;
  const uint32_t plans_T[kPlans] = {0u, 0u, pow2_at_least(2 * h2), pow2_at_least(h2), pow2_at_least(2 * k2),
                                    pow2_at_least(k2), pow2_at_least(2 * k2), pow2_at_least(k2)};
  const uint32_t plans_D[kPlans] = {dtab_n, dtab_n, 0u, 0u, 0u, 0u, 0u, 0u};
  const bool plans_stage[kPlans] = {true, false, false, false, true, true, false, false};
  int plan = -1;
  LdsLayout lay{};
  for (int i = 0; i < kPlans && plan < 0; ++i) {
    if (i < 2 && dtab_n == 0) continue;
    if ((i == 2 || i == 3) && !pg) continue;
    lay = lds_layout(a->K, a->H, plans_T[i], plans_stage[i], hbt_n, sbt_n, plans_D[i]);
    if (static_cast<int>(lay.total) <= di.max_lds) plan = i;
  }
  if (plan < 0)
    return set_error(HS_ERANGE, "K=%d, H=%d need %u bytes of LDS; the device allows %d", a->K,
                     a->H, lay.total, di.max_lds);
  const uint32_t T = plans_T[plan];
  const uint32_t dtab = plans_D[plan];
  const bool stage = plans_stage[plan];
  const bool lookup = plan < 4;   // the direct table or the paged key hash
  uint32_t log2T = 0;
  while ((1u << log2T) < T) ++log2T;
  const bool sr = a->slot_rows != nullptr, prw = a->pool_rows != nullptr;
  const bool exact = a->K % (kKU * kThreads) == 0 && a->H % (kHU * kThreads) == 0;
  const void* resolve_fn = pick_resolve<0>(sr, prw, pg, exact, lookup);
  if (lay.total > 65536) {
    rc = allow_lds(di.device, resolve_fn, lay.total);
    if (rc != HS_OK) return rc;
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
  const char* pool_v_dev = nullptr;
  if (kv) {
    // The V pool lives where the K pool does (one copy strategy for both).
    hipPointerAttribute_t va;
    if (hipPointerGetAttributes(&va, a->pool_v) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(HS_EMEMKIND, "pool_v is not a HIP allocation (device or pinned host)");
    }
    if (va.type != attr.type)
      return set_error(HS_EMEMKIND, "pool_v must be the same kind of memory as pool");
    pool_v_dev = static_cast<const char*>(
        (va.type == hipMemoryTypeHost && va.devicePointer) ? va.devicePointer : a->pool_v);
  }
  // Over the host link each request's workgroup copies its own misses (the
  // link, not the CU count, bounds the copy); an HBM pool gets the wide copy
  // kernel, which spreads every request over many CUs.
  const void* fused_fn = nullptr;
  if (attr.type == hipMemoryTypeHost) {
    fused_fn = W == 16 ? pick_resolve<16>(sr, prw, pg, exact, lookup)
                       : pick_resolve<4>(sr, prw, pg, exact, lookup);
    if (lay.total > 65536) {
      rc = allow_lds(di.device, fused_fn, lay.total);
      if (rc != HS_OK) return rc;
    }
  }

  SwapArgs& s = pl->s;
  s.topk = a->topk_ids;
  s.topk_stride = a->topk_stride;
  s.req_rows = a->req_rows;
  s.seq_lens = a->seq_lens;
  s.num_real = a->num_real;
  s.slot_tokens = a->slot_tokens;
  s.lru = a->lru;
  s.slot_rows = a->slot_rows;
  s.pool_rows = a->pool_rows;
  s.ctx_stride = a->ctx_stride;
  s.pool = pool_dev;
  s.pool_v = pool_v_dev;
  s.hot_v = static_cast<char*>(a->hot_v);
  if (pg) {
    s.hbt = pa->hot_block_table;
    s.hbt_stride = pa->hot_table_stride;
    s.hbs = pa->hot_block_size;
    s.sbt = pa->src_block_table;
    s.sbt_stride = pa->src_table_stride;
    s.sbt_nblocks = pa->src_num_blocks;
    s.sbs = pa->src_block_table ? pa->src_block_size : 1;
    s.rbt = pa->resident_block_table;
    s.rbt_stride = pa->resident_table_stride;
    s.rbt_nblocks = pa->resident_num_blocks;
    s.rbs = pa->resident_block_table ? pa->resident_block_size : 1;
    s.r_null = pa->resident_null_block;
    s.att = pa->attention_indices;
    s.att_stride = pa->attention_row_stride;
    s.att_block_stride = pa->attention_block_stride;
  } else {
    s.hbt = nullptr;
    s.sbt = nullptr;
    s.rbt = nullptr;
    s.att = nullptr;
    s.hbs = s.sbs = s.rbs = 1;
  }
  s.pool_nrows = a->pool_nrows;
  s.hot = static_cast<char*>(a->hot);
  s.hot_nrows = a->hot_nrows;
  s.row_bytes = a->row_bytes;
  s.out_rows = a->out_rows;
  s.miss_counts = a->miss_counts;
  s.miss_mask = a->miss_mask;
  s.stats = reinterpret_cast<unsigned long long*>(a->stats);
  s.B = a->B;
  s.K = a->K;
  s.H = a->H;
  s.S_r = a->S_r;
  s.R = a->R;
  s.T = T;
  s.dtab = dtab;
  s.shift = 32 - log2T;
  s.stage_tokens = stage ? 1 : 0;
  s.hbt_n = static_cast<int32_t>(hbt_n);
  s.sbt_n = static_cast<int32_t>(sbt_n);
  s.hbs_div = make_fastdiv(static_cast<uint32_t>(s.hbs));
  s.sbs_div = make_fastdiv(static_cast<uint32_t>(s.sbs));
  s.rbs_div = make_fastdiv(static_cast<uint32_t>(s.rbs));
  s.cdiv = make_fastdiv(static_cast<uint32_t>(C));

  if (bind_later) {
    s.count = nullptr;
    s.src = nullptr;
    s.dst = nullptr;
  } else {
    bind_workspace(pl, workspace);
  }

  pl->resolve_fn = resolve_fn;
  pl->fused_fn = fused_fn;
  pl->lay = lay;
  pl->host_pool = attr.type == hipMemoryTypeHost;
  pl->W = W;
  pl->C = C;
  pl->num_cus = di.num_cus;
  return HS_OK;
}

int launch_resolve(Plan& pl, const void* fn, hipStream_t stream) {
  void* params[] = {&pl.s};
  hipError_t e = hipLaunchKernel(fn, dim3(pl.s.B), dim3(kThreads), params, pl.lay.total, stream);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return set_error(HS_ELAUNCH, "resolve launch: %s", hipGetErrorString(e));
  return HS_OK;
}

int launch_copy(Plan& pl, hipStream_t stream) {
  MissList l{};
  l.count = pl.s.count;
  l.src = pl.s.src;
  l.dst = pl.s.dst;
  l.pool = pl.s.pool;
  l.hot = pl.s.hot;
  l.pool_v = pl.s.pool_v;
  l.hot_v = pl.s.hot_v;
  l.pool_layers = nullptr;
  l.hot_layers = nullptr;
  l.pool_nrows = pl.s.pool_nrows;
  l.hot_nrows = pl.s.hot_nrows;
  l.row_bytes = pl.s.row_bytes;
  l.B = pl.s.B;
  l.K = pl.s.K;
  l.layers = 1;
  l.cdiv = pl.s.cdiv;
  l.ldiv = make_fastdiv(1);
  return launch_swap_copy(l, pl.W, pl.num_cus, stream, pl.host_pool);
}

}  // namespace

extern "C" size_t hs_swap_in_workspace_bytes(int32_t B, int32_t K) {
  if (B <= 0 || K <= 0) return 0;
  return ws_layout(B, K).total;
}

extern "C" size_t hs_swap_in_workspace_layout(int32_t B, int32_t K, size_t* count_offset,
                                              size_t* src_offset, size_t* dst_offset) {
  if (B <= 0 || K <= 0) return 0;
  const WsLayout w = ws_layout(B, K);
  if (count_offset) *count_offset = w.count;
  if (src_offset) *src_offset = w.src;
  if (dst_offset) *dst_offset = w.dst;
  return w.total;
}

extern "C" int hisparse_swap_in(const hs_swap_in_args* a, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  Plan pl;
  const int rc = prepare(a, workspace, workspace_bytes, &pl);
  if (rc != HS_OK) return rc == kEmptyCall ? HS_OK : rc;
  if (pl.fused_fn) return launch_resolve(pl, pl.fused_fn, stream);
  const int r1 = launch_resolve(pl, pl.resolve_fn, stream);
  if (r1 != HS_OK) return r1;
  return launch_copy(pl, stream);
}

extern "C" int hisparse_resolve(const hs_swap_in_args* a, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  Plan pl;
  const int rc = prepare(a, workspace, workspace_bytes, &pl);
  if (rc != HS_OK) return rc == kEmptyCall ? HS_OK : rc;
  return launch_resolve(pl, pl.resolve_fn, stream);
}

extern "C" int hisparse_gather_compact(const hs_swap_in_args* a, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  Plan pl;
  const int rc = prepare(a, workspace, workspace_bytes, &pl);
  if (rc != HS_OK) return rc == kEmptyCall ? HS_OK : rc;
  return launch_copy(pl, stream);
}

extern "C" int hisparse_gather_compact_layers(const void* workspace, size_t workspace_bytes,
                                              int32_t B, int32_t K, const uint64_t* pool_layer_ptrs,
                                              int64_t pool_nrows, const uint64_t* hot_layer_ptrs,
                                              int64_t hot_nrows, int32_t num_layers,
                                              int64_t row_bytes, hipStream_t stream) {
  if (B < 0 || K < 0 || num_layers < 0) return set_error(HS_EINVAL, "B, K and num_layers must be >= 0");
  if (B == 0 || K == 0 || num_layers == 0) return HS_OK;
  if (!pool_layer_ptrs || !hot_layer_ptrs) return set_error(HS_EINVAL, "a required pointer is NULL");
  if (row_bytes <= 0 || (row_bytes & 3) != 0)
    return set_error(HS_EINVAL, "row_bytes=%lld must be a positive multiple of 4", (long long)row_bytes);
  if (row_bytes > (1ll << 20)) return set_error(HS_ERANGE, "row_bytes above 1 MiB");
  if (pool_nrows < 0 || hot_nrows < 0) return set_error(HS_EINVAL, "row counts must be >= 0");
  if (hot_nrows > 0x7fffffffll) return set_error(HS_ERANGE, "hot_nrows exceeds int32 hot-row indices");
  const int W = (row_bytes & 15) == 0 ? 16 : 4;
  const int64_t C = row_bytes / W;
  if (static_cast<int64_t>(K) * num_layers * C >= (1ll << 31))
    return set_error(HS_ERANGE, "top_k * num_layers * chunks per row exceeds 2^31");
  const WsLayout wl = ws_layout(B, K);
  if (!workspace || workspace_bytes < wl.total || !aligned(workspace, 256))
    return set_error(HS_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned", wl.total);
  DeviceInfo di;
  const int rc = device_info(&di);
  if (rc != HS_OK) return rc;
  const char* ws = static_cast<const char*>(workspace);
  MissList l{};
  l.count = reinterpret_cast<const int32_t*>(ws + wl.count);
  l.src = reinterpret_cast<const int64_t*>(ws + wl.src);
  l.dst = reinterpret_cast<const int32_t*>(ws + wl.dst);
  l.pool = nullptr;
  l.hot = nullptr;
  l.pool_v = nullptr;
  l.hot_v = nullptr;
  l.pool_layers = pool_layer_ptrs;
  l.hot_layers = hot_layer_ptrs;
  l.pool_nrows = pool_nrows;
  l.hot_nrows = hot_nrows;
  l.row_bytes = row_bytes;
  l.B = B;
  l.K = K;
  l.layers = num_layers;
  l.cdiv = make_fastdiv(static_cast<uint32_t>(C));
  l.ldiv = make_fastdiv(static_cast<uint32_t>(num_layers));
  return launch_swap_copy(l, W, di.num_cus, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free swap-in, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// it): the miss list that hisparse_swap_in keeps in the caller's workspace
// lives in `scratch`, a fixed array that each device holds for the life of
// the process. Every call on a device shares that device's array, so calls
// that overlap on one device (different streams, no ordering) race on it.
// Nothing in it has to start at zero: the resolve kernel writes each row's
// count and list entries before the copy reads them.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[HS_NOALLOC_SCRATCH_BYTES];

// Device address of this device's `scratch`, looked up once per device with
// that device current. In host code the array's name is only a stand-in for
// the symbol: passing it to a kernel would fault, so only this address is used.
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64];
  static bool have[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return set_error(HS_ELAUNCH, "hipGetDevice failed");
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!have[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return set_error(HS_ELAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                       hipGetErrorString(e));
    }
    addr[dev] = p;
    have[dev] = true;
  }
  *out = addr[dev];
  return HS_OK;
}

}  // namespace

extern "C" int hisparse_swap_in_noalloc(const hs_swap_in_args* a, hipStream_t stream) {
  if (!a) return set_error(HS_EINVAL, "args is NULL");
  if (a->B > 0 && a->K > 0) {
    const size_t need = ws_layout(a->B, a->K).total;
    if (need > HS_NOALLOC_SCRATCH_BYTES)
      return set_error(HS_ERANGE,
                       "B=%d, K=%d need a %zu-byte miss list; the allocation-free swap-in holds "
                       "%zu bytes (use hisparse_swap_in with a workspace)",
                       a->B, a->K, need, static_cast<size_t>(HS_NOALLOC_SCRATCH_BYTES));
  }
  Plan pl;
  int rc = prepare(a, nullptr, 0, &pl, /*bind_later=*/true);
  if (rc != HS_OK) return rc == kEmptyCall ? HS_OK : rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != HS_OK) return rc;
  bind_workspace(&pl, ws);
  if (pl.fused_fn) return launch_resolve(pl, pl.fused_fn, stream);
  rc = launch_resolve(pl, pl.resolve_fn, stream);
  if (rc != HS_OK) return rc;
  return launch_copy(pl, stream);
}
