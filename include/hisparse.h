/*
 * hisparse.h -- C ABI of the MI355X HiSparse swap-in library (libhisparse.so).
 *
 * HiSparse keeps each request's whole KV cache in a pool (pinned host memory
 * or HBM) and only a small per-request working set of rows in an HBM "hot
 * buffer". Every decode step, sparse attention names the top-k token ids it
 * will read; the swap-in makes those rows resident and returns the hot-buffer
 * row of each one.
 *
 * Sources, cited by page title and the function on it:
 *   SGLang hisparse.cuh        -- load_cache_to_device_buffer_kernel (the swap-in),
 *                                 transfer_cache_dsv4_mla_kernel (all-layer copy).
 *   vLLM hisparse_kernels.cu   -- hisparse_resolve_residency_kernel (the swap-in's
 *                                 resolution half), hisparse_gather_compact_kernel
 *                                 (its copy half), hisparse_gather_plan_kernel
 *                                 (plan replay on index-sharing layers), host
 *                                 argument checks.
 *   tokenspeed kvcache/triton.py -- _kv_transfer_all_layer_mla_kernel,
 *                                 _kv_transfer_all_layer_kernel (K+V),
 *                                 _store_kv_cache_kernel.
 *
 * Conventions for every call:
 *   - All pointers are caller-owned. The library allocates no device memory
 *     and keeps no state between calls beyond a per-device attribute cache.
 *   - "device" pointers are HBM allocations of the current HIP device. The
 *     swap-in pool may instead be pinned host memory (hipHostMalloc), which
 *     kernels read directly over the host link.
 *   - Work is enqueued on `stream` and is asynchronous: outputs and updated
 *     state are valid once the stream reaches that point.
 *   - Host-side validation failures return a negative hs_status, enqueue
 *     nothing, and leave a message for hisparse_last_error(). Nothing else is
 *     reported from the device: entries a kernel cannot serve are written as -1.
 *   - Everything is integer or opaque bytes; there is no floating point.
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HS_OK = 0,
  HS_EINVAL = -1,      /* a NULL pointer, bad size, stride or alignment */
  HS_ERANGE = -2,      /* sizes beyond what the kernels support (see each call) */
  HS_EMEMKIND = -3,    /* pool is neither device memory nor pinned host memory */
  HS_ELAUNCH = -4,     /* the HIP runtime rejected a launch */
  HS_EWORKSPACE = -5   /* workspace missing, too small or misaligned */
} hs_status;

/*
 * Arguments of one swap-in call.
 *
 * Per-request state, one row per request ("state row"), persists across calls:
 *   slot_tokens [R, S_r] int32 : token held by each slot of the request's hot
 *                                region, -1 = empty. Slots 0..H-1 are managed by
 *                                the LRU; slot H holds the request's newest token
 *                                and is written by the caller (store_kv_scatter),
 *                                never by the swap-in (SGLang hisparse.cuh,
 *                                region comment and newest_slot).
 *   lru         [R, H]   int16 : permutation of 0..H-1, least recently used first
 *                                (both pages' lru_slots).
 * Initial state: slot_tokens all -1, lru = 0..H-1 (hisparse_state_reset).
 *
 * Row(r, s) = slot_rows ? slot_rows[r*S_r + s] : r*S_r + s   is the hot-buffer
 * row of slot s of state row r (SGLang: device_buffer_locs).
 * pool_row(r, t) = pool_rows ? pool_rows[r*ctx_stride + t] : r*ctx_stride + t
 * is the pool row holding token t of state row r (SGLang: host_cache_locs).
 */
/*
 * vLLM-style paged addressing (vLLM hisparse_kernels.cu:
 * hisparse_resolve_residency_kernel, get_physical_hot_row, store_hot_index).
 * With hs_swap_in_args.paged set, the swap-in keys slots by global pool rows
 * instead of in-request positions:
 *   - Row(r, s) = hot_block_table[r][s / hot_block_size] * hot_block_size
 *                 + s % hot_block_size: a paged hot buffer. Every row a slot
 *                 can name must lie in [0, hot_nrows) (precondition); a row
 *                 outside is never written, and one past int32 reads as -1;
 *   - position t of state row r has global id g: with src_block_table, the
 *     physical block p = src_block_table[r][t / src_block_size] (blocks past
 *     src_num_blocks: none) gives g = p * src_block_size + t % src_block_size
 *     when p > 0, else no row; without it the id is already global (g = t).
 *     Ids at or past pool_nrows have no row. slot_tokens holds global ids,
 *     and g is the pool row a miss copies;
 *   - with resident_block_table, a position whose block maps to p >= 0,
 *     p != resident_null_block, is resident in the device cache at row
 *     p * resident_block_size + t % resident_block_size and is output as is,
 *     with no slot or copy (a row past INT32_MAX, which no int32 output can
 *     hold, counts as not resident). As the vLLM page's host checks require, a
 *     resident table needs src_block_table, resident_block_size ==
 *     hot_block_size and resident_null_block >= 0 (HS_EINVAL otherwise);
 *   - an id with no row outputs -1; there is no newest-token slot and no
 *     seq_len check (seq_lens may be NULL; ctx_stride is unused);
 *   - attention_indices (optional output, [B, attention_row_stride]) gets, for
 *     each entry, -1 or (out / hot_block_size) * attention_block_stride
 *     + out % hot_block_size.
 * Every table is a device int32 array indexed by the batch row's state row
 * (row r at r * stride). slot_rows and pool_rows must be NULL. pool_nrows and
 * hot_nrows must fit int32. Victim choice, LRU update, padding, the miss list
 * and the copies are as without paging.
 */
typedef struct hs_paged_addressing {
  const int32_t* hot_block_table;       /* [R, hot_table_stride], required     */
  int64_t hot_table_stride;             /* >= ceil(H / hot_block_size)         */
  int32_t hot_block_size;               /* > 0                                 */
  const int32_t* src_block_table;       /* [R, src_table_stride] or NULL       */
  int64_t src_table_stride;
  int32_t src_num_blocks, src_block_size;
  const int32_t* resident_block_table;  /* [R, resident_table_stride] or NULL  */
  int64_t resident_table_stride;
  int32_t resident_num_blocks, resident_block_size, resident_null_block;
  int32_t* attention_indices;           /* [B, attention_row_stride] or NULL   */
  int64_t attention_row_stride, attention_block_stride;
} hs_paged_addressing;

typedef struct hs_swap_in_args {
  int32_t B;                 /* batch rows in this call                          */
  int32_t K;                 /* top_k ids per batch row, 0 < K <= H              */
  int32_t H;                 /* hot_size: LRU slots per request, H <= 32768      */
  int64_t S_r;               /* region_stride of slot_tokens / slot_rows, >= H+1 */
  int64_t R;                 /* state rows in slot_tokens / lru                  */

  const int32_t* topk_ids;   /* device [B, topk_stride]: in-request token ids    */
  int64_t topk_stride;       /* elements between batch rows, >= K                */
  const int64_t* req_rows;   /* device [B]: state row of each batch row          */
  const int64_t* seq_lens;   /* device [B]: tokens so far; newest id = seq_len-1 */
  const int32_t* num_real;   /* device [1] or NULL: rows b >= *num_real are      */
                             /* padding (all outputs -1, count 0)                */

  int32_t* slot_tokens;      /* device [R, S_r], in/out                          */
  int16_t* lru;              /* device [R, H], in/out                            */
  const int32_t* slot_rows;  /* device [R, S_r] or NULL (flat regions)           */
  const int64_t* pool_rows;  /* device [R, ctx_stride] or NULL (flat pool)       */
  int64_t ctx_stride;        /* pool rows per request; ids >= ctx_stride invalid */

  const void* pool;          /* [pool_nrows, row_bytes] pinned host or device    */
  int64_t pool_nrows;
  void* hot;                 /* device [hot_nrows, row_bytes]                    */
  int64_t hot_nrows;
  int64_t row_bytes;         /* opaque row size, > 0 and a multiple of 4         */

  int32_t* out_rows;         /* device [B, K] out: hot row per entry, or -1      */
  int32_t* miss_counts;      /* device [B] out, or NULL: rows copied per row     */
  int32_t* miss_mask;        /* device [B, K] out, or NULL: 1 where the entry    */
                             /* missed and was given a slot (step 3), else 0     */
                             /* (vLLM hisparse_kernels.cu, miss_mask)            */

  /* Non-MLA caches (SGLang hisparse.cuh, !IsMLA): a V pool and a V hot buffer
   * with the same rows, row_bytes and kind of memory as pool / hot. Each miss
   * then copies its V row with the same pool row and hot row as its K row.
   * Both NULL for MLA (one latent row per token). */
  const void* pool_v;        /* [pool_nrows, row_bytes], or NULL                 */
  void* hot_v;               /* device [hot_nrows, row_bytes], or NULL           */

  /* vLLM-style paged addressing (host pointer to a struct whose tables are
   * device arrays), or NULL for the addressing described above. */
  const hs_paged_addressing* paged;

  /* Running counters (vLLM hisparse_kernels.cu, stats), or NULL: device
   * uint64 [2], in/out. Every real batch row adds its hits (step 2) to
   * stats[0] and its misses (step 3) to stats[1] with device atomics, so calls
   * accumulate; the caller zeroes them when it wants a fresh count. Must be
   * 8-byte aligned (HS_EINVAL otherwise). */
  uint64_t* stats;
} hs_swap_in_args;

/* Bytes of device workspace hisparse_swap_in needs for B rows of K ids
 * (the compacted miss list handed from resolution to the copy). */
size_t hs_swap_in_workspace_bytes(int32_t B, int32_t K);

/*
 * hisparse_swap_in -- one decode step of the HiSparse swap-in.
 * SGLang hisparse.cuh, load_cache_to_device_buffer_kernel; vLLM
 * hisparse_kernels.cu, hisparse_resolve_residency_kernel +
 * hisparse_gather_compact_kernel.
 *
 * For each real batch row b with state row r and seq_len L:
 *   1. id t is invalid if t < 0, t >= L, t >= ctx_stride, or pool_row(r,t) is
 *      outside [0, pool_nrows): out = -1. t == L-1 (the newest token) gets
 *      out = Row(r, H). Every other id is pending.
 *   2. Walking lru[r] oldest first, a slot whose token is pending is a hit: that
 *      entry gets out = Row(r, slot). All other slots are evictable, in LRU order.
 *   3. Pending ids that were not hit, in ascending top-k index, are misses; miss
 *      m takes the m-th oldest evictable slot v: out = Row(r, v),
 *      slot_tokens[r][v] = t, and row_bytes bytes are copied from pool row
 *      pool_row(r, t) to hot row Row(r, v).
 *   4. lru[r] becomes: remaining evictables, then the filled slots in miss order,
 *      then the hits, each group in its previous order.
 *   5. miss_counts[b] = number of misses; stats[0] += hits, stats[1] += misses.
 *
 * Preconditions the caller guarantees (not checked on the device): valid ids
 * are unique within a batch row; real rows name distinct state rows; lru rows
 * are permutations; resident tokens in slots 0..H-1 are distinct; pool, hot
 * buffer and state arrays do not overlap. Breaking them cannot make a kernel
 * access memory outside the buffers described here, but results are then
 * unspecified.
 *
 * workspace: device memory of at least hs_swap_in_workspace_bytes(B, K) bytes,
 * 256-byte aligned, owned by the caller; its contents need not be initialised
 * (it carries each request's miss list from the resolve kernel to the copy
 * kernel). Calls that share a workspace must be ordered on one stream.
 *
 * Returns HS_OK; HS_EINVAL / HS_ERANGE / HS_EMEMKIND / HS_EWORKSPACE on bad
 * arguments (nothing enqueued); HS_ELAUNCH if a launch failed. B == 0 or
 * K == 0 returns HS_OK with nothing enqueued. HS_ERANGE also covers K and H
 * whose per-request scratch does not fit one workgroup's LDS (the membership
 * table, the staged ids and outputs, and the old and new LRU rows all live
 * there). With the flat layout (no slot_rows, pool_rows or paged) and
 * ctx_stride <= 65536 the table is a direct-address table of ctx_stride int16
 * entries (the slot holding each position) when that fits; with paged
 * addressing it is a hash of the slots' keys with 2H to 4H entries when that
 * fits; otherwise it is a hash table of the top-k ids with 2K to 4K entries,
 * and with 160 KB per workgroup that allows K <= 4096 for H <= 8192,
 * K <= 3016 at H = 16384 and K <= 584 at H = 32768.
 */
int hisparse_swap_in(const hs_swap_in_args* args, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * hisparse_swap_in_noalloc -- hisparse_swap_in without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Computes exactly what hisparse_swap_in computes (same arguments, same
 * kernels, same results). The miss list that hisparse_swap_in keeps in the
 * caller's workspace lives instead in a fixed device array of
 * HS_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends; the call itself allocates nothing (no hipMalloc,
 * hipFree or allocating library routine). The array needs no initialisation.
 * Every call on a device shares that device's array: calls that overlap on
 * one device (different streams with no ordering between them) race and give
 * unspecified results; order them on one stream. The list is not published
 * for hisparse_gather_compact_layers (use hisparse_resolve with a workspace).
 *
 * Returns HS_ERANGE, with nothing enqueued, when the list of B rows of K ids
 * (hs_swap_in_workspace_bytes(B, K)) exceeds HS_NOALLOC_SCRATCH_BYTES: 4 MiB
 * holds B * K up to about 349,000 (B = 128 at K = 2048). Every other status as
 * for hisparse_swap_in (never HS_EWORKSPACE).
 */
#define HS_NOALLOC_SCRATCH_BYTES (4u << 20)
int hisparse_swap_in_noalloc(const hs_swap_in_args* args, hipStream_t stream);

/*
 * hisparse_resolve / hisparse_gather_compact -- the two halves of
 * hisparse_swap_in, for callers that want to run the row copy later, on
 * another stream, or once per layer group.
 * vLLM hisparse_kernels.cu, hisparse_resolve_residency_kernel (resolution
 * half, compact swap lists) and hisparse_gather_compact_kernel (copy half).
 *
 * hisparse_resolve performs steps 1-5 of hisparse_swap_in except the byte
 * copy: outputs, state and miss counts are final, and the workspace holds
 * each row's miss list (see hs_swap_in_workspace_layout).
 * hisparse_gather_compact copies the rows that list names, from pool to hot.
 * Both take the same argument struct and check it the same way. The gather
 * kernel uses only B, K, pool, pool_nrows, hot, hot_nrows, row_bytes and
 * pool_v / hot_v from it (it leaves outputs, state and stats alone), plus the
 * workspace, which must hold the list of a resolve call with the same B and K
 * enqueued before it (on the same stream, or ordered by an event). Resolve
 * then gather is exactly hisparse_swap_in. Errors as for hisparse_swap_in.
 * Per list entry (as vLLM's hisparse_gather_compact_kernel): the count is
 * clamped to [0, K]; an entry whose pool row is negative or whose hot row is
 * outside [0, hot_nrows) is skipped; a pool row >= pool_nrows writes zeros to
 * the hot row. A list written by a resolve on the same pool never hits the
 * last two cases.
 */
int hisparse_resolve(const hs_swap_in_args* args, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);
int hisparse_gather_compact(const hs_swap_in_args* args, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * hisparse_gather_compact_layers -- replay one resolved plan on several layers.
 * vLLM hisparse_kernels.cu, hisparse_gather_plan_kernel: layers that share the
 * index-producing layer's top-k ids get the same slots, so they reuse its
 * plan and copy only their own bytes; no LRU work is redone.
 *
 * workspace / workspace_bytes / B / K: a workspace holding the miss list of a
 * hisparse_resolve call with the same B and K, enqueued before this call.
 * pool_layer_ptrs, hot_layer_ptrs: device uint64 [num_layers] arrays of layer
 * base addresses, as the device sees them (a pinned host pool's address, or
 * HBM); every layer holds pool_nrows (hot_nrows) rows of row_bytes, with the
 * row numbering of the layer the plan was resolved on. Bases must be 4-byte
 * aligned; 16-byte aligned bases with row_bytes % 16 == 0 take the 16-byte
 * path. For every layer l and list entry (pool row s, hot row d), with the
 * entry rules of hisparse_gather_compact:
 *   hot_layer_ptrs[l] + d*row_bytes  <-  pool_layer_ptrs[l] + s*row_bytes.
 * All layers move in one launch. Hot rows of different layers must not
 * overlap. B, K or num_layers == 0 returns HS_OK with nothing enqueued; other
 * errors as for hisparse_swap_in, and HS_ERANGE when K * num_layers *
 * (row_bytes / 16, or / 4) reaches 2^31.
 */
int hisparse_gather_compact_layers(const void* workspace, size_t workspace_bytes, int32_t B,
                                   int32_t K, const uint64_t* pool_layer_ptrs, int64_t pool_nrows,
                                   const uint64_t* hot_layer_ptrs, int64_t hot_nrows,
                                   int32_t num_layers, int64_t row_bytes, hipStream_t stream);

/*
 * Workspace layout of the miss list, for callers that read it (vLLM
 * hisparse_kernels.cu: swap_counts, swap_host_physical_rows,
 * swap_device_physical_rows). Byte offsets from the workspace start:
 *   count: int32 [B]      misses of batch row b
 *   src:   int64 [B, K]   pool row of miss m of row b (m < count[b]), miss order
 *   dst:   int32 [B, K]   hot row of that miss, or -1 when it was not copied
 * Returns the total size (== hs_swap_in_workspace_bytes), 0 for B or K <= 0.
 * Any offset pointer may be NULL.
 */
size_t hs_swap_in_workspace_layout(int32_t B, int32_t K, size_t* count_offset, size_t* src_offset,
                                   size_t* dst_offset);

/*
 * transfer_rows_all_layer -- fused multi-layer indexed row copy.
 * tokenspeed kvcache/triton.py, _kv_transfer_all_layer_mla_kernel; SGLang
 * hisparse.cuh, transfer_cache_dsv4_mla_kernel (generic row layout).
 *
 * For every pair i < n and layer l < num_layers:
 *   dst_layer_ptrs[l] + dst_idx[i]*row_bytes  <-  src_layer_ptrs[l] + src_idx[i]*row_bytes
 * src_layer_ptrs / dst_layer_ptrs: device uint64 [num_layers] arrays of layer
 * base addresses; each layer holds src_nrows (dst_nrows) rows of row_bytes.
 * Every layer base must be 4-byte aligned (16-byte aligned bases take the
 * 16-byte copy path when row_bytes is a multiple of 16).
 * Either side may be pinned host memory (offload and load directions).
 * src_idx / dst_idx: device int64 [n]; indices stay 64-bit (no truncation).
 * Pairs with an index outside [0, src_nrows) / [0, dst_nrows) are skipped.
 * dst indices must be unique and source and destination rows must not overlap.
 * row_bytes > 0, multiple of 4; n == 0 or num_layers == 0 returns HS_OK.
 * flags: 0, or HS_TRANSFER_HOST_LINK when one side is pinned host memory (the
 * offload and load directions; hs_transfer_flags_for works it out from one
 * pair of layer bases). The library cannot see where the layer bases
 * point; with the flag the launch uses one workgroup per two CUs, each lane
 * keeping 8 chunks in flight, which moves more over the host link than the
 * HBM-sized launch and leaves the other CUs to concurrent work. The bytes
 * written are the same either way. Any other bit set: HS_EINVAL.
 */
#define HS_TRANSFER_HOST_LINK 1u
int transfer_rows_all_layer(const uint64_t* src_layer_ptrs, const uint64_t* dst_layer_ptrs,
                            const int64_t* src_idx, const int64_t* dst_idx, int64_t n,
                            int32_t num_layers, int64_t row_bytes, int64_t src_nrows,
                            int64_t dst_nrows, uint32_t flags, hipStream_t stream);

/*
 * hs_transfer_flags_for -- the flags argument of transfer_rows_all_layer and
 * transfer_kv_all_layer for layers that live where src_layer and dst_layer do.
 * Not on the pages: the transfers take their layer bases from device arrays
 * the library cannot read on the host, so the caller names the memory kind;
 * this reads it from one source and one destination layer base (host
 * pointers as the caller holds them) and is meant to run once, where the
 * caches are set up. *flags becomes HS_TRANSFER_HOST_LINK when either side
 * is pinned host memory, else 0. Enqueues nothing.
 * Errors: NULL argument -> HS_EINVAL; a pointer HIP does not know, or memory
 * other than device or pinned host -> HS_EMEMKIND (*flags unchanged).
 */
int hs_transfer_flags_for(const void* src_layer, const void* dst_layer, uint32_t* flags);

/*
 * transfer_kv_all_layer -- the non-MLA form of transfer_rows_all_layer.
 * tokenspeed kvcache/triton.py, _kv_transfer_all_layer_kernel.
 *
 * For every pair i < n and layer l < num_layers, the K row and the V row:
 *   k_dst_layer_ptrs[l] + dst_idx[i]*row_bytes  <-  k_src_layer_ptrs[l] + src_idx[i]*row_bytes
 *   v_dst_layer_ptrs[l] + dst_idx[i]*row_bytes  <-  v_src_layer_ptrs[l] + src_idx[i]*row_bytes
 * Four device uint64 [num_layers] arrays of layer base addresses; K and V
 * layers have the same row counts (src_nrows, dst_nrows) and row_bytes.
 * Everything else (alignment, directions, skipped pairs, index width,
 * uniqueness, flags, errors) is as for transfer_rows_all_layer; all
 * 2 * num_layers streams move in one launch.
 */
int transfer_kv_all_layer(const uint64_t* k_src_layer_ptrs, const uint64_t* v_src_layer_ptrs,
                          const uint64_t* k_dst_layer_ptrs, const uint64_t* v_dst_layer_ptrs,
                          const int64_t* src_idx, const int64_t* dst_idx, int64_t n,
                          int32_t num_layers, int64_t row_bytes, int64_t src_nrows,
                          int64_t dst_nrows, uint32_t flags, hipStream_t stream);

/*
 * store_kv_scatter -- write rows into a cache at given row indices.
 * tokenspeed kvcache/triton.py, _store_kv_cache_kernel (one cache, the MLA case).
 *
 * For j < n with 0 <= loc[j] < dst_nrows:
 *   dst + loc[j]*dst_row_stride_bytes  <-  src + j*src_row_stride_bytes  (row_bytes bytes)
 * src, dst: device; strides in bytes, >= row_bytes, multiples of 4; loc: device
 * int64 [n], unique among entries that are written. Entries with loc < 0 (the
 * pages' padding value) or loc >= dst_nrows are skipped. n == 0 returns HS_OK.
 */
int store_kv_scatter(const void* src, int64_t src_row_stride_bytes, void* dst,
                     int64_t dst_row_stride_bytes, int64_t dst_nrows, const int64_t* loc,
                     int64_t n, int64_t row_bytes, hipStream_t stream);

/*
 * store_kv_cache -- the K+V form of store_kv_scatter, both halves in one
 * launch (tokenspeed kvcache/triton.py, _store_kv_cache_kernel).
 *
 * For j < n with 0 <= loc[j] < dst_nrows:
 *   k_dst + loc[j]*k_dst_row_stride_bytes  <-  k_src + j*k_src_row_stride_bytes
 *   v_dst + loc[j]*v_dst_row_stride_bytes  <-  v_src + j*v_src_row_stride_bytes
 * (row_bytes bytes each). Each of the four arrays has its own row stride
 * (bytes, >= row_bytes, multiple of 4); K and V caches have dst_nrows rows.
 * Skipped entries, loc uniqueness and errors as for store_kv_scatter.
 */
int store_kv_cache(const void* k_src, int64_t k_src_row_stride_bytes, const void* v_src,
                   int64_t v_src_row_stride_bytes, void* k_dst, int64_t k_dst_row_stride_bytes,
                   void* v_dst, int64_t v_dst_row_stride_bytes, int64_t dst_nrows,
                   const int64_t* loc, int64_t n, int64_t row_bytes, hipStream_t stream);

/*
 * hisparse_invalidate_written -- drop hot copies of rewritten pool rows.
 * vLLM hisparse_kernels.cu, hisparse_invalidate_written_slots_kernel.
 *
 * For every j < n with 0 <= rows[j] < R and written[j] >= 0, every entry of
 * slot_keys[rows[j]][0..S_r) equal to written[j] becomes -1 (empty), so the
 * next swap-in that wants that global row copies it again instead of serving
 * the stale hot row. For slot tables keyed by global ids (paged addressing).
 * The LRU order is left as is: an emptied slot is simply evictable.
 * slot_keys: device int32 [R, S_r]; rows, written: device int64 [n].
 * n == 0 returns HS_OK.
 */
int hisparse_invalidate_written(int32_t* slot_keys, int64_t R, int64_t S_r, const int64_t* rows,
                                const int64_t* written, int64_t n, hipStream_t stream);

/*
 * hisparse_state_reset -- put state rows into the initial state: every entry
 * of slot_tokens[r][0..S_r) = -1 and lru[r] = 0..H-1, for r in rows[0..n_rows).
 * rows: device int64 [n_rows]; rows outside [0, R) are skipped.
 */
int hisparse_state_reset(int32_t* slot_tokens, int16_t* lru, const int64_t* rows, int64_t n_rows,
                         int32_t H, int64_t S_r, int64_t R, hipStream_t stream);

/* Text describing the last non-OK status returned on the calling thread. */
const char* hisparse_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H */
