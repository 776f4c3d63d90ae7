/*
 * HiSparse CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded C reference of what the HiSparse decode-time
 * swap-in, the fused all-layer indexed row transfer and the KV-row scatter
 * compute. Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it. The GPU library neither includes nor links it, and
 * this file shares no code with the GPU library.
 *
 * Sources (cited by page title and function):
 *   [SGL]  SGLang hisparse.cuh, load_cache_to_device_buffer_kernel and
 *          transfer_cache_dsv4_mla_kernel.
 *   [VLLM] vLLM hisparse_kernels.cu, hisparse_resolve_residency_kernel,
 *          hisparse_gather_compact_kernel, hisparse_gather_plan_kernel.
 *   [TS]   tokenspeed kvcache/triton.py, _store_kv_cache_kernel,
 *          _kv_transfer_all_layer_mla_kernel and _kv_transfer_all_layer_kernel.
 *
 * All arrays are host memory and row-major. Nothing here is floating point.
 */
#ifndef HISPARSE_ORACLE_H
#define HISPARSE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ORACLE_OK = 0,
  ORACLE_EARG = -1,      /* bad sizes or NULL pointers */
  ORACLE_EDUP_ID = -2,   /* a valid top-k id repeats within one batch row */
  ORACLE_ELRU = -3,      /* lru row is not a permutation of [0, H) */
  ORACLE_EROWS = -4,     /* two real batch rows share one state row */
  ORACLE_EHOT = -5,      /* a hot-row index falls outside the hot buffer */
  ORACLE_ESTATE = -6,    /* one valid token resident in two LRU slots */
  ORACLE_EINDEX = -7     /* transfer/scatter index outside its buffer */
};

/* vLLM-style addressing ([VLLM] hisparse_resolve_residency_kernel and
 * get_physical_hot_row). With it, slots are keyed by global pool rows instead
 * of in-request positions, there is no newest-token slot and no seq_len
 * check, and slot_rows / pool_rows / ctx_stride are not used. Every table is
 * indexed by the batch row's state row r. */
typedef struct {
  /* Row(r, s) = hot_block_table[r][s / hot_block_size] * hot_block_size
   *             + s % hot_block_size. */
  const int32_t *hot_block_table;
  int64_t hot_table_stride;
  int32_t hot_block_size;
  /* Global id of position t: with a source table, block t / src_block_size
   * (below src_num_blocks) maps to physical block p; p > 0 gives
   * g = p * src_block_size + t % src_block_size, anything else no row.
   * Without one, the id is the global id. Ids at or past pool_nrows have no
   * row either. */
  const int32_t *src_block_table;
  int64_t src_table_stride;
  int32_t src_num_blocks, src_block_size;
  /* Optional: positions still resident in the device cache. Block
   * t / resident_block_size (below resident_num_blocks) maps to p; p >= 0 and
   * p != resident_null_block makes the entry resident at row
   * p * resident_block_size + t % resident_block_size, served as is.
   * As the vLLM page's host checks require: the table needs a source block
   * table, resident_block_size == hot_block_size and resident_null_block >= 0;
   * otherwise the call returns ORACLE_EARG. */
  const int32_t *resident_block_table;
  int64_t resident_table_stride;
  int32_t resident_num_blocks, resident_block_size, resident_null_block;
  /* Optional output: attention_indices[b][i] = -1 for out < 0, else
   * (out / hot_block_size) * attention_block_stride + out % hot_block_size. */
  int32_t *attention_indices;
  int64_t attention_row_stride, attention_block_stride;
} oracle_paged;

typedef struct {
  int32_t B, K, H;          /* batch rows, top_k, hot_size */
  int64_t S_r, R;           /* region_stride (>= H+1), state rows */
  const int32_t *topk;      /* [B, topk_stride] in-request token positions */
  int64_t topk_stride;
  const int64_t *req_rows;  /* [B] state row of each batch row */
  const int64_t *seq_lens;  /* [B]; newest token = seq_len - 1 */
  int32_t num_real;         /* rows b >= num_real are padding; < 0 = none */
  int32_t *slot_tokens;     /* [R, S_r] in/out, -1 = empty */
  int16_t *lru;             /* [R, H] in/out, LRU first */
  const int32_t *slot_rows; /* [R, S_r] or NULL: hot row = r*S_r + s */
  const int64_t *pool_rows; /* [R, ctx_stride] or NULL: pool row = r*ctx_stride + t */
  int64_t ctx_stride;
  const uint8_t *pool;      /* [pool_nrows, row_bytes] */
  int64_t pool_nrows;
  uint8_t *hot;             /* [hot_nrows, row_bytes] */
  int64_t hot_nrows;
  int64_t row_bytes;
  int32_t *out_rows;        /* [B, K] */
  int32_t *miss_counts;     /* [B] or NULL */
  /* Optional plan outputs (all NULL, or each as documented): */
  int32_t *miss_mask;       /* [B, K] or NULL: 1 where the entry missed and got a slot */
  int32_t *list_count;      /* [B] or NULL: misses of row b (the compact plan's length) */
  int64_t *list_src;        /* [B, K]: pool row of miss m of row b, m < list_count[b] */
  int32_t *list_dst;        /* [B, K]: hot row of miss m of row b */
  /* Non-MLA caches ([SGL] !IsMLA): a V pool and V hot buffer with the K
   * pool's and K hot buffer's geometry; every miss copies its V row too. */
  const uint8_t *pool_v;    /* [pool_nrows, row_bytes] or NULL */
  uint8_t *hot_v;           /* [hot_nrows, row_bytes], NULL when pool_v is */
  const oracle_paged *paged; /* NULL: SGLang-style addressing (above) */
  /* Optional running counters ([VLLM] stats): every real row adds its hits
   * (step 2) to stats[0] and its misses (step 3) to stats[1]. */
  uint64_t *stats;          /* [2] in/out, or NULL */
} oracle_swap_in_args;

/* One decode-step swap-in call. Returns ORACLE_OK or a negative code when a
 * precondition of the pages is broken; outputs are then unspecified. */
int oracle_swap_in(const oracle_swap_in_args *a);

/* Replay of a compact miss plan on num_layers (pool, hot) pairs that share
 * the plan's indices ([VLLM] hisparse_gather_compact_kernel, and the
 * index-sharing layers of hisparse_gather_plan_kernel): for every layer l,
 * row b and miss m < count[b] (count clamped to [0, K]), with s = src[b][m]
 * and d = dst[b][m]: skip when s < 0 or d is outside [0, hot_nrows); copy
 * pool row s of layer l to hot row d of layer l when s < pool_nrows;
 * otherwise (no such source row) write zeros to that hot row. Returns the
 * number of rows zeroed (summed over layers), or ORACLE_EARG. */
int64_t oracle_gather_compact_layers(const int32_t *count, const int64_t *src, const int32_t *dst,
                                     int32_t B, int32_t K, const uint8_t *const *pool_layers,
                                     int64_t pool_nrows, uint8_t *const *hot_layers,
                                     int64_t hot_nrows, int32_t num_layers, int64_t row_bytes);

/* dst_layers[l][dst_idx[i]] <- src_layers[l][src_idx[i]] for every pair i and
 * layer l (row_bytes bytes each). Pairs with an index outside [0, nrows) are
 * skipped and counted; returns the number skipped, or ORACLE_EARG. */
int64_t oracle_transfer_rows_all_layer(const uint8_t *const *src_layers, uint8_t *const *dst_layers,
                                       int64_t src_nrows, int64_t dst_nrows,
                                       const int64_t *src_idx, const int64_t *dst_idx, int64_t n,
                                       int32_t num_layers, int64_t row_bytes);

/* The K+V all-layer transfer ([TS] _kv_transfer_all_layer_kernel): for every
 * index pair i and layer l, the K row src_idx[i] of k_src_layers[l] goes to
 * row dst_idx[i] of k_dst_layers[l], then the V row likewise. Pairs with an
 * index outside [0, nrows) are skipped and counted; returns that count, or
 * ORACLE_EARG. */
int64_t oracle_transfer_kv_all_layer(const uint8_t *const *k_src_layers,
                                     const uint8_t *const *v_src_layers,
                                     uint8_t *const *k_dst_layers, uint8_t *const *v_dst_layers,
                                     int64_t src_nrows, int64_t dst_nrows, const int64_t *src_idx,
                                     const int64_t *dst_idx, int64_t n, int32_t num_layers,
                                     int64_t row_bytes);

/* The K+V scatter ([TS] _store_kv_cache_kernel, both halves): for j < n with
 * 0 <= loc[j] < dst_nrows, K row j goes to K row loc[j] and V row j to V row
 * loc[j], each side with its own row stride in bytes. Returns the number of
 * entries skipped, or ORACLE_EARG. */
int64_t oracle_store_kv_cache(const uint8_t *k_src, int64_t k_src_stride, const uint8_t *v_src,
                              int64_t v_src_stride, uint8_t *k_dst, int64_t k_dst_stride,
                              uint8_t *v_dst, int64_t v_dst_stride, int64_t dst_nrows,
                              const int64_t *loc, int64_t n, int64_t row_bytes);

/* dst row loc[j] <- src row j for j < n; entries with loc outside
 * [0, dst_nrows) are skipped. Returns the number skipped, or ORACLE_EARG. */
int64_t oracle_store_kv_scatter(const uint8_t *src, int64_t src_row_stride_bytes,
                                uint8_t *dst, int64_t dst_row_stride_bytes, int64_t dst_nrows,
                                const int64_t *loc, int64_t n, int64_t row_bytes);

/* Write invalidation ([VLLM] hisparse_invalidate_written_slots_kernel): for
 * each written token j with state row rows[j] in [0, R) and global row
 * written[j] >= 0, every slot of that state row (all S_r of them) holding
 * written[j] becomes empty (-1). LRU order is untouched. Returns the number
 * of slots cleared, or ORACLE_EARG. */
int64_t oracle_invalidate_written(int32_t *slot_keys, int64_t R, int64_t S_r, const int64_t *rows,
                                  const int64_t *written, int64_t n);

/* Initial state of the listed state rows: every token -1, LRU = 0..H-1. Each
 * row has its H LRU slots and the newest slot (S_r >= H + 1); rows outside
 * [0, R) are an error. */
int oracle_state_reset(int32_t *slot_tokens, int16_t *lru, const int64_t *rows, int64_t n_rows,
                       int32_t H, int64_t S_r, int64_t R);

#ifdef __cplusplus
}
#endif

#endif
