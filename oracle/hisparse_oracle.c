/*
 * HiSparse CPU oracle -- TEST INFRASTRUCTURE ONLY (see hisparse_oracle.h).
 *
 * Written for a reader checking it against the pages by eye: one batch row at
 * a time, the steps in the order the pages' swap-in kernels take them, plain
 * arrays and libc qsort/bsearch for membership. The GPU library shares no code
 * with this file.
 *
 * Readings where the pages are silent or disagree (each also applies to the
 * GPU path):
 *  - Membership instead of a hash. Both pages insert the top-k ids into an
 *    open-addressing table and probe it with each resident slot's token; the
 *    result they use is only "is this token among the pending ids, and at
 *    which top-k index". A sorted array answers the same question.
 *  - Invalid ids. An id outside [0, seq_len), at or past ctx_stride, or whose
 *    pool row falls outside the pool, is output as -1, is not copied and is
 *    not counted (the vLLM page maps out-of-range ids to -1 the same way).
 *  - Padding. A batch row at or past num_real, or whose state row lies
 *    outside [0, R), gets -1 in every output and a miss count of 0 (the vLLM
 *    page's choice for padded rows; the SGLang page writes nothing).
 *  - The newest token is bound to slot H of its region (SGLang page,
 *    "newest_slot"), is never hashed, copied or counted, and slot H never
 *    enters the LRU.
 */
#include "hisparse_oracle.h"

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t token;  /* in-request position */
  int32_t index;  /* top-k column */
  int32_t hit;    /* set when an LRU slot holds this token */
} pending_t;

static int cmp_by_token(const void *x, const void *y) {
  const pending_t *a = (const pending_t *)x, *b = (const pending_t *)y;
  return (a->token > b->token) - (a->token < b->token);
}

static int cmp_by_index(const void *x, const void *y) {
  const pending_t *a = (const pending_t *)x, *b = (const pending_t *)y;
  return (a->index > b->index) - (a->index < b->index);
}

/* Row(r, s): the hot-buffer row of slot s of state row r. The SGLang page
 * reads it from device_buffer_locs; with no table it is the flat region; the
 * vLLM page pages it through a hot block table (get_physical_hot_row). */
static int64_t hot_row(const oracle_swap_in_args *a, int64_t r, int64_t s) {
  if (a->paged) {
    const oracle_paged *p = a->paged;
    const int64_t blk = p->hot_block_table[r * p->hot_table_stride + s / p->hot_block_size];
    return blk * p->hot_block_size + s % p->hot_block_size;
  }
  return a->slot_rows ? (int64_t)a->slot_rows[r * a->S_r + s] : r * a->S_r + s;
}

/* vLLM page, first phase of hisparse_resolve_residency_kernel: position t of
 * state row r becomes a global id *g (or -1: no row) and, with a resident
 * table, a row *res of the device cache that already holds it (or -1). */
static void paged_translate(const oracle_swap_in_args *a, int64_t r, int64_t t, int64_t *g,
                            int64_t *res) {
  const oracle_paged *p = a->paged;
  *g = t;
  *res = -1;
  if (p->src_block_table) {
    const int64_t blk = t >= 0 ? t / p->src_block_size : -1;
    *g = -1;
    if (blk >= 0 && blk < p->src_num_blocks) {
      const int64_t pb = p->src_block_table[r * p->src_table_stride + blk];
      if (pb > 0) *g = pb * p->src_block_size + t % p->src_block_size;
    }
  }
  if (*g >= a->pool_nrows) *g = -1;
  if (p->resident_block_table) {
    const int64_t blk = t >= 0 ? t / p->resident_block_size : -1;
    if (blk >= 0 && blk < p->resident_num_blocks) {
      const int64_t pb = p->resident_block_table[r * p->resident_table_stride + blk];
      if (pb != p->resident_null_block && pb >= 0)
        *res = pb * p->resident_block_size + t % p->resident_block_size;
    }
    /* Rows are output as int32 (both pages store int32 rows): a resident row
     * past INT32_MAX cannot be output, so its position is not resident. */
    if (*res > INT32_MAX) *res = -1;
  }
}

/* vLLM page, store_hot_index: the attention kernel's index of a row. */
static void store_attention(const oracle_swap_in_args *a, int32_t b, const int32_t *out) {
  const oracle_paged *p = a->paged;
  if (!p || !p->attention_indices) return;
  int32_t *att = p->attention_indices + (int64_t)b * p->attention_row_stride;
  for (int32_t i = 0; i < a->K; ++i) {
    const int64_t o = out[i];
    att[i] = o < 0 ? -1
                   : (int32_t)((o / p->hot_block_size) * p->attention_block_stride +
                               o % p->hot_block_size);
  }
}

/* The pool row holding token t of state row r (SGLang page: host_cache_locs). */
static int64_t pool_row(const oracle_swap_in_args *a, int64_t r, int64_t t) {
  return a->pool_rows ? a->pool_rows[r * a->ctx_stride + t] : r * a->ctx_stride + t;
}

static int check_args(const oracle_swap_in_args *a) {
  if (!a || a->B < 0 || a->K < 0 || a->H < 0 || a->R < 0) return ORACLE_EARG;
  if (a->B == 0 || a->K == 0) return ORACLE_OK;
  if (!a->topk || !a->req_rows || (!a->seq_lens && !a->paged) || !a->slot_tokens || !a->lru ||
      !a->pool || !a->hot || !a->out_rows)
    return ORACLE_EARG;
  if (a->H < a->K || a->S_r < (int64_t)a->H + 1 || a->topk_stride < a->K || a->row_bytes <= 0 ||
      (a->ctx_stride <= 0 && !a->paged))
    return ORACLE_EARG;
  if (a->list_count && (!a->list_src || !a->list_dst)) return ORACLE_EARG;
  if ((a->pool_v == NULL) != (a->hot_v == NULL)) return ORACLE_EARG;
  if (a->paged) {
    const oracle_paged *p = a->paged;
    if (!p->hot_block_table || p->hot_block_size <= 0 || p->hot_table_stride * p->hot_block_size < a->H)
      return ORACLE_EARG;
    if (p->src_block_table && (p->src_block_size <= 0 || p->src_num_blocks < 0)) return ORACLE_EARG;
    if (p->resident_block_table && (p->resident_block_size <= 0 || p->resident_num_blocks < 0))
      return ORACLE_EARG;
    /* vLLM page, host checks of hisparse_resolve_residency: a resident lookup
     * needs the source block table, the resident and hot block sizes must
     * match, and the resident null block must be non-negative. */
    if (p->resident_block_table &&
        (!p->src_block_table || p->resident_block_size != p->hot_block_size ||
         p->resident_null_block < 0))
      return ORACLE_EARG;
    if (a->pool_nrows > INT32_MAX) return ORACLE_EARG;   /* keys are int32 global ids */
  }
  return ORACLE_OK;
}

/* Preconditions the pages state or imply, checked up front so a broken input
 * never produces a plausible-looking answer. */
static int check_state_rows(const oracle_swap_in_args *a, int32_t nreal) {
  /* One block owns one request's region (SGLang page, one block per request):
   * real rows must name distinct state rows. */
  for (int32_t b = 0; b < nreal; ++b) {
    int64_t r = a->req_rows[b];
    if (r < 0 || r >= a->R) continue;
    for (int32_t c = b + 1; c < nreal; ++c)
      if (a->req_rows[c] == r) return ORACLE_EROWS;
    /* The LRU row is a permutation of the H slot ids. */
    char *seen = (char *)calloc((size_t)a->H, 1);
    if (!seen) return ORACLE_EARG;
    for (int32_t p = 0; p < a->H; ++p) {
      int32_t s = a->lru[r * a->H + p];
      if (s < 0 || s >= a->H || seen[s]) { free(seen); return ORACLE_ELRU; }
      seen[s] = 1;
    }
    free(seen);
    /* Every hot row a slot can name lies inside the hot buffer (paged
     * addressing has no newest slot). */
    for (int64_t s = 0; s < (a->paged ? a->H : a->H + 1); ++s) {
      int64_t hr = hot_row(a, r, s);
      if (hr < 0 || hr >= a->hot_nrows) return ORACLE_EHOT;
    }
  }
  return ORACLE_OK;
}

int oracle_swap_in(const oracle_swap_in_args *a) {
  int rc = check_args(a);
  if (rc != ORACLE_OK || a->B == 0 || a->K == 0) return rc;
  const int32_t B = a->B, K = a->K, H = a->H;
  const int32_t nreal = (a->num_real >= 0 && a->num_real < B) ? a->num_real : B;
  rc = check_state_rows(a, nreal);
  if (rc != ORACLE_OK) return rc;

  pending_t *pending = (pending_t *)malloc(sizeof(pending_t) * (size_t)K);
  int16_t *hits = (int16_t *)malloc(sizeof(int16_t) * (size_t)H);
  int16_t *evict = (int16_t *)malloc(sizeof(int16_t) * (size_t)H);
  int16_t *new_lru = (int16_t *)malloc(sizeof(int16_t) * (size_t)H);
  if (!pending || !hits || !evict || !new_lru) {
    free(pending); free(hits); free(evict); free(new_lru);
    return ORACLE_EARG;
  }

  for (int32_t b = 0; b < B; ++b) {
    int32_t *out = a->out_rows + (int64_t)b * K;
    const int32_t *ids = a->topk + (int64_t)b * a->topk_stride;
    const int64_t r = a->req_rows[b];

    int32_t *mask = a->miss_mask ? a->miss_mask + (int64_t)b * K : NULL;
    if (mask)
      for (int32_t i = 0; i < K; ++i) mask[i] = 0;
    if (a->list_count) a->list_count[b] = 0;

    /* Padding rows: -1 outputs and a zero count (vLLM page, V2 padding). */
    if (b >= nreal || r < 0 || r >= a->R) {
      for (int32_t i = 0; i < K; ++i) out[i] = -1;
      if (a->miss_counts) a->miss_counts[b] = 0;
      store_attention(a, b, out);
      continue;
    }
    const int64_t L = a->paged ? 0 : a->seq_lens[b];
    const int64_t newest = L - 1;
    int32_t *tokens = a->slot_tokens + r * a->S_r;
    int16_t *lru = a->lru + r * H;

    /* Step 1 (both pages' first loop): classify each top-k entry. The newest
     * token binds to slot H; everything else valid becomes pending. */
    int32_t np = 0;
    for (int32_t i = 0; i < K; ++i) {
      const int64_t t = ids[i];
      if (a->paged) {
        /* vLLM addressing: a resident entry is served from the device cache
         * as is, an entry without a global id is -1, and every other entry
         * is pending under its global id (no newest slot). */
        int64_t g, res;
        paged_translate(a, r, t, &g, &res);
        if (res >= 0) { out[i] = (int32_t)res; continue; }
        if (g < 0) { out[i] = -1; continue; }
        pending[np].token = (int32_t)g;
        pending[np].index = i;
        pending[np].hit = 0;
        ++np;
        continue;
      }
      if (t < 0 || t >= L || t >= a->ctx_stride) { out[i] = -1; continue; }
      const int64_t pr = pool_row(a, r, t);
      if (pr < 0 || pr >= a->pool_nrows) { out[i] = -1; continue; }
      if (t == newest) { out[i] = (int32_t)hot_row(a, r, H); continue; }
      pending[np].token = (int32_t)t;
      pending[np].index = i;
      pending[np].hit = 0;
      ++np;
    }
    qsort(pending, (size_t)np, sizeof(pending_t), cmp_by_token);
    for (int32_t j = 1; j < np; ++j)
      if (pending[j].token == pending[j - 1].token) { rc = ORACLE_EDUP_ID; goto done; }

    /* Step 2 (both pages' LRU scan): walk slots oldest first. A slot whose
     * token is pending is a hit and serves that entry; every other slot is
     * evictable. Both lists keep LRU order. */
    int32_t nh = 0, ne = 0;
    for (int32_t p = 0; p < H; ++p) {
      const int16_t s = lru[p];
      const int32_t tok = tokens[s];
      pending_t key = {tok, 0, 0};
      pending_t *f = tok >= 0 ? (pending_t *)bsearch(&key, pending, (size_t)np, sizeof(pending_t),
                                                     cmp_by_token)
                              : NULL;
      if (f) {
        if (f->hit) { rc = ORACLE_ESTATE; goto done; }
        f->hit = 1;
        out[f->index] = (int32_t)hot_row(a, r, s);
        hits[nh++] = s;
      } else {
        evict[ne++] = s;
      }
    }

    /* Step 3 (both pages' miss pass): pending entries that were not hit, in
     * ascending top-k index; miss m takes the m-th oldest evictable slot,
     * the table records the new owner and the row is copied in. */
    qsort(pending, (size_t)np, sizeof(pending_t), cmp_by_index);
    int32_t M = 0;
    for (int32_t j = 0; j < np; ++j) {
      if (pending[j].hit) continue;
      const int16_t v = evict[M];   /* M < ne because H >= K */
      const int64_t dst = hot_row(a, r, v);
      /* The pool row: the key itself under global keying. */
      const int64_t src = a->paged ? pending[j].token : pool_row(a, r, pending[j].token);
      out[pending[j].index] = (int32_t)dst;
      tokens[v] = pending[j].token;
      memcpy(a->hot + dst * a->row_bytes, a->pool + src * a->row_bytes, (size_t)a->row_bytes);
      /* Non-MLA caches: the V row travels with the K row (SGLang page,
       * !IsMLA branch of the miss copy: same source and destination rows). */
      if (a->pool_v)
        memcpy(a->hot_v + dst * a->row_bytes, a->pool_v + src * a->row_bytes, (size_t)a->row_bytes);
      /* The plan (vLLM page: miss_mask, and the compact swap lists in miss
       * order) that index-sharing layers replay. */
      if (mask) mask[pending[j].index] = 1;
      if (a->list_count) {
        a->list_src[(int64_t)b * K + M] = src;
        a->list_dst[(int64_t)b * K + M] = (int32_t)dst;
      }
      ++M;
    }
    if (a->list_count) a->list_count[b] = M;

    /* Step 4 (LRU write-back): stale evictables first, then the slots just
     * filled in miss order, then the hits, each group in its old order. */
    int32_t q = 0;
    for (int32_t e = M; e < ne; ++e) new_lru[q++] = evict[e];
    for (int32_t e = 0; e < M; ++e) new_lru[q++] = evict[e];
    for (int32_t h = 0; h < nh; ++h) new_lru[q++] = hits[h];
    memcpy(lru, new_lru, sizeof(int16_t) * (size_t)H);

    if (a->miss_counts) a->miss_counts[b] = M;
    if (a->stats) {
      a->stats[0] += (uint64_t)nh;
      a->stats[1] += (uint64_t)M;
    }
    store_attention(a, b, out);
  }

done:
  free(pending); free(hits); free(evict); free(new_lru);
  return rc;
}

int64_t oracle_gather_compact_layers(const int32_t *count, const int64_t *src, const int32_t *dst,
                                     int32_t B, int32_t K, const uint8_t *const *pool_layers,
                                     int64_t pool_nrows, uint8_t *const *hot_layers,
                                     int64_t hot_nrows, int32_t num_layers, int64_t row_bytes) {
  if (B < 0 || K < 0 || num_layers < 0 || row_bytes <= 0) return ORACLE_EARG;
  if (B > 0 && K > 0 && num_layers > 0 && (!count || !src || !dst || !pool_layers || !hot_layers))
    return ORACLE_EARG;
  int64_t zeroed = 0;
  for (int32_t l = 0; l < num_layers; ++l) {
    for (int32_t b = 0; b < B && K > 0; ++b) {
      int32_t n = count[b];
      if (n < 0) n = 0;
      if (n > K) n = K;
      for (int32_t m = 0; m < n; ++m) {
        const int64_t s = src[(int64_t)b * K + m];
        const int64_t d = dst[(int64_t)b * K + m];
        if (s < 0 || d < 0 || d >= hot_nrows) continue;
        uint8_t *to = hot_layers[l] + d * row_bytes;
        if (s < pool_nrows) {
          memcpy(to, pool_layers[l] + s * row_bytes, (size_t)row_bytes);
        } else {
          /* No source row: the vLLM page zeroes the planned slot rather than
           * leave stale bytes behind. */
          memset(to, 0, (size_t)row_bytes);
          ++zeroed;
        }
      }
    }
  }
  return zeroed;
}

int64_t oracle_transfer_rows_all_layer(const uint8_t *const *src_layers, uint8_t *const *dst_layers,
                                       int64_t src_nrows, int64_t dst_nrows,
                                       const int64_t *src_idx, const int64_t *dst_idx, int64_t n,
                                       int32_t num_layers, int64_t row_bytes) {
  if (n < 0 || num_layers < 0 || row_bytes <= 0) return ORACLE_EARG;
  if (n == 0 || num_layers == 0) return 0;
  if (!src_layers || !dst_layers || !src_idx || !dst_idx) return ORACLE_EARG;
  int64_t skipped = 0;
  /* tokenspeed page, all-layer MLA transfer: for every index pair, for every
   * layer, copy one row. */
  for (int64_t i = 0; i < n; ++i) {
    const int64_t s = src_idx[i], d = dst_idx[i];
    if (s < 0 || s >= src_nrows || d < 0 || d >= dst_nrows) { ++skipped; continue; }
    for (int32_t l = 0; l < num_layers; ++l)
      memcpy(dst_layers[l] + d * row_bytes, src_layers[l] + s * row_bytes, (size_t)row_bytes);
  }
  return skipped;
}

int64_t oracle_transfer_kv_all_layer(const uint8_t *const *k_src_layers,
                                     const uint8_t *const *v_src_layers,
                                     uint8_t *const *k_dst_layers, uint8_t *const *v_dst_layers,
                                     int64_t src_nrows, int64_t dst_nrows, const int64_t *src_idx,
                                     const int64_t *dst_idx, int64_t n, int32_t num_layers,
                                     int64_t row_bytes) {
  if (n < 0 || num_layers < 0 || row_bytes <= 0) return ORACLE_EARG;
  if (n == 0 || num_layers == 0) return 0;
  if (!k_src_layers || !v_src_layers || !k_dst_layers || !v_dst_layers || !src_idx || !dst_idx)
    return ORACLE_EARG;
  int64_t skipped = 0;
  /* tokenspeed page, all-layer K+V transfer: for every index pair, for every
   * layer, the K row and then the V row. */
  for (int64_t i = 0; i < n; ++i) {
    const int64_t s = src_idx[i], d = dst_idx[i];
    if (s < 0 || s >= src_nrows || d < 0 || d >= dst_nrows) { ++skipped; continue; }
    for (int32_t l = 0; l < num_layers; ++l) {
      memcpy(k_dst_layers[l] + d * row_bytes, k_src_layers[l] + s * row_bytes, (size_t)row_bytes);
      memcpy(v_dst_layers[l] + d * row_bytes, v_src_layers[l] + s * row_bytes, (size_t)row_bytes);
    }
  }
  return skipped;
}

int64_t oracle_store_kv_cache(const uint8_t *k_src, int64_t k_src_stride, const uint8_t *v_src,
                              int64_t v_src_stride, uint8_t *k_dst, int64_t k_dst_stride,
                              uint8_t *v_dst, int64_t v_dst_stride, int64_t dst_nrows,
                              const int64_t *loc, int64_t n, int64_t row_bytes) {
  if (n < 0 || row_bytes <= 0) return ORACLE_EARG;
  if (n == 0) return 0;
  if (!k_src || !v_src || !k_dst || !v_dst || !loc) return ORACLE_EARG;
  int64_t skipped = 0;
  /* tokenspeed page, _store_kv_cache_kernel: row j of each source goes to row
   * loc[j] of its destination. */
  for (int64_t j = 0; j < n; ++j) {
    if (loc[j] < 0 || loc[j] >= dst_nrows) { ++skipped; continue; }
    memcpy(k_dst + loc[j] * k_dst_stride, k_src + j * k_src_stride, (size_t)row_bytes);
    memcpy(v_dst + loc[j] * v_dst_stride, v_src + j * v_src_stride, (size_t)row_bytes);
  }
  return skipped;
}

int64_t oracle_store_kv_scatter(const uint8_t *src, int64_t src_row_stride_bytes,
                                uint8_t *dst, int64_t dst_row_stride_bytes, int64_t dst_nrows,
                                const int64_t *loc, int64_t n, int64_t row_bytes) {
  if (n < 0 || row_bytes <= 0) return ORACLE_EARG;
  if (n == 0) return 0;
  if (!src || !dst || !loc) return ORACLE_EARG;
  int64_t skipped = 0;
  /* tokenspeed page, _store_kv_cache_kernel (K half): row j goes to loc[j]. */
  for (int64_t j = 0; j < n; ++j) {
    if (loc[j] < 0 || loc[j] >= dst_nrows) { ++skipped; continue; }
    memcpy(dst + loc[j] * dst_row_stride_bytes, src + j * src_row_stride_bytes, (size_t)row_bytes);
  }
  return skipped;
}

int64_t oracle_invalidate_written(int32_t *slot_keys, int64_t R, int64_t S_r, const int64_t *rows,
                                  const int64_t *written, int64_t n) {
  if (R < 0 || S_r < 0 || n < 0) return ORACLE_EARG;
  if (n == 0) return 0;
  if (!slot_keys || !rows || !written) return ORACLE_EARG;
  int64_t cleared = 0;
  /* vLLM page, hisparse_invalidate_written_slots_kernel: a rewritten global
   * row must not be served from a stale hot copy. */
  for (int64_t j = 0; j < n; ++j) {
    const int64_t r = rows[j], g = written[j];
    if (r < 0 || r >= R || g < 0) continue;
    for (int64_t s = 0; s < S_r; ++s)
      if (slot_keys[r * S_r + s] == g) { slot_keys[r * S_r + s] = -1; ++cleared; }
  }
  return cleared;
}

int oracle_state_reset(int32_t *slot_tokens, int16_t *lru, const int64_t *rows, int64_t n_rows,
                       int32_t H, int64_t S_r, int64_t R) {
  if (!slot_tokens || !lru || !rows || n_rows < 0 || H < 0 || S_r < (int64_t)H + 1) return ORACLE_EARG;
  for (int64_t j = 0; j < n_rows; ++j) {
    const int64_t r = rows[j];
    if (r < 0 || r >= R) return ORACLE_EARG;
    for (int64_t s = 0; s < S_r; ++s) slot_tokens[r * S_r + s] = -1;
    for (int32_t p = 0; p < H; ++p) lru[r * H + p] = (int16_t)p;
  }
  return ORACLE_OK;
}
