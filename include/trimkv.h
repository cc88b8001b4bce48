/*
 * trimkv.h -- C ABI of the retention-scored KV eviction + decode library
 * (libtrimkv.so, HIP for gfx950 / MI355X).
 *
 * The method (DBTrimKV and TRIM-KV pages): every cached KV entry i of a head
 * carries a retention beta_i in [0,1] fixed at creation; at decode step t its
 * score is ln r = (t - i) ln beta_i.  One global budget M over all layers and
 * heads keeps the top-M scores; evicted entries are physically removed from
 * per-head page tables; decode attention runs over the retained entries with
 * forced (renormalised) weights and also reports the softmax mass that was
 * dropped (ContourKV page).
 *
 * Conventions shared by every entry point
 *  - All data pointers are DEVICE memory owned by the caller; the library
 *    never allocates, frees or keeps pointers after a call returns.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; no entry point synchronises the device except
 *    trimkv_validate_cache.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    negative status means nothing was launched.
 *  - Outputs never alias inputs, except trimkv_append (in place).
 *  - Calls that share a workspace or output buffers must be ordered (same
 *    stream or explicit events); otherwise they race.
 *  - State the library keeps between calls (host side, none of it holds
 *    caller data): the resident-wave count of each decode kernel per device
 *    (one occupancy query, cached per host thread); the per-device address
 *    of the static scratch of trimkv_decode_attn_noalloc (32 MiB of device
 *    memory held until the process ends); and the events that
 *    trimkv_profile_next arms for the next call (per host thread).
 *
 * Data layout ("paged, per-head variable length", DBTrimKV page, Method 4)
 *  - A head is one flat KV head h = (b * L + l) * H_kv + h_kv.
 *  - Page size is 16 entries.  Logical page c (0-based) of head h is CSR
 *    entry page_off[h] + c; it lives in physical page page_ids[page_off[h]+c].
 *    Entry i of head h is slot i % 16 of its logical page i / 16; entries
 *    i < len[h] are valid, and their positions are distinct; they ascend
 *    with i except after trimkv_evict_tailfill.
 *  - Pools: k, v [n_pages][16][head_dim] (bf16 or fp32); meta
 *    [n_pages][2][16] 32-bit words: for page p, meta[p][0][j] holds ln(beta)
 *    (fp32 bits) of slot j and meta[p][1][j] its token position (int32).  A
 *    page's metadata is one 128-byte block, so reading it costs one cache
 *    line whatever the physical page order.
 *  - "CSR plane": a per-slot array indexed by CSR slot
 *    s = (page_off[h] + i / 16) * 16 + i % 16, of length
 *    page_off[n_heads] * 16 (<= n_pages * 16).  Scores, keep flags and
 *    attention masses are CSR planes, so selection streams them
 *    contiguously whatever the physical page order.  Keep planes (uint8)
 *    must start on a 16-byte boundary (EINVAL otherwise).
 */
#ifndef TRIMKV_H
#define TRIMKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRIMKV_PAGE_SIZE 16

/* element type of K, V and q */
enum { TRIMKV_F32 = 0, TRIMKV_BF16 = 1 };

/* status codes */
enum {
  TRIMKV_OK = 0,
  TRIMKV_EINVAL = -1,       /* null / inconsistent arguments */
  TRIMKV_EUNSUPPORTED = -2, /* page_size != 16, head_dim not 64/128, dtype, group > 16 */
  TRIMKV_EWORKSPACE = -3,   /* workspace missing or smaller than trimkv_workspace_size() */
  TRIMKV_ECAPACITY = -4,    /* destination pool too small for the worst case */
  TRIMKV_EHIP = -5,         /* the HIP runtime reported an error */
  TRIMKV_EINVARIANT = -6    /* trimkv_validate_cache found a broken precondition */
};

typedef struct trimkv_cache {
  int32_t n_heads;   /* flat KV heads */
  int32_t head_dim;  /* 64 or 128 */
  int32_t page_size; /* must be 16 */
  int32_t dtype;     /* TRIMKV_F32 or TRIMKV_BF16 */
  int64_t n_pages;   /* pool capacity in pages */
  void* k;           /* [n_pages][16][head_dim] */
  void* v;           /* [n_pages][16][head_dim] */
  uint32_t* meta;    /* [n_pages][2][16]  ln(beta) (fp32 bits), then position (int32) */
  int32_t* page_off; /* [n_heads + 1]  CSR offsets, page_off[0] = 0, nondecreasing */
  int32_t* page_ids; /* [n_pages]      physical page of each CSR entry */
  int32_t* len;      /* [n_heads]      valid entries per head */
} trimkv_cache_t;

/* operation ids for trimkv_workspace_size */
enum {
  TRIMKV_OP_SCORE = 0,
  TRIMKV_OP_SELECT = 1,
  TRIMKV_OP_COMPACT = 2,
  TRIMKV_OP_DECODE_ATTN = 3,
  TRIMKV_OP_ATTN_MASS = 4,
  TRIMKV_OP_VALIDATE = 5,
  TRIMKV_OP_DECODE_ERR = 6,
  TRIMKV_OP_COMPACT_INPLACE = 7,
  TRIMKV_OP_EVICT_TAILFILL = 8,
  TRIMKV_OP_DECODE_EVICT = 9
};

/*
 * trimkv_log_beta -- ln(beta[i]) rounded to nearest fp32, for i < n.
 * TRIM-KV page, section 2: beta in [0,1] is assigned once, when the token is
 * created, so its logarithm is computed once per entry.  beta = 1 gives +0.0,
 * beta = 0 gives -inf.
 *   beta: [n] fp32, contiguous
 *   lnb:  output; element i goes to lnb[(i / 16) * out_page_stride + i % 16]:
 *         out_page_stride 16 writes a contiguous array, 32 writes the ln(beta)
 *         half of a cache's meta plane (lnb = (float*)meta).
 * Errors: EINVAL (null pointer with n > 0, n < 0, out_page_stride < 16).
 */
int trimkv_log_beta(const float* beta, float* lnb, int64_t n, int32_t out_page_stride, void* stream);

/*
 * trimkv_score -- retention score of every valid slot.
 * DBTrimKV page, Method 2 (r = beta^(t-i)); TRIM-KV page, section 2.
 * For each head h in segment s (heads seg_head_begin[s] .. seg_head_begin[s+1]-1)
 * and valid entry i:  score[csr slot] = (float)(t[s] - pos) * lnb, one fp32
 * product.  Padding slots of the head's pages receive a quiet NaN.
 *   seg_head_begin: device int32 [n_seg + 1], 0 .. n_heads, nondecreasing
 *   t:              device int32 [n_seg]; requires pos < t <= pos + 2^24
 *   score:          device fp32 CSR plane
 * Errors: EINVAL, EUNSUPPORTED.
 */
int trimkv_score(const trimkv_cache_t* cache, int32_t n_seg, const int32_t* seg_head_begin,
                 const int32_t* t, float* score, void* stream);

/*
 * trimkv_select_global -- exact global top-M per segment.
 * DBTrimKV page, Method 3 (one global budget: rank every cached entry of all
 * layers and heads, keep the top M_global); TRIM-KV page, section 2 (evict the
 * lowest current scores once the budget is exceeded).
 * Total order: score descending (-0.0 == +0.0, -inf below every finite
 * score, NaN below -inf), then flat head ascending, then position
 * descending (read from meta): among equal scores of one head the more
 * recent entry ranks first, so with beta = 1 everywhere (every score 0) each
 * head keeps its most recent entries.  Segment s keeps exactly min(max(budget[s], 0), N_s) entries,
 * N_s = valid entries of its heads.
 *   score:   device fp32 CSR plane (any fp32 key: retention scores or masses)
 *   cache->meta: positions rank tied entries (required)
 *   budget:  device int64 [n_seg]
 *   keep:    device uint8 CSR plane, out: 1 kept, 0 evicted (valid slots),
 *            0 in padding slots
 *   kept:    device int32 [n_heads], out: kept entries per head
 *   keptsum: device fp64 [n_heads] or NULL, out: sum of the kept scores of
 *            each head (a fixed-order tree within each 1024-slot chunk, chunks in order)
 *   status:  device int32 [1] or NULL: a failure counter that the call only
 *            increments (the caller clears it): +1 for every wait on the
 *            tie counts of earlier heads that gave up after its bounded spin
 *            (never expected; the keep plane of that segment is then not
 *            exact).  One counter may serve many calls and be read once.
 *   ws:      workspace of trimkv_workspace_size(TRIMKV_OP_SELECT, cache, n_seg, 0) bytes
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_select_global(const trimkv_cache_t* cache, const float* score, int32_t n_seg,
                         const int32_t* seg_head_begin, const int64_t* budget, uint8_t* keep,
                         int32_t* kept, double* keptsum, int32_t* status, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * trimkv_score_select -- trimkv_score and trimkv_select_global in one call:
 * the retention score of every valid slot is formed inside the selection's
 * first pass (DBTrimKV page, Method 2: r = beta^(t-i), ln r = (t - i) ln beta;
 * Method 3: one global top M over every layer and head), so the score plane
 * is written once and not read back for the first histogram.
 * Outputs are bit for bit those of trimkv_score (score, NaN in padding
 * slots) followed by trimkv_select_global on that plane.
 *   n_seg, seg_head_begin, t: as trimkv_score;  budget: as trimkv_select_global
 *   score:   device fp32 CSR plane, out (16-byte aligned)
 *   keep, kept, keptsum, status: as trimkv_select_global
 *   ws:      trimkv_workspace_size(TRIMKV_OP_SELECT, cache, n_seg, 0) bytes
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_score_select(const trimkv_cache_t* cache, int32_t n_seg, const int32_t* seg_head_begin,
                        const int32_t* t, const int64_t* budget, float* score, uint8_t* keep, int32_t* kept,
                        double* keptsum, int32_t* status, void* ws, size_t ws_bytes, void* stream);

/*
 * trimkv_append_score_select -- a generated step's append, score and
 * selection in one call, for streaming decode: trimkv_append followed by
 * trimkv_score_select, with the new entries written by the selection's first
 * kernel (one launch fewer per step).
 * TRIM-KV page, section 2 (a new entry per head with its retention, then the
 * lowest current scores are evicted once the budget is exceeded); DBTrimKV
 * page, Methods 2-3.
 * Entry len[h] of head h receives k_new[h], v_new[h], ln(beta_new[h]) and
 * position t[s] - 1, s the head's segment, and len[h] += 1, for every head
 * with a free slot; then every entry is scored at its segment's t and the top
 * budget[s] of each segment are kept.  With one segment the outputs, the
 * cache included, are bit for bit those of trimkv_append(t) followed by
 * trimkv_score_select.
 *   k_new, v_new, beta_new: as trimkv_append
 *   n_seg, seg_head_begin, t, budget, score, keep, kept, keptsum: as trimkv_score_select
 *   append_status: as trimkv_append's status (heads without a free slot)
 *   select_status: as trimkv_select_global's status
 *   ws:      trimkv_workspace_size(TRIMKV_OP_SELECT, cache, n_seg, 0) bytes
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_append_score_select(trimkv_cache_t* cache, const void* k_new, const void* v_new,
                               const float* beta_new, int32_t n_seg, const int32_t* seg_head_begin,
                               const int32_t* t, const int64_t* budget, float* score, uint8_t* keep,
                               int32_t* kept, double* keptsum, int32_t* append_status, int32_t* select_status,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * trimkv_compact -- physical eviction: stable out-of-place compaction.
 * DBTrimKV page, Method 4 (paged per-head variable length); ContourKV page,
 * section 2 (the budget must shrink storage, not just mask it).
 * Every kept entry of src (keep == 1) is copied, in slot order, to dst:
 * head h gets ceil((kept_h + reserve) / 16) pages numbered by a prefix sum
 * over heads in flat order, dst->page_ids[c] = c, dst->len[h] = kept_h.
 * K, V rows and their ln(beta) and position are copied bit for bit; padding slots are left
 * unspecified.  `reserve` spare slots per head let trimkv_append add entries.
 *   kept:          device int32 [n_heads] or NULL: the number of nonzero keep
 *                  bytes of each head's valid slots, as trimkv_select_global
 *                  wrote it for this keep plane; NULL counts them here (one
 *                  more kernel).  Counts that disagree with keep give an
 *                  unspecified layout (writes stay inside dst and ws).
 *   dst:           same n_heads/head_dim/dtype as src; its pools, page_off,
 *                  page_ids and len are written; must not overlap src.
 *   max_kept_total: host-side upper bound on the number of kept entries;
 *                  dst->n_pages must be >= ceil((max_kept_total +
 *                  n_heads*reserve)/16) + n_heads, else ECAPACITY.
 *   pages_used:    device int64 [1], out: dst->page_off[n_heads]
 *   ws:            trimkv_workspace_size(TRIMKV_OP_COMPACT, src, 0, 0) bytes
 *                  (it holds an 8-byte (source, destination) slot pair per
 *                  kept entry, so it grows with src->n_pages)
 * Slots are carried as 32-bit indices: n_pages * 16 of src and dst must fit
 * in 32 bits (EUNSUPPORTED otherwise).
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, ECAPACITY.
 */
int trimkv_compact(const trimkv_cache_t* src, const uint8_t* keep, const int32_t* kept, int32_t reserve,
                   int64_t max_kept_total, trimkv_cache_t* dst, int64_t* pages_used, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * trimkv_compact_inplace -- incremental eviction inside each head's own pages.
 * DBTrimKV page, Method 4 (paged per-head storage) and ContourKV page,
 * section 2 (eviction must shrink storage), without a second pool: suited to
 * streaming decode, where each step drops a few entries per head.
 * Every head keeps its kept entries (keep == 1), in slot order, in the first
 * slots of its own pages; only the entries after its first dropped entry
 * move.  The head's new page list is the first
 * min(ceil((kept_h + reserve) / 16), home pages of h) pages of its home list,
 * numbered by a prefix sum over heads into new_page_off / new_page_ids; then
 * cache->len[h] = kept_h.  The pools and len of `cache` are updated in place;
 * its page_off / page_ids are only read.  The caller's next view of the
 * cache is {the same pools, new_page_off, new_page_ids, len}.
 *   cache:        current view; each head's page list must be a prefix of its
 *                 home list (true of a home table itself and of every table
 *                 this call writes); n_pages * 16 must fit in 32 bits
 *   keep, kept:   as trimkv_compact (kept may be NULL: counted here)
 *   reserve:      spare slots per head for trimkv_append, within the head's
 *                 home pages
 *   home_off, home_ids: device int32 [n_heads + 1] and [home_off[n_heads]]:
 *                 each head's own pages (for example the prefill table)
 *   new_page_off: device int32 [n_heads + 1], out
 *   new_page_ids: device int32 [home_off[n_heads]], out; both distinct from
 *                 the cache's and the home table's arrays
 *   ws:           trimkv_workspace_size(TRIMKV_OP_COMPACT_INPLACE, cache, 0, 0) bytes
 * Counts that disagree with keep give an unspecified layout, with len
 * clamped to the new pages.  Calls that overlap on one cache race.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_compact_inplace(trimkv_cache_t* cache, const uint8_t* keep, const int32_t* kept, int32_t reserve,
                           const int32_t* home_off, const int32_t* home_ids, int32_t* new_page_off,
                           int32_t* new_page_ids, void* ws, size_t ws_bytes, void* stream);

/*
 * trimkv_evict_tailfill -- eviction in place that moves only the entries it
 * must.  DBTrimKV page, Method 4 (paged per-head storage) and ContourKV
 * page, section 2 (eviction must shrink storage), for streaming decode,
 * where each step drops a few entries per head.
 * Per head with kept_h kept entries: the dropped entries among its first
 * kept_h slots (holes) take, one each, the kept entries from slot kept_h on,
 * both counted in slot order; every other kept entry stays in its slot.  At
 * most the head's drops move.  The page table and len are then as
 * trimkv_compact_inplace writes them.  Afterwards the head's slots are no
 * longer in position order: selection ranks ties by position and attention
 * is order-free, so both are unaffected; trimkv_mark_recent and
 * trimkv_validate_cache's ascending-position check assume position order
 * and do not apply to such a cache.
 *   arguments: as trimkv_compact_inplace
 *   ws: trimkv_workspace_size(TRIMKV_OP_EVICT_TAILFILL, cache, 0, 0) bytes
 *       (a 4-byte slot per CSR slot for the holes)
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_evict_tailfill(trimkv_cache_t* cache, const uint8_t* keep, const int32_t* kept, int32_t reserve,
                          const int32_t* home_off, const int32_t* home_ids, int32_t* new_page_off,
                          int32_t* new_page_ids, void* ws, size_t ws_bytes, void* stream);

/*
 * trimkv_decode_attn_evict_tailfill -- an eviction step's attention and
 * its in-place eviction in one call, for streaming decode: mask-mode
 * trimkv_decode_attn over the cache as it is, then trimkv_evict_tailfill of
 * the same keep plane, with the attention's merge and the eviction in one
 * launch after the attention's main kernel (neither waits for the other).
 * ContourKV page, problem definition and section 3 (renormalised output
 * over the kept set, dropped mass); DBTrimKV page, Method 4 and ContourKV
 * page, section 2 (the eviction).
 * Outputs (out, dropped, the cache's rows, len and the new table) are bit
 * for bit those of the two calls.
 *   keep, q, group, scale, out, dropped: as trimkv_decode_attn (mask mode)
 *   kept:    device int32 [n_heads], the selection's counts (required)
 *   reserve, home_off, home_ids, new_page_off, new_page_ids: as
 *            trimkv_evict_tailfill
 *   ws: trimkv_workspace_size(TRIMKV_OP_DECODE_EVICT, cache, 0, group) bytes
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_decode_attn_evict_tailfill(trimkv_cache_t* cache, const uint8_t* keep, const int32_t* kept,
                                      const void* q, int32_t group, float scale, float* out, float* dropped,
                                      int32_t reserve, const int32_t* home_off, const int32_t* home_ids,
                                      int32_t* new_page_off, int32_t* new_page_ids, void* ws, size_t ws_bytes,
                                      void* stream);

/*
 * trimkv_decode_attn -- renormalised GQA decode attention with dropped mass.
 * ContourKV page, problem definition (keep a subset, renormalise the weights
 * over it, weights not re-optimised) and section 3 (dropped mass = total
 * softmax weight of the discarded keys).
 * Q head qh uses KV head qh / group.  z_j = scale * <q, k_j>; U = valid
 * entries of the head; A = U (keep == NULL) or {j : keep[j] == 1}.
 *   out[qh]     = sum_{A} e^{z_j} v_j / sum_{A} e^{z_j}   (0 if A is empty)
 *   dropped[qh] = sum_{U\A} e^{z_j} / sum_{U} e^{z_j}       (1 if A is empty)
 *   lse_out[qh] = ln sum_{A} e^{z_j}                        (-inf if A is empty)
 * With lse_ref (reference log-sum-exp of a larger set no longer stored,
 * e.g. from trimkv_attn_mass), dropped[qh] = 1 - exp(lse_out - lse_ref).
 * keep and lse_ref must not both be given.  The kept and the dropped keys'
 * weights are each formed against their own running maximum (fp32), so out
 * stays the kept set's average however far the dropped logits lie above it.
 *   q:       device [n_heads * group][head_dim], same dtype as K/V
 *   group:   1 .. 16
 *   out:     device fp32 [n_heads * group][head_dim]
 *   dropped: device fp32 [n_heads * group]
 *   lse_out: device fp32 [n_heads * group] or NULL
 *   ws:      trimkv_workspace_size(TRIMKV_OP_DECODE_ATTN, cache, 0, group) bytes
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_decode_attn(const trimkv_cache_t* cache, const uint8_t* keep, const float* lse_ref,
                       const void* q, int32_t group, float scale, float* out, float* dropped,
                       float* lse_out, void* ws, size_t ws_bytes, void* stream);

/*
 * trimkv_decode_attn_noalloc -- trimkv_decode_attn without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * outputs and kernels as trimkv_decode_attn, minus ws / ws_bytes: the
 * partial results live in a static scratch array of
 * TRIMKV_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds
 * until the process ends.  The call allocates and frees nothing.  All calls
 * on one GPU share that GPU's scratch: calls that overlap on one GPU (other
 * streams, other host threads without ordering) race; calls ordered on one
 * stream do not.  No part of the scratch needs clearing between calls.
 * Errors: as trimkv_decode_attn; EWORKSPACE when the call would need more
 * than TRIMKV_NOALLOC_SCRATCH_BYTES of partial results (about
 * (waves + n_heads) * group * (head_dim + 3) * 4 bytes, waves = 2048 for the
 * bf16 kernels on an MI355X); EHIP if the scratch address cannot be
 * obtained.
 */
#define TRIMKV_NOALLOC_SCRATCH_BYTES (32u << 20)
int trimkv_decode_attn_noalloc(const trimkv_cache_t* cache, const uint8_t* keep, const float* lse_ref,
                               const void* q, int32_t group, float scale, float* out, float* dropped,
                               float* lse_out, void* stream);

/*
 * trimkv_decode_attn_gated -- retention-gated decode attention.
 * TRIM-KV page, section 2 (attention modulation: the retention score
 * multiplies the attention weights; the page applies it in training) used
 * at decode time.  As trimkv_decode_attn with every weight e^{z_j} replaced
 * by e^{z_j} * r_j, r_j = beta_j^(t - pos_j): the logit gains
 * ln r_j = fp32(t - pos_j) * ln beta_j, formed exactly as trimkv_score forms
 * the score (t of the head's segment, ln beta and position from meta).
 *   out[qh]     = sum_{A} e^{z_j} r_j v_j / sum_{A} e^{z_j} r_j   (0 if A is empty)
 *   dropped[qh] = sum_{U\A} e^{z_j} r_j / sum_{U} e^{z_j} r_j     (1 if A is empty)
 *   lse_out[qh] = ln sum_{A} e^{z_j} r_j                          (-inf if A is empty)
 * keep == NULL means A = U.  Entries with beta = 0 need t > pos (0 * -inf).
 *   n_seg, seg_head_begin, t: as trimkv_score (device int32)
 *   other arguments as trimkv_decode_attn (no lse_ref); bf16 caches only
 *   ws: trimkv_workspace_size(TRIMKV_OP_DECODE_ATTN, cache, 0, group) bytes
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_decode_attn_gated(const trimkv_cache_t* cache, int32_t n_seg, const int32_t* seg_head_begin,
                             const int32_t* t, const uint8_t* keep, const void* q, int32_t group, float scale,
                             float* out, float* dropped, float* lse_out, void* ws, size_t ws_bytes, void* stream);

/*
 * trimkv_decode_attn_err -- mask-mode decode attention that also measures
 * what the forced weights cost: e_s(A) = || mu - m_A ||_2 per query head.
 * ContourKV page, section 1 (theoretical analysis): mu is the dense
 * attention output over every valid entry U of the head, m_A the output
 * renormalised over the kept set A; the norm is the Euclidean norm over the
 * head_dim output components (the page leaves the norm unnamed).
 *   keep:    device uint8 CSR plane (16-byte aligned), A = {j : keep[j] == 1}
 *   out, dropped: as trimkv_decode_attn with this keep plane (out = m_A)
 *   mu:      device fp32 [n_heads * group][head_dim] or NULL: the dense output
 *            (0 for a head without valid entries)
 *   err:     device fp32 [n_heads * group]: || mu - m_A ||_2, with m_A = 0 when
 *            A is empty (so err = || mu ||)
 *   ws:      trimkv_workspace_size(TRIMKV_OP_DECODE_ERR, cache, 0, group) bytes
 * Reads every V row (the mask mode reads only the kept ones).  bf16 caches
 * only (EUNSUPPORTED for fp32).
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_decode_attn_err(const trimkv_cache_t* cache, const uint8_t* keep, const void* q, int32_t group,
                           float scale, float* out, float* dropped, float* mu, float* err, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * trimkv_attn_mass -- query-aware attention mass of every cached key.
 * ContourKV page, sections 1 and 3 (top-mass selection; the dropped-mass
 * statistic).  For KV head h with Q heads g = 0..group-1:
 *   lse_full[h*group+g] = ln sum_{j in U} e^{z_gj}
 *   mass[csr slot j]    = (1/group) sum_g e^{z_gj - lse_full[h*group+g]}
 * Padding slots receive a quiet NaN.
 *   mass:     device fp32 CSR plane;  lse_full: device fp32 [n_heads * group]
 *   ws:       trimkv_workspace_size(TRIMKV_OP_ATTN_MASS, cache, 0, group) bytes
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE.
 */
int trimkv_attn_mass(const trimkv_cache_t* cache, const void* q, int32_t group, float scale,
                     float* mass, float* lse_full, void* ws, size_t ws_bytes, void* stream);

/*
 * trimkv_allocate -- per-head budgets proportional to dropped mass.
 * ContourKV page, section 3 (give budget to the heads whose top-mass set
 * leaves the most mass behind).  With keptsum_h the mass of head h's top-s
 * set (trimkv_select_global on trimkv_attn_mass output):
 *   mbar_h = 1 - keptsum_h;  S = sum_h mbar_h (fp64, head order);
 *   x_h = (B * mbar_h) / S  (B / n_heads if S == 0);  b_h = floor(x_h);
 *   the B - sum b_h leftover units go one each to the largest x_h - b_h
 *   (ties: lower head); then b_h is capped at len_h and the excess is
 *   offered again, one unit per head per pass in the same order, to heads
 *   below their length.
 *   keptsum: device fp64 [n_heads];  len: device int32 [n_heads]
 *   mbar_out: device fp64 [n_heads] or NULL;  budget_out: device int64 [n_heads]
 * Errors: EINVAL (n_heads < 1 or > 16384, total_budget < 0).
 */
int trimkv_allocate(const double* keptsum, const int32_t* len, int32_t n_heads,
                    int64_t total_budget, double* mbar_out, int64_t* budget_out, void* stream);

/*
 * trimkv_allocate_floor -- trimkv_allocate with ContourKV's recency floor.
 * ContourKV page, section 3 (a recency floor kept in every head while the
 * budget goes to the flat heads).  Head h first keeps its most recent
 * floor_h = min(floor, len_h) entries; B' = max(total_budget - sum_h floor_h,
 * 0) is shared out by the rule of trimkv_allocate with caps len_h - floor_h;
 * budget_out[h] = floor_h + share_h (so the floors are kept even when their
 * sum exceeds total_budget).  floor = 0 gives trimkv_allocate.
 *   arguments as trimkv_allocate;  floor >= 0
 * Errors: EINVAL (as trimkv_allocate, or floor < 0).
 */
int trimkv_allocate_floor(const double* keptsum, const int32_t* len, int32_t n_heads, int64_t total_budget,
                          int32_t floor, double* mbar_out, int64_t* budget_out, void* stream);

/*
 * trimkv_mark_recent -- mark each head's recency floor in a CSR plane.
 * ContourKV page, section 3 (recency floor).  plane[csr slot of entry i of
 * head h] = +inf for len_h - min(floor, len_h) <= i < len_h, every other slot
 * unchanged.  A per-head trimkv_select_global with budget_out of
 * trimkv_allocate_floor on a plane of finite scores (attention masses) then
 * keeps the floor plus the top share_h of the other entries.
 *   plane: device fp32 CSR plane;  floor >= 0
 * Errors: EINVAL, EUNSUPPORTED (cache shape).
 */
int trimkv_mark_recent(const trimkv_cache_t* cache, int32_t floor, float* plane, void* stream);

/*
 * trimkv_append -- add one new entry per head at decode step *t.
 * TRIM-KV page, section 2 (beta assigned when the token is created).
 * Entry len[h] of head h receives k_new[h], v_new[h], ln(beta_new[h]) (as
 * trimkv_log_beta) and position *t - 1; then len[h] += 1.  The head must have
 * a free slot in its pages (trimkv_compact with reserve >= 1); a head without
 * one is left unchanged and counted in *status.
 *   k_new, v_new: device [n_heads][head_dim] (cache dtype); beta_new: fp32 [n_heads]
 *   t: device int32 [1]
 *   status: device int32 [1] or NULL: a failure counter that the call only
 *           increments (the caller clears it), by the number of heads that
 *           had no free slot.  One counter may serve a whole decode loop and
 *           be read once at its end (0: every entry was appended).
 * Errors: EINVAL, EUNSUPPORTED.
 */
int trimkv_append(trimkv_cache_t* cache, const void* k_new, const void* v_new,
                  const float* beta_new, const int32_t* t, int32_t* status, void* stream);

/* Bytes of workspace an operation needs for this cache (0 if none). */
size_t trimkv_workspace_size(int op, const trimkv_cache_t* cache, int32_t n_seg, int32_t group);

/*
 * trimkv_validate_cache -- debug check of the preconditions (synchronises):
 * page_off nondecreasing, within n_pages; page_ids in range; len within the
 * head's pages; positions ascending within each head and < *t; ln(beta) <= 0
 * and not NaN.
 * Returns TRIMKV_OK or TRIMKV_EINVARIANT (or an argument / HIP error).
 *   t: device int32 [1];  ws: trimkv_workspace_size(TRIMKV_OP_VALIDATE, ...) bytes
 */
int trimkv_validate_cache(const trimkv_cache_t* cache, const int32_t* t, void* ws,
                          size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* trimkv_strerror(int status);

/*
 * trimkv_profile_next -- measurement hook, not part of the method.
 * The next call on this host thread that launches its main kernel(s)
 * records `start` (a hipEvent_t created by the caller) on its stream right
 * before them and `stop` right after, then disarms the hook.  Main kernels:
 * trimkv_score -> the score kernel; trimkv_select_global -> the three
 * histogram passes and the decision pass; trimkv_compact -> the row copy;
 * trimkv_decode_attn / trimkv_attn_mass -> the attention kernel (not its
 * work-list preparation or the merge).  Both NULL disarms.
 * Errors: EINVAL (exactly one of the two is NULL).
 */
int trimkv_profile_next(void* start, void* stop);

#ifdef __cplusplus
}
#endif
#endif /* TRIMKV_H */
