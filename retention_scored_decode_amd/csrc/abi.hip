// C ABI entry points: host-side validation, then the internal launchers.
// Nothing is enqueued unless every argument check passes.
#include <limits.h>

#include "common.h"
#include "launch.h"

using namespace trimkv;

namespace {

bool cache_shape_ok(const trimkv_cache_t* c, int* rc) {
  if (!c || c->n_heads < 0 || c->n_pages < 0 || c->n_pages > INT32_MAX) {
    *rc = TRIMKV_EINVAL;
    return false;
  }
  if (c->page_size != TRIMKV_PAGE_SIZE || (c->head_dim != 64 && c->head_dim != 128) ||
      (c->dtype != TRIMKV_F32 && c->dtype != TRIMKV_BF16)) {
    *rc = TRIMKV_EUNSUPPORTED;
    return false;
  }
  return true;
}

bool table_ok(const trimkv_cache_t* c) { return c->page_off && c->len && (c->n_pages == 0 || c->page_ids); }
bool pools_ok(const trimkv_cache_t* c) { return c->n_pages == 0 || (c->k && c->v && c->meta); }

int ws_check(void* ws, size_t have, size_t need) {
  if (need == 0) return TRIMKV_OK;
  return (ws && have >= need) ? TRIMKV_OK : TRIMKV_EWORKSPACE;
}

hipStream_t S(void* s) { return (hipStream_t)s; }

// ---------------------------------------------------------------------------
// validate_cache kernels
// ---------------------------------------------------------------------------
enum { BAD_TABLE = 1, BAD_LEN = 2, BAD_PAGEID = 4, BAD_POS_ORDER = 8, BAD_POS_T = 16, BAD_LNB = 32 };

__global__ void k_check_table(const int32_t* page_off, const int32_t* len, int n_heads, int64_t n_pages,
                              int32_t* flag) {
  for (int h = blockIdx.x * blockDim.x + threadIdx.x; h < n_heads; h += gridDim.x * blockDim.x) {
    const int64_t a = page_off[h], b = page_off[h + 1];
    int bad = 0;
    if (a < 0 || b < a || b > n_pages) bad |= BAD_TABLE;
    if (len[h] < 0 || (int64_t)len[h] > (b - a) * PAGE) bad |= BAD_LEN;
    if (bad) atomicOr(flag, bad);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && page_off[0] != 0) atomicOr(flag, BAD_TABLE);
}

__global__ void k_check_ids(const int32_t* page_off, const int32_t* page_ids, int n_heads, int64_t n_pages,
                            int32_t* flag) {
  const int64_t total = page_off[n_heads];
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (int64_t)gridDim.x * blockDim.x)
    if (page_ids[c] < 0 || page_ids[c] >= n_pages) atomicOr(flag, BAD_PAGEID);
}

__global__ void k_check_slots(const int32_t* page_off, const int32_t* page_ids, const int32_t* len,
                              const uint32_t* meta, int n_heads, const int32_t* t, int32_t* flag) {
  const int64_t total = page_off[n_heads];
  const int64_t c = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  if (c >= total) return;
  const int h = upper_index(page_off, n_heads + 1, c);
  const int64_t i = (c - page_off[h]) * PAGE + j;
  if (i >= len[h]) return;
  const uint32_t* mp = meta + (int64_t)page_ids[c] * (2 * PAGE);
  const int32_t pos = (int32_t)mp[PAGE + j];
  int bad = 0;
  if (pos >= t[0]) bad |= BAD_POS_T;
  const float l = __uint_as_float(mp[j]);
  if (!(l <= 0.0f)) bad |= BAD_LNB;
  if (i + 1 < len[h]) {
    const int64_t i1 = i + 1;
    const uint32_t* mp1 = meta + (int64_t)page_ids[page_off[h] + i1 / PAGE] * (2 * PAGE);
    if ((int32_t)mp1[PAGE + i1 % PAGE] <= pos) bad |= BAD_POS_ORDER;
  }
  if (bad) atomicOr(flag, bad);
}

}  // namespace

namespace {
thread_local hipEvent_t g_prof_start = nullptr;
thread_local hipEvent_t g_prof_stop = nullptr;
}  // namespace

// A measurement aid: a failed record leaves the caller's events unrecorded,
// which the caller sees when it reads them; the call itself goes on.
void trimkv::prof_begin(hipStream_t st) {
  if (g_prof_start) (void)hipEventRecord(g_prof_start, st);
}

void trimkv::prof_end(hipStream_t st) {
  if (g_prof_stop) (void)hipEventRecord(g_prof_stop, st);
  g_prof_start = g_prof_stop = nullptr;
}

extern "C" {

int trimkv_profile_next(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return TRIMKV_EINVAL;
  g_prof_start = (hipEvent_t)start;
  g_prof_stop = (hipEvent_t)stop;
  return TRIMKV_OK;
}

const char* trimkv_strerror(int s) {
  switch (s) {
    case TRIMKV_OK: return "ok";
    case TRIMKV_EINVAL: return "invalid argument";
    case TRIMKV_EUNSUPPORTED: return "unsupported configuration";
    case TRIMKV_EWORKSPACE: return "workspace missing or too small";
    case TRIMKV_ECAPACITY: return "destination pool too small";
    case TRIMKV_EHIP: return "HIP runtime error";
    case TRIMKV_EINVARIANT: return "cache invariant violated";
    default: return "unknown status";
  }
}

size_t trimkv_workspace_size(int op, const trimkv_cache_t* c, int32_t n_seg, int32_t group) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return 0;
  switch (op) {
    case TRIMKV_OP_SELECT: return n_seg >= 1 ? select_ws_layout(c, n_seg).total : 0;
    case TRIMKV_OP_COMPACT: return compact_ws_layout(c).total;
    case TRIMKV_OP_DECODE_ATTN: return (group >= 1 && group <= 16) ? attn_ws_layout(c, group).total : 0;
    case TRIMKV_OP_ATTN_MASS: return (group >= 1 && group <= 16) ? mass_ws_layout(c, group).total : 0;
    case TRIMKV_OP_VALIDATE: return 256;
    case TRIMKV_OP_DECODE_ERR: return (group >= 1 && group <= 16) ? err_ws_layout(c, group).total : 0;
    case TRIMKV_OP_COMPACT_INPLACE: return (size_t)c->n_heads * 4 + 256;
    case TRIMKV_OP_EVICT_TAILFILL: return tailfill_ws_layout(c).total;
    case TRIMKV_OP_DECODE_EVICT: return (group >= 1 && group <= 16) ? attn_evict_ws_layout(c, group).total : 0;
    default: return 0;
  }
}

int trimkv_log_beta(const float* beta, float* lnb, int64_t n, int32_t out_page_stride, void* stream) {
  if (n < 0 || out_page_stride < PAGE || (n > 0 && (!beta || !lnb))) return TRIMKV_EINVAL;
  return launch_log_beta(beta, lnb, n, out_page_stride, S(stream));
}

int trimkv_score(const trimkv_cache_t* c, int32_t n_seg, const int32_t* seg, const int32_t* t, float* score,
                 void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (n_seg < 1 || !seg || !t || !score || !table_ok(c) || !c->meta) return TRIMKV_EINVAL;
  if (c->n_heads == 0 || c->n_pages == 0) return TRIMKV_OK;
  return launch_score(c, n_seg, seg, t, score, S(stream));
}

int trimkv_select_global(const trimkv_cache_t* c, const float* score, int32_t n_seg, const int32_t* seg,
                         const int64_t* budget, uint8_t* keep, int32_t* kept, double* keptsum, int32_t* status,
                         void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  // meta: positions rank ties within a head
  if (n_seg < 1 || n_seg > c->n_heads || !score || !seg || !budget || !keep || !kept || !table_ok(c) ||
      (c->n_pages > 0 && !c->meta) || ((uintptr_t)keep & 15))
    return TRIMKV_EINVAL;
  if ((rc = ws_check(ws, ws_bytes, select_ws_layout(c, n_seg).total))) return rc;
  return launch_select(c, score, n_seg, seg, budget, keep, kept, keptsum, status, ws, S(stream));
}

int trimkv_score_select(const trimkv_cache_t* c, int32_t n_seg, const int32_t* seg, const int32_t* t,
                        const int64_t* budget, float* score, uint8_t* keep, int32_t* kept, double* keptsum,
                        int32_t* status, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (n_seg < 1 || n_seg > c->n_heads || !seg || !t || !budget || !score || !keep || !kept || !table_ok(c) ||
      (c->n_pages > 0 && !c->meta) || ((uintptr_t)keep & 15) || ((uintptr_t)score & 15))
    return TRIMKV_EINVAL;
  if ((rc = ws_check(ws, ws_bytes, select_ws_layout(c, n_seg).total))) return rc;
  return launch_score_select(c, n_seg, seg, t, budget, score, keep, kept, keptsum, status, ws, S(stream));
}

int trimkv_append_score_select(trimkv_cache_t* c, const void* k_new, const void* v_new, const float* beta_new,
                               int32_t n_seg, const int32_t* seg, const int32_t* t, const int64_t* budget,
                               float* score, uint8_t* keep, int32_t* kept, double* keptsum, int32_t* append_status,
                               int32_t* select_status, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (!k_new || !v_new || !beta_new || !pools_ok(c) || n_seg < 1 || n_seg > c->n_heads || !seg || !t || !budget ||
      !score || !keep || !kept || !table_ok(c) || (c->n_pages > 0 && !c->meta) || ((uintptr_t)keep & 15) ||
      ((uintptr_t)score & 15))
    return TRIMKV_EINVAL;
  if ((rc = ws_check(ws, ws_bytes, select_ws_layout(c, n_seg).total))) return rc;
  return launch_append_score_select(c, k_new, v_new, beta_new, n_seg, seg, t, budget, score, keep, kept, keptsum,
                                    append_status, select_status, ws, S(stream));
}

int trimkv_compact(const trimkv_cache_t* src, const uint8_t* keep, const int32_t* kept, int32_t reserve,
                   int64_t max_kept_total, trimkv_cache_t* dst, int64_t* pages_used, void* ws, size_t ws_bytes,
                   void* stream) {
  int rc;
  if (!cache_shape_ok(src, &rc)) return rc;
  if (!cache_shape_ok(dst, &rc)) return rc;
  if (!keep || !pages_used || reserve < 0 || max_kept_total < 0 || !table_ok(src) || !pools_ok(src) ||
      !table_ok(dst) || !pools_ok(dst) || !dst->page_ids || ((uintptr_t)keep & 15))
    return TRIMKV_EINVAL;
  // slots are carried as 32-bit indices
  if (src->n_pages * PAGE > (int64_t)UINT32_MAX || dst->n_pages * PAGE > (int64_t)UINT32_MAX)
    return TRIMKV_EUNSUPPORTED;
  if (dst->n_heads != src->n_heads || dst->head_dim != src->head_dim || dst->dtype != src->dtype)
    return TRIMKV_EINVAL;
  if (dst->k == src->k || dst->v == src->v || dst->meta == src->meta ||
      dst->page_off == src->page_off || dst->len == src->len)
    return TRIMKV_EINVAL;
  const int64_t H = src->n_heads;
  const int64_t need = (max_kept_total + H * reserve + PAGE - 1) / PAGE + H;
  if (dst->n_pages < need) return TRIMKV_ECAPACITY;
  if ((rc = ws_check(ws, ws_bytes, compact_ws_layout(src).total))) return rc;
  if (H == 0) return TRIMKV_OK;
  return launch_compact(src, keep, kept, reserve, max_kept_total, dst, pages_used, ws, S(stream));
}

int trimkv_compact_inplace(trimkv_cache_t* c, const uint8_t* keep, const int32_t* kept, int32_t reserve,
                           const int32_t* home_off, const int32_t* home_ids, int32_t* new_page_off,
                           int32_t* new_page_ids, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (!keep || reserve < 0 || !home_off || !home_ids || !new_page_off || !new_page_ids || !table_ok(c) ||
      !pools_ok(c) || ((uintptr_t)keep & 15))
    return TRIMKV_EINVAL;
  // the new table is written while the current one is still read
  if (new_page_off == c->page_off || new_page_ids == c->page_ids || new_page_off == home_off ||
      new_page_ids == home_ids)
    return TRIMKV_EINVAL;
  if (c->n_pages * PAGE > (int64_t)UINT32_MAX) return TRIMKV_EUNSUPPORTED;
  if ((rc = ws_check(ws, ws_bytes, (size_t)c->n_heads * 4 + 256))) return rc;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_compact_inplace(c, keep, kept, reserve, home_off, home_ids, new_page_off, new_page_ids, ws,
                                S(stream));
}

int trimkv_evict_tailfill(trimkv_cache_t* c, const uint8_t* keep, const int32_t* kept, int32_t reserve,
                          const int32_t* home_off, const int32_t* home_ids, int32_t* new_page_off,
                          int32_t* new_page_ids, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (!keep || reserve < 0 || !home_off || !home_ids || !new_page_off || !new_page_ids || !table_ok(c) ||
      !pools_ok(c) || ((uintptr_t)keep & 15))
    return TRIMKV_EINVAL;
  // the new table is written while the current one is still read
  if (new_page_off == c->page_off || new_page_ids == c->page_ids || new_page_off == home_off ||
      new_page_ids == home_ids)
    return TRIMKV_EINVAL;
  if (c->n_pages * PAGE > (int64_t)UINT32_MAX) return TRIMKV_EUNSUPPORTED;
  if ((rc = ws_check(ws, ws_bytes, tailfill_ws_layout(c).total))) return rc;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_evict_tailfill(c, keep, kept, reserve, home_off, home_ids, new_page_off, new_page_ids, ws,
                               S(stream));
}

int trimkv_decode_attn_evict_tailfill(trimkv_cache_t* c, const uint8_t* keep, const int32_t* kept, const void* q,
                                      int32_t group, float scale, float* out, float* dropped, int32_t reserve,
                                      const int32_t* home_off, const int32_t* home_ids, int32_t* new_page_off,
                                      int32_t* new_page_ids, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (group < 1 || group > 16) return TRIMKV_EUNSUPPORTED;
  if (!keep || !kept || !q || !out || !dropped || reserve < 0 || !home_off || !home_ids || !new_page_off ||
      !new_page_ids || !table_ok(c) || !pools_ok(c) || ((uintptr_t)keep & 15))
    return TRIMKV_EINVAL;
  // the new table is written while the current one is still read
  if (new_page_off == c->page_off || new_page_ids == c->page_ids || new_page_off == home_off ||
      new_page_ids == home_ids)
    return TRIMKV_EINVAL;
  if (c->n_pages * PAGE > (int64_t)UINT32_MAX) return TRIMKV_EUNSUPPORTED;
  if ((rc = ws_check(ws, ws_bytes, attn_evict_ws_layout(c, group).total))) return rc;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_decode_attn_evict_tailfill(c, keep, kept, q, group, scale, out, dropped, reserve, home_off, home_ids,
                                           new_page_off, new_page_ids, ws, S(stream));
}

int trimkv_decode_attn(const trimkv_cache_t* c, const uint8_t* keep, const float* lse_ref, const void* q,
                       int32_t group, float scale, float* out, float* dropped, float* lse_out, void* ws,
                       size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (group < 1 || group > 16) return TRIMKV_EUNSUPPORTED;
  if ((keep && lse_ref) || !q || !out || !dropped || !table_ok(c) || !pools_ok(c) || ((uintptr_t)keep & 15))
    return TRIMKV_EINVAL;
  if ((rc = ws_check(ws, ws_bytes, attn_ws_layout(c, group).total))) return rc;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_decode_attn(c, keep, lse_ref, q, group, scale, out, dropped, lse_out, ws, S(stream));
}

int trimkv_decode_attn_noalloc(const trimkv_cache_t* c, const uint8_t* keep, const float* lse_ref, const void* q,
                               int32_t group, float scale, float* out, float* dropped, float* lse_out, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (group < 1 || group > 16) return TRIMKV_EUNSUPPORTED;
  if ((keep && lse_ref) || !q || !out || !dropped || !table_ok(c) || !pools_ok(c) || ((uintptr_t)keep & 15))
    return TRIMKV_EINVAL;
  // a bound that needs no device query: too large for the scratch whatever the launch
  if (noalloc_min_bytes(c, group) > (int64_t)TRIMKV_NOALLOC_SCRATCH_BYTES) return TRIMKV_EWORKSPACE;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_decode_attn_noalloc(c, keep, lse_ref, q, group, scale, out, dropped, lse_out, S(stream));
}

int trimkv_decode_attn_gated(const trimkv_cache_t* c, int32_t n_seg, const int32_t* seg, const int32_t* t,
                             const uint8_t* keep, const void* q, int32_t group, float scale, float* out, float* dropped,
                             float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (group < 1 || group > 16 || c->dtype != TRIMKV_BF16) return TRIMKV_EUNSUPPORTED;
  if (n_seg < 1 || n_seg > c->n_heads || !seg || !t || !q || !out || !dropped || !table_ok(c) || !pools_ok(c) ||
      ((uintptr_t)keep & 15))
    return TRIMKV_EINVAL;
  if ((rc = ws_check(ws, ws_bytes, attn_ws_layout(c, group).total))) return rc;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_decode_attn_gated(c, n_seg, seg, t, keep, q, group, scale, out, dropped, lse_out, ws, S(stream));
}

int trimkv_decode_attn_err(const trimkv_cache_t* c, const uint8_t* keep, const void* q, int32_t group, float scale,
                           float* out, float* dropped, float* mu, float* err, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (group < 1 || group > 16 || c->dtype != TRIMKV_BF16) return TRIMKV_EUNSUPPORTED;
  if (!keep || !q || !out || !dropped || !err || !table_ok(c) || !pools_ok(c) || ((uintptr_t)keep & 15))
    return TRIMKV_EINVAL;
  if ((rc = ws_check(ws, ws_bytes, err_ws_layout(c, group).total))) return rc;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_decode_attn_err(c, keep, q, group, scale, out, dropped, mu, err, ws, S(stream));
}

int trimkv_attn_mass(const trimkv_cache_t* c, const void* q, int32_t group, float scale, float* mass,
                     float* lse_full, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (group < 1 || group > 16) return TRIMKV_EUNSUPPORTED;
  if (!q || !mass || !lse_full || !table_ok(c) || !pools_ok(c)) return TRIMKV_EINVAL;
  if ((rc = ws_check(ws, ws_bytes, mass_ws_layout(c, group).total))) return rc;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_attn_mass(c, q, group, scale, mass, lse_full, ws, S(stream));
}

int trimkv_allocate(const double* keptsum, const int32_t* len, int32_t n_heads, int64_t total_budget,
                    double* mbar_out, int64_t* budget_out, void* stream) {
  if (n_heads < 1 || n_heads > 16384 || total_budget < 0 || !keptsum || !len || !budget_out) return TRIMKV_EINVAL;
  return launch_allocate(keptsum, len, n_heads, total_budget, mbar_out, budget_out, S(stream));
}

int trimkv_allocate_floor(const double* keptsum, const int32_t* len, int32_t n_heads, int64_t total_budget,
                          int32_t floor, double* mbar_out, int64_t* budget_out, void* stream) {
  if (n_heads < 1 || n_heads > 16384 || total_budget < 0 || floor < 0 || !keptsum || !len || !budget_out)
    return TRIMKV_EINVAL;
  return launch_allocate_floor(keptsum, len, n_heads, total_budget, floor, mbar_out, budget_out, S(stream));
}

int trimkv_mark_recent(const trimkv_cache_t* c, int32_t floor, float* plane, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (floor < 0 || !plane || !table_ok(c)) return TRIMKV_EINVAL;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_mark_recent(c, floor, plane, S(stream));
}

int trimkv_append(trimkv_cache_t* c, const void* k_new, const void* v_new, const float* beta_new, const int32_t* t,
                  int32_t* status, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (!k_new || !v_new || !beta_new || !t || !table_ok(c) || !pools_ok(c)) return TRIMKV_EINVAL;
  if (c->n_heads == 0) return TRIMKV_OK;
  return launch_append(c, k_new, v_new, beta_new, t, status, S(stream));
}

int trimkv_validate_cache(const trimkv_cache_t* c, const int32_t* t, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if (!cache_shape_ok(c, &rc)) return rc;
  if (!t || !table_ok(c) || !pools_ok(c)) return TRIMKV_EINVAL;
  if ((rc = ws_check(ws, ws_bytes, 256))) return rc;
  if (c->n_heads == 0) return TRIMKV_OK;
  hipStream_t st = S(stream);
  int32_t* flag = (int32_t*)ws;
  int32_t host = 0;
  if (hipMemsetAsync(flag, 0, 4, st) != hipSuccess) return TRIMKV_EHIP;
  hipLaunchKernelGGL(k_check_table, dim3(64), dim3(256), 0, st, c->page_off, c->len, c->n_heads, c->n_pages, flag);
  if (hipMemcpyAsync(&host, flag, 4, hipMemcpyDeviceToHost, st) != hipSuccess) return TRIMKV_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return TRIMKV_EHIP;
  if (host) return TRIMKV_EINVARIANT;
  hipLaunchKernelGGL(k_check_ids, dim3(256), dim3(256), 0, st, c->page_off, c->page_ids, c->n_heads, c->n_pages,
                     flag);
  if (hipMemcpyAsync(&host, flag, 4, hipMemcpyDeviceToHost, st) != hipSuccess) return TRIMKV_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return TRIMKV_EHIP;
  if (host) return TRIMKV_EINVARIANT;
  if (c->n_pages > 0) {
    const int64_t blocks = (c->n_pages + 15) / 16;
    hipLaunchKernelGGL(k_check_slots, dim3((unsigned)blocks), dim3(256), 0, st, c->page_off, c->page_ids, c->len,
                       c->meta, c->n_heads, t, flag);
  }
  if (hipMemcpyAsync(&host, flag, 4, hipMemcpyDeviceToHost, st) != hipSuccess) return TRIMKV_EHIP;
  if (hipStreamSynchronize(st) != hipSuccess) return TRIMKV_EHIP;
  return host ? TRIMKV_EINVARIANT : TRIMKV_OK;
}

}  // extern "C"
