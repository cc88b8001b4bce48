// Internal launchers behind the C ABI (abi.hip validates, these enqueue).
#pragma once

#include "common.h"

namespace trimkv {

inline int check_launch() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? TRIMKV_OK : TRIMKV_EHIP;
}

// Measurement hook (trimkv_profile_next): events recorded on the call's
// stream right before and right after the call's main kernel(s).
void prof_begin(hipStream_t st);
void prof_end(hipStream_t st);

// Byte offsets of the pieces of one workspace; every piece 256-B aligned.
struct WsLayout {
  size_t off[16];
  size_t total;
  int n;
  void add(size_t bytes) {
    size_t a = (total + 255) & ~size_t(255);
    off[n++] = a;
    total = a + bytes;
  }
  WsLayout() : total(0), n(0) {}
};

// Upper bound on the number of chunks of `cp` pages over all heads.
inline int64_t max_chunks(const trimkv_cache_t* c, int cp) { return c->n_pages / cp + c->n_heads + 1; }

WsLayout select_ws_layout(const trimkv_cache_t* c, int n_seg);
WsLayout err_ws_layout(const trimkv_cache_t* c, int group);
WsLayout compact_ws_layout(const trimkv_cache_t* c);
WsLayout tailfill_ws_layout(const trimkv_cache_t* c);
WsLayout attn_ws_layout(const trimkv_cache_t* c, int group, int64_t slots = -1);
WsLayout attn_evict_ws_layout(const trimkv_cache_t* c, int group);
WsLayout mass_ws_layout(const trimkv_cache_t* c, int group);

int launch_log_beta(const float* beta, float* lnb, int64_t n, int out_page_stride, hipStream_t st);
int launch_score(const trimkv_cache_t* c, int n_seg, const int32_t* seg, const int32_t* t, float* score,
                 hipStream_t st);
int launch_append(trimkv_cache_t* c, const void* kn, const void* vn, const float* bn, const int32_t* t,
                  int32_t* status, hipStream_t st);
int launch_select(const trimkv_cache_t* c, const float* score, int n_seg, const int32_t* seg,
                  const int64_t* budget, uint8_t* keep, int32_t* kept, double* keptsum, int32_t* status, void* ws,
                  hipStream_t st);
int launch_score_select(const trimkv_cache_t* c, int n_seg, const int32_t* seg, const int32_t* t,
                        const int64_t* budget, float* score, uint8_t* keep, int32_t* kept, double* keptsum,
                        int32_t* status, void* ws, hipStream_t st);
int launch_append_score_select(trimkv_cache_t* c, const void* k_new, const void* v_new, const float* beta_new,
                               int n_seg, const int32_t* seg, const int32_t* t, const int64_t* budget, float* score,
                               uint8_t* keep, int32_t* kept, double* keptsum, int32_t* append_status,
                               int32_t* select_status, void* ws, hipStream_t st);
int launch_compact(const trimkv_cache_t* src, const uint8_t* keep, const int32_t* kept, int reserve,
                   int64_t max_kept_total, trimkv_cache_t* dst, int64_t* pages_used, void* ws, hipStream_t st);
int launch_compact_inplace(trimkv_cache_t* c, const uint8_t* keep, const int32_t* kept, int reserve,
                           const int32_t* home_off, const int32_t* home_ids, int32_t* new_off, int32_t* new_ids,
                           void* ws, hipStream_t st);
int launch_decode_attn_evict_tailfill(trimkv_cache_t* c, const uint8_t* keep, const int32_t* kept, const void* q,
                                      int group, float scale, float* out, float* dropped, int reserve,
                                      const int32_t* home_off, const int32_t* home_ids, int32_t* new_off,
                                      int32_t* new_ids, void* ws, hipStream_t st);
int launch_evict_tailfill(trimkv_cache_t* c, const uint8_t* keep, const int32_t* kept, int reserve,
                          const int32_t* home_off, const int32_t* home_ids, int32_t* new_off, int32_t* new_ids,
                          void* ws, hipStream_t st);
int launch_decode_attn_gated(const trimkv_cache_t* c, int n_seg, const int32_t* seg, const int32_t* t,
                             const uint8_t* keep, const void* q, int group, float scale, float* out, float* dropped,
                             float* lse_out, void* ws, hipStream_t st);
int launch_decode_attn_err(const trimkv_cache_t* c, const uint8_t* keep, const void* q, int group, float scale,
                           float* out, float* dropped, float* mu, float* err, void* ws, hipStream_t st);
int launch_decode_attn(const trimkv_cache_t* c, const uint8_t* keep, const float* lse_ref, const void* q,
                       int group, float scale, float* out, float* dropped, float* lse_out, void* ws,
                       hipStream_t st);
// allocation-free decode: partials in a static per-device scratch array
int64_t noalloc_min_bytes(const trimkv_cache_t* c, int group);
int launch_decode_attn_noalloc(const trimkv_cache_t* c, const uint8_t* keep, const float* lse_ref, const void* q,
                               int group, float scale, float* out, float* dropped, float* lse_out, hipStream_t st);
int launch_attn_mass(const trimkv_cache_t* c, const void* q, int group, float scale, float* mass,
                     float* lse_full, void* ws, hipStream_t st);
int launch_allocate_floor(const double* keptsum, const int32_t* len, int n_heads, int64_t budget, int floor_w,
                          double* mbar, int64_t* out, hipStream_t st);
int launch_mark_recent(const trimkv_cache_t* c, int floor_w, float* plane, hipStream_t st);
int launch_allocate(const double* keptsum, const int32_t* len, int n_heads, int64_t budget, double* mbar,
                    int64_t* out, hipStream_t st);
int launch_validate(const trimkv_cache_t* c, const int32_t* t, void* ws, hipStream_t st, int* bad);

}  // namespace trimkv
