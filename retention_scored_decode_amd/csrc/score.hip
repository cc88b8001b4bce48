// ln(beta) once per entry, the retention score of every cached entry, and
// the one-entry-per-head append of a decode step.
//
// DBTrimKV page, Method 2: r_{t,i} = beta_i^(t-i), so ln r = (t-i) ln beta_i.
// TRIM-KV page, section 2: beta in [0,1] is produced once, when the token is
// created; the decay beta^(t-i) is re-evaluated at every step.
#include "common.h"
#include "ln_table.h"
#include "launch.h"

namespace trimkv {

// ln(x) correctly rounded to float32 for x in [0, 1].
// A float64 log (error far below 8 float64 ulps) rounds to the correct
// float32 unless the true value lies close to a float32 rounding midpoint;
// those few inputs (ln within 40 float64 ulps of a midpoint) are listed in
// ln_table.h with their correctly rounded logarithm.  The check below flags
// every input whose float64 log lies within |y| * 2^-48 (16..32 ulps) of a
// midpoint, which covers every listed input and nothing that could round
// wrongly otherwise.
__device__ __forceinline__ float ln_f32_cr(float x) {
  double y = log((double)x);
  float f = (float)y;
  if (!(y < 0.0) || isinf(y)) return f;  // x == 1 -> +0, x == 0 -> -inf
  uint32_t fb = __float_as_uint(f);      // f < 0
  double fd = (double)f;
  double toward0 = (double)__uint_as_float(fb - 1u);
  double away = (double)__uint_as_float(fb + 1u);
  double thr = fabs(y) * 0x1p-48;
  if (fabs(y - 0.5 * (fd + toward0)) < thr || fabs(y - 0.5 * (fd + away)) < thr) {
    uint32_t xb = __float_as_uint(x);
    int lo = 0, hi = TRIMKV_LN_TABLE_N;
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (kLnHardIn[mid] < xb) lo = mid + 1; else hi = mid;
    }
    if (lo < TRIMKV_LN_TABLE_N && kLnHardIn[lo] == xb) return __uint_as_float(kLnHardOut[lo]);
  }
  return f;
}

__global__ void __launch_bounds__(256) k_log_beta(const float* __restrict__ beta, float* __restrict__ lnb,
                                                  int64_t n, int out_page_stride) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    lnb[(i / PAGE) * out_page_stride + i % PAGE] = ln_f32_cr(beta[i]);
}

// 64 CSR pages per block, 4 slots per thread (16-byte loads and stores).
__global__ void __launch_bounds__(256) k_score(const int32_t* __restrict__ page_off,
                                               const int32_t* __restrict__ page_ids,
                                               const int32_t* __restrict__ len,
                                               const uint32_t* __restrict__ meta, int n_heads,
                                               const int32_t* __restrict__ seg_head_begin, int n_seg,
                                               const int32_t* __restrict__ t, float* __restrict__ score) {
  __shared__ PageHeads sh;
  const int64_t total = page_off[n_heads];
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  if (c0 >= total) return;
  const PageHeads r = block_page_heads(page_off, n_heads, c0, min(c0 + 63, total - 1), &sh);
  const int64_t c = c0 + (threadIdx.x >> 2);
  const int j0 = (threadIdx.x & 3) * 4;
  if (c >= total) return;
  const int h = r.hf == r.hl ? r.hf : head_in_range(page_off, r, c);
  const int s = upper_index(seg_head_begin, n_seg + 1, h);
  const int64_t i0 = (c - page_off[h]) * PAGE + j0;
  const int64_t n = len[h];
  float4 out = make_float4(qnan(), qnan(), qnan(), qnan());
  if (i0 < n) {
    // ln(beta) and positions of one page share a 128-byte block
    const uint32_t* mp = meta + (int64_t)page_ids[c] * (2 * PAGE) + j0;
    const float4 l = *reinterpret_cast<const float4*>(mp);
    const int4 p = *reinterpret_cast<const int4*>(mp + PAGE);
    const int tt = t[s];
    out.x = __fmul_rn((float)(tt - p.x), l.x);
    if (i0 + 1 < n) out.y = __fmul_rn((float)(tt - p.y), l.y);
    if (i0 + 2 < n) out.z = __fmul_rn((float)(tt - p.z), l.z);
    if (i0 + 3 < n) out.w = __fmul_rn((float)(tt - p.w), l.w);
  }
  *reinterpret_cast<float4*>(score + c * PAGE + j0) = out;
}

// One wave per head: write entry len[h] and bump len[h].
template <typename T, int D>
__global__ void __launch_bounds__(64) k_append(const int32_t* __restrict__ page_off,
                                               const int32_t* __restrict__ page_ids,
                                               int32_t* __restrict__ len, T* __restrict__ k,
                                               T* __restrict__ v, uint32_t* __restrict__ meta,
                                               const T* __restrict__ k_new,
                                               const T* __restrict__ v_new,
                                               const float* __restrict__ beta_new,
                                               const int32_t* __restrict__ t) {
  const int h = blockIdx.x;
  const int n = len[h];
  const int64_t cap = (int64_t)(page_off[h + 1] - page_off[h]) * PAGE;
  if (n >= cap) return;
  const int64_t page = page_ids[page_off[h] + n / PAGE];
  const int64_t slot = page * PAGE + n % PAGE;
  for (int d = threadIdx.x; d < D; d += 64) {
    k[slot * D + d] = k_new[(int64_t)h * D + d];
    v[slot * D + d] = v_new[(int64_t)h * D + d];
  }
  if (threadIdx.x == 0) {
    meta[page * (2 * PAGE) + n % PAGE] = __float_as_uint(ln_f32_cr(beta_new[h]));
    meta[page * (2 * PAGE) + PAGE + n % PAGE] = (uint32_t)(t[0] - 1);
    len[h] = n + 1;
  }
}

int launch_log_beta(const float* beta, float* lnb, int64_t n, int out_page_stride, hipStream_t st) {
  if (n == 0) return TRIMKV_OK;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_log_beta, dim3((unsigned)blocks), dim3(256), 0, st, beta, lnb, n, out_page_stride);
  return check_launch();
}

int launch_score(const trimkv_cache_t* c, int n_seg, const int32_t* seg, const int32_t* t, float* score,
                 hipStream_t st) {
  int64_t blocks = (c->n_pages + 63) / 64;
  if (blocks == 0) return TRIMKV_OK;
  prof_begin(st);
  hipLaunchKernelGGL(k_score, dim3((unsigned)blocks), dim3(256), 0, st, c->page_off, c->page_ids, c->len,
                     c->meta, c->n_heads, seg, n_seg, t, score);
  prof_end(st);
  return check_launch();
}

template <typename T, int D>
static void append_t(trimkv_cache_t* c, const void* kn, const void* vn, const float* bn, const int32_t* t,
                     hipStream_t st) {
  hipLaunchKernelGGL((k_append<T, D>), dim3(c->n_heads), dim3(64), 0, st, c->page_off, c->page_ids, c->len,
                     (T*)c->k, (T*)c->v, c->meta, (const T*)kn, (const T*)vn, bn, t);
}

int launch_append(trimkv_cache_t* c, const void* kn, const void* vn, const float* bn, const int32_t* t,
                  hipStream_t st) {
  if (c->n_heads == 0) return TRIMKV_OK;
  if (c->dtype == TRIMKV_BF16) {
    if (c->head_dim == 128) append_t<uint16_t, 128>(c, kn, vn, bn, t, st);
    else append_t<uint16_t, 64>(c, kn, vn, bn, t, st);
  } else {
    if (c->head_dim == 128) append_t<float, 128>(c, kn, vn, bn, t, st);
    else append_t<float, 64>(c, kn, vn, bn, t, st);
  }
  return check_launch();
}

}  // namespace trimkv
