// ln(beta) once per entry, the retention score of every cached entry, and
// the one-entry-per-head append of a decode step.
//
// DBTrimKV page, Method 2: r_{t,i} = beta_i^(t-i), so ln r = (t-i) ln beta_i.
// TRIM-KV page, section 2: beta in [0,1] is produced once, when the token is
// created; the decay beta^(t-i) is re-evaluated at every step.
#include "common.h"
#include "launch.h"
#include "ln_cr.h"

namespace trimkv {

__global__ void __launch_bounds__(256) k_log_beta(const float* __restrict__ beta, float* __restrict__ lnb,
                                                  int64_t n, int out_page_stride) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    lnb[(i / PAGE) * out_page_stride + i % PAGE] = ln_f32_cr(beta[i]);
}

// TILES tiles of 64 CSR pages per block, 4 slots per thread (16-byte loads
// and stores).  A thread's physical pages depend only on its CSR pages, so
// they are requested before the block's head search; the metadata lines and
// the heads' table words are then requested together, so a block waits for
// about four round trips in all.  Large caches take 4 tiles per block
// (measured against 1, 2 and 8 on the 8B, batched and streaming caches: best
// or within 2% everywhere; batched 805 MB: 175 us against 187 and 196);
// small ones take 1, so that the grid still fills the GPU.
template <int SC_TILES>
__global__ void __launch_bounds__(256) k_score(const int32_t* __restrict__ page_off,
                                               const int32_t* __restrict__ page_ids,
                                               const int32_t* __restrict__ len,
                                               const uint32_t* __restrict__ meta, int n_heads,
                                               const int32_t* __restrict__ seg_head_begin, int n_seg,
                                               const int32_t* __restrict__ t, float* __restrict__ score) {
  __shared__ PageHeads sh;
  const int64_t total = page_off[n_heads];
  const int64_t b0 = (int64_t)blockIdx.x * (64 * SC_TILES);
  if (b0 >= total) return;
  const int64_t blast = min(b0 + 64 * SC_TILES - 1, total - 1);
  const int j0 = (threadIdx.x & 3) * 4;
  int64_t cc[SC_TILES];
  int pid[SC_TILES];
#pragma unroll
  for (int k = 0; k < SC_TILES; ++k) {
    cc[k] = b0 + k * 64 + (threadIdx.x >> 2);
    pid[k] = cc[k] <= blast ? page_ids[cc[k]] : 0;
  }
  const PageHeads r = block_page_heads(page_off, n_heads, b0, blast, &sh);
  // segments of the block's first and last heads (segments are head ranges)
  const int sf = upper_index(seg_head_begin, n_seg + 1, r.hf);
  const int sl = r.hl == r.hf ? sf : upper_index(seg_head_begin, n_seg + 1, r.hl);
  float4 lb[SC_TILES];
  int4 ps[SC_TILES];
  int hh[SC_TILES];
#pragma unroll
  for (int k = 0; k < SC_TILES; ++k) {
    if (cc[k] <= blast) {
      // ln(beta) and positions of one page share a 128-byte block
      const uint32_t* mp = meta + (int64_t)pid[k] * (2 * PAGE) + j0;
      lb[k] = *reinterpret_cast<const float4*>(mp);
      ps[k] = *reinterpret_cast<const int4*>(mp + PAGE);
      hh[k] = r.hf == r.hl ? r.hf : head_in_range(page_off, r, cc[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < SC_TILES; ++k) {
    if (cc[k] > blast) continue;
    const int h = hh[k];
    const int64_t i0 = (cc[k] - page_off[h]) * PAGE + j0;
    const int64_t n = len[h];
    float4 out = make_float4(qnan(), qnan(), qnan(), qnan());
    if (i0 < n) {
      const int s = sf == sl ? sf : upper_index(seg_head_begin, n_seg + 1, h);
      const int tt = t[s];
      out.x = __fmul_rn((float)(tt - ps[k].x), lb[k].x);
      if (i0 + 1 < n) out.y = __fmul_rn((float)(tt - ps[k].y), lb[k].y);
      if (i0 + 2 < n) out.z = __fmul_rn((float)(tt - ps[k].z), lb[k].z);
      if (i0 + 3 < n) out.w = __fmul_rn((float)(tt - ps[k].w), lb[k].w);
    }
    *reinterpret_cast<float4*>(score + cc[k] * PAGE + j0) = out;
  }
}

// One wave per head: write entry len[h] and bump len[h].  A head without a
// free slot is left unchanged and counted in *status (when given).
template <typename T, int D>
__global__ void __launch_bounds__(64) k_append(const int32_t* __restrict__ page_off,
                                               const int32_t* __restrict__ page_ids,
                                               int32_t* __restrict__ len, T* __restrict__ k,
                                               T* __restrict__ v, uint32_t* __restrict__ meta,
                                               const T* __restrict__ k_new,
                                               const T* __restrict__ v_new,
                                               const float* __restrict__ beta_new,
                                               const int32_t* __restrict__ t, int32_t* __restrict__ status) {
  const int h = blockIdx.x;
  const int n = len[h];
  const int64_t cap = (int64_t)(page_off[h + 1] - page_off[h]) * PAGE;
  if (n >= cap) {
    if (threadIdx.x == 0 && status) atomicAdd(status, 1);
    return;
  }
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
  const int64_t big = (c->n_pages + 255) / 256;   // blocks of 4 tiles
  if (big == 0) return TRIMKV_OK;
  prof_begin(st);
  if (big >= 1024)
    hipLaunchKernelGGL(k_score<4>, dim3((unsigned)big), dim3(256), 0, st, c->page_off, c->page_ids, c->len,
                       c->meta, c->n_heads, seg, n_seg, t, score);
  else
    hipLaunchKernelGGL(k_score<1>, dim3((unsigned)((c->n_pages + 63) / 64)), dim3(256), 0, st, c->page_off,
                       c->page_ids, c->len, c->meta, c->n_heads, seg, n_seg, t, score);
  prof_end(st);
  return check_launch();
}

template <typename T, int D>
static void append_t(trimkv_cache_t* c, const void* kn, const void* vn, const float* bn, const int32_t* t,
                     int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL((k_append<T, D>), dim3(c->n_heads), dim3(64), 0, st, c->page_off, c->page_ids, c->len,
                     (T*)c->k, (T*)c->v, c->meta, (const T*)kn, (const T*)vn, bn, t, status);
}

int launch_append(trimkv_cache_t* c, const void* kn, const void* vn, const float* bn, const int32_t* t,
                  int32_t* status, hipStream_t st) {
  if (c->n_heads == 0) return TRIMKV_OK;
  if (c->dtype == TRIMKV_BF16) {
    if (c->head_dim == 128) append_t<uint16_t, 128>(c, kn, vn, bn, t, status, st);
    else append_t<uint16_t, 64>(c, kn, vn, bn, t, status, st);
  } else {
    if (c->head_dim == 128) append_t<float, 128>(c, kn, vn, bn, t, status, st);
    else append_t<float, 64>(c, kn, vn, bn, t, status, st);
  }
  return check_launch();
}

}  // namespace trimkv
