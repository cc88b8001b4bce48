// Exact global top-M per segment over fp32 keys, ties by (head, slot).
//
// DBTrimKV page, Method 3: one global budget M_global; every cached entry of
// every layer and head is ranked by predicted utility and the top M_global
// are kept.  TRIM-KV page, section 2: the lowest current scores are evicted
// once the budget is exceeded.
//
// Algorithm (per segment = contiguous range of heads sharing one budget):
//   1. scores -> order-preserving uint32 keys (-0.0 == +0.0);
//   2. three radix passes (11, 11, 10 bits) find K*, the M-th largest key,
//      and need = M - #{key > K*}: per-block LDS histograms, flushed with
//      device atomics into a per-segment histogram; the last block to finish
//      a segment scans its histogram and narrows the prefix;
//   3. per 1024-slot chunk: #{key > K*} and #{key == K*};
//   4. one block scans the tie counts in (head, slot) order: chunk c keeps
//      gt_c + clamp(need - E_c, 0, eq_c), E_c = ties in earlier chunks;
//   5. per chunk: keep = key > K*, or key == K* and its tie rank < need.
// Since CSR order within a segment is head order and, within a head, slot
// (= position) order, this realises "score desc, head asc, position asc".
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace trimkv {

namespace {

constexpr int CP = 64;          // pages per chunk
constexpr int CS = CP * PAGE;   // slots per chunk
constexpr int NT = 256;         // threads per chunk block (4 slots each)
constexpr int CPB = 8;          // chunks per histogram block
constexpr int HIST_WORDS = 2048 + 2048 + 1024;

enum { MODE_NORMAL = 0, MODE_ALL = 1, MODE_NONE = 2 };

struct SegState {
  int64_t remaining;  // 1-based rank of the target key among keys matching `prefix`
  int64_t n_valid;
  uint32_t prefix;
  int32_t mode;
  int32_t chunk_begin, chunk_end;
};

struct SelWs {
  int32_t* chunk_off;   // [H + 1]
  int32_t* chunk_head;  // [Tmax]
  int32_t* seg_of;      // [H]
  SegState* seg;        // [n_seg]
  uint32_t* hist;       // [n_seg][HIST_WORDS]
  uint32_t* done;       // [n_seg][4]
  int32_t* cnt;         // [Tmax][2]  (gt, eq)
  int64_t* p_gt;        // [Tmax + 1] exclusive prefix over chunks of gt
  int64_t* p_eq;        // [Tmax + 1] exclusive prefix over chunks of eq
  double* part;         // [Tmax]
};

struct CacheView {
  const int32_t* page_off;
  const int32_t* len;
  int n_heads;
};

__device__ __forceinline__ int pass_bits(int pass) { return pass == 2 ? 10 : 11; }
__device__ __forceinline__ uint32_t* pass_hist(const SelWs& w, int s, int pass) {
  return w.hist + (size_t)s * HIST_WORDS + (pass == 0 ? 0 : pass == 1 ? 2048 : 4096);
}

// valid entries and first CSR slot of chunk c of head h
__device__ __forceinline__ void chunk_geom(const CacheView& cv, const SelWs& w, int c, int h, int* nv,
                                           int64_t* csr0, int* nslots) {
  const int64_t e0 = (int64_t)(c - w.chunk_off[h]) * CS;
  const int64_t np = (int64_t)cv.page_off[h + 1] - cv.page_off[h];
  int64_t v = (int64_t)cv.len[h] - e0;
  *nv = (int)(v < 0 ? 0 : (v > CS ? CS : v));
  *csr0 = (int64_t)cv.page_off[h] * PAGE + e0;
  int64_t ns = np * PAGE - e0;
  *nslots = (int)(ns > CS ? CS : ns);
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_sel_prep(CacheView cv, int n_seg, const int32_t* __restrict__ seg_hb,
                                                   const int64_t* __restrict__ budget, SelWs w) {
  // every block: clear histograms and completion counters
  const size_t nclear = (size_t)n_seg * HIST_WORDS;
  for (size_t i = (size_t)blockIdx.x * 1024 + threadIdx.x; i < nclear; i += (size_t)gridDim.x * 1024)
    w.hist[i] = 0u;
  for (size_t i = (size_t)blockIdx.x * 1024 + threadIdx.x; i < (size_t)n_seg * 4; i += (size_t)gridDim.x * 1024)
    w.done[i] = 0u;
  if (blockIdx.x != 0) return;
  __shared__ int64_t tmp[1024 / WAVE + 1];
  build_chunk_list<1024>(cv.page_off, cv.n_heads, CP, w.chunk_off, w.chunk_head, tmp);
  __syncthreads();
  for (int s = threadIdx.x; s < n_seg; s += 1024) {
    const int hb = seg_hb[s], he = seg_hb[s + 1];
    for (int h = hb; h < he; ++h) w.seg_of[h] = s;
    SegState st;
    st.remaining = budget[s];
    st.n_valid = 0;
    st.prefix = 0u;
    st.chunk_begin = w.chunk_off[hb];
    st.chunk_end = w.chunk_off[he];
    st.mode = (budget[s] <= 0 || st.chunk_begin == st.chunk_end) ? MODE_NONE : MODE_NORMAL;
    w.seg[s] = st;
  }
}

// Last block of a segment: locate the bin holding the target rank.
__device__ void sel_find(const SelWs& w, int s, int pass) {
  __shared__ int64_t tmp[NT / WAVE + 1];
  const int nb = pass == 2 ? 1024 : 2048;
  const int per = nb / NT;  // 8 or 4
  const uint32_t* g = pass_hist(w, s, pass);
  uint32_t c[8];
  int64_t tsum = 0;
  for (int k = 0; k < per; ++k) {
    c[k] = __hip_atomic_load(g + threadIdx.x * per + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tsum += c[k];
  }
  int64_t total;
  const int64_t ex = block_exclusive_scan<NT>(tsum, tmp, &total);
  const int64_t above = total - ex - tsum;  // keys in bins of higher threads
  SegState st = w.seg[s];
  if (pass == 0) {
    if (threadIdx.x == 0) {
      w.seg[s].n_valid = total;
      if (st.remaining >= total) w.seg[s].mode = total == 0 ? MODE_NONE : MODE_ALL;
    }
    if (st.remaining >= total) return;
  }
  const int64_t r = st.remaining;
  if (above < r && r <= above + tsum) {
    int64_t cum = above;
    for (int k = per - 1; k >= 0; --k) {
      if (cum + c[k] >= r) {
        w.seg[s].remaining = r - cum;
        w.seg[s].prefix = (st.prefix << pass_bits(pass)) | (uint32_t)(threadIdx.x * per + k);
        break;
      }
      cum += c[k];
    }
  }
}

template <int PASS>
__global__ void __launch_bounds__(NT) k_sel_hist(CacheView cv, const float* __restrict__ score, SelWs w) {
  constexpr int NB = PASS == 2 ? 1024 : 2048;
  __shared__ uint32_t lh[NB];
  __shared__ int sh_mode, sh_last;
  __shared__ uint32_t sh_prefix;
  const int T = w.chunk_off[cv.n_heads];
  const int c0 = blockIdx.x * CPB;
  if (c0 >= T) return;
  const int c1 = min(c0 + CPB, T);
  for (int b = threadIdx.x; b < NB; b += NT) lh[b] = 0u;
  int cur = -1;
  auto flush = [&](int s) {
    __syncthreads();
    uint32_t* g = pass_hist(w, s, PASS);
    for (int b = threadIdx.x; b < NB; b += NT) {
      uint32_t v = lh[b];
      if (v) { atomicAdd(g + b, v); lh[b] = 0u; }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const SegState& st = w.seg[s];
      const int nblk = (st.chunk_end - 1) / CPB - st.chunk_begin / CPB + 1;
      uint32_t old = __hip_atomic_fetch_add(w.done + (size_t)s * 4 + PASS, 1u, __ATOMIC_ACQ_REL,
                                            __HIP_MEMORY_SCOPE_AGENT);
      sh_last = (old + 1u == (uint32_t)nblk);
    }
    __syncthreads();
    if (sh_last) {
      __threadfence();
      sel_find(w, s, PASS);
    }
    __syncthreads();
  };
  for (int c = c0; c < c1; ++c) {
    const int h = w.chunk_head[c];
    const int s = w.seg_of[h];
    if (s != cur) {
      if (cur >= 0 && sh_mode == MODE_NORMAL) flush(cur);
      __syncthreads();
      if (threadIdx.x == 0) {
        sh_mode = w.seg[s].mode;
        sh_prefix = w.seg[s].prefix;
      }
      __syncthreads();
      cur = s;
    }
    if (sh_mode != MODE_NORMAL) continue;
    int nv, nslots;
    int64_t csr0;
    chunk_geom(cv, w, c, h, &nv, &csr0, &nslots);
    const int i0 = threadIdx.x * 4;
    if (i0 < nv) {
      const float4 sv = *reinterpret_cast<const float4*>(score + csr0 + i0);
      const float a[4] = {sv.x, sv.y, sv.z, sv.w};
      const uint32_t pre = sh_prefix;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (i0 + k < nv) {
          const uint32_t key = score_key(a[k]);
          if (PASS == 0) {
            atomicAdd(&lh[key >> 21], 1u);
          } else if (PASS == 1) {
            if ((key >> 21) == pre) atomicAdd(&lh[(key >> 10) & 2047u], 1u);
          } else {
            if ((key >> 10) == pre) atomicAdd(&lh[key & 1023u], 1u);
          }
        }
      }
    }
  }
  if (cur >= 0 && sh_mode == MODE_NORMAL) flush(cur);
}

__device__ __forceinline__ int64_t block_sum_i64(int64_t v, int64_t* tmp) {
  int64_t tot;
  block_exclusive_scan<NT>(v, tmp, &tot);
  return tot;
}

__global__ void __launch_bounds__(NT) k_sel_count(CacheView cv, const float* __restrict__ score, SelWs w) {
  __shared__ int64_t tmp[NT / WAVE + 1];
  const int c = blockIdx.x;
  const int T = w.chunk_off[cv.n_heads];
  if (c >= T) return;
  const int h = w.chunk_head[c];
  const SegState st = w.seg[w.seg_of[h]];
  int nv, nslots;
  int64_t csr0;
  chunk_geom(cv, w, c, h, &nv, &csr0, &nslots);
  int gt = 0, eq = 0;
  const int i0 = threadIdx.x * 4;
  if (st.mode == MODE_ALL) {
    gt = max(0, min(4, nv - i0));
  } else if (st.mode == MODE_NORMAL && i0 < nv) {
    const float4 sv = *reinterpret_cast<const float4*>(score + csr0 + i0);
    const float a[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (i0 + k < nv) {
        const uint32_t key = score_key(a[k]);
        gt += key > st.prefix;
        eq += key == st.prefix;
      }
    }
  }
  const int64_t packed = ((int64_t)gt << 32) | (int64_t)eq;
  const int64_t tot = block_sum_i64(packed, tmp);
  if (threadIdx.x == 0) {
    w.cnt[2 * (size_t)c] = (int32_t)(tot >> 32);
    w.cnt[2 * (size_t)c + 1] = (int32_t)(tot & 0xFFFFFFFF);
  }
}

// Prefix sums of (gt, eq) over all chunks; kept[h] follows by telescoping:
// the ties a head takes from its consecutive chunks are
// clamp(need - E_first, 0, E_end - E_first), E = ties before, in the segment.
__global__ void __launch_bounds__(1024) k_sel_scan(CacheView cv, SelWs w, int32_t* __restrict__ kept) {
  __shared__ int64_t tmp[1024 / WAVE + 1];
  const int H = cv.n_heads;
  const int T = w.chunk_off[H];
  const int32_t* cnt = w.cnt;
  block_scan_runs<1024>(T, [cnt](int i) { return (int64_t)cnt[2 * (size_t)i]; }, w.p_gt, tmp);
  block_scan_runs<1024>(T, [cnt](int i) { return (int64_t)cnt[2 * (size_t)i + 1]; }, w.p_eq, tmp);
  __syncthreads();
  for (int h = threadIdx.x; h < H; h += 1024) {
    const SegState st = w.seg[w.seg_of[h]];
    const int cb = w.chunk_off[h], ce = w.chunk_off[h + 1];
    const int64_t gt = w.p_gt[ce] - w.p_gt[cb];
    int64_t k = 0;
    if (st.mode == MODE_ALL) {
      k = gt;
    } else if (st.mode == MODE_NORMAL) {
      const int64_t e_first = w.p_eq[cb] - w.p_eq[st.chunk_begin];
      const int64_t e_end = w.p_eq[ce] - w.p_eq[st.chunk_begin];
      int64_t take = st.remaining - e_first;
      take = take < 0 ? 0 : (take > e_end - e_first ? e_end - e_first : take);
      k = gt + take;
    }
    kept[h] = (int32_t)k;
  }
}

__device__ __forceinline__ double block_sum_f64(double v, double* tmpd) {
  // fixed-order tree: xor butterfly in each wave, then waves in order
  for (int d = WAVE / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, WAVE);
  const int wid = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) tmpd[wid] = v;
  __syncthreads();
  double r = 0.0;
  if (threadIdx.x == 0)
    for (int i = 0; i < NT / WAVE; ++i) r += tmpd[i];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(NT) k_sel_decide(CacheView cv, const float* __restrict__ score, SelWs w,
                                                   uint8_t* __restrict__ keep, int want_sum) {
  __shared__ int64_t tmp[NT / WAVE + 1];
  __shared__ double tmpd[NT / WAVE];
  const int c = blockIdx.x;
  const int T = w.chunk_off[cv.n_heads];
  if (c >= T) return;
  const int h = w.chunk_head[c];
  const SegState st = w.seg[w.seg_of[h]];
  int nv, nslots;
  int64_t csr0;
  chunk_geom(cv, w, c, h, &nv, &csr0, &nslots);
  const int i0 = threadIdx.x * 4;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  if (i0 < nv && st.mode != MODE_NONE) {
    const float4 sv = *reinterpret_cast<const float4*>(score + csr0 + i0);
    a[0] = sv.x; a[1] = sv.y; a[2] = sv.z; a[3] = sv.w;
  }
  uint32_t gtm = 0, eqm = 0;
  if (st.mode == MODE_NORMAL) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (i0 + k < nv) {
        const uint32_t key = score_key(a[k]);
        gtm |= (uint32_t)(key > st.prefix) << k;
        eqm |= (uint32_t)(key == st.prefix) << k;
      }
    }
  } else if (st.mode == MODE_ALL) {
#pragma unroll
    for (int k = 0; k < 4; ++k) gtm |= (uint32_t)(i0 + k < nv) << k;
  }
  int64_t tot;
  int64_t rank = (w.p_eq[c] - w.p_eq[st.chunk_begin]) + block_exclusive_scan<NT>((int64_t)__popc(eqm), tmp, &tot);
  uint32_t km = gtm;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (eqm & (1u << k)) {
      if (rank < st.remaining) km |= 1u << k;
      ++rank;
    }
  }
  if (i0 < nslots) {
    const uint32_t word = (km & 1u) | ((km & 2u) << 7) | ((km & 4u) << 14) | ((km & 8u) << 21);
    *reinterpret_cast<uint32_t*>(keep + csr0 + i0) = word;
  }
  if (want_sum) {
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (km & (1u << k)) sum += (double)a[k];
    const double bs = block_sum_f64(sum, tmpd);
    if (threadIdx.x == 0) w.part[c] = bs;
  }
}

__global__ void k_sel_headsum(CacheView cv, SelWs w, double* __restrict__ keptsum) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= cv.n_heads) return;
  double s = 0.0;
  for (int c = w.chunk_off[h]; c < w.chunk_off[h + 1]; ++c) s += w.part[c];
  keptsum[h] = s;
}

SelWs carve(const trimkv_cache_t* c, int n_seg, void* ws) {
  WsLayout L = select_ws_layout(c, n_seg);
  char* b = (char*)ws;
  SelWs w;
  w.chunk_off = (int32_t*)(b + L.off[0]);
  w.chunk_head = (int32_t*)(b + L.off[1]);
  w.seg_of = (int32_t*)(b + L.off[2]);
  w.seg = (SegState*)(b + L.off[3]);
  w.hist = (uint32_t*)(b + L.off[4]);
  w.done = (uint32_t*)(b + L.off[5]);
  w.cnt = (int32_t*)(b + L.off[6]);
  w.p_gt = (int64_t*)(b + L.off[7]);
  w.p_eq = (int64_t*)(b + L.off[8]);
  w.part = (double*)(b + L.off[9]);
  return w;
}

}  // namespace

WsLayout select_ws_layout(const trimkv_cache_t* c, int n_seg) {
  const int64_t T = max_chunks(c, CP);
  const int64_t H = c->n_heads;
  WsLayout L;
  L.add((H + 1) * 4);
  L.add(T * 4);
  L.add(H * 4);
  L.add((size_t)n_seg * sizeof(SegState));
  L.add((size_t)n_seg * HIST_WORDS * 4);
  L.add((size_t)n_seg * 16);
  L.add(T * 8);
  L.add((T + 1) * 8);
  L.add((T + 1) * 8);
  L.add(T * 8);
  return L;
}

int launch_select(const trimkv_cache_t* c, const float* score, int n_seg, const int32_t* seg,
                  const int64_t* budget, uint8_t* keep, int32_t* kept, double* keptsum, void* ws,
                  hipStream_t st) {
  SelWs w = carve(c, n_seg, ws);
  CacheView cv{c->page_off, c->len, c->n_heads};
  const int64_t T = max_chunks(c, CP);
  int prep_blocks = (int)std::min<int64_t>(64, ((int64_t)n_seg * HIST_WORDS + 1023) / 1024 + 1);
  hipLaunchKernelGGL(k_sel_prep, dim3(prep_blocks), dim3(1024), 0, st, cv, n_seg, seg, budget, w);
  const unsigned hb = (unsigned)((T + CPB - 1) / CPB);
  hipLaunchKernelGGL(k_sel_hist<0>, dim3(hb), dim3(NT), 0, st, cv, score, w);
  hipLaunchKernelGGL(k_sel_hist<1>, dim3(hb), dim3(NT), 0, st, cv, score, w);
  hipLaunchKernelGGL(k_sel_hist<2>, dim3(hb), dim3(NT), 0, st, cv, score, w);
  hipLaunchKernelGGL(k_sel_count, dim3((unsigned)T), dim3(NT), 0, st, cv, score, w);
  hipLaunchKernelGGL(k_sel_scan, dim3(1), dim3(1024), 0, st, cv, w, kept);
  hipLaunchKernelGGL(k_sel_decide, dim3((unsigned)T), dim3(NT), 0, st, cv, score, w, keep, keptsum != nullptr);
  if (keptsum)
    hipLaunchKernelGGL(k_sel_headsum, dim3((unsigned)((c->n_heads + 255) / 256)), dim3(256), 0, st, cv, w,
                       keptsum);
  return check_launch();
}

}  // namespace trimkv
