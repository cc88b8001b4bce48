// Per-head budgets proportional to the dropped-mass statistic.
//
// ContourKV page, section 3: the dropped mass of a head's top-mass set
// predicts where selection leaves a large gap, and the budget is given to
// those ("flat") heads.  Here b_h is proportional to mbar_h = 1 - keptsum_h
// with largest-remainder rounding, then capped at the head length with the
// excess offered again in remainder order.  With a recency floor w, every
// head first keeps its most recent min(w, len_h) entries; the budget left,
// max(B - sum of the floors, 0), is shared out as above over the entries
// above the floors, and b_h is the floor plus the share.
#include "common.h"
#include "launch.h"

namespace trimkv {

namespace {

constexpr int NT = 1024;

__device__ __forceinline__ int64_t block_sum(int64_t v, int64_t* tmp) {
  int64_t tot;
  block_exclusive_scan<NT>(v, tmp, &tot);
  return tot;
}

__device__ __forceinline__ double xval(double S, int64_t B, double mbar, int H) {
  return S > 0.0 ? ((double)B * mbar) / S : (double)B / (double)H;
}

// One block; H <= 16384.  Values every thread needs (the dropped masses for
// the head-order sum S, then the fractional parts for the ranks) are staged
// through LDS one chunk of NT heads at a time, each computed once.
__global__ void __launch_bounds__(NT) k_allocate(const double* __restrict__ keptsum, const int32_t* __restrict__ len,
                                                 int H, int64_t B_total, int floor_w, double* __restrict__ mbar_out,
                                                 int64_t* __restrict__ b) {
  __shared__ int64_t tmp[NT / WAVE + 1];
  __shared__ double sS;
  __shared__ double sbuf[NT];
  __shared__ int32_t srank[16384];
  auto fl_of = [&](int h) -> int64_t { return min((int64_t)floor_w, (int64_t)len[h]); };
  auto cap = [&](int h) -> int64_t { return (int64_t)len[h] - fl_of(h); };   // entries above the floor
  int64_t fsum = 0;
  for (int h = threadIdx.x; h < H; h += NT) fsum += fl_of(h);
  const int64_t B = max(B_total - block_sum(fsum, tmp), (int64_t)0);
  // S = sum of the dropped masses in head order (one thread adds, chunk by chunk)
  double S = 0.0;
  for (int c0 = 0; c0 < H; c0 += NT) {
    const int h = c0 + (int)threadIdx.x;
    if (h < H) sbuf[threadIdx.x] = 1.0 - keptsum[h];
    __syncthreads();
    if (threadIdx.x == 0) {
      const int n = min(NT, H - c0);
      for (int i = 0; i < n; ++i) S += sbuf[i];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) sS = S;
  __syncthreads();
  S = sS;
  auto frac_of = [&](int h) {
    const double x = xval(S, B, 1.0 - keptsum[h], H);
    return x - floor(x);
  };
  // rank in (fraction desc, head asc) order: every thread's heads against
  // each chunk of fractions
  constexpr int PER = 16384 / NT;
  double mine[PER];
  int32_t rk[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int h = (int)threadIdx.x + u * NT;
    mine[u] = h < H ? frac_of(h) : 0.0;
    rk[u] = 0;
  }
  for (int c0 = 0; c0 < H; c0 += NT) {
    const int o = c0 + (int)threadIdx.x;
    if (o < H) sbuf[threadIdx.x] = frac_of(o);
    __syncthreads();
    const int n = min(NT, H - c0);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int h = (int)threadIdx.x + u * NT;
      if (u * NT < H) {   // block-uniform
        // eight fractions requested per step, so their LDS latencies overlap
        // (one dependent read per element took about 20 us at 288 heads)
        int32_t r = 0;
        int i = 0;
        for (; i + 8 <= n; i += 8) {
          double fo[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) fo[k] = sbuf[i + k];
#pragma unroll
          for (int k = 0; k < 8; ++k) r += (fo[k] > mine[u]) || (fo[k] == mine[u] && c0 + i + k < h);
        }
        for (; i < n; ++i) {
          const double fo = sbuf[i];
          r += (fo > mine[u]) || (fo == mine[u] && c0 + i < h);
        }
        rk[u] += r;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int h = (int)threadIdx.x + u * NT;
    if (h < H) srank[h] = rk[u];
  }
  __syncthreads();
  int64_t part = 0;
  for (int h = threadIdx.x; h < H; h += NT) {
    const double m = 1.0 - keptsum[h];
    if (mbar_out) mbar_out[h] = m;
    const int64_t fl = (int64_t)floor(xval(S, B, m, H));
    b[h] = fl;
    part += fl;
  }
  const int64_t R = B - block_sum(part, tmp);
  int64_t excess = 0, maxroom = 0;
  for (int h = threadIdx.x; h < H; h += NT) {
    const int64_t rk = srank[h];
    int64_t v = b[h] + R / H + (rk < R % H ? 1 : 0);
    const int64_t L = cap(h);
    if (v > L) {
      excess += v - L;
      v = L;
    }
    b[h] = v;
    maxroom = max(maxroom, L - v);
  }
  excess = block_sum(excess, tmp);
  if (excess == 0) {
    for (int h = threadIdx.x; h < H; h += NT) b[h] += fl_of(h);
    return;
  }
  // water-fill: largest k with F(k) = sum_h min(room_h, k) <= excess
  __shared__ int64_t s_maxroom;
  if (threadIdx.x == 0) s_maxroom = 0;
  __syncthreads();
  atomicMax((unsigned long long*)&s_maxroom, (unsigned long long)maxroom);
  __syncthreads();
  int64_t lo = 0, hi = s_maxroom;  // F(lo) <= excess
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    int64_t f = 0;
    for (int h = threadIdx.x; h < H; h += NT) f += min(cap(h) - b[h], mid);
    f = block_sum(f, tmp);
    if (f <= excess) lo = mid; else hi = mid - 1;
  }
  const int64_t k = lo;
  int64_t f = 0;
  for (int h = threadIdx.x; h < H; h += NT) f += min(cap(h) - b[h], k);
  const int64_t left = excess - block_sum(f, tmp);
  // heads with room > k take one more unit, in rank order, while units remain
  int64_t add[16];
  int na = 0;
  for (int h = threadIdx.x; h < H; h += NT) {
    const int64_t room = cap(h) - b[h];
    int64_t v = b[h] + min(room, k);
    if (room > k && left > 0) {
      const int32_t rk = srank[h];
      int64_t er = 0;
      for (int o = 0; o < H; ++o)
        if (cap(o) - b[o] > k && srank[o] < rk) ++er;
      if (er < left) v += 1;
    }
    if (na < 16) add[na++] = v;
  }
  __syncthreads();
  na = 0;
  for (int h = threadIdx.x; h < H; h += NT) b[h] = add[na++] + fl_of(h);
}

// Entries of each head's most recent min(w, len_h) slots set to +inf in a
// CSR plane, so that a per-head selection takes them first.
__global__ void __launch_bounds__(256) k_mark_recent(const int32_t* __restrict__ page_off,
                                                     const int32_t* __restrict__ len, int w,
                                                     float* __restrict__ plane) {
  const int h = blockIdx.x;
  const int n = len[h];
  const int fl = min(w, n);
  const int64_t base = (int64_t)page_off[h] * PAGE;
  for (int i = n - fl + (int)threadIdx.x; i < n; i += 256) plane[base + i] = INFINITY;
}

}  // namespace

int launch_allocate(const double* keptsum, const int32_t* len, int n_heads, int64_t budget, double* mbar,
                    int64_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_allocate, dim3(1), dim3(NT), 0, st, keptsum, len, n_heads, budget, 0, mbar, out);
  return check_launch();
}

int launch_allocate_floor(const double* keptsum, const int32_t* len, int n_heads, int64_t budget, int floor_w,
                          double* mbar, int64_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_allocate, dim3(1), dim3(NT), 0, st, keptsum, len, n_heads, budget, floor_w, mbar, out);
  return check_launch();
}

int launch_mark_recent(const trimkv_cache_t* c, int floor_w, float* plane, hipStream_t st) {
  hipLaunchKernelGGL(k_mark_recent, dim3(c->n_heads), dim3(256), 0, st, c->page_off, c->len, floor_w, plane);
  return check_launch();
}

}  // namespace trimkv
