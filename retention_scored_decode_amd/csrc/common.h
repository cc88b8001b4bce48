// Shared device helpers for the trimkv HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "trimkv.h"

namespace trimkv {

constexpr int PAGE = TRIMKV_PAGE_SIZE;
constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// fp32 score -> order-preserving uint32 key (larger score => larger key).
// -0.0 is folded onto +0.0; NaN (padding slots) maps to 0, below every real
// score (the smallest real key, that of -inf, is 0x007FFFFF).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s != s) return 0u;
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float qnan() { return __uint_as_float(0x7FC00000u); }

// Last index h in [0, n) with a[h] <= x (a nondecreasing, a[0] <= x).
__device__ __forceinline__ int upper_index(const int32_t* a, int n, int64_t x) {
  int lo = 0, hi = n;  // invariant: a[lo] <= x, answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of one int64 per thread (blockDim.x == NT).
// `tmp` is LDS of NT/64 + 1 int64.  Returns the exclusive prefix; *total is
// the block sum.  All threads must call it.
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* tmp, int64_t* total) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int wid = threadIdx.x / WAVE;
  int64_t x = v;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    int64_t y = __shfl_up(x, d, WAVE);
    if (lane >= d) x += y;
  }
  if (lane == WAVE - 1) tmp[wid] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t run = 0;
    for (int w = 0; w < NT / WAVE; ++w) {
      int64_t t = tmp[w];
      tmp[w] = run;
      run += t;
    }
    tmp[NT / WAVE] = run;
  }
  __syncthreads();
  int64_t r = tmp[wid] + x - v;
  *total = tmp[NT / WAVE];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Per-head work list over chunks of CP logical pages:
//   chunk_off[h] = sum_{h' < h} ceil(pages(h') / CP),  chunk_off[H] = total
//   chunk_head[c] = head of chunk c
// Computed by one block of NT threads.
// ---------------------------------------------------------------------------
template <int NT>
__device__ void build_chunk_list(const int32_t* __restrict__ page_off, int n_heads, int cp,
                                 int32_t* __restrict__ chunk_off, int32_t* __restrict__ chunk_head,
                                 int64_t* tmp) {
  int64_t carry = 0;
  for (int base = 0; base < n_heads; base += NT) {
    int h = base + threadIdx.x;
    int64_t n = 0;
    if (h < n_heads) {
      int64_t np = (int64_t)page_off[h + 1] - page_off[h];
      n = (np + cp - 1) / cp;
    }
    int64_t tot;
    int64_t ex = block_exclusive_scan<NT>(n, tmp, &tot);
    if (h < n_heads) chunk_off[h] = (int32_t)(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) chunk_off[n_heads] = (int32_t)carry;
  __syncthreads();
  for (int h = threadIdx.x; h < n_heads; h += NT) {
    int b = chunk_off[h], e = chunk_off[h + 1];
    for (int c = b; c < e; ++c) chunk_head[c] = h;
  }
}

// ---------------------------------------------------------------------------
// Exclusive prefix sums out[0..n] (out[n] = total) of load(0..n-1), by one
// block of NT threads, each scanning a contiguous run.
// ---------------------------------------------------------------------------
template <int NT, typename Load>
__device__ void block_scan_runs(int n, Load load, int64_t* __restrict__ out, int64_t* tmp) {
  const int R = (n + NT - 1) / NT;
  const int b = min((int)threadIdx.x * R, n), e = min(b + R, n);
  int64_t s = 0;
  for (int i = b; i < e; ++i) s += load(i);
  int64_t tot;
  int64_t base = block_exclusive_scan<NT>(s, tmp, &tot);
  for (int i = b; i < e; ++i) {
    out[i] = base;
    base += load(i);
  }
  if (threadIdx.x == 0) out[n] = tot;
}

// bf16 bits -> fp32
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace trimkv
