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
// Workgroup barrier ordering LDS only.  __syncthreads() also drains every
// outstanding global store and atomic of the wave (a workgroup release on
// all address spaces); where a barrier only hands LDS data between threads
// this one waits for LDS operations alone.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The value of lane i - D of the same 16-lane DPP row, 0 for the row's
// first D lanes (row_shr with bound_ctrl off keeps the `old` operand, 0).
template <int D>
__device__ __forceinline__ int64_t row_shr(int64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, 0x110 + D, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)((uint64_t)v >> 32), 0x110 + D, 0xF, 0xF, false);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
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
  lds_barrier();
  static_assert(NT / WAVE <= 16, "the wave totals fit one DPP row");
  if (wid == 0) {   // wave totals scanned in the first row of wave 0: two live registers, not NT/32
    const int64_t t = lane < NT / WAVE ? tmp[lane] : 0;
    int64_t s = t;
    if constexpr (NT / WAVE > 1) s += row_shr<1>(s);
    if constexpr (NT / WAVE > 2) s += row_shr<2>(s);
    if constexpr (NT / WAVE > 4) s += row_shr<4>(s);
    if constexpr (NT / WAVE > 8) s += row_shr<8>(s);
    if (lane < NT / WAVE) tmp[lane] = s - t;
    if (lane == NT / WAVE - 1) tmp[NT / WAVE] = s;
  }
  lds_barrier();
  int64_t r = tmp[wid] + x - v;
  *total = tmp[NT / WAVE];
  lds_barrier();
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

// ---------------------------------------------------------------------------
// Heads of the CSR pages [c0, c0 + npages) for a block: the first and last
// head are found once (thread 0, binary search over page_off) and shared;
// a page between them is then located by a search over that short range.
// ---------------------------------------------------------------------------
struct PageHeads {
  int hf, hl;
};

// upper_index by a whole wave: 64 probes per step (one per lane) and a
// ballot, so n entries take ceil(log64 n) dependent loads instead of log2 n.
// Every lane returns the same index.
__device__ __forceinline__ int wave_upper_index(const int32_t* __restrict__ a, int n, int64_t x) {
  const int lane = threadIdx.x & (WAVE - 1);
  int lo = 0, hi = n;  // invariant: a[lo] <= x, answer in [lo, hi)
  while (hi - lo > 1) {
    const int step = (hi - lo + WAVE - 1) / WAVE;
    const int i = lo + lane * step;
    const uint64_t le = __ballot(i < hi && (int64_t)a[i] <= x);   // a prefix of the lanes, lane 0 included
    lo += (63 - __clzll((long long)le)) * step;
    hi = min(lo + step, hi);
  }
  return lo;
}

// Heads of the first and last CSR page of a block (waves 0 and 1 search in
// parallel; blockDim.x >= 128).
__device__ __forceinline__ PageHeads block_page_heads(const int32_t* __restrict__ page_off, int n_heads, int64_t c0,
                                                      int64_t clast, PageHeads* sh) {
  const int wid = threadIdx.x / WAVE;
  if (wid < 2) {
    const int h = wave_upper_index(page_off, n_heads + 1, wid == 0 ? c0 : clast);
    if ((threadIdx.x & (WAVE - 1)) == 0) (wid == 0 ? sh->hf : sh->hl) = h;
  }
  __syncthreads();
  return *sh;
}

__device__ __forceinline__ int head_in_range(const int32_t* __restrict__ page_off, PageHeads r, int64_t c) {
  int lo = r.hf, hi = r.hl + 1;  // page_off[lo] <= c < page_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)page_off[mid] <= c) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Chunk list shared by the prep kernels.  Every block rebuilds, in LDS, the
// exclusive scan over heads of ceil(pages(h) / cp) together with copies of
// page_off and len (n_heads <= PREP_HMAX); block 0 also stores the scan to
// chunk_off_g.  With more heads the caller launches a single block and the
// scan lives in chunk_off_g (global memory) instead.
// ---------------------------------------------------------------------------
constexpr int PREP_HMAX = 4096;

struct PrepLDS {
  int32_t off[PREP_HMAX + 1];
  int32_t pg[PREP_HMAX + 1];
  int32_t len[PREP_HMAX];
};

// grow (LDS list only): count one more entry in every head with a free slot
// (an append that the lengths in memory do not show yet).
template <int NT>
__device__ int prep_chunks(const int32_t* __restrict__ page_off, const int32_t* __restrict__ len, int n_heads,
                           int cp, PrepLDS& L, int64_t* tmp, int32_t* __restrict__ chunk_off_g, bool grow = false) {
  const bool lds = n_heads <= PREP_HMAX;
  int64_t carry = 0;
  for (int base = 0; base < n_heads; base += NT) {
    const int h = base + threadIdx.x;
    int64_t n = 0;
    if (h < n_heads) {
      const int32_t a = page_off[h], b = page_off[h + 1];
      n = ((int64_t)b - a + cp - 1) / cp;
      if (lds) {
        L.pg[h] = a;
        const int32_t n0 = len[h];
        L.len[h] = n0 + ((grow && (int64_t)n0 < ((int64_t)b - a) * PAGE) ? 1 : 0);
        if (h == n_heads - 1) L.pg[n_heads] = b;
      }
    }
    int64_t tot;
    const int64_t ex = block_exclusive_scan<NT>(n, tmp, &tot);
    if (h < n_heads) {
      if (lds) L.off[h] = (int32_t)(carry + ex);
      if (!lds || blockIdx.x == 0) chunk_off_g[h] = (int32_t)(carry + ex);
    }
    carry += tot;
  }
  if (threadIdx.x == 0) {
    if (lds) L.off[n_heads] = (int32_t)carry;
    if (!lds || blockIdx.x == 0) chunk_off_g[n_heads] = (int32_t)carry;
  }
  __syncthreads();
  return (int)carry;
}

// Head, first chunk of the head, first CSR page, valid entries and pages of
// chunk c (after prep_chunks).
struct ChunkInfo {
  int h, c0, page0, nv, npg;
};

__device__ __forceinline__ ChunkInfo chunk_info(const PrepLDS& L, const int32_t* __restrict__ chunk_off_g,
                                                const int32_t* __restrict__ page_off,
                                                const int32_t* __restrict__ len, int n_heads, int cp, int c) {
  ChunkInfo r;
  if (n_heads <= PREP_HMAX) {
    r.h = upper_index(L.off, n_heads + 1, c);
    r.c0 = L.off[r.h];
    const int64_t e0 = (int64_t)(c - r.c0) * cp * PAGE;
    const int64_t v = (int64_t)L.len[r.h] - e0;
    r.nv = (int)(v < 0 ? 0 : (v > cp * PAGE ? cp * PAGE : v));
    r.page0 = L.pg[r.h] + (int)(e0 / PAGE);
    const int np = L.pg[r.h + 1] - r.page0;
    r.npg = np > cp ? cp : np;
  } else {
    r.h = upper_index(chunk_off_g, n_heads + 1, c);
    r.c0 = chunk_off_g[r.h];
    const int64_t e0 = (int64_t)(c - r.c0) * cp * PAGE;
    const int64_t v = (int64_t)len[r.h] - e0;
    r.nv = (int)(v < 0 ? 0 : (v > cp * PAGE ? cp * PAGE : v));
    r.page0 = page_off[r.h] + (int)(e0 / PAGE);
    const int np = page_off[r.h + 1] - r.page0;
    r.npg = np > cp ? cp : np;
  }
  return r;
}

inline int prep_grid(int n_heads, int64_t tmax, int per_block) {
  if (n_heads > PREP_HMAX) return 1;
  int64_t b = (tmax + per_block - 1) / per_block;
  return (int)(b < 1 ? 1 : (b > 128 ? 128 : b));
}

// bf16 bits -> fp32
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace trimkv
