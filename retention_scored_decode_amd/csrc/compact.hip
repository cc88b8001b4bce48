// Physical eviction: stable, out-of-place compaction of the kept entries
// into a fresh pool, with a prefix-sum page table.
//
// DBTrimKV page, Method 4: per-head variable-length KV in a paged layout.
// ContourKV page, section 2: a budget that only masks the full cache
// overstates compression; storage itself must shrink (ragged storage).
//
// Head h receives ceil((kept_h + reserve) / 16) destination pages numbered
// by a prefix sum over heads; kept rows keep their slot order, so positions
// stay ascending within every head.
//
// Kernels: count (one block per head: kept entries of the head), index (one
// block per head: the kept entries of all earlier heads and their destination
// pages by a strided reduction over the head counts, then the (source slot,
// destination slot) pair of every kept entry in kept order, staged through LDS
// so that the pair list is written with coalesced stores) and copy (a
// grid-stride row gather over the pair list: random 256-byte reads,
// contiguous writes).  Planning is kept out of the copy so that every wave of
// the copy issues its row loads after a single dependent load.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "tailfill.h"

namespace trimkv {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;     // copy kernel
constexpr int NTP = 1024;   // planning kernels: one block per head, one page per thread and tile
constexpr int NWP = NTP / WAVE;

struct CmpWs {
  int32_t* head_kept;   // [H] kept entries per head (the caller's counts when given)
  int64_t* total;       // [1] kept entries over all heads
  uint2* pairs;         // [n_pages * 16] (source slot, destination slot) per kept entry
};

// Bit b (0..15) set iff keep byte b of page p of a head is nonzero and the
// slot is valid (below nv, the head's valid entries).
__device__ __forceinline__ uint32_t page_keep_mask(const uint8_t* __restrict__ keep, int page0, int nv, int p) {
  const int nvb = min(max(nv - PAGE * p, 0), PAGE);
  if (nvb == 0) return 0u;
  const uint4 q = *reinterpret_cast<const uint4*>(keep + ((int64_t)page0 + p) * PAGE);
  auto nz4 = [](uint32_t x) -> uint32_t {   // one bit per nonzero byte
    const uint32_t t = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
    return ((t >> 7) & 1u) | ((t >> 14) & 2u) | ((t >> 21) & 4u) | ((t >> 28) & 8u);
  };
  const uint32_t m = nz4(q.x) | (nz4(q.y) << 4) | (nz4(q.z) << 8) | (nz4(q.w) << 12);
  return m & ((1u << nvb) - 1u);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, WAVE);
  return v;
}

// Valid entries of a head: its length, bounded by the slots of its pages.
__device__ __forceinline__ int head_valid(const int32_t* __restrict__ page_off, const int32_t* __restrict__ len,
                                          int h, int* p0) {
  *p0 = page_off[h];
  const int64_t slots = ((int64_t)page_off[h + 1] - *p0) * PAGE;
  return (int)min((int64_t)max(len[h], 0), slots);
}

__global__ void __launch_bounds__(NTP) k_cmp_count(const int32_t* __restrict__ page_off,
                                                   const int32_t* __restrict__ len,
                                                   const uint8_t* __restrict__ keep, CmpWs w) {
  __shared__ int part[NWP];
  const int h = blockIdx.x;
  int p0;
  const int nv = head_valid(page_off, len, h, &p0);
  const int np = (nv + PAGE - 1) / PAGE;
  int n = 0;
  // four pages per thread in flight
  for (int p = threadIdx.x; p < np; p += 4 * NTP) {
    uint32_t m[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) m[u] = page_keep_mask(keep, p0, nv, p + u * NTP);
#pragma unroll
    for (int u = 0; u < 4; ++u) n += __popc(m[u]);
  }
  n = wave_sum(n);
  if ((threadIdx.x & (WAVE - 1)) == 0) part[threadIdx.x / WAVE] = n;
  lds_barrier();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < NWP; ++i) t += part[i];
    w.head_kept[h] = t;
  }
}

// Destination layout: head h owns ceil((kept_h + reserve) / 16) pages,
// numbered by a prefix sum over heads; its kept entries fill them in kept
// order.  Every block recomputes the prefix of its own head from the head
// counts (a strided reduction: O(H / 1024) loads per thread).
__global__ void __launch_bounds__(NTP) k_cmp_index(int n_heads, int reserve, const int32_t* __restrict__ page_off,
                                                   const int32_t* __restrict__ len,
                                                   const int32_t* __restrict__ page_ids,
                                                   const uint8_t* __restrict__ keep, CmpWs w,
                                                   int32_t* __restrict__ dst_off, int32_t* __restrict__ dst_len,
                                                   int64_t* __restrict__ pages_used, int64_t cap) {
  __shared__ uint32_t stage[NWP][WAVE * PAGE];   // source slots of each wave's kept entries
  __shared__ int64_t red[2][NWP];
  __shared__ int wtot[NWP];
  const int h = blockIdx.x;
  const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
  int p0;
  const int nv = head_valid(page_off, len, h, &p0);
  const int np = (nv + PAGE - 1) / PAGE;
  // first tile's keep bits and page ids, in flight during the head prefix
  uint32_t mask = page_keep_mask(keep, p0, nv, threadIdx.x);
  int pid = (int)threadIdx.x < np ? page_ids[p0 + threadIdx.x] : 0;
  int64_t kb = 0, pb = 0;
  for (int j = threadIdx.x; j < h; j += NTP) {
    const int64_t kj = w.head_kept[j];
    kb += kj;
    pb += (kj + reserve + PAGE - 1) / PAGE;
  }
  kb = wave_sum(kb);
  pb = wave_sum(pb);
  if (lane == 0) {
    red[0][wid] = kb;
    red[1][wid] = pb;
  }
  lds_barrier();
  kb = 0;
  pb = 0;
#pragma unroll
  for (int i = 0; i < NWP; ++i) {
    kb += red[0][i];
    pb += red[1][i];
  }
  const int kh = w.head_kept[h];
  if (threadIdx.x == 0) {
    dst_off[h] = (int32_t)pb;
    dst_len[h] = kh;
    if (h == n_heads - 1) {
      const int64_t pend = pb + ((int64_t)kh + reserve + PAGE - 1) / PAGE;
      dst_off[n_heads] = (int32_t)pend;
      pages_used[0] = pend;
      w.total[0] = kb + kh;
    }
  }
  const uint32_t d_base = (uint32_t)pb * PAGE;
  int carry = 0;   // kept entries of the head's earlier tiles
  for (int t0 = 0; t0 < np; t0 += NTP) {
    // next tile's loads ahead of this tile's scan
    const int pn = t0 + NTP + (int)threadIdx.x;
    const uint32_t mask_n = page_keep_mask(keep, p0, nv, pn);
    const int pid_n = pn < np ? page_ids[p0 + pn] : 0;
    const int cnt = __popc(mask);
    int inc = cnt;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
      const int o = __shfl_up(inc, d, WAVE);
      if (lane >= d) inc += o;
    }
    const int wt = __shfl(inc, WAVE - 1, WAVE);
    uint32_t mm = mask;
    for (int r = inc - cnt; mm; ++r) {
      const int b = __ffs(mm) - 1;
      mm &= mm - 1;
      stage[wid][r] = (uint32_t)pid * PAGE + b;
    }
    if (lane == 0) wtot[wid] = wt;
    lds_barrier();
    int wex = 0, ttot = 0;
#pragma unroll
    for (int i = 0; i < NWP; ++i) {
      const int x = wtot[i];
      wex += i < wid ? x : 0;
      ttot += x;
    }
    const int o = carry + wex;   // ordinal within the head of the wave's first entry
    for (int j = lane; j < wt; j += WAVE) {
      const int64_t k = kb + o + j;
      if (k >= 0 && k < cap) w.pairs[k] = make_uint2(stage[wid][j], d_base + (uint32_t)(o + j));
    }
    carry += ttot;
    mask = mask_n;
    pid = pid_n;
    lds_barrier();   // stage and wtot are rewritten by the next tile
  }
  // a caller's count above the head's nonzero keep bytes: the pairs this
  // head owns but did not fill become no-ops for the copy (source slot out
  // of range), not stale words of an earlier call
  for (int64_t j = (int64_t)carry + threadIdx.x; j < kh; j += NTP) {
    const int64_t k = kb + j;
    if (k >= 0 && k < cap) w.pairs[k] = make_uint2(~0u, ~0u);
  }
}

// Grid-stride copy of kept rows: LPR lanes of 16 bytes per row, UNR rows per
// lane group in flight.  Rows are read at random, written contiguously.  A
// pair whose source slot lies outside the source pool (left by counts that
// disagree with the keep plane) copies nothing.  K
// and V rows are loaded and stored non-temporally: each is touched once, and
// the compacted pool is read next by decode attention, where write-back lines
// left in the caches would otherwise be evicted during that read, competing
// with it for HBM.
template <int ROWB>
__global__ void __launch_bounds__(NT) k_cmp_copy(int n_heads, const uint8_t* __restrict__ src_k,
                                                 const uint8_t* __restrict__ src_v,
                                                 const uint32_t* __restrict__ src_meta, CmpWs w,
                                                 const int32_t* __restrict__ dst_off, int32_t* __restrict__ dst_ids,
                                                 uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v,
                                                 uint32_t* __restrict__ dst_meta, int64_t dst_pages,
                                                 int64_t src_slots) {
  constexpr int LPR = ROWB / 16;  // lanes per row
  constexpr int RPB = NT / LPR;   // rows per block pass
  constexpr int UNR = 4;
  // identity page ids of the destination pool (writes are bounded by the
  // destination capacity even if the caller's max_kept_total was wrong)
  const int64_t total_dst = min((int64_t)dst_off[n_heads], dst_pages);
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total_dst; i += (int64_t)gridDim.x * NT)
    dst_ids[i] = (int32_t)i;
  const int64_t total = min(w.total[0], src_slots);   // the pair list holds at most src_slots pairs
  if (total == 0) return;
  const int64_t dcap = dst_pages * PAGE;
  const int part = threadIdx.x % LPR;
  for (int64_t k0 = (int64_t)blockIdx.x * RPB * UNR + threadIdx.x / LPR; k0 < total;
       k0 += (int64_t)gridDim.x * RPB * UNR) {
    uint2 pr[UNR];
    u32x4 kv[UNR], vv[UNR];
    uint32_t mv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) pr[u] = w.pairs[min(k0 + u * RPB, total - 1)];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t s = (int64_t)pr[u].x < src_slots ? (int64_t)pr[u].x : 0;
      kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src_k + s * ROWB + part * 16));
      vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src_v + s * ROWB + part * 16));
      // lanes 0 and 1 of a row carry its ln(beta) and position
      mv[u] = src_meta[(s / PAGE) * (2 * PAGE) + (part & 1) * PAGE + s % PAGE];
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t d = pr[u].y;
      if (k0 + u * RPB < total && d < dcap && (int64_t)pr[u].x < src_slots) {
        __builtin_nontemporal_store(kv[u], reinterpret_cast<u32x4*>(dst_k + d * ROWB + part * 16));
        __builtin_nontemporal_store(vv[u], reinterpret_cast<u32x4*>(dst_v + d * ROWB + part * 16));
        if (part < 2) dst_meta[(d / PAGE) * (2 * PAGE) + part * PAGE + d % PAGE] = mv[u];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Incremental eviction in place: every head keeps its kept entries, in slot
// order, in the first slots of its own pages, and its page list becomes the
// first min(ceil((kept + reserve) / 16), home pages) pages of its home list
// (the head's own allocation, of which the current list is a prefix).  Only
// entries after the head's first dropped entry move, each to an earlier
// slot, so a streaming step that drops a few entries per head moves a
// suffix of each head instead of rewriting the cache into a second pool.
//
// One block per head walks the head in windows of NTP slots: a block scan of
// the keep flags gives every kept entry its destination slot, and the
// window's moves run in passes whose rows are all read before any is
// written.  A destination never lies after its source and sources increase
// from pass to pass, so no pass overwrites a row a later pass still reads,
// and only this pass's reads can be overwritten by this pass's writes.
template <int ROWB>
__global__ void __launch_bounds__(NTP) k_cmp_shift(int n_heads, int reserve, const int32_t* __restrict__ page_off,
                                                   const int32_t* __restrict__ page_ids, int32_t* __restrict__ len,
                                                   const uint8_t* __restrict__ keep,
                                                   const int32_t* __restrict__ head_kept,
                                                   const int32_t* __restrict__ home_off,
                                                   const int32_t* __restrict__ home_ids,
                                                   int32_t* __restrict__ new_off, int32_t* __restrict__ new_ids,
                                                   uint8_t* __restrict__ pk, uint8_t* __restrict__ pv,
                                                   uint32_t* __restrict__ meta) {
  constexpr int LPR = ROWB / 16;          // lanes per row
  constexpr int GROUPS = NTP / LPR;       // row groups per block
  constexpr int UNR = 4;                  // rows per group in flight
  constexpr int PASS = GROUPS * UNR;      // rows per pass
  __shared__ uint32_t s_src[NTP], s_dst[NTP];
  __shared__ int64_t red[NWP + 1];
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;
  auto pages_of = [&](int j) -> int64_t {
    const int64_t want = ((int64_t)max(head_kept[j], 0) + reserve + PAGE - 1) / PAGE;
    return min(want, (int64_t)home_off[j + 1] - home_off[j]);
  };
  // the new page list: a prefix sum over the earlier heads, then the head's home prefix
  int64_t pb = 0;
  for (int j = tid; j < h; j += NTP) pb += pages_of(j);
  pb = wave_sum(pb);
  if (lane == 0) red[wid] = pb;
  lds_barrier();
  pb = 0;
#pragma unroll
  for (int i = 0; i < NWP; ++i) pb += red[i];
  const int64_t nh = pages_of(h);
  const int64_t hb = home_off[h];
  for (int64_t c = tid; c < nh; c += NTP) new_ids[pb + c] = home_ids[hb + c];
  if (tid == 0) {
    new_off[h] = (int32_t)pb;
    if (h == n_heads - 1) new_off[n_heads] = (int32_t)(pb + nh);
  }
  lds_barrier();   // red is the scan's scratch below

  int p0;
  const int nv = head_valid(page_off, len, h, &p0);
  const int part = tid % LPR, grp = tid / LPR;
  int carry = 0;   // kept entries before the window
  for (int s0 = 0; s0 < nv; s0 += NTP) {
    const int i = s0 + tid;
    int kf = 0;
    uint32_t src = 0;
    if (i < nv) {
      kf = keep[((int64_t)p0 + i / PAGE) * PAGE + i % PAGE] != 0;
      src = (uint32_t)page_ids[p0 + i / PAGE] * PAGE + i % PAGE;
    }
    int64_t tot64;
    const int rank = (int)block_exclusive_scan<NTP>(kf, red, &tot64);
    const int tot = (int)tot64;
    if (carry == s0 && tot == min(NTP, nv - s0)) {   // nothing dropped yet: every entry stays
      carry += tot;
      continue;
    }
    if (kf) {
      const int j = carry + rank;
      s_src[rank] = src;
      s_dst[rank] = (uint32_t)page_ids[p0 + j / PAGE] * PAGE + j % PAGE;
    }
    lds_barrier();
    for (int r0 = 0; r0 < tot; r0 += PASS) {
      u32x4 kv[UNR], vv[UNR];
      uint32_t mv[UNR], dsl[UNR];
      bool mov[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int r = r0 + grp + u * GROUPS;
        const uint32_t s = r < tot ? s_src[r] : 0u;
        dsl[u] = r < tot ? s_dst[r] : 0u;
        mov[u] = r < tot && s != dsl[u];
        if (mov[u]) {
          kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pk + (int64_t)s * ROWB + part * 16));
          vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pv + (int64_t)s * ROWB + part * 16));
          mv[u] = meta[(int64_t)(s / PAGE) * (2 * PAGE) + (part & 1) * PAGE + s % PAGE];
        }
      }
      // every row of the pass is in registers before any thread overwrites one
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (mov[u]) {
          const int64_t d = dsl[u];
          __builtin_nontemporal_store(kv[u], reinterpret_cast<u32x4*>(pk + d * ROWB + part * 16));
          __builtin_nontemporal_store(vv[u], reinterpret_cast<u32x4*>(pv + d * ROWB + part * 16));
          if (part < 2) meta[(d / PAGE) * (2 * PAGE) + part * PAGE + d % PAGE] = mv[u];
        }
      }
    }
    carry += tot;
    lds_barrier();   // s_src and s_dst are rewritten by the next window
  }
  if (tid == 0) len[h] = (int32_t)min((int64_t)carry, nh * PAGE);
}

// In-place eviction by tail fill: one block per head (tailfill.h).
template <int ROWB>
__global__ void __launch_bounds__(tf::NT) k_cmp_tailfill(tf::Args a) {
  __shared__ tf::LDS L;
  tf::evict_head<ROWB>(blockIdx.x, a, L);
}

CmpWs carve(const trimkv_cache_t* c, void* ws) {
  WsLayout L = compact_ws_layout(c);
  char* b = (char*)ws;
  return CmpWs{(int32_t*)(b + L.off[0]), (int64_t*)(b + L.off[1]), (uint2*)(b + L.off[2])};
}

}  // namespace

WsLayout tailfill_ws_layout(const trimkv_cache_t* c) {
  WsLayout L;
  L.add((int64_t)c->n_heads * 4);        // kept counts when the caller gives none
  L.add(c->n_pages * PAGE * 4);          // hole lists (a slot per CSR slot)
  return L;
}

WsLayout compact_ws_layout(const trimkv_cache_t* c) {
  WsLayout L;
  L.add((int64_t)c->n_heads * 4);
  L.add(8);
  L.add(c->n_pages * PAGE * 8);
  return L;
}

int launch_compact_inplace(trimkv_cache_t* c, const uint8_t* keep, const int32_t* kept, int reserve,
                           const int32_t* home_off, const int32_t* home_ids, int32_t* new_off, int32_t* new_ids,
                           void* ws, hipStream_t st) {
  const int H = c->n_heads;
  CmpWs w{};
  if (kept) {
    w.head_kept = const_cast<int32_t*>(kept);
  } else {
    w.head_kept = (int32_t*)ws;
    hipLaunchKernelGGL(k_cmp_count, dim3(H), dim3(NTP), 0, st, c->page_off, c->len, keep, w);
  }
  const int elt = c->dtype == TRIMKV_BF16 ? 2 : 4;
#define TRIMKV_SHIFT(RB)                                                                                        \
  hipLaunchKernelGGL(k_cmp_shift<RB>, dim3(H), dim3(NTP), 0, st, H, reserve, c->page_off, c->page_ids, c->len, \
                     keep, w.head_kept, home_off, home_ids, new_off, new_ids, (uint8_t*)c->k, (uint8_t*)c->v,   \
                     c->meta)
  prof_begin(st);
  switch (c->head_dim * elt) {
    case 128: TRIMKV_SHIFT(128); break;
    case 256: TRIMKV_SHIFT(256); break;
    case 512: TRIMKV_SHIFT(512); break;
    default: return TRIMKV_EUNSUPPORTED;
  }
  prof_end(st);
#undef TRIMKV_SHIFT
  return check_launch();
}

int launch_evict_tailfill(trimkv_cache_t* c, const uint8_t* keep, const int32_t* kept, int reserve,
                          const int32_t* home_off, const int32_t* home_ids, int32_t* new_off, int32_t* new_ids,
                          void* ws, hipStream_t st) {
  const int H = c->n_heads;
  WsLayout L = tailfill_ws_layout(c);
  char* b = (char*)ws;
  CmpWs w{};
  uint32_t* holes = (uint32_t*)(b + L.off[1]);
  if (kept) {
    w.head_kept = const_cast<int32_t*>(kept);
  } else {
    w.head_kept = (int32_t*)(b + L.off[0]);
    hipLaunchKernelGGL(k_cmp_count, dim3(H), dim3(NTP), 0, st, c->page_off, c->len, keep, w);
  }
  const int elt = c->dtype == TRIMKV_BF16 ? 2 : 4;
  const tf::Args ta{H, reserve, c->page_off, c->page_ids, c->len, keep, w.head_kept, home_off, home_ids, new_off,
                    new_ids, (uint8_t*)c->k, (uint8_t*)c->v, c->meta, holes};
#define TRIMKV_TAILFILL(RB) hipLaunchKernelGGL(k_cmp_tailfill<RB>, dim3(H), dim3(tf::NT), 0, st, ta)
  prof_begin(st);
  switch (c->head_dim * elt) {
    case 128: TRIMKV_TAILFILL(128); break;
    case 256: TRIMKV_TAILFILL(256); break;
    case 512: TRIMKV_TAILFILL(512); break;
    default: return TRIMKV_EUNSUPPORTED;
  }
  prof_end(st);
#undef TRIMKV_TAILFILL
  return check_launch();
}

int launch_compact(const trimkv_cache_t* src, const uint8_t* keep, const int32_t* kept, int reserve,
                   int64_t max_kept_total, trimkv_cache_t* dst, int64_t* pages_used, void* ws, hipStream_t st) {
  CmpWs w = carve(src, ws);
  const int H = src->n_heads;
  if (kept) w.head_kept = const_cast<int32_t*>(kept);   // only read from here on
  else hipLaunchKernelGGL(k_cmp_count, dim3(H), dim3(NTP), 0, st, src->page_off, src->len, keep, w);
  hipLaunchKernelGGL(k_cmp_index, dim3(H), dim3(NTP), 0, st, H, reserve, src->page_off, src->len, src->page_ids,
                     keep, w, dst->page_off, dst->len, pages_used, src->n_pages * PAGE);
  const int elt = src->dtype == TRIMKV_BF16 ? 2 : 4;
  const int rowb = src->head_dim * elt;
  // enough blocks for every destination page id and every row of the bound
  const int64_t rows_per_block = (int64_t)(NT / (rowb / 16)) * 4;
  const int64_t want = std::max((max_kept_total + rows_per_block - 1) / rows_per_block,
                                (dst->n_pages + NT - 1) / NT);
  const unsigned grid = (unsigned)std::min<int64_t>(std::max<int64_t>(want, 1), 65536);
#define TRIMKV_COPY(RB)                                                                                      \
  hipLaunchKernelGGL(k_cmp_copy<RB>, dim3(grid), dim3(NT), 0, st, H, (const uint8_t*)src->k,                 \
                     (const uint8_t*)src->v, src->meta, w, dst->page_off, dst->page_ids, (uint8_t*)dst->k,    \
                     (uint8_t*)dst->v, dst->meta, dst->n_pages, src->n_pages * PAGE)
  prof_begin(st);
  switch (rowb) {
    case 128: TRIMKV_COPY(128); break;
    case 256: TRIMKV_COPY(256); break;
    case 512: TRIMKV_COPY(512); break;
    default: return TRIMKV_EUNSUPPORTED;
  }
  prof_end(st);
#undef TRIMKV_COPY
  return check_launch();
}

}  // namespace trimkv
