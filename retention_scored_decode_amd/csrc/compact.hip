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
// Kernels: prep (chunk list of 64 pages), count (kept per chunk and per
// head; one wave per chunk), head scan (destination page table and the
// number of kept entries before each head), index (one wave per chunk: the
// (source slot, destination slot) pair of every kept entry, in kept order)
// and copy (a grid-stride row gather over the pair list: random 256-byte
// reads, contiguous writes).  Planning is kept out of the copy so that every
// wave of the copy issues its row loads after a single dependent load.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace trimkv {

namespace {

constexpr int CP = 64;          // pages per chunk: one keep byte per lane-slot, 16 per lane
constexpr int NT = 256;
constexpr int CPB = NT / WAVE;  // chunks per block of the count and index kernels

// chunk metadata: x = head, y = first chunk of the head, z = first CSR page,
// w = valid entries | (pages of the chunk << 16)
struct CmpWs {
  int32_t* chunk_off;   // [H + 1]
  int4* meta;           // [Tmax + CPB]
  int32_t* cnt;         // [Tmax] kept entries per chunk
  int32_t* head_kept;   // [H]
  int64_t* kept_before; // [H + 1] kept entries of the earlier heads; [H] = total
  uint2* pairs;         // [n_pages * 16] (source slot, destination slot) per kept entry
};

__global__ void __launch_bounds__(1024) k_cmp_prep(const int32_t* __restrict__ page_off,
                                                   const int32_t* __restrict__ len, int n_heads, CmpWs w) {
  __shared__ int64_t tmp[1024 / WAVE + 1];
  __shared__ PrepLDS L;
  for (int h = blockIdx.x * 1024 + threadIdx.x; h < n_heads; h += gridDim.x * 1024) w.head_kept[h] = 0;
  const int T = prep_chunks<1024>(page_off, len, n_heads, CP, L, tmp, w.chunk_off);
  for (int c = blockIdx.x * 1024 + threadIdx.x; c < T; c += gridDim.x * 1024) {
    const ChunkInfo ci = chunk_info(L, w.chunk_off, page_off, len, n_heads, CP, c);
    w.meta[c] = make_int4(ci.h, ci.c0, ci.page0, ci.nv | (ci.npg << 16));
  }
}

// Bit b (0..15) set iff keep byte b of this lane's 16 bytes is nonzero and
// the slot is valid.  Lane l of a chunk's wave covers page l of the chunk.
__device__ __forceinline__ uint32_t lane_keep_mask(const uint8_t* __restrict__ keep, int page0, int nv,
                                                   int lane) {
  const int nvb = min(max(nv - 16 * lane, 0), 16);
  if (nvb == 0) return 0u;
  const uint4 q = *reinterpret_cast<const uint4*>(keep + ((int64_t)page0 + lane) * PAGE);
  auto nz4 = [](uint32_t x) -> uint32_t {   // one bit per nonzero byte
    const uint32_t t = (((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
    return ((t >> 7) & 1u) | ((t >> 14) & 2u) | ((t >> 21) & 4u) | ((t >> 28) & 8u);
  };
  const uint32_t m = nz4(q.x) | (nz4(q.y) << 4) | (nz4(q.z) << 8) | (nz4(q.w) << 12);
  return m & ((1u << nvb) - 1u);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, WAVE);
  return v;
}

__global__ void __launch_bounds__(NT) k_cmp_count(int n_heads, const uint8_t* __restrict__ keep, CmpWs w) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int c = blockIdx.x * CPB + (threadIdx.x >> 6);
  const int T = w.chunk_off[n_heads];
  const int4 m = w.meta[c];   // padded: in bounds for every launched wave
  if (c >= T) return;
  const int n = wave_sum(__popc(lane_keep_mask(keep, m.z, m.w & 0xFFFF, lane)));
  if (lane == 0) {
    w.cnt[c] = n;
    if (n) atomicAdd(w.head_kept + m.x, n);
  }
}

__global__ void __launch_bounds__(1024) k_cmp_headscan(int n_heads, int reserve, CmpWs w,
                                                       int32_t* __restrict__ dst_off, int32_t* __restrict__ dst_len,
                                                       int64_t* __restrict__ pages_used) {
  __shared__ int64_t tmp[1024 / WAVE + 1];
  int64_t carry = 0, kcarry = 0;
  for (int base = 0; base < n_heads; base += 1024) {
    const int h = base + threadIdx.x;
    int64_t pages = 0, kh = 0;
    if (h < n_heads) {
      kh = w.head_kept[h];
      dst_len[h] = (int32_t)kh;
      pages = (kh + reserve + PAGE - 1) / PAGE;
    }
    int64_t tot, ktot;
    const int64_t ex = block_exclusive_scan<1024>(pages, tmp, &tot);
    const int64_t kex = block_exclusive_scan<1024>(kh, tmp, &ktot);
    if (h < n_heads) {
      dst_off[h] = (int32_t)(carry + ex);
      w.kept_before[h] = kcarry + kex;
    }
    carry += tot;
    kcarry += ktot;
  }
  if (threadIdx.x == 0) {
    dst_off[n_heads] = (int32_t)carry;
    w.kept_before[n_heads] = kcarry;
    pages_used[0] = carry;
  }
}

// One wave per chunk: the kept entries of the chunk in slot order get
// consecutive kept indices after those of the head's earlier chunks.
__global__ void __launch_bounds__(NT) k_cmp_index(int n_heads, const int32_t* __restrict__ page_ids,
                                                  const uint8_t* __restrict__ keep, CmpWs w,
                                                  const int32_t* __restrict__ dst_off, int64_t cap) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int c = blockIdx.x * CPB + (threadIdx.x >> 6);
  const int T = w.chunk_off[n_heads];
  const int4 m = w.meta[c];
  if (c >= T) return;
  const int h = m.x, nv = m.w & 0xFFFF, npg = m.w >> 16;
  int before = 0;
  for (int j = m.y + lane; j < c; j += WAVE) before += w.cnt[j];
  const int pid = lane < npg ? page_ids[m.z + lane] : 0;
  const uint32_t mask = lane_keep_mask(keep, m.z, nv, lane);
  before = wave_sum(before);
  // exclusive prefix of the per-lane counts
  const int cntl = __popc(mask);
  int inc = cntl;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int o = __shfl_up(inc, d, WAVE);
    if (lane >= d) inc += o;
  }
  const int64_t k0 = w.kept_before[h] + before + (inc - cntl);
  const uint32_t d0 = (uint32_t)dst_off[h] * PAGE + (uint32_t)(before + inc - cntl);
  uint32_t mm = mask;
  for (int r = 0; mm; ++r) {
    const int b = __ffs(mm) - 1;
    mm &= mm - 1;
    if (k0 + r < cap) w.pairs[k0 + r] = make_uint2((uint32_t)pid * PAGE + b, d0 + r);
  }
}

// Grid-stride copy of kept rows: LPR lanes of 16 bytes per row, UNR rows per
// lane group in flight.  Rows are read at random, written contiguously.
template <int ROWB>
__global__ void __launch_bounds__(NT) k_cmp_copy(int n_heads, const uint8_t* __restrict__ src_k,
                                                 const uint8_t* __restrict__ src_v,
                                                 const uint32_t* __restrict__ src_meta, CmpWs w,
                                                 const int32_t* __restrict__ dst_off, int32_t* __restrict__ dst_ids,
                                                 uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v,
                                                 uint32_t* __restrict__ dst_meta, int64_t dst_pages,
                                                 int64_t pair_cap) {
  constexpr int LPR = ROWB / 16;  // lanes per row
  constexpr int RPB = NT / LPR;   // rows per block pass
  constexpr int UNR = 4;
  // identity page ids of the destination pool (writes are bounded by the
  // destination capacity even if the caller's max_kept_total was wrong)
  const int64_t total_dst = min((int64_t)dst_off[n_heads], dst_pages);
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total_dst; i += (int64_t)gridDim.x * NT)
    dst_ids[i] = (int32_t)i;
  const int64_t total = min(w.kept_before[n_heads], pair_cap);
  if (total == 0) return;
  const int64_t dcap = dst_pages * PAGE;
  const int part = threadIdx.x % LPR;
  for (int64_t k0 = (int64_t)blockIdx.x * RPB * UNR + threadIdx.x / LPR; k0 < total;
       k0 += (int64_t)gridDim.x * RPB * UNR) {
    uint2 pr[UNR];
    uint4 kv[UNR], vv[UNR];
    uint32_t mv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) pr[u] = w.pairs[min(k0 + u * RPB, total - 1)];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t s = pr[u].x;
      kv[u] = *reinterpret_cast<const uint4*>(src_k + s * ROWB + part * 16);
      vv[u] = *reinterpret_cast<const uint4*>(src_v + s * ROWB + part * 16);
      // lanes 0 and 1 of a row carry its ln(beta) and position
      mv[u] = src_meta[(s / PAGE) * (2 * PAGE) + (part & 1) * PAGE + s % PAGE];
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t d = pr[u].y;
      if (k0 + u * RPB < total && d < dcap) {
        *reinterpret_cast<uint4*>(dst_k + d * ROWB + part * 16) = kv[u];
        *reinterpret_cast<uint4*>(dst_v + d * ROWB + part * 16) = vv[u];
        if (part < 2) dst_meta[(d / PAGE) * (2 * PAGE) + part * PAGE + d % PAGE] = mv[u];
      }
    }
  }
}

CmpWs carve(const trimkv_cache_t* c, void* ws) {
  WsLayout L = compact_ws_layout(c);
  char* b = (char*)ws;
  return CmpWs{(int32_t*)(b + L.off[0]), (int4*)(b + L.off[1]), (int32_t*)(b + L.off[2]),
               (int32_t*)(b + L.off[3]), (int64_t*)(b + L.off[4]), (uint2*)(b + L.off[5])};
}

}  // namespace

WsLayout compact_ws_layout(const trimkv_cache_t* c) {
  const int64_t T = max_chunks(c, CP);
  WsLayout L;
  L.add(((int64_t)c->n_heads + 1) * 4);
  L.add((T + CPB) * 16);
  L.add(T * 4);
  L.add((int64_t)c->n_heads * 4);
  L.add(((int64_t)c->n_heads + 1) * 8);
  L.add(c->n_pages * PAGE * 8);
  return L;
}

int launch_compact(const trimkv_cache_t* src, const uint8_t* keep, int reserve, int64_t max_kept_total,
                   trimkv_cache_t* dst, int64_t* pages_used, void* ws, hipStream_t st) {
  CmpWs w = carve(src, ws);
  const int64_t T = max_chunks(src, CP);
  const int H = src->n_heads;
  const unsigned cgrid = (unsigned)((T + CPB - 1) / CPB);
  hipLaunchKernelGGL(k_cmp_prep, dim3(prep_grid(H, T, 1024)), dim3(1024), 0, st, src->page_off, src->len, H, w);
  hipLaunchKernelGGL(k_cmp_count, dim3(cgrid), dim3(NT), 0, st, H, keep, w);
  hipLaunchKernelGGL(k_cmp_headscan, dim3(1), dim3(1024), 0, st, H, reserve, w, dst->page_off, dst->len,
                     pages_used);
  hipLaunchKernelGGL(k_cmp_index, dim3(cgrid), dim3(NT), 0, st, H, src->page_ids, keep, w, dst->page_off,
                     src->n_pages * PAGE);
  const int elt = src->dtype == TRIMKV_BF16 ? 2 : 4;
  const int rowb = src->head_dim * elt;
  // enough blocks for every destination page id and every row of the bound
  const int64_t rows_per_block = (int64_t)(NT / (rowb / 16)) * 4;
  const int64_t want = std::max((max_kept_total + rows_per_block - 1) / rows_per_block,
                                (dst->n_pages + NT - 1) / NT);
  const unsigned grid = (unsigned)std::min<int64_t>(std::max<int64_t>(want, 1), 8192);
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
