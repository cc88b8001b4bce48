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
// Kernels: prep (chunk list), count (kept per chunk and per head), head scan
// (destination page table), scatter (row copies; a chunk's offset within its
// head is the sum of the counts of the head's earlier chunks).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace trimkv {

namespace {

constexpr int CP = 64;
constexpr int CS = CP * PAGE;
constexpr int NT = 256;

// chunk metadata: x = head, y = first chunk of the head, z = first CSR page,
// w = valid entries | (pages of the chunk << 16)
struct CmpWs {
  int32_t* chunk_off;   // [H + 1]
  int4* meta;           // [Tmax]
  int32_t* cnt;         // [Tmax] kept entries per chunk
  int32_t* head_kept;   // [H]
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

__device__ __forceinline__ uint32_t keep_bits(const uint8_t* keep, int64_t csr0, int i0, int nv) {
  if (i0 >= nv) return 0u;
  const uint32_t word = *reinterpret_cast<const uint32_t*>(keep + csr0 + i0);
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (i0 + k < nv && ((word >> (8 * k)) & 0xFFu)) m |= 1u << k;
  return m;
}

__global__ void __launch_bounds__(NT) k_cmp_count(int n_heads, const uint8_t* __restrict__ keep, CmpWs w) {
  __shared__ int64_t tmp[NT / WAVE + 1];
  const int c = blockIdx.x;
  if (c >= w.chunk_off[n_heads]) return;
  const int4 m = w.meta[c];
  const uint32_t bits = keep_bits(keep, (int64_t)m.z * PAGE, threadIdx.x * 4, m.w & 0xFFFF);
  int64_t tot;
  block_exclusive_scan<NT>((int64_t)__popc(bits), tmp, &tot);
  if (threadIdx.x == 0) {
    w.cnt[c] = (int32_t)tot;
    if (tot) atomicAdd(w.head_kept + m.x, (int32_t)tot);
  }
}

__global__ void __launch_bounds__(1024) k_cmp_headscan(int n_heads, int reserve, CmpWs w,
                                                       int32_t* __restrict__ dst_off, int32_t* __restrict__ dst_len,
                                                       int64_t* __restrict__ pages_used) {
  __shared__ int64_t tmp[1024 / WAVE + 1];
  int64_t carry = 0;
  for (int base = 0; base < n_heads; base += 1024) {
    const int h = base + threadIdx.x;
    int64_t pages = 0;
    if (h < n_heads) {
      const int64_t kh = w.head_kept[h];
      dst_len[h] = (int32_t)kh;
      pages = (kh + reserve + PAGE - 1) / PAGE;
    }
    int64_t tot;
    const int64_t ex = block_exclusive_scan<1024>(pages, tmp, &tot);
    if (h < n_heads) dst_off[h] = (int32_t)(carry + ex);
    carry += tot;
  }
  if (threadIdx.x == 0) {
    dst_off[n_heads] = (int32_t)carry;
    pages_used[0] = carry;
  }
}

template <int ROWB>
__global__ void __launch_bounds__(NT) k_cmp_scatter(int n_heads, const int32_t* __restrict__ page_ids,
                                                    const uint8_t* __restrict__ src_k,
                                                    const uint8_t* __restrict__ src_v,
                                                    const uint32_t* __restrict__ src_meta,
                                                    const uint8_t* __restrict__ keep, CmpWs w,
                                                    const int32_t* __restrict__ dst_off,
                                                    int32_t* __restrict__ dst_ids, uint8_t* __restrict__ dst_k,
                                                    uint8_t* __restrict__ dst_v, uint32_t* __restrict__ dst_meta,
                                                    int64_t dst_pages) {
  constexpr int LPR = ROWB / 16;  // lanes per row (16 B each)
  constexpr int RPI = NT / LPR;   // rows per iteration
  constexpr int UNR = 4;          // row iterations whose loads are issued together
  __shared__ int64_t tmp[NT / WAVE + 1];
  __shared__ int64_t src_slot[CS];
  __shared__ int32_t pids[CP];
  // identity page ids of the destination pool (writes are bounded by the
  // destination capacity even if the caller's max_kept_total was wrong)
  const int64_t total_dst = min((int64_t)dst_off[n_heads], dst_pages);
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < total_dst; i += (int64_t)gridDim.x * NT)
    dst_ids[i] = (int32_t)i;
  const int c = blockIdx.x;
  if (c >= w.chunk_off[n_heads]) return;
  if (w.cnt[c] == 0) return;
  const int4 m = w.meta[c];
  const int h = m.x, nv = m.w & 0xFFFF;
  const int64_t csr0 = (int64_t)m.z * PAGE;
  // kept entries of the head's earlier chunks
  int64_t before = 0;
  for (int j = m.y + threadIdx.x; j < c; j += NT) before += w.cnt[j];
  const int npg = (nv + PAGE - 1) / PAGE;
  if (threadIdx.x < npg) pids[threadIdx.x] = page_ids[m.z + threadIdx.x];
  int64_t tb;
  block_exclusive_scan<NT>(before, tmp, &tb);
  const int i0 = threadIdx.x * 4;
  const uint32_t bits = keep_bits(keep, csr0, i0, nv);
  int64_t nk;
  int64_t r = block_exclusive_scan<NT>((int64_t)__popc(bits), tmp, &nk);  // syncs: pids visible
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (bits & (1u << k)) {
      const int i = i0 + k;
      src_slot[r++] = (int64_t)pids[i / PAGE] * PAGE + (i % PAGE);
    }
  }
  __syncthreads();
  const int64_t dbase = (int64_t)dst_off[h] * PAGE + tb;
  const int64_t dcap = dst_pages * PAGE;
  const int part = threadIdx.x % LPR;
  for (int row0 = threadIdx.x / LPR; row0 < nk; row0 += RPI * UNR) {
    uint4 kv[UNR], vv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      // rows past the end re-read the last kept row (not stored)
      const int row = min(row0 + u * RPI, (int)nk - 1);
      const int64_t s = src_slot[row];
      kv[u] = *reinterpret_cast<const uint4*>(src_k + s * ROWB + part * 16);
      vv[u] = *reinterpret_cast<const uint4*>(src_v + s * ROWB + part * 16);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int row = row0 + u * RPI;
      const int64_t d = dbase + row;
      if (row < nk && d < dcap) {
        *reinterpret_cast<uint4*>(dst_k + d * ROWB + part * 16) = kv[u];
        *reinterpret_cast<uint4*>(dst_v + d * ROWB + part * 16) = vv[u];
      }
    }
  }
  // ln beta and position of the kept rows (one 128-byte metadata block per page)
  for (int row = threadIdx.x; row < nk; row += NT) {
    const int64_t d = dbase + row;
    if (d < dcap) {
      const int64_t s = src_slot[row];
      const uint32_t* sm = src_meta + (s / PAGE) * (2 * PAGE) + s % PAGE;
      uint32_t* dm = dst_meta + (d / PAGE) * (2 * PAGE) + d % PAGE;
      dm[0] = sm[0];
      dm[PAGE] = sm[PAGE];
    }
  }
}

CmpWs carve(const trimkv_cache_t* c, void* ws) {
  WsLayout L = compact_ws_layout(c);
  char* b = (char*)ws;
  return CmpWs{(int32_t*)(b + L.off[0]), (int4*)(b + L.off[1]), (int32_t*)(b + L.off[2]),
               (int32_t*)(b + L.off[3])};
}

}  // namespace

WsLayout compact_ws_layout(const trimkv_cache_t* c) {
  const int64_t T = max_chunks(c, CP);
  WsLayout L;
  L.add(((int64_t)c->n_heads + 1) * 4);
  L.add(T * 16);
  L.add(T * 4);
  L.add((int64_t)c->n_heads * 4);
  return L;
}

int launch_compact(const trimkv_cache_t* src, const uint8_t* keep, int reserve, trimkv_cache_t* dst,
                   int64_t* pages_used, void* ws, hipStream_t st) {
  CmpWs w = carve(src, ws);
  const int64_t T = max_chunks(src, CP);
  const int H = src->n_heads;
  hipLaunchKernelGGL(k_cmp_prep, dim3(prep_grid(H, T, 1024)), dim3(1024), 0, st, src->page_off, src->len, H, w);
  hipLaunchKernelGGL(k_cmp_count, dim3((unsigned)T), dim3(NT), 0, st, H, keep, w);
  hipLaunchKernelGGL(k_cmp_headscan, dim3(1), dim3(1024), 0, st, H, reserve, w, dst->page_off, dst->len,
                     pages_used);
  const int elt = src->dtype == TRIMKV_BF16 ? 2 : 4;
  const int rowb = src->head_dim * elt;
#define TRIMKV_SCATTER(RB)                                                                                   \
  hipLaunchKernelGGL(k_cmp_scatter<RB>, dim3((unsigned)T), dim3(NT), 0, st, H, src->page_ids,                \
                     (const uint8_t*)src->k, (const uint8_t*)src->v, src->meta, keep, w, dst->page_off,           \
                     dst->page_ids, (uint8_t*)dst->k, (uint8_t*)dst->v, dst->meta, dst->n_pages)
  switch (rowb) {
    case 128: TRIMKV_SCATTER(128); break;
    case 256: TRIMKV_SCATTER(256); break;
    case 512: TRIMKV_SCATTER(512); break;
    default: return TRIMKV_EUNSUPPORTED;
  }
#undef TRIMKV_SCATTER
  return check_launch();
}

}  // namespace trimkv
