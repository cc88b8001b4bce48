// In-place eviction of one head by tail fill, as a block-level routine, so
// that the eviction kernel and the kernel that runs it beside the attention
// merge share one body.
//
// DBTrimKV page, Method 4 (paged per-head variable-length KV); ContourKV
// page, section 2 (storage itself must shrink), for the streaming loop.
//
// Head h keeps its kept entries in the first slots of its own (home) pages:
// the j-th dropped slot below the new length kept_h (a hole, in slot order)
// takes the j-th kept entry at or above kept_h (a mover, in slot order), and
// every other entry stays where it is.  Only as many rows move as there are
// holes, at most the head's drops.  Holes lie below kept_h and movers at or
// above it, so no move reads a row that another move writes.  Slot order
// then no longer follows position order (selection ranks ties by position,
// so it is unaffected; attention is order-free).
//
// One block of NT threads per head: a first walk over the head's first
// kept_h slots ranks its holes (block scan per window of 4 NT slots, 4 per
// thread) and lists their physical slots in the workspace at the head's CSR
// offset; a second walk over the rest ranks the movers, and mover r moves to
// hole r (LPR lanes of 16 bytes per row).  Counts that disagree with the
// keep plane move only min(holes, movers) rows.  The new page table is the
// head's home-list prefix after a prefix sum of the earlier heads' pages.
#pragma once
#include "common.h"

namespace trimkv {
namespace tf {

constexpr int NT = 1024;   // threads per block (one block per head)
constexpr int NW = NT / WAVE;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Args {
  int n_heads;
  int reserve;
  const int32_t* page_off;   // the current table
  const int32_t* page_ids;
  int32_t* len;              // in: current lengths; out: the new lengths
  const uint8_t* keep;       // CSR keep plane of the current table
  const int32_t* head_kept;  // kept entries per head
  const int32_t* home_off;   // each head's home page list
  const int32_t* home_ids;
  int32_t* new_off;          // out: the new table
  int32_t* new_ids;
  uint8_t* pk;               // K and V planes, rows of ROWB bytes
  uint8_t* pv;
  uint32_t* meta;            // [n_pages][2][16]: ln beta bits, positions
  uint32_t* holes;           // workspace: one word per CSR slot
};

struct LDS {
  uint32_t src[4 * NT], dst[4 * NT];   // a window's movers (4 slots per thread)
  int64_t red[NW + 1];
};

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, WAVE);
  return v;
}

template <int ROWB>
__device__ void evict_head(int h, const Args& A, LDS& L) {
  constexpr int LPR = ROWB / 16;   // lanes per row
  constexpr int GROUPS = NT / LPR; // rows moved at once by the block
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;
  auto pages_of = [&](int j) -> int64_t {
    const int64_t want = ((int64_t)max(A.head_kept[j], 0) + A.reserve + PAGE - 1) / PAGE;
    return min(want, (int64_t)A.home_off[j + 1] - A.home_off[j]);
  };
  // the new page list: a prefix sum over the earlier heads, then the head's home prefix
  int64_t pb = 0;
  for (int j = tid; j < h; j += NT) pb += pages_of(j);
  pb = wave_sum(pb);
  if (lane == 0) L.red[wid] = pb;
  lds_barrier();
  pb = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) pb += L.red[i];
  const int64_t nh = pages_of(h);
  const int64_t hb = A.home_off[h];
  for (int64_t c = tid; c < nh; c += NT) A.new_ids[pb + c] = A.home_ids[hb + c];
  if (tid == 0) {
    A.new_off[h] = (int32_t)pb;
    if (h == A.n_heads - 1) A.new_off[A.n_heads] = (int32_t)(pb + nh);
  }
  lds_barrier();   // red is the scans' scratch below

  // valid entries: the length, bounded by the slots of the head's pages
  const int p0 = A.page_off[h];
  const int nv = (int)min((int64_t)max(A.len[h], 0), ((int64_t)A.page_off[h + 1] - p0) * PAGE);
  const int kh = min(max(A.head_kept[h], 0), nv);
  uint32_t* const hl = A.holes + (int64_t)p0 * PAGE;   // this head's hole list (its CSR slots)
  auto phys = [&](int i) -> uint32_t { return (uint32_t)A.page_ids[p0 + i / PAGE] * PAGE + i % PAGE; };
  // 1. holes: dropped slots below kh, in slot order (4 consecutive slots
  //    per thread: one 4-byte keep load, one block scan per 4,096 slots)
  const uint8_t* kh_bytes = A.keep + (int64_t)p0 * PAGE;   // the head's keep bytes, in slot order
  int n_holes = 0;
  for (int s0 = 0; s0 < kh; s0 += 4 * NT) {
    const int i = s0 + 4 * tid;   // a multiple of 4: its 4 bytes lie in one page
    const uint32_t kb = i < kh ? *reinterpret_cast<const uint32_t*>(kh_bytes + i) : ~0u;
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) bits |= (uint32_t)(i + j < kh && ((kb >> (8 * j)) & 0xFFu) == 0) << j;
    int64_t tot;
    int r = (int)block_exclusive_scan<NT>(__popc(bits), L.red, &tot);
    for (uint32_t b = bits; b; b &= b - 1) hl[n_holes + r++] = phys(i + __builtin_ctz(b));
    n_holes += __builtin_amdgcn_readfirstlane((int)tot);   // block-uniform: the loop below stays uniform
  }
  __syncthreads();   // the hole list (global memory) is complete and visible to the block
  // 2. movers: kept slots from kh on; mover r takes hole r
  int n_movers = 0;
  for (int s0 = kh & ~3; s0 < nv && n_movers < n_holes; s0 += 4 * NT) {
    const int i = s0 + 4 * tid;
    const uint32_t kb = i < nv ? *reinterpret_cast<const uint32_t*>(kh_bytes + i) : 0u;
    uint32_t bits = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bits |= (uint32_t)(i + j >= kh && i + j < nv && ((kb >> (8 * j)) & 0xFFu) != 0) << j;
    int64_t tot;
    int r = (int)block_exclusive_scan<NT>(__popc(bits), L.red, &tot);
    const int n_here = min(__builtin_amdgcn_readfirstlane((int)tot), n_holes - n_movers);
    for (uint32_t b = bits; b && r < n_here; b &= b - 1, ++r) {
      L.src[r] = phys(i + __builtin_ctz(b));
      L.dst[r] = hl[n_movers + r];
    }
    lds_barrier();
    const int part = tid % LPR;
    for (int q = tid / LPR; q < n_here; q += GROUPS) {
      const int64_t s = L.src[q], d = L.dst[q];
      const u32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(A.pk + s * ROWB + part * 16));
      const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(A.pv + s * ROWB + part * 16));
      const uint32_t mv = A.meta[(s / PAGE) * (2 * PAGE) + (part & 1) * PAGE + s % PAGE];
      __builtin_nontemporal_store(kv, reinterpret_cast<u32x4*>(A.pk + d * ROWB + part * 16));
      __builtin_nontemporal_store(vv, reinterpret_cast<u32x4*>(A.pv + d * ROWB + part * 16));
      if (part < 2) A.meta[(d / PAGE) * (2 * PAGE) + part * PAGE + d % PAGE] = mv;
    }
    n_movers += n_here;
    lds_barrier();   // src and dst are rewritten by the next window
  }
  if (tid == 0) A.len[h] = (int32_t)min((int64_t)kh, nh * PAGE);
}

}  // namespace tf
}  // namespace trimkv
