// Ragged, paged GQA decode attention renormalised over the retained set,
// with the dropped softmax mass; and the full-cache attention mass.
//
// ContourKV page, problem definition: deployed eviction keeps a subset and
// renormalises the attention weights over it (forced weights, not
// re-optimised).  ContourKV page, section 3: the dropped mass is the total
// weight of the discarded keys; sections 1 and 3: top-mass selection uses
// each key's attention mass.  DBTrimKV page, Method 4: paged per-head
// variable-length KV.
//
// bf16 caches: the CSR page list (all heads, in order) is split evenly over
// exactly as many waves as the GPU holds at once; a wave streams its pages
// and writes one partial (running max, kept sum, dropped sum, O[G][D]) per
// head its range touches, at index wave + head (unique: both ranges are
// monotone).  All G query heads of a KV head are processed together, so K
// and V are read once.  K and V pages reach LDS through direct global->LDS
// loads; S = K q^T and O += P V run on MFMA.  A second kernel merges the
// partials of each head in a fixed order, so results are run-to-run
// identical.  fp32 caches (small configurations) use one block per
// (head, 16-page chunk) and VALU arithmetic.
#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"
#include "launch.h"
#include "tailfill.h"

// Scratch of trimkv_decode_attn_noalloc: the partials of the flat split (or
// the fp32 work list) live here instead of in a caller's workspace.  Each
// GPU holds its own copy for the life of the process; host code reaches it
// only through the address hipGetSymbolAddress returns for that device.
static __device__ __align__(256) unsigned char scratch[TRIMKV_NOALLOC_SCRATCH_BYTES];

namespace trimkv {

namespace {

// Cache policy of the K/V page loads: non-temporal.  Every K/V byte is read
// once per call, and streaming reads that do not allocate in the caches
// reached 6.9-7.1 TB/s here against 5.0-6.3 TB/s for ordinary loads.
constexpr int CPOL_NT = 2;

constexpr int CHA_F32 = 16;     // pages per work item of the fp32 kernel (one key per thread)
constexpr int NT = 256;
constexpr int GMAX = 16;
constexpr int FLAT_WMAX = 8192;   // most waves of one bf16 launch (workspace bound)
// Threads per block of the bf16 kernel: eight waves, each staging two K and
// two V pages (16 KB at D = 128) in LDS, one block per CU.  Each SIMD then
// holds two waves of the same block (waves w and w + 4), which keep their
// progress even by wave priority (below).  Measured against four-wave
// blocks (two per CU), two- and one-wave blocks: those were 1-2%, 5% and 25%
// slower.
constexpr int NTA = 512;
// floats of a partial's statistics per query head: the kept keys' base-2
// maximum and sum relative to it, the dropped keys' sum and maximum
constexpr int NST = 4;
constexpr int SIMD_PAIR = 4;   // waves w and w ^ SIMD_PAIR share a SIMD
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

enum { A_PLAIN = 0, A_MASK = 1, A_LOGITS = 2, A_ERR = 3, A_GPLAIN = 4, A_GMASK = 5 };

struct AttnWs {
  int32_t* item_off;   // [H + 1]          (fp32 work list)
  int4* item;          // [Tmax + 4]       (fp32 work list: head, first CSR page, valid entries, pages)
  float* stats;        // [Smax][G][NST]   partials: base-2 kept max, kept sum, dropped sum, dropped max
  float* acc;          // [Smax][G][D]     partials: unnormalised outputs
  float* acc2;         // [Smax][G][D]     partials of the dropped keys (error mode), else null
  float* lse2;         // [H * G] base-2 LSE (mass op)
  float* logits;       // [n_pages][G][16] (mass op): page-major, so a page's logits are one 64 * G-byte run
};

struct AttnArgs {
  const int32_t* page_off;
  const int32_t* page_ids;
  const int32_t* len;
  const void* k;
  const void* v;
  const uint8_t* keep;   // CSR plane or null
  const void* q;
  int n_heads;
  int group;
  float scale2;          // scale * log2(e)
  int cha;               // pages per work item (fp32 path)
  int waves;             // waves of the launch (bf16 path; 0 = fp32 work list)
  AttnWs w;
  // outputs written by the merge of each head
  const float* lse_ref;
  float* out;
  float* dropped;
  float* lse_out;
  float* mu;             // error mode: dense output over every key, or null
  float* err;            // error mode: || mu - out ||_2 per query head
  // retention-gated modes: ln r = fp32(t - pos) * ln beta joins each logit
  const uint32_t* meta;  // [n_pages][2][16]: ln beta bits, positions
  const int32_t* seg;    // [n_seg + 1] first head of each segment
  const int32_t* tseg;   // [n_seg] decode step of each segment
  int n_seg;
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // plain vector loads/stores (no struct copies)

// Read-only inputs addressed with wave-uniform indices are read through the
// constant address space, which turns them into scalar loads.
typedef const __attribute__((address_space(4))) int32_t* c_i32;
typedef const __attribute__((address_space(4))) u32x4* c_u32x4;

// Work list of (head, chunk of cha pages) for the fp32 path: one 16-byte record per item.
// Work list of (head, chunk of cha pages): one 16-byte record per item.
__global__ void __launch_bounds__(1024) k_attn_prep(const int32_t* __restrict__ page_off,
                                                    const int32_t* __restrict__ len, int n_heads, int cha,
                                                    AttnWs w) {
  __shared__ int64_t tmp[1024 / WAVE + 1];
  __shared__ PrepLDS L;
  const int T = prep_chunks<1024>(page_off, len, n_heads, cha, L, tmp, w.item_off);
  for (int it = blockIdx.x * 1024 + threadIdx.x; it < T; it += gridDim.x * 1024) {
    const ChunkInfo ci = chunk_info(L, w.item_off, page_off, len, n_heads, cha, it);
    w.item[it] = make_int4(ci.h, ci.page0, ci.nv, ci.npg);
  }
}


// First CSR page of the flat range of wave w out of W over P pages, and the
// wave whose range holds page p.
__device__ __forceinline__ int64_t flat_begin(int64_t w, int64_t W, int64_t P) { return w * P / W; }
__device__ __forceinline__ int64_t flat_wave(int64_t p, int64_t W, int64_t P) { return ((p + 1) * W - 1) / P; }

// Merge all partials of query row g of KV head h.  The kept keys' sums are
// rescaled to Mk, the largest partial kept maximum, the dropped keys' to Md,
// the largest dropped maximum; O is rescaled like the kept sums and divided
// by theirs, and the dropped mass is Ld 2^Md / (Lk 2^Mk + Ld 2^Md), formed
// relative to the larger of the two.  A head without partials has an empty
// kept set: out = 0, dropped = 1, lse = -inf.  Partials of head h: fp32
// path, items item_off[h] .. item_off[h+1]-1 (add = 0); bf16 path, index
// w + h (add = h) for every wave w in [b, e), whose ranges meet the head's
// pages.  With fewer pages than waves (every = false) waves with an empty
// range wrote no partial and are skipped.
//
// One wave per query row and no block barriers: lane j holds the statistics
// of partial j, lane l accumulates output dimensions l, l + 64 (D = 128).
// The first MB partials' outputs are requested together with the
// statistics, so a row costs one round trip.  Every sum runs in a fixed
// order (partials ascending per lane, then a xor butterfly), so results are
// run-to-run identical whichever wave merges.
// ERR_OK = false compiles out the error mode's dense output (callers that
// never pass acc2).
template <int D, bool ERR_OK = true>
__device__ void merge_row(const AttnArgs& a, int h, int g, int b, int e, int add, bool every, int64_t P,
                          int with_out) {
  constexpr int DL = D / WAVE;   // output dimensions per lane
  constexpr int MB = 16;         // partial outputs per batch of loads
  const AttnWs& w = a.w;
  const int G = a.group;
  const int lane = threadIdx.x & (WAVE - 1);
  const int n = e - b;
  auto has = [&](int it) { return every || flat_begin(it, a.waves, P) < flat_begin(it + 1, a.waves, P); };
  const int ss = NST * G;   // floats between consecutive partials' statistics
  const float* st = w.stats + (size_t)(b + add) * ss + g * NST;        // partial j: st + j * ss
  const float* ac = w.acc + ((size_t)(b + add) * G + g) * D + lane;    // partial j, dim lane + 64k: ac + j * G * D + 64k
  const float* ac2 = w.acc2 ? w.acc2 + ((size_t)(b + add) * G + g) * D + lane : nullptr;
  const bool err = ERR_OK && ac2 != nullptr;   // wave-uniform

  // batch of MB partial outputs starting at partial j0 (zeros past the end)
  const int gs = G * D;   // floats between consecutive partials of the row
  float v[MB][DL], v2[MB][DL];
  auto load = [&](int j0) {
#pragma unroll
    for (int u = 0; u < MB; ++u)
#pragma unroll
      for (int k = 0; k < DL; ++k) v[u][k] = j0 + u < n ? ac[(j0 + u) * gs + 64 * k] : 0.f;
    if (err) {
#pragma unroll
      for (int u = 0; u < MB; ++u)
#pragma unroll
        for (int k = 0; k < DL; ++k) v2[u][k] = j0 + u < n ? ac2[(j0 + u) * gs + 64 * k] : 0.f;
    }
  };
  if (with_out) load(0);   // in flight with the statistics
  // statistics of partial j = lane (+ 64 per further batch)
  float m0 = -INFINITY, l0 = 0.f, d0 = 0.f, md0 = -INFINITY;
  const bool v0 = lane < n && has(b + lane);
  if (v0) {
    m0 = st[lane * ss];
    l0 = st[lane * ss + 1];
    d0 = st[lane * ss + 2];
    md0 = st[lane * ss + 3];
  }
  float Mk = m0, Md = md0;
  for (int j = WAVE + lane; j - lane < n; j += WAVE)
    if (j < n && has(b + j)) {
      Mk = fmaxf(Mk, st[j * ss]);
      Md = fmaxf(Md, st[j * ss + 3]);
    }
#pragma unroll
  for (int s = WAVE / 2; s > 0; s >>= 1) {
    Mk = fmaxf(Mk, __shfl_xor(Mk, s, WAVE));
    Md = fmaxf(Md, __shfl_xor(Md, s, WAVE));
  }
  // weights of each partial: 2^(m_j - Mk) and 2^(md_j - Md), zero for
  // partials without data and for a set without a finite logit
  auto weight = [&](float mj, float M, bool valid) { return valid && M != -INFINITY ? exp2f(mj - M) : 0.f; };
  const float w0 = weight(m0, Mk, v0), wd0 = weight(md0, Md, v0);
  // explicit roundings (no contraction left to the compiler), so that every
  // instantiation of the merge gives the same bits
  float la = __fmul_rn(l0, w0), ld = __fmul_rn(d0, wd0);
  for (int j = WAVE + lane; j - lane < n; j += WAVE) {
    if (j < n && has(b + j)) {
      la = fmaf(st[j * ss + 1], weight(st[j * ss], Mk, true), la);
      ld = fmaf(st[j * ss + 2], weight(st[j * ss + 3], Md, true), ld);
    }
  }
#pragma unroll
  for (int s = WAVE / 2; s > 0; s >>= 1) {
    la += __shfl_xor(la, s, WAVE);
    ld += __shfl_xor(ld, s, WAVE);
  }
  // the kept and dropped sums relative to the larger maximum T (ek, ed: the
  // scale factors; a set without a finite logit has a zero sum)
  const float T = fmaxf(Mk, Md);
  const float ek = la > 0.f ? exp2f(Mk - T) : 0.f, ed = ld > 0.f ? exp2f(Md - T) : 0.f;
  const float lat = __fmul_rn(la, ek), ldt = __fmul_rn(ld, ed), den = __fadd_rn(lat, ldt);
  if (lane == 0) {
    const int qh = h * G + g;
    const float l2 = la > 0.f ? Mk + log2f(la) : -INFINITY;  // base-2 LSE of the kept set
    const float lse = l2 * LN2;
    if (a.lse_out) a.lse_out[qh] = lse;
    if (w.lse2) w.lse2[qh] = l2;
    if (a.dropped) {
      float dm = 1.f;
      if (la > 0.f) dm = a.lse_ref ? -expm1f(lse - a.lse_ref[qh]) : ldt / den;
      a.dropped[qh] = dm;
    }
  }
  if (!with_out) return;
  float s[DL], s2[DL];
#pragma unroll
  for (int k = 0; k < DL; ++k) s[k] = s2[k] = 0.f;
  float wl = w0, wdl = wd0;   // weights of partial j0 - j0 % 64 + lane
  for (int j0 = 0; j0 < n; j0 += MB) {
    if (j0 > 0) {
      if (j0 % WAVE == 0) {
        const int j = j0 + lane;
        const bool vj = j < n && has(b + j);
        wl = weight(vj ? st[j * ss] : -INFINITY, Mk, vj);
        if (err) wdl = weight(vj ? st[j * ss + 3] : -INFINITY, Md, vj);
      }
      load(j0);
    }
    // partials without data hold stale words: selected away, never multiplied
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const float wt = __shfl(wl, j0 % WAVE + u, WAVE);
      const bool use = j0 + u < n && wt != 0.f;
#pragma unroll
      for (int k = 0; k < DL; ++k) s[k] = use ? fmaf(v[u][k], wt, s[k]) : s[k];
    }
    if (err) {   // the dropped keys' outputs, against their own maximum
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        const float wt = __shfl(wdl, j0 % WAVE + u, WAVE);
        const bool use = j0 + u < n && wt != 0.f;
#pragma unroll
        for (int k = 0; k < DL; ++k) s2[k] = use ? fmaf(v2[u][k], wt, s2[k]) : s2[k];
      }
    }
  }
  float q2 = 0.f;
#pragma unroll
  for (int k = 0; k < DL; ++k) {
    const size_t o = ((size_t)h * G + g) * D + lane + 64 * k;
    const float mA = la > 0.f ? s[k] / la : 0.f;
    a.out[o] = mA;
    if (err) {
      // dense output over every key: both sums relative to T
      const float mu = den > 0.f ? fmaf(s[k], ek, __fmul_rn(s2[k], ed)) / den : 0.f;
      if (a.mu) a.mu[o] = mu;
      q2 += (mu - mA) * (mu - mA);
    }
  }
  if (err) {   // e_s(A) = || mu - m_A ||_2, fixed-order sum over the D dimensions
#pragma unroll
    for (int s = WAVE / 2; s > 0; s >>= 1) q2 += __shfl_xor(q2, s, WAVE);
    if (lane == 0) a.err[(size_t)h * G + g] = sqrtf(q2);
  }
}

// Query row `row` of the merge (wave-uniform); rows past the last return.
template <int D, bool ERR_OK = true>
__device__ void merge_query_row(const AttnArgs& a, int row, int with_out) {
  const AttnWs& w = a.w;
  const int G = a.group;
  if (row >= a.n_heads * G) return;   // per-wave exit: no block barriers below
  const int h = row / G, g = row % G;
  int b, e, add;
  const int64_t P = a.page_off[a.n_heads];
  if (a.waves) {
    const int64_t p0 = a.page_off[h], p1 = a.page_off[h + 1];
    b = 0, e = 0, add = h;
    if (p1 > p0) {
      b = (int)flat_wave(p0, a.waves, P);
      e = (int)flat_wave(p1 - 1, a.waves, P) + 1;
    }
  } else {
    b = w.item_off[h], e = w.item_off[h + 1], add = 0;
  }
  // waves with an empty range (fewer pages than waves) wrote no partial; with
  // at least as many pages as waves every range is nonempty (no divisions)
  const bool every = !a.waves || P >= a.waves;
  merge_row<D, ERR_OK>(a, h, g, b, e, add, every, P, with_out);
}

// Merge kernel: one wave per query row, over the partials the main kernel
// left in the workspace (ERR: the error mode's launches, which pass acc2).
template <int D, bool ERR>
__global__ void __launch_bounds__(NT) k_attn_merge(AttnArgs a, int with_out) {
  merge_query_row<D, ERR>(a, blockIdx.x * (NT / WAVE) + __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE),
                          with_out);
}

// The merge beside a tail-filled eviction of the same cache, in one launch:
// neither reads what the other writes (the merge reads the partials and the
// page offsets, the eviction the keep plane and the rows, and writes rows,
// lengths and a new table), and both wait only for the main kernel.  Blocks
// [0, merge_blocks) merge, one wave per query row; each later block evicts
// one head.
template <int D, int ROWB>
__global__ void __launch_bounds__(tf::NT) k_attn_merge_evict(AttnArgs a, tf::Args t, int merge_blocks) {
  __shared__ tf::LDS L;
  if ((int)blockIdx.x < merge_blocks) {   // block-uniform
    merge_query_row<D, false>(a, blockIdx.x * (tf::NT / WAVE) + __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), 1);
    return;
  }
  tf::evict_head<ROWB>(blockIdx.x - merge_blocks, t, L);
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only
constexpr int wait_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// LDS operand reads as inline assembly (see the staging notes in the kernel);
// their results may be used only after lds_wait_all, which ties every result
// register to the wait so no use can be scheduled before it.
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

__device__ __forceinline__ short4_t lds_read_tr_b64(uint32_t addr) {
  short4_t v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

template <int NK, int NV>
__device__ __forceinline__ void lds_wait_all(u32x4 (&k)[NK], short4_t (&v)[NV]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int u = 0; u < NK; ++u) asm volatile("" : "+v"(k[u]));
#pragma unroll
  for (int n = 0; n < NV; ++n) asm volatile("" : "+v"(v[n]));
}

// 16-byte chunks of zeros: the source of V rows that take no part
__device__ const uint32_t kZeroChunks[64 * 4] = {};

// Threshold (log2 units) of the lazily updated running maximum: between two
// rescalings every exp2(z - m) stays below 2^RESCALE_T, far inside fp32.
constexpr float RESCALE_T = 10.f;

// Page tiles in LDS, one K and one V tile per wave and buffer.  A tile is 16
// rows of CH 16-byte chunks; chunk c of row k is stored at chunk position
// c ^ swz(k) of its row.  The swizzles make every LDS access of the kernel
// free of bank conflicts: the K operand reads (16 lanes = 16 keys, one chunk
// each) and the transposing V reads (lanes of a half-wave touch 8 rows x 2
// chunks).
template <int D>
struct Tile {
  static constexpr int CH = D / 8;    // 16-byte chunks per row
  static constexpr int LPP = CH / 4;  // 16-byte loads per lane per tile
  static __device__ __forceinline__ int slot_k(int k, int c) { return k * CH + (c ^ (D == 128 ? k : (k >> 1))); }
  static __device__ __forceinline__ int slot_v(int k, int c) {
    return k * CH + (c ^ (D == 128 ? ((2 * k) & 15) : ((2 * (k >> 1)) & 7)));
  }
};

__device__ __forceinline__ short4_t pack_hi(const float (&p)[4]) {
  // upper halves of the fp32 bit patterns: bf16 truncations of p
  const uint32_t w0 = __builtin_amdgcn_perm(__float_as_uint(p[1]), __float_as_uint(p[0]), 0x07060302u);
  const uint32_t w1 = __builtin_amdgcn_perm(__float_as_uint(p[3]), __float_as_uint(p[2]), 0x07060302u);
  return __builtin_bit_cast(short4_t, make_uint2(w0, w1));
}

__device__ __forceinline__ short4_t pack_rne(float a, float b, float c, float d) {
  const bf16x2_t x = __builtin_convertvector((float2_t){a, b}, bf16x2_t);
  const bf16x2_t y = __builtin_convertvector((float2_t){c, d}, bf16x2_t);
  return __builtin_bit_cast(short4_t, make_uint2(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y)));
}

__device__ __forceinline__ uint32_t pick4(u32x4 v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// bf16 K/V.  MODE: A_PLAIN (every valid key kept), A_MASK (keep plane;
// dropped keys only enter the dropped sum and their V rows are not read),
// A_ERR (as A_MASK, and the dropped keys' P V goes to a second accumulator,
// so that the merge has the dense output as well; every V row is read),
// A_LOGITS (base-2 logits of every valid key and (max, sum) partials),
// A_GPLAIN / A_GMASK (as A_PLAIN / A_MASK with retention-gated weights: each
// base-2 logit gains ln r * log2(e), r = beta^(t - pos), read from the page's
// metadata line together with its K and V).
//
// Wave w of W streams CSR pages [w P / W, (w + 1) P / W) and, per head
// segment of that range, writes the partial with index w + head.  Each
// page's K and V tiles are loaded with direct global->LDS loads (contiguous
// 1 KB per instruction; two pages in flight) into the wave's swizzled LDS
// tiles and read back as MFMA operands:
//   S = K q^T     v_mfma_f32_16x16x32_bf16: key = lane % 16, 8 dims per lane;
//                 lane (r, col) receives S[key 4r + j][query head col];
//   O += P V      v_mfma_f32_16x16x16_bf16, A = P exactly as S is laid out
//                 (row = query head, keys 4r..4r+3), B = V through the
//                 transposing LDS read; P is split into a bf16 truncation and
//                 a bf16 remainder (two MFMAs), so each weight carries a
//                 relative error below 2^-16.
// One running maximum per query head (shared by the four 16-lane rows), and
// in the mask modes a second one for the dropped keys, is raised only when a
// logit exceeds it by more than RESCALE_T, a wave-uniform branch; the common
// page costs one FMA and one exp2 per logit.  With its own maximum the kept
// set's weights stay in range however far the dropped keys' logits lie above
// them (retention gates can put them hundreds of units apart).
// Where a wave's range crosses into another head (D = 128, all modes but
// A_ERR and A_LOGITS), the next segment's first two pages, and for groups of
// up to 8 query heads its query rows (staged in LDS), are requested during
// the last page of the segment before, so that the crossing costs no load
// latency.
// ---------------------------------------------------------------------------
template <int D, int MODE>
__global__ void __launch_bounds__(NTA, D == 64 ? 4 : 2) k_attn_bf16(AttnArgs a) {
  typedef Tile<D> TL;
  constexpr int CH = TL::CH, LPP = TL::LPP;
  constexpr int KU = D / 32;    // QK MFMAs per page
  constexpr int NV = D / 16;    // PV output column blocks
  constexpr bool LOGITS = MODE == A_LOGITS;
  constexpr bool MASKED = MODE == A_MASK || MODE == A_ERR || MODE == A_GMASK;
  constexpr bool ERR = MODE == A_ERR;
  constexpr bool GATED = MODE == A_GPLAIN || MODE == A_GMASK;
  // Segments requested ahead, during the last page of the segment before
  // (D = 128).  Not in the error mode, whose second accumulator leaves no
  // registers to spare, nor in the logits mode, whose ranges hold hundreds of
  // pages, nor for D = 64, where the registers it takes would halve the
  // blocks per compute unit.
  constexpr bool XS = D == 128 && !ERR && !LOGITS;
  // load instructions per page; pages in flight are tracked by vmcnt.  The
  // logits mode also stores each page's logits inside the loop; those stores
  // are not counted: loads complete in issue order among themselves, so once
  // no more than the next page's LPP loads (or stores) are outstanding, the
  // current page has arrived, whether or not the stores complete in order
  // with the loads (at worst the wait also covers a store)
  constexpr int PER_PAGE = LOGITS ? LPP : 2 * LPP + (GATED ? 2 : 0);
  __shared__ u32x4 lds_k[NTA / WAVE][2][16 * CH];
  __shared__ u32x4 lds_v[NTA / WAVE][2][LOGITS ? 1 : 16 * CH];
  // the next segment's query rows (G x D bf16, row-major), one area of 128
  // chunks per wave: rows of up to 8 query heads (larger groups load the
  // query at the segment's start)
  constexpr int QSL = XS ? 128 : 1;
  __shared__ u32x4 lds_q[NTA / WAVE][QSL];
  const AttnWs& w = a.w;
  const int lane = threadIdx.x & 63, r = lane >> 4, col = lane & 15, wv = threadIdx.x >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(wv);
  const int H = a.n_heads, G = a.group;
  const c_i32 cpo = (c_i32)a.page_off;
  const c_i32 cids = (c_i32)a.page_ids;
  const c_i32 clen = (c_i32)a.len;
  // page offsets are wave-uniform; readfirstlane keeps everything derived from them in scalar registers
  auto pg = [&](int hh) -> int { return __builtin_amdgcn_readfirstlane(cpo[hh]); };
  auto head_of = [&](int p) -> int {   // head whose pages hold CSR page p (64 probes per step)
    return __builtin_amdgcn_readfirstlane(wave_upper_index(a.page_off, H + 1, p));
  };
  const int64_t P = pg(H);
  const int W = a.waves;
  const int wave = blockIdx.x * (NTA / WAVE) + wu;
  // pages done by each wave of the block: the wave behind its SIMD partner
  // takes the higher issue priority, so that the two finish together
  // instead of the older one first (the younger, then alone on its SIMD,
  // keeping half as many pages in flight)
  __shared__ int prog[NTA / WAVE];
  if (lane == 0) prog[wu] = 0;
  int p = (int)flat_begin(wave, W, P);
  const int pbeg = p;
  const int pend = (int)flat_begin(wave + 1, W, P);
  if (p >= pend) return;   // per-wave exit: no block barriers below

  const uint8_t* kbase = (const uint8_t*)a.k;
  const uint8_t* vbase = (const uint8_t*)a.v;
  // per-lane byte offsets within a page of the chunks each load instruction
  // fetches: LDS slot s of a tile receives the chunk the swizzle places there
  uint32_t gk[LPP], gv[LPP];
#pragma unroll
  for (int u = 0; u < LPP; ++u) {
    const int sl = 64 * u + lane, row = sl / CH;
    gk[u] = row * (D * 2) + ((sl % CH) ^ (TL::slot_k(row, 0) - row * CH)) * 16;
    gv[u] = row * (D * 2) + ((sl % CH) ^ (TL::slot_v(row, 0) - row * CH)) * 16;
  }
  // LDS byte offsets of this lane's operand chunks within a tile
  const int vrow = 4 * r + (col >> 2), vhalf = col & 1, vc = (col & 3) >> 1;
  uint32_t koff[KU], voff[LOGITS ? 1 : NV];
#pragma unroll
  for (int u = 0; u < KU; ++u) koff[u] = TL::slot_k(col, 4 * u + r) * 16;
  if (!LOGITS) {
#pragma unroll
    for (int n = 0; n < NV; ++n) voff[n] = TL::slot_v(vrow, 2 * n + vc) * 16 + 8 * vhalf;
  }
  typedef __attribute__((address_space(1))) const void* gptr;
  typedef __attribute__((address_space(3))) void* lptr;

  // where a segment starts at CSR page s: its head (the first head from hh
  // on whose pages reach past s), its end, its valid entries, its first two
  // physical pages and their keep words (indices clamped into the wave's
  // range: a page past the segment is unused); scalar loads only
  const u32x4 all_kept_c = (u32x4){~0u, ~0u, ~0u, ~0u};
  struct Seg { int h, send, nv, id0, id1, id2; u32x4 kw0, kw1; };
  auto seg_at = [&](int s, int hh) -> Seg {
    Seg g;
    // the physical pages and keep words depend only on s: requested first
    g.id0 = cids[s];
    g.id1 = cids[min(s + 1, pend - 1)];
    g.id2 = cids[min(s + 2, pend - 1)];
    g.kw0 = g.kw1 = all_kept_c;
    if (MASKED) {
      const c_u32x4 ck = (c_u32x4)a.keep;   // 16 keep bytes per page
      g.kw0 = ck[s];
      g.kw1 = ck[min(s + 1, pend - 1)];   // unused where the segment has one page
    }
    int hb = pg(hh), he = pg(hh + 1), hlen = __builtin_amdgcn_readfirstlane(clen[hh]);
    while (he <= s) {   // heads without pages hold no page
      ++hh;
      hb = he;
      he = pg(hh + 1);
      hlen = __builtin_amdgcn_readfirstlane(clen[hh]);
    }
    g.h = hh;
    g.send = min(pend, he);
    const int cnt = g.send - s, v0 = hlen - (s - hb) * PAGE;
    g.nv = v0 < 0 ? 0 : (v0 > cnt * PAGE ? cnt * PAGE : v0);
    return g;
  };
  u32x4 g_lnb[GATED ? 2 : 1], g_pos[GATED ? 2 : 1];
  // page i's loads into tile buffer B; phys = its physical page, kw4 = its 16
  // keep bytes (mask mode), nvv = the valid entries of its segment.  Gated
  // modes: ln beta bits and positions of keys 4r..4r+3 of the page in
  // register buffer B (loaded with the page, two pages in flight like the tiles)
  auto dma = [&](auto B, int i, int64_t phys, u32x4 kw4, int nvv) {
    constexpr int buf = decltype(B)::value;
    const uint8_t* kpage = kbase + phys * (PAGE * D * 2);
    const uint8_t* vpage = vbase + phys * (PAGE * D * 2);
#pragma unroll
    for (int u = 0; u < LPP; ++u)
      __builtin_amdgcn_global_load_lds((gptr)(kpage + gk[u]), (lptr)(&lds_k[wu][buf][64 * u]), 16, 0, CPOL_NT);
    if (!LOGITS) {
      const bool full = (i + 1) * PAGE <= nvv;   // wave-uniform
      if ((MODE == A_PLAIN || MODE == A_GPLAIN || ERR) && full) {
#pragma unroll
        for (int u = 0; u < LPP; ++u)
          __builtin_amdgcn_global_load_lds((gptr)(vpage + gv[u]), (lptr)(&lds_v[wu][buf][64 * u]), 16, 0, CPOL_NT);
      } else {
#pragma unroll
        for (int u = 0; u < LPP; ++u) {
          const int row = (64 * u + lane) / CH;
          bool need = i * PAGE + row < nvv;
          if (MODE == A_MASK || MODE == A_GMASK) need &= ((pick4(kw4, row >> 2) >> (8 * (row & 3))) & 0xFFu) != 0;
          // rows that take no part read zeros
          const uint8_t* src = need ? vpage + gv[u] : reinterpret_cast<const uint8_t*>(kZeroChunks) + 16 * lane;
          __builtin_amdgcn_global_load_lds((gptr)src, (lptr)(&lds_v[wu][buf][64 * u]), 16, 0, 0);
        }
      }
    }
    if (GATED) {   // counted in PER_PAGE: issued after the page's tiles
      const uint32_t* mrow = a.meta + phys * (2 * PAGE) + 4 * r;
      g_lnb[buf & (GATED ? 1 : 0)] = *reinterpret_cast<const u32x4*>(mrow);
      g_pos[buf & (GATED ? 1 : 0)] = *reinterpret_cast<const u32x4*>(mrow + PAGE);
    }
  };
  // B operand of QK MFMA u for head hq: dims 32u + 8r .. +7 of query head
  // col.  Columns col >= G repeat query head 0: their logits, weights and
  // outputs follow column 0's and are never stored.
  auto load_q = [&](int hq, u32x4 (&qo)[KU]) {
    const uint8_t* qrow = (const uint8_t*)a.q + ((size_t)hq * G + (col < G ? col : 0)) * D * 2 + 16 * r;
#pragma unroll
    for (int u = 0; u < KU; ++u) qo[u] = *reinterpret_cast<const u32x4*>(qrow + 64 * u);
  };
  // Query rows of head hq copied into the wave's LDS area by the same
  // asynchronous loads as the pages, so that the next segment's query is
  // requested ahead of that segment like its pages: one load instruction per
  // 64 chunks, lanes past the rows idle (every instruction has lane 0
  // active, so each one is issued and counted).
  const int qch = G * D / 8;   // 16-byte chunks of the rows
  const bool qst = XS && qch <= QSL;
  auto stage_q = [&](int hq) {
    const uint8_t* qh = (const uint8_t*)a.q + (size_t)hq * G * D * 2;
#pragma unroll
    for (int c = 0; c < (QSL + 63) / 64; ++c) {
      if (64 * c < qch) {   // wave-uniform
        if (64 * c + lane < qch)
          __builtin_amdgcn_global_load_lds((gptr)(qh + 16 * (64 * c + lane)), (lptr)(&lds_q[wu][64 * c]), 16, 0, 0);
      }
    }
  };
  // each segment's first two pages (and staged query) are requested before
  // the segment starts: the first segment's here, each later one's during
  // the last page of the segment before it (both tiles are free by then).
  // The compiler's own waits do not count the asynchronous LDS loads, so a
  // query held in registers across them would be awaited with every page in
  // flight; staged in LDS, it is awaited by the explicit counts only.
  Seg nx = seg_at(p, head_of(p));
  if (XS) {
    if (qst) stage_q(nx.h);
    dma(std::integral_constant<int, 0>{}, 0, nx.id0, nx.kw0, nx.nv);
    if (nx.send - p > 1) dma(std::integral_constant<int, 1>{}, 1, nx.id1, nx.kw1, nx.nv);
  }
  while (true) {
    // ---- one head segment: CSR pages [p, send) of head h ----
    const Seg cur = nx;
    const int h = cur.h, send = cur.send, nv = cur.nv;
    const int page0 = p, cnt = send - p;
    u32x4 qop[KU];
    if (qst) {
      // the staged query rows and the segment's first page, issued in that
      // order and followed by at most the second page's loads, have arrived
      // once no more than one page's loads are outstanding
      __builtin_amdgcn_s_waitcnt(wait_vm(PER_PAGE));
      const uint32_t ql = lds_addr(&lds_q[wu][0]) + (col < G ? col : 0) * D * 2 + 16 * r;
#pragma unroll
      for (int u = 0; u < KU; ++u) qop[u] = lds_read_b128(ql + 64 * u);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int u = 0; u < KU; ++u) asm volatile("" : "+v"(qop[u]));
    } else {
      load_q(h, qop);
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
      if (!XS) {   // the segment's first two pages, requested only now
        dma(std::integral_constant<int, 0>{}, 0, cur.id0, cur.kw0, nv);
        if (cnt > 1) dma(std::integral_constant<int, 1>{}, 1, cur.id1, cur.kw1, nv);
      }
    }
    const c_u32x4 ckeep = (c_u32x4)(a.keep + (int64_t)page0 * PAGE);   // 16 keep bytes per page
    int t_h = 0;   // decode step of the head's segment (gated modes)
    if (GATED) {
      const c_i32 cseg = (c_i32)a.seg;
      int lo = 0, hi = a.n_seg;   // last segment whose first head is <= h
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cseg[mid] <= h) lo = mid; else hi = mid;
      }
      t_h = __builtin_amdgcn_readfirstlane(((c_i32)a.tseg)[lo]);
    }
    const bool has_next = send < pend;   // wave-uniform
    if (XS && has_next) nx = seg_at(send, h + 1);

    float m = -INFINITY, la = 0.f, ld = 0.f;
    float nm = INFINITY;   // -m, or +inf while m = -inf (every finite logit then forces an update)
    float md = -INFINITY, nmd = INFINITY;   // the same for the dropped keys (mask modes)
    float4_t acc[LOGITS ? 1 : NV], acc2[ERR ? NV : 1];
#pragma unroll
    for (int n = 0; n < (LOGITS ? 1 : NV); ++n) acc[n] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < (ERR ? NV : 1); ++n) acc2[n] = (float4_t){0.f, 0.f, 0.f, 0.f};

  auto math = [&](int i, const u32x4 (&kop)[KU], const short4_t (&vop)[LOGITS ? 1 : NV], uint32_t kwr,
                  u32x4 glnb, u32x4 gpos, auto&& after_qk) {
    // ---- S = K q^T ----
    float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KU; ++u)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[u]),
                                                  __builtin_bit_cast(bf16x8_t, qop[u]), s, 0, 0, 0);
    after_qk();   // the query operand is free from here on
    // base-2 offset of each logit: 0, or ln r * log2(e) with ln r formed as
    // the score kernel forms it (one fp32 product)
    float gate[4] = {0.f, 0.f, 0.f, 0.f};
    if (GATED) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        gate[j] = __fmul_rn((float)(t_h - (int)gpos[j]), __uint_as_float(glnb[j])) * LOG2E;
    }
    const int i0 = i * PAGE + 4 * r;          // entry of key 4r within the item
    const bool full = (i + 1) * PAGE <= nv;   // wave-uniform
    // keys 4r..4r+3 in the kept set (mask modes: kept and valid; the other
    // modes keep every key).  Dropped keys are weighed against a running
    // maximum of their own, so that a kept set far below the dropped keys
    // keeps its relative weights instead of underflowing against them.
    bool kj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kj[j] = !MASKED || (((kwr >> (8 * j)) & 0xFFu) && (full || i0 + j < nv));
    float pj[4];
    bool slow = !full;
    if (full) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float off = kj[j] ? nm : nmd;
        pj[j] = fmaf(s[j], a.scale2, GATED ? gate[j] + off : off);
      }
      // NaN (gated: a -inf gate while the maximum is -inf) takes the exact path too
      slow = __any(!(fmaxf(fmaxf(pj[0], pj[1]), fmaxf(pj[2], pj[3])) <= RESCALE_T));
    }
    if (slow) {
      float z[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = i0 + j < nv ? (GATED ? fmaf(s[j], a.scale2, gate[j]) : s[j] * a.scale2) : -INFINITY;
      // maxima of the page for query head col, kept and dropped keys
      float pk = -INFINITY, pdm = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (kj[j]) pk = fmaxf(pk, z[j]);
        else pdm = fmaxf(pdm, z[j]);
      }
      pk = fmaxf(pk, __shfl_xor(pk, 16, WAVE));
      pk = fmaxf(pk, __shfl_xor(pk, 32, WAVE));
      const float mn = fmaxf(m, pk);
      float alpha = 1.f;
      if (mn != -INFINITY) {
        alpha = exp2f(m - mn);   // 0 while m = -inf
        m = mn;
        nm = -mn;
      }
      la *= alpha;
      float alphad = 1.f;
      if (MASKED) {
        pdm = fmaxf(pdm, __shfl_xor(pdm, 16, WAVE));
        pdm = fmaxf(pdm, __shfl_xor(pdm, 32, WAVE));
        const float mnd = fmaxf(md, pdm);
        if (mnd != -INFINITY) {
          alphad = exp2f(md - mnd);
          md = mnd;
          nmd = -mnd;
        }
        ld *= alphad;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) pj[j] = z[j] - (kj[j] ? m : md);
      if (!LOGITS) {
        // output row g = 4r + j belongs to query head 4r + j: its factors live in lane 4r + j
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float aj = __shfl(alpha, 4 * r + j, WAVE);
#pragma unroll
          for (int n = 0; n < NV; ++n) acc[n][j] *= aj;
          if (ERR) {
            const float adj = __shfl(alphad, 4 * r + j, WAVE);
#pragma unroll
            for (int n = 0; n < NV; ++n) acc2[n][j] *= adj;
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) pj[j] = __builtin_amdgcn_exp2f(pj[j]);   // exp2(-inf) = 0
    if (slow) {   // a key whose set has no finite logit yet weighs nothing (-inf - -inf)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((kj[j] ? m : md) == -INFINITY) pj[j] = 0.f;
    }
    if (LOGITS) {
      if (col < G) {
        float* dst = w.logits + ((int64_t)(page0 + i) * G + col) * PAGE + 4 * r;
        if (full) {
          *reinterpret_cast<float4*>(dst) = make_float4(s[0] * a.scale2, s[1] * a.scale2, s[2] * a.scale2,
                                                        s[3] * a.scale2);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (i0 + j < nv) dst[j] = s[j] * a.scale2;
        }
      }
      la += (pj[0] + pj[1]) + (pj[2] + pj[3]);
      return;
    }
    float pd[4] = {0.f, 0.f, 0.f, 0.f};   // weights of the dropped keys (error mode)
    if (MASKED) {
      float sk = 0.f, sd = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sk += kj[j] ? pj[j] : 0.f;
        sd += kj[j] ? 0.f : pj[j];
        if (ERR) pd[j] = kj[j] ? 0.f : pj[j];
        if (!kj[j]) pj[j] = 0.f;
      }
      la += sk;
      ld += sd;
    } else {
      la += (pj[0] + pj[1]) + (pj[2] + pj[3]);
    }
    // ---- O += P V (P = hi + lo, both bf16) ----
    const short4_t phi = pack_hi(pj);
    float rem[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) rem[j] = pj[j] - __uint_as_float(__float_as_uint(pj[j]) & 0xFFFF0000u);
    const short4_t plo = pack_rne(rem[0], rem[1], rem[2], rem[3]);
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vop[n], acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vop[n], acc[n], 0, 0, 0);
    }
    if (ERR) {   // dropped keys: same split, second accumulator
      const short4_t dhi = pack_hi(pd);
      float drem[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) drem[j] = pd[j] - __uint_as_float(__float_as_uint(pd[j]) & 0xFFFF0000u);
      const short4_t dlo = pack_rne(drem[0], drem[1], drem[2], drem[3]);
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        acc2[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dhi, vop[n], acc2[n], 0, 0, 0);
        acc2[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dlo, vop[n], acc2[n], 0, 0, 0);
      }
    }
  };


    // Page i + 1 is in flight while page i is read and computed; page i + 2
    // is requested as soon as page i's operands are in registers.  The
    // operand reads are inline assembly with explicit waits: the compiler
    // would otherwise wait for every outstanding page before any LDS read.
    // The page id and keep bytes that a step needs are read one step earlier
    // (scalar loads), so no load is issued behind a dependent table read.
    const u32x4 all_kept = (u32x4){~0u, ~0u, ~0u, ~0u};
    auto keep4 = [&](int i) -> u32x4 { return MASKED ? ckeep[i] : all_kept; };
    int64_t id_n = cur.id2;                                 // page of the next load (i + 2)
    u32x4 kwd_n = cnt > 2 ? keep4(2) : all_kept;         // its keep bytes
    u32x4 kwm_n = keep4(0);                              // keep bytes of the next page computed
    // B: the tile buffer, i & 1 (a constant, or at run time for the last page)
    auto step = [&](auto B, int i, auto LAST) {
      const int buf = B;
      const u32x4 kwm = kwm_n;
      const uint32_t kwr = pick4(kwm, r);   // keep word of keys 4r..4r+3 (mask mode)
      asm volatile("" ::: "memory");
      if (PER_PAGE && i + 1 < cnt) __builtin_amdgcn_s_waitcnt(wait_vm(PER_PAGE));
      else __builtin_amdgcn_s_waitcnt(wait_vm(0));
      const uint32_t kl = lds_addr(&lds_k[wu][buf][0]), vl = lds_addr(&lds_v[wu][buf][0]);
      u32x4 kop[KU];
      short4_t vop[LOGITS ? 1 : NV];
#pragma unroll
      for (int u = 0; u < KU; ++u) kop[u] = lds_read_b128(kl + koff[u]);
      if (!LOGITS) {
#pragma unroll
        for (int n = 0; n < NV; ++n) vop[n] = lds_read_tr_b64(vl + voff[n]);
      }
      lds_wait_all(kop, vop);   // the tile may be overwritten once these reads are done
      {
        const int done = page0 - pbeg + i;
        if (lane == 0) prog[wu] = done;
        const int other = __builtin_amdgcn_readfirstlane(prog[wu ^ SIMD_PAIR]);
        if (done <= other) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(0);
      }
      // page i's gate words, taken before page i + 2's loads reuse their registers
      const u32x4 glnb = (buf & 1) ? g_lnb[GATED ? 1 : 0] : g_lnb[0];
      const u32x4 gpos = (buf & 1) ? g_pos[GATED ? 1 : 0] : g_pos[0];
      if constexpr (!decltype(LAST)::value) {
        if (i + 2 < cnt) dma(B, i + 2, id_n, kwd_n, nv);
      }
      if (i + 3 < cnt) {
        id_n = cids[page0 + i + 3];
        kwd_n = keep4(i + 3);
      }
      if (i + 1 < cnt) kwm_n = keep4(i + 1);
      asm volatile("" ::: "memory");
      math(i, kop, vop, kwr, glnb, gpos, [&] {
        if constexpr (XS && decltype(LAST)::value == 1) {
          // the segment's last page, once its logits are formed, where
          // another segment follows: that segment's query operand, then its
          // first two pages (both tiles are free by now)
          if (qst) stage_q(nx.h);
          dma(std::integral_constant<int, 0>{}, 0, nx.id0, nx.kw0, nx.nv);
          if (nx.send - send > 1) dma(std::integral_constant<int, 1>{}, 1, nx.id1, nx.kw1, nx.nv);
        }
      });
    };
    constexpr std::integral_constant<int, 0> B0{};
    constexpr std::integral_constant<int, 1> B1{};
    // kinds of step: a page before the last, the last page where another
    // segment follows, the wave's last page
    constexpr std::integral_constant<int, 0> MID{};
    constexpr std::integral_constant<int, 1> NEXT{};
    constexpr std::integral_constant<int, 2> LASTSEG{};

    // ---- partial of this segment: the maxima are common to the four rows ----
    auto finish = [&] {
    const size_t part = (size_t)wave + h;
    la += __shfl_xor(la, 16, WAVE);
    la += __shfl_xor(la, 32, WAVE);
    ld += __shfl_xor(ld, 16, WAVE);
    ld += __shfl_xor(ld, 32, WAVE);
    if (r == 0 && col < G) {
      float* st = w.stats + (part * G + col) * NST;
      st[0] = m;
      st[1] = la;
      st[2] = ld;
      st[3] = md;
    }
    if (!LOGITS) {
      // lane (r, col) holds O[query head 4r + j][dim 16n + col]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int g = 4 * r + j;
        if (g < G) {
          float* dst = w.acc + (part * G + g) * D + col;
#pragma unroll
          for (int n = 0; n < NV; ++n) dst[16 * n] = acc[n][j];
          if (ERR) {
            float* dst2 = w.acc2 + (part * G + g) * D + col;
#pragma unroll
            for (int n = 0; n < NV; ++n) dst2[16 * n] = acc2[n][j];
          }
        }
      }
    }
    };
    if constexpr (!XS) {
      for (int i = 0; i < cnt; i += 2) {
        step(B0, i, MID);
        if (i + 1 < cnt) step(B1, i + 1, MID);
      }
      finish();
      if (!has_next) break;
      p = send;
      nx = seg_at(p, h + 1);
      continue;
    }
    int i = 0;
    for (; i + 2 < cnt; i += 2) {
      step(B0, i, MID);
      step(B1, i + 1, MID);
    }
    if (i + 1 < cnt) step(B0, i++, MID);
    // the last page: one code path whichever its buffer; the wave's last
    // segment leaves the loop on its own path, so that every path around the
    // loop issues the next segment's loads
    if (!has_next) {
      step(i & 1, i, LASTSEG);
      finish();
      break;
    }
    step(i & 1, i, NEXT);
    finish();
    p = send;
  }
}

// ---------------------------------------------------------------------------
// fp32 K/V (any D in {64,128}, G <= 16): one thread per key of the item.
// ---------------------------------------------------------------------------
template <int D, bool LOGITS>
__global__ void __launch_bounds__(NT) k_attn_f32(AttnArgs a) {
  constexpr int NKEY = CHA_F32 * PAGE;  // 256 keys per item = one per thread
  __shared__ float sq[GMAX][D];
  __shared__ float sp[GMAX][NKEY];
  __shared__ float red[NT / WAVE];
  const AttnWs& w = a.w;
  const int item = blockIdx.x;
  if (item >= w.item_off[a.n_heads]) return;
  const int G = a.group;
  const int4 rec = w.item[item];
  const int h = rec.x, page0 = rec.y, nv = rec.z, cnt = rec.w;
  const float* qf = (const float*)a.q;
  for (int i = threadIdx.x; i < G * D; i += NT) sq[i / D][i % D] = qf[(size_t)h * G * D + i];
  __syncthreads();
  const int t = threadIdx.x;
  const int p = t / PAGE;   // page within the item
  const bool valid = p < cnt && t < nv;
  int64_t slot = 0;
  bool kept = valid;
  if (valid) {
    slot = (int64_t)a.page_ids[page0 + p] * PAGE + t % PAGE;
    if (!LOGITS && a.keep) kept = a.keep[(int64_t)(page0 + p) * PAGE + t % PAGE] != 0;
  }
  const float* krow = (const float*)a.k + slot * D;
  for (int g = 0; g < G; ++g) {
    float z = -INFINITY;
    if (valid) {
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(sq[g][d], krow[d], dot);
      z = dot * a.scale2;
      if (LOGITS) w.logits[((int64_t)(page0 + p) * G + g) * PAGE + t % PAGE] = z;
    }
    sp[g][t] = z;
  }
  __syncthreads();
  auto block_reduce = [&](float v, bool is_max) {
    for (int d = 32; d > 0; d >>= 1) {
      float o = __shfl_xor(v, d, 64);
      v = is_max ? fmaxf(v, o) : v + o;
    }
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < NT / WAVE; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    __syncthreads();
    return r;
  };
  for (int g = 0; g < G; ++g) {
    // kept and dropped keys, each against its own maximum
    const float z = sp[g][t];
    const float Mk = block_reduce(kept ? z : -INFINITY, true);
    const float Md = block_reduce(valid && !kept ? z : -INFINITY, true);
    const float M = kept ? Mk : Md;
    const float pr = (M == -INFINITY || !valid) ? 0.f : exp2f(z - M);
    const float ka = block_reduce(kept ? pr : 0.f, false);
    const float kd = block_reduce(kept ? 0.f : pr, false);
    __syncthreads();
    sp[g][t] = kept ? pr : 0.f;
    if (t == 0) {
      float* st = w.stats + ((size_t)item * G + g) * NST;
      st[0] = Mk;
      st[1] = ka;
      st[2] = kd;
      st[3] = Md;
    }
  }
  __syncthreads();
  if (!LOGITS) {
    const float* vb = (const float*)a.v;
    for (int i = t; i < G * D; i += NT) {
      const int g = i / D, d = i % D;
      float s = 0.f;
      for (int k = 0; k < NKEY; ++k) {
        const float pk = sp[g][k];
        if (pk != 0.f) {
          const int64_t sl = (int64_t)a.page_ids[page0 + k / PAGE] * PAGE + k % PAGE;
          s = fmaf(pk, vb[sl * D + d], s);
        }
      }
      w.acc[(size_t)item * G * D + i] = s;
    }
  }
}


// mass[j] = (1/G) sum_g 2^(z2_gj - lse2_g); NaN in padding slots.
// 64 CSR pages per block, 4 slots per thread.
template <int GM>
__global__ void __launch_bounds__(256) k_mass(const int32_t* __restrict__ page_off, const int32_t* __restrict__ len,
                                              int n_heads, int group, int64_t n_pages, const AttnWs w,
                                              float* __restrict__ mass) {
  __shared__ PageHeads sh;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const int64_t c = c0 + (threadIdx.x >> 2);
  const int j0 = (threadIdx.x & 3) * 4;
  // a page's logits depend only on the page: requested before the block's
  // head search (pages past the pool read nothing)
  float4 zg[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g)
    if (g < group && c < n_pages) zg[g] = *reinterpret_cast<const float4*>(w.logits + (c * group + g) * PAGE + j0);
  const int64_t total = page_off[n_heads];
  if (c0 >= total) return;
  const PageHeads r = block_page_heads(page_off, n_heads, c0, min(c0 + 63, total - 1), &sh);
  if (c >= total) return;
  const int h = r.hf == r.hl ? r.hf : head_in_range(page_off, r, c);
  const int64_t i0 = (c - page_off[h]) * PAGE + j0;
  const int64_t n = len[h];
  const int64_t slot = c * PAGE + j0;
  float o[4] = {qnan(), qnan(), qnan(), qnan()};
  if (i0 < n) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g < group) {
        const float4 z = zg[g];
        const float l2 = w.lse2[(size_t)h * group + g];
        s[0] += exp2f(z.x - l2);
        s[1] += exp2f(z.y - l2);
        s[2] += exp2f(z.z - l2);
        s[3] += exp2f(z.w - l2);
      }
    }
    const float inv = 1.f / (float)group;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i0 + k < n) o[k] = s[k] * inv;
  }
  *reinterpret_cast<float4*>(mass + slot) = make_float4(o[0], o[1], o[2], o[3]);
}


AttnWs carve(const trimkv_cache_t* c, int group, void* ws, bool mass, bool err = false, int64_t slots = -1) {
  WsLayout L = mass ? mass_ws_layout(c, group) : err ? err_ws_layout(c, group) : attn_ws_layout(c, group, slots);
  char* b = (char*)ws;
  AttnWs w;
  w.item_off = (int32_t*)(b + L.off[0]);
  w.item = (int4*)(b + L.off[1]);
  w.stats = (float*)(b + L.off[2]);
  w.acc = (float*)(b + L.off[3]);
  w.acc2 = err ? (float*)(b + L.off[4]) : nullptr;
  w.lse2 = mass ? (float*)(b + L.off[4]) : nullptr;
  w.logits = mass ? (float*)(b + L.off[5]) : nullptr;
  return w;
}

// Waves that the device holds at once for a kernel of NTA threads per block
// (cached per kernel and device).
template <typename K>
int resident_waves(K kernel) {
  struct Entry { const void* k; int dev; int waves; };
  static thread_local Entry cache[16];
  static thread_local int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  for (int i = 0; i < used; ++i)
    if (cache[i].k == (const void*)kernel && cache[i].dev == dev) return cache[i].waves;
  // failed queries fall back to an MI355X's 256 CUs and one block per CU:
  // the split stays correct for any wave count
  int cus = 0, blocks = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, NTA, 0) != hipSuccess) blocks = 1;
  const int wv = std::min(FLAT_WMAX, std::max(1, blocks) * std::max(1, cus) * (NTA / WAVE));
  if (used < 16) cache[used++] = Entry{(const void*)kernel, dev, wv};
  return wv;
}

template <int MODE>
int launch_main(const trimkv_cache_t* c, AttnArgs& a, hipStream_t st) {
  constexpr bool LOGITS = MODE == A_LOGITS;
  const dim3 blk(NT);
  if (c->dtype == TRIMKV_F32) {
    if (MODE == A_ERR || MODE == A_GPLAIN || MODE == A_GMASK) return TRIMKV_EUNSUPPORTED;
    const int64_t T = max_chunks(c, CHA_F32);   // bound on the number of items
    if (c->head_dim == 128) hipLaunchKernelGGL((k_attn_f32<128, LOGITS>), dim3((unsigned)T), blk, 0, st, a);
    else hipLaunchKernelGGL((k_attn_f32<64, LOGITS>), dim3((unsigned)T), blk, 0, st, a);
    return TRIMKV_OK;
  }
  auto go = [&](auto kernel) {
    a.waves = resident_waves(kernel);
    hipLaunchKernelGGL(kernel, dim3((unsigned)(a.waves / (NTA / WAVE))), dim3(NTA), 0, st, a);
  };
  if (c->head_dim == 128) go(k_attn_bf16<128, MODE>);
  else go(k_attn_bf16<64, MODE>);
  return TRIMKV_OK;
}

// Merge launch: one wave per query row.
void launch_merge(const trimkv_cache_t* c, const AttnArgs& a, int with_out, hipStream_t st) {
  const unsigned blocks = (unsigned)(((int64_t)c->n_heads * a.group + NT / WAVE - 1) / (NT / WAVE));
  const bool err = a.w.acc2 != nullptr;
  if (c->head_dim == 128) {
    if (err) hipLaunchKernelGGL((k_attn_merge<128, true>), dim3(blocks), dim3(NT), 0, st, a, with_out);
    else hipLaunchKernelGGL((k_attn_merge<128, false>), dim3(blocks), dim3(NT), 0, st, a, with_out);
  } else {
    if (err) hipLaunchKernelGGL((k_attn_merge<64, true>), dim3(blocks), dim3(NT), 0, st, a, with_out);
    else hipLaunchKernelGGL((k_attn_merge<64, false>), dim3(blocks), dim3(NT), 0, st, a, with_out);
  }
}

// Partial slots: fp32 work items, or flat waves + heads.
int64_t partial_slots(const trimkv_cache_t* c) {
  return c->dtype == TRIMKV_F32 ? max_chunks(c, CHA_F32) : (int64_t)FLAT_WMAX + c->n_heads;
}

}  // namespace

WsLayout attn_ws_layout(const trimkv_cache_t* c, int group, int64_t slots) {
  const int64_t S = slots >= 0 ? slots : partial_slots(c);
  const int64_t T = c->dtype == TRIMKV_F32 ? max_chunks(c, CHA_F32) : 0;
  WsLayout L;
  L.add(((int64_t)c->n_heads + 1) * 4);
  L.add((T + 4) * 16);
  L.add(S * group * NST * 4);
  L.add(S * group * (int64_t)c->head_dim * 4);
  return L;
}

WsLayout err_ws_layout(const trimkv_cache_t* c, int group) {
  WsLayout L = attn_ws_layout(c, group);
  L.add(partial_slots(c) * group * (int64_t)c->head_dim * 4);   // dropped keys' partial outputs
  return L;
}

WsLayout mass_ws_layout(const trimkv_cache_t* c, int group) {
  const int64_t S = partial_slots(c);
  const int64_t T = c->dtype == TRIMKV_F32 ? max_chunks(c, CHA_F32) : 0;
  WsLayout L;
  L.add(((int64_t)c->n_heads + 1) * 4);
  L.add((T + 4) * 16);
  L.add(S * group * NST * 4);
  L.add(0);
  L.add((int64_t)c->n_heads * group * 4);
  L.add((int64_t)group * c->n_pages * PAGE * 4);
  return L;
}

namespace {

// The decode call on a workspace laid out for `slots` partial slots (-1:
// the public layout, sized for the most waves a launch may use).
int decode_attn_on(const trimkv_cache_t* c, const uint8_t* keep, const float* lse_ref, const void* q, int group,
                   float scale, float* out, float* dropped, float* lse_out, void* ws, int64_t slots, hipStream_t st) {
  AttnWs w = carve(c, group, ws, false, false, slots);
  const bool f32 = c->dtype == TRIMKV_F32;
  if (f32)
    hipLaunchKernelGGL(k_attn_prep, dim3(prep_grid(c->n_heads, max_chunks(c, CHA_F32), 2048)), dim3(1024), 0, st,
                       c->page_off, c->len, c->n_heads, CHA_F32, w);
  AttnArgs a{c->page_off, c->page_ids, c->len, c->k, c->v, keep, q, c->n_heads, group, scale * LOG2E,
             CHA_F32, 0, w, lse_ref, out, dropped, lse_out};
  prof_begin(st);
  int rc = keep ? launch_main<A_MASK>(c, a, st) : launch_main<A_PLAIN>(c, a, st);
  prof_end(st);
  if (rc) return rc;
  launch_merge(c, a, 1, st);
  return check_launch();
}

// Address of this device's scratch, looked up once per device (with that
// device current) and kept.
std::mutex g_scratch_mu;
constexpr int SCRATCH_MAX_DEV = 64;
void* g_scratch_ptr[SCRATCH_MAX_DEV] = {};

int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TRIMKV_EHIP;
  if (dev < 0 || dev >= SCRATCH_MAX_DEV) return TRIMKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TRIMKV_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TRIMKV_OK;
}

}  // namespace

int launch_decode_attn(const trimkv_cache_t* c, const uint8_t* keep, const float* lse_ref, const void* q,
                       int group, float scale, float* out, float* dropped, float* lse_out, void* ws,
                       hipStream_t st) {
  return decode_attn_on(c, keep, lse_ref, q, group, scale, out, dropped, lse_out, ws, -1, st);
}

WsLayout attn_evict_ws_layout(const trimkv_cache_t* c, int group) {
  WsLayout L = attn_ws_layout(c, group);
  L.add(c->n_pages * PAGE * 4);   // the eviction's hole lists (a word per CSR slot)
  return L;
}

int launch_decode_attn_evict_tailfill(trimkv_cache_t* c, const uint8_t* keep, const int32_t* kept, const void* q,
                                      int group, float scale, float* out, float* dropped, int reserve,
                                      const int32_t* home_off, const int32_t* home_ids, int32_t* new_off,
                                      int32_t* new_ids, void* ws, hipStream_t st) {
  const int elt = c->dtype == TRIMKV_BF16 ? 2 : 4;
  const int rowb = c->head_dim * elt;
  if (rowb != 128 && rowb != 256 && rowb != 512) return TRIMKV_EUNSUPPORTED;
  AttnWs w = carve(c, group, ws, false, false);
  const WsLayout L = attn_evict_ws_layout(c, group);
  uint32_t* holes = (uint32_t*)((char*)ws + L.off[4]);
  if (c->dtype == TRIMKV_F32)
    hipLaunchKernelGGL(k_attn_prep, dim3(prep_grid(c->n_heads, max_chunks(c, CHA_F32), 2048)), dim3(1024), 0, st,
                       c->page_off, c->len, c->n_heads, CHA_F32, w);
  AttnArgs a{c->page_off, c->page_ids, c->len, c->k, c->v, keep, q, c->n_heads, group, scale * LOG2E,
             CHA_F32, 0, w, nullptr, out, dropped, nullptr};
  prof_begin(st);
  const int rc = launch_main<A_MASK>(c, a, st);
  prof_end(st);
  if (rc) return rc;
  const tf::Args t{c->n_heads, reserve, c->page_off, c->page_ids, c->len, keep, kept, home_off, home_ids, new_off,
                   new_ids, (uint8_t*)c->k, (uint8_t*)c->v, c->meta, holes};
  const int rows_per_block = tf::NT / WAVE;
  const int mb = (int)(((int64_t)c->n_heads * group + rows_per_block - 1) / rows_per_block);
  const dim3 grid((unsigned)(mb + c->n_heads)), blk(tf::NT);
  if (c->head_dim == 128) {
    if (rowb == 256) hipLaunchKernelGGL((k_attn_merge_evict<128, 256>), grid, blk, 0, st, a, t, mb);
    else hipLaunchKernelGGL((k_attn_merge_evict<128, 512>), grid, blk, 0, st, a, t, mb);
  } else {
    if (rowb == 128) hipLaunchKernelGGL((k_attn_merge_evict<64, 128>), grid, blk, 0, st, a, t, mb);
    else hipLaunchKernelGGL((k_attn_merge_evict<64, 256>), grid, blk, 0, st, a, t, mb);
  }
  return check_launch();
}

int64_t noalloc_min_bytes(const trimkv_cache_t* c, int group) {
  const int64_t slots = c->dtype == TRIMKV_F32 ? max_chunks(c, CHA_F32) : (int64_t)c->n_heads + 1;
  return (int64_t)attn_ws_layout(c, group, slots).total;
}

int launch_decode_attn_noalloc(const trimkv_cache_t* c, const uint8_t* keep, const float* lse_ref, const void* q,
                               int group, float scale, float* out, float* dropped, float* lse_out, hipStream_t st) {
  // partial slots: the waves this launch will use (plus one per head), not
  // the most any launch may use, so that the scratch stays small
  int64_t slots = max_chunks(c, CHA_F32);
  if (c->dtype != TRIMKV_F32) {
    int waves;
    if (keep) waves = c->head_dim == 128 ? resident_waves(k_attn_bf16<128, A_MASK>) : resident_waves(k_attn_bf16<64, A_MASK>);
    else waves = c->head_dim == 128 ? resident_waves(k_attn_bf16<128, A_PLAIN>) : resident_waves(k_attn_bf16<64, A_PLAIN>);
    slots = (int64_t)waves + c->n_heads;
  }
  if (attn_ws_layout(c, group, slots).total > (size_t)TRIMKV_NOALLOC_SCRATCH_BYTES) return TRIMKV_EWORKSPACE;
  void* ws = nullptr;
  const int rc = device_scratch(&ws);
  if (rc) return rc;
  return decode_attn_on(c, keep, lse_ref, q, group, scale, out, dropped, lse_out, ws, slots, st);
}

int launch_decode_attn_err(const trimkv_cache_t* c, const uint8_t* keep, const void* q, int group, float scale,
                           float* out, float* dropped, float* mu, float* err, void* ws, hipStream_t st) {
  AttnWs w = carve(c, group, ws, false, true);
  AttnArgs a{c->page_off, c->page_ids, c->len, c->k, c->v, keep, q, c->n_heads, group, scale * LOG2E,
             CHA_F32, 0, w, nullptr, out, dropped, nullptr, mu, err};
  prof_begin(st);
  int rc = launch_main<A_ERR>(c, a, st);
  prof_end(st);
  if (rc) return rc;
  launch_merge(c, a, 1, st);
  return check_launch();
}

int launch_decode_attn_gated(const trimkv_cache_t* c, int n_seg, const int32_t* seg, const int32_t* t,
                             const uint8_t* keep, const void* q, int group, float scale, float* out, float* dropped,
                             float* lse_out, void* ws, hipStream_t st) {
  AttnWs w = carve(c, group, ws, false);
  AttnArgs a{c->page_off, c->page_ids, c->len, c->k, c->v, keep, q, c->n_heads, group, scale * LOG2E,
             CHA_F32, 0, w, nullptr, out, dropped, lse_out, nullptr, nullptr,
             c->meta, seg, t, n_seg};
  prof_begin(st);
  int rc = keep ? launch_main<A_GMASK>(c, a, st) : launch_main<A_GPLAIN>(c, a, st);
  prof_end(st);
  if (rc) return rc;
  launch_merge(c, a, 1, st);
  return check_launch();
}

int launch_attn_mass(const trimkv_cache_t* c, const void* q, int group, float scale, float* mass,
                     float* lse_full, void* ws, hipStream_t st) {
  AttnWs w = carve(c, group, ws, true);
  const bool f32 = c->dtype == TRIMKV_F32;
  if (f32)
    hipLaunchKernelGGL(k_attn_prep, dim3(prep_grid(c->n_heads, max_chunks(c, CHA_F32), 2048)), dim3(1024), 0, st,
                       c->page_off, c->len, c->n_heads, CHA_F32, w);
  AttnArgs a{c->page_off, c->page_ids, c->len, c->k, c->v, nullptr, q, c->n_heads, group, scale * LOG2E,
             CHA_F32, 0, w, nullptr, nullptr, nullptr, lse_full};
  prof_begin(st);
  int rc = launch_main<A_LOGITS>(c, a, st);
  prof_end(st);
  if (rc) return rc;
  launch_merge(c, a, 0, st);
  const int64_t blocks = (c->n_pages + 63) / 64;
  if (group <= 4)
    hipLaunchKernelGGL(k_mass<4>, dim3((unsigned)blocks), dim3(256), 0, st, c->page_off, c->len, c->n_heads, group,
                       c->n_pages, w, mass);
  else if (group <= 8)
    hipLaunchKernelGGL(k_mass<8>, dim3((unsigned)blocks), dim3(256), 0, st, c->page_off, c->len, c->n_heads, group,
                       c->n_pages, w, mass);
  else
    hipLaunchKernelGGL(k_mass<GMAX>, dim3((unsigned)blocks), dim3(256), 0, st, c->page_off, c->len, c->n_heads, group,
                       c->n_pages, w, mass);
  return check_launch();
}

}  // namespace trimkv
