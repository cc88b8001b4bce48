// Exact global top-M per segment over fp32 keys, ties by head ascending, then
// position descending (the more recent entry of a head first).
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
//      device atomics into a per-segment histogram; every block of the next
//      kernel scans the finished histogram of its segment to narrow the
//      prefix (no inter-block waits, no cache flushes inside a kernel);
//   3. one pass over 1024-slot chunks: each chunk keeps key > K*.  When the
//      ties (key == K*) straddle the budget, the segment's heads are taken
//      in order by a per-segment ticket; each counts its ties, obtains the
//      ties of every earlier head by a decoupled look-back (one wave reads 64
//      predecessor words at a time; value and flag share one 64-bit word),
//      and keeps its q most recent ties, q = clamp(need - earlier ties, 0,
//      ties), found by a radix selection over their positions (read from the
//      cache's metadata, so slot order does not matter).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "ln_cr.h"

namespace trimkv {

namespace {

constexpr int CP = 64;          // pages per chunk
constexpr int CS = CP * PAGE;   // slots per chunk
constexpr int NT = 1024;        // threads per histogram and decision block
constexpr int GT = CS / 4;      // threads per chunk (4 slots each)
constexpr int CG = NT / GT;     // chunks in flight per block: thread t works on chunk t / GT of each round
constexpr int CPB = 32;         // chunks per block (most)
static_assert(CPB % CG == 0 && CPB <= NT, "chunk rounds");
// Histogram layout per segment and pass: HC copies (block b adds into copy
// b % HC), 32 words apart, so that each copy's bins take only a quarter of
// the device atomics; readers sum the copies.
constexpr int HC = 4;
__host__ __device__ constexpr int copy_words(int nb) { return nb + 32; }
constexpr int HIST_WORDS = HC * (2 * copy_words(2048) + copy_words(1024));
constexpr uint32_t SPIN_LIMIT = 1u << 26;

constexpr unsigned N_CU = 256;  // compute units of an MI355X

enum { MODE_NORMAL = 0, MODE_ALL = 1, MODE_NONE = 2 };

struct SegState {
  int64_t remaining;  // 1-based rank of the target key among keys matching `prefix`
  int64_t n_valid;
  int64_t ties;       // keys in the located bin (after the last pass: keys equal to K*)
  uint32_t prefix;
  int32_t mode;
  int32_t chunk_begin, chunk_end;
};

// chunk metadata: x = head, y = segment, z = first CSR page,
// w = valid entries | (pages of the chunk << 16)
struct SelWs {
  int32_t* chunk_off;   // [H + 1]
  int4* meta;           // [Tmax]
  SegState* seg;        // [4][n_seg]: state before radix pass 0, 1, 2 and the final state
  int n_seg;
  uint32_t* hist;       // [n_seg][HIST_WORDS]
  uint64_t* look;       // [Tmax > n_heads] tie look-back word of each head: 0 | flag<<62 | value
  uint32_t* ticket;     // [2 + n_seg]: [2 + s] ticket of segment s
  int32_t* status;      // caller's failure counter (nullable): +1 per timed-out look-back wait
  double* part;         // [Tmax]
};

constexpr uint64_t LB_AGG = 1ull << 62, LB_PREFIX = 2ull << 62, LB_VAL = (1ull << 62) - 1;

__device__ __forceinline__ int pass_bits(int pass) { return pass == 2 ? 10 : 11; }
__device__ __forceinline__ uint32_t* pass_hist(const SelWs& w, int s, int pass) {
  return w.hist + (size_t)s * HIST_WORDS + (pass == 0 ? 0 : pass == 1 ? 1 : 2) * HC * copy_words(2048);
}

// The step's new entries, when the selection also appends them (one per
// head, at slot len[h] with position t_s - 1 of the head's segment s, as
// trimkv_append writes them); k_new == null: no append.
struct AppendSrc {
  const uint8_t* k_new;    // [n_heads][row bytes]
  const uint8_t* v_new;
  const float* beta_new;   // [n_heads]
  uint8_t* k;              // the cache's K and V planes, rows of `rowb` bytes
  uint8_t* v;
  uint32_t* meta;          // [n_pages][2][16]: ln beta bits, positions
  const int32_t* page_ids;
  const int32_t* t;        // decode step of each segment
  int rowb;                // bytes per K or V row
  int elt;                 // bytes per element (2: bf16, 4: fp32)
  int32_t* status;         // +1 per head without a free slot (nullable)
};

// One wave's append of head h, as trimkv_append writes it: entry len[h]
// takes the new row, ln beta and position t_s - 1 (s the head's segment); a
// head without a free slot is counted.  Beta and the step are requested
// before the length is known.
__device__ __forceinline__ void append_head(int h, const int32_t* __restrict__ page_off, const int32_t* len,
                                            int n_seg, const int32_t* __restrict__ seg_hb, const AppendSrc& ap) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int s = upper_index(seg_hb, n_seg + 1, h);
  const float b = ap.beta_new[h];
  const int tt = ap.t[s];
  const int n = len[h];
  const int64_t cap = (int64_t)(page_off[h + 1] - page_off[h]) * PAGE;
  if (n >= cap) {
    if (lane == 0 && ap.status) atomicAdd(ap.status, 1);
    return;
  }
  const int64_t page = ap.page_ids[page_off[h] + n / PAGE];
  const int64_t slot = page * PAGE + n % PAGE;
  // element-wise, as trimkv_append copies (inputs need only element alignment)
  if (ap.elt == 2) {
    const uint16_t* kn = reinterpret_cast<const uint16_t*>(ap.k_new) + (int64_t)h * (ap.rowb / 2);
    const uint16_t* vn = reinterpret_cast<const uint16_t*>(ap.v_new) + (int64_t)h * (ap.rowb / 2);
    uint16_t* kd = reinterpret_cast<uint16_t*>(ap.k) + slot * (ap.rowb / 2);
    uint16_t* vd = reinterpret_cast<uint16_t*>(ap.v) + slot * (ap.rowb / 2);
    for (int d = lane; d < ap.rowb / 2; d += WAVE) {
      kd[d] = kn[d];
      vd[d] = vn[d];
    }
  } else {
    const uint32_t* kn = reinterpret_cast<const uint32_t*>(ap.k_new) + (int64_t)h * (ap.rowb / 4);
    const uint32_t* vn = reinterpret_cast<const uint32_t*>(ap.v_new) + (int64_t)h * (ap.rowb / 4);
    uint32_t* kd = reinterpret_cast<uint32_t*>(ap.k) + slot * (ap.rowb / 4);
    uint32_t* vd = reinterpret_cast<uint32_t*>(ap.v) + slot * (ap.rowb / 4);
    for (int d = lane; d < ap.rowb / 4; d += WAVE) {
      kd[d] = kn[d];
      vd[d] = vn[d];
    }
  }
  if (lane == 0) {
    ap.meta[page * (2 * PAGE) + n % PAGE] = __float_as_uint(ln_f32_cr(b));
    ap.meta[page * (2 * PAGE) + PAGE + n % PAGE] = (uint32_t)(tt - 1);
  }
}

// ---------------------------------------------------------------------------
// prep: chunk list + metadata + segment state (block 0); the first n_prep
// blocks clear histograms, kept[] and look-back words.  With an append, the
// chunk list counts one more entry in every head with a free slot, and the
// entries themselves are written by further blocks, one wave per head,
// beside the prep blocks (neither reads what the other writes); the lengths
// are raised by the first histogram pass, which no selection kernel before
// it needs.  With more heads than the LDS list holds, one block does
// everything in order: the appends, the lengths, then the list.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_sel_prep(const int32_t* __restrict__ page_off,
                                                   int32_t* __restrict__ len, int n_heads, int n_seg,
                                                   const int32_t* __restrict__ seg_hb,
                                                   const int64_t* __restrict__ budget, int64_t tmax, SelWs w,
                                                   int32_t* __restrict__ kept, AppendSrc ap, int n_prep) {
  const bool grow = ap.k_new != nullptr;
  constexpr int WPB = 1024 / WAVE;
  if (grow && (int)blockIdx.x >= n_prep) {   // append blocks (block-uniform; no barriers)
    const int h = (blockIdx.x - n_prep) * WPB + __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    if (h < n_heads) append_head(h, page_off, len, n_seg, seg_hb, ap);
    return;
  }
  const size_t gtid = (size_t)blockIdx.x * 1024 + threadIdx.x, gstride = (size_t)n_prep * 1024;
  for (size_t i = gtid; i < (size_t)n_seg * HIST_WORDS; i += gstride) w.hist[i] = 0u;
  for (size_t i = gtid; i < (size_t)tmax; i += gstride) w.look[i] = 0ull;
  for (size_t i = gtid; i < (size_t)n_heads; i += gstride) kept[i] = 0;
  for (size_t i = gtid; i < (size_t)n_seg + 2; i += gstride) w.ticket[i] = 0u;
  __shared__ int64_t tmp[1024 / WAVE + 1];
  __shared__ PrepLDS L;
  if (grow && n_heads > PREP_HMAX) {   // one block (n_prep = 1, no append blocks)
    for (int h = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE); h < n_heads; h += WPB)
      append_head(h, page_off, len, n_seg, seg_hb, ap);
    __syncthreads();   // every wave has read its heads' old lengths
    for (int h = threadIdx.x; h < n_heads; h += 1024) {
      const int n = len[h];
      if ((int64_t)n < (int64_t)(page_off[h + 1] - page_off[h]) * PAGE) len[h] = n + 1;
    }
    __syncthreads();
  }
  const int T = prep_chunks<1024>(page_off, len, n_heads, CP, L, tmp, w.chunk_off,
                                  grow && n_heads <= PREP_HMAX);
  const bool single = n_heads > PREP_HMAX;   // then one block and a global scan
  if (blockIdx.x == 0) {
    for (int s = threadIdx.x; s < n_seg; s += 1024) {
      const int hb = seg_hb[s], he = seg_hb[s + 1];
      SegState st;
      st.remaining = budget[s];
      st.n_valid = 0;
      st.ties = 0;
      st.prefix = 0u;
      st.chunk_begin = single ? w.chunk_off[hb] : L.off[hb];
      st.chunk_end = single ? w.chunk_off[he] : L.off[he];
      st.mode = (budget[s] <= 0 || st.chunk_begin == st.chunk_end) ? MODE_NONE : MODE_NORMAL;
      w.seg[s] = st;
    }
  }
  for (int c = blockIdx.x * 1024 + threadIdx.x; c < T; c += n_prep * 1024) {
    const ChunkInfo ci = chunk_info(L, w.chunk_off, page_off, len, n_heads, CP, c);
    const int s = upper_index(seg_hb, n_seg + 1, ci.h);
    w.meta[c] = make_int4(ci.h, s, ci.page0, ci.nv | (ci.npg << 16));
  }
}

// State of segment s after radix pass `pass`, computed by a whole block from
// the finished histogram of that pass (every thread gets the result); the
// block holding the segment's first chunk stores it as the state before the
// next pass.  The histogram words are loaded together with the state.
__device__ SegState state_after(const SelWs& w, int s, int pass, int cpb) {
  __shared__ int64_t tmp[NT / WAVE + 1];
  __shared__ uint32_t sh_prefix;
  __shared__ int64_t sh_rem, sh_ties;
  const int nb = pass == 2 ? 1024 : 2048;
  const int per = nb / NT;  // 2 or 1
  const uint32_t* g = pass_hist(w, s, pass);
  uint32_t c[2] = {0u, 0u};
  for (int k = 0; k < per; ++k) {
    uint32_t v = 0;
#pragma unroll
    for (int r = 0; r < HC; ++r) v += g[r * copy_words(nb) + threadIdx.x * per + k];
    c[k] = v;
  }
  SegState st = w.seg[(size_t)pass * w.n_seg + s];
  const int64_t tsum = (int64_t)c[0] + c[1];
  int64_t total;
  const int64_t ex = block_exclusive_scan<NT>(tsum, tmp, &total);   // a histogram not filled reads zero
  if (st.mode == MODE_NORMAL) {
    const int64_t above = total - ex - tsum;  // keys in bins of higher threads
    if (pass == 0) {
      st.n_valid = total;
      if (st.remaining >= total) st.mode = total == 0 ? MODE_NONE : MODE_ALL;
    }
    if (st.mode == MODE_NORMAL) {
      const int64_t r = st.remaining;
      if (above < r && r <= above + tsum) {
        int64_t cum = above;
        for (int k = per - 1; k >= 0; --k) {
          if (cum + c[k] >= r) {
            sh_rem = r - cum;
            sh_ties = c[k];
            sh_prefix = (st.prefix << pass_bits(pass)) | (uint32_t)(threadIdx.x * per + k);
            break;
          }
          cum += c[k];
        }
      }
      lds_barrier();
      st.remaining = sh_rem;
      st.prefix = sh_prefix;
      st.ties = sh_ties;
      lds_barrier();
    }
  }
  if (threadIdx.x == 0 && (int)blockIdx.x == st.chunk_begin / cpb) w.seg[(size_t)(pass + 1) * w.n_seg + s] = st;
  return st;
}

// Chunk metadata from LDS, in scalar registers: every wave works on one
// chunk per round.
__device__ __forceinline__ int4 umeta(const int4* sm, int k) {
  const int4 m = sm[k];
  return make_int4(__builtin_amdgcn_readfirstlane(m.x), __builtin_amdgcn_readfirstlane(m.y),
                   __builtin_amdgcn_readfirstlane(m.z), __builtin_amdgcn_readfirstlane(m.w));
}

// Smallest fp32 value whose key is >= K, for 1 <= K <= 2^32: a score s has
// key(s) >= K exactly when s is not NaN and s >= key_floor(K) (the float
// comparison also equates -0.0 and +0.0, as the keys do).  NaN when no value
// qualifies.  Lets later passes classify scores with two float comparisons
// and convert to keys only the few that fall inside the located bin.
__device__ __forceinline__ float key_floor(uint64_t K) {
  if (K <= 0x007FFFFFull) return -INFINITY;                              // at or below the key of -inf
  if (K < 0x80000000ull) return __uint_as_float(~(uint32_t)K);           // negative values, -0.0
  if (K <= 0xFF800000ull) return __uint_as_float((uint32_t)K & 0x7FFFFFFFu);   // +0.0 .. +inf
  return qnan();
}

// Marks values as changed at this point so that quantities derived from
// them are computed where used rather than hoisted out of the segment-run
// loop (32 extra live registers).  Emits no instruction.
template <typename T, int R>
__device__ __forceinline__ void opaque(T (&x)[R][4]) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(x[r][j]));
}

// Inputs of the retention score, for the pass that forms the scores itself.
struct ScoreSrc {
  const int32_t* page_ids;   // physical page of each CSR page
  const uint32_t* meta;      // [n_pages][2][16]: ln beta bits, positions
  const int32_t* t;          // decode step of each segment
  float* score;              // CSR plane, written
  int32_t* grow_len;         // with an append planned by prep: the lengths to raise (block 0), else null
  const int32_t* page_off;
};

// Block b histograms chunks [b*CPB, b*CPB + CPB), CG chunks per round
// (GT threads of 4 slots per chunk): metadata first, then every key load in
// flight while the previous pass's bin is located.  The block's histogram is
// merged into the segment's once per segment run, so the number of device
// atomics per bin falls with the number of chunks per block.
// FUSED (pass 0 only): the retention score of every slot is formed here from
// its page's ln beta and position, fp32(t - pos) * ln beta with one rounding
// exactly as trimkv_score forms it, written to the CSR score plane (NaN in
// padding slots) and histogrammed in the same pass.
template <int PASS, int HB, bool FUSED = false>
__global__ void __launch_bounds__(NT) k_sel_hist(int n_heads, const float* __restrict__ score, SelWs w,
                                                 ScoreSrc src) {
  static_assert(!FUSED || PASS == 0, "scores are formed in the first pass");
  constexpr int RND = HB / CG;   // rounds of CG chunks
  static_assert(HB % CG == 0 && HB <= CPB, "chunk rounds");
  constexpr int NB = PASS == 2 ? 1024 : 2048;
  constexpr int SH = PASS == 0 ? 32 : PASS == 1 ? 21 : 10;   // key bits below the known prefix
  constexpr int BSH = SH - (PASS == 2 ? 10 : 11);               // shift of this pass's bin
  __shared__ uint32_t lh[NB];
  __shared__ int4 sm[HB];
  const int c0 = blockIdx.x * HB;
  if (PASS == 0 && src.grow_len && blockIdx.x == 0) {
    // the append planned by prep: every head with a free slot grows by one
    for (int h = threadIdx.x; h < n_heads; h += NT) {
      const int n = src.grow_len[h];
      if ((int64_t)n < (int64_t)(src.page_off[h + 1] - src.page_off[h]) * PAGE) src.grow_len[h] = n + 1;
    }
  }
  int4 mv = make_int4(0, 0, 0, 0);
  if (threadIdx.x < HB) mv = w.meta[c0 + threadIdx.x];   // padded by CPB >= HB entries
  const int T = w.chunk_off[n_heads];
  if (c0 >= T) return;
  const int nc = min(HB, T - c0);
  if (threadIdx.x < nc) sm[threadIdx.x] = mv;
  for (int b = threadIdx.x; b < NB; b += NT) lh[b] = 0u;
  lds_barrier();
  const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / GT), i0 = (threadIdx.x % GT) * 4;
  float a[RND][4];
  SegState st0;
  {
    float4 kv[RND];
    if constexpr (FUSED) {
      // page ids, then every page's ln beta and positions in flight at once
      int pid[RND];
#pragma unroll
      for (int r = 0; r < RND; ++r) {
        const int k = r * CG + grp;
        const int4 m = umeta(sm, k);
        pid[r] = (k < nc && i0 < (m.w >> 16) * PAGE) ? src.page_ids[m.z + i0 / PAGE] : -1;
      }
      float4 lb[RND];
      int4 ps[RND];
#pragma unroll
      for (int r = 0; r < RND; ++r) {
        if (pid[r] >= 0) {
          const uint32_t* mp = src.meta + (int64_t)pid[r] * (2 * PAGE) + (i0 % PAGE);
          lb[r] = *reinterpret_cast<const float4*>(mp);
          ps[r] = *reinterpret_cast<const int4*>(mp + PAGE);
        }
      }
#pragma unroll
      for (int r = 0; r < RND; ++r) {
        const int k = r * CG + grp;
        const int4 m = umeta(sm, k);
        kv[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (pid[r] >= 0) {
          const int nv = m.w & 0xFFFF;
          const int tt = src.t[m.y];
          float4 o = make_float4(qnan(), qnan(), qnan(), qnan());
          if (i0 < nv) o.x = __fmul_rn((float)(tt - ps[r].x), lb[r].x);
          if (i0 + 1 < nv) o.y = __fmul_rn((float)(tt - ps[r].y), lb[r].y);
          if (i0 + 2 < nv) o.z = __fmul_rn((float)(tt - ps[r].z), lb[r].z);
          if (i0 + 3 < nv) o.w = __fmul_rn((float)(tt - ps[r].w), lb[r].w);
          *reinterpret_cast<float4*>(src.score + (int64_t)m.z * PAGE + i0) = o;
          kv[r] = o;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < RND; ++r) {
        const int k = r * CG + grp;
        const int4 m = umeta(sm, k);
        kv[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (k < nc && i0 < (m.w & 0xFFFF)) kv[r] = *reinterpret_cast<const float4*>(score + (int64_t)m.z * PAGE + i0);
      }
    }
    // state for the first segment run while the scores are in flight
    if (PASS > 0) st0 = state_after(w, sm[0].y, PASS - 1, HB);
#pragma unroll
    for (int r = 0; r < RND; ++r) {
      a[r][0] = kv[r].x;
      a[r][1] = kv[r].y;
      a[r][2] = kv[r].z;
      a[r][3] = kv[r].w;
    }
  }
  int i = 0;
  while (i < nc) {
    // run of consecutive chunks of one segment (block-uniform)
    const int s = sm[i].y;
    int e = i + 1;
    while (e < nc && sm[e].y == s) ++e;
    SegState st;
    if (PASS == 0) st = w.seg[s];
    else st = i == 0 ? st0 : state_after(w, s, PASS - 1, HB);
    opaque(a);
    if (st.mode == MODE_NORMAL) {
      const uint32_t pre = st.prefix;
      // keys of the located bin: [lo, hi); lo == 0 holds NaN, which no float
      // comparison finds, so that bin is classified on the keys themselves
      const uint64_t lo = PASS == 0 ? 0 : (uint64_t)pre << SH, hi = PASS == 0 ? 0 : (uint64_t)(pre + 1) << SH;
      const bool by_key = PASS == 0 || lo == 0;
      const float flo = key_floor(lo), fhi = key_floor(hi);
      // one loop per classification, chosen once per run (block-uniform)
      auto count = [&](auto exact) {
#pragma unroll
        for (int r = 0; r < RND; ++r) {
          const int k = r * CG + grp;
          if (k >= i && k < e) {
            const int nv = umeta(sm, k).w & 0xFFFF;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              if (i0 + j < nv) {
                bool in;
                if constexpr (decltype(exact)::value) {
                  if constexpr (PASS == 0) in = true;   // no prefix yet: every valid key
                  else in = (score_key(a[r][j]) >> SH) == pre;
                } else {
                  in = a[r][j] >= flo && !(a[r][j] >= fhi);
                }
                if (in) atomicAdd(&lh[(score_key(a[r][j]) >> BSH) & (NB - 1)], 1u);
              }
            }
          }
        }
      };
      if (by_key) count(std::true_type{});
      else count(std::false_type{});
      lds_barrier();
      uint32_t* g = pass_hist(w, s, PASS) + (blockIdx.x % HC) * copy_words(NB);
      for (int b = threadIdx.x; b < NB; b += NT) {
        const uint32_t v = lh[b];
        lh[b] = 0u;
        if (v) atomicAdd(g + b, v);
      }
      lds_barrier();
    }
    i = e;
  }
}

__device__ __forceinline__ double block_sum_f64(double v, double* tmpd) {
  // fixed-order tree: xor butterfly in each wave, then waves in order
  for (int d = WAVE / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, WAVE);
  const int wid = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) tmpd[wid] = v;
  lds_barrier();
  double r = 0.0;
  if (threadIdx.x == 0)
    for (int i = 0; i < NT / WAVE; ++i) r += tmpd[i];
  lds_barrier();
  return r;
}

// The block's sum in every thread.
__device__ __forceinline__ int block_sum_all_i32(int v, int* red) {
  for (int d = WAVE / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, WAVE);
  if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = v;
  lds_barrier();
  int r = 0;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) r += red[i];
  lds_barrier();
  return r;
}

__device__ __forceinline__ int block_sum_i32(int v, int* red) {
  for (int d = WAVE / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, WAVE);
  if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = v;
  lds_barrier();
  int r = 0;
  if (threadIdx.x == 0)
    for (int i = 0; i < NT / WAVE; ++i) r += red[i];
  lds_barrier();
  return r;   // valid in thread 0
}

// Keep bits of four consecutive slots (bit j: slot i0 + j) under state st:
// gtm marks key > K*, eqm key == K* (K* = st.prefix after the last pass),
// decided on the scores with K*'s float bounds.
__device__ __forceinline__ void classify(const SegState& st, const float (&a)[4], int i0, int nv, uint32_t& gtm,
                                         uint32_t& eqm) {
  gtm = 0;
  eqm = 0;
  if (st.mode == MODE_NORMAL) {
    const uint32_t ks = st.prefix;
    if (ks != 0u) {
      const float fa = key_floor((uint64_t)ks + 1), fe = key_floor(ks);   // fe: the value whose key is K*
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (i0 + j < nv) {
          gtm |= (uint32_t)(a[j] >= fa) << j;
          eqm |= (uint32_t)(a[j] == fe) << j;
        }
      }
    } else {   // K* is the key of NaN, below every other score
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (i0 + j < nv) {
          const bool nan = a[j] != a[j];
          gtm |= (uint32_t)!nan << j;
          eqm |= (uint32_t)nan << j;
        }
      }
    }
  } else if (st.mode == MODE_ALL) {
#pragma unroll
    for (int j = 0; j < 4; ++j) gtm |= (uint32_t)(i0 + j < nv) << j;
  }
}

__device__ __forceinline__ uint32_t keep_word(uint32_t km) {
  return (km & 1u) | ((km & 2u) << 7) | ((km & 4u) << 14) | ((km & 8u) << 21);
}

// ---------------------------------------------------------------------------
// decide: block b handles chunk positions b*CB .. b*CB + CB - 1.  The state
// after the last radix pass is computed once per segment run of the block.
// In the common case every key equal to K* is kept and chunks are
// independent: keep words, then one kept-count atomic per head run.  When
// the ties straddle the budget (more keys equal K* than `need`), the heads
// of that segment are processed in the order of a per-segment ticket, one
// head per ticket and block, with a decoupled look-back for the ties of
// earlier heads; a ticket is taken only when its head is processed, so
// every head a block waits for belongs to a block that is already running.
// Optional per-chunk kept-score sums (fixed-order trees).
// ---------------------------------------------------------------------------
template <int CB>
__global__ void __launch_bounds__(NT) k_sel_decide(int n_heads, const float* __restrict__ score, SelWs w,
                                                   uint8_t* __restrict__ keep, int32_t* __restrict__ kept,
                                                   int want_sum, const int32_t* __restrict__ page_ids,
                                                   const uint32_t* __restrict__ meta) {
  constexpr int RNDB = CB / CG;   // rounds of CG chunks
  static_assert(CB % CG == 0 && CB <= CPB, "chunk rounds");
  __shared__ double tmpd[NT / WAVE];
  __shared__ double tmps[RNDB][NT / WAVE];   // per-round wave sums of kept scores
  __shared__ int cnt[RNDB][NT / WAVE];        // per-round wave counts of kept slots
  __shared__ int red[NT / WAVE];
  __shared__ int sh_c;
  __shared__ int64_t sh_excl;
  __shared__ uint32_t lhist[256];   // ranked ties: histogram of position bytes
  __shared__ uint32_t sh_pre;
  __shared__ int64_t sh_rem;
  __shared__ int4 sm[CB];
  const int c0 = blockIdx.x * CB;
  int4 mv = make_int4(0, 0, 0, 0);
  if (threadIdx.x < CB) mv = w.meta[c0 + threadIdx.x];   // padded by CPB >= CB entries
  const int T = w.chunk_off[n_heads];
  if (c0 >= T) return;
  const int nc = min(CB, T - c0);
  if (threadIdx.x < nc) sm[threadIdx.x] = mv;
  lds_barrier();
  const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
  const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / GT), i0 = (threadIdx.x % GT) * 4;
  // scores of the block's own chunk positions, all loads in flight at once
  float ka[RNDB][4];
  SegState st0;
  {
    float4 kv[RNDB];
#pragma unroll
    for (int r = 0; r < RNDB; ++r) {
      const int k = r * CG + grp;
      const int4 m = umeta(sm, k);
      kv[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < nc && i0 < (m.w & 0xFFFF)) kv[r] = *reinterpret_cast<const float4*>(score + (int64_t)m.z * PAGE + i0);
    }
    // state for the first segment run while the scores are in flight
    st0 = state_after(w, sm[0].y, 2, CB);
#pragma unroll
    for (int r = 0; r < RNDB; ++r) {
      ka[r][0] = kv[r].x;
      ka[r][1] = kv[r].y;
      ka[r][2] = kv[r].z;
      ka[r][3] = kv[r].w;
    }
  }
  int i = 0;
  while (i < nc) {
    const int sg = sm[i].y;
    int e = i + 1;
    while (e < nc && sm[e].y == sg) ++e;
    const SegState st = i == 0 ? st0 : state_after(w, sg, 2, CB);
    opaque(ka);
    const bool ranked = st.mode == MODE_NORMAL && st.ties > st.remaining;
    if (!ranked) {
      // every tie is kept: key >= K*, i.e. (K* above the key of NaN) one
      // comparison with the smallest value whose key is K*
      uint32_t kmr[RNDB];
      auto mark = [&](auto cmp_only) {
#pragma unroll
        for (int r = 0; r < RNDB; ++r) {
          const int k = r * CG + grp;
          kmr[r] = 0;
          if (k >= i && k < e) {
            const int4 m = umeta(sm, k);
            const int nv = m.w & 0xFFFF;
            if constexpr (decltype(cmp_only)::value) {
              const float fe = key_floor(st.prefix);
#pragma unroll
              for (int j = 0; j < 4; ++j) kmr[r] |= (uint32_t)(i0 + j < nv && ka[r][j] >= fe) << j;
            } else {
              uint32_t gtm, eqm;
              classify(st, ka[r], i0, nv, gtm, eqm);
              kmr[r] = gtm | eqm;
            }
            if (i0 < (m.w >> 16) * PAGE)
              *reinterpret_cast<uint32_t*>(keep + (int64_t)m.z * PAGE + i0) = keep_word(kmr[r]);
          }
        }
      };
      if (st.mode == MODE_NORMAL && st.prefix != 0u) mark(std::true_type{});
      else mark(std::false_type{});
      // kept entries per head, one atomic per head run: a run of one head
      // takes one block sum; a run over several heads (short heads) stages
      // every round's per-wave counts and takes one barrier in all, instead
      // of a block sum per head (measured both ways: each form is faster in
      // its own case)
      if (sm[i].x == sm[e - 1].x) {   // block-uniform
        int n = 0;
#pragma unroll
        for (int r = 0; r < RNDB; ++r) {
          const int k = r * CG + grp;
          if (k >= i && k < e) n += __popc(kmr[r]);
        }
        n = block_sum_i32(n, red);
        if (threadIdx.x == 0 && n) atomicAdd(kept + sm[i].x, n);
      } else {
#pragma unroll
        for (int r = 0; r < RNDB; ++r) {
          const int k = r * CG + grp;
          int n = (k >= i && k < e) ? __popc(kmr[r]) : 0;
          for (int d = WAVE / 2; d > 0; d >>= 1) n += __shfl_xor(n, d, WAVE);
          if (lane == 0) cnt[r][wid] = n;
        }
        lds_barrier();
        if (threadIdx.x == 0) {
          int j = i;
          while (j < e) {
            const int h = sm[j].x;
            int n = 0;
            for (; j < e && sm[j].x == h; ++j)   // chunk j = round j / CG, group j % CG
              for (int q = 0; q < GT / WAVE; ++q) n += cnt[j / CG][(j % CG) * (GT / WAVE) + q];
            if (n) atomicAdd(kept + h, n);
          }
        }
        lds_barrier();   // cnt is written again by the block's next segment run
      }
      if (want_sum) {
        // every round's wave sums first, then one barrier; each chunk's sum
        // then adds its waves' sums in the same fixed order as before
#pragma unroll
        for (int r = 0; r < RNDB; ++r) {
          const int k = r * CG + grp;
          const bool mine = k >= i && k < e;
          double sum = 0.0;
          if (mine) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (kmr[r] & (1u << q)) sum += (double)ka[r][q];
          }
          for (int d = WAVE / 2; d > 0; d >>= 1) sum += __shfl_xor(sum, d, WAVE);
          if (lane == 0) tmps[r][wid] = sum;
        }
        lds_barrier();
        if (threadIdx.x % GT == 0) {
#pragma unroll
          for (int r = 0; r < RNDB; ++r) {
            const int k = r * CG + grp;
            if (k >= i && k < e) {
              double t = 0.0;
              for (int q = 0; q < GT / WAVE; ++q) t += tmps[r][grp * (GT / WAVE) + q];
              w.part[c0 + k] = t;
            }
          }
        }
        lds_barrier();   // tmps is written again by the block's next segment run
      }
    } else {
      // Ties straddle the budget: they rank by head ascending, then position
      // descending.  Heads are taken in the order of a per-segment ticket,
      // one head per ticket and block: the block counts the head's keys above
      // K* and its ties, obtains the ties of every earlier head by a
      // decoupled look-back over the tickets, keeps the head's q most recent
      // ties (a radix selection on their positions when 0 < q < ties), then
      // writes the head's keep bytes.  A ticket is taken only when its head
      // is processed, so every head a block waits for belongs to a block
      // that is already running.  Slot order never matters here, so caches
      // whose slots are not in position order rank the same.
      // Control flow of this loop stays wave-uniform at both ends (the ticket
      // is taken and the head's count stored by the whole of wave 0, never
      // under a one-thread branch): with one-thread branches at both ends
      // the compiler threaded them into a nested loop whose inner back edge,
      // taken by every lane but thread 0, re-read the previous ticket, so
      // those lanes never left the loop.
      // look-back words are indexed by head (heads of different segments are
      // disjoint; a head without pages has no chunk but still takes a ticket)
      const int cb = st.chunk_begin;
      const int h_first = __builtin_amdgcn_readfirstlane(w.meta[cb].x);
      const int n_th = __builtin_amdgcn_readfirstlane(w.meta[st.chunk_end - 1].x) - h_first + 1;
      const int wave0 = __builtin_amdgcn_readfirstlane(wid) == 0;
      const float f_gt = key_floor((uint64_t)st.prefix + 1), f_eq = key_floor(st.prefix);
      const bool nan_tie = st.prefix == 0u;   // K* is the key of NaN
      auto tie_of = [&](float x, bool& gt, bool& eq) {
        if (nan_tie) {
          gt = x == x;
          eq = !gt;
        } else {
          gt = x >= f_gt;
          eq = x == f_eq;
        }
      };
      while (true) {
        if (wave0) {
          // lane 0 adds 1, the others 0: lane 0's old value is the ticket
          const uint32_t v = atomicAdd(w.ticket + 2 + sg, lane == 0 ? 1u : 0u);
          sh_c = __builtin_amdgcn_readfirstlane((int)v);
        }
        lds_barrier();
        const int t = __builtin_amdgcn_readfirstlane(sh_c);
        lds_barrier();   // every thread has read sh_c
        if (t >= n_th) break;
        const int h = h_first + t;
        const int ch0 = w.chunk_off[h], ch1 = w.chunk_off[h + 1];
        // 1. ties of the head (one slot per thread per chunk)
        int n_eq = 0;
        for (int c = ch0; c < ch1; ++c) {
          const int4 m = w.meta[c];
          const bool valid = (int)threadIdx.x < (m.w & 0xFFFF);
          if (valid) {
            bool gt, eq;
            tie_of(score[(int64_t)m.z * PAGE + threadIdx.x], gt, eq);
            n_eq += eq;
          }
        }
        const int64_t eq_h = __builtin_amdgcn_readfirstlane(block_sum_all_i32(n_eq, red));   // < 2^31 (one head)
        // 2. ties of the earlier heads of the segment (look-back over tickets)
        if (wave0) {
          int64_t excl = 0;
          if (t != 0) {
            if (lane == 0)
              __hip_atomic_store(w.look + h, LB_AGG | (uint64_t)eq_h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int base = t - 1;   // window: tickets base, base-1, ..., base-63
            uint32_t spins = 0;
            while (true) {
              const int jj = base - lane;
              // before the segment's first ticket: a zero prefix
              const uint64_t v = jj >= 0 ? __hip_atomic_load(w.look + h_first + jj, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                         : LB_PREFIX;
              const uint64_t zm = __ballot(v == 0ull);
              const uint64_t pm = __ballot((v & ~LB_VAL) == LB_PREFIX);
              const int first = pm ? __ffsll((long long)pm) - 1 : WAVE;   // nearest prefix in the window
              const uint64_t need = first == WAVE ? ~0ull : ((2ull << first) - 1ull);
              if (zm & need) {  // a predecessor has not published yet
                if (++spins > SPIN_LIMIT) {  // never expected; keeps every wave finite, reported
                  if (lane == 0 && w.status) atomicAdd(w.status, 1);
                  break;
                }
                __builtin_amdgcn_s_sleep(1);
                continue;
              }
              int64_t val = (lane <= first) ? (int64_t)(v & LB_VAL) : 0;
              for (int d = WAVE / 2; d > 0; d >>= 1) val += __shfl_xor(val, d, WAVE);
              excl += val;
              if (pm) break;
              base -= WAVE;
            }
          }
          if (lane == 0) {
            __hip_atomic_store(w.look + h, LB_PREFIX | (uint64_t)(excl + eq_h), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            sh_excl = excl;
          }
        }
        lds_barrier();
        // ties of this head kept (0 .. eq_h)
        const int64_t q = __builtin_amdgcn_readfirstlane((int)min(max(st.remaining - sh_excl, (int64_t)0), eq_h));
        lds_barrier();
        // 3. q < ties: the q-th largest position among the head's ties
        //    (positions are distinct within a head), by four 8-bit passes
        uint32_t pstar = 0u;
        if (q > 0 && q < eq_h) {
          int64_t rem = q;
          for (int pass = 0; pass < 4; ++pass) {
            const int sh = 24 - 8 * pass;
            if (threadIdx.x < 256) lhist[threadIdx.x] = 0u;
            lds_barrier();
            for (int c = ch0; c < ch1; ++c) {
              const int4 m = w.meta[c];
              if ((int)threadIdx.x < (m.w & 0xFFFF)) {
                bool gt, eq;
                tie_of(score[(int64_t)m.z * PAGE + threadIdx.x], gt, eq);
                if (eq) {
                  const int64_t pid = page_ids[m.z + (int)threadIdx.x / PAGE];
                  const uint32_t pos = meta[pid * (2 * PAGE) + PAGE + threadIdx.x % PAGE];
                  if (pass == 0 || (pos >> (sh + 8)) == pstar) atomicAdd(&lhist[(pos >> sh) & 255u], 1u);
                }
              }
            }
            lds_barrier();
            if (wave0) {
              // bins 4*lane .. 4*lane+3; counts of the bins above, from the top
              uint32_t cb4[4];
              int64_t own = 0;
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                cb4[u] = lhist[4 * lane + u];
                own += cb4[u];
              }
              int64_t above = own;   // inclusive suffix sum over lanes >= lane
              for (int d = 1; d < WAVE; d <<= 1) {
                const int64_t o = __shfl_down(above, d, WAVE);
                if (lane + d < WAVE) above += o;
              }
              above -= own;          // keys in bins of higher lanes
              if (above < rem && rem <= above + own) {
                int64_t cum = above;
                for (int u = 3; u >= 0; --u) {
                  if (cum + cb4[u] >= rem) {
                    sh_pre = (pstar << 8) | (uint32_t)(4 * lane + u);
                    sh_rem = rem - cum;
                    break;
                  }
                  cum += cb4[u];
                }
              }
            }
            lds_barrier();
            pstar = sh_pre;
            rem = sh_rem;
            lds_barrier();
          }
        }
        // 4. keep bytes of the head, kept count, kept-score sums per chunk
        int nk = 0;
        for (int c = ch0; c < ch1; ++c) {
          const int4 m = w.meta[c];
          const bool valid = (int)threadIdx.x < (m.w & 0xFFFF);
          float x = 0.f;
          bool k1 = false;
          if (valid) {
            x = score[(int64_t)m.z * PAGE + threadIdx.x];
            bool gt, eq;
            tie_of(x, gt, eq);
            k1 = gt;
            if (eq && q > 0) {
              if (q == eq_h) {
                k1 = true;
              } else {
                const int64_t pid = page_ids[m.z + (int)threadIdx.x / PAGE];
                k1 = meta[pid * (2 * PAGE) + PAGE + threadIdx.x % PAGE] >= pstar;
              }
            }
          }
          if ((int)threadIdx.x < (m.w >> 16) * PAGE) keep[(int64_t)m.z * PAGE + threadIdx.x] = k1 ? 1 : 0;
          nk += k1;
          if (want_sum) {
            const double bs = block_sum_f64(k1 ? (double)x : 0.0, tmpd);
            if (threadIdx.x == 0) w.part[c] = bs;
          }
        }
        nk = block_sum_all_i32(nk, red);
        if (wave0) kept[h] = nk;   // one value, stored by the whole wave
      }
    }
    i = e;
  }
}

// Kept-score sum of each head: its chunks' sums added in chunk order.  One
// wave per head: the lanes load 64 chunk sums at once, and the additions
// run in chunk order through lane shuffles (every lane forms the same sum).
__global__ void __launch_bounds__(256) k_sel_headsum(int n_heads, SelWs w, double* __restrict__ keptsum) {
  const int h = blockIdx.x * (256 / WAVE) + __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  if (h >= n_heads) return;   // per-wave exit: no block barriers
  const int lane = threadIdx.x & (WAVE - 1);
  const int c0 = w.chunk_off[h], c1 = w.chunk_off[h + 1];
  double s = 0.0;
  for (int b = c0; b < c1; b += WAVE) {
    const double v = b + lane < c1 ? w.part[b + lane] : 0.0;
    const int n = min(WAVE, c1 - b);
    for (int j = 0; j < n; ++j) s += __shfl(v, j, WAVE);
  }
  if (lane == 0) keptsum[h] = s;
}

SelWs carve(const trimkv_cache_t* c, int n_seg, void* ws) {
  WsLayout L = select_ws_layout(c, n_seg);
  char* b = (char*)ws;
  SelWs w;
  w.chunk_off = (int32_t*)(b + L.off[0]);
  w.meta = (int4*)(b + L.off[1]);
  w.seg = (SegState*)(b + L.off[2]);
  w.n_seg = n_seg;
  w.hist = (uint32_t*)(b + L.off[3]);
  w.look = (uint64_t*)(b + L.off[4]);
  w.ticket = (uint32_t*)(b + L.off[5]);
  w.status = nullptr;
  w.part = (double*)(b + L.off[6]);
  return w;
}

}  // namespace

WsLayout select_ws_layout(const trimkv_cache_t* c, int n_seg) {
  const int64_t T = max_chunks(c, CP);
  const int64_t H = c->n_heads;
  WsLayout L;
  L.add((H + 1) * 4);
  L.add((T + CPB) * 16);
  L.add((size_t)4 * n_seg * sizeof(SegState));
  L.add((size_t)n_seg * HIST_WORDS * 4);
  L.add(T * 8);
  L.add(((size_t)n_seg + 2) * 4);
  L.add(T * 8);
  return L;
}

namespace {

// The selection's kernels; with `src.score` set, the first pass forms the
// scores itself (score + select in one call).
int select_kernels(const trimkv_cache_t* c, const float* score, int n_seg, const int32_t* seg,
                   const int64_t* budget, uint8_t* keep, int32_t* kept, double* keptsum, int32_t* status, void* ws,
                   ScoreSrc src, AppendSrc ap, hipStream_t st) {
  SelWs w = carve(c, n_seg, ws);
  w.status = status;
  const int64_t T = max_chunks(c, CP);
  const int prep_blocks = prep_grid(c->n_heads, T, 1024);
  if (ap.k_new && c->n_heads <= PREP_HMAX) src.grow_len = c->len;   // raised by the first pass
  src.page_off = c->page_off;
  // append blocks (one wave per head) beside the prep blocks, unless one block must do everything
  const int app_blocks = ap.k_new && c->n_heads <= PREP_HMAX ? (c->n_heads + 15) / 16 : 0;
  hipLaunchKernelGGL(k_sel_prep, dim3(prep_blocks + app_blocks), dim3(1024), 0, st, c->page_off, c->len, c->n_heads,
                     n_seg, seg, budget, T, w, kept, ap, prep_blocks);
  // Chunks per block: 32 for pools of at least 4,096 chunks (about 4M
  // entries); smaller pools take 16, 8 or 4, the fewest that still gives at
  // most 256 blocks, so that a small selection (a streaming step's 0.5M
  // entries) spreads over many CUs instead of a dozen.  Counted, like the
  // grids, from the pool's capacity.
  const int cb = T >= 4096 ? CPB : T <= 4 * (int64_t)N_CU ? 4 : T <= 8 * (int64_t)N_CU ? 8 : 16;
  const unsigned hb = (unsigned)((T + cb - 1) / cb);
  prof_begin(st);
#define TRIMKV_SEL_PASSES(CBV)                                                                                    \
  {                                                                                                                \
    if (src.score)                                                                                                 \
      hipLaunchKernelGGL((k_sel_hist<0, CBV, true>), dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, src);       \
    else                                                                                                           \
      hipLaunchKernelGGL((k_sel_hist<0, CBV>), dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, src);             \
    hipLaunchKernelGGL((k_sel_hist<1, CBV>), dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, src);               \
    hipLaunchKernelGGL((k_sel_hist<2, CBV>), dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, src);               \
  }
  if (cb == CPB) {
    if (src.score) {
      // the pass that also forms the scores holds 94 VGPRs at CPB chunks per
      // block (one block per CU) and 54 at half (two): half measured faster
      // (8B pool: score + select 67.0 -> 64.4 us; the plain passes are
      // slower at half there, 56.1 -> 57.7 us for select)
      const unsigned hb0 = (unsigned)((T + CPB / 2 - 1) / (CPB / 2));
      hipLaunchKernelGGL((k_sel_hist<0, CPB / 2, true>), dim3(hb0), dim3(NT), 0, st, c->n_heads, score, w, src);
    } else {
      hipLaunchKernelGGL((k_sel_hist<0, CPB>), dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, src);   // 48 VGPRs
    }
    // Later passes (78 VGPRs at CPB chunks per block: one block per CU), when
    // there are more blocks with work than CUs (counted as if the pool's pages
    // were all in use): half the chunks per block, whose fewer live keys (64
    // VGPRs) let two blocks share a CU.
    if ((c->n_pages / CP + CPB - 1) / CPB > N_CU) {
      const unsigned hb2 = (unsigned)((T + CPB / 2 - 1) / (CPB / 2));
      hipLaunchKernelGGL((k_sel_hist<1, CPB / 2>), dim3(hb2), dim3(NT), 0, st, c->n_heads, score, w, src);
      hipLaunchKernelGGL((k_sel_hist<2, CPB / 2>), dim3(hb2), dim3(NT), 0, st, c->n_heads, score, w, src);
    } else {
      hipLaunchKernelGGL((k_sel_hist<1, CPB>), dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, src);
      hipLaunchKernelGGL((k_sel_hist<2, CPB>), dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, src);
    }
    hipLaunchKernelGGL(k_sel_decide<CPB>, dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, keep, kept,
                       keptsum != nullptr, c->page_ids, c->meta);
  } else if (cb == 16) {
    TRIMKV_SEL_PASSES(16)
    hipLaunchKernelGGL(k_sel_decide<16>, dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, keep, kept,
                       keptsum != nullptr, c->page_ids, c->meta);
  } else if (cb == 8) {
    TRIMKV_SEL_PASSES(8)
    hipLaunchKernelGGL(k_sel_decide<8>, dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, keep, kept,
                       keptsum != nullptr, c->page_ids, c->meta);
  } else {
    TRIMKV_SEL_PASSES(4)
    hipLaunchKernelGGL(k_sel_decide<4>, dim3(hb), dim3(NT), 0, st, c->n_heads, score, w, keep, kept,
                       keptsum != nullptr, c->page_ids, c->meta);
  }
#undef TRIMKV_SEL_PASSES
  prof_end(st);
  if (keptsum)
    hipLaunchKernelGGL(k_sel_headsum, dim3((unsigned)((c->n_heads + 3) / 4)), dim3(256), 0, st, c->n_heads, w,
                       keptsum);
  return check_launch();
}

}  // namespace

int launch_select(const trimkv_cache_t* c, const float* score, int n_seg, const int32_t* seg,
                  const int64_t* budget, uint8_t* keep, int32_t* kept, double* keptsum, int32_t* status, void* ws,
                  hipStream_t st) {
  return select_kernels(c, score, n_seg, seg, budget, keep, kept, keptsum, status, ws, ScoreSrc{}, AppendSrc{}, st);
}

int launch_score_select(const trimkv_cache_t* c, int n_seg, const int32_t* seg, const int32_t* t,
                        const int64_t* budget, float* score, uint8_t* keep, int32_t* kept, double* keptsum,
                        int32_t* status, void* ws, hipStream_t st) {
  return select_kernels(c, score, n_seg, seg, budget, keep, kept, keptsum, status, ws,
                        ScoreSrc{c->page_ids, c->meta, t, score, nullptr, nullptr}, AppendSrc{}, st);
}

int launch_append_score_select(trimkv_cache_t* c, const void* k_new, const void* v_new, const float* beta_new,
                               int n_seg, const int32_t* seg, const int32_t* t, const int64_t* budget, float* score,
                               uint8_t* keep, int32_t* kept, double* keptsum, int32_t* append_status,
                               int32_t* select_status, void* ws, hipStream_t st) {
  const int elt = c->dtype == TRIMKV_BF16 ? 2 : 4;
  AppendSrc ap{(const uint8_t*)k_new, (const uint8_t*)v_new, beta_new, (uint8_t*)c->k, (uint8_t*)c->v, c->meta,
               c->page_ids, t, c->head_dim * elt, elt, append_status};
  return select_kernels(c, score, n_seg, seg, budget, keep, kept, keptsum, select_status, ws,
                        ScoreSrc{c->page_ids, c->meta, t, score, nullptr, nullptr}, ap, st);
}

}  // namespace trimkv
