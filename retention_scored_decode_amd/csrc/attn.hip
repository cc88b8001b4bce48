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
// Split-K over work items = (KV head, chunk of 16 pages).  A work-group of
// four waves handles one item; every (wave, 16-lane row) is an independent
// online-softmax stream over 4 keys of each page it visits.  All G query
// heads of the KV head are processed together, so K and V are read once.
//
// bf16 path: S = K q^T on MFMA (v_mfma_f32_16x16x16_bf16: 16 keys x 16
// query columns, G <= 16 of them live), P V on the VALU with fp32
// accumulation.  Logits are kept in base 2 (scale * log2 e folded in).
// Partials (max, kept sum, dropped sum, acc[G][D]) are merged per query head
// in a fixed order by a second kernel, so results are run-to-run identical.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace trimkv {

namespace {

constexpr int CHA_F32 = 16;  // pages per work item of the fp32 kernel (one key per thread)
constexpr int CHA_MIN = 16;  // smallest item size (workspace bound)
constexpr int NT = 256;
constexpr int GMAX = 16;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

enum { A_PLAIN = 0, A_MASK = 1, A_LOGITS = 2 };

struct AttnWs {
  int32_t* item_off;   // [H + 1]
  int4* item;          // [Wmax + 4] (head, first CSR page, valid entries, pages)
  float* stats;        // [Wmax][G][3]   (max2, kept sum, dropped sum)
  float* acc;          // [Wmax][G][D]
  float* lse2;         // [H * G] base-2 LSE (mass op)
  float* logits;       // [G][n_pages * 16] (mass op)
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
  int64_t plane;         // logits plane stride (n_pages * 16)
  int cha;               // pages per work item
  AttnWs w;
  // outputs written by the merge of each head
  const float* lse_ref;
  float* out;
  float* dropped;
  float* lse_out;
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

template <int L>
__device__ __forceinline__ float bcast_row(float v) {
  // DPP row_newbcast: every lane of a 16-lane row reads lane L of that row
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + L, 0xF, 0xF, true));
}

template <int GM, typename F>
__device__ __forceinline__ void for_g(F f) {
#pragma unroll
  for (int g = 0; g < GM; ++g) f(g);
}

__device__ __forceinline__ float bcast_dyn(float v, int g) {
  switch (g) {
    case 0: return bcast_row<0>(v);   case 1: return bcast_row<1>(v);
    case 2: return bcast_row<2>(v);   case 3: return bcast_row<3>(v);
    case 4: return bcast_row<4>(v);   case 5: return bcast_row<5>(v);
    case 6: return bcast_row<6>(v);   case 7: return bcast_row<7>(v);
    case 8: return bcast_row<8>(v);   case 9: return bcast_row<9>(v);
    case 10: return bcast_row<10>(v); case 11: return bcast_row<11>(v);
    case 12: return bcast_row<12>(v); case 13: return bcast_row<13>(v);
    case 14: return bcast_row<14>(v); default: return bcast_row<15>(v);
  }
}

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

// Merge all partials of KV head h: per query head g, M = max of the item
// maxima, kept and dropped sums rescaled to M, acc rescaled and divided by
// the kept sum.  A head without items has an empty kept set: out = 0,
// dropped = 1, lse = -inf.  One block per KV head; fixed summation order.
template <int D>
__global__ void __launch_bounds__(NT) k_attn_merge(AttnArgs a, int with_out) {
  const AttnWs& w = a.w;
  const int h = blockIdx.x;
  const int G = a.group;
  const int b = w.item_off[h], e = w.item_off[h + 1];
  __shared__ float sM[GMAX], sLA[GMAX];
  const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;  // 16 groups of 16 lanes
  if (grp < G) {
    float M = -INFINITY;
    for (int it = b + sub; it < e; it += 16) M = fmaxf(M, w.stats[((size_t)it * G + grp) * 3]);
#pragma unroll
    for (int d = 8; d > 0; d >>= 1) M = fmaxf(M, __shfl_xor(M, d, 16));
    float la = 0.f, ld = 0.f;
    if (M != -INFINITY) {
      for (int it = b + sub; it < e; it += 16) {
        const float* st = w.stats + ((size_t)it * G + grp) * 3;
        const float sc = exp2f(st[0] - M);
        la += st[1] * sc;
        ld += st[2] * sc;
      }
    }
#pragma unroll
    for (int d = 8; d > 0; d >>= 1) {
      la += __shfl_xor(la, d, 16);
      ld += __shfl_xor(ld, d, 16);
    }
    if (sub == 0) {
      sM[grp] = M;
      sLA[grp] = la;
      const int qh = h * G + grp;
      const float l2 = la > 0.f ? M + log2f(la) : -INFINITY;  // base-2 LSE of the kept set
      const float lse = l2 * LN2;
      if (a.lse_out) a.lse_out[qh] = lse;
      if (w.lse2) w.lse2[qh] = l2;
      if (a.dropped) {
        float dm = 1.f;
        if (la > 0.f) dm = a.lse_ref ? -expm1f(lse - a.lse_ref[qh]) : ld / (la + ld);
        a.dropped[qh] = dm;
      }
    }
  }
  __syncthreads();
  if (with_out) {
    for (int i = threadIdx.x; i < G * D; i += NT) {
      const int g = i / D;
      const float M = sM[g], la = sLA[g];
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
      if (M != -INFINITY) {
        int it = b;
        for (; it + 4 <= e; it += 4) {
          s0 += w.acc[(size_t)it * G * D + i] * exp2f(w.stats[((size_t)it * G + g) * 3] - M);
          s1 += w.acc[(size_t)(it + 1) * G * D + i] * exp2f(w.stats[((size_t)(it + 1) * G + g) * 3] - M);
          s2 += w.acc[(size_t)(it + 2) * G * D + i] * exp2f(w.stats[((size_t)(it + 2) * G + g) * 3] - M);
          s3 += w.acc[(size_t)(it + 3) * G * D + i] * exp2f(w.stats[((size_t)(it + 3) * G + g) * 3] - M);
        }
        for (; it < e; ++it) s0 += w.acc[(size_t)it * G * D + i] * exp2f(w.stats[((size_t)it * G + g) * 3] - M);
      }
      const float s = (s0 + s1) + (s2 + s3);
      a.out[(size_t)h * G * D + i] = la > 0.f ? s / la : 0.f;
    }
  }
}

template <int D> struct VRow;
template <> struct VRow<128> { typedef uint4 T; };
template <> struct VRow<64> { typedef uint2 T; };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Threshold (log2 units) of the lazily updated running maximum: between two
// rescalings every exp2(z - m) stays below 2^RESCALE_T, far inside fp32.
constexpr float RESCALE_T = 10.f;

// ---------------------------------------------------------------------------
// bf16 K/V, MFMA logits.  MODE: A_PLAIN (every valid key kept), A_MASK (keep
// plane; dropped keys only enter the dropped sum, their V is not read),
// A_LOGITS (write base-2 logits of every valid key, (max, sum) partials).
//
// One wave per work item (head, up to a.cha consecutive pages); waves never
// wait for each other.  S = K q^T on v_mfma_f32_16x16x32_bf16: lane (r, col)
// feeds key `col`, dims 32u + 8r .. +7 of K and the same dims of query head
// `col`, straight from 16-byte loads; it receives S[key 4r + j][head col].
// Each 16-lane row r is an online-softmax stream over keys 4r..4r+3 of every
// page; its running maximum is raised only when a logit exceeds it by more
// than RESCALE_T (a wave-uniform branch), so the common page costs one FMA
// and one exp2 per logit.  P V runs on the VALU in fp32.  K and V tiles of
// page i + LA are in flight while page i is processed.
// ---------------------------------------------------------------------------
template <int D, int GM, int MODE>
__global__ void __launch_bounds__(NT) k_attn_bf16(AttnArgs a) {
  constexpr int KU = D / 32;    // 16-byte K pieces per lane per page = MFMAs per page
  constexpr int DS = D / 16;    // V dims per lane
  constexpr bool LOGITS = MODE == A_LOGITS;
  typedef typename VRow<D>::T VT;
  const AttnWs& w = a.w;
  const int lane = threadIdx.x & 63, r = lane >> 4, col = lane & 15;
  const int item = blockIdx.x * (NT / WAVE) + (threadIdx.x >> 6);
  const int total = w.item_off[a.n_heads];
  const int4 rec = w.item[item];   // (head, first CSR page, valid entries, pages); padded past the end
  if (item >= total) return;       // per-wave exit: no block barriers below
  const int G = a.group;
  const int h = rec.x, page0 = rec.y, nv = rec.z, cnt = rec.w;

  // lane l: page id of page l; keep words: lane l of kw[b] covers page 16b + l/4, keys 4(l%4)..+3
  const int pid_l = lane < cnt ? a.page_ids[page0 + lane] : 0;
  uint32_t kw0 = 0xFFFFFFFFu, kw1 = 0xFFFFFFFFu;
  if (MODE == A_MASK) {
    const uint8_t* kb = a.keep + (int64_t)page0 * PAGE;
    if (lane / 4 < cnt) kw0 = *reinterpret_cast<const uint32_t*>(kb + 4 * lane);
    if (16 + lane / 4 < cnt) kw1 = *reinterpret_cast<const uint32_t*>(kb + 256 + 4 * lane);
  }
  auto kword = [&](int i) -> uint32_t {
    if (MODE != A_MASK) return 0xFFFFFFFFu;
    const uint32_t src = (i < 16) ? kw0 : kw1;
    return (uint32_t)__shfl((int)src, ((i & 15) << 2) + r, WAVE);
  };

  // B operand of MFMA u: dims 32u + 8r .. +7 of query head col (zero for col >= G)
  uint4 qop[KU];
  {
    const uint8_t* qrow = (const uint8_t*)a.q + ((size_t)h * G + (col < G ? col : 0)) * D * 2 + 16 * r;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      qop[u] = *reinterpret_cast<const uint4*>(qrow + 64 * u);
      if (col >= G) qop[u] = make_uint4(0, 0, 0, 0);
    }
  }

  float m = -INFINITY, la = 0.f, ld = 0.f;
  float nm = INFINITY;   // -m, or +inf while m = -inf (every finite logit then forces an update)
  float acc[GM][DS];
  for_g<GM>([&](int g) {
#pragma unroll
    for (int d = 0; d < DS; ++d) acc[g][d] = 0.f;
  });
  const uint8_t* kbase = (const uint8_t*)a.k;
  const uint8_t* vbase = (const uint8_t*)a.v;
  const uint32_t koff = col * D * 2 + 16 * r;            // this lane's K bytes within a page
  const uint32_t voff = (4 * r * D + col * DS) * 2;      // this lane's V bytes of key 4r

  // Every load is issued unconditionally so the compiler can count outstanding
  // loads exactly and wait only for the page being processed: a V row that is
  // not needed (dropped or past the end) is read from the start of the page's
  // K tile instead, a line this wave has just requested.
  auto load = [&](int i, uint32_t kwi, uint4 (&kd)[KU], VT (&vd)[4]) {
    const int64_t phys = __builtin_amdgcn_readlane(pid_l, i);
    const uint8_t* kpage = kbase + phys * (PAGE * D * 2);
    const uint8_t* vpage = vbase + phys * (PAGE * D * 2);
#pragma unroll
    for (int u = 0; u < KU; ++u) kd[u] = *reinterpret_cast<const uint4*>(kpage + koff + 64 * u);
    if (MODE == A_PLAIN) {
      // every row of an allocated page is readable; rows past the end are
      // zeroed before use
#pragma unroll
      for (int j = 0; j < 4; ++j) vd[j] = *reinterpret_cast<const VT*>(vpage + voff + j * D * 2);
    } else if (MODE == A_MASK) {
      const int i0 = i * PAGE + 4 * r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool need = i0 + j < nv && ((kwi >> (8 * j)) & 0xFFu);
        const uint8_t* src = need ? vpage + voff + j * D * 2 : kpage + col * 16;
        vd[j] = *reinterpret_cast<const VT*>(src);
      }
    }
  };

  auto compute = [&](int i, uint32_t kwi, uint4 (&kc)[KU], VT (&vc)[4]) {
    float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KU; ++u)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kc[u]),
                                                  __builtin_bit_cast(bf16x8_t, qop[u]), s, 0, 0, 0);
    const int i0 = i * PAGE + 4 * r;      // entry of key 4r within the item
    const bool full = (i + 1) * PAGE <= nv;   // wave-uniform
    float pj[4];
    bool slow = !full;
    if (full) {
#pragma unroll
      for (int j = 0; j < 4; ++j) pj[j] = fmaf(s[j], a.scale2, nm);
      slow = __any(fmaxf(fmaxf(pj[0], pj[1]), fmaxf(pj[2], pj[3])) > RESCALE_T);
    }
    float alpha = 1.f;
    if (slow) {
      float z[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = i0 + j < nv ? s[j] * a.scale2 : -INFINITY;
      const float mn = fmaxf(m, fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
      if (mn != -INFINITY) {
        alpha = exp2f(m - mn);   // 0 while m = -inf
        m = mn;
        nm = -mn;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) pj[j] = z[j] - m;
      la *= alpha;
      ld *= alpha;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) pj[j] = __builtin_amdgcn_exp2f(pj[j]);   // exp2(-inf) = 0; NaN only while m = -inf
    if (slow && m == -INFINITY) pj[0] = pj[1] = pj[2] = pj[3] = 0.f;
    if (LOGITS) {
      if (col < G) {
        float* dst = w.logits + (int64_t)col * a.plane + (int64_t)(page0 + i) * PAGE + 4 * r;
        if (full) {
          *reinterpret_cast<float4*>(dst) = make_float4(s[0] * a.scale2, s[1] * a.scale2, s[2] * a.scale2,
                                                        s[3] * a.scale2);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (i0 + j < nv) dst[j] = s[j] * a.scale2;
        }
      }
    }
    if (MODE == A_MASK) {
      float sk = 0.f, sd = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool kept = ((kwi >> (8 * j)) & 0xFFu) && (full || i0 + j < nv);
        sk += kept ? pj[j] : 0.f;
        sd += kept ? 0.f : pj[j];
        if (!kept) pj[j] = 0.f;
      }
      la += sk;
      ld += sd;
    } else {
      la += (pj[0] + pj[1]) + (pj[2] + pj[3]);
    }
    if (!LOGITS) {
      if (slow) {
        for_g<GM>([&](int g) {
          const float av = bcast_dyn(alpha, g);
#pragma unroll
          for (int d = 0; d < DS; ++d) acc[g][d] *= av;
        });
      }
      // P V: lanes of row r own dims [col*DS, col*DS+DS) of keys 4r..4r+3
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool kept = MODE == A_PLAIN ? true : (((kwi >> (8 * j)) & 0xFFu) && (full || i0 + j < nv));
        if (MODE == A_PLAIN || kept) {
          VT vv = vc[j];
          if (MODE == A_PLAIN && !full && i0 + j >= nv) vv = VT{};   // unwritten rows may hold non-finite bits
          float vf[DS];
          if constexpr (DS == 8) {
            vf[0] = bf16lo(vv.x); vf[1] = bf16hi(vv.x); vf[2] = bf16lo(vv.y); vf[3] = bf16hi(vv.y);
            vf[4] = bf16lo(vv.z); vf[5] = bf16hi(vv.z); vf[6] = bf16lo(vv.w); vf[7] = bf16hi(vv.w);
          } else {
            vf[0] = bf16lo(vv.x); vf[1] = bf16hi(vv.x); vf[2] = bf16lo(vv.y); vf[3] = bf16hi(vv.y);
          }
          for_g<GM>([&](int g) {
            const float pk = bcast_dyn(pj[j], g);
#pragma unroll
            for (int d = 0; d < DS; ++d) acc[g][d] = fmaf(pk, vf[d], acc[g][d]);
          });
        }
      }
    }
  };

  // ring of LA + 1 page buffers: page ii + LA is loaded while page ii is
  // processed (indices past the item's last page reload that page)
  constexpr int LA = GM <= 4 ? 2 : 1;
  constexpr int NB = LA + 1;
  uint4 kb[NB][KU];
  VT vb[NB][4];
  uint32_t kwb[NB];
#pragma unroll
  for (int u = 0; u < LA; ++u) {
    const int pi = min(u, cnt - 1);
    kwb[u] = kword(pi);
    load(pi, kwb[u], kb[u], vb[u]);
  }
  for (int i = 0; i < cnt; i += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int ii = i + u;
      if (ii >= cnt) break;
      const int nb = (u + LA) % NB;
      const int pi = min(ii + LA, cnt - 1);
      kwb[nb] = kword(pi);
      load(pi, kwb[nb], kb[nb], vb[nb]);
      compute(ii, kwb[u], kb[u], vb[u]);
    }
  }

  // ---- combine the four row streams of the wave and write the partial ----
  float M = fmaxf(m, __shfl_xor(m, 16, WAVE));
  M = fmaxf(M, __shfl_xor(M, 32, WAVE));
  const float sc = (M == -INFINITY) ? 0.f : exp2f(m - M);
  float las = la * sc, lds = ld * sc;
  las += __shfl_xor(las, 16, WAVE);
  las += __shfl_xor(las, 32, WAVE);
  lds += __shfl_xor(lds, 16, WAVE);
  lds += __shfl_xor(lds, 32, WAVE);
  if (r == 0 && col < G) {
    float* st = w.stats + ((size_t)item * G + col) * 3;
    st[0] = M;
    st[1] = las;
    st[2] = lds;
  }
  if (!LOGITS) {
    for_g<GM>([&](int g) {
      const float sg = bcast_dyn(sc, g);   // scale of this row's stream for query column g
#pragma unroll
      for (int d = 0; d < DS; ++d) {
        float x = acc[g][d] * sg;
        x += __shfl_xor(x, 16, WAVE);
        x += __shfl_xor(x, 32, WAVE);
        acc[g][d] = x;
      }
      if (r == 0 && g < G) {
        float* dst = w.acc + ((size_t)item * G + g) * D + col * DS;
#pragma unroll
        for (int d = 0; d < DS; ++d) dst[d] = acc[g][d];
      }
    });
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
      if (LOGITS) w.logits[(int64_t)g * a.plane + (int64_t)(page0 + p) * PAGE + t % PAGE] = z;
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
    const float z = sp[g][t];
    const float M = block_reduce(z, true);
    const float pr = (M == -INFINITY || !valid) ? 0.f : exp2f(z - M);
    const float ka = block_reduce(kept ? pr : 0.f, false);
    const float kd = block_reduce(kept ? 0.f : pr, false);
    __syncthreads();
    sp[g][t] = kept ? pr : 0.f;
    if (t == 0) {
      float* st = w.stats + ((size_t)item * G + g) * 3;
      st[0] = M;
      st[1] = ka;
      st[2] = kd;
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
__global__ void __launch_bounds__(256) k_mass(const int32_t* __restrict__ page_off, const int32_t* __restrict__ len,
                                              int n_heads, int group, int64_t plane, const AttnWs w,
                                              float* __restrict__ mass) {
  __shared__ PageHeads sh;
  const int64_t total = page_off[n_heads];
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  if (c0 >= total) return;
  const PageHeads r = block_page_heads(page_off, n_heads, c0, min(c0 + 63, total - 1), &sh);
  const int64_t c = c0 + (threadIdx.x >> 2);
  const int j0 = (threadIdx.x & 3) * 4;
  if (c >= total) return;
  const int h = r.hf == r.hl ? r.hf : head_in_range(page_off, r, c);
  const int64_t i0 = (c - page_off[h]) * PAGE + j0;
  const int64_t n = len[h];
  const int64_t slot = c * PAGE + j0;
  float o[4] = {qnan(), qnan(), qnan(), qnan()};
  if (i0 < n) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < group; ++g) {
      const float4 z = *reinterpret_cast<const float4*>(w.logits + (int64_t)g * plane + slot);
      const float l2 = w.lse2[(size_t)h * group + g];
      s[0] += exp2f(z.x - l2);
      s[1] += exp2f(z.y - l2);
      s[2] += exp2f(z.z - l2);
      s[3] += exp2f(z.w - l2);
    }
    const float inv = 1.f / (float)group;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (i0 + k < n) o[k] = s[k] * inv;
  }
  *reinterpret_cast<float4*>(mass + slot) = make_float4(o[0], o[1], o[2], o[3]);
}

AttnWs carve(const trimkv_cache_t* c, int group, void* ws, bool mass) {
  WsLayout L = mass ? mass_ws_layout(c, group) : attn_ws_layout(c, group);
  char* b = (char*)ws;
  AttnWs w;
  w.item_off = (int32_t*)(b + L.off[0]);
  w.item = (int4*)(b + L.off[1]);
  w.stats = (float*)(b + L.off[2]);
  w.acc = (float*)(b + L.off[3]);
  w.lse2 = mass ? (float*)(b + L.off[4]) : nullptr;
  w.logits = mass ? (float*)(b + L.off[5]) : nullptr;
  return w;
}

int gm_for(int g) { return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : g <= 8 ? 8 : 16; }

template <int MODE>
int launch_main(const trimkv_cache_t* c, AttnArgs& a, hipStream_t st) {
  constexpr bool LOGITS = MODE == A_LOGITS;
  const int64_t W = max_chunks(c, a.cha);   // bound on the number of items
  const dim3 blk(NT);
  if (c->dtype == TRIMKV_F32) {
    const dim3 grid((unsigned)W);   // one item per block
    if (c->head_dim == 128) hipLaunchKernelGGL((k_attn_f32<128, LOGITS>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_attn_f32<64, LOGITS>), grid, blk, 0, st, a);
    return TRIMKV_OK;
  }
  const dim3 grid((unsigned)((W + NT / WAVE - 1) / (NT / WAVE)));   // one item per wave
  const int gm = gm_for(a.group);
#define TRIMKV_BF16(DD, GG) hipLaunchKernelGGL((k_attn_bf16<DD, GG, MODE>), grid, blk, 0, st, a)
  if (c->head_dim == 128) {
    switch (gm) {
      case 1: TRIMKV_BF16(128, 1); break;
      case 2: TRIMKV_BF16(128, 2); break;
      case 4: TRIMKV_BF16(128, 4); break;
      case 8: TRIMKV_BF16(128, 8); break;
      default: TRIMKV_BF16(128, 16); break;
    }
  } else {
    switch (gm) {
      case 1: TRIMKV_BF16(64, 1); break;
      case 2: TRIMKV_BF16(64, 2); break;
      case 4: TRIMKV_BF16(64, 4); break;
      case 8: TRIMKV_BF16(64, 8); break;
      default: TRIMKV_BF16(64, 16); break;
    }
  }
#undef TRIMKV_BF16
  return TRIMKV_OK;
}

}  // namespace

WsLayout attn_ws_layout(const trimkv_cache_t* c, int group) {
  const int64_t W = max_chunks(c, CHA_MIN);
  WsLayout L;
  L.add(((int64_t)c->n_heads + 1) * 4);
  L.add((W + 4) * 16);
  L.add(W * group * 3 * 4);
  L.add(W * group * (int64_t)c->head_dim * 4);
  return L;
}

WsLayout mass_ws_layout(const trimkv_cache_t* c, int group) {
  const int64_t W = max_chunks(c, CHA_MIN);
  WsLayout L;
  L.add(((int64_t)c->n_heads + 1) * 4);
  L.add((W + 4) * 16);
  L.add(W * group * 3 * 4);
  L.add(0);
  L.add((int64_t)c->n_heads * group * 4);
  L.add((int64_t)group * c->n_pages * PAGE * 4);
  return L;
}

int launch_decode_attn(const trimkv_cache_t* c, const uint8_t* keep, const float* lse_ref, const void* q,
                       int group, float scale, float* out, float* dropped, float* lse_out, void* ws,
                       hipStream_t st) {
  AttnWs w = carve(c, group, ws, false);
  // items of 32 pages when every key is read (mask mode), 16 otherwise
  const int cha = c->dtype == TRIMKV_F32 ? CHA_F32 : (keep ? 32 : 16);
  hipLaunchKernelGGL(k_attn_prep, dim3(prep_grid(c->n_heads, max_chunks(c, cha), 2048)), dim3(1024), 0, st,
                     c->page_off, c->len, c->n_heads, cha, w);
  AttnArgs a{c->page_off, c->page_ids, c->len, c->k, c->v, keep, q, c->n_heads, group, scale * LOG2E,
             c->n_pages * PAGE, cha, w, lse_ref, out, dropped, lse_out};
  prof_begin(st);
  int rc = keep ? launch_main<A_MASK>(c, a, st) : launch_main<A_PLAIN>(c, a, st);
  prof_end(st);
  if (rc) return rc;
  if (c->head_dim == 128) hipLaunchKernelGGL(k_attn_merge<128>, dim3(c->n_heads), dim3(NT), 0, st, a, 1);
  else hipLaunchKernelGGL(k_attn_merge<64>, dim3(c->n_heads), dim3(NT), 0, st, a, 1);
  return check_launch();
}

int launch_attn_mass(const trimkv_cache_t* c, const void* q, int group, float scale, float* mass,
                     float* lse_full, void* ws, hipStream_t st) {
  AttnWs w = carve(c, group, ws, true);
  const int cha = c->dtype == TRIMKV_F32 ? CHA_F32 : 32;
  hipLaunchKernelGGL(k_attn_prep, dim3(prep_grid(c->n_heads, max_chunks(c, cha), 2048)), dim3(1024), 0, st,
                     c->page_off, c->len, c->n_heads, cha, w);
  AttnArgs a{c->page_off, c->page_ids, c->len, c->k, c->v, nullptr, q, c->n_heads, group, scale * LOG2E,
             c->n_pages * PAGE, cha, w, nullptr, nullptr, nullptr, lse_full};
  prof_begin(st);
  int rc = launch_main<A_LOGITS>(c, a, st);
  prof_end(st);
  if (rc) return rc;
  if (c->head_dim == 128) hipLaunchKernelGGL(k_attn_merge<128>, dim3(c->n_heads), dim3(NT), 0, st, a, 0);
  else hipLaunchKernelGGL(k_attn_merge<64>, dim3(c->n_heads), dim3(NT), 0, st, a, 0);
  const int64_t blocks = (c->n_pages + 63) / 64;
  hipLaunchKernelGGL(k_mass, dim3((unsigned)blocks), dim3(256), 0, st, c->page_off, c->len, c->n_heads, group,
                     c->n_pages * PAGE, w, mass);
  return check_launch();
}

}  // namespace trimkv
