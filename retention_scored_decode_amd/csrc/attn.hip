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

constexpr int CHA = 16;   // pages per work item
constexpr int NT = 256;
constexpr int GMAX = 16;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct AttnWs {
  int32_t* item_off;   // [H + 1]
  int32_t* item_head;  // [Wmax]
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
  AttnWs w;
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

template <int L>
__device__ __forceinline__ float bcast_row(float v) {
  // DPP row_newbcast: every lane of a 16-lane row reads lane L of that row
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + L, 0xF, 0xF, false));
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

__global__ void __launch_bounds__(1024) k_attn_prep(const int32_t* __restrict__ page_off, int n_heads, AttnWs w) {
  __shared__ int64_t tmp[1024 / WAVE + 1];
  build_chunk_list<1024>(page_off, n_heads, CHA, w.item_off, w.item_head, tmp);
}

// Combine the 16 streams of a work-group and write the item's partial.
// m/la/ld: this lane's stream values for g = lane % 16 (lanes with
// lane % 16 >= G hold don't-care values); acc: this lane's dims slice.
template <int D, int GM>
__device__ __forceinline__ void combine_streams(float m, float la, float ld, float (&acc)[GM][D / 16], int G,
                                                int item, const AttnWs& w, bool with_acc) {
  constexpr int DS = D / 16;
  __shared__ float sm[16][GMAX], sla[16][GMAX], sld[16][GMAX];
  __shared__ float sacc[4][GM][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane >> 4, col = lane & 15;
  const int stream = wave * 4 + r;
  if (col < G) sm[stream][col] = m;
  __syncthreads();
  float scale_own[GM];
  for_g<GM>([&](int g) {
    float M = -INFINITY;
    if (g < G)
      for (int s = 0; s < 16; ++s) M = fmaxf(M, sm[s][g]);
    const float ms = g < G ? sm[stream][g] : -INFINITY;
    scale_own[g] = (M == -INFINITY) ? 0.f : exp2f(ms - M);
  });
  if (col < G) {
    float sc = 0.f;
    for_g<GM>([&](int g) { if (g == col) sc = scale_own[g]; });
    sla[stream][col] = la * sc;
    sld[stream][col] = ld * sc;
  }
  if (with_acc) {
    for_g<GM>([&](int g) {
#pragma unroll
      for (int d = 0; d < DS; ++d) {
        float x = acc[g][d] * scale_own[g];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        acc[g][d] = x;
      }
    });
    if (r == 0) {
      for_g<GM>([&](int g) {
#pragma unroll
        for (int d = 0; d < DS; ++d) sacc[wave][g][col * DS + d] = acc[g][d];
      });
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float M = -INFINITY, a = 0.f, b = 0.f;
    for (int s = 0; s < 16; ++s) {
      M = fmaxf(M, sm[s][g]);
      a += sla[s][g];
      b += sld[s][g];
    }
    float* st = w.stats + ((size_t)item * G + g) * 3;
    st[0] = M;
    st[1] = a;
    st[2] = b;
  }
  if (with_acc) {
    for (int i = threadIdx.x; i < G * D; i += NT) {
      const int g = i / D, d = i % D;
      float s = 0.f;
      for_g<GM>([&](int gg) {
        if (gg == g) s = sacc[0][gg][d] + sacc[1][gg][d] + sacc[2][gg][d] + sacc[3][gg][d];
      });
      w.acc[(size_t)item * G * D + i] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 K/V, MFMA logits.  LOGITS=false: attention partials; LOGITS=true:
// write base-2 logits of every valid key and (max, sum) partials.
// ---------------------------------------------------------------------------
template <int D, int GM, bool LOGITS>
__global__ void __launch_bounds__(NT) k_attn_bf16(AttnArgs a) {
  constexpr int KU = D / 32;   // uint4 of K per lane per page
  constexpr int NK = D / 16;   // MFMAs per page
  constexpr int DS = D / 16;   // V dims per lane
  const int item = blockIdx.x;
  const AttnWs& w = a.w;
  if (item >= w.item_off[a.n_heads]) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane >> 4, col = lane & 15;
  const int G = a.group;
  const int h = w.item_head[item];
  const int pbase = a.page_off[h];
  const int np = a.page_off[h + 1] - pbase;
  const int p0 = (item - w.item_off[h]) * CHA;
  const int p1 = min(p0 + CHA, np);
  const int n = a.len[h];
  const uint16_t* kq = (const uint16_t*)a.q;

  // B operand: query column g = col; MFMA kk covers dims 32*(kk/2) + 8r + 4*(kk%2) + [0,4)
  short4_t qop[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    short4_t x = {0, 0, 0, 0};
    if (col < G) {
      const uint16_t* src = kq + ((size_t)h * G + col) * D + 32 * (kk / 2) + 8 * r + 4 * (kk % 2);
      const uint2 u = *reinterpret_cast<const uint2*>(src);
      x[0] = (short)(u.x & 0xFFFF); x[1] = (short)(u.x >> 16);
      x[2] = (short)(u.y & 0xFFFF); x[3] = (short)(u.y >> 16);
    }
    qop[kk] = x;
  }

  float m = -INFINITY, la = 0.f, ld = 0.f;
  float acc[GM][DS];
  for_g<GM>([&](int g) {
#pragma unroll
    for (int d = 0; d < DS; ++d) acc[g][d] = 0.f;
  });
  const uint8_t* kbase = (const uint8_t*)a.k;
  const uint8_t* vbase = (const uint8_t*)a.v;

  for (int p = p0 + wave; p < p1; p += 4) {
    const int64_t phys = a.page_ids[pbase + p];
    // ---- logits S[key = 4r + j][g = col] ----
    const uint8_t* krow = kbase + ((phys * PAGE + col) * D) * 2 + 16 * r;
    uint4 kr[KU];
#pragma unroll
    for (int u = 0; u < KU; ++u) kr[u] = *reinterpret_cast<const uint4*>(krow + 64 * u);
    float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      short4_t a0 = {(short)(kr[u].x & 0xFFFF), (short)(kr[u].x >> 16), (short)(kr[u].y & 0xFFFF),
                     (short)(kr[u].y >> 16)};
      short4_t a1 = {(short)(kr[u].z & 0xFFFF), (short)(kr[u].z >> 16), (short)(kr[u].w & 0xFFFF),
                     (short)(kr[u].w >> 16)};
      s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a0, qop[2 * u], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a1, qop[2 * u + 1], s, 0, 0, 0);
    }
    const int i0 = p * PAGE + 4 * r;   // entry index of key 4r within the head
    uint32_t kw = 0xFFFFFFFFu;         // keep bytes of keys 4r..4r+3
    if (!LOGITS && a.keep) kw = *reinterpret_cast<const uint32_t*>(a.keep + (int64_t)(pbase + p) * PAGE + 4 * r);
    float z[4];
    bool valid[4], kept[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      valid[j] = i0 + j < n;
      kept[j] = valid[j] && ((kw >> (8 * j)) & 0xFFu);
      z[j] = valid[j] ? s[j] * a.scale2 : -INFINITY;
    }
    if (LOGITS) {
      if (col < G) {
        float* dst = w.logits + (int64_t)col * a.plane + (int64_t)(pbase + p) * PAGE + 4 * r;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (valid[j]) dst[j] = z[j];
      }
    }
    const float pm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    const float mn = fmaxf(m, pm);
    float alpha, pj[4];
    if (mn == -INFINITY) {
      alpha = 1.f;
      pj[0] = pj[1] = pj[2] = pj[3] = 0.f;
    } else {
      alpha = exp2f(m - mn);
#pragma unroll
      for (int j = 0; j < 4; ++j) pj[j] = valid[j] ? exp2f(z[j] - mn) : 0.f;
    }
    m = mn;
    float sk = 0.f, sd = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kept[j]) sk += pj[j];
      else sd += pj[j];
    }
    la = la * alpha + sk;
    ld = ld * alpha + sd;
    if (!LOGITS) {
      // ---- P V: lanes of row r own dims [col*DS, col*DS+DS) of keys 4r..4r+3 ----
      bool any = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) any |= kept[j];
      float av[GM];
      float pk[GM][4];
      for_g<GM>([&](int g) {
        av[g] = bcast_dyn(alpha, g);
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[g][j] = bcast_dyn(kept[j] ? pj[j] : 0.f, g);
      });
      for_g<GM>([&](int g) {
#pragma unroll
        for (int d = 0; d < DS; ++d) acc[g][d] *= av[g];
      });
      if (any) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (kept[j]) {
            const uint8_t* vrow = vbase + ((phys * PAGE + 4 * r + j) * D + col * DS) * 2;
            float vf[DS];
            if (DS == 8) {
              const uint4 vv = *reinterpret_cast<const uint4*>(vrow);
              vf[0] = bf16lo(vv.x); vf[1] = bf16hi(vv.x); vf[2] = bf16lo(vv.y); vf[3] = bf16hi(vv.y);
              vf[4] = bf16lo(vv.z); vf[5] = bf16hi(vv.z); vf[6] = bf16lo(vv.w); vf[7] = bf16hi(vv.w);
            } else {
              const uint2 vv = *reinterpret_cast<const uint2*>(vrow);
              vf[0] = bf16lo(vv.x); vf[1] = bf16hi(vv.x); vf[2] = bf16lo(vv.y); vf[3] = bf16hi(vv.y);
            }
            for_g<GM>([&](int g) {
#pragma unroll
              for (int d = 0; d < DS; ++d) acc[g][d] = fmaf(pk[g][j], vf[d], acc[g][d]);
            });
          }
        }
      }
    }
  }
  combine_streams<D, GM>(m, la, ld, acc, G, item, w, !LOGITS);
}

// ---------------------------------------------------------------------------
// fp32 K/V (any D in {64,128}, G <= 16): one thread per key of the item.
// ---------------------------------------------------------------------------
template <int D, bool LOGITS>
__global__ void __launch_bounds__(NT) k_attn_f32(AttnArgs a) {
  constexpr int NKEY = CHA * PAGE;  // 256 keys per item = one per thread
  __shared__ float sq[GMAX][D];
  __shared__ float sp[GMAX][NKEY];
  __shared__ float red[NT / WAVE];
  const AttnWs& w = a.w;
  const int item = blockIdx.x;
  if (item >= w.item_off[a.n_heads]) return;
  const int G = a.group;
  const int h = w.item_head[item];
  const int pbase = a.page_off[h];
  const int np = a.page_off[h + 1] - pbase;
  const int p0 = (item - w.item_off[h]) * CHA;
  const int n = a.len[h];
  const float* qf = (const float*)a.q;
  for (int i = threadIdx.x; i < G * D; i += NT) sq[i / D][i % D] = qf[(size_t)h * G * D + i];
  __syncthreads();
  const int t = threadIdx.x;
  const int p = p0 + t / PAGE;
  const int e = p * PAGE + t % PAGE;
  const bool valid = p < np && e < n;
  int64_t slot = 0;
  bool kept = valid;
  if (valid) {
    slot = (int64_t)a.page_ids[pbase + p] * PAGE + t % PAGE;
    if (!LOGITS && a.keep) kept = a.keep[(int64_t)(pbase + p) * PAGE + t % PAGE] != 0;
  }
  const float* krow = (const float*)a.k + slot * D;
  for (int g = 0; g < G; ++g) {
    float z = -INFINITY;
    if (valid) {
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(sq[g][d], krow[d], dot);
      z = dot * a.scale2;
      if (LOGITS) w.logits[(int64_t)g * a.plane + (int64_t)(pbase + p) * PAGE + t % PAGE] = z;
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
  if (LOGITS) return;
  const float* vb = (const float*)a.v;
  for (int i = t; i < G * D; i += NT) {
    const int g = i / D, d = i % D;
    float s = 0.f;
    for (int k = 0; k < NKEY; ++k) {
      const float pk = sp[g][k];
      if (pk != 0.f) {
        const int pp = p0 + k / PAGE;
        const int64_t sl = (int64_t)a.page_ids[pbase + pp] * PAGE + k % PAGE;
        s = fmaf(pk, vb[sl * D + d], s);
      }
    }
    w.acc[(size_t)item * G * D + i] = s;
  }
}

// Per query head: merge the partials of its KV head's items in order.
template <int D>
__global__ void __launch_bounds__(64) k_attn_merge(const AttnWs w, int group, const float* __restrict__ lse_ref,
                                                   float* __restrict__ out, float* __restrict__ dropped,
                                                   float* __restrict__ lse_out, float* __restrict__ lse2_out) {
  const int qh = blockIdx.x;
  const int h = qh / group, g = qh % group;
  const int b = w.item_off[h], e = w.item_off[h + 1];
  float M = -INFINITY;
  for (int it = b; it < e; ++it) M = fmaxf(M, w.stats[((size_t)it * group + g) * 3]);
  float la = 0.f, ld = 0.f;
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  for (int it = b; it < e; ++it) {
    const float* st = w.stats + ((size_t)it * group + g) * 3;
    const float sc = (M == -INFINITY) ? 0.f : exp2f(st[0] - M);
    la += st[1] * sc;
    ld += st[2] * sc;
    if (out) {
      const float* ac = w.acc + ((size_t)it * group + g) * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] += ac[threadIdx.x + 64 * k] * sc;
    }
  }
  if (out) {
    const float inv = la > 0.f ? 1.f / la : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) out[(size_t)qh * D + threadIdx.x + 64 * k] = acc[k] * inv;
  }
  if (threadIdx.x == 0) {
    const float l2 = la > 0.f ? M + log2f(la) : -INFINITY;  // base-2 LSE of the kept set
    const float lse = l2 * LN2;
    if (lse_out) lse_out[qh] = lse;
    if (lse2_out) lse2_out[qh] = l2;
    if (dropped) {
      float dm;
      if (lse_ref) dm = la > 0.f ? -expm1f(lse - lse_ref[qh]) : 1.f;
      else dm = (la + ld) > 0.f ? ld / (la + ld) : 1.f;
      if (!(la > 0.f)) dm = 1.f;
      dropped[qh] = dm;
    }
  }
}

// mass[j] = (1/G) sum_g 2^(z2_gj - lse2_g); NaN in padding slots
__global__ void __launch_bounds__(256) k_mass(const int32_t* __restrict__ page_off, const int32_t* __restrict__ len,
                                              int n_heads, int group, int64_t plane, const AttnWs w,
                                              float* __restrict__ mass) {
  const int64_t total = page_off[n_heads];
  const int64_t c = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  if (c >= total) return;
  const int h = upper_index(page_off, n_heads + 1, c);
  const int64_t i = (c - page_off[h]) * PAGE + j;
  const int64_t slot = c * PAGE + j;
  float out = qnan();
  if (i < len[h]) {
    float s = 0.f;
    for (int g = 0; g < group; ++g) s += exp2f(w.logits[(int64_t)g * plane + slot] - w.lse2[(size_t)h * group + g]);
    out = s / (float)group;
  }
  mass[slot] = out;
}

AttnWs carve(const trimkv_cache_t* c, int group, void* ws, bool mass) {
  WsLayout L = mass ? mass_ws_layout(c, group) : attn_ws_layout(c, group);
  char* b = (char*)ws;
  AttnWs w;
  w.item_off = (int32_t*)(b + L.off[0]);
  w.item_head = (int32_t*)(b + L.off[1]);
  w.stats = (float*)(b + L.off[2]);
  w.acc = (float*)(b + L.off[3]);
  w.lse2 = mass ? (float*)(b + L.off[4]) : nullptr;
  w.logits = mass ? (float*)(b + L.off[5]) : nullptr;
  return w;
}

int gm_for(int g) { return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : g <= 8 ? 8 : 16; }

template <bool LOGITS>
int launch_main(const trimkv_cache_t* c, AttnArgs& a, hipStream_t st) {
  const int64_t W = max_chunks(c, CHA);
  const dim3 grid((unsigned)W), blk(NT);
  if (c->dtype == TRIMKV_F32) {
    if (c->head_dim == 128) hipLaunchKernelGGL((k_attn_f32<128, LOGITS>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((k_attn_f32<64, LOGITS>), grid, blk, 0, st, a);
    return TRIMKV_OK;
  }
  const int gm = gm_for(a.group);
#define TRIMKV_BF16(DD, GG) hipLaunchKernelGGL((k_attn_bf16<DD, GG, LOGITS>), grid, blk, 0, st, a)
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
  const int64_t W = max_chunks(c, CHA);
  WsLayout L;
  L.add(((int64_t)c->n_heads + 1) * 4);
  L.add(W * 4);
  L.add(W * group * 3 * 4);
  L.add(W * group * (int64_t)c->head_dim * 4);
  return L;
}

WsLayout mass_ws_layout(const trimkv_cache_t* c, int group) {
  const int64_t W = max_chunks(c, CHA);
  WsLayout L;
  L.add(((int64_t)c->n_heads + 1) * 4);
  L.add(W * 4);
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
  hipLaunchKernelGGL(k_attn_prep, dim3(1), dim3(1024), 0, st, c->page_off, c->n_heads, w);
  AttnArgs a{c->page_off, c->page_ids, c->len, c->k, c->v, keep, q, c->n_heads, group, scale * LOG2E,
             c->n_pages * PAGE, w};
  int rc = launch_main<false>(c, a, st);
  if (rc) return rc;
  const int nq = c->n_heads * group;
  if (c->head_dim == 128)
    hipLaunchKernelGGL(k_attn_merge<128>, dim3(nq), dim3(64), 0, st, w, group, lse_ref, out, dropped, lse_out,
                       (float*)nullptr);
  else
    hipLaunchKernelGGL(k_attn_merge<64>, dim3(nq), dim3(64), 0, st, w, group, lse_ref, out, dropped, lse_out,
                       (float*)nullptr);
  return check_launch();
}

int launch_attn_mass(const trimkv_cache_t* c, const void* q, int group, float scale, float* mass,
                     float* lse_full, void* ws, hipStream_t st) {
  AttnWs w = carve(c, group, ws, true);
  hipLaunchKernelGGL(k_attn_prep, dim3(1), dim3(1024), 0, st, c->page_off, c->n_heads, w);
  AttnArgs a{c->page_off, c->page_ids, c->len, c->k, c->v, nullptr, q, c->n_heads, group, scale * LOG2E,
             c->n_pages * PAGE, w};
  int rc = launch_main<true>(c, a, st);
  if (rc) return rc;
  const int nq = c->n_heads * group;
  if (c->head_dim == 128)
    hipLaunchKernelGGL(k_attn_merge<128>, dim3(nq), dim3(64), 0, st, w, group, (const float*)nullptr,
                       (float*)nullptr, (float*)nullptr, lse_full, w.lse2);
  else
    hipLaunchKernelGGL(k_attn_merge<64>, dim3(nq), dim3(64), 0, st, w, group, (const float*)nullptr,
                       (float*)nullptr, (float*)nullptr, lse_full, w.lse2);
  const int64_t blocks = (c->n_pages + 15) / 16;
  hipLaunchKernelGGL(k_mass, dim3((unsigned)blocks), dim3(256), 0, st, c->page_off, c->len, c->n_heads, group,
                     c->n_pages * PAGE, w, mass);
  return check_launch();
}

}  // namespace trimkv
