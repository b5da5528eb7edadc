// Row quantizers shared by the append, re-tier and prologue kernels: group reductions over the
// lanes of a 128-channel row (32 lanes, 4 channels each; a group of g channels spans g/4
// lanes), the outlier predicate and the fits of every storage format.
//
// "Hierarchical Token Routing and Sub-2-Bit Non-Linear KV Compression ...", section
// "Paradigm 2": outliers beyond tau standard deviations kept apart at higher precision, the
// rest coded against a 4-centroid codebook fitted by k-means; "The Sub-10ms Barrier ...",
// section "2. FP4/INT4 KV-Cache Quantization": per-group scale (max - min)/(2^b - 1);
// "Hierarchical Token Gating and Tiered KV-Cache Paging ...", section "2. Entropy-Guided
// Tiered KV-Cache Quantization": FP8 tier rows.
//
// Bit-exactness contract: every decision is taken in float32 with round-to-nearest-even, no
// fused multiply-add (contraction is off from here to the end of every file that includes this
// one), correctly rounded division, and every sum over a group follows one fixed pairwise tree:
// for w = g/2, g/4, ..., 1: a[i] += a[i + w] for i < w.  With L = g/4 lanes per group and lane
// j holding group elements j, j+L, j+2L, j+3L, the steps w = 2L and w = L are in-lane and the
// steps w < L are xor exchanges between lanes (every lane then holds the root by commutativity
// of addition).
#pragma once
#pragma clang fp contract(off)

#include <type_traits>

#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kRowLanes = 32;  // lanes per row: 128 channels, 4 per lane

// compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// ---------------------------------------------------------------- group reductions
template <int L>
__device__ __forceinline__ float group_sum_tree(float a0, float a1, float a2, float a3) {
  float t = (a0 + a2) + (a1 + a3);   // tree steps w = 2L, w = L
  if constexpr (L >= 32) t = t + xor_f32<16>(t);
  if constexpr (L >= 16) t = t + xor_f32<8>(t);
  if constexpr (L >= 8) t = t + xor_f32<4>(t);
  if constexpr (L >= 4) t = t + xor_f32<2>(t);
  if constexpr (L >= 2) t = t + xor_f32<1>(t);
  return t;
}
template <int L>
__device__ __forceinline__ int group_isum(int v) {
  if constexpr (L >= 32) v += xor_i32<16>(v);
  if constexpr (L >= 16) v += xor_i32<8>(v);
  if constexpr (L >= 8) v += xor_i32<4>(v);
  if constexpr (L >= 4) v += xor_i32<2>(v);
  if constexpr (L >= 2) v += xor_i32<1>(v);
  return v;
}
template <int L>
__device__ __forceinline__ int group_ior(int v) {
  if constexpr (L >= 32) v |= xor_i32<16>(v);
  if constexpr (L >= 16) v |= xor_i32<8>(v);
  if constexpr (L >= 8) v |= xor_i32<4>(v);
  if constexpr (L >= 4) v |= xor_i32<2>(v);
  if constexpr (L >= 2) v |= xor_i32<1>(v);
  return v;
}
template <int L>
__device__ __forceinline__ float group_min(float v) {
  if constexpr (L >= 32) v = fminf(v, xor_f32<16>(v));
  if constexpr (L >= 16) v = fminf(v, xor_f32<8>(v));
  if constexpr (L >= 8) v = fminf(v, xor_f32<4>(v));
  if constexpr (L >= 4) v = fminf(v, xor_f32<2>(v));
  if constexpr (L >= 2) v = fminf(v, xor_f32<1>(v));
  return v;
}
template <int L>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (L >= 32) v = fmaxf(v, xor_f32<16>(v));
  if constexpr (L >= 16) v = fmaxf(v, xor_f32<8>(v));
  if constexpr (L >= 8) v = fmaxf(v, xor_f32<4>(v));
  if constexpr (L >= 4) v = fmaxf(v, xor_f32<2>(v));
  if constexpr (L >= 2) v = fmaxf(v, xor_f32<1>(v));
  return v;
}

// lane Q of the lane's quad (DPP quad_perm [Q, Q, Q, Q])
template <int Q>
__device__ __forceinline__ float quad_bcast_f32(float v) {
  return as_f32((uint32_t)__builtin_amdgcn_mov_dpp((int)as_u32(v), Q * 0x55, 0xF, 0xF, false));
}

// ---------------------------------------------------------------- per-row state
struct RowOut {
  uint32_t code[4];   // per element
  uint32_t flag[4];   // outlier flags
  uint32_t meta[2];   // group metadata held by the group's lane 0 (up to 8 bytes)
};

// nearest of 4 centroids by |x - c| (fl32), first index on ties
__device__ __forceinline__ uint32_t nearest4(float x, const float c[4]) {
  float best = __builtin_fabsf(x - c[0]);
  uint32_t k = 0;
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    const float d = __builtin_fabsf(x - c[j]);
    if (d < best) { best = d; k = (uint32_t)j; }
  }
  return k;
}

// Outlier predicate: e * (g-1) > fl32(tau^2) * Q2 with e = (x - mean)^2, Q2 = sum of e.
template <int G>
__device__ __forceinline__ void outlier_flags(const float x[4], float tau2, bool keep[4]) {
  constexpr int L = G / 4;
  const float mean = group_sum_tree<L>(x[0], x[1], x[2], x[3]) * (1.0f / (float)G);
  float e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { const float d = x[i] - mean; e[i] = d * d; }
  const float q2 = group_sum_tree<L>(e[0], e[1], e[2], e[3]);
  const float rhs = tau2 * q2;
#pragma unroll
  for (int i = 0; i < 4; ++i) keep[i] = !(e[i] * (float)(G - 1) > rhs);
}

// Asymmetric integer fit ("The Sub-10ms Barrier ...", section "2. FP4/INT4 KV-Cache
// Quantization"): S = (max - min) / (2^b - 1) over the non-outliers, fp16 S and zero =
// fp16(min), code = rint(clamp((x - z) / S)).  LEVELS = 2^b - 1: 15 for INT4, 7 for the
// asymmetric 3-bit codes of "Sub-5ms MoE Inference ...", section "Sub-Byte KV-Cache
// Quantization".
template <int G, int LEVELS = 15>
__device__ __forceinline__ void fit_int4(const float x[4], const bool keep[4], RowOut& o) {
  constexpr int L = G / 4;
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (keep[i]) { mn = fminf(mn, x[i]); mx = fmaxf(mx, x[i]); }
  mn = group_min<L>(mn) + 0.0f;  // a zero minimum is taken as +0
  mx = group_max<L>(mx) + 0.0f;
  const float s = (mx - mn) / (float)LEVELS;
  const uint32_t sh = f32_to_half_bits(s), zh = f32_to_half_bits(mn);
  const float S = half_bits_to_f32(sh), Z = half_bits_to_f32(zh);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float xx = keep[i] ? x[i] : 0.0f;
    uint32_t q = 0;
    if (S > 0.0f) {
      const float y = (xx - Z) / S;
      q = (uint32_t)__builtin_rintf(fminf(fmaxf(y, 0.0f), (float)LEVELS));
    }
    o.code[i] = q;
  }
  o.meta[0] = sh | (zh << 16);
  o.meta[1] = 0;
}

template <int G>
__device__ __forceinline__ void fit_fp4(const float x[4], const bool keep[4], RowOut& o) {
  constexpr int L = G / 4;
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (keep[i]) a = fmaxf(a, __builtin_fabsf(x[i]));
  a = group_max<L>(a);
  const uint32_t s8 = f32_to_e4m3(a / 6.0f);
  const float sv = e4m3_to_f32(s8);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float xx = keep[i] ? x[i] : 0.0f;
    o.code[i] = sv > 0.0f ? f32_to_e2m1(xx / sv) : 0u;
  }
  o.meta[0] = s8;
  o.meta[1] = 0;
}

// Symmetric INT4 ("The Sub-10ms Barrier ...", section "2. FP4/INT4 KV-Cache Quantization", the
// quantize_kv_cache_fp4 listing): scale absmax/7 over the non-outliers, at least 1e-5, stored as
// fp16 S; code = clamp(round(x / S), -8, 7) + 8, stored as INT4 with zero -8 S.
template <int G>
__device__ __forceinline__ void fit_int4sym(const float x[4], const bool keep[4], RowOut& o) {
  constexpr int L = G / 4;
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (keep[i]) a = fmaxf(a, __builtin_fabsf(x[i]));
  a = group_max<L>(a);
  const uint32_t sh = f32_to_half_bits(fmaxf(a / 7.0f, 1e-5f));
  const float S = half_bits_to_f32(sh);
  const uint32_t zh = f32_to_half_bits(-8.0f * S);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float xx = keep[i] ? x[i] : 0.0f;
    o.code[i] = (uint32_t)((int)fminf(fmaxf(__builtin_rintf(xx / S), -8.0f), 7.0f) + 8);
  }
  o.meta[0] = sh | (zh << 16);
  o.meta[1] = 0;
}

// Uniform 2-bit codebook ("Hierarchical Token Routing and Sub-2-Bit Non-Linear KV Compression
// ...", the compress_kv_head listing): the group's values with the outlier slots set to 0, 4
// centroids linspace(min, max) formed as torch.linspace does (step fl32((max - min) / 3); min,
// min + step, max - step, max), fp16 centroids, nearest centroid (first index on ties).
template <int G>
__device__ __forceinline__ void fit_u2(const float x[4], const bool keep[4], RowOut& o) {
  constexpr int L = G / 4;
  float xx[4], mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xx[i] = keep[i] ? x[i] : 0.0f;
    mn = fminf(mn, xx[i]);
    mx = fmaxf(mx, xx[i]);
  }
  mn = group_min<L>(mn) + 0.0f;  // a zero end is taken as +0
  mx = group_max<L>(mx) + 0.0f;
  const float step = (mx - mn) / 3.0f;
  const float c[4] = {mn, mn + step, mx - step, mx};
  uint32_t hb[4];
  float ch[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { hb[j] = f32_to_half_bits(c[j]); ch[j] = half_bits_to_f32(hb[j]); }
#pragma unroll
  for (int i = 0; i < 4; ++i) o.code[i] = nearest4(xx[i], ch);
  o.meta[0] = hb[0] | (hb[1] << 16);
  o.meta[1] = hb[2] | (hb[3] << 16);
}

// 2-bit centroids: seeds at ranks floor((2j+1) n / 8) of the sorted non-outliers, then
// `iters` Lloyd iterations (empty clusters keep their centroid), fp16 centroids.
template <int G>
__device__ __forceinline__ void fit_c2(const float x[4], const bool keep[4], int jg, int iters, RowOut& o) {
  constexpr int L = G / 4;
  int nloc = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) nloc += keep[i] ? 1 : 0;
  const int n = group_isum<L>(nloc);
  // stable rank of each kept element among the kept elements of the group: element (src, e)
  // of the group (index src + L e, broadcast from lane src of the 16-lane row that holds the
  // group) precedes my element i (index jg + L i) when it is smaller, or equal with a lower
  // index.  Outliers compare as +inf, which precedes no kept element.
  static_assert(G == 64, "one group per 16-lane DPP row");
  float xs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xs[i] = keep[i] ? x[i] : INFINITY;
  int rank[4] = {0, 0, 0, 0};
  const uint32_t xb[4] = {as_u32(x[0]), as_u32(x[1]), as_u32(x[2]), as_u32(x[3])};
  static_for<L>([&](auto src_c) {
    constexpr int src = decltype(src_c)::value;
    const bool before_me = src < jg;   // same e: the source's index is lower when src < jg
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = as_f32((uint32_t)row_bcast_i32<src>((int)as_u32(xs[e])));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool less = e < i ? v <= xs[i] : e > i ? v < xs[i] : (before_me ? v <= xs[i] : v < xs[i]);
        rank[i] += less ? 1 : 0;
      }
    }
  });
  float c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = ((2 * j + 1) * n) >> 3;
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) bits |= (keep[i] && rank[i] == r) ? xb[i] : 0u;
    c[j] = as_f32((uint32_t)group_ior<L>((int)bits));
  }
  // Each Lloyd iteration: the members' sums by the fixed tree, the four member counts in one
  // reduction (a byte each: a group has at most 64 members), and the four divisions spread
  // over the lanes of each quad (lane jg computes centroid jg % 4; a quad broadcast gives every
  // lane all four), the same correctly rounded quotients in fewer instructions.
  const int jq = jg & 3;
  for (int it = 0; it < iters; ++it) {
    uint32_t a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = nearest4(x[i], c);
    uint32_t pk = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) pk += keep[i] ? 1u << (8u * a[i]) : 0u;
    const uint32_t cnts = (uint32_t)group_isum<L>((int)pk);
    float sum[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = keep[i] && a[i] == (uint32_t)j ? x[i] : 0.0f;
      sum[j] = group_sum_tree<L>(s[0], s[1], s[2], s[3]);
    }
    const float my_sum = jq == 0 ? sum[0] : jq == 1 ? sum[1] : jq == 2 ? sum[2] : sum[3];
    const float my_c = jq == 0 ? c[0] : jq == 1 ? c[1] : jq == 2 ? c[2] : c[3];
    const int my_cnt = (int)((cnts >> (8 * jq)) & 0xFFu);
    const float my_nc = my_cnt > 0 ? my_sum / (float)my_cnt : my_c;
    c[0] = quad_bcast_f32<0>(my_nc);
    c[1] = quad_bcast_f32<1>(my_nc);
    c[2] = quad_bcast_f32<2>(my_nc);
    c[3] = quad_bcast_f32<3>(my_nc);
  }
  uint32_t hb[4];
  float ch[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) { hb[j] = f32_to_half_bits(c[j]); ch[j] = half_bits_to_f32(hb[j]); }
#pragma unroll
  for (int i = 0; i < 4; ++i) o.code[i] = nearest4(keep[i] ? x[i] : 0.0f, ch);
  o.meta[0] = hb[0] | (hb[1] << 16);
  o.meta[1] = hb[2] | (hb[3] << 16);
}

// FP8 tier row: scale = absmax/448 over the 128 channels (1 if zero), codes E4M3(x/scale)
__device__ __forceinline__ void fit_fp8row(const float x[4], RowOut& o) {
  float a = fmaxf(fmaxf(__builtin_fabsf(x[0]), __builtin_fabsf(x[1])),
                  fmaxf(__builtin_fabsf(x[2]), __builtin_fabsf(x[3])));
  a = group_max<32>(a);
  const float s = a > 0.0f ? a / 448.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) { o.code[i] = f32_to_e4m3(x[i] / s); o.flag[i] = 0; }
  o.meta[0] = as_u32(s);
  o.meta[1] = 0;
}

// One row's quantization (32 lanes; lane = gi * (G / 4) + jg holds channels gi * G + jg + (G / 4) e,
// e = 0..3): the FP8-tier row fit, or outlier isolation (the static channel mask of list
// (kv, h) when the cache has one, else the tau predicate) followed by the format's fit.
// o.flag[e] = 1 for an outlier.
template <int FMT, int G>
__device__ __forceinline__ void quantize_row(const float x[4], int tier1, const uint32_t* chan_mask,
                                             int outl, float tau2, int fit, int lloyd, int kv,
                                             int h, int H, int gi, int jg, RowOut& o) {
  constexpr int L = G / 4;
  // the flags are set once, after the branches, from keep (all kept in an FP8-tier row)
  bool keep[4] = {true, true, true, true};
  if (tier1) {
    fit_fp8row(x, o);
  } else {
    if (outl != KVQ_OUTL_NONE) {
      if (chan_mask) {   // static channel mask: the masked channels are the outliers
        const uint32_t* mw = chan_mask + ((size_t)kv * H + h) * (kHeadDim / 32);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = gi * G + jg + L * e;
          keep[e] = ((mw[c >> 5] >> (c & 31)) & 1u) == 0u;
        }
      } else {
        outlier_flags<G>(x, tau2, keep);
      }
    }
    if constexpr (FMT == FMT_INT4) {
      if (fit == kFitSym) fit_int4sym<G>(x, keep, o);
      else fit_int4<G>(x, keep, o);
    } else if constexpr (FMT == FMT_INT3) {
      fit_int4<G, 7>(x, keep, o);
    } else if constexpr (FMT == FMT_FP4) {
      fit_fp4<G>(x, keep, o);
    } else {
      if (fit == kFitUniform) fit_u2<G>(x, keep, o);
      else fit_c2<G>(x, keep, jg, lloyd, o);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) o.flag[e] = keep[e] ? 0u : 1u;
}

// 32-bit word `w` of a packed row from its 128 codes (one byte each), for `bits` = 2, 4 or 8
// (2-bit: channel 4s + j of the word's 16 in byte j, bit pair s; otherwise LSB first) and 3 (one
// LSB-first bit stream: channel c in stream bits 3c .. 3c + 2; word w holds stream bits 32 w ..
// 32 w + 31, the channels that start in it and the head of one that starts in the word before)
__device__ __forceinline__ uint32_t pack_word(const uint8_t* code, int w, int bits) {
  uint32_t out = 0;
  if (bits == 3) {
    const int c0 = (32 * w) / 3, c1 = (32 * w + 31) / 3;
    for (int c = c0; c <= c1; ++c) {
      const int sh = 3 * c - 32 * w;
      const uint32_t v = code[c];
      out |= sh >= 0 ? v << sh : v >> -sh;
    }
    return out;
  }
  const int per_word = 32 / bits;
  for (int k = 0; k < per_word; ++k) {
    const int sh = bits == 2 ? 8 * (k & 3) + 2 * (k >> 2) : bits * k;
    out |= (uint32_t)code[w * per_word + k] << sh;
  }
  return out;
}

// ---------------------------------------------------------------- appending a row to a list
// The helpers below take any launch descriptor `a` with the fields L (Layout), cache
// (kvq_cache), block_table, outl, tau2, fit and lloyd.

// LDS staging of the rows quantized together (NS row slots of 32 lanes)
template <int NS>
struct RowStage {
  uint8_t code[NS][kHeadDim];
  uint8_t flag[NS][kHeadDim];
  float x[NS][kHeadDim];
  uint32_t meta[NS][8];
};

// The records of list (b, h, kv) of tokens < t: those before t's 16-token block plus those of
// the block's rows before t (a block holds at most 16 rows of D records, and the list is sorted,
// so each of the n lanes stops at its first record of a token >= t); the lanes' counts are
// summed over the n-lane group (n a power of two, aligned in the wave).
template <int N, class A>
__device__ int64_t records_before(const A& a, int b, int h, int kv, int t, int lane) {
  const Layout& Lo = a.L;
  int64_t start = 0;
  int cnt = 0;
  if (t > 0) {
    const size_t lid = list_id(Lo, b, h, kv);
    const uint32_t* oidx = a.cache.outl_idx[kv] + ((size_t)b * Lo.H + h) * (size_t)Lo.outl_cap;
    start = max((int64_t)0, min((int64_t)a.cache.outl_block_start[lid * (size_t)Lo.nblk + ((t - 1) >> 4)],
                                Lo.outl_cap));
    const int64_t old = max((int64_t)0, min((int64_t)a.cache.outl_count[lid], Lo.outl_cap));
    const int64_t lim = min(old, start + (int64_t)kBlock * kHeadDim);
    for (int64_t r = start + lane; r < lim; r += N) {
      if (oidx[r] >= (uint32_t)t * kHeadDim) break;
      ++cnt;
    }
  }
#pragma unroll
  for (int o = N / 2; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, N);
  return start + cnt;
}

// Appends one token's row (32 lanes of one slot; lane = gi * (G / 4) + jg holds channels
// gi * G + jg + (G / 4) e) to list (b, h, kv) at token t, after the `running` records of tokens
// < t (the list is cut back to them): the row is quantized (FP8 tier or outlier isolation + fit),
// its codes and metadata are written to its row slot and its outlier records appended in channel
// order.  sync() orders the staging's LDS accesses between the lanes that call this together
// (a workgroup barrier when the slots span waves; a wave fence when they share one wave): every
// lane of those calls it once per round, and the staging is free again on return.  `valid` false:
// the slot has no row this round.  Returns the list's record count after the row.
template <int FMT, int G, class A, int NS, class Sync>
__device__ int64_t append_row(const A& a, bool valid, int b, int h, int kv, int t, int64_t running,
                              const float x[4], int lane, int slot, RowStage<NS>& st, Sync sync) {
  constexpr int L = G / 4;
  constexpr int CB = kHeadDim * code_bits(FMT) / 8;
  const Layout& Lo = a.L;
  const int gi = lane / L, jg = lane % L;
  if (valid && t >= Lo.S_cap) {
    if (lane == 0) report(a.cache.status, KVQ_ERR_INVALID_ARG);
    valid = false;
  }
  const size_t lid = list_id(Lo, b, h, kv);
  int32_t* bstart = a.cache.outl_block_start + lid * (size_t)Lo.nblk;
  uint32_t* oidx = a.cache.outl_idx[kv] + ((size_t)b * Lo.H + h) * (size_t)Lo.outl_cap;
  uint8_t* oval = (uint8_t*)a.cache.outl_val[kv] +
                  ((size_t)b * Lo.H + h) * (size_t)Lo.outl_cap * (a.outl == KVQ_OUTL_FP16 ? 2 : 1);

  int tier1 = 0;
  size_t pslot = 0;
  bool row_ok = valid;
  if (Lo.paged && valid) {
    row_ok = page_slot(Lo, a.block_table, b, t, &tier1, &pslot);
    if (!row_ok && lane == 0) report(a.cache.status, KVQ_ERR_INVALID_ARG);
  }
  RowOut o;
  quantize_row<FMT, G>(x, tier1, a.cache.chan_mask, a.outl, a.tau2, a.fit, a.lloyd, kv, h, Lo.H, gi,
                       jg, o);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = gi * G + jg + L * e;
    st.code[slot][c] = (uint8_t)o.code[e];
    st.flag[slot][c] = valid ? (uint8_t)o.flag[e] : 0;
    st.x[slot][c] = x[e];
  }
  if (tier1) {
    if (lane == 0) st.meta[slot][0] = o.meta[0];
  } else if (jg == 0) {
    constexpr int MB = meta_bytes_per_group(FMT);
    if constexpr (MB == 8) { st.meta[slot][2 * gi] = o.meta[0]; st.meta[slot][2 * gi + 1] = o.meta[1]; }
    else if constexpr (MB == 4) { st.meta[slot][gi] = o.meta[0]; }
    else { ((uint8_t*)st.meta[slot])[gi] = (uint8_t)o.meta[0]; }
  }
  sync();

  if (row_ok) {
    uint8_t* codes_dst;
    uint8_t* meta_dst;
    int cb, mb;
    if (!Lo.paged) {
      const size_t row = ((size_t)b * Lo.H + h) * (size_t)Lo.S_cap + (size_t)t;
      codes_dst = (uint8_t*)a.cache.codes[kv] + row * CB;
      meta_dst = (uint8_t*)a.cache.meta[kv] + row * Lo.meta_bytes;
      cb = CB; mb = Lo.meta_bytes;
    } else {
      const size_t prow = (pslot * Lo.H + h) * kBlock + (t & 15);
      if (tier1) {
        codes_dst = (uint8_t*)a.cache.codes8[kv] + prow * kHeadDim;
        meta_dst = (uint8_t*)(a.cache.scale8[kv] + prow);
        cb = kHeadDim; mb = 4;
      } else {
        codes_dst = (uint8_t*)a.cache.codes[kv] + prow * CB;
        meta_dst = (uint8_t*)a.cache.meta[kv] + prow * Lo.meta_bytes;
        cb = CB; mb = Lo.meta_bytes;
      }
    }
    const int bits = tier1 ? 8 : code_bits(FMT);
    if (lane < cb / 4) ((uint32_t*)codes_dst)[lane] = pack_word(st.code[slot], lane, bits);
    if (lane < mb / 4) ((uint32_t*)meta_dst)[lane] = st.meta[slot][lane];
    else if (mb < 4 && lane == 0) {
      for (int k = 0; k < mb; ++k) meta_dst[k] = ((uint8_t*)st.meta[slot])[k];
    }
  }

  // the row's outlier records in channel order: channels 4 lane .. 4 lane + 3
  uint32_t fl = 0;
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t f = st.flag[slot][4 * lane + k];
    fl |= f << k;
    cnt += (int)f;
  }
  int incl = cnt;
#pragma unroll
  for (int dd = 1; dd < kRowLanes; dd <<= 1) {
    const int y = __shfl_up(incl, dd, kRowLanes);
    if (lane >= dd) incl += y;
  }
  const int total = __shfl(incl, kRowLanes - 1, kRowLanes);
  const int64_t count = min(running + total, Lo.outl_cap);
  if (valid) {
    if ((t & 15) == 0 && lane == 0) bstart[t >> 4] = (int32_t)min(running, (int64_t)INT32_MAX);
    int64_t k = running + (incl - cnt);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if ((fl >> q) & 1u) {
        const int c = 4 * lane + q;
        if (k < Lo.outl_cap) {
          oidx[k] = (uint32_t)t * kHeadDim + (uint32_t)c;
          const float xv = st.x[slot][c];
          if (a.outl == KVQ_OUTL_FP16) ((uint16_t*)oval)[k] = (uint16_t)f32_to_half_bits(xv);
          else oval[k] = (uint8_t)f32_to_e4m3(xv);
        } else {
          report(a.cache.status, KVQ_ERR_CAPACITY);
        }
        ++k;
      }
    }
    if (lane == 0) a.cache.outl_count[lid] = (int32_t)count;
  }
  sync();   // the staging is reused by the next round
  return count;
}

}  // namespace
}  // namespace kvq
