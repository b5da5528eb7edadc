// Fused dequantize + flash-decoding attention, VALU (fp32) variant for every format and
// layout, plus the log-sum-exp merge of split-K partials.
//
// "Hierarchical Token Routing and Sub-2-Bit Non-Linear KV Compression ...", section
// "Hardware-Kernel Fusion: Eliminating DRAM Round-Trips": compressed codes are streamed from
// HBM and expanded on chip, never written back dequantized; "The Sub-10ms Barrier ...",
// figure in "The Twin Bottlenecks": the attention phase is a flash-decoding engine fed by the
// quantized cache.  Chunks of tokens produce partial (max, sum, unnormalized output) states
// that a second kernel merges by log-sum-exp.
//
// Work unit: one workgroup per (chunk, KV head, sequence) holding the GQA group's query rows.
// Each 64-token step dequantizes K and V rows into LDS as fp32 (outlier positions overwritten
// from the side lists), computes scores in fp32, updates the online softmax and accumulates
// P.V in fp32.  Exact fp32 dequantization makes this the path for formats whose values are
// not fp16-representable (INT4 scale * code + zero).  Short contexts make it latency-bound, so
// the dependent loads are few: the queries go out with the sequence length, each step's
// outlier bounds and first records with its codes.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

constexpr int kT = 64;      // tokens per step
constexpr int kStride = kHeadDim + 1;
constexpr int kMaxRows = 16;

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return as_f32((uint32_t)v << 16); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) v = fmaxf(v, __shfl_xor(v, w, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) v += __shfl_xor(v, w, 64);
  return v;
}

// dequantize channels [32*part, 32*part + 32) of one row into dst (fp32)
template <int FMT, int GS>
__device__ __forceinline__ void dequant32(const RowRef& r, int part, float* dst) {
  if (r.tier1) {
    const uint32_t* cw = (const uint32_t*)(r.codes + 32 * part);
    const float s = *(const float*)r.meta;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t u = cw[w];
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[4 * w + k] = e4m3_to_f32((u >> (8 * k)) & 0xFFu) * s;
    }
    return;
  }
  if constexpr (FMT == FMT_C2) {
    const uint2 cw = *(const uint2*)(r.codes + 8 * part);
    const uint2 mw = *(const uint2*)(r.meta + 8 * (part >> 1));
    const float c[4] = {half_bits_to_f32(mw.x & 0xFFFFu), half_bits_to_f32(mw.x >> 16),
                        half_bits_to_f32(mw.y & 0xFFFFu), half_bits_to_f32(mw.y >> 16)};
    // channel 4s + j of a 16-channel word sits in byte j, bit pair s
#pragma unroll
    for (int k = 0; k < 16; ++k) dst[k] = c[(cw.x >> (8 * (k & 3) + 2 * (k >> 2))) & 3u];
#pragma unroll
    for (int k = 0; k < 16; ++k) dst[16 + k] = c[(cw.y >> (8 * (k & 3) + 2 * (k >> 2))) & 3u];
  } else if constexpr (FMT == FMT_INT3) {
    // 32 channels = 96 stream bits = words 3 part .. 3 part + 2; channel c at stream bit 3c
    const uint32_t* cp = (const uint32_t*)(r.codes + 12 * part);
    const uint32_t w[4] = {cp[0], cp[1], cp[2], 0u};
    const int gi = (32 * part) / GS;
    const uint32_t m = *(const uint32_t*)(r.meta + 4 * gi);
    const float S = half_bits_to_f32(m & 0xFFFFu), Z = half_bits_to_f32(m >> 16);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int o = 3 * k, i = o >> 5, sh = o & 31;
      const uint32_t v = sh > 29 ? (w[i] >> sh) | (w[i + 1] << (32 - sh)) : w[i] >> sh;
      dst[k] = fmaf((float)(v & 7u), S, Z);
    }
  } else {
    const uint4 cw = *(const uint4*)(r.codes + 16 * part);
    const uint32_t wv[4] = {cw.x, cw.y, cw.z, cw.w};
    const int gi = (32 * part) / GS;
    if constexpr (FMT == FMT_INT4) {
      const uint32_t m = *(const uint32_t*)(r.meta + 4 * gi);
      const float S = half_bits_to_f32(m & 0xFFFFu), Z = half_bits_to_f32(m >> 16);
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[8 * w + k] = fmaf((float)((wv[w] >> (4 * k)) & 15u), S, Z);
    } else {  // FP4
      const float s = e4m3_to_f32(r.meta[gi]);
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[8 * w + k] = e2m1_to_f32((wv[w] >> (4 * k)) & 15u) * s;
    }
  }
}

__device__ __forceinline__ float outlier_value(const void* vals, int64_t i, int outl) {
  if (outl == KVQ_OUTL_FP16) return half_bits_to_f32(((const uint16_t*)vals)[i]);
  return e4m3_to_f32(((const uint8_t*)vals)[i]);
}

template <int FMT, int GS>
__global__ void __launch_bounds__(256) decode_generic_kernel(DecodeLaunch d) {
  __shared__ float s_q[kMaxRows][kHeadDim];
  __shared__ float s_k[kT][kStride];
  __shared__ float s_v[kT][kStride];
  __shared__ float s_s[kMaxRows][kT];
  __shared__ float s_alpha[kMaxRows];
  __shared__ float s_m[kMaxRows];
  __shared__ float s_l[kMaxRows];

  const Layout& L = d.L;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = d.Hq / L.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // the group's query rows (contiguous in q) are loaded with the sequence length
  float qv[kMaxRows * kHeadDim / 256];
  const uint16_t* qg = d.q + ((size_t)b * d.Hq + (size_t)h * G) * kHeadDim;
#pragma unroll
  for (int k = 0; k < kMaxRows * kHeadDim / 256; ++k) {
    const int i = tid + 256 * k;
    qv[k] = i < G * kHeadDim ? bf16_to_f32(qg[i]) : 0.0f;
  }
  const int S = d.seq_lens[b];
  if (S < 1 || S > L.S_cap) {
    if (threadIdx.x == 0 && chunk == 0 && h == 0) report(d.cache.status, KVQ_ERR_INVALID_ARG);
    return;
  }
  const int t0 = chunk * d.chunk;
  if (t0 >= S) return;
  const int t1 = min(t0 + d.chunk, S);

#pragma unroll
  for (int k = 0; k < kMaxRows * kHeadDim / 256; ++k) {
    const int i = tid + 256 * k;
    if (i < G * kHeadDim) s_q[i / kHeadDim][i % kHeadDim] = qv[k];
  }
  if (tid < kMaxRows) { s_m[tid] = -INFINITY; s_l[tid] = 0.0f; }
  float o[kMaxRows / 2];
#pragma unroll
  for (int k = 0; k < kMaxRows / 2; ++k) o[k] = 0.0f;

  const size_t lidK = list_id(L, b, h, 0), lidV = lidK + 1;
  const int32_t* bsK = d.cache.outl_block_start + lidK * (size_t)L.nblk;
  const int32_t* bsV = d.cache.outl_block_start + lidV * (size_t)L.nblk;
  const size_t lbase = ((size_t)b * L.H + h) * (size_t)L.outl_cap;
  const size_t vbytes = d.outl == KVQ_OUTL_FP16 ? 2 : 1;
  __syncthreads();

  const bool has_outl = d.outl != KVQ_OUTL_NONE;
  const int64_t cntK = has_outl ? d.cache.outl_count[lidK] : 0;
  const int64_t cntV = has_outl ? d.cache.outl_count[lidV] : 0;
  const uint32_t* idxK = d.cache.outl_idx[0] + lbase;
  const uint32_t* idxV = d.cache.outl_idx[1] + lbase;
  const void* valsK = (const uint8_t*)d.cache.outl_val[0] + lbase * vbytes;
  const void* valsV = (const uint8_t*)d.cache.outl_val[1] + lbase * vbytes;
  constexpr uint32_t kNoRec = 0xFFFFFFFFu;

  for (int ts = t0; ts < t1; ts += kT) {
    const int te = min(ts + kT, t1);
    // the step's outlier records [r0, r1) of K and V, and each thread's first record of each
    int64_t rk0 = 0, rk1 = 0, rv0 = 0, rv1 = 0;
    uint32_t fk = kNoRec, fv = kNoRec;
    float vk = 0.0f, vv = 0.0f;
    if (has_outl) {
      rk0 = max((int64_t)0, min((int64_t)bsK[ts >> 4], L.outl_cap));
      rk1 = max(rk0, min((te < S) ? (int64_t)bsK[te >> 4] : cntK, L.outl_cap));
      rv0 = max((int64_t)0, min((int64_t)bsV[ts >> 4], L.outl_cap));
      rv1 = max(rv0, min((te < S) ? (int64_t)bsV[te >> 4] : cntV, L.outl_cap));
      if (rk0 + tid < rk1) { fk = idxK[rk0 + tid]; vk = outlier_value(valsK, rk0 + tid, d.outl); }
      if (rv0 + tid < rv1) { fv = idxV[rv0 + tid]; vv = outlier_value(valsV, rv0 + tid, d.outl); }
    }
    {  // dequantize 64 rows of K and V: thread -> (token tid/4, 32 channels)
      const int tt = tid >> 2, part = tid & 3;
      float buf[32];
      const int t = ts + tt;
      const RowRef rk = row_ref(L, d.cache, 0, b, h, t < te ? t : ts, d.block_table);
      if (t < te && rk.ok) {
        dequant32<FMT, GS>(rk, part, buf);
      } else {
#pragma unroll
        for (int k = 0; k < 32; ++k) buf[k] = 0.0f;
      }
#pragma unroll
      for (int k = 0; k < 32; ++k) s_k[tt][32 * part + k] = buf[k];
      const RowRef rv = row_ref(L, d.cache, 1, b, h, t < te ? t : ts, d.block_table);
      if (t < te && rv.ok) dequant32<FMT, GS>(rv, part, buf);
      if (t < te && (!rk.ok || !rv.ok) && part == 0) report(d.cache.status, KVQ_ERR_INVALID_ARG);
#pragma unroll
      for (int k = 0; k < 32; ++k) s_v[tt][32 * part + k] = buf[k];
    }
    __syncthreads();
    if (has_outl) {  // overwrite outlier positions of this step
      for (int kv = 0; kv < 2; ++kv) {
        const uint32_t f = kv ? fv : fk;
        const int64_t r0 = kv ? rv0 : rk0, r1 = kv ? rv1 : rk1;
        const uint32_t* idx = kv ? idxV : idxK;
        const void* vals = kv ? valsV : valsK;
        float (*tile)[kStride] = kv ? s_v : s_k;
        if (f != kNoRec) {
          const int t = (int)(f / kHeadDim), ch = (int)(f % kHeadDim);
          if (t >= ts && t < te) tile[t - ts][ch] = kv ? vv : vk;
        }
        for (int64_t r = r0 + tid + 256; r < r1; r += 256) {
          const uint32_t ix = idx[r];
          const int t = (int)(ix / kHeadDim), ch = (int)(ix % kHeadDim);
          if (t >= ts && t < te) tile[t - ts][ch] = outlier_value(vals, r, d.outl);
        }
      }
    }
    __syncthreads();
    {  // scores (log2 domain): thread -> (token lane, rows wave, wave+4, ...)
      const int t = ts + lane;
      for (int r = wave; r < G; r += 4) {
        float acc = 0.0f;
#pragma unroll 8
        for (int ch = 0; ch < kHeadDim; ++ch) acc = fmaf(s_q[r][ch], s_k[lane][ch], acc);
        s_s[r][lane] = t < te ? acc * d.scale_log2 : -INFINITY;
      }
    }
    __syncthreads();
    for (int r = wave; r < G; r += 4) {  // online softmax, one row per wave
      const float v = s_s[r][lane];
      const float mold = s_m[r];
      const float mnew = fmaxf(mold, wave_max(v));
      const float p = exp2f(v - mnew);
      const float sum = wave_sum(p);
      const float alpha = exp2f(mold - mnew);
      s_s[r][lane] = p;
      if (lane == 0) { s_l[r] = s_l[r] * alpha + sum; s_m[r] = mnew; s_alpha[r] = alpha; }
    }
    __syncthreads();
    {  // P.V: thread -> (channel tid % 128, rows tid/128, +2, ...)
      const int ch = tid & 127, rh = tid >> 7;
#pragma unroll
      for (int k = 0; k < kMaxRows / 2; ++k) {
        const int r = rh + 2 * k;
        if (r < G) {
          float acc = o[k] * s_alpha[r];
#pragma unroll 8
          for (int tt = 0; tt < kT; ++tt) acc = fmaf(s_s[r][tt], s_v[tt][ch], acc);
          o[k] = acc;
        }
      }
    }
    __syncthreads();
  }
  const int ch = tid & 127, rh = tid >> 7;
#pragma unroll
  for (int k = 0; k < kMaxRows / 2; ++k) {
    const int r = rh + 2 * k;
    if (r >= G) continue;
    const size_t hq = (size_t)h * G + r;
    if (d.n_chunks == 1) {
      d.out[((size_t)b * d.Hq + hq) * kHeadDim + ch] = o[k] / s_l[r];
    } else {
      float* pp = d.partials + (((size_t)b * d.Hq + hq) * d.n_chunks + chunk) * (kHeadDim + 2);
      if (ch == 0) { pp[0] = s_m[r]; pp[1] = s_l[r]; }
      pp[2 + ch] = o[k];
    }
  }
}

// out[b][hq] = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c over the chunks holding tokens,
// M = max_c m_c.  Latency-bound, so built for few dependent memory round trips: one workgroup per
// query head, thread (g, ch) owns channel ch of the chunks c = g mod kMergeGroups and folds them
// into a running (max, sum, output) state in chunk order (every load of a thread is independent
// of its arithmetic, so an unrolled batch of chunks is in flight at once); the kMergeGroups
// states of a channel are then combined through LDS in group order.  Deterministic.
constexpr int kMergeGroups = 4;

__global__ void __launch_bounds__(kMergeGroups * kHeadDim) lse_merge_kernel(DecodeLaunch d) {
  __shared__ float s_st[kMergeGroups][3][kHeadDim];
  const int hq = blockIdx.x, b = blockIdx.y;
  const int ch = threadIdx.x % kHeadDim, g = threadIdx.x / kHeadDim;
  const int S = d.seq_lens[b];
  if (S < 1 || S > d.L.S_cap) return;   // reported by the decode kernel; out[b] is not written
  const int nc = min((S + d.chunk - 1) / d.chunk, d.n_chunks);
  const float* pp = d.partials + ((size_t)b * d.Hq + hq) * d.n_chunks * (kHeadDim + 2);
  float M = -INFINITY, den = 0.0f, num = 0.0f;
#pragma unroll 4
  for (int c = g; c < nc; c += kMergeGroups) {
    const float* q = pp + (size_t)c * (kHeadDim + 2);
    const float m = q[0], l = q[1], o = q[2 + ch];      // a chunk holding tokens: m finite
    const float Mn = fmaxf(M, m);
    const float a = exp2f(M - Mn), w = exp2f(m - Mn);    // a = 0 while M is -inf
    den = fmaf(w, l, den * a);
    num = fmaf(w, o, num * a);
    M = Mn;
  }
  s_st[g][0][ch] = M;
  s_st[g][1][ch] = den;
  s_st[g][2][ch] = num;
  __syncthreads();
  if (g != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMergeGroups; ++i) Mt = fmaxf(Mt, s_st[i][0][ch]);
  float D = 0.0f, N = 0.0f;
#pragma unroll
  for (int i = 0; i < kMergeGroups; ++i) {
    const float Mi = s_st[i][0][ch];
    const float f = Mi == -INFINITY ? 0.0f : exp2f(Mi - Mt);   // a group with no chunk
    D = fmaf(f, s_st[i][1][ch], D);
    N = fmaf(f, s_st[i][2][ch], N);
  }
  d.out[((size_t)b * d.Hq + hq) * kHeadDim + ch] = N / D;
  if (d.total_lse && ch == 0) d.total_lse[(size_t)b * d.Hq + hq] = Mt + __builtin_log2f(D);
}

}  // namespace

hipError_t launch_decode_generic(const DecodeLaunch& d, hipStream_t st) {
  dim3 grid(d.n_chunks, d.L.H, d.L.B);
  switch (d.fmt) {
    case FMT_INT4:
      if (d.group == 32) decode_generic_kernel<FMT_INT4, 32><<<grid, 256, 0, st>>>(d);
      else decode_generic_kernel<FMT_INT4, 64><<<grid, 256, 0, st>>>(d);
      break;
    case FMT_FP4:
      if (d.group == 32) decode_generic_kernel<FMT_FP4, 32><<<grid, 256, 0, st>>>(d);
      else decode_generic_kernel<FMT_FP4, 64><<<grid, 256, 0, st>>>(d);
      break;
    case FMT_C2: decode_generic_kernel<FMT_C2, 64><<<grid, 256, 0, st>>>(d); break;
    case FMT_INT3:
      if (d.group == 32) decode_generic_kernel<FMT_INT3, 32><<<grid, 256, 0, st>>>(d);
      else decode_generic_kernel<FMT_INT3, 64><<<grid, 256, 0, st>>>(d);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lse_merge(const DecodeLaunch& d, hipStream_t st) {
  lse_merge_kernel<<<dim3(d.Hq, d.L.B), kMergeGroups * kHeadDim, 0, st>>>(d);
  return hipGetLastError();
}

}  // namespace kvq
