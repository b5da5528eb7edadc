// Fused dequantize + flash-decoding attention on the MFMA matrix cores (gfx950) for caches whose
// dequantized values are exact in fp16: 2-bit centroid codes (fp16 centroids, E4M3 or fp16
// outliers) and FP4 E2M1 codes with E4M3 block scales (E2M1 x E4M3 has at most 6 significant
// bits and stays inside the fp16 range).
//
// "Hierarchical Token Routing and Sub-2-Bit Non-Linear KV Compression ...", section
// "Hardware-Kernel Fusion: Eliminating DRAM Round-Trips" (stream packed codes, expand on chip);
// "Sub-5ms MoE Inference ...", section "Engineering Real-Time Autonomous Workflows", item 3
// (bit-unpacked matrix products in matrix-core operand registers); "The Sub-10ms Barrier ...",
// section "2. FP4/INT4 KV-Cache Quantization", item 3 (dequantize into fp16 operand space inside
// the flash-attention reduction).
//
// Work unit: a workgroup of 4 waves per (split-K chunk, KV head, sequence).  Waves take 32-token
// steps of the chunk in turn.  Per step a lane owns (token, 64-channel half row): it loads the
// packed codes and group metadata with 128-bit loads (prefetched two steps ahead), expands them
// to fp16 in registers and writes the rows into the wave's LDS tile; outlier records of the step
// are written over their positions.  Scores are computed transposed, S^T = K^ Q^T, with
// v_mfma_f32_16x16x32_f16 (16 tokens x 16 padded query rows), which leaves every lane holding
// the probabilities of one query row for 4+4 tokens - exactly the B operand of O^T = V^T P^T.
// V^T operands come out of the LDS tile with ds_read_b64_tr_b16.  P is split into fp16 hi + lo
// parts so that large outlier values in V see fp32-grade probabilities.  The 4 waves' states are
// merged in LDS; a chunk writes either the final output or a (max, sum, output) partial.
//
// 2-bit expansion: per 64-bit centroid word, two byte tables (low bytes and high bytes of the 4
// fp16 centroids) are built once; four codes spread into the four bytes of a selector give the
// low and high bytes of their centroids with one v_perm each, and two more v_perm interleave
// them into two fp16 pairs.  This writes each 16-channel block in 4x4-transposed order
// (position 4*(c%4) + c/4); queries, outlier positions and the output use the same order.
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef _Float16 __attribute__((address_space(3))) lds_half;

// 4 x 16-bit transposed LDS read (see the lane mapping in the file comment)
__device__ __forceinline__ half4v read_tr16(const lds_half* p) {
  const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)p);
  return __builtin_bit_cast(half4v, v);
}

constexpr int kWaves = 4;
constexpr int kStep = 32;                  // tokens per wave step
constexpr int kRow = 136;                  // LDS row stride in halfs (272 bytes)
constexpr int kTile = kStep * kRow;        // halfs per tile
constexpr int kWaveLds = 2 * kTile;        // K tile + V tile

// position of channel c in the LDS row
template <int FMT>
__device__ __forceinline__ int chan_pos(int c) {
  if constexpr (FMT == FMT_C2) return (c & ~15) | ((c & 3) << 2) | ((c >> 2) & 3);
  else return c;
}

template <int FMT> struct Buf;
template <> struct Buf<FMT_C2> { uint4 kc, vc; uint2 km, vm; };
template <> struct Buf<FMT_FP4> { uint4 kc0, kc1, vc0, vc1; uint32_t km, vm; };

struct Recs {       // up to 128 outlier records per list per step, two per lane
  uint32_t kidx0, kidx1, vidx0, vidx1;
  uint32_t kval0, kval1, vval0, vval1;
  int kr0, kr1, vr0, vr1;   // record range of the step (uniform)
};

template <int FMT>
__device__ __forceinline__ void load_codes(Buf<FMT>& bf, const uint8_t* ck, const uint8_t* cv,
                                           const uint8_t* mk, const uint8_t* mv) {
  if constexpr (FMT == FMT_C2) {
    bf.kc = *(const uint4*)ck;
    bf.vc = *(const uint4*)cv;
    bf.km = *(const uint2*)mk;
    bf.vm = *(const uint2*)mv;
  } else {
    bf.kc0 = *(const uint4*)ck;
    bf.kc1 = *(const uint4*)(ck + 16);
    bf.vc0 = *(const uint4*)cv;
    bf.vc1 = *(const uint4*)(cv + 16);
    bf.km = *(const uint16_t*)mk;
    bf.vm = *(const uint16_t*)mv;
  }
}

// 64 channels of one 2-bit row -> 64 fp16 in transposed-block order at dst
__device__ __forceinline__ void expand_c2(uint4 c, uint2 m, _Float16* dst) {
  const uint32_t tl = __builtin_amdgcn_perm(m.y, m.x, 0x06040200u);  // low bytes of C0..C3
  const uint32_t th = __builtin_amdgcn_perm(m.y, m.x, 0x07050301u);  // high bytes
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t o[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t x = (w[k] >> (2 * s)) & 0x03030303u;
      const uint32_t lo = __builtin_amdgcn_perm(th, tl, x);
      const uint32_t hi = __builtin_amdgcn_perm(tl, th, x);
      o[2 * s] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
      o[2 * s + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    }
    uint4* d = (uint4*)(dst + 16 * k);
    d[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
}

// 64 channels of one FP4 row (two groups of 32) -> fp16 in natural order
__device__ __forceinline__ void expand_fp4(uint4 c0, uint4 c1, uint32_t m, _Float16* dst) {
  const _Float16 s0 = (_Float16)e4m3_to_f32(m & 0xFFu);
  const _Float16 s1 = (_Float16)e4m3_to_f32((m >> 8) & 0xFFu);
  const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const half2v sc = k < 4 ? half2v{s0, s0} : half2v{s1, s1};
    const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 0) * sc;
    const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 1) * sc;
    const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 2) * sc;
    const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[k], 1.0f, 3) * sc;
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, a);
    v.y = __builtin_bit_cast(uint32_t, b);
    v.z = __builtin_bit_cast(uint32_t, c);
    v.w = __builtin_bit_cast(uint32_t, d);
    *(uint4*)(dst + 8 * k) = v;
  }
}

__device__ __forceinline__ uint32_t outl_half_bits(uint32_t v, int outl) {
  return outl == KVQ_OUTL_FP16 ? v : f32_to_half_bits(e4m3_to_f32(v));
}

template <int FMT>
__device__ __forceinline__ void patch(_Float16* tile, uint32_t idx, uint32_t val, int ts, int nval,
                                      int outl) {
  if (idx == 0xFFFFFFFFu) return;
  const int t = (int)(idx >> 7) - ts;
  if (t < 0 || t >= nval) return;
  const int c = (int)(idx & 127u);
  tile[t * kRow + chan_pos<FMT>(c)] = __builtin_bit_cast(_Float16, (uint16_t)outl_half_bits(val, outl));
}

template <int FMT>
__global__ void __launch_bounds__(256) decode_mfma_kernel(DecodeLaunch d) {
  __shared__ __attribute__((aligned(16))) _Float16 s_lds[kWaves * kWaveLds];
  __shared__ float s_ml[kWaves][16][2];

  const Layout& L = d.L;
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int S = d.seq_lens[b];
  if (S < 1 || S > L.S_cap) {
    if (threadIdx.x == 0 && chunk == 0 && h == 0) report(d.cache.status, KVQ_ERR_INVALID_ARG);
    return;
  }
  const int t0 = chunk * d.chunk;
  if (t0 >= S) return;
  const int t1 = min(t0 + d.chunk, S);
  const int G = d.Hq / L.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kg = lane >> 4;           // MFMA lane coordinates
  const int trow = lane & 31, half = lane >> 5;      // dequant lane coordinates
  constexpr int CB = FMT == FMT_C2 ? 32 : 64;
  constexpr int MB = FMT == FMT_C2 ? 16 : 4;

  _Float16* ktile = s_lds + wave * kWaveLds;
  _Float16* vtile = ktile + kTile;

  // query operand (B of S^T = K^ Q^T): lane (row r, k-group kg), positions 32*ks + 8*kg + e
  half8 qop[4];
  {
    const uint16_t* qrow = d.q + ((size_t)b * d.Hq + (size_t)h * G + (r < G ? r : 0)) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = chan_pos<FMT>(32 * ks + 8 * kg + e);  // the order is an involution
        const float v = r < G ? as_f32((uint32_t)qrow[c] << 16) : 0.0f;
        qop[ks][e] = (_Float16)v;
      }
  }

  const size_t rowbase = ((size_t)b * L.H + h) * (size_t)L.S_cap;
  const uint8_t* codesK = (const uint8_t*)d.cache.codes[0] + rowbase * CB + half * (CB / 2);
  const uint8_t* codesV = (const uint8_t*)d.cache.codes[1] + rowbase * CB + half * (CB / 2);
  const uint8_t* metaK = (const uint8_t*)d.cache.meta[0] + rowbase * MB + half * (MB / 2);
  const uint8_t* metaV = (const uint8_t*)d.cache.meta[1] + rowbase * MB + half * (MB / 2);
  const size_t lidK = list_id(L, b, h, 0), lidV = lidK + 1;
  const int32_t* bsK = d.cache.outl_block_start + lidK * (size_t)L.nblk;
  const int32_t* bsV = d.cache.outl_block_start + lidV * (size_t)L.nblk;
  const size_t lbase = ((size_t)b * L.H + h) * (size_t)L.outl_cap;
  const uint32_t* oidxK = d.cache.outl_idx[0] + lbase;
  const uint32_t* oidxV = d.cache.outl_idx[1] + lbase;
  const int outl = d.outl;
  const int vbytes = outl == KVQ_OUTL_FP16 ? 2 : 1;
  const uint8_t* ovalK = (const uint8_t*)d.cache.outl_val[0] + lbase * vbytes;
  const uint8_t* ovalV = (const uint8_t*)d.cache.outl_val[1] + lbase * vbytes;
  const int cntK = d.cache.outl_count[lidK], cntV = d.cache.outl_count[lidV];
  const int cap = (int)min(L.outl_cap, (int64_t)INT32_MAX);

  const int nsteps = (t1 - t0 + kStep - 1) / kStep;
  const int nmine = wave < nsteps ? (nsteps - wave + kWaves - 1) / kWaves : 0;
  auto step_ts = [&](int j) { return t0 + kStep * (wave + kWaves * j); };

  // ---- per-step loaders
  auto issue_codes = [&](Buf<FMT>& bf, int j) {
    const int ts = step_ts(j);
    const int t = min(ts + trow, t1 - 1);
    load_codes<FMT>(bf, codesK + (size_t)t * CB, codesV + (size_t)t * CB,
                    metaK + (size_t)t * MB, metaV + (size_t)t * MB);
  };
  // lane 0..3 loads {K start, K end, V start, V end} of step j's records
  auto issue_bounds = [&](int j) -> int {
    if (outl == KVQ_OUTL_NONE) return 0;
    const int ts = step_ts(j);
    const int blk = ts >> 4;
    const bool last = ts + kStep >= S;
    int v = 0;
    if (lane == 0) v = bsK[blk];
    else if (lane == 1) v = last ? cntK : bsK[blk + 2];
    else if (lane == 2) v = bsV[blk];
    else if (lane == 3) v = last ? cntV : bsV[blk + 2];
    return v;
  };
  auto issue_recs = [&](Recs& rc, int bnd) {
    if (outl == KVQ_OUTL_NONE) { rc.kr0 = rc.kr1 = rc.vr0 = rc.vr1 = 0; return; }
    rc.kr0 = max(0, min(__builtin_amdgcn_readlane(bnd, 0), cap));
    rc.kr1 = max(rc.kr0, min(__builtin_amdgcn_readlane(bnd, 1), cap));
    rc.vr0 = max(0, min(__builtin_amdgcn_readlane(bnd, 2), cap));
    rc.vr1 = max(rc.vr0, min(__builtin_amdgcn_readlane(bnd, 3), cap));
    const int a0 = rc.kr0 + lane, a1 = rc.kr0 + 64 + lane;
    const int c0 = rc.vr0 + lane, c1 = rc.vr0 + 64 + lane;
    rc.kidx0 = a0 < rc.kr1 ? oidxK[a0] : 0xFFFFFFFFu;
    rc.kidx1 = a1 < rc.kr1 ? oidxK[a1] : 0xFFFFFFFFu;
    rc.vidx0 = c0 < rc.vr1 ? oidxV[c0] : 0xFFFFFFFFu;
    rc.vidx1 = c1 < rc.vr1 ? oidxV[c1] : 0xFFFFFFFFu;
    if (vbytes == 2) {
      rc.kval0 = a0 < rc.kr1 ? ((const uint16_t*)ovalK)[a0] : 0u;
      rc.kval1 = a1 < rc.kr1 ? ((const uint16_t*)ovalK)[a1] : 0u;
      rc.vval0 = c0 < rc.vr1 ? ((const uint16_t*)ovalV)[c0] : 0u;
      rc.vval1 = c1 < rc.vr1 ? ((const uint16_t*)ovalV)[c1] : 0u;
    } else {
      rc.kval0 = a0 < rc.kr1 ? ovalK[a0] : 0u;
      rc.kval1 = a1 < rc.kr1 ? ovalK[a1] : 0u;
      rc.vval0 = c0 < rc.vr1 ? ovalV[c0] : 0u;
      rc.vval1 = c1 < rc.vr1 ? ovalV[c1] : 0u;
    }
  };

  // ---- state
  floatx4 oacc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) oacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = d.scale_log2;

  auto consume = [&](const Buf<FMT>& bf, const Recs& rc, int j) {
    const int ts = step_ts(j);
    const int nval = min(kStep, t1 - ts);
    // expand rows into the tiles
    _Float16* krow = ktile + trow * kRow + 64 * half;
    _Float16* vrow = vtile + trow * kRow + 64 * half;
    if constexpr (FMT == FMT_C2) {
      expand_c2(bf.kc, bf.km, krow);
      expand_c2(bf.vc, bf.vm, vrow);
    } else {
      expand_fp4(bf.kc0, bf.kc1, bf.km, krow);
      expand_fp4(bf.vc0, bf.vc1, bf.vm, vrow);
    }
    if (outl != KVQ_OUTL_NONE) {
      patch<FMT>(ktile, rc.kidx0, rc.kval0, ts, nval, outl);
      patch<FMT>(ktile, rc.kidx1, rc.kval1, ts, nval, outl);
      patch<FMT>(vtile, rc.vidx0, rc.vval0, ts, nval, outl);
      patch<FMT>(vtile, rc.vidx1, rc.vval1, ts, nval, outl);
      // more than 128 records in this step: the rest, read directly
      for (int a = rc.kr0 + 128 + lane; a < rc.kr1; a += 64) {
        const uint32_t v = vbytes == 2 ? ((const uint16_t*)ovalK)[a] : ovalK[a];
        patch<FMT>(ktile, oidxK[a], v, ts, nval, outl);
      }
      for (int a = rc.vr0 + 128 + lane; a < rc.vr1; a += 64) {
        const uint32_t v = vbytes == 2 ? ((const uint16_t*)ovalV)[a] : ovalV[a];
        patch<FMT>(vtile, oidxV[a], v, ts, nval, outl);
      }
    }
    // S^T for tokens 0..15 and 16..31 of the step
    floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const half8 a0 = *(const half8*)(ktile + r * kRow + 32 * ks + 8 * kg);
      const half8 a1 = *(const half8*)(ktile + (16 + r) * kRow + 32 * ks + 8 * kg);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qop[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qop[ks], s1, 0, 0, 0);
    }
    // online softmax: lane holds query row r, tokens 4kg+v (tile 0) and 16+4kg+v (tile 1)
    float sc[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      sc[v] = (4 * kg + v) < nval ? s0[v] * sl2 : -INFINITY;
      sc[4 + v] = (16 + 4 * kg + v) < nval ? s1[v] * sl2 : -INFINITY;
    }
    float mx = sc[0];
#pragma unroll
    for (int v = 1; v < 8; ++v) mx = fmaxf(mx, sc[v]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    half8 phi, plo;
    float psum = 0.0f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const float p = __builtin_amdgcn_exp2f(sc[v] - m_new);
      psum += p;
      const _Float16 hi = (_Float16)p;
      phi[v] = hi;
      plo[v] = (_Float16)(p - (float)hi);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) oacc[mt] *= alpha;
    }
    // O^T += V^T P^T: A = V^T (16 channels x 32 tokens) through transposing LDS reads
    const lds_half* vbase = (const lds_half*)vtile;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int col = 16 * mt + 4 * (r & 3);
      const int rowo = 4 * kg + (r >> 2);
      const half4v t0v = read_tr16(vbase + rowo * kRow + col);
      const half4v t1v = read_tr16(vbase + (16 + rowo) * kRow + col);
      const half8 av = {t0v[0], t0v[1], t0v[2], t0v[3], t1v[0], t1v[1], t1v[2], t1v[3]};
      oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, phi, oacc[mt], 0, 0, 0);
      oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, plo, oacc[mt], 0, 0, 0);
    }
  };

  // ---- software pipeline: codes and records two steps ahead, record bounds three ahead
  Buf<FMT> buf[3];
  Recs rec[3];
  int bnd[3];
  if (nmine > 0) {
    bnd[0] = issue_bounds(0);
    if (nmine > 1) bnd[1] = issue_bounds(1);
    if (nmine > 2) bnd[2] = issue_bounds(2);
    issue_codes(buf[0], 0);
    issue_recs(rec[0], bnd[0]);
    if (nmine > 1) { issue_codes(buf[1], 1); issue_recs(rec[1], bnd[1]); }
  }
  for (int j = 0; j < nmine; j += 3) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int jj = j + u;
      if (jj < nmine) {
        if (jj + 3 < nmine) bnd[u] = issue_bounds(jj + 3);
        if (jj + 2 < nmine) {
          issue_recs(rec[(u + 2) % 3], bnd[(u + 2) % 3]);
          issue_codes(buf[(u + 2) % 3], jj + 2);
        }
        consume(buf[u], rec[u], jj);
      }
    }
  }

  // ---- merge the waves of the workgroup
  float l_row = l_run + __shfl_xor(l_run, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);
  float* s_o = (float*)(s_lds + wave * kWaveLds);   // [16 rows][128 channels] of this wave
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) s_o[r * kHeadDim + chan_pos<FMT>(16 * mt + 4 * kg + v)] = oacc[mt][v];
  if (kg == 0) { s_ml[wave][r][0] = m_run; s_ml[wave][r][1] = l_row; }
  __syncthreads();
  for (int i = threadIdx.x; i < G * kHeadDim; i += 256) {
    const int row = i / kHeadDim, ch = i % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][row][0]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_ml[w][row][0];
      const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      den += f * s_ml[w][row][1];
      num += f * ((const float*)(s_lds + w * kWaveLds))[row * kHeadDim + ch];
    }
    const size_t hq = (size_t)h * G + row;
    if (d.n_chunks == 1) {
      d.out[((size_t)b * d.Hq + hq) * kHeadDim + ch] = num / den;
    } else {
      float* pp = d.partials + (((size_t)b * d.Hq + hq) * d.n_chunks + chunk) * (kHeadDim + 2);
      if (ch == 0) { pp[0] = M; pp[1] = den; }
      pp[2 + ch] = num;
    }
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeLaunch& d, hipStream_t st, bool* handled) {
  *handled = false;
  if (d.L.paged) return hipSuccess;
  if (d.fmt != FMT_C2 && !(d.fmt == FMT_FP4 && d.group == 32)) return hipSuccess;
  if (d.chunk % kStep) return hipSuccess;
  dim3 grid(d.n_chunks, d.L.H, d.L.B);
  if (d.fmt == FMT_C2) decode_mfma_kernel<FMT_C2><<<grid, 256, 0, st>>>(d);
  else decode_mfma_kernel<FMT_FP4><<<grid, 256, 0, st>>>(d);
  *handled = true;
  return hipGetLastError();
}

}  // namespace kvq
