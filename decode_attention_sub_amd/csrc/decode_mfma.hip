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
#ifndef KVQ_TILE_ROW
#define KVQ_TILE_ROW 136
#endif
constexpr int kRow = KVQ_TILE_ROW;         // LDS row stride in halfs (272 bytes by default)
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
  int kr0, nk, vr0, nv;     // first record and record count of the step (uniform)
};

// raw buffer resource (gfx9 family): loads at byte offsets >= num_records return zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint2 ld64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
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

// stored outlier value -> fp16 bits (E4M3 values are exact in fp16)
// E4M3 bits placed as fp16 bits ((code & 0x7F) << 7 | sign << 15) encode value * 2^-8 for every
// code, subnormals included (both formats' subnormal steps line up); one exact fp16 multiply by
// 256 restores the value.
template <int OUTL>
__device__ __forceinline__ _Float16 outl_half(uint32_t v) {
  if constexpr (OUTL == KVQ_OUTL_FP16) {
    return __builtin_bit_cast(_Float16, (uint16_t)v);
  } else {
    const uint32_t h = ((v & 0x7Fu) << 7) | ((v & 0x80u) << 8);
    return __builtin_bit_cast(_Float16, (uint16_t)h) * (_Float16)256.0f;
  }
}

// Overwrite one outlier position in a tile.  Records outside the step (or past the step's
// record count) are written to a pad slot (row 0, column 128) that no operand read touches.
template <int FMT, int OUTL>
__device__ __forceinline__ void patch(_Float16* tile, bool have, uint32_t idx, uint32_t val,
                                      int ts, int nval) {
  const uint32_t t = (idx >> 7) - (uint32_t)ts;
  const uint32_t c = idx & 127u;
  const bool ok = have && t < (uint32_t)nval;
  const uint32_t at = ok ? t * (uint32_t)kRow + (uint32_t)chan_pos<FMT>((int)c) : (uint32_t)kHeadDim;
  tile[at] = outl_half<OUTL>(val);
}

template <int FMT, int OUTL>
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
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, kg = lane >> 4;           // MFMA lane coordinates
  const int trow = lane & 31, half = lane >> 5;      // dequant lane coordinates
  constexpr int CB = FMT == FMT_C2 ? 32 : 64;
  constexpr int MB = FMT == FMT_C2 ? 16 : 4;
  constexpr int VB = OUTL == KVQ_OUTL_FP16 ? 2 : 1;
  constexpr bool HAS_OUTL = OUTL != KVQ_OUTL_NONE;

  _Float16* ktile = s_lds + wave * kWaveLds;
  _Float16* vtile = ktile + kTile;

  // query operand (B of S^T = K^ Q^T): lane (row r, k-group kg), positions 32*ks + 8*kg + e
  half8 qop[4];
  {
    // every lane reads a valid row (padding rows read row 0 and are zeroed after the load)
    const uint16_t* qrow = d.q + ((size_t)b * d.Hq + (size_t)h * G + (r < G ? r : 0)) * kHeadDim;
    uint16_t raw[4][8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) raw[ks][e] = qrow[chan_pos<FMT>(32 * ks + 8 * kg + e)];
    const float keep = r < G ? 1.0f : 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[ks][e] = (_Float16)(as_f32((uint32_t)raw[ks][e] << 16) * keep);
  }

  // buffer resources: rows [0, t1) of this (sequence, KV head); rows past t1 read as zero
  const size_t rowbase = ((size_t)b * L.H + h) * (size_t)L.S_cap;
  const __amdgpu_buffer_rsrc_t rcK = make_rsrc((const uint8_t*)d.cache.codes[0] + rowbase * CB, (uint32_t)t1 * CB);
  const __amdgpu_buffer_rsrc_t rcV = make_rsrc((const uint8_t*)d.cache.codes[1] + rowbase * CB, (uint32_t)t1 * CB);
  const __amdgpu_buffer_rsrc_t rmK = make_rsrc((const uint8_t*)d.cache.meta[0] + rowbase * MB, (uint32_t)t1 * MB);
  const __amdgpu_buffer_rsrc_t rmV = make_rsrc((const uint8_t*)d.cache.meta[1] + rowbase * MB, (uint32_t)t1 * MB);
  const uint32_t coff = (uint32_t)(trow * CB + half * (CB / 2));
  const uint32_t moff = (uint32_t)(trow * MB + half * (MB / 2));

  const size_t lidK = list_id(L, b, h, 0);
  const int cap = (int)min(L.outl_cap, (int64_t)INT32_MAX);
  __amdgpu_buffer_rsrc_t riK, riV, rvK, rvV, rbs;
  int cntK = 0, cntV = 0;
  const uint32_t* oidxK = nullptr;
  const uint32_t* oidxV = nullptr;
  const uint8_t* ovalK = nullptr;
  const uint8_t* ovalV = nullptr;
  if constexpr (HAS_OUTL) {
    const size_t lbase = ((size_t)b * L.H + h) * (size_t)L.outl_cap;
    oidxK = d.cache.outl_idx[0] + lbase;
    oidxV = d.cache.outl_idx[1] + lbase;
    ovalK = (const uint8_t*)d.cache.outl_val[0] + lbase * VB;
    ovalV = (const uint8_t*)d.cache.outl_val[1] + lbase * VB;
    riK = make_rsrc(oidxK, (uint32_t)cap * 4);
    riV = make_rsrc(oidxV, (uint32_t)cap * 4);
    rvK = make_rsrc(ovalK, (uint32_t)cap * VB);
    rvV = make_rsrc(ovalV, (uint32_t)cap * VB);
    rbs = make_rsrc(d.cache.outl_block_start + lidK * (size_t)L.nblk, (uint32_t)L.nblk * 8);
    cntK = max(0, min(d.cache.outl_count[lidK], cap));
    cntV = max(0, min(d.cache.outl_count[lidK + 1], cap));
  }

  const int nsteps = (t1 - t0 + kStep - 1) / kStep;
  const int nmine = wave < nsteps ? (nsteps - wave + kWaves - 1) / kWaves : 0;
  auto step_ts = [&](int j) { return t0 + kStep * (wave + kWaves * j); };

  auto issue_codes = [&](Buf<FMT>& bf, int j) {
    const uint32_t ts = (uint32_t)step_ts(j);
    if constexpr (FMT == FMT_C2) {
      bf.kc = ld128(rcK, ts * CB + coff);
      bf.vc = ld128(rcV, ts * CB + coff);
      bf.km = ld64(rmK, ts * MB + moff);
      bf.vm = ld64(rmV, ts * MB + moff);
    } else {
      bf.kc0 = ld128(rcK, ts * CB + coff);
      bf.kc1 = ld128(rcK, ts * CB + coff + 16);
      bf.vc0 = ld128(rcV, ts * CB + coff);
      bf.vc1 = ld128(rcV, ts * CB + coff + 16);
      bf.km = ld16(rmK, ts * MB + moff);
      bf.vm = ld16(rmV, ts * MB + moff);
    }
  };
  // lanes 0..3 load {K start, K end, V start, V end} of step j's records (block starts)
  auto issue_bounds = [&](int j) -> uint32_t {
    if constexpr (!HAS_OUTL) return 0u;
    const int blk = step_ts(j) >> 4;
    const int which = lane & 3;  // 0: K blk, 1: K blk+2, 2: V blk, 3: V blk+2
    const uint32_t off = (uint32_t)(((which >> 1) * L.nblk + blk + 2 * (which & 1)) * 4);
    return ld32(rbs, off);
  };
  auto issue_recs = [&](Recs& rc, uint32_t bnd, int j) {
    if constexpr (HAS_OUTL) {
      const bool last = step_ts(j) + kStep >= S;
      const int k0 = max(0, min(__builtin_amdgcn_readlane((int)bnd, 0), cap));
      const int k1 = last ? cntK : max(0, min(__builtin_amdgcn_readlane((int)bnd, 1), cap));
      const int v0 = max(0, min(__builtin_amdgcn_readlane((int)bnd, 2), cap));
      const int v1 = last ? cntV : max(0, min(__builtin_amdgcn_readlane((int)bnd, 3), cap));
      rc.kr0 = k0; rc.nk = max(k1 - k0, 0);
      rc.vr0 = v0; rc.nv = max(v1 - v0, 0);
      const uint32_t a0 = (uint32_t)(k0 + lane), a1 = a0 + 64u;
      const uint32_t c0 = (uint32_t)(v0 + lane), c1 = c0 + 64u;
      rc.kidx0 = ld32(riK, a0 * 4);
      rc.kidx1 = ld32(riK, a1 * 4);
      rc.vidx0 = ld32(riV, c0 * 4);
      rc.vidx1 = ld32(riV, c1 * 4);
      if constexpr (VB == 2) {
        rc.kval0 = ld16(rvK, a0 * 2); rc.kval1 = ld16(rvK, a1 * 2);
        rc.vval0 = ld16(rvV, c0 * 2); rc.vval1 = ld16(rvV, c1 * 2);
      } else {
        rc.kval0 = ld8(rvK, a0); rc.kval1 = ld8(rvK, a1);
        rc.vval0 = ld8(rvV, c0); rc.vval1 = ld8(rvV, c1);
      }
    }
  };

  floatx4 oacc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) oacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = d.scale_log2;

  auto consume = [&](const Buf<FMT>& bf, const Recs& rc, int j) {
    const int ts = step_ts(j);
    const int nval = min(kStep, t1 - ts);
    _Float16* krow = ktile + trow * kRow + 64 * half;
    _Float16* vrow = vtile + trow * kRow + 64 * half;
    if constexpr (FMT == FMT_C2) {
      expand_c2(bf.kc, bf.km, krow);
      expand_c2(bf.vc, bf.vm, vrow);
    } else {
      expand_fp4(bf.kc0, bf.kc1, bf.km, krow);
      expand_fp4(bf.vc0, bf.vc1, bf.vm, vrow);
    }
    if constexpr (HAS_OUTL) {
      patch<FMT, OUTL>(ktile, lane < rc.nk, rc.kidx0, rc.kval0, ts, nval);
      patch<FMT, OUTL>(ktile, lane + 64 < rc.nk, rc.kidx1, rc.kval1, ts, nval);
      patch<FMT, OUTL>(vtile, lane < rc.nv, rc.vidx0, rc.vval0, ts, nval);
      patch<FMT, OUTL>(vtile, lane + 64 < rc.nv, rc.vidx1, rc.vval1, ts, nval);
      if (rc.nk > 128 || rc.nv > 128) {  // rare: the rest of a crowded step, read directly
        for (int a = 128 + lane; a < rc.nk; a += 64) {
          const int at = rc.kr0 + a;
          const uint32_t v = VB == 2 ? ((const uint16_t*)ovalK)[at] : ovalK[at];
          patch<FMT, OUTL>(ktile, true, oidxK[at], v, ts, nval);
        }
        for (int a = 128 + lane; a < rc.nv; a += 64) {
          const int at = rc.vr0 + a;
          const uint32_t v = VB == 2 ? ((const uint16_t*)ovalV)[at] : ovalV[at];
          patch<FMT, OUTL>(vtile, true, oidxV[at], v, ts, nval);
        }
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
    for (int v = 0; v < 4; ++v) { sc[v] = s0[v] * sl2; sc[4 + v] = s1[v] * sl2; }
    if (nval < kStep) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (4 * kg + v >= nval) sc[v] = -INFINITY;
        if (16 + 4 * kg + v >= nval) sc[4 + v] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    half8 phi, plo;
    float psum = 0.0f;
#pragma unroll
    for (int v = 0; v < 8; v += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sc[v] - m_new);
      const float p1 = __builtin_amdgcn_exp2f(sc[v + 1] - m_new);
      psum += p0 + p1;
      const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(p0, p1));
      const half2v lo = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(p0 - (float)hi[0], p1 - (float)hi[1]));
      phi[v] = hi[0]; phi[v + 1] = hi[1];
      plo[v] = lo[0]; plo[v + 1] = lo[1];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) oacc[mt] *= alpha;
    }
    // O^T += V^T P^T: A = V^T (16 channels x 32 tokens) through transposing LDS reads
    const lds_half* vbase = (const lds_half*)vtile;
    const int col0 = 4 * (r & 3);
    const int rowo = 4 * kg + (r >> 2);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const half4v t0v = read_tr16(vbase + rowo * kRow + 16 * mt + col0);
      const half4v t1v = read_tr16(vbase + (16 + rowo) * kRow + 16 * mt + col0);
      const half8 av = {t0v[0], t0v[1], t0v[2], t0v[3], t1v[0], t1v[1], t1v[2], t1v[3]};
      oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, phi, oacc[mt], 0, 0, 0);
      oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, plo, oacc[mt], 0, 0, 0);
    }
  };

  // ---- software pipeline: codes and records two steps ahead, record bounds three ahead
  Buf<FMT> buf[3];
  Recs rec[3];
  uint32_t bnd[3] = {0u, 0u, 0u};
  // Loads for steps past the wave's last step are issued anyway: their offsets lie past the
  // buffer ranges (codes) or are clamped (records), so they return zeros or unused data without
  // touching memory, and keeping every load unconditional lets the wait counters stay exact.
  if (nmine > 0) {
    bnd[0] = issue_bounds(0);
    bnd[1] = issue_bounds(1);
    bnd[2] = issue_bounds(2);
    issue_recs(rec[0], bnd[0], 0);
    issue_codes(buf[0], 0);
    issue_recs(rec[1], bnd[1], 1);
    issue_codes(buf[1], 1);
  }
  for (int j = 0; j < nmine; j += 3) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int jj = j + u;
      if (jj < nmine) {
        bnd[u] = issue_bounds(jj + 3);
        issue_recs(rec[(u + 2) % 3], bnd[(u + 2) % 3], jj + 2);
        issue_codes(buf[(u + 2) % 3], jj + 2);
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

template <int FMT>
void launch_fmt(const DecodeLaunch& d, dim3 grid, hipStream_t st) {
  switch (d.outl) {
    case KVQ_OUTL_NONE: decode_mfma_kernel<FMT, KVQ_OUTL_NONE><<<grid, 256, 0, st>>>(d); break;
    case KVQ_OUTL_FP16: decode_mfma_kernel<FMT, KVQ_OUTL_FP16><<<grid, 256, 0, st>>>(d); break;
    default: decode_mfma_kernel<FMT, KVQ_OUTL_FP8_E4M3><<<grid, 256, 0, st>>>(d); break;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeLaunch& d, hipStream_t st, bool* handled) {
  *handled = false;
  if (d.L.paged) return hipSuccess;
  if (d.fmt != FMT_C2 && !(d.fmt == FMT_FP4 && d.group == 32)) return hipSuccess;
  if (d.chunk % kStep) return hipSuccess;
  dim3 grid(d.n_chunks, d.L.H, d.L.B);
  if (d.fmt == FMT_C2) launch_fmt<FMT_C2>(d, grid, st);
  else launch_fmt<FMT_FP4>(d, grid, st);
  *handled = true;
  return hipGetLastError();
}

}  // namespace kvq
