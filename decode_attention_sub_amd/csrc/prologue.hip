// Attention prologue of a decode step in one kernel: RMSNorm of every sequence's hidden state,
// the joint Q / K / V projection on the MFMA matrix cores, and the KV-cache write of the new
// token's K and V rows (quantized exactly as an append of those rows).
//
// "Sub-5ms MoE Inference: Sub-Byte KV Quantization and Expert Pipelining at Scale", section
// "Engineering Real-Time Autonomous Workflows", item 1: RMSNorm, the self-attention projection
// and the KV-cache write fused into a single kernel.
//
// Arithmetic.  y = W (g * h) / rms(h), rms(h) = sqrt(mean(h^2) + eps), is formed as r * (W a)
// with a = bf16(h * g) (a bf16 x bf16 product is exact in fp32; it is rounded once to bf16) and
// r = 1 / sqrt(sum(h^2) / d + eps) applied to each row after the product (r is one number per
// row).  W a runs on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; sum(h^2) is an fp32 sum of
// exact squares.  A row's value is the fp32 sum of its K-slice partials in slice order, times r:
// the result does not depend on which workgroup finishes last.
//
// Work split.  A tile is one head's 128 output columns (K heads, then V heads, then Q heads, so
// that the K / V tiles are dispatched first) for up to 64 batch rows; the d_model reduction of a
// tile is split over several workgroups (K / V tiles more finely, so that their epilogues, which
// quantize the rows, start early and overlap the Q tiles' weight streaming).  A workgroup streams
// its weight slice from HBM straight into MFMA operand registers (every weight is read once),
// stages bf16(h * g) of its slice in LDS 128 columns at a time, and writes a partial tile; the
// last workgroup of a tile to arrive sums the partials and finishes the tile: q rows in bf16, or
// the K / V rows quantized into the cache.  Partials cross workgroups on different XCDs, whose L2
// caches are not coherent with each other: they are stored and loaded with agent-scope atomics
// (which carry the coherence cache policy), the arrival counter is an agent-scope atomic, and the
// last workgroup returns the counter to zero.
#include "kvq_device.h"
#include "kvq_launch.h"
#include "quant_row.h"

namespace kvq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPThreads = 512;            // 8 waves, 16 output columns each
constexpr int kPRows = kPrologueRows;     // batch rows of a row block
constexpr int kPKc = 128;                 // d_model columns per LDS stage
constexpr int kPStride = kPKc + 8;        // bf16 per staged row: 272 bytes, conflict-free reads
constexpr int kPSlots = kPThreads / kRowLanes;   // rows quantized at once in a K / V epilogue

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return as_f32(b << 16); }
// nearest-even bfloat16 of a finite float
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  const uint32_t u = as_u32(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Partials: 16-byte buffer loads and stores carrying the cache policy bit sc1 of gfx940-family
// memory instructions, which agent-scope atomic loads and stores carry: they reach the device's
// coherence point, past the XCD's own L2.
constexpr int kSc1 = 16;
constexpr int kNT = 2;    // cache policy of data read once (non-temporal)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kSc1);
}
__device__ __forceinline__ floatx4 load_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kSc1));
}

// A workgroup barrier that orders LDS accesses only: global loads in flight stay in flight
// across it (a full __syncthreads also waits for every outstanding global load, which would
// drain the weight stream at every stage).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int FMT, int G>
__global__ void __launch_bounds__(kPThreads, 4) prologue_kernel(PrologueLaunch a) {
  // the staged activations of two 128-column stages; the last workgroup of a tile reuses them
  // for the tile's summed rows
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][kPRows * kPStride];
  __shared__ float s_r[kPRows];
  __shared__ RowStage<kPSlots> s_st;
  __shared__ int s_word;
  static_assert(sizeof(s_a) >= kPRows * (kHeadDim + 1) * sizeof(float), "row tile fits the staging");

  const Layout& L = a.L;
  const int H = L.H, Hq = a.Hq, d = a.d;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nkv = 2 * H * a.splits_kv, nx = nkv + Hq * a.splits_q;
  const int nall = nx * a.row_blocks;
  // Roles are handed out in the order the workgroups start (an arrival ticket), K / V slices of
  // a row block before its Q slices: a Q workgroup that waits for K / V rows below only waits for
  // workgroups that have started before it, which never wait themselves.
  if (tid == 0) s_word = __hip_atomic_fetch_add(a.ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int ticket = s_word;
  __syncthreads();   // s_word is written again below
  if (ticket >= nall) {   // the control words were not zero before the call
    if (tid == 0) report(a.cache.status, KVQ_ERR_WORKSPACE);
    return;
  }
  const int rb = ticket / nx, wg = ticket % nx, row0 = rb * kPRows;
  const int nrows = min(kPRows, L.B - row0);
  // tile and K-slice of this role; the tile's slices are consecutive
  int tile, split, splits, first;
  if (wg < nkv) {
    tile = wg / a.splits_kv; split = wg % a.splits_kv; splits = a.splits_kv; first = tile * a.splits_kv;
  } else {
    tile = 2 * H + (wg - nkv) / a.splits_q; split = (wg - nkv) % a.splits_q; splits = a.splits_q;
    first = nkv + (tile - 2 * H) * a.splits_q;
  }
  // output rows of the projection: K head j at Hq + j, V head j at Hq + H + j, Q head j at j
  const int head_row = tile < 2 * H ? Hq + tile : tile - 2 * H;
  const int col0 = head_row * kHeadDim;
  const int nch = d / kPKc;
  const int per = (nch + splits - 1) / splits;
  const int c0 = min(nch, split * per), c1 = min(nch, c0 + per);

  // staging map: thread -> 8 columns (kseg) of rows srow + 32 i
  constexpr int kSR = kPThreads / 16;   // rows staged per pass
  constexpr int kSI = kPRows / kSR;     // passes
  const int kseg = tid & 15, srow = tid >> 4;
  // MFMA map: lane (r16, kg); wave -> columns 16 wave .. 16 wave + 15
  const int r16 = lane & 15, kg = lane >> 4;

  float ss[kSI];
#pragma unroll
  for (int i = 0; i < kSI; ++i) ss[i] = 0.0f;
  floatx4 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Activations one stage and weights two stages ahead of their use; weights are read once:
  // non-temporal loads.  Every stage issues the same loads without conditions (past the slice,
  // or past the row block, an offset beyond the buffer range reads zeros without touching
  // memory), so the wait counters stay exact and the loads in flight are never drained.
  constexpr uint32_t kOOB = 0xFFFFFFF0u;
  // the wave's 16 output rows: d / 32 consecutive 1 KB blocks of the packed weights
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(a.weight + (size_t)(col0 / 16 + wave) * (d / 32) * 512, (uint32_t)(d / 32) * 1024u);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.hidden + (size_t)row0 * d, (uint32_t)(nrows * d * 2));
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gain, (uint32_t)(d * 2));
  const uint32_t wlane = (uint32_t)lane * 16u;   // lane (r16, kg) of a block: row r16, columns 8 kg ..
  struct HSlot { u32x4 h[kSI]; u32x4 g; };
  HSlot h0, h1;
  u32x4 w0[4], w1[4], w2[4];
  auto load_h = [&](HSlot& hs, int c) {
    const bool in = c < c1;
    const uint32_t k0 = (uint32_t)(c * kPKc + 8 * kseg) * 2u;
    hs.g = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, (int)(in ? k0 : kOOB), 0, 0));
#pragma unroll
    for (int i = 0; i < kSI; ++i) {
      const int r = srow + kSR * i;
      const uint32_t off = in && r < nrows ? (uint32_t)(r * d) * 2u + k0 : kOOB;
      hs.h[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, (int)off, 0, 0));
    }
  };
  auto load_w = [&](u32x4 (&w)[4], int c) {
    const uint32_t base = c < c1 ? wlane + (uint32_t)c * 4096u : kOOB;   // 4 blocks per stage
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      w[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rw, (int)(base == kOOB ? kOOB : base + 1024u * ks), 0, kNT));
  };
  // bf16(h * g) of the staged columns into LDS, h^2 into the row sums
  auto stage = [&](const HSlot& hs, int buf) {
    const uint32_t g[4] = {hs.g[0], hs.g[1], hs.g[2], hs.g[3]};
#pragma unroll
    for (int i = 0; i < kSI; ++i) {
      const uint32_t hw[4] = {hs.h[i][0], hs.h[i][1], hs.h[i][2], hs.h[i][3]};
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float f0 = bf16_to_f32(hw[j] & 0xFFFFu), f1 = bf16_to_f32(hw[j] >> 16);
        const float g0 = bf16_to_f32(g[j] & 0xFFFFu), g1 = bf16_to_f32(g[j] >> 16);
        ss[i] += f0 * f0;
        ss[i] += f1 * f1;
        o[j] = f32_to_bf16(f0 * g0) | (f32_to_bf16(f1 * g1) << 16);
      }
      *(uint4*)&s_a[buf][(srow + kSR * i) * kPStride + 8 * kseg] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };
  auto mfma = [&](int buf, const u32x4 (&w)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 bw = __builtin_bit_cast(bf16x8, w[ks]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, *(const uint4*)&s_a[buf][(16 * mt + r16) * kPStride + 32 * ks + 8 * kg]);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw, acc[mt], 0, 0, 0);
      }
    }
  };

  // ---- the K-slice: stage c, issue the loads of c + 1 (activations) and c + 2 (weights),
  // multiply c.  Six stages per turn: the activation slots alternate, the weight slots rotate.
  if (c0 < c1) {
    load_h(h0, c0);
    load_w(w0, c0);
    load_w(w1, c0 + 1);
    int buf = 0;
    auto one = [&](int c, HSlot& hs, HSlot& hn, const u32x4 (&w)[4], u32x4 (&wn)[4]) {
      stage(hs, buf);
      load_h(hn, c + 1);
      load_w(wn, c + 2);
      lds_barrier();
      mfma(buf, w);
      buf ^= 1;
    };
    for (int c = c0; c < c1; c += 6) {
      one(c, h0, h1, w0, w2);
      if (c + 1 >= c1) break;
      one(c + 1, h1, h0, w1, w0);
      if (c + 2 >= c1) break;
      one(c + 2, h0, h1, w2, w1);
      if (c + 3 >= c1) break;
      one(c + 3, h1, h0, w0, w2);
      if (c + 4 >= c1) break;
      one(c + 4, h0, h1, w1, w0);
      if (c + 5 >= c1) break;
      one(c + 5, h1, h0, w2, w1);
    }
  }
  // row sums of h^2 over the slice: the 16 threads of a row are one 16-lane DPP row
#pragma unroll
  for (int i = 0; i < kSI; ++i) {
    ss[i] += xor_f32<8>(ss[i]);
    ss[i] += xor_f32<4>(ss[i]);
    ss[i] += xor_f32<2>(ss[i]);
    ss[i] += xor_f32<1>(ss[i]);
  }

  // ---- partial tile: [128 columns][64 rows] (a lane's four rows of a column are contiguous),
  // then the [64] row sums of h^2
  constexpr int kPart = kPRows * kHeadDim + kPRows;
  const __amdgpu_buffer_rsrc_t rpart = make_rsrc(a.partials + ((size_t)rb * nx + wg) * kPart, kPart * 4);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    store_coherent(rpart, ((16 * wave + r16) * kPRows + 16 * mt + 4 * kg) * 4, acc[mt]);
  if (kseg == 0) {
#pragma unroll
    for (int i = 0; i < kSI; ++i) s_r[srow + kSR * i] = ss[i];
  }
  __syncthreads();
  if (tid < kPRows / 4)
    store_coherent(rpart, (kPRows * kHeadDim + 4 * tid) * 4,
                   floatx4{s_r[4 * tid], s_r[4 * tid + 1], s_r[4 * tid + 2], s_r[4 * tid + 3]});
  // every store of the workgroup has completed before it arrives
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int* ctr = a.arrive + (size_t)rb * (2 * H + Hq) + tile;
  if (tid == 0) s_word = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
  __syncthreads();
  const bool last = s_word != 0;
  __syncthreads();   // s_word is written again below

  if (last) {
    // ---- the last workgroup of the tile: rows y = r * (sum of the partials in slice order)
    float* s_y = (float*)&s_a[0][0];   // [64][129]
    const __amdgpu_buffer_rsrc_t rall = make_rsrc(a.partials + ((size_t)rb * nx + first) * kPart,
                                                  (uint32_t)splits * kPart * 4);
    // every thread's vectors of 4 consecutive rows of a column (or of the row sums), summed over
    // the slices in slice order; the loads of two slices are in flight at once
    constexpr int kVec = kPart / 4, kPer = (kVec + kPThreads - 1) / kPThreads;
    floatx4 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) v[u] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int sl = 0; sl < splits; ++sl) {
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = tid + kPThreads * u;
        if (i < kVec) v[u] += load_coherent(rall, ((uint32_t)sl * kPart + 4 * i) * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + kPThreads * u;
      if (i >= kVec) continue;
      if (4 * i < kPRows * kHeadDim) {
        const int c = (4 * i) / kPRows, r = (4 * i) % kPRows;
#pragma unroll
        for (int j = 0; j < 4; ++j) s_y[(r + j) * (kHeadDim + 1) + c] = v[u][j];
      } else {
        const int r = 4 * i - kPRows * kHeadDim;
#pragma unroll
        for (int j = 0; j < 4; ++j) s_r[r + j] = 1.0f / sqrtf(v[u][j] / (float)d + a.eps);
      }
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int ncols = (Hq + 2 * H) * kHeadDim;
    if (a.proj_out) {
      for (int i = tid; i < nrows * kHeadDim; i += kPThreads) {
        const int r = i >> 7, c = i & 127;
        a.proj_out[(size_t)(row0 + r) * ncols + col0 + c] = s_y[r * (kHeadDim + 1) + c] * s_r[r];
      }
    }
    if (tile >= 2 * H) {   // query head: bf16 q
      for (int i = tid; i < nrows * kHeadDim; i += kPThreads) {
        const int r = i >> 7, c = i & 127;
        const float y = s_y[r * (kHeadDim + 1) + c] * s_r[r];
        a.q_out[((size_t)(row0 + r) * Hq + head_row) * kHeadDim + c] = (uint16_t)f32_to_bf16(y);
      }
    } else {
      // key or value head: the rows for the quantizing workgroups, then the tile's ready flag
      const __amdgpu_buffer_rsrc_t rrows =
          make_rsrc(a.kvrows + ((size_t)rb * 2 * H + tile) * kPRows * kHeadDim, kPRows * kHeadDim * 4);
      for (int i = tid; i < kPRows * kHeadDim / 4; i += kPThreads) {
        const int r = (4 * i) >> 7, c = (4 * i) & 127;
        const float* y = &s_y[r * (kHeadDim + 1) + c];
        store_coherent(rrows, 4 * i * 4, floatx4{y[0] * s_r[r], y[1] * s_r[r], y[2] * s_r[r], y[3] * s_r[r]});
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(a.ready + (size_t)rb * 2 * H + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
  }

  // ---- Q slices, once their own part is done, quantize the K / V rows of their row block into
  // the cache, kPSlots rows of one tile at a time (claimed in order from a counter)
  if (wg >= nkv) {
    constexpr int Lg = G / 4;
    const int slot = tid / kRowLanes, l32 = tid % kRowLanes;
    const int gi = l32 / Lg, jg = l32 % Lg;
    const int nbt = (nrows + kPSlots - 1) / kPSlots;   // batches per tile
    for (;;) {
      if (tid == 0) s_word = __hip_atomic_fetch_add(a.claim + rb, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const int batch = s_word;
      __syncthreads();
      if (batch >= 2 * H * nbt) break;
      const int kvtile = batch / nbt, r = (batch % nbt) * kPSlots + slot;
      const int kv = kvtile < H ? 0 : 1, hk = kvtile < H ? kvtile : kvtile - H;
      // the tile's rows are ready once its last slice has written them (bounded wait: the slices
      // started before this workgroup and wait for nothing)
      if (tid == 0) {
        const int* flag = a.ready + (size_t)rb * 2 * H + kvtile;
        int ok = 0;
        for (int it = 0; it < (1 << 22); ++it) {
          if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) { ok = 1; break; }
          __builtin_amdgcn_s_sleep(2);
        }
        if (!ok) report(a.cache.status, KVQ_ERR_HIP);
        s_word = ok;
      }
      __syncthreads();
      const bool ready = s_word != 0;
      __syncthreads();
      if (!ready) continue;
      const int b = row0 + min(r, nrows - 1);
      const int t = a.positions[b];
      const bool valid = r < nrows && t >= 0;
      const float* yrow = a.kvrows + (((size_t)rb * 2 * H + kvtile) * kPRows + min(r, nrows - 1)) * kHeadDim;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[e] = valid ? __hip_atomic_load(const_cast<float*>(yrow + gi * G + jg + Lg * e), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : 0.0f;
      const int64_t run = records_before<kRowLanes>(a, b, hk, kv, valid && t < L.S_cap ? t : 0, l32);
      append_row<FMT, G>(a, valid, b, hk, kv, t, run, x, l32, slot, s_st, [] { lds_barrier(); });
    }
  }

  // ---- the last workgroup to finish returns the control words to zero
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (tid == 0 && __hip_atomic_fetch_add(a.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nall - 1) {
    for (int i = 0; i < a.row_blocks * 2 * H; ++i)
      __hip_atomic_store(a.ready + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int i = 0; i < a.row_blocks; ++i)
      __hip_atomic_store(a.claim + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int FMT, int G>
hipError_t launch_fmt(const PrologueLaunch& a, dim3 grid, hipStream_t st) {
  prologue_kernel<FMT, G><<<grid, kPThreads, 0, st>>>(a);
  return hipGetLastError();
}

// Packed projection weights: for each group of 16 output rows (cg) and each step of 32 inputs
// (ks), one 1 KB block at (cg * d / 32 + ks) * 1 KB whose 16-byte lane l = 16 q + j holds
// W[16 cg + j][32 ks + 8 q .. 32 ks + 8 q + 7]: the B operand of one MFMA for one wave.  A
// wave's stream through d is then contiguous.
__global__ void __launch_bounds__(256) pack_weights_kernel(const uint4* __restrict__ w, uint4* __restrict__ out,
                                                            int d, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 16-byte unit of the output
  if (i >= n16) return;
  const int64_t blk = i >> 6;
  const int l = (int)(i & 63), j = l & 15, q = l >> 4;
  const int nks = d / 32;
  const int64_t cg = blk / nks, ks = blk % nks;
  const int64_t row = 16 * cg + j, col = 32 * ks + 8 * q;
  out[i] = w[(row * d + col) / 8];
}

}  // namespace

hipError_t launch_pack_weights(const void* w, void* out, int d, int64_t rows, hipStream_t st) {
  const int64_t n16 = rows * d / 8;
  pack_weights_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, st>>>((const uint4*)w, (uint4*)out, d, n16);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueLaunch& a, hipStream_t st) {
  const dim3 grid((2 * a.L.H * a.splits_kv + a.Hq * a.splits_q) * a.row_blocks);
  const bool g32 = a.group == 32;
  switch (a.fmt) {
    case FMT_C2: return g32 ? hipErrorInvalidValue : launch_fmt<FMT_C2, 64>(a, grid, st);
    case FMT_INT4: return g32 ? launch_fmt<FMT_INT4, 32>(a, grid, st) : launch_fmt<FMT_INT4, 64>(a, grid, st);
    case FMT_FP4: return g32 ? launch_fmt<FMT_FP4, 32>(a, grid, st) : launch_fmt<FMT_FP4, 64>(a, grid, st);
    case FMT_INT3: return g32 ? launch_fmt<FMT_INT3, 32>(a, grid, st) : launch_fmt<FMT_INT3, 64>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
