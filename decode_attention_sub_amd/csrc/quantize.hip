// Quantize-on-append: group statistics, outlier isolation, quantizer fit, encoding, packing
// and ordered compaction of outlier records into the per-list COO side lists.
//
// "Hierarchical Token Routing and Sub-2-Bit Non-Linear KV Compression ...", section
// "Paradigm 2": outliers beyond tau standard deviations kept apart at higher precision, the
// rest coded against a 4-centroid codebook fitted by k-means; "The Sub-10ms Barrier ...",
// section "2. FP4/INT4 KV-Cache Quantization": per-group scale (max - min)/(2^b - 1) computed
// at token insertion; "Hierarchical Token Gating and Tiered KV-Cache Paging ...", section
// "2. Entropy-Guided Tiered KV-Cache Quantization": FP8 tier rows.
//
// Bit-exactness contract: every decision is taken in float32 with round-to-nearest-even, no
// fused multiply-add (contraction is off in this file), correctly rounded division, and every
// sum over a group follows one fixed pairwise tree: for w = g/2, g/4, ..., 1:
// a[i] += a[i + w] for i < w.  With L = g/4 lanes per group and lane j holding group elements
// j, j+L, j+2L, j+3L, the steps w = 2L and w = L are in-lane and the steps w < L are xor
// exchanges between lanes (every lane then holds the root by commutativity of addition).
#pragma clang fp contract(off)

#include <type_traits>

#include "kvq_device.h"
#include "kvq_launch.h"
#include "quant_row.h"

namespace kvq {
namespace {


struct QArgs {
  Layout L;
  kvq_cache cache;
  const float* k_new;
  const float* v_new;
  const int32_t* positions;
  const int32_t* counts;
  const int32_t* block_table;
  int max_new;
  int outl;          // kvq_outlier_dtype
  float tau2;        // fl32(tau * tau)
  int lloyd;
  int fit;           // kFitDefault, or a variant fit of the storage format
};

// ---------------------------------------------------------------- kernel
template <int FMT, int G, int NW>
__global__ void __launch_bounds__(64 * NW) quantize_append_kernel(QArgs a) {
  constexpr int L = G / 4;          // lanes per group
  constexpr int RPI = 2 * NW;       // rows per iteration
  constexpr int CB = kHeadDim * code_bits(FMT) / 8;
  __shared__ uint8_t s_code[RPI][kHeadDim];
  __shared__ uint8_t s_flag[RPI][kHeadDim];
  __shared__ float s_x[RPI][kHeadDim];
  __shared__ uint32_t s_meta[RPI][8];
  __shared__ int s_tier[RPI];
  __shared__ int s_rowtot[RPI];
  __shared__ int s_trunc;

  const Layout& Lo = a.L;
  const int list = blockIdx.x;
  const int kv = list & 1;
  const int h = (list >> 1) % Lo.H;
  const int b = (list >> 1) / Lo.H;
  const int tid = threadIdx.x;
  const int slot = tid / kRowLanes;
  const int lane = tid % kRowLanes;
  const int gi = lane / L;          // group within the row
  const int jg = lane % L;          // lane within the group

  const int p = a.positions[b];
  const int n = a.counts[b];
  // the first rows' values are loaded with the position and count (row min(slot, max_new - 1)
  // is inside k_new / v_new whatever the count; rows past it are zeroed below)
  const float* src = (kv == 0 ? a.k_new : a.v_new) + ((size_t)b * Lo.H + h) * (size_t)a.max_new * kHeadDim;
  float x0[4];
  {
    const int srow = min(slot, a.max_new - 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) x0[e] = src[(size_t)srow * kHeadDim + gi * G + jg + L * e];
  }
  if (n <= 0) return;
  if (p < 0 || n > a.max_new || (int64_t)p + n > Lo.S_cap) {
    if (tid == 0) report(a.cache.status, KVQ_ERR_INVALID_ARG);
    return;
  }
  const size_t lid = list_id(Lo, b, h, kv);
  int32_t* bstart = a.cache.outl_block_start + lid * (size_t)Lo.nblk;
  uint32_t* oidx = a.cache.outl_idx[kv] + ((size_t)b * Lo.H + h) * (size_t)Lo.outl_cap;
  uint8_t* oval = (uint8_t*)a.cache.outl_val[kv] +
                  ((size_t)b * Lo.H + h) * (size_t)Lo.outl_cap * (a.outl == KVQ_OUTL_FP16 ? 2 : 1);

  // The list is truncated to the records of tokens < p: the records before the start of p's
  // 16-token block, plus those of the block's rows before p.  A block holds at most 16 rows of D
  // records, and the list is sorted, so each thread stops at its first record of a token >= p.
  // The scan's bounds and first loads are issued here; it is finished after the first rows'
  // fits (which do not need it), before their records are written.
  if (tid == 0) s_trunc = 0;
  int64_t start = 0, lim = 0;
  uint32_t first_idx = 0xFFFFFFFFu;
  if (p > 0) {
    start = max((int64_t)0, min((int64_t)bstart[(p - 1) >> 4], Lo.outl_cap));
    const int64_t old = max((int64_t)0, min((int64_t)a.cache.outl_count[lid], Lo.outl_cap));
    lim = min(old, start + (int64_t)kBlock * kHeadDim);
    if (start + tid < lim) first_idx = oidx[start + tid];
  }
  int64_t running = 0;

  for (int i0 = 0; i0 < n; i0 += RPI) {
    const int r = i0 + slot;
    const bool valid = r < n;
    const int t = p + r;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = !valid ? 0.0f : i0 == 0 ? x0[e] : src[(size_t)r * kHeadDim + gi * G + jg + L * e];
    int tier1 = 0;
    size_t pslot = 0;
    bool row_ok = valid;
    if (Lo.paged && valid) {
      row_ok = page_slot(Lo, a.block_table, b, t, &tier1, &pslot);
      if (!row_ok && lane == 0) report(a.cache.status, KVQ_ERR_INVALID_ARG);
    }
    RowOut o;
    if (tier1) {
      fit_fp8row(x, o);
    } else {
      bool keep[4] = {true, true, true, true};
      if (a.outl != KVQ_OUTL_NONE) {
        if (a.cache.chan_mask) {   // static channel mask: the masked channels are the outliers
          const uint32_t* mw = a.cache.chan_mask + ((size_t)kv * Lo.H + h) * (kHeadDim / 32);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = gi * G + jg + L * e;
            keep[e] = ((mw[c >> 5] >> (c & 31)) & 1u) == 0u;
          }
        } else {
          outlier_flags<G>(x, a.tau2, keep);
        }
      }
      if constexpr (FMT == FMT_INT4) {
        if (a.fit == kFitSym) fit_int4sym<G>(x, keep, o);
        else fit_int4<G>(x, keep, o);
      } else if constexpr (FMT == FMT_INT3) {
        fit_int4<G, 7>(x, keep, o);
      } else if constexpr (FMT == FMT_FP4) {
        fit_fp4<G>(x, keep, o);
      } else {
        if (a.fit == kFitUniform) fit_u2<G>(x, keep, o);
        else fit_c2<G>(x, keep, jg, a.lloyd, o);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) o.flag[e] = keep[e] ? 0u : 1u;
    }
    // stage the row in LDS
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = gi * G + jg + L * e;
      s_code[slot][c] = (uint8_t)o.code[e];
      s_flag[slot][c] = valid ? (uint8_t)o.flag[e] : 0;
      s_x[slot][c] = x[e];
    }
    if (tier1) {
      if (lane == 0) s_meta[slot][0] = o.meta[0];
    } else if (jg == 0) {
      constexpr int MB = meta_bytes_per_group(FMT);
      if constexpr (MB == 8) { s_meta[slot][2 * gi] = o.meta[0]; s_meta[slot][2 * gi + 1] = o.meta[1]; }
      else if constexpr (MB == 4) { s_meta[slot][gi] = o.meta[0]; }
      else { ((uint8_t*)s_meta[slot])[gi] = (uint8_t)o.meta[0]; }
    }
    if (lane == 0) s_tier[slot] = tier1;
    __syncthreads();
    if (i0 == 0 && p > 0) {   // the truncation scan, finished (every thread of the workgroup)
      int cnt = 0;
      if (first_idx < (uint32_t)p * kHeadDim) {
        cnt = 1;
        for (int64_t rr = start + tid + blockDim.x; rr < lim; rr += blockDim.x) {
          if (oidx[rr] >= (uint32_t)p * kHeadDim) break;
          ++cnt;
        }
      }
      if (cnt) atomicAdd(&s_trunc, cnt);
      __syncthreads();
      running = start + s_trunc;
    }

    // pack codes and write the row
    if (row_ok) {
      const int tr = s_tier[slot];
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
        if (tr) {
          codes_dst = (uint8_t*)a.cache.codes8[kv] + prow * kHeadDim;
          meta_dst = (uint8_t*)(a.cache.scale8[kv] + prow);
          cb = kHeadDim; mb = 4;
        } else {
          codes_dst = (uint8_t*)a.cache.codes[kv] + prow * CB;
          meta_dst = (uint8_t*)a.cache.meta[kv] + prow * Lo.meta_bytes;
          cb = CB; mb = Lo.meta_bytes;
        }
      }
      const int bits = tr ? 8 : code_bits(FMT);
      if (lane < cb / 4) ((uint32_t*)codes_dst)[lane] = pack_word(s_code[slot], lane, bits);
      if (lane < mb / 4) ((uint32_t*)meta_dst)[lane] = s_meta[slot][lane];
      else if (mb < 4 && lane == 0) {
        for (int k = 0; k < mb; ++k) meta_dst[k] = ((uint8_t*)s_meta[slot])[k];
      }
    }

    // ordered compaction of outlier records: channels 4*lane .. 4*lane+3 of this row
    uint32_t fl = 0;
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t f = s_flag[slot][4 * lane + k];
      fl |= f << k;
      cnt += (int)f;
    }
    int incl = cnt;  // inclusive scan over the 32 lanes of the row
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const int y = __shfl_up(incl, d, 32);
      if (lane >= d) incl += y;
    }
    if (lane == 31) s_rowtot[slot] = incl;
    __syncthreads();
    int64_t base = running;
    for (int s = 0; s < slot; ++s) base += s_rowtot[s];
    int64_t total = 0;
    for (int s = 0; s < RPI; ++s) total += s_rowtot[s];
    if (valid) {
      if ((t & 15) == 0 && lane == 0) bstart[t >> 4] = (int32_t)min(base, (int64_t)INT32_MAX);
      int64_t k = base + (incl - cnt);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if ((fl >> q) & 1u) {
          const int c = 4 * lane + q;
          if (k < Lo.outl_cap) {
            oidx[k] = (uint32_t)t * kHeadDim + (uint32_t)c;
            const float xv = s_x[slot][c];
            if (a.outl == KVQ_OUTL_FP16) ((uint16_t*)oval)[k] = (uint16_t)f32_to_half_bits(xv);
            else oval[k] = (uint8_t)f32_to_e4m3(xv);
          } else {
            report(a.cache.status, KVQ_ERR_CAPACITY);
          }
          ++k;
        }
      }
    }
    running += total;
    __syncthreads();
  }
  if (tid == 0) a.cache.outl_count[lid] = (int32_t)min(running, Lo.outl_cap);
}

// ---------------------------------------------------------------- tiering: FP8 pages to 2-bit
// The rows of a moved page (one workgroup per (moved page, KV head, K or V); 16 rows of 32
// lanes): x' = fl32(e4m3(code) * row scale) from the page's FP8 slot, the outlier predicate (or
// the static channel mask) and the 2-bit fit as in an append, codes and centroids written to the
// page's new 2-bit slot, the outlier flags kept as a bitmap (16 rows x 4 words) for the list pass.
__global__ void __launch_bounds__(16 * kRowLanes) retier_quantize_kernel(RetierLaunch r) {
  constexpr int G = 64, L = G / 4;
  __shared__ uint8_t s_code[kBlock][kHeadDim];
  __shared__ uint8_t s_flag[kBlock][kHeadDim];
  const Layout& Lo = r.L;
  const int item = blockIdx.x;
  const int kv = item & 1, h = (item >> 1) % Lo.H, rank = (item >> 1) / Lo.H;
  if (rank >= *r.n_moved) return;
  const int32_t e = r.moved[rank];
  if (e < 0) return;
  const int b = e / Lo.max_pages, p = e % Lo.max_pages;
  const int S = r.seq_lens[b];
  const int tid = threadIdx.x, row = tid / kRowLanes, lane = tid % kRowLanes;
  const int gi = lane / L, jg = lane % L;
  const bool valid = kBlock * p + row < S;
  const uint32_t slot8 = (uint32_t)r.block_table[e] & 0x7FFFFFFFu;   // not yet rewritten
  const uint32_t slot2 = (uint32_t)r.moves[e];
  const size_t r8 = ((size_t)slot8 * Lo.H + h) * kBlock + row;
  const uint8_t* c8 = (const uint8_t*)r.cache.codes8[kv] + r8 * kHeadDim;
  const float s8 = valid ? r.cache.scale8[kv][r8] : 0.0f;
  float x[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) x[k] = valid ? e4m3_to_f32(c8[gi * G + jg + L * k]) * s8 : 0.0f;
  bool keep[4] = {true, true, true, true};
  if (r.outl != KVQ_OUTL_NONE) {
    if (r.cache.chan_mask) {
      const uint32_t* mw = r.cache.chan_mask + ((size_t)kv * Lo.H + h) * (kHeadDim / 32);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = gi * G + jg + L * k;
        keep[k] = ((mw[c >> 5] >> (c & 31)) & 1u) == 0u;
      }
    } else {
      outlier_flags<G>(x, r.tau2, keep);
    }
  }
  RowOut o;
  fit_c2<G>(x, keep, jg, r.lloyd, o);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = gi * G + jg + L * k;
    s_code[row][c] = (uint8_t)o.code[k];
    s_flag[row][c] = valid && !keep[k] ? 1 : 0;
  }
  __syncthreads();
  uint32_t* bm = r.bitmaps + ((size_t)rank * Lo.H * 2 + (size_t)h * 2 + kv) * (kBlock * 4);
  if (lane < 4) {
    uint32_t w = 0;
    for (int k = 0; k < 32; ++k) w |= (uint32_t)s_flag[row][32 * lane + k] << k;
    bm[row * 4 + lane] = w;
  }
  if (!valid) return;
  const size_t r2 = ((size_t)slot2 * Lo.H + h) * kBlock + row;
  if (lane < 8) {   // 2-bit: channel 4s + j of the word's 16 goes to byte j, bit pair s
    uint32_t w = 0;
    for (int k = 0; k < 16; ++k) w |= (uint32_t)s_code[row][lane * 16 + k] << (8 * (k & 3) + 2 * (k >> 2));
    ((uint32_t*)((uint8_t*)r.cache.codes[kv] + r2 * 32))[lane] = w;
  }
  if (jg == 0) {
    uint32_t* md = (uint32_t*)((uint8_t*)r.cache.meta[kv] + r2 * 16);
    md[2 * gi] = o.meta[0];
    md[2 * gi + 1] = o.meta[1];
  }
}

// One list (sequence, KV head, K or V): the record counts of its pages (a moved page: its bitmap;
// any other: its old range), new block starts by a prefix sum, the old records moved to their
// new places (back to front, a block of 256 at a time: records only move up), the moved pages'
// records written in token and channel order, then the block starts and the count.  Records
// past the list's capacity are dropped and reported, as in an append.
__global__ void __launch_bounds__(256) retier_lists_kernel(RetierLaunch r) {
  __shared__ int s_new[kRetierMaxPages + 1];
  __shared__ int s_part[256];
  const Layout& Lo = r.L;
  const int list = blockIdx.x;
  const int kv = list & 1, h = (list >> 1) % Lo.H, b = (list >> 1) / Lo.H;
  const int S = r.seq_lens[b];
  if (S < 1 || S > Lo.S_cap) return;
  const int np = (S + kBlock - 1) / kBlock;
  const int tid = threadIdx.x;
  const size_t lid = list_id(Lo, b, h, kv);
  int32_t* bstart = r.cache.outl_block_start + lid * (size_t)Lo.nblk;
  uint32_t* oidx = r.cache.outl_idx[kv] + ((size_t)b * Lo.H + h) * (size_t)Lo.outl_cap;
  const int VB = r.outl == KVQ_OUTL_FP16 ? 2 : 1;
  uint8_t* oval = (uint8_t*)r.cache.outl_val[kv] + ((size_t)b * Lo.H + h) * (size_t)Lo.outl_cap * VB;
  const int64_t cap = Lo.outl_cap;
  const int old = (int)max((int64_t)0, min((int64_t)r.cache.outl_count[lid], cap));
  const int32_t* mv = r.moves + (size_t)b * Lo.max_pages;
  const int32_t* rk = r.rank + (size_t)b * Lo.max_pages;
  // a sequence with no moved page keeps its lists as they are
  int any = 0;
  for (int p = tid; p < np; p += 256) any |= mv[p] >= 0;
  if (!__syncthreads_or(any)) return;
  auto bitmap = [&](int p) {
    return r.bitmaps + ((size_t)rk[p] * Lo.H * 2 + (size_t)h * 2 + kv) * (kBlock * 4);
  };
  auto old_start = [&](int p) { return p < np ? max(0, min(bstart[p], old)) : old; };
  // counts per page, then an exclusive scan in place (chunks of pages per thread)
  for (int p = tid; p < np; p += 256) {
    int c;
    if (mv[p] >= 0) {
      const uint32_t* bm = bitmap(p);
      c = 0;
      for (int i = 0; i < kBlock * 4; ++i) c += __builtin_popcount(bm[i]);
    } else {
      c = max(0, old_start(p + 1) - old_start(p));
    }
    s_new[p] = c;
  }
  __syncthreads();
  const int per = (np + 255) / 256;
  const int q0 = min(np, per * tid), q1 = min(np, q0 + per);
  int sum = 0;
  for (int q = q0; q < q1; ++q) sum += s_new[q];
  s_part[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int run = s_part[tid] - sum;
  for (int q = q0; q < q1; ++q) { const int c = s_new[q]; s_new[q] = run; run += c; }
  if (tid == 255) s_new[np] = s_part[255];
  __syncthreads();
  const int total = s_new[np];
  // old records move up by the records inserted before their page
  for (int j = old; j > 0; j -= 256) {
    const int i = j - 256 + tid;
    uint32_t ix = 0, vl = 0;
    int dst = -1;
    if (i >= 0) {
      ix = oidx[i];
      vl = VB == 2 ? ((const uint16_t*)oval)[i] : oval[i];
      const int pg = min((int)(ix / kHeadDim) / kBlock, np);
      dst = i + (pg < np ? s_new[pg] - old_start(pg) : total - old);
    }
    __syncthreads();
    if (i >= 0 && dst < cap) {
      oidx[dst] = ix;
      if (VB == 2) ((uint16_t*)oval)[dst] = (uint16_t)vl;
      else oval[dst] = (uint8_t)vl;
    }
  }
  __syncthreads();
  // records of the moved pages: one thread per (page, row)
  for (int q = tid; q < np * kBlock; q += 256) {
    const int p = q / kBlock, row = q % kBlock;
    if (mv[p] < 0) continue;
    const uint32_t* bm = bitmap(p);
    int pos = s_new[p];
    for (int i = 0; i < row * 4; ++i) pos += __builtin_popcount(bm[i]);
    const uint32_t slot8 = (uint32_t)r.block_table[(size_t)b * Lo.max_pages + p] & 0x7FFFFFFFu;
    const size_t r8 = ((size_t)slot8 * Lo.H + h) * kBlock + row;
    const uint8_t* c8 = (const uint8_t*)r.cache.codes8[kv] + r8 * kHeadDim;
    const float s8 = r.cache.scale8[kv][r8];
    const uint32_t t = (uint32_t)(kBlock * p + row);
    for (int w = 0; w < 4; ++w) {
      uint32_t bits = bm[row * 4 + w];
      while (bits) {
        const int c = 32 * w + __builtin_ctz(bits);
        bits &= bits - 1;
        if (pos < cap) {
          const float xv = e4m3_to_f32(c8[c]) * s8;
          oidx[pos] = t * kHeadDim + (uint32_t)c;
          if (VB == 2) ((uint16_t*)oval)[pos] = (uint16_t)f32_to_half_bits(xv);
          else oval[pos] = (uint8_t)f32_to_e4m3(xv);
        }
        ++pos;
      }
    }
  }
  for (int p = tid; p < np; p += 256) bstart[p] = s_new[p];
  if (tid == 0) {
    if (total > cap) report(r.cache.status, KVQ_ERR_CAPACITY);
    r.cache.outl_count[lid] = (int32_t)min((int64_t)total, cap);
  }
}

template <int FMT, int G>
hipError_t launch_quantize_t(const QArgs& qa, int nlists, int max_new, hipStream_t st) {
  if (max_new <= 2) {
    quantize_append_kernel<FMT, G, 1><<<nlists, 64, 0, st>>>(qa);
  } else {
    quantize_append_kernel<FMT, G, 4><<<nlists, 256, 0, st>>>(qa);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_retier_demote(const RetierLaunch& r, hipStream_t st) {
  if (r.n_cand > 0) {
    retier_quantize_kernel<<<(unsigned)((int64_t)r.n_cand * r.L.H * 2), 16 * kRowLanes, 0, st>>>(r);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  retier_lists_kernel<<<(unsigned)(r.L.B * r.L.H * 2), 256, 0, st>>>(r);
  return hipGetLastError();
}

hipError_t launch_quantize_append(const QuantizeLaunch& q, hipStream_t st) {
  QArgs qa;
  qa.L = q.L;
  qa.cache = q.cache;
  qa.k_new = q.k_new;
  qa.v_new = q.v_new;
  qa.positions = q.positions;
  qa.counts = q.counts;
  qa.block_table = q.block_table;
  qa.max_new = q.max_new;
  qa.outl = q.outl;
  qa.tau2 = q.tau2;
  qa.lloyd = q.lloyd;
  qa.fit = q.fit;
  const int nlists = q.L.B * q.L.H * 2;
  switch (q.fmt) {
    case FMT_INT4: return q.group == 32 ? launch_quantize_t<FMT_INT4, 32>(qa, nlists, q.max_new, st)
                                        : launch_quantize_t<FMT_INT4, 64>(qa, nlists, q.max_new, st);
    case FMT_FP4: return q.group == 32 ? launch_quantize_t<FMT_FP4, 32>(qa, nlists, q.max_new, st)
                                       : launch_quantize_t<FMT_FP4, 64>(qa, nlists, q.max_new, st);
    case FMT_C2: return launch_quantize_t<FMT_C2, 64>(qa, nlists, q.max_new, st);
    case FMT_INT3: return q.group == 32 ? launch_quantize_t<FMT_INT3, 32>(qa, nlists, q.max_new, st)
                                        : launch_quantize_t<FMT_INT3, 64>(qa, nlists, q.max_new, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
