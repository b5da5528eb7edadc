// Entropy-guided tiering of paged caches: page attention masses from a decode's per-page
// log-sum-exps, the choice of the pages that keep the FP8 tier, the assignment of 2-bit pool
// slots to the FP8 pages that leave it, and the block-table update.  The rows of those pages are
// re-quantized and their outlier records merged into the lists by the kernels of quantize.hip.
//
// "Hierarchical Token Gating and Tiered KV-Cache Paging ...", section "2. Entropy-Guided Tiered
// KV-Cache Quantization" ("Dual-Tier Paged Compression Protocol": the highest-attention part of
// the cache stays FP8, the rest is 2-bit) and "Operational Blueprint for AI Systems Engineers",
// item 2 (the ranking is refreshed every N decode steps).
#include "kvq_device.h"
#include "kvq_launch.h"

namespace kvq {
namespace {

// mass[b][p] = (1/Hq) sum_hq 2^(page_lse[b][hq][p] - total_lse[b][hq]) for the pages holding
// tokens < S_b (the mean over query heads of the page's share of the softmax weight); 0 for the
// other entries of the row and for sequences whose length the decode rejected
__global__ void __launch_bounds__(256) mass_normalize_kernel(MassLaunch m) {
  const int b = blockIdx.y;
  const int p = blockIdx.x * 256 + (int)threadIdx.x;
  if (p >= m.max_pages) return;
  const int S = m.seq_lens[b];
  const int np = S >= 1 && S <= m.S_cap ? (S + kBlock - 1) / kBlock : 0;
  float sum = 0.0f;
  if (p < np) {
    for (int hq = 0; hq < m.Hq; ++hq) {
      const size_t bh = (size_t)b * m.Hq + hq;
      sum += exp2f(m.page_lse[bh * m.max_pages + p] - m.total_lse[bh]);
    }
    sum /= (float)m.Hq;
  }
  m.mass[(size_t)b * m.max_pages + p] = sum;
}

// Per sequence: the hot pages are the ceil(keep_frac * n) pages of largest mass, ties to the
// lower page (a bitonic sort of keys ~mass_bits << 32 | page: masses are non-negative, so their
// bit patterns order like their values).  An FP8 page that is not hot is a candidate.
__global__ void __launch_bounds__(1024) retier_select_kernel(RetierLaunch r) {
  __shared__ uint64_t s_key[kRetierMaxPages];
  __shared__ uint8_t s_hot[kRetierMaxPages];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int S = r.seq_lens[b];
  const int np = S >= 1 && S <= r.L.S_cap ? (S + kBlock - 1) / kBlock : 0;
  int n2 = 1;
  while (n2 < np) n2 <<= 1;
  for (int i = tid; i < n2; i += 1024) {
    s_key[i] = i < np ? ((uint64_t)(~__float_as_uint(r.mass[(size_t)b * r.L.max_pages + i])) << 32) | (uint32_t)i
                      : ~0ull;
    s_hot[i] = 0;
  }
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += 1024) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t a = s_key[i], c = s_key[l];
          const bool up = (i & k) == 0;
          if ((a > c) == up) { s_key[i] = c; s_key[l] = a; }
        }
      }
      __syncthreads();
    }
  }
  const int keep = min(np, (int)ceil((double)r.keep_frac * (double)np));
  for (int i = tid; i < keep; i += 1024) s_hot[(uint32_t)s_key[i]] = 1;
  __syncthreads();
  const int32_t* bt = r.block_table + (size_t)b * r.L.max_pages;
  for (int p = tid; p < r.L.max_pages; p += 1024) {
    const bool fp8 = p < np && ((uint32_t)bt[p] >> 31) != 0;
    r.cand[(size_t)b * r.L.max_pages + p] = fp8 && !s_hot[p] ? 1 : 0;
  }
}

// One workgroup: the candidates in (sequence, page) order take the free 2-bit slots in order;
// candidates past the free slots stay FP8.  moves[b][p] = the page's new 2-bit slot or -1;
// rank[b][p] = its place among the moved pages; moved[rank] = b * max_pages + p (-1: a free
// slot outside the pool, the page stays); freed[rank] = its FP8 slot; *n_moved = the number of
// ranks handed out.
__global__ void __launch_bounds__(1024) retier_assign_kernel(RetierLaunch r) {
  __shared__ int s_part[1024];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)r.L.B * r.L.max_pages;
  const int64_t per = (n + 1023) / 1024;
  const int64_t e0 = min(n, per * tid), e1 = min(n, e0 + per);
  int cnt = 0;
  for (int64_t e = e0; e < e1; ++e) cnt += r.cand[e];
  s_part[tid] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive scan of the per-thread counts
    const int v = tid >= o ? s_part[tid - o] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int rank = s_part[tid] - cnt;
  for (int64_t e = e0; e < e1; ++e) {
    int32_t mv = -1, rk = -1;
    if (r.cand[e]) {
      if (rank < r.n_cand) {   // n_cand: at most the free slots and the FP8 pool's size
        const int32_t slot = r.free_slots[rank];
        r.moved[rank] = -1;
        if (slot >= 0 && slot < r.L.num_pages) {
          mv = slot;
          rk = rank;
          r.moved[rank] = (int32_t)e;
          r.freed[rank] = r.block_table[e] & 0x7FFFFFFF;
        } else {
          report(r.cache.status, KVQ_ERR_INVALID_ARG);   // a free slot outside the 2-bit pool
          r.freed[rank] = -1;
        }
      }
      ++rank;
    }
    r.moves[e] = mv;
    r.rank[e] = rk;
  }
  if (tid == 1023) {
    const int total = s_part[1023];
    *r.n_moved = min(total, r.n_cand);
  }
}

// the moved pages' block-table entries now name their 2-bit slots (after their rows and
// records are written)
__global__ void __launch_bounds__(256) retier_commit_kernel(RetierLaunch r) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)r.L.B * r.L.max_pages) return;
  const int32_t mv = r.moves[e];
  if (mv >= 0) r.block_table[e] = mv;
}

}  // namespace

hipError_t launch_mass_normalize(const MassLaunch& m, hipStream_t st) {
  mass_normalize_kernel<<<dim3((m.max_pages + 255) / 256, m.B), 256, 0, st>>>(m);
  return hipGetLastError();
}

hipError_t launch_retier_select(const RetierLaunch& r, hipStream_t st) {
  retier_select_kernel<<<r.L.B, 1024, 0, st>>>(r);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  retier_assign_kernel<<<1, 1024, 0, st>>>(r);
  return hipGetLastError();
}

hipError_t launch_retier_commit(const RetierLaunch& r, hipStream_t st) {
  const int64_t n = (int64_t)r.L.B * r.L.max_pages;
  retier_commit_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(r);
  return hipGetLastError();
}

}  // namespace kvq
