/* Plain C client of include/kvq.h on the GPU: device buffers from hipMalloc, one append of two
 * tokens and one decode, no C++ or Python in between.  The packed 2-bit codes and the centroids
 * of every appended row are read back and checked against the packing order and metadata
 * layout the header states; the decode uses the header's default softmax scale (NaN).
 *
 * Every 64-channel group of the K and V rows holds four values, each in 16 channels, so the
 * 2-bit fit (quartile seeds, Lloyd iterations) reproduces them exactly in fp16 and no value lies
 * beyond 3 standard deviations of its group.  Both tokens have the same K row, so each query
 * gives them equal weight and the output is the mean of the two V rows, to fp32 rounding. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvq.h"

enum { B = 2, HQ = 8, H = 2, D = 128, SCAP = 64, NT = 2 };

static const float kLevels[4] = {-1.5f, -0.5f, 0.5f, 2.0f};

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));                  \
      return 1;                                                               \
    }                                                                         \
  } while (0)

static void* dev_zero(size_t bytes) {
  void* p = NULL;
  if (bytes == 0) bytes = 4;
  if (hipMalloc(&p, bytes) != hipSuccess) return NULL;
  if (hipMemset(p, 0, bytes) != hipSuccess) return NULL;
  return p;
}

int main(void) {
  kvq_params p;
  memset(&p, 0, sizeof p);
  p.batch = B; p.num_q_heads = HQ; p.num_kv_heads = H; p.head_dim = D; p.max_seq_len = SCAP;
  p.format = KVQ_FMT_CENTROID2; p.group_size = 64; p.outlier_dtype = KVQ_OUTL_FP8_E4M3;
  p.outlier_sigma = 3.0f; p.lloyd_iters = 8;

  const int64_t cap = 1024;
  kvq_cache_sizes_t sz;
  if (kvq_cache_sizes(&p, cap, &sz) != KVQ_OK) { printf("FAIL kvq_cache_sizes\n"); return 1; }
  kvq_cache c;
  memset(&c, 0, sizeof c);
  for (int kv = 0; kv < 2; ++kv) {
    c.codes[kv] = dev_zero(sz.codes);
    c.meta[kv] = dev_zero(sz.meta);
    c.outl_idx[kv] = (uint32_t*)dev_zero(sz.outl_idx);
    c.outl_val[kv] = dev_zero(sz.outl_val);
    if (!c.codes[kv] || !c.meta[kv] || !c.outl_idx[kv] || !c.outl_val[kv]) { printf("FAIL alloc\n"); return 1; }
  }
  c.outl_count = (int32_t*)dev_zero(sz.outl_count);
  c.outl_block_start = (int32_t*)dev_zero(sz.outl_block_start);
  c.outl_capacity = cap;
  c.status = (int32_t*)dev_zero(sizeof(int32_t));
  if (!c.outl_count || !c.outl_block_start || !c.status) { printf("FAIL alloc\n"); return 1; }

  /* new rows [B][H][NT][D]: K the same for both tokens, V token 0 and token 1 differ */
  static float k[B * H * NT * D], v[B * H * NT * D];
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int t = 0; t < NT; ++t)
        for (int ch = 0; ch < D; ++ch) {
          const size_t i = (((size_t)b * H + h) * NT + t) * D + ch;
          k[i] = kLevels[(ch + b + h) % 4];
          v[i] = kLevels[(ch + b + 2 * h + 3 * t) % 4];
        }
  int32_t pos[B] = {0, 0}, cnt[B] = {NT, NT}, lens[B] = {NT, NT};
  static uint16_t q[B * HQ * D];
  for (size_t i = 0; i < (size_t)B * HQ * D; ++i) q[i] = (uint16_t)(0x3E80u + (i % 7) * 0x10u);

  float *dk, *dv, *dout;
  int32_t *dpos, *dcnt, *dlens;
  uint16_t* dq;
  HIP_OK(hipMalloc((void**)&dk, sizeof k));
  HIP_OK(hipMalloc((void**)&dv, sizeof v));
  HIP_OK(hipMalloc((void**)&dq, sizeof q));
  HIP_OK(hipMalloc((void**)&dout, sizeof(float) * B * HQ * D));
  HIP_OK(hipMalloc((void**)&dpos, sizeof pos));
  HIP_OK(hipMalloc((void**)&dcnt, sizeof cnt));
  HIP_OK(hipMalloc((void**)&dlens, sizeof lens));
  HIP_OK(hipMemcpy(dk, k, sizeof k, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, v, sizeof v, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dq, q, sizeof q, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dpos, pos, sizeof pos, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dcnt, cnt, sizeof cnt, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dlens, lens, sizeof lens, hipMemcpyHostToDevice));

  int fails = 0;
  int32_t st = kvq_quantize_append(&p, &c, dk, dv, NT, dpos, dcnt, NULL, NULL);
  printf("%s append returned %d\n", st == KVQ_OK ? "ok" : "FAIL", st);
  fails += st != KVQ_OK;
  uint64_t ws = 0;
  st = kvq_workspace_bytes(&p, 0, &ws);
  void* work = ws ? dev_zero(ws) : NULL;
  st = st ? st : kvq_decode_attention(&p, &c, dq, dlens, NULL, NAN, 0, dout, work, ws, NULL);
  printf("%s decode returned %d\n", st == KVQ_OK ? "ok" : "FAIL", st);
  fails += st != KVQ_OK;
  HIP_OK(hipDeviceSynchronize());
  int32_t status = -99;
  HIP_OK(hipMemcpy(&status, c.status, sizeof status, hipMemcpyDeviceToHost));
  printf("%s device status %d\n", status == KVQ_OK ? "ok" : "FAIL", status);
  fails += status != KVQ_OK;
  /* packed rows: channel 16k + 4s + j in bits 2s..2s+1 of byte 4k + j; the code of a level is
   * its rank (the fit reproduces the four levels as its ascending centroids) */
  {
    static uint8_t codes[2][B * H * SCAP * 32];
    static uint16_t meta[2][B * H * SCAP * 8];
    HIP_OK(hipMemcpy(codes[0], c.codes[0], sizeof codes[0], hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(codes[1], c.codes[1], sizeof codes[1], hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(meta[0], c.meta[0], sizeof meta[0], hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(meta[1], c.meta[1], sizeof meta[1], hipMemcpyDeviceToHost));
    static const uint16_t kLevelBits[4] = {0xBE00u, 0xB800u, 0x3800u, 0x4000u};  /* fp16 */
    int badp = 0;
    for (int kv = 0; kv < 2; ++kv)
      for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
          for (int t = 0; t < NT; ++t) {
            const size_t row = ((size_t)b * H + h) * SCAP + t;
            const uint8_t* pk = codes[kv] + row * 32;
            for (int byte = 0; byte < 32; ++byte) {
              unsigned want = 0;
              for (int s = 0; s < 4; ++s) {
                const int ch = 16 * (byte / 4) + 4 * s + byte % 4;
                const int lvl = kv == 0 ? (ch + b + h) % 4 : (ch + b + 2 * h + 3 * t) % 4;
                want |= (unsigned)lvl << (2 * s);
              }
              if (pk[byte] != want) {
                if (badp < 5) printf("  kv=%d b=%d h=%d t=%d byte %d: 0x%02x want 0x%02x\n", kv, b,
                                     h, t, byte, pk[byte], want);
                ++badp;
              }
            }
            for (int i = 0; i < 8; ++i)
              if (meta[kv][row * 8 + i] != kLevelBits[i % 4]) ++badp;
          }
    printf("%s packed 2-bit rows and centroids follow the header's layout (%d mismatches)\n",
           badp ? "FAIL" : "ok", badp);
    fails += badp != 0;
  }
  static float out[B * HQ * D];
  HIP_OK(hipMemcpy(out, dout, sizeof out, hipMemcpyDeviceToHost));
  int bad = 0;
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < HQ; ++hq)
      for (int ch = 0; ch < D; ++ch) {
        const int h = hq / (HQ / H);
        const float v0 = v[(((size_t)b * H + h) * NT + 0) * D + ch];
        const float v1 = v[(((size_t)b * H + h) * NT + 1) * D + ch];
        const float want = 0.5f * (v0 + v1), got = out[((size_t)b * HQ + hq) * D + ch];
        const float tol = 1e-6f * (want < 0 ? -want : want) + 1e-6f;
        if (got - want > tol || want - got > tol) {
          if (bad < 5) printf("  b=%d hq=%d ch=%d got %.9g want %.9g\n", b, hq, ch, got, want);
          ++bad;
        }
      }
  printf("%s outputs equal the mean of the two V rows (%d mismatches)\n", bad ? "FAIL" : "ok", bad);
  fails += bad != 0;
  return fails ? 1 : 0;
}
