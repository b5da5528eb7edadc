/* Plain C client of include/kvq.h: the host-only entry points (byte counts, buffer sizes,
 * workspace size, status text and argument checks), built with gcc and linked against libkvq.so
 * with no C++ or Python in between.  Prints one line per check; exits non-zero on a mismatch. */
#include <stdio.h>
#include <string.h>

#include "kvq.h"

static int fails = 0;
#define CHECK(cond, what)                                              \
  do {                                                                 \
    if (cond) printf("ok %s\n", what);                                 \
    else { printf("FAIL %s\n", what); ++fails; }                       \
  } while (0)

int main(void) {
  /* 2-bit centroids, g = 64, E4M3 outliers: 32 code bytes + 2 x 8 centroid bytes per row */
  kvq_params p;
  memset(&p, 0, sizeof p);
  p.batch = 64; p.num_q_heads = 64; p.num_kv_heads = 8; p.head_dim = 128;
  p.max_seq_len = 32768; p.format = KVQ_FMT_CENTROID2; p.group_size = 64;
  p.outlier_dtype = KVQ_OUTL_FP8_E4M3; p.outlier_sigma = 3.0f; p.lloyd_iters = 8;

  uint64_t bytes = 0;
  CHECK(kvq_kv_bytes(&p, 1, 32768, 1000, &bytes) == KVQ_OK &&
        bytes == 2ull * 8 * 32768 * 48 + 1000ull * 5, "kv_bytes 2-bit + E4M3 records");

  kvq_params f = p;
  f.format = KVQ_FMT_FP16;
  CHECK(kvq_kv_bytes(&f, 80, 1, 0, &bytes) == KVQ_OK && bytes == 327680ull,
        "kv_bytes FP16: 2 x 80 layers x 8 heads x 128 x 2 bytes per token");

  kvq_cache_sizes_t s;
  CHECK(kvq_cache_sizes(&p, 4096, &s) == KVQ_OK && s.code_bytes_per_row == 32 &&
        s.meta_bytes_per_row == 16 && s.codes == 64ull * 8 * 32768 * 32,
        "cache_sizes 2-bit rows");

  kvq_params i3 = p;
  i3.format = KVQ_FMT_INT3_ASYM; i3.group_size = 32;
  CHECK(kvq_cache_sizes(&i3, 4096, &s) == KVQ_OK && s.code_bytes_per_row == 48 &&
        s.meta_bytes_per_row == 16, "cache_sizes INT3 rows");

  uint64_t ws = 1;
  CHECK(kvq_workspace_bytes(&p, 0, &ws) == KVQ_OK && ws == 256ull * (2 * 8 * (128 + 2) * 4 + 32),
        "workspace of 256 workgroups");
  CHECK(kvq_workspace_bytes(&p, 4096, &ws) == KVQ_OK &&
        ws == 4096ull * (2 * 8 * (128 + 2) * 4 + 32), "workspace of one workgroup per 4096 tokens");

  kvq_params bad = p;
  bad.head_dim = 96;
  CHECK(kvq_workspace_bytes(&bad, 0, &ws) == KVQ_ERR_UNSUPPORTED, "head_dim 96 unsupported");
  bad = p;
  bad.num_q_heads = 60;
  CHECK(kvq_workspace_bytes(&bad, 0, &ws) == KVQ_ERR_INVALID_ARG, "Hq not a multiple of H");
  CHECK(kvq_workspace_bytes(&p, 100, &ws) == KVQ_ERR_INVALID_ARG, "split not a multiple of 64");
  CHECK(kvq_decode_attention(&p, NULL, NULL, NULL, NULL, 0.1f, 0, NULL, NULL, 0, NULL) ==
        KVQ_ERR_INVALID_ARG, "decode with null cache rejected before any launch");
  CHECK(strcmp(kvq_status_string(KVQ_ERR_CAPACITY), "unknown status") != 0,
        "status text for capacity");

  /* hostile arguments: every call must return an error status without touching memory it was
   * not given (run under AddressSanitizer and UndefinedBehaviorSanitizer by the CPU suite) */
  {
    int hostile_ok = 1;
    kvq_cache c;
    memset(&c, 0, sizeof c);
    kvq_params h = p;
    hostile_ok &= kvq_kv_bytes(NULL, 1, 1, 0, &bytes) < 0;
    hostile_ok &= kvq_kv_bytes(&p, 1, 1, 0, NULL) < 0;
    hostile_ok &= kvq_kv_bytes(&p, -1, 1, 0, &bytes) < 0;
    hostile_ok &= kvq_cache_sizes(NULL, 1, &s) < 0 && kvq_cache_sizes(&p, 1, NULL) < 0;
    hostile_ok &= kvq_cache_sizes(&p, -5, &s) < 0;
    hostile_ok &= kvq_workspace_bytes(NULL, 0, &ws) < 0 && kvq_workspace_bytes(&p, 0, NULL) < 0;
    hostile_ok &= kvq_workspace_bytes(&p, -64, &ws) < 0;
    const int32_t formats[] = {-1, 0, 1, 5, 9, 99};
    for (unsigned i = 0; i < sizeof formats / sizeof formats[0]; ++i) {
      h = p;
      h.format = formats[i];
      hostile_ok &= kvq_workspace_bytes(&h, 0, &ws) < 0;
    }
    const int32_t groups[] = {-64, 0, 1, 16, 48, 128};
    for (unsigned i = 0; i < sizeof groups / sizeof groups[0]; ++i) {
      h = p;
      h.group_size = groups[i];
      hostile_ok &= kvq_workspace_bytes(&h, 0, &ws) < 0;
      /* the byte formula takes any group size that divides the head dimension */
      hostile_ok &= (kvq_kv_bytes(&h, 1, 1, 0, &bytes) < 0) == (groups[i] < 1 || 128 % groups[i] != 0);
    }
    h = p; h.num_kv_heads = 0; hostile_ok &= kvq_cache_sizes(&h, 1, &s) < 0;
    h = p; h.num_q_heads = 8 * 17; hostile_ok &= kvq_cache_sizes(&h, 1, &s) < 0;
    h = p; h.max_seq_len = 0x7FFFFFFF; hostile_ok &= kvq_cache_sizes(&h, 1, &s) < 0;
    h = p; h.outlier_sigma = -1.0f; hostile_ok &= kvq_cache_sizes(&h, 1, &s) < 0;
    h = p; h.outlier_dtype = 7; hostile_ok &= kvq_cache_sizes(&h, 1, &s) < 0;
    h = p; h.lloyd_iters = 1000; hostile_ok &= kvq_cache_sizes(&h, 1, &s) < 0;
    h = p; h.page_size = 16; h.max_pages_per_seq = 1; hostile_ok &= kvq_cache_sizes(&h, 1, &s) < 0;
    h = p; h.page_size = 8; hostile_ok &= kvq_cache_sizes(&h, 1, &s) < 0;
    float dummy[4];
    int32_t idummy[4];
    hostile_ok &= kvq_quantize_append(NULL, &c, dummy, dummy, 1, idummy, idummy, NULL, NULL) < 0;
    hostile_ok &= kvq_quantize_append(&p, NULL, dummy, dummy, 1, idummy, idummy, NULL, NULL) < 0;
    hostile_ok &= kvq_quantize_append(&p, &c, dummy, dummy, 1, idummy, idummy, NULL, NULL) < 0;
    hostile_ok &= kvq_decode_attention(&p, &c, dummy, idummy, NULL, 0.1f, 0, dummy, NULL, 0,
                                       NULL) < 0;
    {
      /* a workspace that is not 16-byte aligned is rejected before anything is launched (the
         buffers are host stand-ins that the rejected call never touches) */
      static uint64_t wsbuf[64];
      kvq_cache cf;
      memset(&cf, 0, sizeof cf);
      for (int kv = 0; kv < 2; ++kv) {
        cf.codes[kv] = dummy; cf.meta[kv] = dummy; cf.outl_idx[kv] = (uint32_t*)idummy;
        cf.outl_val[kv] = dummy;
      }
      cf.outl_count = idummy; cf.outl_block_start = idummy; cf.outl_capacity = 1;
      kvq_params pi = p;
      pi.batch = 1; pi.num_q_heads = 8; pi.num_kv_heads = 2; pi.max_seq_len = 1024;
      pi.format = KVQ_FMT_INT4_ASYM; pi.group_size = 32; pi.outlier_dtype = KVQ_OUTL_FP16;
      hostile_ok &= kvq_decode_attention(&pi, &cf, dummy, idummy, NULL, 0.1f, 0, dummy,
                                         (char*)wsbuf + 4, sizeof wsbuf - 4, NULL) == KVQ_ERR_WORKSPACE;
      hostile_ok &= kvq_decode_attention(&p, &cf, dummy, idummy, NULL, 0.1f, 0, dummy,
                                         (char*)wsbuf + 8, 1ull << 40, NULL) == KVQ_ERR_WORKSPACE;
    }
    hostile_ok &= kvq_probe_read(NULL, 16, dummy, NULL) < 0 && kvq_probe_read(dummy, 15, dummy, NULL) < 0;
    hostile_ok &= kvq_probe_copy(dummy, NULL, 16, NULL) < 0 && kvq_probe_copy(dummy, dummy, 0, NULL) < 0;
    hostile_ok &= strcmp(kvq_status_string(-12345), "unknown status") == 0;
    CHECK(hostile_ok, "hostile arguments rejected with an error status");
  }
  return fails ? 1 : 0;
}
