/* One S3R round driven from plain C through libs3r, with no Python or torch:
 * page bounds, page select, sparse draft attention (step 0), dense verify and
 * speculative sampling on inputs read from raw files in a directory. Device
 * memory comes from the HIP runtime's C API. Outputs are written back as raw
 * files next to the inputs; tests/test_gpu_c_round.py compares them with the
 * oracle.
 *
 * usage: round_gpu DIR B HQ HKV D P MAX_PAGES N_PHYS BUDGET GAMMA V KV_F32
 * inputs  (DIR/<name>.bin): k_pool, v_pool, page_table, seq_lens0, seq_lens_v,
 *                      q_draft, q_verify, draft_logits, target_logits, draft_tokens
 * outputs (DIR/<name>.bin): bounds, selected, num_selected, draft_out, verify_out,
 *                      out_tokens, num_accepted (attention outputs fp32)
 * Prints "ok" and returns 0, or names the failing call and returns 1. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "s3r.h"

static const char* g_dir;

static void* upload(const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s.bin", g_dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(1); }
  void* host = malloc(bytes ? bytes : 1);
  if (fread(host, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(1); }
  fclose(f);
  void* dev = NULL;
  if (hipMalloc(&dev, bytes ? bytes : 16) != hipSuccess ||
      hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "upload %s failed\n", name);
    exit(1);
  }
  free(host);
  return dev;
}

static void* device(size_t bytes) {
  void* dev = NULL;
  if (hipMalloc(&dev, bytes ? bytes : 16) != hipSuccess) { fprintf(stderr, "hipMalloc failed\n"); exit(1); }
  return dev;
}

static void download(const char* name, const void* dev, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s.bin", g_dir, name);
  void* host = malloc(bytes ? bytes : 1);
  if (hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    fprintf(stderr, "download %s failed\n", name);
    exit(1);
  }
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(host, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(1); }
  fclose(f);
  free(host);
}

#define CALL(x)                                                                   \
  do {                                                                            \
    s3r_status st_ = (x);                                                         \
    if (st_ != S3R_OK) {                                                          \
      fprintf(stderr, "%s failed: %s\n", #x, s3r_status_string(st_));             \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 13) { fprintf(stderr, "usage: see the header comment\n"); return 2; }
  g_dir = argv[1];
  const int B = atoi(argv[2]), Hq = atoi(argv[3]), Hkv = atoi(argv[4]), D = atoi(argv[5]);
  const int P = atoi(argv[6]), max_pages = atoi(argv[7]), n_phys = atoi(argv[8]);
  const int budget = atoi(argv[9]), gamma = atoi(argv[10]), V = atoi(argv[11]);
  const int f32 = atoi(argv[12]);
  const size_t esz = f32 ? 4 : 2, k = (size_t)budget / P;
  const size_t pool = (size_t)n_phys * Hkv * P * D * esz;
  const float scale = 1.0f / sqrtf((float)D);

  s3r_paged_kv kv = {0};
  kv.num_seqs = B;
  kv.num_q_heads = Hq;
  kv.num_kv_heads = Hkv;
  kv.head_dim = D;
  kv.page_size = P;
  kv.max_pages_per_seq = max_pages;
  kv.total_pages_hint = 0;
  kv.kv_dtype = f32 ? S3R_F32 : S3R_BF16;
  kv.k_pool = upload("k_pool", pool);
  kv.v_pool = upload("v_pool", pool);
  kv.page_table = (const int32_t*)upload("page_table", sizeof(int32_t) * B * max_pages);
  const int32_t* seq0 = (const int32_t*)upload("seq_lens0", sizeof(int32_t) * B);
  const int32_t* seqv = (const int32_t*)upload("seq_lens_v", sizeof(int32_t) * B);
  kv.num_phys_pages = n_phys;
  kv.seq_lens = seq0;
  const void* q_draft = upload("q_draft", (size_t)B * Hq * D * esz);
  const void* q_verify = upload("q_verify", (size_t)B * (gamma + 1) * Hq * D * esz);
  const float* dl = (const float*)upload("draft_logits", sizeof(float) * B * gamma * V);
  const float* tl = (const float*)upload("target_logits", sizeof(float) * B * (gamma + 1) * V);
  const int32_t* dt = (const int32_t*)upload("draft_tokens", sizeof(int32_t) * B * gamma);

  const size_t bounds_bytes = (size_t)n_phys * Hkv * 2 * D * esz;
  void* bounds = device(bounds_bytes);
  int32_t* sel = (int32_t*)device(sizeof(int32_t) * B * Hkv * k);
  int32_t* nsel = (int32_t*)device(sizeof(int32_t) * B);
  float* d_out = (float*)device(sizeof(float) * B * Hq * D);
  float* v_out = (float*)device(sizeof(float) * B * (gamma + 1) * Hq * D);
  int32_t* tok = (int32_t*)device(sizeof(int32_t) * B * (gamma + 1));
  int32_t* nacc = (int32_t*)device(sizeof(int32_t) * B);

  CALL(s3r_page_bounds_update(&kv, bounds, NULL, 0, NULL));
  const size_t ws_sel = s3r_page_select_workspace(&kv, budget);
  void* w1 = device(ws_sel);
  CALL(s3r_page_select(&kv, bounds, q_draft, budget, scale, sel, nsel, w1, ws_sel, NULL));
  const size_t ws_d = s3r_attn_workspace(&kv, 1, (int32_t)k);
  void* w2 = device(ws_d);
  CALL(s3r_sparse_draft_attn(&kv, q_draft, sel, (int32_t)k, scale, S3R_F32, d_out, w2, ws_d, NULL));
  kv.seq_lens = seqv;
  const size_t ws_v = s3r_attn_workspace(&kv, gamma + 1, max_pages);
  void* w3 = device(ws_v);
  CALL(s3r_dense_verify_attn(&kv, q_verify, gamma + 1, scale, S3R_F32, v_out, w3, ws_v, NULL));
  const size_t ws_s = s3r_spec_sample_workspace(B, gamma, V);
  void* w4 = device(ws_s);
  CALL(s3r_spec_sample(B, gamma, V, dl, tl, dt, 1.0f, 0, 7, tok, nacc, w4, ws_s, NULL));
  if (hipDeviceSynchronize() != hipSuccess) { fprintf(stderr, "device error\n"); return 1; }

  download("bounds", bounds, bounds_bytes);
  download("selected", sel, sizeof(int32_t) * B * Hkv * k);
  download("num_selected", nsel, sizeof(int32_t) * B);
  download("draft_out", d_out, sizeof(float) * B * Hq * D);
  download("verify_out", v_out, sizeof(float) * B * (gamma + 1) * Hq * D);
  download("out_tokens", tok, sizeof(int32_t) * B * (gamma + 1));
  download("num_accepted", nacc, sizeof(int32_t) * B);
  printf("ok\n");
  return 0;
}
