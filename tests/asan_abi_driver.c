/*
 * Host-side checks of libkvfuse under AddressSanitizer (no GPU needed).
 *
 * Built by rag_kv_cache_kvf_amd/csrc/build.py::build_asan against a copy of
 * the library whose host code is instrumented, and run by
 * tests/test_asan_abi.py.  Every call below is rejected by the host-side
 * validation before anything is enqueued, or is pure host bookkeeping
 * (workspace sizes, budgets, static-rule counts), so an out-of-bounds access
 * or use of freed memory in that code stops the run with an ASan report.
 * Host arrays are heap-allocated at their exact sizes so that reading one
 * element past the end is caught.
 *
 * With KVF_ASAN_LAUNCH=1 (set by the test only on a machine without a GPU)
 * it also makes one fully valid call, whose kernel launch must fail with
 * KVF_ERR_HIP naming the call; with KVF_SYNC_CHECK=1 that failure goes
 * through the synchronising check.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvfuse.h"

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);  \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

/* a pointer that is never dereferenced on the host (validation rejects the
 * call before any use) */
static void* const FAKE = (void*)(uintptr_t)0x1000;

static int32_t* ivec(int n, const int32_t* vals) {
  int32_t* p = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  for (int i = 0; i < n; ++i) p[i] = vals[i];
  return p;
}

/* a batch of n requests, each T rows of which N are context */
typedef struct {
  kvf_batch b;
  int32_t* cu;
  int32_t* nc;
} batch_t;

static batch_t make_batch(int n, int T, int N) {
  batch_t x;
  x.cu = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n + 1));
  x.nc = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  x.cu[0] = 0;
  for (int r = 0; r < n; ++r) {
    x.cu[r + 1] = x.cu[r] + T;
    x.nc[r] = N;
  }
  x.b.n_req = n;
  x.b.cu_T = x.cu;
  x.b.n_ctx = x.nc;
  return x;
}

static void free_batch(batch_t* x) {
  free(x->cu);
  free(x->nc);
}

static void check_strings(void) {
  CHECK(strcmp(kvf_status_string(KVF_OK), "KVF_OK") == 0);
  CHECK(strcmp(kvf_status_string(KVF_ERR_HIP), "KVF_ERR_HIP") == 0);
  CHECK(strcmp(kvf_status_string((kvf_status)99), "KVF_UNKNOWN_STATUS") == 0);
  CHECK(kvf_abi_version() == KVF_ABI_VERSION);
  CHECK(kvf_last_error() != NULL);
}

static void check_budgets(void) {
  CHECK(kvf_recompute_budget(5120, 30) == 1536);
  CHECK(kvf_recompute_budget(32768, 20) == 6553);
  CHECK(kvf_recompute_budget(2147483647, 100) == 2147483647);
  CHECK(kvf_recompute_budget(-1, 10) == -1);
  CHECK(kvf_recompute_budget(10, 101) == -1);
  CHECK(kvf_anchor_budget(512, 1, 10) == 52);
  CHECK(kvf_anchor_budget(2147483647, 1, 1) == 2147483647);
  CHECK(kvf_anchor_budget(5, 1, 0) == -1);
}

static void check_layer_validation(void) {
  kvf_layer_desc bad_dim = {4096, 32, 8, 96, KVF_BF16};
  kvf_layer_desc bad_group = {4096, 30, 8, 128, KVF_BF16};
  kvf_layer_desc bad_type = {4096, 32, 8, 128, 7};
  kvf_layer_desc ok = {4096, 32, 8, 128, KVF_BF16};
  batch_t b = make_batch(1, 5184, 5120);
  CHECK(kvf_score(KVF_SCORE_DEVIATION, NULL, &b.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  CHECK(kvf_score(KVF_SCORE_DEVIATION, &bad_dim, &b.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
        KVF_ERR_UNSUPPORTED);
  CHECK(kvf_score(KVF_SCORE_DEVIATION, &bad_group, &b.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0,
                  NULL) == KVF_ERR_UNSUPPORTED);
  CHECK(kvf_score(KVF_SCORE_DEVIATION, &bad_type, &b.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0,
                  NULL) == KVF_ERR_INVALID_ARG);
  CHECK(strlen(kvf_last_error()) > 0);
  /* unknown flags, missing tensors, workspace too small */
  CHECK(kvf_score((kvf_score_mode)0x200, &ok, &b.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  CHECK(kvf_score(KVF_SCORE_DEVIATION, &ok, &b.b, FAKE, NULL, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  size_t need = kvf_score_workspace_size(KVF_SCORE_ATTN_MASS, &ok, &b.b, 0);
  CHECK(need > 65536);
  CHECK(kvf_score(KVF_SCORE_ATTN_MASS, &ok, &b.b, FAKE, NULL, FAKE, 0, NULL, FAKE, FAKE, need - 1,
                  NULL) == KVF_ERR_WORKSPACE);
  CHECK(kvf_score_workspace_size(KVF_SCORE_DEVIATION, &ok, &b.b, 0) == 0);
  free_batch(&b);
  /* more 128-key context tiles than the counter region holds */
  batch_t huge = make_batch(1, 16384 * 128 + 200, 16384 * 128 + 1);
  CHECK(kvf_score(KVF_SCORE_ATTN_MASS, &ok, &huge.b, FAKE, NULL, FAKE, 0, NULL, FAKE, FAKE,
                  (size_t)1 << 40, NULL) == KVF_ERR_UNSUPPORTED);
  free_batch(&huge);
}

static void check_batch_validation(void) {
  kvf_layer_desc ok = {256, 4, 4, 64, KVF_F32};
  batch_t none = make_batch(0, 10, 5);
  CHECK(kvf_score(KVF_SCORE_DEVIATION, &ok, &none.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  free_batch(&none);
  batch_t many = make_batch(KVF_MAX_REQ + 1, 10, 5);
  CHECK(kvf_score(KVF_SCORE_DEVIATION, &ok, &many.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  free_batch(&many);
  batch_t b = make_batch(3, 10, 5);
  b.cu[2] = 5;                                   /* decreasing offsets */
  CHECK(kvf_score(KVF_SCORE_DEVIATION, &ok, &b.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  b.cu[2] = 20;
  b.nc[1] = 11;                                  /* more context than rows */
  CHECK(kvf_score(KVF_SCORE_DEVIATION, &ok, &b.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  b.nc[1] = 5;
  b.cu[0] = 1;
  CHECK(kvf_score(KVF_SCORE_DEVIATION, &ok, &b.b, FAKE, FAKE, NULL, 0, NULL, FAKE, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  free_batch(&b);
}

static void check_select(void) {
  batch_t b = make_batch(2, 100, 90);
  int32_t* k = ivec(2, (const int32_t[]){30, 91});
  CHECK(kvf_select_topk(FAKE, NULL, &b.b, k, FAKE, NULL, NULL, NULL, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  k[1] = 30;
  CHECK(kvf_select_topk(FAKE, NULL, &b.b, k, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  CHECK(kvf_select_topk(FAKE, NULL, &b.b, k, FAKE, FAKE, NULL, NULL, NULL, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  CHECK(kvf_select_workspace_size(&b.b) == 0);
  CHECK(kvf_select_topk_segmented(FAKE, NULL, &b.b, NULL, 3, k, FAKE, NULL, NULL, NULL) ==
        KVF_ERR_INVALID_ARG);
  CHECK(kvf_select_topk_segmented(FAKE, NULL, &b.b, FAKE, -1, k, FAKE, NULL, NULL, NULL) ==
        KVF_ERR_INVALID_ARG);
  kvf_static_rules neg = {-1, 0, 0};
  CHECK(kvf_select_static(&b.b, FAKE, 1, &neg, FAKE, NULL) == KVF_ERR_INVALID_ARG);
  free(k);
  free_batch(&b);
}

/* brute-force count of the static rules over one request's context */
static int32_t brute_static(int N, const int* starts, int n_starts, kvf_static_rules r) {
  char* m = (char*)calloc((size_t)(N > 0 ? N : 1), 1);
  for (int t = 0; t < r.sink && t < N; ++t) m[t] = 1;
  for (int i = 0; i < n_starts; ++i) {
    int p = starts[i];
    for (int t = p; t < p + r.boundary && t < N; ++t) m[t] = 1;
    if (p > 0)
      for (int t = p - r.seam < 0 ? 0 : p - r.seam; t < p; ++t) m[t] = 1;
  }
  int32_t c = 0;
  for (int t = 0; t < N; ++t) c += m[t];
  free(m);
  return c;
}

static void check_static_counts(void) {
  unsigned seed = 7;
  for (int trial = 0; trial < 200; ++trial) {
    int n_req = 1 + (int)((seed = seed * 1103515245u + 12345u) >> 16) % 4;
    int* N = (int*)malloc(sizeof(int) * (size_t)n_req);
    batch_t b = make_batch(n_req, 0, 0);
    for (int r = 0; r < n_req; ++r) {
      N[r] = (int)((seed = seed * 1103515245u + 12345u) >> 16) % 300;
      b.cu[r + 1] = b.cu[r] + N[r] + 7;
      b.nc[r] = N[r];
    }
    int per = 5;
    int n_chunks = n_req * per;
    kvf_chunk* ch = (kvf_chunk*)calloc((size_t)n_chunks, sizeof(kvf_chunk));
    int* starts = (int*)malloc(sizeof(int) * (size_t)n_chunks);
    for (int r = 0; r < n_req; ++r)
      for (int i = 0; i < per; ++i) {
        int p = N[r] ? (i == 0 ? 0 : (int)((seed = seed * 1103515245u + 12345u) >> 16) % N[r]) : 0;
        starts[r * per + i] = p;
        ch[r * per + i].dst_row = b.cu[r] + p;
        ch[r * per + i].len = 1;
      }
    kvf_static_rules rules = {(int)(seed >> 20) % 9, (int)(seed >> 24) % 5, 16};
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_req);
    CHECK(kvf_static_counts(&b.b, ch, n_chunks, &rules, counts) == KVF_OK);
    for (int r = 0; r < n_req; ++r) {
      int n_st = 0;
      int* st = (int*)malloc(sizeof(int) * (size_t)per);
      for (int i = 0; i < per; ++i)
        if (N[r] && starts[r * per + i] < N[r]) st[n_st++] = starts[r * per + i];
      CHECK(counts[r] == (N[r] ? brute_static(N[r], st, n_st, rules) : 0));
      free(st);
    }
    free(counts);
    free(starts);
    free(ch);
    free(N);
    free_batch(&b);
  }
}

static void check_projection_and_attention(void) {
  kvf_layer_desc ok = {4096, 32, 8, 128, KVF_BF16};
  kvf_layer_desc f32 = {4096, 32, 8, 128, KVF_F32};
  /* projection */
  CHECK(kvf_recompute_qkv(&ok, FAKE, 10, NULL, FAKE, 11, FAKE, 7, FAKE, FAKE, 10, FAKE, FAKE, FAKE,
                          NULL, 0, NULL, 0, NULL) == KVF_ERR_INVALID_ARG);   /* M > x_rows */
  CHECK(kvf_recompute_qkv(&ok, FAKE, 10, NULL, FAKE, 4, FAKE, 8, FAKE, FAKE, 10, FAKE, FAKE, FAKE,
                          NULL, 0, NULL, 0, NULL) == KVF_ERR_INVALID_ARG);   /* unknown bit */
  size_t wr = kvf_recompute_workspace_size(&ok, 64, 7);
  CHECK(wr >= 4096);
  CHECK(kvf_recompute_qkv(&ok, FAKE, 100, FAKE, FAKE, 64, FAKE, 7, FAKE, FAKE, 100, FAKE, FAKE, FAKE,
                          NULL, 0, FAKE, wr - 1, NULL) == KVF_ERR_WORKSPACE);
  /* scatter */
  CHECK(kvf_scatter_kv(&ok, FAKE, NULL, 4, NULL, NULL, 0, FAKE, 5, FAKE, FAKE, 10, NULL) ==
        KVF_ERR_INVALID_ARG);
  CHECK(kvf_scatter_kv(&ok, FAKE, FAKE, 4, NULL, NULL, 0, NULL, 5, FAKE, FAKE, 10, NULL) ==
        KVF_ERR_INVALID_ARG);
  /* attention: workspace sizes for several shapes; too small; bad cu_q */
  batch_t b = make_batch(1, 5184, 5120);
  int32_t* cq = ivec(2, (const int32_t[]){0, 1600});
  size_t need = kvf_attention_workspace_size(&ok, &b.b, cq);
  CHECK(need == 4096 + (size_t)50 * 8 * 2 * 17 * 256 * 16);
  CHECK(kvf_attention_workspace_size(&f32, &b.b, cq) == 0);
  CHECK(kvf_sparse_q_attention(&ok, &b.b, FAKE, FAKE, cq, FAKE, FAKE, 0.088f, FAKE, NULL, FAKE,
                               need - 1, NULL) == KVF_ERR_WORKSPACE);
  CHECK(kvf_sparse_q_attention(&ok, &b.b, FAKE, FAKE, cq, FAKE, FAKE, -1.f, FAKE, NULL, NULL, 0,
                               NULL) == KVF_ERR_INVALID_ARG);
  cq[0] = 1;
  CHECK(kvf_attention_workspace_size(&ok, &b.b, cq) == 0);
  free(cq);
  free_batch(&b);
  batch_t b8 = make_batch(8, 10368, 10240);
  int32_t* cq8 = (int32_t*)malloc(sizeof(int32_t) * 9);
  for (int r = 0; r <= 8; ++r) cq8[r] = r * 3200;
  CHECK(kvf_attention_workspace_size(&ok, &b8.b, cq8) == 0);   /* large grid: no key split */
  free(cq8);
  free_batch(&b8);
  /* re-positioning */
  kvf_chunk* ch = (kvf_chunk*)calloc(1, sizeof(kvf_chunk));
  CHECK(kvf_rerotate(&ok, ch, 1, 4, FAKE, FAKE, NULL, 4, FAKE, FAKE, 4, FAKE, FAKE, 4, 2, NULL) ==
        KVF_ERR_INVALID_ARG);
  CHECK(kvf_rerotate(&ok, ch, 1, 4, NULL, NULL, NULL, 4, FAKE, FAKE, 4, FAKE, NULL, 4, 1, NULL) ==
        KVF_ERR_INVALID_ARG);
  CHECK(kvf_rerotate(&ok, ch, -1, 4, FAKE, FAKE, NULL, 4, FAKE, FAKE, 4, FAKE, FAKE, 4, 0, NULL) ==
        KVF_ERR_INVALID_ARG);
  free(ch);
  CHECK(kvf_rope_table(1.0, 64, 4, FAKE, FAKE, NULL) == KVF_ERR_INVALID_ARG);
  CHECK(kvf_rope_table(1e4, 63, 4, FAKE, FAKE, NULL) == KVF_ERR_INVALID_ARG);
}

/* the re-positioning passes that also score: their batch checks read the
 * host arrays (exact sizes here), then their own and kvf_rerotate's checks */
static void check_fused_passes(void) {
  const kvf_layer_desc bf = {2048, 16, 2, 128, KVF_BF16};
  const kvf_layer_desc wide = {4096, 32, 16, 128, KVF_BF16};   /* 128 units per row */
  batch_t b = make_batch(3, 100, 90);
  kvf_chunk* ch = (kvf_chunk*)calloc(1, sizeof(kvf_chunk));
  kvf_q8_cache q8 = {(uint8_t*)FAKE, (uint8_t*)FAKE, (float*)FAKE, (float*)FAKE, 300};
  /* deviation, bf16 cache */
  CHECK(kvf_rerotate_deviation(&bf, &b.b, ch, 1, 4, FAKE, FAKE, NULL, 4, FAKE, FAKE, 4, FAKE, FAKE,
                               300, 0, FAKE, NULL, 2, FAKE, NULL) == KVF_ERR_INVALID_ARG);
  CHECK(kvf_rerotate_deviation(&wide, &b.b, ch, 1, 4, FAKE, FAKE, NULL, 4, FAKE, FAKE, 4, FAKE, FAKE,
                               300, 0, FAKE, NULL, 0, FAKE, NULL) == KVF_ERR_UNSUPPORTED);
  CHECK(kvf_rerotate_deviation(&bf, &b.b, ch, 1, 4, FAKE, FAKE, NULL, 4, FAKE, FAKE, 4, FAKE, FAKE,
                               300, 0, NULL, NULL, 0, FAKE, NULL) == KVF_ERR_INVALID_ARG);
  CHECK(kvf_rerotate_deviation(&bf, &b.b, ch, 1, 4, FAKE, FAKE, NULL, 4, FAKE, FAKE, 4, FAKE, NULL,
                               300, 0, FAKE, NULL, 0, FAKE, NULL) == KVF_ERR_INVALID_ARG);
  /* deviation, int8-resident cache */
  CHECK(kvf_rerotate_q8_deviation(&bf, &b.b, ch, 1, 4, FAKE, FAKE, NULL, 4, FAKE, FAKE, 4, &q8, FAKE,
                                  NULL, 3, FAKE, NULL) == KVF_ERR_INVALID_ARG);
  CHECK(kvf_rerotate_q8_deviation(&wide, &b.b, ch, 1, 4, FAKE, FAKE, NULL, 4, FAKE, FAKE, 4, &q8, FAKE,
                                  NULL, 0, FAKE, NULL) == KVF_ERR_UNSUPPORTED);
  CHECK(kvf_rerotate_q8_deviation(&bf, &b.b, ch, 1, 4, FAKE, FAKE, NULL, 4, FAKE, FAKE, 4, NULL, FAKE,
                                  NULL, 0, FAKE, NULL) == KVF_ERR_INVALID_ARG);
  /* attention mass with keys-only re-positioning */
  CHECK(kvf_rerotate_score_attn_mass(&bf, &b.b, ch, 1, 4, FAKE, 100, FAKE, FAKE, 4, FAKE, 299, FAKE, 0,
                                     NULL, 0, FAKE, FAKE, 1 << 30, NULL) == KVF_ERR_INVALID_ARG);
  CHECK(kvf_rerotate_score_attn_mass(&bf, &b.b, ch, 1, 4, NULL, 100, FAKE, FAKE, 4, FAKE, 300, FAKE, 0,
                                     NULL, 0, FAKE, FAKE, 1 << 30, NULL) == KVF_ERR_INVALID_ARG);
  CHECK(kvf_rerotate_score_attn_mass(&bf, &b.b, ch, 1, 4, FAKE, 100, FAKE, FAKE, 4, FAKE, 300, FAKE, 0,
                                     NULL, 5, FAKE, FAKE, 1 << 30, NULL) == KVF_ERR_INVALID_ARG);
  CHECK(kvf_rerotate_score_attn_mass(&bf, &b.b, ch, 1, 4, FAKE, 100, FAKE, FAKE, 4, FAKE, 300, FAKE, 0,
                                     NULL, 0, FAKE, FAKE, 0, NULL) == KVF_ERR_WORKSPACE);
  free(ch);
  free_batch(&b);
}

static void check_launch_failure(void) {
  /* a valid call on a machine without a GPU: the launch fails and the call
   * reports it as its own KVF_ERR_HIP */
  kvf_status st = kvf_rope_table(1e4, 64, 4, FAKE, FAKE, NULL);
  CHECK(st == KVF_ERR_HIP);
  CHECK(strstr(kvf_last_error(), "kvf_rope_table") != NULL);
  fprintf(stderr, "launch without a GPU: %s (%s)\n", kvf_status_string(st), kvf_last_error());
}

int main(void) {
  check_strings();
  check_budgets();
  check_layer_validation();
  check_batch_validation();
  check_select();
  check_static_counts();
  check_projection_and_attention();
  check_fused_passes();
  const char* launch = getenv("KVF_ASAN_LAUNCH");
  if (launch && strcmp(launch, "1") == 0) check_launch_failure();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("asan abi driver: all checks passed\n");
  return 0;
}
