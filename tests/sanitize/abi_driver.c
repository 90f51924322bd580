/* Host-side exercise of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_host_sanitize.py builds the
 * library's host code with both and runs this program on the CPU).
 *
 * It makes no call that reaches the GPU: every size and plan query runs on a
 * grid of problem sizes (ragged, empty and long sequences, bf16 and float32,
 * the layer variants), and every entry point is called with invalid
 * arguments (expecting an error status and a message) and with valid
 * arguments but a workspace one byte short of the size it reports, which
 * runs the whole host-side plan and stops at the workspace check, before any
 * launch. Pointers stand in for device memory and are never dereferenced on
 * the host. Exit status 0 when every expectation holds; the sanitizers abort
 * on the first error they find. */
#include "dspark.h"

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static int failures = 0;
static int checks = 0;

#define EXPECT(cond, ...)                                                  \
  do {                                                                     \
    ++checks;                                                              \
    if (!(cond)) {                                                         \
      ++failures;                                                          \
      fprintf(stderr, "FAIL line %d: ", __LINE__);                         \
      fprintf(stderr, __VA_ARGS__);                                        \
      fprintf(stderr, " (last error: %s)\n", dspark_last_error());         \
    }                                                                      \
  } while (0)

/* a non-OK status with a message */
#define EXPECT_ERR(st, what)                                                          \
  do {                                                                                \
    const dspark_status s_ = (st);                                                    \
    EXPECT(s_ != DSPARK_OK && dspark_last_error() && dspark_last_error()[0] != '\0', \
           "%s: status %d", what, (int)s_);                                           \
  } while (0)

#define EXPECT_STATUS(st, want, what)                                         \
  do {                                                                        \
    const dspark_status s_ = (st);                                            \
    EXPECT(s_ == (want), "%s: status %d, expected %d", what, (int)s_, (int)(want)); \
  } while (0)

static char* arena; /* stand-in device memory: aligned, never read or written here */
#define P(off) ((void*)(arena + (off)))

static dspark_dims make_dims(int dtype, int m, int H, int d, int heads, int gamma, int layers, int ff) {
  dspark_dims x;
  memset(&x, 0, sizeof(x));
  x.m = m;
  x.H = H;
  x.d = d;
  x.n_heads = heads;
  x.gamma = gamma;
  x.n_layers = layers;
  x.ff = ff;
  x.eps = 1e-6f;
  x.dtype = dtype;
  return x;
}

static void make_layers(dspark_layer_weights* lw, int n) {
  for (int i = 0; i < n; ++i) {
    lw[i].attn_norm = (const float*)P(4096);
    lw[i].wq = P(8192);
    lw[i].wk = P(12288);
    lw[i].wv = P(16384);
    lw[i].wo = P(20480);
    lw[i].ff_norm = (const float*)P(24576);
    lw[i].w_gate = P(28672);
    lw[i].w_up = P(32768);
    lw[i].w_down = P(36864);
    lw[i].q_norm = (const float*)P(40960);
    lw[i].k_norm = (const float*)P(45056);
  }
}

/* cu prefix sums of the lengths */
static void prefix(const int* len, int A, int32_t* cu) {
  cu[0] = 0;
  for (int b = 0; b < A; ++b) cu[b + 1] = cu[b] + len[b];
}

static void exercise_forward(const dspark_dims* dm, int A, const int32_t* cu) {
  dspark_layer_weights lw[8];
  make_layers(lw, dm->n_layers);
  const void* taps[8];
  for (int j = 0; j < dm->m; ++j) taps[j] = P(65536 + 4096 * j);
  const int32_t* cu_dev = (const int32_t*)P(49152);

  /* every op's size and plan */
  for (int op = DSPARK_OP_CTX_FUSE; op <= DSPARK_OP_BLOCK_PROPOSE; ++op) {
    const size_t need = dspark_workspace_size(op, dm, A, cu);
    EXPECT(need > 0, "workspace_size op %d", op);
    int64_t info[DSPARK_PLAN_COUNT + 4];
    const int32_t n = dspark_plan_info(op, dm, A, cu, info, DSPARK_PLAN_COUNT + 4);
    EXPECT(n == DSPARK_PLAN_COUNT, "plan_info op %d returned %d", op, n);
    if (n == DSPARK_PLAN_COUNT) EXPECT((size_t)info[DSPARK_PLAN_WORKSPACE_BYTES] == need, "plan bytes op %d", op);
  }

  const size_t nf = dspark_workspace_size(DSPARK_OP_CTX_FUSE, dm, A, cu);
  const size_t nl = dspark_workspace_size(DSPARK_OP_BLOCK_LAYER, dm, A, cu);
  const size_t nw = dspark_workspace_size(DSPARK_OP_BLOCK_FORWARD, dm, A, cu);
  const int64_t T = cu[A];
  if (T > 0)
    EXPECT_STATUS(dspark_ctx_fuse(dm, A, cu, cu_dev, taps, dm->H, P(0), (const float*)P(256), P(512), P(1024),
                                  nf - 1, NULL),
                  DSPARK_EWORKSPACE, "ctx_fuse short workspace");
  EXPECT_STATUS(dspark_block_layer(dm, A, cu, cu_dev, P(512), (const float*)P(768), (float*)P(1024), lw, P(1280),
                                   nl - 1, NULL),
                DSPARK_EWORKSPACE, "block_layer short workspace");
  EXPECT_STATUS(dspark_block_forward(dm, A, cu, cu_dev, taps, dm->H, P(0), (const float*)P(256),
                                     (const float*)P(512), (const float*)P(768), lw, (const float*)P(1024), NULL,
                                     (float*)P(1280), P(1536), nw - 1, NULL),
                DSPARK_EWORKSPACE, "block_forward short workspace");

  /* invalid arguments */
  EXPECT_ERR(dspark_block_forward(NULL, A, cu, cu_dev, taps, dm->H, P(0), (const float*)P(256),
                                  (const float*)P(512), (const float*)P(768), lw, NULL, NULL, (float*)P(1280),
                                  P(1536), nw, NULL),
             "forward NULL dims");
  EXPECT_ERR(dspark_block_forward(dm, A, cu, cu_dev, taps, dm->H, NULL, (const float*)P(256),
                                  (const float*)P(512), (const float*)P(768), lw, NULL, NULL, (float*)P(1280),
                                  P(1536), nw, NULL),
             "forward NULL w_c");
  EXPECT_ERR(dspark_block_forward(dm, A, cu, cu_dev, taps, dm->H - 1, P(0), (const float*)P(256),
                                  (const float*)P(512), (const float*)P(768), lw, NULL, NULL, (float*)P(1280),
                                  P(1536), nw, NULL),
             "forward ld_tap < H");
  EXPECT_ERR(dspark_block_forward(dm, A, cu, cu_dev, taps, dm->H, P(2), (const float*)P(256),
                                  (const float*)P(512), (const float*)P(768), lw, NULL, NULL, (float*)P(1280),
                                  P(1536), nw, NULL),
             "forward misaligned w_c");
  EXPECT_ERR(dspark_block_layer(dm, A, cu, cu_dev, P(512), (const float*)P(768), (float*)P(1024), NULL, P(1280),
                                nl, NULL),
             "layer NULL weights");
  EXPECT_ERR(dspark_block_layer_noalloc(dm, A, cu, cu_dev, NULL, (const float*)P(768), (float*)P(1024), lw, NULL),
             "noalloc NULL h_ctx");
  if (A > 1) {
    int32_t bad[65];
    memcpy(bad, cu, sizeof(int32_t) * (A + 1));
    bad[1] = bad[2] + 1; /* not monotone */
    EXPECT(dspark_workspace_size(DSPARK_OP_BLOCK_FORWARD, dm, A, bad) == 0, "non-monotone cu accepted");
  }
  EXPECT(dspark_workspace_size(DSPARK_OP_BLOCK_FORWARD, dm, 0, cu) == 0, "A = 0 accepted");
  EXPECT(dspark_workspace_size(17, dm, A, cu) == 0, "unknown op accepted");
  EXPECT(dspark_workspace_size(DSPARK_OP_BLOCK_FORWARD, dm, A, NULL) == 0, "NULL cu accepted");
}

static void exercise_cache(const dspark_dims* dm, int A, const int* lens, int cap) {
  dspark_layer_weights lw[8];
  make_layers(lw, dm->n_layers);
  const void* taps[8];
  for (int j = 0; j < dm->m; ++j) taps[j] = P(65536 + 4096 * j);
  const size_t cb = dspark_cache_bytes(dm, A, cap);
  EXPECT(cb > 0, "cache_bytes");
  EXPECT(dspark_cache_bytes(dm, A, 0) == 0, "cache of 0 rows accepted");
  EXPECT_ERR(dspark_cache_reset(dm, A, cap, NULL, NULL), "cache_reset NULL cache");

  int32_t ncu[65], pos[64], cu[65];
  int news[64];
  for (int b = 0; b < A; ++b) {
    pos[b] = lens[b] / 2;
    news[b] = lens[b] - pos[b];
  }
  prefix(news, A, ncu);
  const size_t na = dspark_workspace_size(DSPARK_OP_CTX_APPEND, dm, A, ncu);
  EXPECT(na > 0, "append workspace");
  if (ncu[A] > 0)
    EXPECT_STATUS(dspark_ctx_append(dm, A, cap, ncu, (const int32_t*)P(49152), pos, (const int32_t*)P(49408), taps,
                                    dm->H, P(0), (const float*)P(256), lw, P(2048), P(4096), na - 1, NULL),
                  DSPARK_EWORKSPACE, "append short workspace");
  /* rows that do not fit the cache */
  int32_t over[64];
  for (int b = 0; b < A; ++b) over[b] = cap;
  if (ncu[A] > 0)
    EXPECT_ERR(dspark_ctx_append(dm, A, cap, ncu, (const int32_t*)P(49152), over, (const int32_t*)P(49408), taps,
                                 dm->H, P(0), (const float*)P(256), lw, P(2048), P(4096), na, NULL),
               "append past the cache");
  EXPECT_ERR(dspark_ctx_append(dm, A, cap, ncu, (const int32_t*)P(49152), NULL, (const int32_t*)P(49408), taps,
                               dm->H, P(0), (const float*)P(256), lw, P(2048), P(4096), na, NULL),
             "append NULL pos_host");

  prefix(lens, A, cu);
  const size_t np = dspark_workspace_size(DSPARK_OP_BLOCK_PROPOSE, dm, A, cu);
  EXPECT(np > 0, "propose workspace");
  EXPECT_STATUS(dspark_block_propose(dm, A, cap, cu, (const int32_t*)P(49152), P(2048), (const float*)P(512),
                                     (const float*)P(768), lw, (const float*)P(1024), (float*)P(1280), P(4096),
                                     np - 1, NULL),
                DSPARK_EWORKSPACE, "propose short workspace");
  EXPECT_ERR(dspark_block_propose(dm, A, cap, cu, (const int32_t*)P(49152), NULL, (const float*)P(512),
                                  (const float*)P(768), lw, (const float*)P(1024), (float*)P(1280), P(4096), np,
                                  NULL),
             "propose NULL cache");
}

static void exercise_padded(const dspark_dims* dm, int A, int L) {
  dspark_layer_weights lw[8];
  make_layers(lw, dm->n_layers);
  const void* taps[8];
  for (int j = 0; j < dm->m; ++j) taps[j] = P(65536 + 4096 * j);
  const size_t need = dspark_padded_workspace_size(dm, A, L);
  EXPECT(need > 0, "padded workspace");
  EXPECT_STATUS(dspark_block_forward_padded(dm, A, L, taps, dm->H, P(0), (const float*)P(256),
                                            (const uint8_t*)P(512), (const float*)P(768), (const float*)P(1024), lw,
                                            NULL, NULL, (float*)P(1280), P(1536), need - 1, NULL),
                DSPARK_EWORKSPACE, "padded short workspace");
  EXPECT_ERR(dspark_block_forward_padded(dm, A, L, taps, dm->H, P(0), (const float*)P(256), NULL,
                                         (const float*)P(768), (const float*)P(1024), lw, NULL, NULL,
                                         (float*)P(1280), P(1536), need, NULL),
             "padded NULL mask");
  EXPECT(dspark_padded_workspace_size(dm, A, 0) > 0, "padded batch without context rows");
  EXPECT(dspark_padded_workspace_size(dm, A, -1) == 0, "padded L = -1 accepted");
  EXPECT_ERR(dspark_block_build(dm, A, NULL, P(0), (const float*)P(256), (float*)P(512), NULL),
             "block_build NULL anchor");
}

static void exercise_markov(const dspark_dims* dm, int A, int vocab, int rank) {
  const size_t need = dspark_markov_workspace_size(dm, A, vocab, rank);
  EXPECT(need > 0, "markov workspace A %d vocab %d rank %d", A, vocab, rank);
  EXPECT_STATUS(dspark_markov_draft(dm, A, vocab, rank, (const float*)P(0), (const float*)P(256),
                                    (const int32_t*)P(512), P(768), P(1024), (const float*)P(1280),
                                    (const float*)P(1536), (int32_t*)P(1792), (float*)P(2048), (float*)P(2304),
                                    P(4096), need - 1, NULL),
                DSPARK_EWORKSPACE, "markov short workspace");
  EXPECT(dspark_markov_workspace_size(dm, A, vocab + 4, rank) == 0, "vocab not a multiple of 8 accepted");
  EXPECT(dspark_markov_workspace_size(dm, A, vocab, rank + 32) == 0, "rank not a multiple of 64 accepted");
  EXPECT(dspark_markov_workspace_size(dm, 0, vocab, rank) == 0, "markov A = 0 accepted");
  EXPECT_ERR(dspark_markov_draft(dm, A, vocab, rank, (const float*)P(0), (const float*)P(256), NULL, P(768),
                                 P(1024), (const float*)P(1280), (const float*)P(1536), (int32_t*)P(1792),
                                 (float*)P(2048), (float*)P(2304), P(4096), need, NULL),
             "markov NULL anchor");
}

int main(void) {
  arena = (char*)aligned_alloc(4096, 1 << 20);
  if (!arena) return 2;

  EXPECT(dspark_version() && dspark_version()[0], "version");
  const int32_t kinds = dspark_kernel_kinds();
  EXPECT(kinds > 0, "kernel kinds");
  for (int k = 0; k < kinds; ++k) EXPECT(dspark_kernel_name(k) && dspark_kernel_name(k)[0], "kernel name %d", k);
  EXPECT(dspark_kernel_name(kinds) && dspark_kernel_name(kinds)[0] == '\0', "kernel name past the end");
  EXPECT(dspark_kernel_name(-1) && dspark_kernel_name(-1)[0] == '\0', "kernel name -1");
  EXPECT_ERR(dspark_trace_end(NULL, NULL, 0), "trace_end NULL outputs");
  EXPECT_ERR(dspark_trace_begin(~0ull, 0), "trace_begin capacity 0");

  /* shapes: bf16 with head_dim 128, 64, 32; float32; grouped K/V heads with
   * q/k norms and rotary positions; the context length mixes of the tests */
  static const int ragged[] = {37, 0, 250, 1, 64, 65, 300, 129, 7, 0, 200, 33, 128, 5, 90, 311};
  static const int longs[] = {30011, 0, 11111};
  static const int big[] = {16384, 512, 9000, 2048, 16000, 700, 12000, 4096,
                            8000, 15000, 600, 3000, 10000, 5000, 14000, 1024};
  int32_t cu[65];
  struct {
    int dtype, m, H, d, heads, gamma, layers, ff, kv, variant;
    float theta;
  } shapes[] = {
      {DSPARK_BF16, 2, 64, 256, 2, 5, 2, 512, 0, 0, 0.f},
      {DSPARK_BF16, 4, 2560, 1024, 8, 5, 5, 2048, 0, 0, 0.f},
      {DSPARK_BF16, 1, 64, 256, 4, 16, 1, 512, 0, 0, 0.f},
      {DSPARK_BF16, 2, 128, 128, 4, 1, 1, 384, 0, 0, 0.f},
      {DSPARK_F32, 2, 128, 128, 4, 5, 2, 256, 0, 0, 0.f},
      {DSPARK_BF16, 2, 128, 512, 4, 8, 2, 1024, 2, DSPARK_QK_NORM | DSPARK_GELU_FFN, 10000.f},
      {DSPARK_BF16, 2, 128, 256, 2, 6, 1, 512, 0, DSPARK_PLAIN_CTX_KV, 0.f},
  };
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    dspark_dims dm = make_dims(shapes[s].dtype, shapes[s].m, shapes[s].H, shapes[s].d, shapes[s].heads,
                               shapes[s].gamma, shapes[s].layers, shapes[s].ff);
    dm.n_kv_heads = shapes[s].kv;
    dm.variant = shapes[s].variant;
    dm.rope_theta = shapes[s].theta;
    prefix(ragged, 16, cu);
    exercise_forward(&dm, 16, cu);
    prefix(longs, 3, cu);
    exercise_forward(&dm, 3, cu);
    prefix(big, 16, cu);
    exercise_forward(&dm, 16, cu);
    exercise_cache(&dm, 3, longs, 32768);
    exercise_cache(&dm, 16, ragged, 512);
    exercise_padded(&dm, 2, 1600);
    exercise_markov(&dm, 17, 5000, 256);
    exercise_markov(&dm, 1, 131072, 256);
    exercise_markov(&dm, 2, 1000, 576);

    /* invalid dims */
    dspark_dims bad = dm;
    bad.n_heads = 3; /* d % n_heads != 0 */
    EXPECT(dspark_workspace_size(DSPARK_OP_BLOCK_FORWARD, &bad, 16, cu) == 0, "d %% n_heads accepted");
    bad = dm;
    bad.gamma = 17;
    EXPECT(dspark_workspace_size(DSPARK_OP_BLOCK_FORWARD, &bad, 16, cu) == 0, "gamma 17 accepted");
    bad = dm;
    bad.gamma = 0;
    EXPECT(dspark_workspace_size(DSPARK_OP_BLOCK_LAYER, &bad, 16, cu) == 0, "gamma 0 accepted");
    bad = dm;
    bad.dtype = 7;
    EXPECT(dspark_workspace_size(DSPARK_OP_CTX_FUSE, &bad, 16, cu) == 0, "dtype 7 accepted");
  }

  free(arena);
  printf("%d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
