/*
 * Host-side check of libtsa.so's validation, run against a build of the
 * library's host code with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_host_sanitized.py builds and runs it; no GPU is used).
 *
 * Every call below either fails validation, which include/tsa.h says happens
 * before anything is enqueued, or passes it with TSA_FAULT_INJECT=launch set,
 * which makes the library return TSA_ERR_HIP where it would launch.  So no
 * call reaches the HIP runtime: the pointers are host addresses that are
 * never dereferenced.
 */
#define _POSIX_C_SOURCE 200809L /* setenv */

#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tsa.h"

static int g_checks = 0, g_failures = 0;

#define CHECK(cond, ...)                                        \
  do {                                                          \
    ++g_checks;                                                 \
    if (!(cond)) {                                              \
      ++g_failures;                                             \
      fprintf(stderr, "FAIL line %d: ", __LINE__);              \
      fprintf(stderr, __VA_ARGS__);                             \
      fprintf(stderr, " [last error: %s]\n", tsa_last_error()); \
    }                                                           \
  } while (0)

/* Stand-in tensor and workspace addresses: 256-byte aligned, never read. */
static unsigned char* g_buf;
#define P(i) ((void*)(g_buf + 256 * (i)))
#define MIS ((void*)(g_buf + 8)) /* 8-byte aligned only */

static tsa_problem good(void) {
  tsa_problem p = {1, 8, 2, 4096, 128, 64, 0.05f, TSA_BF16, 0};
  return p;
}

/* Every entry point that takes a problem, called with stand-in arguments
 * that are valid except, possibly, the problem itself.  Returns nonzero (and
 * names the entry points) if any status differs from `want`. */
static int all_entry_points(const tsa_problem* p, tsa_status want, const char* what) {
  const size_t big = (size_t)1 << 60; /* any workspace size check passes */
  int32_t* i32 = (int32_t*)P(5);
  float* f32 = (float*)P(6);
  tsa_status st[14];
  const char* names[14] = {"tsa_score", "tsa_budget", "tsa_select", "tsa_gather", "tsa_gather_kv",
                           "tsa_attention", "tsa_attention_block_sparse", "tsa_scatter",
                           "tsa_forward", "tsa_attention_indexed", "tsa_attention_qo_indexed",
                           "tsa_zero_unselected", "tsa_forward_fused",
                           "tsa_forward_fused_noalloc"};
  const int group = (p && p->Hkv > 0 && p->Hq % (p->Hkv ? p->Hkv : 1) == 0) ? p->Hq / p->Hkv : 1;
  st[0] = tsa_score(p, P(1), P(2), f32, P(8), big, NULL);
  st[1] = tsa_budget(p, f32, i32, P(8), big, NULL);
  st[2] = tsa_select(p, f32, i32, i32, i32, P(8), big, NULL);
  st[3] = tsa_gather(p, P(1), P(2), P(3), i32, i32, P(4), P(4), P(4), NULL);
  st[4] = tsa_gather_kv(p, P(2), P(3), i32, P(4), P(4), NULL);
  st[5] = tsa_attention(p, P(1), P(2), P(3), i32, group > 0 ? group : 1, P(4), NULL);
  st[6] = tsa_attention_block_sparse(p, P(1), P(2), P(3), i32, 1, (const uint32_t*)P(7), P(4),
                                     NULL);
  st[7] = tsa_scatter(p, P(4), i32, P(1), NULL);
  st[8] = tsa_forward(p, P(1), P(2), P(3), P(4), i32, i32, P(8), big, NULL);
  st[9] = tsa_attention_indexed(p, P(1), P(2), P(3), i32, i32, P(4), NULL);
  st[10] = tsa_attention_qo_indexed(p, P(1), P(2), P(3), i32, i32, P(4), NULL);
  st[11] = tsa_zero_unselected(p, i32, P(4), NULL);
  st[12] = tsa_forward_fused(p, P(1), P(2), P(3), P(4), i32, i32, P(8), big, NULL);
  st[13] = tsa_forward_fused_noalloc(p, P(1), P(2), P(3), P(4), i32, i32, NULL);
  int bad = 0;
  for (int i = 0; i < 14; ++i) {
    /* the no-allocation entry point refuses problems beyond its scratch first */
    if (i == 13 && want == TSA_ERR_HIP && st[i] == TSA_ERR_UNSUPPORTED) continue;
    if (st[i] != want) {
      fprintf(stderr, "  %s: %s returned %s, expected %s\n", what, names[i],
              tsa_status_string(st[i]), tsa_status_string(want));
      bad = 1;
    }
  }
  return bad;
}

static void check_bad_problems(void) {
  struct {
    const char* what;
    tsa_problem p;
    tsa_status want;
  } cases[64];
  int n = 0;
#define ADD(desc, field, value, status)  \
  do {                                   \
    cases[n].what = desc;                \
    cases[n].p = good();                 \
    cases[n].p.field = value;            \
    cases[n].want = status;              \
    ++n;                                 \
  } while (0)
  ADD("B=0", B, 0, TSA_ERR_INVALID_ARG);
  ADD("B<0", B, -1, TSA_ERR_INVALID_ARG);
  ADD("Hq=0", Hq, 0, TSA_ERR_INVALID_ARG);
  ADD("Hkv=0", Hkv, 0, TSA_ERR_INVALID_ARG);
  ADD("Hkv<0", Hkv, -2, TSA_ERR_INVALID_ARG);
  ADD("L=0", L, 0, TSA_ERR_INVALID_ARG);
  ADD("d=0", d, 0, TSA_ERR_INVALID_ARG);
  ADD("w=0", w, 0, TSA_ERR_INVALID_ARG);
  ADD("Hq%Hkv", Hkv, 3, TSA_ERR_INVALID_ARG);
  ADD("w>L", w, 4097, TSA_ERR_INVALID_ARG);
  ADD("L>2^22", L, (1 << 22) + 1, TSA_ERR_INVALID_ARG);
  ADD("L=INT32_MAX", L, INT32_MAX, TSA_ERR_INVALID_ARG);
  ADD("tau NaN", tau, NAN, TSA_ERR_INVALID_ARG);
  ADD("tau<0", tau, -0.01f, TSA_ERR_INVALID_ARG);
  ADD("tau=1", tau, 1.0f, TSA_ERR_INVALID_ARG);
  ADD("tau=inf", tau, INFINITY, TSA_ERR_INVALID_ARG);
  ADD("flags", flags, 8, TSA_ERR_UNSUPPORTED);
  ADD("flags<0", flags, -1, TSA_ERR_UNSUPPORTED);
  ADD("dtype", dtype, 2, TSA_ERR_UNSUPPORTED);
  ADD("dtype<0", dtype, -1, TSA_ERR_UNSUPPORTED);
  ADD("d=96", d, 96, TSA_ERR_UNSUPPORTED);
  ADD("d=256", d, 256, TSA_ERR_UNSUPPORTED);
  ADD("B*Hq>65535", B, 8192, TSA_ERR_UNSUPPORTED);
  ADD("B=INT32_MAX", B, INT32_MAX, TSA_ERR_UNSUPPORTED);
#undef ADD
  cases[n].what = "Hq>4096";
  cases[n].p = good();
  cases[n].p.Hq = 4097;
  cases[n].p.Hkv = 4097;
  cases[n].want = TSA_ERR_INVALID_ARG;
  ++n;
  cases[n].what = "Hq=INT32_MAX";
  cases[n].p = good();
  cases[n].p.Hq = INT32_MAX;
  cases[n].p.Hkv = INT32_MAX;
  cases[n].want = TSA_ERR_INVALID_ARG;
  ++n;
  cases[n].what = "bf16 w>2944";
  cases[n].p = good();
  cases[n].p.w = 2945;
  cases[n].want = TSA_ERR_UNSUPPORTED;
  ++n;

  for (int i = 0; i < n; ++i) {
    const tsa_problem* p = &cases[i].p;
    CHECK(!all_entry_points(p, cases[i].want, cases[i].what), "%s: every entry point returns %s",
          cases[i].what, tsa_status_string(cases[i].want));
    CHECK(strlen(tsa_last_error()) > 0, "%s: the error text is set", cases[i].what);
    CHECK(tsa_workspace_bytes(p) == 0 && tsa_forward_workspace_bytes(p) == 0 &&
              tsa_fused_workspace_bytes(p) == 0 && tsa_block_mask_words(p) == 0,
          "%s: size queries return 0", cases[i].what);
  }
  /* f32 has no proxy-tile limit */
  tsa_problem f = good();
  f.dtype = TSA_F32;
  f.w = 2945;
  CHECK(tsa_workspace_bytes(&f) > 0, "f32 w=2945 is accepted");
  /* a null problem */
  CHECK(!all_entry_points(NULL, TSA_ERR_INVALID_ARG, "NULL problem"),
        "NULL problem: every entry point returns TSA_ERR_INVALID_ARG");
  CHECK(tsa_workspace_bytes(NULL) == 0 && tsa_forward_workspace_bytes(NULL) == 0 &&
            tsa_fused_workspace_bytes(NULL) == 0 && tsa_block_mask_words(NULL) == 0,
        "NULL problem: size queries return 0");
}

/* Null and misaligned tensor pointers, one argument at a time. */
static void check_pointers(void) {
  const tsa_problem pr = good();
  const tsa_problem* p = &pr;
  const size_t ws = tsa_forward_workspace_bytes(p);
  int32_t* i32 = (int32_t*)P(5);
  float* f32 = (float*)P(6);
  void* bad[2] = {NULL, MIS};
  for (int b = 0; b < 2; ++b) {
    void* x = bad[b];
    const char* kind = b ? "misaligned" : "NULL";
    CHECK(tsa_score(p, x, P(2), f32, P(8), ws, NULL) == TSA_ERR_INVALID_ARG, "score q %s", kind);
    CHECK(tsa_score(p, P(1), x, f32, P(8), ws, NULL) == TSA_ERR_INVALID_ARG, "score k %s", kind);
    CHECK(tsa_score(p, P(1), P(2), (float*)x, P(8), ws, NULL) == TSA_ERR_INVALID_ARG,
          "score s %s", kind);
    CHECK(tsa_budget(p, (float*)x, i32, P(8), ws, NULL) == TSA_ERR_INVALID_ARG, "budget s %s",
          kind);
    CHECK(tsa_budget(p, f32, (int32_t*)x, P(8), ws, NULL) == TSA_ERR_INVALID_ARG,
          "budget budget %s", kind);
    CHECK(tsa_select(p, f32, i32, (int32_t*)x, i32, P(8), ws, NULL) == TSA_ERR_INVALID_ARG,
          "select idx %s", kind);
    CHECK(tsa_select(p, f32, i32, i32, (int32_t*)x, P(8), ws, NULL) == TSA_ERR_INVALID_ARG,
          "select rank %s", kind);
    CHECK(tsa_gather(p, P(1), P(2), P(3), (int32_t*)x, i32, P(4), P(4), P(4), NULL) ==
              TSA_ERR_INVALID_ARG,
          "gather idx %s", kind);
    CHECK(tsa_gather(p, P(1), P(2), P(3), i32, i32, P(4), x, P(4), NULL) == TSA_ERR_INVALID_ARG,
          "gather kc %s", kind);
    CHECK(tsa_gather_kv(p, P(2), P(3), i32, P(4), x, NULL) == TSA_ERR_INVALID_ARG,
          "gather_kv vc %s", kind);
    CHECK(tsa_attention(p, P(1), P(2), P(3), i32, 4, x, NULL) == TSA_ERR_INVALID_ARG,
          "attention o %s", kind);
    CHECK(tsa_attention_block_sparse(p, P(1), P(2), P(3), i32, 1, (const uint32_t*)x, P(4),
                                     NULL) == TSA_ERR_INVALID_ARG,
          "block_sparse mask %s", kind);
    CHECK(tsa_scatter(p, x, i32, P(1), NULL) == TSA_ERR_INVALID_ARG, "scatter oc %s", kind);
    CHECK(tsa_forward(p, P(1), P(2), P(3), x, i32, i32, P(8), ws, NULL) == TSA_ERR_INVALID_ARG,
          "forward o %s", kind);
    CHECK(tsa_forward(p, P(1), P(2), P(3), P(4), i32, (int32_t*)x, P(8), ws, NULL) ==
              TSA_ERR_INVALID_ARG,
          "forward idx %s", kind);
    CHECK(tsa_attention_indexed(p, P(1), P(2), P(3), (int32_t*)x, i32, P(4), NULL) ==
              TSA_ERR_INVALID_ARG,
          "attention_indexed idx %s", kind);
    CHECK(tsa_attention_qo_indexed(p, P(1), x, P(3), i32, i32, P(4), NULL) ==
              TSA_ERR_INVALID_ARG,
          "attention_qo_indexed kc %s", kind);
    CHECK(tsa_zero_unselected(p, (int32_t*)x, P(4), NULL) == TSA_ERR_INVALID_ARG,
          "zero_unselected rank %s", kind);
    CHECK(tsa_forward_fused(p, x, P(2), P(3), P(4), i32, i32, P(8), ws, NULL) ==
              TSA_ERR_INVALID_ARG,
          "forward_fused q %s", kind);
    CHECK(tsa_forward_fused_noalloc(p, P(1), P(2), P(3), P(4), (int32_t*)x, i32, NULL) ==
              TSA_ERR_INVALID_ARG,
          "forward_fused_noalloc budget %s", kind);
  }
  /* optional pointers: qc of tsa_gather and budget of tsa_attention */
  CHECK(tsa_gather(p, P(1), P(2), P(3), i32, i32, NULL, P(4), P(4), NULL) == TSA_ERR_HIP,
        "gather accepts qc = NULL");
  CHECK(tsa_attention(p, P(1), P(2), P(3), NULL, 4, P(4), NULL) == TSA_ERR_HIP,
        "attention accepts budget = NULL");
  CHECK(tsa_attention(p, P(1), P(2), P(3), (int32_t*)MIS, 4, P(4), NULL) == TSA_ERR_INVALID_ARG,
        "attention rejects a misaligned budget");
  /* kv_group */
  const int32_t groups[4] = {0, -1, 3, 16};
  for (int i = 0; i < 4; ++i) {
    CHECK(tsa_attention(p, P(1), P(2), P(3), i32, groups[i], P(4), NULL) == TSA_ERR_INVALID_ARG,
          "attention kv_group=%d", groups[i]);
    CHECK(tsa_attention_block_sparse(p, P(1), P(2), P(3), i32, groups[i], (const uint32_t*)P(7),
                                     P(4), NULL) == TSA_ERR_INVALID_ARG,
          "block_sparse kv_group=%d", groups[i]);
  }
  CHECK(tsa_attention(p, P(1), P(2), P(3), i32, 8, P(4), NULL) == TSA_ERR_HIP,
        "attention kv_group=8 passes validation");
}

/* Workspace checks: one byte short, NULL and misaligned. */
static void check_workspaces(void) {
  const tsa_problem pr = good();
  const tsa_problem* p = &pr;
  int32_t* i32 = (int32_t*)P(5);
  float* f32 = (float*)P(6);
  const size_t step = tsa_workspace_bytes(p), fwd = tsa_forward_workspace_bytes(p),
               fused = tsa_fused_workspace_bytes(p);
  CHECK(step > 0 && fused > step && fwd > fused, "step < fused < forward workspace");
  CHECK(tsa_score(p, P(1), P(2), f32, P(8), step - 1, NULL) == TSA_ERR_WORKSPACE, "score short");
  CHECK(tsa_budget(p, f32, i32, P(8), step - 1, NULL) == TSA_ERR_WORKSPACE, "budget short");
  CHECK(tsa_select(p, f32, i32, i32, i32, P(8), step - 1, NULL) == TSA_ERR_WORKSPACE,
        "select short");
  CHECK(tsa_forward(p, P(1), P(2), P(3), P(4), i32, i32, P(8), fwd - 1, NULL) ==
            TSA_ERR_WORKSPACE,
        "forward short");
  CHECK(tsa_forward_fused(p, P(1), P(2), P(3), P(4), i32, i32, P(8), fused - 1, NULL) ==
            TSA_ERR_WORKSPACE,
        "forward_fused short");
  CHECK(tsa_forward(p, P(1), P(2), P(3), P(4), i32, i32, NULL, fwd, NULL) == TSA_ERR_WORKSPACE,
        "forward NULL workspace");
  CHECK(tsa_forward(p, P(1), P(2), P(3), P(4), i32, i32, (void*)(g_buf + 16), fwd, NULL) ==
            TSA_ERR_WORKSPACE,
        "forward workspace not 256-byte aligned");
  CHECK(tsa_score(p, P(1), P(2), f32, P(8), step, NULL) == TSA_ERR_HIP, "score exact workspace");
  CHECK(tsa_forward(p, P(1), P(2), P(3), P(4), i32, i32, P(8), fwd, NULL) == TSA_ERR_HIP,
        "forward exact workspace");
}

/* Size queries over shapes up to the limits: monotone, 256-aligned, large
 * enough for the tensors they hold, and computed without overflow. */
static void check_sizes(void) {
  const int32_t Ls[] = {1, 2, 63, 64, 65, 1000, 4096, 131072, 1 << 22};
  const int32_t Hqs[] = {1, 8, 32, 64, 4096};
  const int32_t ds[] = {64, 128};
  int shapes = 0;
  for (int li = 0; li < (int)(sizeof(Ls) / sizeof(Ls[0])); ++li)
    for (int hi = 0; hi < (int)(sizeof(Hqs) / sizeof(Hqs[0])); ++hi)
      for (int di = 0; di < 2; ++di)
        for (int dt = 0; dt < 2; ++dt)
          for (int flags = 0; flags < 8; ++flags)
            for (int B = 1; B <= 15; B += 14) {
              tsa_problem p = {B, Hqs[hi], Hqs[hi] >= 8 ? Hqs[hi] / 8 : 1, Ls[li], ds[di],
                               Ls[li] < 64 ? Ls[li] : 64, 0.05f, dt, flags};
              const size_t step = tsa_workspace_bytes(&p);
              const size_t fused = tsa_fused_workspace_bytes(&p);
              const size_t fwd = tsa_forward_workspace_bytes(&p);
              const double heads = (double)B * p.Hq;
              const double eb = dt == TSA_BF16 ? 2.0 : 4.0;
              ++shapes;
              CHECK(step > 0 && step % 256 == 0 && fused % 256 == 0 && fwd % 256 == 0,
                    "L=%d Hq=%d B=%d: sizes positive and 256-aligned", p.L, p.Hq, B);
              CHECK(step < fused && fused < fwd, "L=%d Hq=%d B=%d: step < fused < forward", p.L,
                    p.Hq, B);
              /* fused holds the scores and the rank map; forward adds compact K and V */
              CHECK((double)(fused - step) >= heads * p.L * 8.0,
                    "L=%d Hq=%d B=%d: fused scratch holds scores and ranks", p.L, p.Hq, B);
              CHECK((double)(fwd - fused) >= 2.0 * heads * p.L * p.d * eb,
                    "L=%d Hq=%d B=%d: forward scratch holds compact K and V", p.L, p.Hq, B);
              CHECK((double)fwd < 1.1 * (2.0 * heads * p.L * p.d * eb) + 64.0 * heads * p.L +
                                      (double)(1 << 24) * (1.0 + heads),
                    "L=%d Hq=%d B=%d: forward scratch within bounds", p.L, p.Hq, B);
              const size_t nb = ((size_t)p.L + 63) / 64, nw = (nb + 31) / 32;
              CHECK(tsa_block_mask_words(&p) == (size_t)B * p.Hq * nb * nw,
                    "L=%d Hq=%d B=%d: block mask words", p.L, p.Hq, B);
              if (li > 0) {
                tsa_problem q = p;
                q.L = Ls[li - 1];
                q.w = q.L < 64 ? q.L : 64;
                CHECK(tsa_forward_workspace_bytes(&q) <= fwd, "L=%d Hq=%d: monotone in L", p.L,
                      p.Hq);
              }
            }
  CHECK(shapes > 1000, "shape sweep ran (%d shapes)", shapes);
}

/* Every valid problem in a small grid passes validation on every entry
 * point (the injected launch failure is the only error). */
static void check_valid_problems(void) {
  for (int flags = 0; flags < 8; ++flags)
    for (int dt = 0; dt < 2; ++dt) {
      tsa_problem p = {2, 8, 2, 300, 64, 33, 0.1f, dt, flags};
      CHECK(!all_entry_points(&p, TSA_ERR_HIP, "valid"), "flags=%d dtype=%d: validation passes",
            flags, dt);
      CHECK(strstr(tsa_last_error(), "injected") != NULL, "flags=%d: the injected failure is named",
            flags);
    }
  /* the limits themselves are accepted */
  tsa_problem edge = {1, 4096, 1, 1 << 22, 128, 2944, 0.0f, TSA_BF16, 0};
  CHECK(tsa_workspace_bytes(&edge) > 0, "Hq=4096, L=2^22, w=2944 accepted");
  tsa_problem heads = {65535, 1, 1, 1, 64, 1, 0.999f, TSA_F32, 0};
  CHECK(tsa_workspace_bytes(&heads) > 0, "B*Hq = 65535 accepted");
  /* the no-allocation entry point refuses what exceeds its scratch */
  tsa_problem huge = {1, 32, 8, 1 << 22, 128, 64, 0.05f, TSA_BF16, 0};
  CHECK(tsa_fused_workspace_bytes(&huge) > TSA_NOALLOC_SCRATCH_BYTES, "huge needs more scratch");
  CHECK(tsa_forward_fused_noalloc(&huge, P(1), P(2), P(3), P(4), (int32_t*)P(5), (int32_t*)P(5),
                                  NULL) == TSA_ERR_UNSUPPORTED,
        "noalloc refuses a problem beyond its scratch");
}

static void check_strings(void) {
  const tsa_status all[5] = {TSA_OK, TSA_ERR_INVALID_ARG, TSA_ERR_UNSUPPORTED, TSA_ERR_WORKSPACE,
                             TSA_ERR_HIP};
  const char* names[5] = {"TSA_OK", "TSA_ERR_INVALID_ARG", "TSA_ERR_UNSUPPORTED",
                          "TSA_ERR_WORKSPACE", "TSA_ERR_HIP"};
  for (int i = 0; i < 5; ++i)
    CHECK(strcmp(tsa_status_string(all[i]), names[i]) == 0, "status string %d", i);
  CHECK(strcmp(tsa_status_string((tsa_status)99), "TSA_ERR_UNKNOWN") == 0, "unknown status");
  CHECK(tsa_version() && strstr(tsa_version(), "gfx950") != NULL, "version names gfx950");
}

/* The error text is per thread. */
struct thread_arg {
  int B;
  char text[256];
};

static void* fail_in_thread(void* arg) {
  struct thread_arg* a = (struct thread_arg*)arg;
  tsa_problem p = good();
  p.B = a->B;
  for (int i = 0; i < 200; ++i) {
    (void)tsa_workspace_bytes(&p);
    tsa_problem q = good();
    (void)tsa_score(&q, P(1), P(2), (float*)P(6), NULL, 0, NULL); /* workspace error */
    (void)tsa_workspace_bytes(&p);
  }
  snprintf(a->text, sizeof(a->text), "%s", tsa_last_error());
  return NULL;
}

static void check_threads(void) {
  struct thread_arg a[4] = {{0, ""}, {-3, ""}, {0, ""}, {-7, ""}};
  pthread_t th[4];
  for (int i = 0; i < 4; ++i) pthread_create(&th[i], NULL, fail_in_thread, &a[i]);
  for (int i = 0; i < 4; ++i) pthread_join(th[i], NULL);
  for (int i = 0; i < 4; ++i) {
    char want[32];
    snprintf(want, sizeof(want), "B=%d ", a[i].B);
    CHECK(strstr(a[i].text, want) != NULL, "thread %d sees its own error text: %s", i, a[i].text);
  }
}

int main(void) {
  if (setenv("TSA_FAULT_INJECT", "launch", 1) != 0) return 2;
  const char* e = getenv("TSA_FAULT_INJECT");
  if (!e || strcmp(e, "launch") != 0) return 2; /* without it valid calls would launch */
  g_buf = (unsigned char*)aligned_alloc(256, 256 * 16);
  if (!g_buf) return 2;
  memset(g_buf, 0, 256 * 16);
  check_strings();
  check_bad_problems();
  check_pointers();
  check_workspaces();
  check_sizes();
  check_valid_problems();
  check_threads();
  free(g_buf);
  printf("%d checks, %d failures\n", g_checks, g_failures);
  return g_failures ? 1 : 0;
}
