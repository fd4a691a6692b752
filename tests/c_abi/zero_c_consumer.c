/*
 * A plain C consumer of the C ABI in include/zero_adam.h, with no Python and no
 * torch: device buffers come from the HIP runtime, the step from libzero.so,
 * and the expected values from the CPU oracle (liboracle.so, test
 * infrastructure) run on the same host inputs.
 *
 *   zero_c_consumer host   host-only checks of the ABI (no device call)
 *   zero_c_consumer gpu    init_states and three fused steps in fp64 (N = 3),
 *                          fp32 (N = 8), bf16 mixed precision (N = 4) and fp16
 *                          mixed precision (N = 5), compared with the oracle:
 *                          fp64 bit-exact, fp32 within 1e-6 * max(1, |ref|),
 *                          bf16 and fp16 within 1 ulp; then a bucketed fp32
 *                          step (zero_step_buckets) whose buckets wait on
 *                          events that a producer stream records after copying
 *                          each bucket's gradients in, against the oracle;
 *                          and a clipped fp32 step (zero_step_clipped): its
 *                          squared norm within the summation-order bound of
 *                          the oracle's, and the step equal to the oracle's
 *                          step from the mean clipped by the device's norm;
 *                          then a bf16 step that stores the averaged gradient
 *                          (zero_step_with_mean) and the no-allocation mean
 *                          (zero_mean_grad_noalloc), bit for bit against the
 *                          oracle's mean and step.
 * Exit status 0 when every check holds.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_adam.h"

/* the oracle's entry points (oracle/zero_oracle.cpp) */
void orc_init_states(int mode, int64_t len, const void* param, void* master, void* m, void* v);
int orc_zero_step(int mode, int64_t n, int64_t N, const void* param_in, const void* const* grads,
                  const void* master_in, const void* m_in, const void* v_in, void* param_out,
                  void* master_out, void* m_out, void* v_out, int64_t t, double lr, double b1,
                  double b2, double eps, double wd, const uint8_t* decay);
int orc_mean_grad(int mode, int64_t n, int64_t N, int64_t rank, const void* const* grads,
                  void* mean_out, double* sumsq_out);
int orc_step_mean(int mode, int64_t n, int64_t N, int64_t rank, const void* param_in,
                  const void* mean, const void* master_in, const void* m_in, const void* v_in,
                  void* param_out, void* master_out, void* m_out, void* v_out, int64_t t,
                  double lr, double b1, double b2, double eps, double wd, const uint8_t* decay,
                  const double* clip_sumsq, double max_norm);

static int g_fail = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, #c);     \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)
#define HIP(x)                                                                      \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, \
              __LINE__);                                                            \
      exit(2);                                                                      \
    }                                                                               \
  } while (0)

/* seeded inputs: a 64-bit linear congruential generator */
static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return g_state;
}
static double uniform(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }
/* a random bf16 bit pattern with exponent in [e_lo, e_hi] */
static uint16_t random_bf16(int e_lo, int e_hi) {
  const uint64_t r = next_u64();
  const uint16_t sign = (uint16_t)((r >> 63) << 15);
  const uint16_t exp = (uint16_t)(e_lo + (int)((r >> 8) % (uint64_t)(e_hi - e_lo + 1)));
  return (uint16_t)(sign | (uint16_t)(exp << 7) | (uint16_t)(r & 0x7F));
}

/* a random fp16 bit pattern with exponent field in [e_lo, e_hi] */
static uint16_t random_fp16(int e_lo, int e_hi) {
  const uint64_t r = next_u64();
  const uint16_t sign = (uint16_t)((r >> 63) << 15);
  const uint16_t exp = (uint16_t)(e_lo + (int)((r >> 12) % (uint64_t)(e_hi - e_lo + 1)));
  return (uint16_t)(sign | (uint16_t)(exp << 10) | (uint16_t)(r & 0x3FF));
}

static int host_checks(void) {
  int64_t a = 0, b = 0;
  CHECK(zero_shard_bounds(10, 4, 1, &a, &b) == ZERO_OK && a == 3 && b == 6);
  CHECK(zero_shard_bounds(3, 5, 4, &a, &b) == ZERO_OK && a == 3 && b == 3);
  zero_mem mem;
  CHECK(zero_memory_bytes(8000000000LL, 64, 0, 3, ZERO_MODE_MIXED_BF16, 0, &mem) == ZERO_OK);
  CHECK(mem.total == 16 * 125000000LL);
  int32_t stage = 0;
  CHECK(zero_min_stage(20000000000LL, 8, ZERO_MODE_MIXED_F16, 10000000000LL, 80000000000LL,
                       &stage) == ZERO_OK && stage == 3);
  CHECK(zero_step(NULL, NULL, NULL, NULL, 1, NULL) == ZERO_EINVAL);
  CHECK(strlen(zero_last_error()) > 0);
  zero_hparams hp;
  memset(&hp, 0, sizeof hp);
  hp.n = 1000;
  hp.n_workers = 4;
  hp.rank = -1;
  hp.mode = ZERO_MODE_F32;
  hp.lr = 1e-3;
  hp.beta1 = 0.9;
  hp.beta2 = 0.999;
  hp.eps = 1e-8;
  zero_step_scalars sc;
  CHECK(zero_step_scalars_fill(&hp, 2, &sc) == ZERO_OK && sc.t == 2);
  CHECK(sc.bias1 == 1.0 - pow(0.9, 2.0) && sc.bias2 == 1.0 - pow(0.999, 2.0));
  CHECK(zero_step_scalars_fill(&hp, 0, &sc) == ZERO_EINVAL);
  printf("host checks: %d failures\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}

static size_t state_size(int mode) { return mode == ZERO_MODE_F64 ? 8 : 4; }
static size_t elem_size(int mode) { return mode == ZERO_MODE_F64 ? 8 : (mode == ZERO_MODE_F32 ? 4 : 2); }

/* |got - ref| within the bar for one mode's element kind; counts bit-exact */
static int64_t compare(const char* what, int kind, const void* got, const void* ref, int64_t n) {
  int64_t exact = 0, bad = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (kind == 0) { /* fp64 bit-exact */
      const int same = memcmp((const char*)got + 8 * i, (const char*)ref + 8 * i, 8) == 0;
      exact += same;
      bad += !same;
    } else if (kind == 1) { /* fp32 */
      const float g = ((const float*)got)[i], r = ((const float*)ref)[i];
      const int same = memcmp(&g, &r, 4) == 0;
      exact += same;
      if (!same && !(fabs((double)g - (double)r) <= 1e-6 * fmax(1.0, fabs((double)r)))) ++bad;
    } else { /* bf16, ordered bit patterns within 1 */
      const uint16_t g = ((const uint16_t*)got)[i], r = ((const uint16_t*)ref)[i];
      const int32_t og = (g & 0x8000) ? -(int32_t)(g & 0x7FFF) : (int32_t)g;
      const int32_t orr = (r & 0x8000) ? -(int32_t)(r & 0x7FFF) : (int32_t)r;
      exact += g == r;
      if (abs(og - orr) > 1) ++bad;
    }
  }
  printf("  %-6s %lld of %lld bit-exact, %lld beyond the bar\n", what, (long long)exact,
         (long long)n, (long long)bad);
  return bad;
}

static void run_mode(int mode, int64_t n, int N) {
  const size_t G = elem_size(mode), S = state_size(mode);
  const int mixed = mode == ZERO_MODE_MIXED_BF16 || mode == ZERO_MODE_MIXED_F16;
  printf("[case] mode %d n %lld N %d\n", mode, (long long)n, N);
  fflush(stdout);
  /* host inputs */
  unsigned char* p_h = malloc(n * G);
  unsigned char* g_h[8];
  for (int k = 0; k < N; ++k) g_h[k] = malloc(n * G);
  for (int64_t i = 0; i < n; ++i) {
    if (mode == ZERO_MODE_F64) ((double*)p_h)[i] = uniform() - 0.5;
    else if (mode == ZERO_MODE_F32) ((float*)p_h)[i] = (float)(0.04 * (uniform() - 0.5));
    else if (mode == ZERO_MODE_MIXED_BF16) ((uint16_t*)p_h)[i] = random_bf16(115, 124);
    else ((uint16_t*)p_h)[i] = random_fp16(5, 12); /* 2^-10 .. 2^-3 */
  }
  /* device buffers */
  void *p_d, *m_d, *v_d, *ms_d = NULL, *g_d[8];
  HIP(hipMalloc(&p_d, n * G));
  HIP(hipMalloc(&m_d, n * S));
  HIP(hipMalloc(&v_d, n * S));
  if (mixed) HIP(hipMalloc(&ms_d, n * S));
  for (int k = 0; k < N; ++k) HIP(hipMalloc(&g_d[k], n * G));
  HIP(hipMemcpy(p_d, p_h, n * G, hipMemcpyHostToDevice));
  /* oracle state */
  unsigned char *op = malloc(n * G), *om = malloc(n * S), *ov = malloc(n * S), *oms = NULL;
  memcpy(op, p_h, n * G);
  if (mixed) oms = malloc(n * S);
  orc_init_states(mode, n, op, oms, om, ov);

  zero_hparams hp;
  memset(&hp, 0, sizeof hp);
  hp.n = n;
  hp.n_workers = N;
  hp.rank = -1;
  hp.mode = mode;
  hp.optimizer = ZERO_OPT_ADAM;
  hp.lr = 1e-3;
  hp.beta1 = 0.9;
  hp.beta2 = 0.95;
  hp.eps = 1e-8;
  hp.weight_decay = 0.05;
  zero_states st = {ms_d, m_d, v_d};
  CHECK(zero_init_states(&hp, p_d, &st, NULL) == ZERO_OK);
  const void* gp[8];
  for (int k = 0; k < N; ++k) gp[k] = g_d[k];
  unsigned char *np_ = malloc(n * G), *nm = malloc(n * S), *nv = malloc(n * S), *nms = NULL;
  if (mixed) nms = malloc(n * S);
  for (int64_t t = 1; t <= 3; ++t) {
    for (int k = 0; k < N; ++k) {
      for (int64_t i = 0; i < n; ++i) {
        if (mode == ZERO_MODE_F64) ((double*)g_h[k])[i] = 2.0 * (uniform() - 0.5);
        else if (mode == ZERO_MODE_F32) ((float*)g_h[k])[i] = (float)(2e-3 * (uniform() - 0.5));
        else if (mode == ZERO_MODE_MIXED_BF16) ((uint16_t*)g_h[k])[i] = random_bf16(110, 121);
        else ((uint16_t*)g_h[k])[i] = random_fp16(1, 9); /* 2^-14 .. 2^-6 */
      }
      HIP(hipMemcpy(g_d[k], g_h[k], n * G, hipMemcpyHostToDevice));
    }
    CHECK(zero_step(&hp, p_d, gp, &st, t, NULL) == ZERO_OK);
    CHECK(orc_zero_step(mode, n, N, op, (const void* const*)g_h, oms, om, ov, np_, nms, nm, nv, t,
                        hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, NULL) == 0);
    memcpy(op, np_, n * G);
    memcpy(om, nm, n * S);
    memcpy(ov, nv, n * S);
    if (mixed) memcpy(oms, nms, n * S);
  }
  HIP(hipDeviceSynchronize());
  unsigned char *dp = malloc(n * G), *dm = malloc(n * S), *dv = malloc(n * S);
  HIP(hipMemcpy(dp, p_d, n * G, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dm, m_d, n * S, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dv, v_d, n * S, hipMemcpyDeviceToHost));
  const int sk = mode == ZERO_MODE_F64 ? 0 : 1;
  CHECK(compare("param", mode == ZERO_MODE_F64 ? 0 : (mixed ? 2 : 1), dp, op, n) == 0);
  CHECK(compare("m", sk, dm, om, n) == 0);
  CHECK(compare("v", sk, dv, ov, n) == 0);
  if (mixed) {
    unsigned char* dms = malloc(n * S);
    HIP(hipMemcpy(dms, ms_d, n * S, hipMemcpyDeviceToHost));
    CHECK(compare("master", 1, dms, oms, n) == 0);
    free(dms);
    free(oms);
    free(nms);
    HIP(hipFree(ms_d));
  }
  for (int k = 0; k < N; ++k) {
    HIP(hipFree(g_d[k]));
    free(g_h[k]);
  }
  HIP(hipFree(p_d));
  HIP(hipFree(m_d));
  HIP(hipFree(v_d));
  free(p_h);
  free(op);
  free(om);
  free(ov);
  free(np_);
  free(nm);
  free(nv);
  free(dp);
  free(dm);
  free(dv);
}

/* Two bucketed steps: a producer stream copies each bucket's gradients from
 * pinned host memory and records an event; zero_step_buckets on a second
 * stream steps each bucket once its event has completed. */
static void run_buckets(void) {
  const int mode = ZERO_MODE_F32, N = 4;
  const int64_t n = 65539, bsize = 8192;
  const int nb = (int)((n + bsize - 1) / bsize);
  printf("[case] buckets with events: fp32 n %lld N %d, %d buckets\n", (long long)n, N, nb);
  fflush(stdout);
  float *p_h, *g_h[4];
  HIP(hipHostMalloc((void**)&p_h, n * 4, hipHostMallocDefault));
  for (int k = 0; k < N; ++k) HIP(hipHostMalloc((void**)&g_h[k], n * 4, hipHostMallocDefault));
  for (int64_t i = 0; i < n; ++i) p_h[i] = (float)(0.04 * (uniform() - 0.5));
  void *p_d, *m_d, *v_d, *g_d[4];
  HIP(hipMalloc(&p_d, n * 4));
  HIP(hipMalloc(&m_d, n * 4));
  HIP(hipMalloc(&v_d, n * 4));
  for (int k = 0; k < N; ++k) HIP(hipMalloc(&g_d[k], n * 4));
  HIP(hipMemcpy(p_d, p_h, n * 4, hipMemcpyHostToDevice));
  float *op = malloc(n * 4), *om = malloc(n * 4), *ov = malloc(n * 4);
  float *np_ = malloc(n * 4), *nm = malloc(n * 4), *nv = malloc(n * 4);
  memcpy(op, p_h, n * 4);
  orc_init_states(mode, n, op, NULL, om, ov);
  zero_hparams hp;
  memset(&hp, 0, sizeof hp);
  hp.n = n;
  hp.n_workers = N;
  hp.rank = -1;
  hp.mode = mode;
  hp.lr = 1e-3;
  hp.beta1 = 0.9;
  hp.beta2 = 0.95;
  hp.eps = 1e-8;
  zero_states st = {NULL, m_d, v_d};
  hipStream_t prod, step;
  HIP(hipStreamCreate(&prod));
  HIP(hipStreamCreate(&step));
  CHECK(zero_init_states(&hp, p_d, &st, step) == ZERO_OK);
  hipEvent_t ev[16];
  int64_t edges[32];
  for (int b = 0; b < nb; ++b) {
    const int i = nb - 1 - b; /* last bucket first, as a backward pass finishes them */
    edges[2 * b] = i * bsize;
    edges[2 * b + 1] = (i + 1) * bsize < n ? (i + 1) * bsize : n;
    HIP(hipEventCreateWithFlags(&ev[b], hipEventDisableTiming));
  }
  const void* gp[4];
  for (int k = 0; k < N; ++k) gp[k] = g_d[k];
  for (int64_t t = 1; t <= 2; ++t) {
    for (int k = 0; k < N; ++k)
      for (int64_t i = 0; i < n; ++i) g_h[k][i] = (float)(2e-3 * (uniform() - 0.5));
    for (int b = 0; b < nb; ++b) {
      const int64_t lo = edges[2 * b], hi = edges[2 * b + 1];
      for (int k = 0; k < N; ++k)
        HIP(hipMemcpyAsync((char*)g_d[k] + lo * 4, g_h[k] + lo, (hi - lo) * 4,
                           hipMemcpyHostToDevice, prod));
      HIP(hipEventRecord(ev[b], prod));
    }
    CHECK(zero_step_buckets(&hp, p_d, gp, &st, t, edges, nb, (void* const*)ev, step) ==
          ZERO_OK);
    HIP(hipStreamSynchronize(step)); /* every bucket waited for its copies */
    CHECK(orc_zero_step(mode, n, N, op, (const void* const*)g_h, NULL, om, ov, np_, NULL, nm, nv,
                        t, hp.lr, hp.beta1, hp.beta2, hp.eps, 0.0, NULL) == 0);
    memcpy(op, np_, n * 4);
    memcpy(om, nm, n * 4);
    memcpy(ov, nv, n * 4);
  }
  float *dp = malloc(n * 4), *dm = malloc(n * 4);
  HIP(hipMemcpy(dp, p_d, n * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dm, m_d, n * 4, hipMemcpyDeviceToHost));
  CHECK(compare("param", 1, dp, op, n) == 0);
  CHECK(compare("m", 1, dm, om, n) == 0);
  for (int b = 0; b < nb; ++b) HIP(hipEventDestroy(ev[b]));
  HIP(hipStreamDestroy(prod));
  HIP(hipStreamDestroy(step));
  for (int k = 0; k < N; ++k) {
    HIP(hipFree(g_d[k]));
    HIP(hipHostFree(g_h[k]));
  }
  HIP(hipFree(p_d));
  HIP(hipFree(m_d));
  HIP(hipFree(v_d));
  HIP(hipHostFree(p_h));
  free(op);
  free(om);
  free(ov);
  free(np_);
  free(nm);
  free(nv);
  free(dp);
  free(dm);
}

/* One clipped step with the clip active (max_norm = half the norm). The device
 * sums the squares in a fixed tree, the oracle in index order: both sum the
 * same exact squares in double, so they agree within 2 n 2^-53 relatively.
 * Given the device's squared norm, the oracle's step is the same arithmetic. */
static void run_clipped(void) {
  const int mode = ZERO_MODE_F32, N = 8;
  const int64_t n = 65539;
  printf("[case] clipped step: fp32 n %lld N %d\n", (long long)n, N);
  fflush(stdout);
  float *p_h = malloc(n * 4), *g_h[8];
  for (int64_t i = 0; i < n; ++i) p_h[i] = (float)(0.04 * (uniform() - 0.5));
  void *p_d, *m_d, *v_d, *g_d[8], *ws_d;
  double* ss_d;
  for (int k = 0; k < N; ++k) {
    g_h[k] = malloc(n * 4);
    for (int64_t i = 0; i < n; ++i) g_h[k][i] = (float)(2e-3 * (uniform() - 0.5));
    HIP(hipMalloc(&g_d[k], n * 4));
    HIP(hipMemcpy(g_d[k], g_h[k], n * 4, hipMemcpyHostToDevice));
  }
  HIP(hipMalloc(&p_d, n * 4));
  HIP(hipMalloc(&m_d, n * 4));
  HIP(hipMalloc(&v_d, n * 4));
  HIP(hipMalloc((void**)&ss_d, sizeof(double)));
  HIP(hipMemcpy(p_d, p_h, n * 4, hipMemcpyHostToDevice));
  zero_hparams hp;
  memset(&hp, 0, sizeof hp);
  hp.n = n;
  hp.n_workers = N;
  hp.rank = -1;
  hp.mode = mode;
  hp.lr = 1e-3;
  hp.beta1 = 0.9;
  hp.beta2 = 0.95;
  hp.eps = 1e-8;
  hp.weight_decay = 0.05;
  size_t wsb = 0;
  CHECK(zero_step_clipped_workspace_bytes(&hp, &wsb) == ZERO_OK && wsb > 0);
  HIP(hipMalloc(&ws_d, wsb));
  zero_states st = {NULL, m_d, v_d};
  CHECK(zero_init_states(&hp, p_d, &st, NULL) == ZERO_OK);
  float *mean_o = malloc(n * 4), *om = malloc(n * 4), *ov = malloc(n * 4);
  float *np_ = malloc(n * 4), *nm = malloc(n * 4), *nv = malloc(n * 4);
  double ss_o = 0.0;
  CHECK(orc_mean_grad(mode, n, N, -1, (const void* const*)g_h, mean_o, &ss_o) == 0);
  const double max_norm = 0.5 * sqrt(ss_o);
  const void* gp[8];
  for (int k = 0; k < N; ++k) gp[k] = g_d[k];
  CHECK(zero_step_clipped(&hp, p_d, gp, &st, 1, max_norm, ss_d, ws_d, wsb, NULL) == ZERO_OK);
  HIP(hipDeviceSynchronize());
  double ss_dev = 0.0;
  HIP(hipMemcpy(&ss_dev, ss_d, sizeof(double), hipMemcpyDeviceToHost));
  CHECK(fabs(ss_dev - ss_o) <= 2.0 * (double)n * ldexp(1.0, -53) * ss_o);
  orc_init_states(mode, n, p_h, NULL, om, ov);
  CHECK(orc_step_mean(mode, n, N, -1, p_h, mean_o, NULL, om, ov, np_, NULL, nm, nv, 1, hp.lr,
                      hp.beta1, hp.beta2, hp.eps, hp.weight_decay, NULL, &ss_dev, max_norm) == 0);
  float *dp = malloc(n * 4), *dm = malloc(n * 4), *dv = malloc(n * 4);
  HIP(hipMemcpy(dp, p_d, n * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dm, m_d, n * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dv, v_d, n * 4, hipMemcpyDeviceToHost));
  CHECK(compare("param", 1, dp, np_, n) == 0);
  CHECK(compare("m", 1, dm, nm, n) == 0);
  CHECK(compare("v", 1, dv, nv, n) == 0);
  for (int k = 0; k < N; ++k) {
    HIP(hipFree(g_d[k]));
    free(g_h[k]);
  }
  HIP(hipFree(p_d));
  HIP(hipFree(m_d));
  HIP(hipFree(v_d));
  HIP(hipFree(ws_d));
  HIP(hipFree(ss_d));
  free(p_h);
  free(mean_o);
  free(om);
  free(ov);
  free(np_);
  free(nm);
  free(nv);
  free(dp);
  free(dm);
  free(dv);
}

/* The fused step that also stores the averaged gradient (bf16 mixed
 * precision), and the no-allocation mean with its squared norm, each against
 * the oracle: the stored mean and every state bit for bit, the norm within the
 * summation-order bound. */
static void run_with_mean_and_noalloc(void) {
  const int mode = ZERO_MODE_MIXED_BF16, N = 4;
  const int64_t n = 40009;
  printf("[case] step with mean store and no-allocation mean: bf16 n %lld N %d\n", (long long)n,
         N);
  fflush(stdout);
  uint16_t *p_h = malloc(n * 2), *g_h[4];
  for (int64_t i = 0; i < n; ++i) p_h[i] = random_bf16(115, 124);
  void *p_d, *ms_d, *m_d, *v_d, *g_d[4], *mean_d, *mean2_d;
  double* ss_d;
  for (int k = 0; k < N; ++k) {
    g_h[k] = malloc(n * 2);
    for (int64_t i = 0; i < n; ++i) g_h[k][i] = random_bf16(110, 121);
    HIP(hipMalloc(&g_d[k], n * 2));
    HIP(hipMemcpy(g_d[k], g_h[k], n * 2, hipMemcpyHostToDevice));
  }
  HIP(hipMalloc(&p_d, n * 2));
  HIP(hipMalloc(&ms_d, n * 4));
  HIP(hipMalloc(&m_d, n * 4));
  HIP(hipMalloc(&v_d, n * 4));
  HIP(hipMalloc(&mean_d, n * 4));
  HIP(hipMalloc(&mean2_d, n * 4));
  HIP(hipMalloc((void**)&ss_d, sizeof(double)));
  HIP(hipMemcpy(p_d, p_h, n * 2, hipMemcpyHostToDevice));
  zero_hparams hp;
  memset(&hp, 0, sizeof hp);
  hp.n = n;
  hp.n_workers = N;
  hp.rank = -1;
  hp.mode = mode;
  hp.lr = 1e-3;
  hp.beta1 = 0.9;
  hp.beta2 = 0.95;
  hp.eps = 1e-8;
  hp.weight_decay = 0.05;
  zero_states st = {ms_d, m_d, v_d};
  CHECK(zero_init_states(&hp, p_d, &st, NULL) == ZERO_OK);
  const void* gp[4];
  for (int k = 0; k < N; ++k) gp[k] = g_d[k];
  CHECK(zero_step_with_mean(&hp, p_d, gp, &st, 1, mean_d, NULL) == ZERO_OK);
  CHECK(zero_mean_grad_noalloc(&hp, gp, mean2_d, ss_d, NULL) == ZERO_OK);
  HIP(hipDeviceSynchronize());
  float *mean_o = malloc(n * 4), *oms = malloc(n * 4), *om = malloc(n * 4), *ov = malloc(n * 4);
  float *nms = malloc(n * 4), *nm = malloc(n * 4), *nv = malloc(n * 4);
  uint16_t* np_ = malloc(n * 2);
  double ss_o = 0.0;
  CHECK(orc_mean_grad(mode, n, N, -1, (const void* const*)g_h, mean_o, &ss_o) == 0);
  orc_init_states(mode, n, p_h, oms, om, ov);
  CHECK(orc_zero_step(mode, n, N, p_h, (const void* const*)g_h, oms, om, ov, np_, nms, nm, nv, 1,
                      hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, NULL) == 0);
  float *dmean = malloc(n * 4), *dmean2 = malloc(n * 4), *dms = malloc(n * 4);
  float *dm = malloc(n * 4), *dv = malloc(n * 4);
  uint16_t* dp = malloc(n * 2);
  double ss_dev = 0.0;
  HIP(hipMemcpy(dmean, mean_d, n * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dmean2, mean2_d, n * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dp, p_d, n * 2, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dms, ms_d, n * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dm, m_d, n * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(dv, v_d, n * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(&ss_dev, ss_d, sizeof(double), hipMemcpyDeviceToHost));
  CHECK(memcmp(dmean, mean_o, n * 4) == 0);
  CHECK(memcmp(dmean2, mean_o, n * 4) == 0);
  CHECK(fabs(ss_dev - ss_o) <= 2.0 * (double)n * ldexp(1.0, -53) * ss_o);
  CHECK(compare("param", 2, dp, np_, n) == 0);
  CHECK(memcmp(dms, nms, n * 4) == 0 && memcmp(dm, nm, n * 4) == 0 && memcmp(dv, nv, n * 4) == 0);
  printf("  mean (stored and no-allocation), master, m and v bit-exact\n");
  for (int k = 0; k < N; ++k) {
    HIP(hipFree(g_d[k]));
    free(g_h[k]);
  }
  HIP(hipFree(p_d));
  HIP(hipFree(ms_d));
  HIP(hipFree(m_d));
  HIP(hipFree(v_d));
  HIP(hipFree(mean_d));
  HIP(hipFree(mean2_d));
  HIP(hipFree(ss_d));
  free(p_h);
  free(mean_o);
  free(oms);
  free(om);
  free(ov);
  free(nms);
  free(nm);
  free(nv);
  free(np_);
  free(dmean);
  free(dmean2);
  free(dms);
  free(dm);
  free(dv);
  free(dp);
}

int main(int argc, char** argv) {
  if (argc != 2 || (strcmp(argv[1], "host") != 0 && strcmp(argv[1], "gpu") != 0)) {
    fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
    return 2;
  }
  if (strcmp(argv[1], "host") == 0) return host_checks();
  run_mode(ZERO_MODE_F64, 100003, 3);
  run_mode(ZERO_MODE_F32, 65539, 8);
  run_mode(ZERO_MODE_MIXED_BF16, 40009, 4);
  run_mode(ZERO_MODE_MIXED_F16, 30011, 5);
  run_buckets();
  run_clipped();
  run_with_mean_and_noalloc();
  printf("gpu run: %d failures\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}
