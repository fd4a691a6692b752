// Oracle driver for the sanitizer test: runs the oracle's entry points on
// random shapes (including empty shards, N > n and ragged splits) under
// AddressSanitizer and UndefinedBehaviorSanitizer, and checks the invariants
// that need no reference: sharded == shard-free bit for bit, and a rank's
// share == the shard of the full step.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
void orc_split_bounds(int64_t n, int64_t N, int64_t r, int64_t* a, int64_t* b);
int orc_zero_step(int mode, int64_t n, int64_t N, const void* param_in, const void* const* grads,
                  const void* master_in, const void* m_in, const void* v_in, void* param_out,
                  void* master_out, void* m_out, void* v_out, int64_t t, double lr, double b1,
                  double b2, double eps, double wd, const uint8_t* decay);
int orc_full_step(int mode, int64_t n, int64_t N, const void* param_in, const void* const* grads,
                  const void* master_in, const void* m_in, const void* v_in, void* param_out,
                  void* master_out, void* m_out, void* v_out, int64_t t, double lr, double b1,
                  double b2, double eps, double wd, const uint8_t* decay);
int orc_mean_grad(int mode, int64_t n, int64_t N, int64_t rank, const void* const* grads,
                  void* mean_out, double* sumsq_out);
int orc_sgd_step(int form, int mode, int64_t n, int64_t N, int64_t rank, const void* param_in,
                 const void* const* grads, const void* master_in, const void* buf_in,
                 void* param_out, void* master_out, void* buf_out, int64_t t, double lr,
                 double wd, double momentum, double dampening, int nesterov,
                 const uint8_t* decay);
}

static int g_fail = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

int main() {
  std::mt19937_64 rng(7);
  std::normal_distribution<float> nd(0.f, 1.f);
  for (int trial = 0; trial < 40; ++trial) {
    const int64_t n = 1 + (int64_t)(rng() % 3000);
    const int64_t N = 1 + (int64_t)(rng() % 70);
    const int mode = (int)(rng() % 2);  // fp64 and fp32 (all-fp layouts)
    const size_t s = mode == 0 ? 8 : 4;
    std::vector<std::vector<unsigned char>> g(N, std::vector<unsigned char>(n * s));
    std::vector<const void*> gp(N);
    for (int64_t k = 0; k < N; ++k) {
      for (int64_t i = 0; i < n; ++i) {
        const float x = nd(rng);
        if (mode == 0) { double d = x; std::memcpy(&g[k][i * 8], &d, 8); }
        else std::memcpy(&g[k][i * 4], &x, 4);
      }
      gp[k] = g[k].data();
    }
    std::vector<unsigned char> p(n * s), m(n * s, 0), v(n * s, 0), dec(n);
    for (int64_t i = 0; i < n; ++i) {
      const float x = nd(rng);
      if (mode == 0) { double d = x; std::memcpy(&p[i * 8], &d, 8); }
      else std::memcpy(&p[i * 4], &x, 4);
      dec[i] = (uint8_t)(rng() & 1);
    }
    std::vector<unsigned char> p1(n * s), m1(n * s), v1(n * s), p2(n * s), m2(n * s), v2(n * s);
    CHECK(orc_zero_step(mode, n, N, p.data(), gp.data(), nullptr, m.data(), v.data(), p1.data(),
                        nullptr, m1.data(), v1.data(), 1, 1e-3, 0.9, 0.95, 1e-8, 0.1,
                        dec.data()) == 0);
    CHECK(orc_full_step(mode, n, N, p.data(), gp.data(), nullptr, m.data(), v.data(), p2.data(),
                        nullptr, m2.data(), v2.data(), 1, 1e-3, 0.9, 0.95, 1e-8, 0.1,
                        dec.data()) == 0);
    CHECK(p1 == p2 && m1 == m2 && v1 == v2);
    std::vector<unsigned char> mean(n * s);
    double ss = -1;
    CHECK(orc_mean_grad(mode, n, N, -1, gp.data(), mean.data(), &ss) == 0 && ss >= 0);
    // each rank's share of the mean gradient, from chunk copies
    for (int64_t r = 0; r < N; r += 1 + N / 4) {
      int64_t a, b;
      orc_split_bounds(n, N, r, &a, &b);
      std::vector<std::vector<unsigned char>> ch(N);
      std::vector<const void*> cp(N);
      for (int64_t k = 0; k < N; ++k) {
        ch[k].assign(g[k].begin() + a * s, g[k].begin() + b * s);
        cp[k] = ch[k].data();
      }
      std::vector<unsigned char> mr((b - a) * s + 1);
      double sr = -1;
      CHECK(orc_mean_grad(mode, n, N, r, cp.data(), mr.data(), &sr) == 0 && sr >= 0);
      CHECK(std::memcmp(mr.data(), mean.data() + a * s, (b - a) * s) == 0);
    }
    std::vector<unsigned char> p3(n * s), b3(n * s);
    CHECK(orc_sgd_step(0, mode, n, N, -1, p.data(), gp.data(), nullptr, m.data(), p3.data(),
                       nullptr, b3.data(), 1, 1e-2, 0.01, 0.9, 0.0, 1, dec.data()) == 0);
  }
  std::printf("oracle driver: %d failures\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}
