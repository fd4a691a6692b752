// Host-only driver for the sanitizer test: exercises the C ABI's host logic
// (validation, shard bounds, memory model, workspace sizes) with the launch
// layer replaced by stubs, so that it runs under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU. Any launch reaching the
// stubs is counted, never executed.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "zero_adam.h"
#include "zero_launch.h"

static int g_launches = 0;

// What each launch reaching the stubs was given: kind 0 step, 1 step from a
// mean, 2 mean (w = mean, m = partials), 3 finalize (w = partials, len = count).
struct Rec {
  int kind;
  int64_t len;
  uintptr_t w, m, v, out, g0, g1;
  int64_t mask_off;
};
static std::vector<Rec> g_rec;

static void record_step(int kind, const zlaunch::StepArgs& a) {
  g_rec.push_back({kind, a.len, (uintptr_t)a.w, (uintptr_t)a.m, (uintptr_t)a.v, (uintptr_t)a.out,
                   (uintptr_t)a.grads[0], a.n_workers > 1 ? (uintptr_t)a.grads[1] : 0,
                   a.mask_bit_offset});
}

namespace zlaunch {
const char* launch_step(const StepArgs& a, void*) {
  ++g_launches;
  record_step(0, a);
  return nullptr;
}
const char* launch_init(const InitArgs&, void*) { ++g_launches; return nullptr; }
const char* launch_step_mean(const StepArgs& a, void*) {
  ++g_launches;
  record_step(1, a);
  return nullptr;
}
const char* launch_mean(const MeanArgs& a, void*) {
  ++g_launches;
  g_rec.push_back({2, a.len, (uintptr_t)a.mean, (uintptr_t)a.partials, 0, 0,
                   (uintptr_t)a.grads[0], 0, 0});
  return nullptr;
}
const char* launch_sumsq_finalize(const double* partials, int64_t count, double* out, void*) {
  ++g_launches;
  g_rec.push_back({3, count, (uintptr_t)partials, 0, 0, (uintptr_t)out, 0, 0, 0});
  return nullptr;
}
int64_t mean_partials(int, int64_t len) { return len / 1024 + 1; }
const char* stream_wait(void*, void*) { ++g_launches; return nullptr; }
// a stand-in address for the library's static device scratch
constexpr uintptr_t kFakeScratch = (uintptr_t)0x7A << 40;
static int g_scratch_lookups = 0;
const char* scratch_address(void*, double** out) {
  ++g_scratch_lookups;
  *out = reinterpret_cast<double*>(kFakeScratch);
  return nullptr;
}
}  // namespace zlaunch

static int g_fail = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static zero_hparams hp(int64_t n, int32_t N, int32_t rank, int32_t mode) {
  zero_hparams h;
  std::memset(&h, 0, sizeof h);
  h.n = n;
  h.n_workers = N;
  h.rank = rank;
  h.mode = mode;
  h.lr = 1e-3;
  h.beta1 = 0.9;
  h.beta2 = 0.999;
  h.eps = 1e-8;
  return h;
}

int main() {
  // shard bounds: cover [0, n) exactly, numpy's rule
  for (int64_t n = 0; n < 300; n += 7)
    for (int32_t N = 1; N < 70; ++N) {
      int64_t prev = 0;
      for (int32_t r = 0; r < N; ++r) {
        int64_t a, b;
        CHECK(zero_shard_bounds(n, N, r, &a, &b) == ZERO_OK);
        CHECK(a == prev && b >= a && b - a >= n / N && b - a <= n / N + 1);
        prev = b;
      }
      CHECK(prev == n);
    }
  int64_t a, b;
  CHECK(zero_shard_bounds(8000000000LL, 8, 7, &a, &b) == ZERO_OK && b == 8000000000LL);
  CHECK(zero_shard_bounds(10, 0, 0, &a, &b) == ZERO_EINVAL && std::strlen(zero_last_error()) > 0);

  // memory model over a wide range, including the largest counts
  zero_mem m;
  for (int32_t stage = 0; stage <= 3; ++stage)
    for (int32_t mode = 0; mode <= 2; ++mode) {
      CHECK(zero_memory_bytes(175000000000LL, 64, 63, stage, mode, 0, &m) == ZERO_OK);
      CHECK(m.total == m.params + m.grads + m.optimizer);
    }
  CHECK(zero_memory_bytes(10, 4, 0, 4, 0, 0, &m) == ZERO_EINVAL);
  int32_t stage = 9;
  CHECK(zero_min_stage(20000000000LL, 8, ZERO_MODE_MIXED_BF16, 10000000000LL, 80000000000LL,
                       &stage) == ZERO_OK && stage == 3);
  CHECK(zero_min_stage(10, 8, ZERO_MODE_F32, 0, 0, &stage) == ZERO_OK && stage == -1);
  CHECK(zero_min_stage(10, 8, ZERO_MODE_F32, 0, 10, nullptr) == ZERO_EINVAL);

  // step validation with fake, aligned, non-overlapping addresses
  const uintptr_t A = (uintptr_t)1 << 32;
  const void* grads[256];
  for (int k = 0; k < 256; ++k) grads[k] = (const void*)(A + ((uintptr_t)(3 + k) << 24));
  zero_states st = {nullptr, (void*)(A + (1u << 24)), (void*)(A + (2u << 24))};
  zero_hparams h = hp(1000, 4, -1, ZERO_MODE_F32);
  CHECK(zero_step(&h, (void*)A, grads, &st, 1, nullptr) == ZERO_OK);
  CHECK(zero_step(&h, (void*)A, grads, &st, 0, nullptr) == ZERO_EINVAL);
  h.beta1 = 1.0;
  CHECK(zero_step(&h, (void*)A, grads, &st, 1, nullptr) == ZERO_EINVAL);
  h = hp(1000, 256, -1, ZERO_MODE_F32);
  CHECK(zero_step(&h, (void*)A, grads, &st, 1, nullptr) == ZERO_OK);
  h = hp(1000, 257, -1, ZERO_MODE_F32);
  CHECK(zero_step(&h, (void*)A, grads, &st, 1, nullptr) == ZERO_EINVAL);
  // rank mode, ragged shards, misaligned slot is fine
  zero_states stm = {(void*)(A + ((uintptr_t)300 << 24)), (void*)(A + (1u << 24)), (void*)(A + (2u << 24))};
  h = hp(8 * 1001 + 3, 8, 3, ZERO_MODE_MIXED_BF16);
  CHECK(zero_step(&h, (void*)A, grads, &stm, 2, nullptr) == ZERO_OK);
  CHECK(zero_step_range(&h, (void*)A, grads, &stm, 2, 8, 800, nullptr) == ZERO_OK);
  CHECK(zero_step_range(&h, (void*)A, grads, &stm, 2, 4, 800, nullptr) == ZERO_EINVAL);
  // step scalars in device memory
  zero_step_scalars sc;
  CHECK(zero_step_scalars_fill(&h, 3, &sc) == ZERO_OK && sc.t == 3);
  const zero_step_scalars* dsc = (const zero_step_scalars*)(A + ((uintptr_t)400 << 24));
  CHECK(zero_step_range_dev(&h, (void*)A, grads, &stm, dsc, 8, 800, nullptr) == ZERO_OK);
  CHECK(zero_step_range_dev(&h, (void*)A, grads, &stm, nullptr, 8, 800, nullptr) == ZERO_EINVAL);
  // buckets in one call, with and without ready events; an invalid bucket enqueues nothing
  {
    const int64_t edges[6] = {400, 800, 0, 400, 800, 1001};  // rank 3 holds 1001 elements
    void* evs[3] = {(void*)(A + 1), nullptr, (void*)(A + 2)};
    const int before_b = g_launches;
    CHECK(zero_step_buckets(&h, (void*)A, grads, &stm, 2, edges, 3, evs, nullptr) == ZERO_OK);
    CHECK(g_launches == before_b + 5);  // 2 waits + 3 launches
    const int64_t bad[4] = {0, 400, 404, 900};  // the second begin is not a multiple of 8
    CHECK(zero_step_buckets(&h, (void*)A, grads, &stm, 2, bad, 2, nullptr, nullptr) == ZERO_EINVAL);
    CHECK(g_launches == before_b + 5);
    CHECK(zero_step_buckets(&h, (void*)A, grads, &stm, 2, nullptr, 1, nullptr, nullptr) == ZERO_EINVAL);
    const int64_t overlap[4] = {0, 400, 392, 500};
    CHECK(zero_step_buckets(&h, (void*)A, grads, &stm, 2, overlap, 2, nullptr, nullptr) == ZERO_EINVAL);
    CHECK(g_launches == before_b + 5);
    CHECK(zero_step_buckets(&h, (void*)A, grads, &stm, 2, edges, -1, nullptr, nullptr) == ZERO_EINVAL);
  }
  // empty shard: nothing launched, pointers may be NULL
  const int before = g_launches;
  h = hp(3, 5, 4, ZERO_MODE_F64);
  CHECK(zero_step(&h, nullptr, nullptr, nullptr, 1, nullptr) == ZERO_OK);
  CHECK(g_launches == before);
  // SGD
  h = hp(1000, 4, -1, ZERO_MODE_F32);
  h.optimizer = ZERO_OPT_SGD;
  h.momentum = 0.9;
  zero_states sts = {nullptr, (void*)(A + (1u << 24)), nullptr};
  CHECK(zero_step(&h, (void*)A, grads, &sts, 1, nullptr) == ZERO_OK);
  CHECK(zero_step_range(&h, (void*)A, grads, &sts, 2, 8, 800, nullptr) == ZERO_OK);
  size_t wsg = 0;
  CHECK(zero_step_clipped_workspace_bytes(&h, &wsg) == ZERO_OK);
  // the SGD state has no v: a workspace at a low address overlaps nothing
  CHECK(zero_step_clipped(&h, (void*)A, grads, &sts, 1, 1.0, nullptr, (void*)(uintptr_t)256, wsg,
                          nullptr) == ZERO_OK);
  h.nesterov = 1;
  h.dampening = 0.5;
  CHECK(zero_step(&h, (void*)A, grads, &sts, 1, nullptr) == ZERO_EINVAL);
  // clipping and mean gradient
  h = hp(100000, 8, -1, ZERO_MODE_F32);
  size_t ws = 0;
  CHECK(zero_step_clipped_workspace_bytes(&h, &ws) == ZERO_OK && ws >= 400000);
  CHECK(zero_step_clipped(&h, (void*)A, grads, &st, 1, 1.0, nullptr, (void*)(A + ((uintptr_t)340 << 24)),
                          ws, nullptr) == ZERO_OK);
  CHECK(zero_step_clipped(&h, (void*)A, grads, &st, 1, NAN, nullptr, (void*)(A + ((uintptr_t)340 << 24)),
                          ws, nullptr) == ZERO_EINVAL);
  size_t mws = 0;
  CHECK(zero_mean_grad_workspace_bytes(&h, &mws) == ZERO_OK);
  CHECK(zero_mean_grad(&h, grads, (void*)(A + ((uintptr_t)350 << 24)), (double*)(A + ((uintptr_t)360 << 24)),
                       (void*)(A + ((uintptr_t)361 << 24)), mws, nullptr) == ZERO_OK);
  CHECK(zero_step_mean(&h, (void*)A, (void*)(A + ((uintptr_t)350 << 24)), &st, 1,
                       (const double*)(A + ((uintptr_t)360 << 24)), 1.0, nullptr) == ZERO_OK);
  // Calls longer than zlaunch::kLaunchElems are enqueued as consecutive
  // launches on offset views: lengths, pointers and mask offsets per piece.
  {
    const int64_t L = zlaunch::kLaunchElems;
    const uintptr_t B = (uintptr_t)1 << 40, S = (uintptr_t)1 << 38;  // 256 GiB apart
    const void* bg[2] = {(const void*)(B + 3 * S), (const void*)(B + 4 * S)};
    zero_states bst = {(void*)(B + 5 * S), (void*)(B + 1 * S), (void*)(B + 2 * S)};
    zero_hparams bh = hp(2 * L + 5, 2, -1, ZERO_MODE_MIXED_BF16);
    bh.weight_decay = 0.1;
    bh.wd_mask = (const uint32_t*)(B + 6 * S);
    g_rec.clear();
    CHECK(zero_step(&bh, (void*)B, bg, &bst, 1, nullptr) == ZERO_OK);
    CHECK(g_rec.size() == 3);
    for (size_t i = 0; i < g_rec.size() && i < 3; ++i) {
      const int64_t off = (int64_t)i * L;
      const Rec& r = g_rec[i];
      CHECK(r.kind == 0 && r.len == (i < 2 ? L : 5) && r.mask_off == off);
      CHECK(r.w == B + 5 * S + 4 * off && r.m == B + 1 * S + 4 * off && r.v == B + 2 * S + 4 * off);
      CHECK(r.out == B + 2 * off && r.g0 == B + 3 * S + 2 * off && r.g1 == B + 4 * S + 2 * off);
    }
    // rank mode: the mask offset is the shard's start plus the piece's offset
    zero_hparams rh = hp(8 * (L + 3) + 1, 8, 3, ZERO_MODE_MIXED_BF16);
    int64_t ra, rb;
    CHECK(zero_shard_bounds(rh.n, 8, 3, &ra, &rb) == ZERO_OK && rb - ra == L + 3);
    rh.weight_decay = 0.1;
    rh.wd_mask = (const uint32_t*)(B + 6 * S);
    const void* rg[8];
    for (int k = 0; k < 8; ++k) rg[k] = (const void*)(B + (8 + k) * S);
    g_rec.clear();
    CHECK(zero_step(&rh, (void*)B, rg, &bst, 1, nullptr) == ZERO_OK);
    CHECK(g_rec.size() == 2);
    if (g_rec.size() == 2) {
      CHECK(g_rec[0].len == L && g_rec[0].mask_off == ra && g_rec[0].out == B + 2 * ra);
      CHECK(g_rec[1].len == 3 && g_rec[1].mask_off == ra + L && g_rec[1].out == B + 2 * (ra + L));
      CHECK(g_rec[1].w == B + 5 * S + 4 * L && g_rec[1].g0 == B + 8 * S + 2 * L);
    }
    // a range: the pieces start at `begin`
    g_rec.clear();
    CHECK(zero_step_range(&bh, (void*)B, bg, &bst, 1, 8, L + 24, nullptr) == ZERO_OK);
    CHECK(g_rec.size() == 2);
    if (g_rec.size() == 2) {
      CHECK(g_rec[0].len == L && g_rec[0].w == B + 5 * S + 4 * 8 && g_rec[0].mask_off == 8);
      CHECK(g_rec[1].len == 16 && g_rec[1].w == B + 5 * S + 4 * (8 + L) &&
            g_rec[1].mask_off == 8 + L);
    }
    // the mean: pieces write their partials back to back, one finalize sums them all
    zero_hparams mh = hp(L + 1, 1, -1, ZERO_MODE_F32);
    size_t mws = 0;
    CHECK(zero_mean_grad_workspace_bytes(&mh, &mws) == ZERO_OK);
    const int64_t p0 = L / 1024 + 1, p1 = 1 / 1024 + 1;  // the stub's mean_partials
    CHECK((int64_t)mws == 8 * (p0 + p1));
    g_rec.clear();
    CHECK(zero_mean_grad(&mh, bg, (void*)(B + 1 * S), (double*)(B + 2 * S), (void*)(B + 5 * S),
                         mws, nullptr) == ZERO_OK);
    CHECK(g_rec.size() == 3);
    if (g_rec.size() == 3) {
      CHECK(g_rec[0].kind == 2 && g_rec[0].len == L && g_rec[0].m == B + 5 * S);
      CHECK(g_rec[1].kind == 2 && g_rec[1].len == 1 && g_rec[1].w == B + 1 * S + 4 * L &&
            g_rec[1].g0 == B + 3 * S + 4 * L && g_rec[1].m == B + 5 * S + 8 * p0);
      CHECK(g_rec[2].kind == 3 && g_rec[2].len == p0 + p1 && g_rec[2].w == B + 5 * S &&
            g_rec[2].out == B + 2 * S);
    }
    CHECK(zero_mean_grad(&mh, bg, (void*)(B + 1 * S), (double*)(B + 2 * S), (void*)(B + 5 * S),
                         mws - 8, nullptr) == ZERO_EINVAL);
    // the clipped step: mean pieces, the finalize, then step pieces from the mean
    zero_states cst = {nullptr, (void*)(B + 1 * S), (void*)(B + 2 * S)};
    size_t cws = 0;
    CHECK(zero_step_clipped_workspace_bytes(&mh, &cws) == ZERO_OK);
    g_rec.clear();
    CHECK(zero_step_clipped(&mh, (void*)(B + 7 * S), bg, &cst, 1, 1.0, nullptr,
                            (void*)(B + 9 * S), cws, nullptr) == ZERO_OK);
    CHECK(g_rec.size() == 5);
    if (g_rec.size() == 5) {
      CHECK(g_rec[0].kind == 2 && g_rec[1].kind == 2 && g_rec[2].kind == 3);
      CHECK(g_rec[3].kind == 1 && g_rec[3].len == L && g_rec[3].g0 == B + 9 * S);
      CHECK(g_rec[4].kind == 1 && g_rec[4].len == 1 && g_rec[4].g0 == B + 9 * S + 4 * L &&
            g_rec[4].w == B + 7 * S + 4 * L);
    }
    // an empty rank shard still writes its (zero) norm: one mean launch, one finalize
    zero_hparams eh = hp(3, 5, 4, ZERO_MODE_F32);
    g_rec.clear();
    CHECK(zero_mean_grad(&eh, nullptr, nullptr, (double*)(B + 2 * S), (void*)(B + 5 * S), 64,
                         nullptr) == ZERO_OK);
    CHECK(g_rec.size() == 2 && g_rec[0].len == 0 && g_rec[1].kind == 3 && g_rec[1].len == 1);
    // the no-alloc mean: the partials go to the library's scratch, looked up only
    // after validation; the same pieces and finalize as with a workspace
    g_rec.clear();
    zlaunch::g_scratch_lookups = 0;
    zero_hparams nh = hp(1 << 20, 2, -1, ZERO_MODE_F32);  // the stub counts 1025 partials
    CHECK(zero_mean_grad_noalloc(&nh, bg, (void*)(B + 1 * S), (double*)(B + 2 * S), nullptr) ==
          ZERO_OK);
    CHECK(zlaunch::g_scratch_lookups == 1 && g_rec.size() == 2);
    if (g_rec.size() == 2) {
      CHECK(g_rec[0].kind == 2 && g_rec[0].m == zlaunch::kFakeScratch && g_rec[0].len == 1 << 20);
      CHECK(g_rec[1].kind == 3 && g_rec[1].w == zlaunch::kFakeScratch && g_rec[1].len == 1025 &&
            g_rec[1].out == B + 2 * S);
    }
    // rejected calls look nothing up and launch nothing
    g_rec.clear();
    zlaunch::g_scratch_lookups = 0;
    CHECK(zero_mean_grad_noalloc(&nh, bg, (void*)(B + 1 * S + 4), (double*)(B + 2 * S),
                                 nullptr) == ZERO_EINVAL);
    zero_hparams huge = hp(zlaunch::kScratchDoubles * 1024 * 2, 1, -1, ZERO_MODE_F32);
    CHECK(zero_mean_grad_noalloc(&huge, bg, (void*)(B + 1 * S), (double*)(B + 2 * S),
                                 nullptr) == ZERO_EINVAL);
    CHECK(zlaunch::g_scratch_lookups == 0 && g_rec.empty());
    // without a squared norm no scratch is needed, whatever the size
    CHECK(zero_mean_grad_noalloc(&huge, bg, (void*)(B + 1 * S), nullptr, nullptr) == ZERO_OK);
    CHECK(zlaunch::g_scratch_lookups == 0);
    // one piece when the call fits one launch
    zero_hparams oh = hp(L, 2, -1, ZERO_MODE_F32);
    g_rec.clear();
    CHECK(zero_step(&oh, (void*)B, bg, &cst, 1, nullptr) == ZERO_OK);
    CHECK(g_rec.size() == 1 && g_rec[0].len == L);
  }

  // NULL everywhere
  CHECK(zero_step(nullptr, nullptr, nullptr, nullptr, 1, nullptr) == ZERO_EINVAL);
  CHECK(zero_init_states(nullptr, nullptr, nullptr, nullptr) == ZERO_EINVAL);
  CHECK(zero_memory_bytes(1, 1, 0, 0, 0, 0, nullptr) == ZERO_EINVAL);

  std::printf("host driver: %d launches reached the stubs, %d failures\n", g_launches, g_fail);
  return g_fail == 0 ? 0 : 1;
}
