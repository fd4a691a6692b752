// Host side of the C ABI declared in include/zero_adam.h: argument validation,
// np.array_split shard bounds, the per-rank memory model and the per-step
// scalars. Touches no HIP API itself; device work goes through zlaunch::.
#include "zero_adam.h"

#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "zero_launch.h"

static_assert(sizeof(zero_step_scalars) == sizeof(zlaunch::DynScalars) &&
                  offsetof(zero_step_scalars, bias2) == offsetof(zlaunch::DynScalars, bias2) &&
                  offsetof(zero_step_scalars, t) == offsetof(zlaunch::DynScalars, t),
              "zero_step_scalars and zlaunch::DynScalars must share one layout");

namespace {

thread_local std::string g_last_error;

// Largest accepted n: 2^56 elements, so that every byte count and address
// range formed from n (at most 32 bytes per element) stays inside int64_t.
constexpr int64_t kMaxN = INT64_C(1) << 56;

zero_status fail(zero_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
zero_status fail(zero_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

zero_status ok() {
  g_last_error.clear();
  return ZERO_OK;
}

// Shard r of np.array_split(np.arange(n), N) ("ZeRO-Sharded Adam Step",
// section "The shards"): q = n / N, rho = n % N; the first rho shards have
// q + 1 elements, so shard r starts at r*q + min(r, rho).
void shard_range(int64_t n, int64_t N, int64_t r, int64_t* a, int64_t* b) {
  const int64_t q = n / N, rho = n % N;
  *a = r * q + (r < rho ? r : rho);
  *b = *a + q + (r < rho ? 1 : 0);
}

// 1 - beta^t in double: the bias correction of step t.
double bias_correction(double beta, int64_t t) { return 1.0 - std::pow(beta, (double)t); }

struct Widths {
  int64_t param, grad, state, optimizer;
};

bool mode_widths(int32_t mode, Widths* w) {
  switch (mode) {
    case ZERO_MODE_F64: *w = {8, 8, 8, 16}; return true;
    case ZERO_MODE_F32: *w = {4, 4, 4, 8}; return true;
    case ZERO_MODE_MIXED_BF16: *w = {2, 2, 4, 12}; return true;
    case ZERO_MODE_MIXED_F16: *w = {2, 2, 4, 12}; return true;
    default: return false;
  }
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  const char* name;
};

bool overlaps(const Range& x, const Range& y) {
  return x.lo < x.hi && y.lo < y.hi && x.lo < y.hi && y.lo < x.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// bf16 or fp16 parameters and gradients with a separate fp32 master
bool mixed_mode(int32_t mode) {
  return mode == ZERO_MODE_MIXED_BF16 || mode == ZERO_MODE_MIXED_F16;
}

// Shared checks of zero_hparams. On success fills the shard range this call
// covers ([a, b): the whole vector in full mode, worker `rank`'s shard in rank
// mode).
zero_status check_hparams(const zero_hparams* hp, bool for_step, Widths* wd, int64_t* a,
                          int64_t* b) {
  if (hp == nullptr) return fail(ZERO_EINVAL, "hparams is NULL");
  if (hp->reserved != 0) return fail(ZERO_EINVAL, "hparams.reserved must be 0");
  if (!mode_widths(hp->mode, wd)) return fail(ZERO_EINVAL, "unknown mode %d", hp->mode);
  if (hp->n < 1) return fail(ZERO_EINVAL, "n must be >= 1 (no parameters), got %lld",
                             (long long)hp->n);
  if (hp->n > kMaxN) return fail(ZERO_EINVAL, "n must be <= 2^56, got %lld", (long long)hp->n);
  if (hp->n_workers < 1 || hp->n_workers > ZERO_MAX_WORKERS)
    return fail(ZERO_EINVAL, "n_workers must be in [1, %d], got %d", ZERO_MAX_WORKERS,
                hp->n_workers);
  if (hp->rank < -1 || hp->rank >= hp->n_workers)
    return fail(ZERO_EINVAL, "rank must be -1 or in [0, %d), got %d", hp->n_workers, hp->rank);
  if (hp->rank >= 0) {
    shard_range(hp->n, hp->n_workers, hp->rank, a, b);
  } else {
    *a = 0;
    *b = hp->n;
  }
  if (hp->optimizer != ZERO_OPT_ADAM && hp->optimizer != ZERO_OPT_SGD)
    return fail(ZERO_EINVAL, "unknown optimizer %d", hp->optimizer);
  if (!for_step) return ZERO_OK;
  if (!std::isfinite(hp->lr)) return fail(ZERO_EINVAL, "lr must be finite");
  if (hp->optimizer == ZERO_OPT_ADAM) {
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0)) return fail(ZERO_EINVAL, "beta1 must be in [0, 1)");
    if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0)) return fail(ZERO_EINVAL, "beta2 must be in [0, 1)");
    if (!(std::isfinite(hp->eps) && hp->eps > 0.0))
      return fail(ZERO_EINVAL, "eps must be finite and > 0");
  } else {
    if (!(std::isfinite(hp->momentum) && hp->momentum >= 0.0))
      return fail(ZERO_EINVAL, "momentum must be finite and >= 0");
    if (!(hp->dampening >= 0.0 && hp->dampening <= 1.0))
      return fail(ZERO_EINVAL, "dampening must be in [0, 1]");
    if (hp->nesterov != 0 && hp->nesterov != 1) return fail(ZERO_EINVAL, "nesterov must be 0 or 1");
    if (hp->nesterov && !(hp->momentum > 0.0 && hp->dampening == 0.0))
      return fail(ZERO_EINVAL, "nesterov needs momentum > 0 and dampening == 0");
  }
  if (!(std::isfinite(hp->weight_decay) && hp->weight_decay >= 0.0))
    return fail(ZERO_EINVAL, "weight_decay must be finite and >= 0");
  if (hp->wd_mask != nullptr && !aligned(hp->wd_mask, 4))
    return fail(ZERO_EINVAL, "wd_mask must be 4-byte aligned");
  return ZERO_OK;
}

// Pointer checks shared by init and step: the state buffers of `len` elements
// and the role of the master pointer per mode.
zero_status check_states(const zero_hparams* hp, const zero_states* st, const Widths& wd) {
  if (st == nullptr) return fail(ZERO_EINVAL, "states is NULL");
  const bool sgd = hp->optimizer == ZERO_OPT_SGD;
  if (st->m == nullptr) return fail(ZERO_EINVAL, "states.m is NULL");
  if (st->v == nullptr && !sgd) return fail(ZERO_EINVAL, "states.v is NULL");
  if (!aligned(st->m, 16) || (st->v != nullptr && !aligned(st->v, 16)))
    return fail(ZERO_EINVAL, "states.m and states.v must be 16-byte aligned");
  const bool need_master = mixed_mode(hp->mode) || hp->rank >= 0;
  if (need_master && st->master == nullptr)
    return fail(ZERO_EINVAL, "states.master is required in mixed mode and in rank mode");
  if (!need_master && st->master != nullptr)
    return fail(ZERO_EINVAL,
                "states.master must be NULL in full fp64/fp32 mode (the parameter is its own "
                "master)");
  if (st->master != nullptr && !aligned(st->master, 16))
    return fail(ZERO_EINVAL, "states.master must be 16-byte aligned");
  (void)wd;
  return ZERO_OK;
}

}  // namespace

extern "C" {

const char* zero_last_error(void) { return g_last_error.c_str(); }

zero_status zero_shard_bounds(int64_t n, int32_t n_workers, int32_t r, int64_t* begin,
                              int64_t* end) {
  if (begin == nullptr || end == nullptr) return fail(ZERO_EINVAL, "begin/end is NULL");
  if (n < 0) return fail(ZERO_EINVAL, "n must be >= 0");
  if (n_workers < 1) return fail(ZERO_EINVAL, "n_workers must be >= 1");
  if (r < 0 || r >= n_workers) return fail(ZERO_EINVAL, "r must be in [0, %d)", n_workers);
  shard_range(n, n_workers, r, begin, end);
  return ok();
}

zero_status zero_memory_bytes(int64_t n, int32_t n_workers, int32_t rank, int32_t stage,
                              int32_t mode, int32_t convention, zero_mem* out) {
  if (out == nullptr) return fail(ZERO_EINVAL, "out is NULL");
  if (n < 1) return fail(ZERO_EINVAL, "n must be >= 1 (no parameters)");
  if (n > kMaxN) return fail(ZERO_EINVAL, "n must be <= 2^56");
  if (n_workers < 1) return fail(ZERO_EINVAL, "n_workers must be >= 1");
  if (rank < 0 || rank >= n_workers) return fail(ZERO_EINVAL, "rank must be in [0, %d)", n_workers);
  if (stage < 0 || stage > 3) return fail(ZERO_EINVAL, "stage must be in [0, 3], got %d", stage);
  Widths w;
  if (!mode_widths(mode, &w)) return fail(ZERO_EINVAL, "unknown mode %d", mode);
  int64_t a, b;
  shard_range(n, n_workers, rank, &a, &b);
  const int64_t c = b - a;
  if (convention == 0) {
    out->params = w.param * (stage >= 3 ? c : n);
    out->grads = w.grad * (stage >= 2 ? c : n);
    out->optimizer = w.optimizer * (stage >= 1 ? c : n);
  } else if (convention == 1) {
    if (mixed_mode(mode))
      return fail(ZERO_EUNSUPPORTED, "convention 1 counts one value width; not for mixed modes");
    const int64_t B = w.param;
    switch (stage) {
      case 0: out->params = B * n; out->grads = B * n; out->optimizer = 2 * B * n; break;
      case 1: out->params = B * n; out->grads = B * n + B * c; out->optimizer = 3 * B * c; break;
      case 2: out->params = B * n; out->grads = B * c; out->optimizer = 3 * B * c; break;
      default: out->params = B * c; out->grads = B * c; out->optimizer = 2 * B * c; break;
    }
  } else {
    return fail(ZERO_EINVAL, "unknown convention %d", convention);
  }
  out->total = out->params + out->grads + out->optimizer;
  return ok();
}

zero_status zero_min_stage(int64_t n, int32_t n_workers, int32_t mode, int64_t activation_bytes,
                           int64_t available_bytes, int32_t* stage) {
  if (stage == nullptr) return fail(ZERO_EINVAL, "stage is NULL");
  if (activation_bytes < 0 || available_bytes < 0)
    return fail(ZERO_EINVAL, "byte counts must be >= 0");
  *stage = -1;
  for (int32_t s = 0; s <= 3; ++s) {
    zero_mem m;
    const zero_status st = zero_memory_bytes(n, n_workers, 0, s, mode, 0, &m);
    if (st != ZERO_OK) return st;
    // m.total + activation_bytes < available_bytes, without overflow
    if (activation_bytes < available_bytes && m.total < available_bytes - activation_bytes) {
      *stage = s;
      break;
    }
  }
  return ok();
}

zero_status zero_init_states(const zero_hparams* hp, const void* param, const zero_states* st,
                             void* stream) {
  Widths wd;
  int64_t a = 0, b = 0;
  zero_status s = check_hparams(hp, false, &wd, &a, &b);
  if (s != ZERO_OK) return s;
  if (b == a) return ok();  // an empty shard: no buffer is touched
  if ((s = check_states(hp, st, wd)) != ZERO_OK) return s;
  if (st->master != nullptr && param == nullptr)
    return fail(ZERO_EINVAL, "param is NULL but a master copy is requested");
  if (param != nullptr && !aligned(param, (uintptr_t)wd.param))
    return fail(ZERO_EINVAL, "param must be aligned to its element size");
  const int64_t len = b - a;
  const Range r_m{(uintptr_t)st->m, (uintptr_t)st->m + (uintptr_t)(len * wd.state), "m"};
  const Range r_v{(uintptr_t)st->v, st->v ? (uintptr_t)st->v + (uintptr_t)(len * wd.state) : 0,
                  "v"};
  const Range r_ms{(uintptr_t)st->master,
                   st->master ? (uintptr_t)st->master + (uintptr_t)(len * wd.state) : 0, "master"};
  const Range r_p{(uintptr_t)param + (uintptr_t)(a * wd.param),
                  param ? (uintptr_t)param + (uintptr_t)(b * wd.param) : 0, "param"};
  const Range written[3] = {r_m, r_v, r_ms};
  const Range all[4] = {r_m, r_v, r_ms, r_p};
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 4; ++j)
      if (i != j && overlaps(written[i], all[j]))
        return fail(ZERO_EINVAL, "%s overlaps %s", written[i].name, all[j].name);
  zlaunch::InitArgs ia;
  ia.mode = hp->mode;
  ia.param = st->master ? static_cast<const char*>(param) + a * wd.param : nullptr;
  ia.master = st->master;
  ia.m = st->m;
  ia.v = st->v;
  ia.len = len;
  const char* err = zlaunch::launch_init(ia, stream);
  if (err) return fail(ZERO_EHIP, "init launch failed: %s", err);
  return ok();
}

}  // extern "C"

namespace {

// Validates one step call and fills the launch arguments. `grads` holds ngp
// device pointers whose elements are gelem bytes (the workers' gradients, or
// the one materialised mean); each holds the call's len elements. Sets *empty
// for an empty rank shard, when nothing is to be launched.
zero_status build_step(const zero_hparams* hp, void* param, const void* const* grads, int ngp,
                       int64_t gelem, const zero_states* st, int64_t t, zlaunch::StepArgs* la,
                       bool* empty, int64_t* a_out, int64_t* b_out) {
  Widths wd;
  int64_t a = 0, b = 0;
  zero_status s = check_hparams(hp, true, &wd, &a, &b);
  if (s != ZERO_OK) return s;
  if (t < 1) return fail(ZERO_EINVAL, "t must be >= 1 (1-based step number), got %lld", (long long)t);
  *empty = b == a;
  *a_out = a;
  *b_out = b;
  if (*empty) return ZERO_OK;  // an empty shard: no buffer is touched
  if ((s = check_states(hp, st, wd)) != ZERO_OK) return s;
  if (param == nullptr) return fail(ZERO_EINVAL, "param is NULL");
  if (grads == nullptr) return fail(ZERO_EINVAL, "grads is NULL");
  const bool rank_mode = hp->rank >= 0;
  if (rank_mode ? !aligned(param, (uintptr_t)wd.param) : !aligned(param, 16))
    return fail(ZERO_EINVAL, rank_mode ? "param must be aligned to its element size"
                                       : "param must be 16-byte aligned");
  for (int k = 0; k < ngp; ++k) {
    if (grads[k] == nullptr) return fail(ZERO_EINVAL, "grads[%d] is NULL", k);
    if (!aligned(grads[k], 16)) return fail(ZERO_EINVAL, "grads[%d] must be 16-byte aligned", k);
  }
  const int64_t len = b - a;
  // Written ranges must not overlap one another or anything read.
  Range written[4];
  int nw = 0;
  written[nw++] = {(uintptr_t)param + (uintptr_t)(a * wd.param),
                   (uintptr_t)param + (uintptr_t)(b * wd.param), "param"};
  written[nw++] = {(uintptr_t)st->m, (uintptr_t)st->m + (uintptr_t)(len * wd.state), "m"};
  const bool adam = hp->optimizer == ZERO_OPT_ADAM;
  if (adam)
    written[nw++] = {(uintptr_t)st->v, (uintptr_t)st->v + (uintptr_t)(len * wd.state), "v"};
  if (st->master)
    written[nw++] = {(uintptr_t)st->master, (uintptr_t)st->master + (uintptr_t)(len * wd.state),
                     "master"};
  for (int i = 0; i < nw; ++i)
    for (int j = i + 1; j < nw; ++j)
      if (overlaps(written[i], written[j]))
        return fail(ZERO_EINVAL, "%s overlaps %s", written[i].name, written[j].name);
  const bool decays = hp->weight_decay != 0.0;
  for (int i = 0; i < nw; ++i) {
    for (int k = 0; k < ngp; ++k) {
      const Range g{(uintptr_t)grads[k], (uintptr_t)grads[k] + (uintptr_t)(len * gelem), "grad"};
      if (overlaps(written[i], g)) return fail(ZERO_EINVAL, "%s overlaps grads[%d]", written[i].name, k);
    }
    if (decays && hp->wd_mask) {
      const Range mk{(uintptr_t)hp->wd_mask,
                     (uintptr_t)hp->wd_mask + (uintptr_t)(((hp->n + 31) / 32) * 4), "wd_mask"};
      if (overlaps(written[i], mk)) return fail(ZERO_EINVAL, "%s overlaps wd_mask", written[i].name);
    }
  }

  *la = zlaunch::StepArgs{};
  la->mode = hp->mode;
  la->n_workers = ngp;
  for (int k = 0; k < ngp; ++k) la->grads[k] = grads[k];
  la->m = st->m;
  la->v = st->v;
  if (rank_mode || mixed_mode(hp->mode)) {
    la->w = st->master;
    la->out = static_cast<char*>(param) + a * wd.param;
  } else {
    la->w = param;  // updated in place: the parameter is its own master
    la->out = nullptr;
  }
  la->len = len;
  la->decay_kind = !decays ? 0 : (hp->wd_mask ? 2 : 1);
  la->mask = decays ? hp->wd_mask : nullptr;
  la->mask_bit_offset = a;
  // Step scalars: formed in double, rounded to the state type by the launch.
  la->beta1 = hp->beta1;
  la->beta2 = hp->beta2;
  la->one_minus_beta1 = 1.0 - hp->beta1;
  la->one_minus_beta2 = 1.0 - hp->beta2;
  la->bias1 = bias_correction(hp->beta1, t);
  la->bias2 = bias_correction(hp->beta2, t);
  la->lr = hp->lr;
  la->eps = hp->eps;
  la->decay_factor = 1.0 - hp->lr * hp->weight_decay;
  la->n_workers_value = (double)ngp;
  la->clip_sumsq = nullptr;
  la->max_norm = 0.0;
  la->optimizer = hp->optimizer;
  la->momentum = hp->momentum;
  la->one_minus_dampening = 1.0 - hp->dampening;
  la->weight_decay = hp->weight_decay;
  la->nesterov = hp->nesterov;
  la->first = t == 1;
  if (adam && (!(la->bias1 > 0.0) || !(la->bias2 > 0.0)))
    return fail(ZERO_EINVAL, "bias correction 1 - beta^t is not positive (beta = 0 is fine; "
                             "check beta and t)");
  return ZERO_OK;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// The ranges a built step launch writes: its master or in-place parameter,
// m, v (NULL for SGD) and the separate gathered output (NULL when in place).
void step_written(const zlaunch::StepArgs& la, const Widths& wd, Range out[4]) {
  const uintptr_t w = (uintptr_t)la.w, m = (uintptr_t)la.m, v = (uintptr_t)la.v,
                  o = (uintptr_t)la.out;
  const uintptr_t sb = (uintptr_t)(la.len * wd.state);
  out[0] = {w, w + sb, "w"};
  out[1] = {m, m + sb, "m"};
  out[2] = {v, v ? v + sb : 0, "v"};
  out[3] = {o, o ? o + (uintptr_t)(la.len * wd.param) : 0, "param"};
}

// A device value of `bytes` bytes that the step kernel reads while it writes
// its outputs must not overlap any of them.
zero_status check_not_written(const zlaunch::StepArgs& la, const Widths& wd, const void* p,
                              size_t bytes, const char* name) {
  Range written[4];
  step_written(la, wd, written);
  const Range r{(uintptr_t)p, (uintptr_t)p + bytes, name};
  for (const Range& x : written)
    if (overlaps(r, x)) return fail(ZERO_EINVAL, "%s overlaps %s", name, x.name);
  return ZERO_OK;
}

// Element widths of hp's mode; only called after the mode has been validated.
Widths range_widths(const zero_hparams* hp) {
  Widths wd{};
  mode_widths(hp->mode, &wd);
  return wd;
}

// Moves a built launch `off` elements forward: the same step on offset views.
// gelem: bytes per element of la->grads.
void offset_step(zlaunch::StepArgs* la, int64_t off, const Widths& wd, int64_t gelem) {
  for (int k = 0; k < la->n_workers; ++k)
    la->grads[k] = static_cast<const char*>(la->grads[k]) + off * gelem;
  la->w = static_cast<char*>(la->w) + off * wd.state;
  la->m = static_cast<char*>(la->m) + off * wd.state;
  if (la->v) la->v = static_cast<char*>(la->v) + off * wd.state;  // NULL for SGD
  if (la->out) la->out = static_cast<char*>(la->out) + off * wd.param;
  if (la->mean_out) la->mean_out = static_cast<char*>(la->mean_out) + off * wd.state;
  la->mask_bit_offset += off;
}

// Enqueues a built step as launches of at most zlaunch::kLaunchElems elements
// each, in order, on consecutive offset views (the step is elementwise, so the
// pieces compute exactly what one launch would).
const char* launch_pieces(const zlaunch::StepArgs& la, const Widths& wd, int64_t gelem,
                          bool from_mean, void* stream) {
  auto one = [&](const zlaunch::StepArgs& x) {
    return from_mean ? zlaunch::launch_step_mean(x, stream) : zlaunch::launch_step(x, stream);
  };
  if (la.len <= zlaunch::kLaunchElems) return one(la);
  for (int64_t off = 0; off < la.len; off += zlaunch::kLaunchElems) {
    zlaunch::StepArgs piece = la;
    offset_step(&piece, off, wd, gelem);
    piece.len = std::min(zlaunch::kLaunchElems, la.len - off);
    if (const char* err = one(piece)) return err;
  }
  return nullptr;
}

// Block partials the mean writes for a range of len, summed over the launches
// the range is split into (at least one launch, also for len == 0).
int64_t partials_count(int mode, int64_t len) {
  int64_t total = 0, off = 0;
  do {
    const int64_t piece = std::min(zlaunch::kLaunchElems, len - off);
    total += zlaunch::mean_partials(mode, piece);
    off += piece;
  } while (off < len);
  return total;
}

// Enqueues the mean of ma's range as launches of at most kLaunchElems
// elements, their partials back to back from ma.partials, then, if sumsq_out,
// the fixed-order sum of all partials_count(mode, len) of them.
const char* launch_mean_pieces(const zlaunch::MeanArgs& ma, const Widths& wd, double* sumsq_out,
                               void* stream) {
  int64_t off = 0, np = 0;
  do {
    zlaunch::MeanArgs piece = ma;
    piece.len = std::min(zlaunch::kLaunchElems, ma.len - off);
    if (off > 0) {
      for (int k = 0; k < ma.n_workers; ++k)
        piece.grads[k] = static_cast<const char*>(ma.grads[k]) + off * wd.grad;
      piece.mean = static_cast<char*>(ma.mean) + off * wd.state;
    }
    piece.partials = ma.partials ? ma.partials + np : nullptr;
    np += zlaunch::mean_partials(ma.mode, piece.len);
    if (const char* err = zlaunch::launch_mean(piece, stream)) return err;
    off += piece.len;
  } while (off < ma.len);
  if (sumsq_out != nullptr) return zlaunch::launch_sumsq_finalize(ma.partials, np, sumsq_out, stream);
  return nullptr;
}

// zero_mean_grad and zero_mean_grad_noalloc: the partial sums of the squared
// norm go to the caller's workspace, or (library_scratch) to the library's
// static device scratch, whose address is looked up only after every argument
// has been validated.
zero_status mean_grad_impl(const zero_hparams* hp, const void* const* grads, void* mean_out,
                           double* sumsq_out, void* workspace, size_t workspace_bytes,
                           bool library_scratch, void* stream) {
  Widths wd;
  int64_t a = 0, b = 0;
  zero_status s = check_hparams(hp, false, &wd, &a, &b);
  if (s != ZERO_OK) return s;
  const int64_t len = b - a;
  const int N = hp->n_workers;
  const int64_t count = partials_count(hp->mode, len);
  const int64_t need = count * 8;
  if (sumsq_out != nullptr) {
    if (!aligned(sumsq_out, 8)) return fail(ZERO_EINVAL, "sumsq_out must be 8-byte aligned");
    if (library_scratch) {
      if (count > zlaunch::kScratchDoubles)
        return fail(ZERO_EINVAL,
                    "%lld elements need %lld partial sums of the squared norm; the library's "
                    "scratch holds %lld (use zero_mean_grad with a workspace)",
                    (long long)len, (long long)count, (long long)zlaunch::kScratchDoubles);
    } else if (workspace == nullptr || !aligned(workspace, 16) ||
               (int64_t)workspace_bytes < need) {
      return fail(ZERO_EINVAL, "workspace must be 16-byte aligned and hold %lld bytes",
                  (long long)need);
    }
  }
  zlaunch::MeanArgs ma{};
  ma.mode = hp->mode;
  ma.n_workers = N;
  ma.len = len;
  ma.n_workers_value = (double)N;
  if (len > 0) {
    if (grads == nullptr) return fail(ZERO_EINVAL, "grads is NULL");
    if (mean_out == nullptr || !aligned(mean_out, 16))
      return fail(ZERO_EINVAL, "mean_out must be non-NULL and 16-byte aligned");
    const Range rm{(uintptr_t)mean_out, (uintptr_t)mean_out + (uintptr_t)(len * wd.state), "mean_out"};
    // the library's scratch is its own static allocation: it overlaps nothing
    const bool ws_used = sumsq_out != nullptr && !library_scratch;
    const Range rw{(uintptr_t)workspace,
                   ws_used ? (uintptr_t)workspace + (uintptr_t)need : (uintptr_t)workspace,
                   "workspace"};
    const Range rs{(uintptr_t)sumsq_out, sumsq_out ? (uintptr_t)sumsq_out + 8 : 0, "sumsq_out"};
    for (int k = 0; k < N; ++k) {
      if (grads[k] == nullptr) return fail(ZERO_EINVAL, "grads[%d] is NULL", k);
      if (!aligned(grads[k], 16)) return fail(ZERO_EINVAL, "grads[%d] must be 16-byte aligned", k);
      const Range g{(uintptr_t)grads[k], (uintptr_t)grads[k] + (uintptr_t)(len * wd.grad), "grad"};
      if (overlaps(rm, g) || overlaps(rw, g) || overlaps(rs, g))
        return fail(ZERO_EINVAL, "an output overlaps grads[%d]", k);
    }
    if (overlaps(rm, rw) || overlaps(rm, rs) || overlaps(rw, rs))
      return fail(ZERO_EINVAL, "mean_out, workspace and sumsq_out must not overlap");
    ma.mean = mean_out;
    for (int k = 0; k < N; ++k) ma.grads[k] = grads[k];
  }
  if (len == 0 && sumsq_out == nullptr) return ok();  // an empty shard: nothing to do
  if (sumsq_out != nullptr) {
    if (library_scratch) {
      double* p = nullptr;
      if (const char* err = zlaunch::scratch_address(stream, &p))
        return fail(ZERO_EHIP, "scratch lookup failed: %s", err);
      ma.partials = p;
    } else {
      ma.partials = static_cast<double*>(workspace);
    }
  }
  const char* err = launch_mean_pieces(ma, wd, sumsq_out, stream);
  if (err) return fail(ZERO_EHIP, "mean launch failed: %s", err);
  return ok();
}

// Validation and launch arguments shared by zero_step_range and
// zero_step_range_dev: the range [begin, end) of the call's index space as
// offset views of the full-length buffers.
zero_status build_range(const zero_hparams* hp, void* param, const void* const* grads,
                        const zero_states* st, int64_t t, int64_t begin, int64_t end,
                        zlaunch::StepArgs* la, bool* nothing) {
  bool empty = false;
  int64_t a, b;
  if (hp == nullptr) return fail(ZERO_EINVAL, "hparams is NULL");
  Widths wd;
  if (!mode_widths(hp->mode, &wd)) return fail(ZERO_EINVAL, "unknown mode %d", hp->mode);
  const int N = hp->n_workers >= 1 && hp->n_workers <= ZERO_MAX_WORKERS ? hp->n_workers : 0;
  zero_status s = build_step(hp, param, grads, N, wd.grad, st, t, la, &empty, &a, &b);
  if (s != ZERO_OK) return s;
  const int64_t len = b - a;
  if (begin < 0 || end < begin || end > len)
    return fail(ZERO_EINVAL, "need 0 <= begin <= end <= %lld, got [%lld, %lld)", (long long)len,
                (long long)begin, (long long)end);
  if (begin % 8 != 0)
    return fail(ZERO_EINVAL, "begin must be a multiple of 8, got %lld", (long long)begin);
  *nothing = empty || begin == end;
  if (*nothing) return ZERO_OK;
  // Elementwise: the sub-range is the same step on offset views.
  offset_step(la, begin, wd, wd.grad);
  la->len = end - begin;
  return ZERO_OK;
}

// Workspace of zero_step_clipped: the mean gradient, the block partials, the
// squared norm.
struct ClipLayout {
  int64_t mean_off, partials_off, sumsq_off, total;
};
ClipLayout clip_layout(int mode, int64_t len, int64_t state_bytes) {
  ClipLayout l;
  l.mean_off = 0;
  l.partials_off = align_up(len * state_bytes, 256);
  l.sumsq_off = l.partials_off + align_up(partials_count(mode, len) * 8, 256);
  l.total = l.sumsq_off + 8;
  return l;
}

zero_status check_max_norm(double max_norm) {
  if (!(std::isfinite(max_norm) && max_norm > 0.0))
    return fail(ZERO_EINVAL, "max_norm must be finite and > 0");
  return ZERO_OK;
}

}  // namespace

extern "C" {

zero_status zero_step(const zero_hparams* hp, void* param, const void* const* grads,
                      const zero_states* st, int64_t t, void* stream) {
  zlaunch::StepArgs la;
  bool empty = false;
  int64_t a, b;
  if (hp == nullptr) return fail(ZERO_EINVAL, "hparams is NULL");
  Widths wd;
  if (!mode_widths(hp->mode, &wd)) return fail(ZERO_EINVAL, "unknown mode %d", hp->mode);
  const int N = hp->n_workers >= 1 && hp->n_workers <= ZERO_MAX_WORKERS ? hp->n_workers : 0;
  zero_status s = build_step(hp, param, grads, N, wd.grad, st, t, &la, &empty, &a, &b);
  if (s != ZERO_OK || empty) return s == ZERO_OK ? ok() : s;
  const char* err = launch_pieces(la, wd, wd.grad, false, stream);
  if (err) return fail(ZERO_EHIP, "step launch failed: %s", err);
  return ok();
}

zero_status zero_step_with_mean(const zero_hparams* hp, void* param, const void* const* grads,
                                const zero_states* st, int64_t t, void* mean_out, void* stream) {
  zlaunch::StepArgs la;
  bool empty = false;
  int64_t a, b;
  if (hp == nullptr) return fail(ZERO_EINVAL, "hparams is NULL");
  Widths wd;
  if (!mode_widths(hp->mode, &wd)) return fail(ZERO_EINVAL, "unknown mode %d", hp->mode);
  const int N = hp->n_workers >= 1 && hp->n_workers <= ZERO_MAX_WORKERS ? hp->n_workers : 0;
  zero_status s = build_step(hp, param, grads, N, wd.grad, st, t, &la, &empty, &a, &b);
  if (s != ZERO_OK || empty) return s == ZERO_OK ? ok() : s;
  if (mean_out == nullptr || !aligned(mean_out, 16))
    return fail(ZERO_EINVAL, "mean_out must be non-NULL and 16-byte aligned");
  const size_t mbytes = (size_t)(la.len * wd.state);
  // the mean is one more written range: it must not overlap the other outputs,
  // the gradients or the decay mask
  if ((s = check_not_written(la, wd, mean_out, mbytes, "mean_out")) != ZERO_OK) return s;
  const Range rm{(uintptr_t)mean_out, (uintptr_t)mean_out + (uintptr_t)mbytes, "mean_out"};
  for (int k = 0; k < N; ++k) {
    const Range g{(uintptr_t)grads[k], (uintptr_t)grads[k] + (uintptr_t)(la.len * wd.grad), "grad"};
    if (overlaps(rm, g)) return fail(ZERO_EINVAL, "mean_out overlaps grads[%d]", k);
  }
  if (la.mask != nullptr) {
    const Range mk{(uintptr_t)hp->wd_mask,
                   (uintptr_t)hp->wd_mask + (uintptr_t)(((hp->n + 31) / 32) * 4), "wd_mask"};
    if (overlaps(rm, mk)) return fail(ZERO_EINVAL, "mean_out overlaps wd_mask");
  }
  la.mean_out = mean_out;
  const char* err = launch_pieces(la, wd, wd.grad, false, stream);
  if (err) return fail(ZERO_EHIP, "step launch failed: %s", err);
  return ok();
}

zero_status zero_step_range(const zero_hparams* hp, void* param, const void* const* grads,
                            const zero_states* st, int64_t t, int64_t begin, int64_t end,
                            void* stream) {
  zlaunch::StepArgs la;
  bool nothing = false;
  zero_status s = build_range(hp, param, grads, st, t, begin, end, &la, &nothing);
  if (s != ZERO_OK || nothing) return s == ZERO_OK ? ok() : s;
  const Widths wd = range_widths(hp);
  const char* err = launch_pieces(la, wd, wd.grad, false, stream);
  if (err) return fail(ZERO_EHIP, "step launch failed: %s", err);
  return ok();
}

zero_status zero_step_buckets(const zero_hparams* hp, void* param, const void* const* grads,
                              const zero_states* st, int64_t t, const int64_t* edges,
                              int32_t nbuckets, void* const* ready_events, void* stream) {
  if (edges == nullptr && nbuckets > 0) return fail(ZERO_EINVAL, "edges is NULL");
  if (nbuckets < 0) return fail(ZERO_EINVAL, "nbuckets must be >= 0, got %d", nbuckets);
  // validate the whole call and every bucket before enqueueing anything
  zlaunch::StepArgs whole;
  bool nothing = false;
  zero_status s = build_range(hp, param, grads, st, t, 0, 0, &whole, &nothing);
  if (s != ZERO_OK) return s;
  int64_t a, b;
  if (hp->rank >= 0) shard_range(hp->n, hp->n_workers, hp->rank, &a, &b);
  else a = 0, b = hp->n;
  const int64_t len = b - a;
  for (int32_t i = 0; i < nbuckets; ++i) {
    const int64_t lo = edges[2 * i], hi = edges[2 * i + 1];
    if (lo < 0 || hi < lo || hi > len)
      return fail(ZERO_EINVAL, "bucket %d: need 0 <= begin <= end <= %lld, got [%lld, %lld)", i,
                  (long long)len, (long long)lo, (long long)hi);
    if (lo % 8 != 0)
      return fail(ZERO_EINVAL, "bucket %d: begin must be a multiple of 8, got %lld", i,
                  (long long)lo);
  }
  {  // disjoint: an element stepped twice would take two updates in one step
    std::vector<std::pair<int64_t, int64_t>> r;
    r.reserve((size_t)nbuckets);
    for (int32_t i = 0; i < nbuckets; ++i)
      if (edges[2 * i + 1] > edges[2 * i]) r.emplace_back(edges[2 * i], edges[2 * i + 1]);
    std::sort(r.begin(), r.end());
    for (size_t i = 1; i < r.size(); ++i)
      if (r[i].first < r[i - 1].second)
        return fail(ZERO_EINVAL, "buckets overlap: [%lld, %lld) and [%lld, %lld)",
                    (long long)r[i - 1].first, (long long)r[i - 1].second, (long long)r[i].first,
                    (long long)r[i].second);
  }
  for (int32_t i = 0; i < nbuckets; ++i) {
    const int64_t lo = edges[2 * i], hi = edges[2 * i + 1];
    if (ready_events != nullptr && ready_events[i] != nullptr) {
      const char* err = zlaunch::stream_wait(stream, ready_events[i]);
      if (err) return fail(ZERO_EHIP, "bucket %d: wait failed: %s", i, err);
    }
    zlaunch::StepArgs la;
    s = build_range(hp, param, grads, st, t, lo, hi, &la, &nothing);
    if (s != ZERO_OK) return s;  // not reached: validated above
    if (nothing) continue;
    const Widths wd = range_widths(hp);
    const char* err = launch_pieces(la, wd, wd.grad, false, stream);
    if (err) return fail(ZERO_EHIP, "bucket %d: step launch failed: %s", i, err);
  }
  return ok();
}

zero_status zero_step_scalars_fill(const zero_hparams* hp, int64_t t, zero_step_scalars* out) {
  Widths wd;
  int64_t a = 0, b = 0;
  if (out == nullptr) return fail(ZERO_EINVAL, "out is NULL");
  zero_status s = check_hparams(hp, true, &wd, &a, &b);
  if (s != ZERO_OK) return s;
  if (t < 1) return fail(ZERO_EINVAL, "t must be >= 1 (1-based step number), got %lld", (long long)t);
  const double b1 = bias_correction(hp->beta1, t), b2 = bias_correction(hp->beta2, t);
  if (hp->optimizer == ZERO_OPT_ADAM && (!(b1 > 0.0) || !(b2 > 0.0)))
    return fail(ZERO_EINVAL, "bias correction 1 - beta^t is not positive (check beta and t)");
  out->bias1 = b1;
  out->bias2 = b2;
  out->t = t;
  return ok();
}

zero_status zero_step_range_dev(const zero_hparams* hp, void* param, const void* const* grads,
                                const zero_states* st, const zero_step_scalars* dev_scalars,
                                int64_t begin, int64_t end, void* stream) {
  zlaunch::StepArgs la;
  bool nothing = false;
  if (dev_scalars == nullptr || !aligned(dev_scalars, 8))
    return fail(ZERO_EINVAL, "dev_scalars must be non-NULL and 8-byte aligned");
  // validated as step 1; the kernel takes the step-dependent values from dev_scalars
  zero_status s = build_range(hp, param, grads, st, 1, begin, end, &la, &nothing);
  if (s != ZERO_OK || nothing) return s == ZERO_OK ? ok() : s;
  Widths wd{};
  if (!mode_widths(hp->mode, &wd)) return fail(ZERO_EINVAL, "unknown mode %d", hp->mode);
  s = check_not_written(la, wd, dev_scalars, sizeof(zero_step_scalars), "dev_scalars");
  if (s != ZERO_OK) return s;
  la.dyn = dev_scalars;
  const char* err = launch_pieces(la, wd, wd.grad, false, stream);
  if (err) return fail(ZERO_EHIP, "step launch failed: %s", err);
  return ok();
}

zero_status zero_mean_grad_workspace_bytes(const zero_hparams* hp, size_t* bytes) {
  Widths wd;
  int64_t a = 0, b = 0;
  if (bytes == nullptr) return fail(ZERO_EINVAL, "bytes is NULL");
  zero_status s = check_hparams(hp, false, &wd, &a, &b);
  if (s != ZERO_OK) return s;
  *bytes = (size_t)(partials_count(hp->mode, b - a) * 8);
  return ok();
}

zero_status zero_mean_grad(const zero_hparams* hp, const void* const* grads, void* mean_out,
                           double* sumsq_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return mean_grad_impl(hp, grads, mean_out, sumsq_out, workspace, workspace_bytes, false, stream);
}

zero_status zero_mean_grad_noalloc(const zero_hparams* hp, const void* const* grads,
                                   void* mean_out, double* sumsq_out, void* stream) {
  return mean_grad_impl(hp, grads, mean_out, sumsq_out, nullptr, 0, true, stream);
}

zero_status zero_step_mean(const zero_hparams* hp, void* param, const void* mean_grad,
                           const zero_states* st, int64_t t, const double* clip_sumsq,
                           double max_norm, void* stream) {
  zlaunch::StepArgs la;
  bool empty = false;
  int64_t a, b;
  if (hp == nullptr) return fail(ZERO_EINVAL, "hparams is NULL");
  Widths wd;
  if (!mode_widths(hp->mode, &wd)) return fail(ZERO_EINVAL, "unknown mode %d", hp->mode);
  if (clip_sumsq != nullptr) {
    zero_status c = check_max_norm(max_norm);
    if (c != ZERO_OK) return c;
    if (!aligned(clip_sumsq, 8)) return fail(ZERO_EINVAL, "clip_sumsq must be 8-byte aligned");
  }
  const void* one[1] = {mean_grad};
  zero_status s = build_step(hp, param, one, 1, wd.state, st, t, &la, &empty, &a, &b);
  if (s != ZERO_OK || empty) return s == ZERO_OK ? ok() : s;
  if (clip_sumsq != nullptr &&
      (s = check_not_written(la, wd, clip_sumsq, sizeof(double), "clip_sumsq")) != ZERO_OK)
    return s;
  la.clip_sumsq = clip_sumsq;
  la.max_norm = max_norm;
  const char* err = launch_pieces(la, wd, wd.state, true, stream);
  if (err) return fail(ZERO_EHIP, "step launch failed: %s", err);
  return ok();
}

zero_status zero_step_clipped_workspace_bytes(const zero_hparams* hp, size_t* bytes) {
  Widths wd;
  int64_t a = 0, b = 0;
  if (bytes == nullptr) return fail(ZERO_EINVAL, "bytes is NULL");
  zero_status s = check_hparams(hp, false, &wd, &a, &b);
  if (s != ZERO_OK) return s;
  *bytes = (size_t)clip_layout(hp->mode, b - a, wd.state).total;
  return ok();
}

zero_status zero_step_clipped(const zero_hparams* hp, void* param, const void* const* grads,
                              const zero_states* st, int64_t t, double max_norm,
                              double* sumsq_out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  zlaunch::StepArgs la;
  bool empty = false;
  int64_t a, b;
  if (hp == nullptr) return fail(ZERO_EINVAL, "hparams is NULL");
  if (hp->rank >= 0)
    return fail(ZERO_EUNSUPPORTED,
                "a clipped step needs every shard's squared norm; in rank mode use "
                "zero_mean_grad, sum the ranks' squared norms, then zero_step_mean");
  Widths wd;
  if (!mode_widths(hp->mode, &wd)) return fail(ZERO_EINVAL, "unknown mode %d", hp->mode);
  zero_status s = check_max_norm(max_norm);
  if (s != ZERO_OK) return s;
  const int N = hp->n_workers >= 1 && hp->n_workers <= ZERO_MAX_WORKERS ? hp->n_workers : 0;
  s = build_step(hp, param, grads, N, wd.grad, st, t, &la, &empty, &a, &b);
  if (s != ZERO_OK) return s;
  const int64_t len = b - a;
  const ClipLayout L = clip_layout(hp->mode, len, wd.state);
  if (workspace == nullptr || !aligned(workspace, 16) || (int64_t)workspace_bytes < L.total)
    return fail(ZERO_EINVAL, "workspace must be 16-byte aligned and hold %lld bytes",
                (long long)L.total);
  if (sumsq_out != nullptr && !aligned(sumsq_out, 8))
    return fail(ZERO_EINVAL, "sumsq_out must be 8-byte aligned");
  // the workspace and sumsq_out must not overlap anything the step reads or writes
  const Range rw{(uintptr_t)workspace, (uintptr_t)workspace + (uintptr_t)L.total, "workspace"};
  const Range rs{(uintptr_t)sumsq_out, sumsq_out ? (uintptr_t)sumsq_out + 8 : 0, "sumsq_out"};
  const Range others[4] = {
      {(uintptr_t)param, (uintptr_t)param + (uintptr_t)(hp->n * wd.param), "param"},
      {(uintptr_t)st->m, (uintptr_t)st->m + (uintptr_t)(len * wd.state), "m"},
      {(uintptr_t)st->v, st->v ? (uintptr_t)st->v + (uintptr_t)(len * wd.state) : 0, "v"},
      {(uintptr_t)st->master, st->master ? (uintptr_t)st->master + (uintptr_t)(len * wd.state) : 0,
       "master"}};
  for (const Range& o : others)
    if (overlaps(rw, o) || overlaps(rs, o)) return fail(ZERO_EINVAL, "workspace/sumsq_out overlaps %s", o.name);
  if (overlaps(rw, rs)) return fail(ZERO_EINVAL, "sumsq_out overlaps the workspace");
  for (int k = 0; k < N; ++k) {
    const Range g{(uintptr_t)grads[k], (uintptr_t)grads[k] + (uintptr_t)(len * wd.grad), "grad"};
    if (overlaps(rw, g) || overlaps(rs, g)) return fail(ZERO_EINVAL, "workspace/sumsq_out overlaps grads[%d]", k);
  }
  if (hp->wd_mask && hp->weight_decay != 0.0) {
    const Range mk{(uintptr_t)hp->wd_mask, (uintptr_t)hp->wd_mask + (uintptr_t)(((hp->n + 31) / 32) * 4), "wd_mask"};
    if (overlaps(rw, mk) || overlaps(rs, mk)) return fail(ZERO_EINVAL, "workspace/sumsq_out overlaps wd_mask");
  }
  char* ws = static_cast<char*>(workspace);
  double* sumsq = sumsq_out ? sumsq_out : reinterpret_cast<double*>(ws + L.sumsq_off);
  zlaunch::MeanArgs ma{};
  ma.mode = hp->mode;
  ma.n_workers = N;
  for (int k = 0; k < N; ++k) ma.grads[k] = grads[k];
  ma.mean = ws + L.mean_off;
  ma.len = len;
  ma.n_workers_value = (double)N;
  ma.partials = reinterpret_cast<double*>(ws + L.partials_off);
  const char* err = launch_mean_pieces(ma, wd, sumsq, stream);
  if (err) return fail(ZERO_EHIP, "mean launch failed: %s", err);
  la.n_workers = 1;
  la.grads[0] = ws + L.mean_off;
  for (int k = 1; k < zlaunch::kMaxWorkers; ++k) la.grads[k] = nullptr;
  la.n_workers_value = 1.0;
  la.clip_sumsq = sumsq;
  la.max_norm = max_norm;
  err = launch_pieces(la, wd, wd.state, true, stream);
  if (err) return fail(ZERO_EHIP, "step launch failed: %s", err);
  return ok();
}

}  // extern "C"
