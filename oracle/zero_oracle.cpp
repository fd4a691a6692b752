// CPU oracle for the ZeRO-sharded Adam step.
//
// TEST INFRASTRUCTURE ONLY. This file is the checker, not the product: only the
// test suite, the smoke check and the CPU-baseline leg of the benchmark may load
// the library built from it. It shares no code, header, table or constant with
// the HIP path (zero_sharded_optimizer_amd/csrc), and neither side includes the
// other.
//
// What it computes, and where that is defined:
//   * "ZeRO-Sharded Adam Step" (scratchllm.com), sections "The step", "The shards",
//     "What to implement", "Requirements": N workers, shard i is
//     np.array_split(np.arange(n), N)[i]; (1) reduce-scatter of the mean gradient,
//     (2) Adam on each shard with that shard's own m and v, (3) all-gather of the
//     updated shards; the outcome must match ordinary Adam over the whole vector
//     driven by the averaged gradient.
//   * "Data parallelism and ZeRO stages 1 to 3" (openlearn L11.3), section
//     "2. Principles" (chunked elementwise update, reduce-scatter then divide by p,
//     the memory table and the emulation's bookkeeping) and section "3. Worked
//     example by hand" (first-step moments m = (1-b1) g, v = (1-b2) g^2 and the
//     byte table).
//   * "Data Parallelism & ZeRO" (pradyotprakash.com), section "ZeRO, stage by
//     stage"; "Data parallelism and ZeRO optimization" (brentwoodlivery.com),
//     sections "Memory Consumption Analysis" and "ZeRO-1/2/3"; "ZeRO One:
//     Sharding the Optimizer" (blog.underfit.ai), sections "Training Memory
//     Requirements", "Sharding Parameters", "Synchronizing Parameters".
//
// Readings where the pages are silent (each is also listed in the design notes):
//   * The Adam formula is not printed (the page treats adam_update as given).
//     Taken as textbook bias-corrected Adam with eps outside the square root,
//     the only form that gives the pages' first step (move by lr against the
//     mean gradient, eps touching the eighth digit).
//   * Weight decay (AdamW with decay is named, no formula): decoupled,
//     multiplicative w <- w * (1 - lr*wd) applied to the pre-update w.
//   * Mean: sum the N worker gradients left to right in rank order, then one
//     division by N.
//   * One fixed operation order per element, every operation a single IEEE
//     round-to-nearest operation in the state type S (double, or float for the
//     fp32 and mixed modes), never fused:
//         gb  = (g_0 + g_1 + ... + g_{N-1}) / N
//         m   = b1*m + (1-b1)*gb
//         v   = b2*v + (1-b2)*(gb*gb)
//         mh  = m / (1-b1^t);  vh = v / (1-b2^t)
//         den = sqrt(vh) + eps
//         w   = w * (1 - lr*wd)            (only where decay applies)
//         w   = w - lr*(mh/den)
//     The step scalars 1-b1, 1-b2, 1-b1^t, 1-b2^t, 1-lr*wd are formed in double
//     and rounded once to S.
//   * bf16 write-back in mixed precision: round to nearest, ties to even; NaN
//     becomes the quiet NaN 0x7FC0.
//   * fp16 mixed precision ("Data parallelism and ZeRO optimization", section
//     "Memory Consumption Analysis": fp16 parameters and gradients, fp32
//     master, momentum and variance): the same step with IEEE binary16
//     parameters and gradients; write-back rounds to nearest, ties to even,
//     with gradual underflow and overflow to infinity; NaN becomes 0x7E00.
//   * Momentum SGD (the other wrapped optimizer of "Data parallelism and ZeRO
//     stages 1 to 3"; no formula printed): torch.optim.SGD's definition with
//     coupled L2 decay, the buffer set to the first step's gradient, optional
//     dampening and Nesterov; see sgd_update.
//   * Global-norm clipping ("Data parallelism and ZeRO stages 1 to 3", section
//     "Going further", which names it as a sum over ranks of the chunks' squared
//     norms before the step, with no formula): each shard's squared norm of its
//     mean gradient, summed in index order in double, then summed over shards
//     in rank order; the factor min(1, max_norm / (sqrt(sum) + 1e-6)) in
//     double, as torch's clip_grad_norm_ defines it, rounded once to S; the
//     mean gradient is multiplied by it before the moments.
//
// Build: g++ -O2 -std=c++17 -ffp-contract=off -fno-fast-math -shared -fPIC.
// Single-threaded and deliberately unfused: every worker materialises its own
// mean-gradient shard and its own m, v and master arrays, as the pages describe.
//
// ORACLE_MUTANT (compile-time, tests only) plants one known mistake so that the
// pin tests can show they catch it; 0 (the default) is the oracle itself.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

namespace {

// ---------------------------------------------------------------------------
// Shards. "ZeRO-Sharded Adam Step", section "The shards": shard r is
// np.array_split(np.arange(n), N)[r]. numpy's rule: the first (n mod N) sections
// hold floor(n/N)+1 indices, the rest floor(n/N); section r starts where the
// sections before it end. Written as that cumulative sum, one shard at a time.
// ---------------------------------------------------------------------------
int64_t section_size(int64_t n, int64_t N, int64_t r) {
  const int64_t each = n / N;
  const int64_t extras = n % N;
  return r < extras ? each + 1 : each;
}

void split_bounds(int64_t n, int64_t N, int64_t r, int64_t* a, int64_t* b) {
  int64_t start = 0;
  for (int64_t k = 0; k < r; ++k) start += section_size(n, N, k);
#if ORACLE_MUTANT == 2
  // planted: a rank beginning at the neighbour's chunk (ignores the extra elements)
  start = r * (n / N);
#endif
  *a = start;
  *b = start + section_size(n, N, r);
}

// ---------------------------------------------------------------------------
// bf16 rounding, from the definition: the two bf16 values that bracket x are the
// truncation of x (towards zero) and the next bf16 value away from zero; take
// the nearer one, and on a tie the one whose last mantissa bit is 0. A value at
// or past the midpoint between the largest finite bf16 and 2^128 rounds to
// infinity, as IEEE overflow does.
// ---------------------------------------------------------------------------
uint32_t float_bits(float x) { uint32_t u; std::memcpy(&u, &x, 4); return u; }
float bits_float(uint32_t u) { float x; std::memcpy(&x, &u, 4); return x; }

uint16_t bf16_round(float x) {
  if (std::isnan(x)) return 0x7FC0;
  if (std::isinf(x)) return (uint16_t)(float_bits(x) >> 16);
  const uint32_t u = float_bits(x);
  const uint32_t lo_bits = u & 0xFFFF0000u;
  const uint32_t hi_bits = lo_bits + 0x10000u;  // next value away from zero
#if ORACLE_MUTANT == 11
  return (uint16_t)(lo_bits >> 16);  // planted: truncation instead of rounding
#endif
  const double xd = std::fabs((double)x);
  const double lo = std::fabs((double)bits_float(lo_bits));
  double hi;
  if ((hi_bits & 0x7FFFFFFFu) == 0x7F800000u)
    hi = std::ldexp(1.0, 128);  // the step past the largest finite value
  else
    hi = std::fabs((double)bits_float(hi_bits));
  const double dlo = xd - lo;
  const double dhi = hi - xd;
  uint32_t pick;
  if (dlo < dhi) pick = lo_bits;
  else if (dhi < dlo) pick = hi_bits;
  else pick = ((lo_bits >> 16) & 1u) ? hi_bits : lo_bits;
  return (uint16_t)(pick >> 16);
}

float bf16_widen(uint16_t h) { return bits_float((uint32_t)h << 16); }

// ---------------------------------------------------------------------------
// IEEE binary16 (fp16), from the definition: 1 sign bit, 5 exponent bits (bias
// 15), 10 fraction bits; exponent field 0 holds the subnormals k * 2^-24
// (k < 1024), field 31 infinity and NaN. The representable magnitudes near a
// value a are a grid of spacing 2^(e-10) in the binade [2^e, 2^(e+1)),
// e in [-14, 15], and of spacing 2^-24 below 2^-14.
// ---------------------------------------------------------------------------
float fp16_widen(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const int f = h & 0x3FF;
  double mag;
  if (e == 0) mag = std::ldexp((double)f, -24);
  else if (e == 31) mag = f ? NAN : INFINITY;
  else mag = std::ldexp((double)(1024 + f), e - 25);
  return (float)((h & 0x8000) ? -mag : mag);
}

// Round to nearest fp16, ties to the value with an even last fraction bit.
// Magnitudes from the midpoint between 65504 and 2^16 upwards overflow to
// infinity, as the grid step past 65504 is 2^16.
uint16_t fp16_round(float x) {
  if (std::isnan(x)) return 0x7E00;
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  if (std::isinf(x)) return sign | 0x7C00;
  const double a = std::fabs((double)x);
  if (a == 0.0) return sign;
  int e2;
  std::frexp(a, &e2);  // a = f * 2^e2, f in [0.5, 1): a is in the binade [2^(e2-1), 2^e2)
  const int binade = e2 - 1 < -14 ? -14 : e2 - 1;
  const double q = std::ldexp(1.0, binade - 10);  // grid spacing around a
  const double k = std::floor(a / q);             // a / q is exact: q is a power of two
  const double dlo = a - k * q, dhi = (k + 1.0) * q - a;
  double r;
#if ORACLE_MUTANT == 19
  r = k;  // planted: truncation instead of rounding
#else
  if (dlo < dhi) r = k;
  else if (dhi < dlo) r = k + 1.0;
  else r = std::fmod(k, 2.0) == 0.0 ? k : k + 1.0;
#endif
  const double v = r * q;
  if (v >= 65536.0) return sign | 0x7C00;
  if (v < std::ldexp(1.0, -14)) return sign | (uint16_t)(v / std::ldexp(1.0, -24));
  int ev;
  std::frexp(v, &ev);  // v in [2^(ev-1), 2^ev)
  const int field = ev - 1 + 15;
  const uint16_t frac = (uint16_t)(v / std::ldexp(1.0, ev - 1 - 10) - 1024.0);
  return sign | (uint16_t)(field << 10) | frac;
}

// ---------------------------------------------------------------------------
// Per-step scalars, formed in double and rounded once to S.
// ---------------------------------------------------------------------------
template <class S>
struct StepConsts {
  S beta1, beta2, one_minus_beta1, one_minus_beta2, bias1, bias2, lr, eps, decay;
};

template <class S>
StepConsts<S> step_consts(double lr, double beta1, double beta2, double eps,
                          double wd, int64_t t) {
  StepConsts<S> c;
#if ORACLE_MUTANT == 10
  lr = 1e-2;  // planted: the optimizer's default lr instead of the caller's
#endif
  double tt = (double)t;
#if ORACLE_MUTANT == 14
  tt = (double)(t + 1);  // planted: off-by-one step count in the bias correction
#endif
  c.beta1 = (S)beta1;
  c.beta2 = (S)beta2;
  c.one_minus_beta1 = (S)(1.0 - beta1);
  c.one_minus_beta2 = (S)(1.0 - beta2);
  c.bias1 = (S)(1.0 - std::pow(beta1, tt));
  c.bias2 = (S)(1.0 - std::pow(beta2, tt));
  c.lr = (S)lr;
  c.eps = (S)eps;
  c.decay = (S)(1.0 - lr * wd);
#if ORACLE_MUTANT == 4
  // planted: the two betas exchanged everywhere
  std::swap(c.beta1, c.beta2);
  std::swap(c.one_minus_beta1, c.one_minus_beta2);
  std::swap(c.bias1, c.bias2);
#endif
  return c;
}

inline float oracle_sqrt(float x) { return std::sqrt(x); }
inline double oracle_sqrt(double x) { return std::sqrt(x); }

// ---------------------------------------------------------------------------
// adam_update: one Adam (or AdamW) step on one array, in place.
// "ZeRO-Sharded Adam Step", section "What to implement" names this routine
// without printing it; the formula is the reading stated at the top of the
// file. decay[i] != 0 selects decoupled weight decay for element i
// ("Data parallelism and ZeRO stages 1 to 3", section "4. The interface" and
// its test catalog, whose differential test runs AdamW with weight decay).
// ---------------------------------------------------------------------------
template <class S>
void adam_update(S* w, const S* g, S* m, S* v, int64_t len,
                 const StepConsts<S>& c, const uint8_t* decay, S wd_raw) {
  for (int64_t i = 0; i < len; ++i) {
#if ORACLE_MUTANT == 7
    // planted: coupled L2 decay, wd*w folded into the gradient before the moments
    const S gi = (decay == nullptr || decay[i] != 0) ? g[i] + wd_raw * w[i] : g[i];
#else
    const S gi = g[i];
#endif
    S b1m = c.beta1 * m[i];
    S gterm = c.one_minus_beta1 * gi;
    const S mi = b1m + gterm;
    S gsq = gi * gi;
    S b2v = c.beta2 * v[i];
    S g2term = c.one_minus_beta2 * gsq;
    const S vi = b2v + g2term;
    S mh = mi / c.bias1;
#if ORACLE_MUTANT == 5
    S vh = vi;  // planted: bias correction of v dropped
#else
    S vh = vi / c.bias2;
#endif
#if ORACLE_MUTANT == 6
    S den = oracle_sqrt(vh + c.eps);  // planted: eps inside the square root
#else
    S den = oracle_sqrt(vh) + c.eps;
#endif
    S wi = w[i];
    const bool dec = decay == nullptr ? true : decay[i] != 0;
#if ORACLE_MUTANT == 12
    const bool use_decay = !dec;  // planted: decay mask inverted
#else
    const bool use_decay = dec;
#endif
#if ORACLE_MUTANT == 7
    (void)use_decay;
#else
    (void)wd_raw;
    if (use_decay) wi = wi * c.decay;
#endif
    S ratio = mh / den;
    S upd = c.lr * ratio;
#if ORACLE_MUTANT == 8
    wi = wi + upd;  // planted: step along the gradient
#else
    wi = wi - upd;
#endif
    w[i] = wi;
    m[i] = mi;
    v[i] = vi;
  }
}

// ---------------------------------------------------------------------------
// Momentum SGD ("Data parallelism and ZeRO stages 1 to 3": the wrapped
// optimizers are M10.2 SGD and M10.3 AdamW; the DDP tests run momentum-SGD
// steps; no formula is printed). Reading: torch.optim.SGD's definition, in S:
//   d = g;  where decay applies: d = d + wd*w         (coupled L2 decay)
//   if momentum != 0:
//     buf = d at the first step (t == 1), else buf = momentum*buf + (1-dampening)*d
//     d = nesterov ? d + momentum*buf : buf
//   w = w - lr*d
// The momentum buffer is the m state array; v is not used.
// ---------------------------------------------------------------------------
struct OptSel {
  int kind;  // 0: Adam/AdamW, 1: momentum SGD
  double momentum, dampening;
  int nesterov;
};
const OptSel kAdam = {0, 0.0, 0.0, 0};

template <class S>
void sgd_update(S* w, const S* g, S* buf, int64_t len, int64_t t, double lr_d, double wd_d,
                const OptSel& o, const uint8_t* decay) {
  const S lr = (S)lr_d, wd = (S)wd_d, mom = (S)o.momentum;
  const S one_minus_damp = (S)(1.0 - o.dampening);
  for (int64_t i = 0; i < len; ++i) {
    S d = g[i];
    const bool dec = decay == nullptr ? true : decay[i] != 0;
#if ORACLE_MUTANT == 18
    if (wd_d != 0.0 && dec) w[i] = w[i] * (S)(1.0 - lr_d * wd_d);  // planted: decoupled decay
#else
    if (wd_d != 0.0 && dec) {
      const S dw = wd * w[i];
      d = d + dw;
    }
#endif
    if (o.momentum != 0.0) {
      S b;
#if ORACLE_MUTANT == 17
      if (false) {  // planted: the buffer starts at zero instead of the first gradient
#else
      if (t == 1) {
#endif
        b = d;
      } else {
        const S kept = mom * buf[i];
        const S added = one_minus_damp * d;
        b = kept + added;
      }
      buf[i] = b;
      if (o.nesterov) {
        const S nb = mom * b;
        d = d + nb;
      } else {
        d = b;
      }
    }
    const S step = lr * d;
    w[i] = w[i] - step;
  }
}

template <class S>
void opt_update(S* w, const S* g, S* m, S* v, int64_t len, const StepConsts<S>& c,
                const uint8_t* decay, S wd_raw, const OptSel& o, int64_t t, double lr,
                double wd) {
  if (o.kind == 0) adam_update<S>(w, g, m, v, len, c, decay, wd_raw);
  else sgd_update<S>(w, g, m, len, t, lr, wd, o, decay);
}

// Element access by mode. mode 0: fp64 everywhere. mode 1: fp32 everywhere.
// mode 2: bf16 gradients and gathered parameters, fp32 master/m/v. mode 3: the
// same with fp16 in place of bf16.
enum { MODE_F64 = 0, MODE_F32 = 1, MODE_MIXED = 2, MODE_MIXED_F16 = 3 };

bool is_mixed(int mode) { return mode == MODE_MIXED || mode == MODE_MIXED_F16; }

template <class S>
S load_grad(const void* g, int64_t i, int mode) {
  if (mode == MODE_F64) return (S)((const double*)g)[i];
  if (mode == MODE_F32) return (S)((const float*)g)[i];
  if (mode == MODE_MIXED_F16) return (S)fp16_widen(((const uint16_t*)g)[i]);
  return (S)bf16_widen(((const uint16_t*)g)[i]);
}

// The gathered parameter value written back for a master value w.
template <class S>
void store_param(void* p, int64_t i, S w, int mode) {
  if (mode == MODE_F64) ((double*)p)[i] = (double)w;
  else if (mode == MODE_F32) ((float*)p)[i] = (float)w;
  else if (mode == MODE_MIXED_F16) ((uint16_t*)p)[i] = fp16_round((float)w);
  else ((uint16_t*)p)[i] = bf16_round((float)w);
}

// Master value of gathered parameter i: the parameter itself in fp64/fp32 mode,
// or the separate fp32 master copy in mixed mode.
template <class S>
S load_master(const void* param, const void* master, int64_t i, int mode) {
  if (is_mixed(mode)) return ((const float*)master)[i];
  if (mode == MODE_F64) return (S)((const double*)param)[i];
  return (S)((const float*)param)[i];
}

// ---------------------------------------------------------------------------
// The reduce-scatter mean for one shard [a, b): worker r receives, for its
// indices only, the mean over all N workers' gradients ("ZeRO-Sharded Adam
// Step", section "The step", item 1; "Data parallelism and ZeRO stages 1 to 3",
// section "2. Principles", stage 2: reduce_scatter, then divide by p).
// grads[k] is indexed by offset + i for i in [a, b).
// ---------------------------------------------------------------------------
template <class S>
std::vector<S> reduce_scatter_mean(const void* const* grads, int64_t N, int64_t a,
                                   int64_t b, int64_t offset, int mode) {
  std::vector<S> out((size_t)(b - a));
  for (int64_t i = a; i < b; ++i) {
    S s = load_grad<S>(grads[0], i - offset, mode);
    for (int64_t k = 1; k < N; ++k) s = s + load_grad<S>(grads[k], i - offset, mode);
#if ORACLE_MUTANT == 1
    out[(size_t)(i - a)] = s;  // planted: sum without dividing by N
#else
    out[(size_t)(i - a)] = s / (S)N;
#endif
  }
  return out;
}

// ---------------------------------------------------------------------------
// The sharded step, all N workers in one process ("ZeRO-Sharded Adam Step",
// sections "The step" and "What to implement"; a loop over the workers is
// allowed there). Functional: inputs are not modified; the new gathered
// parameters and the new (concatenated) per-worker states are written to the
// *_out arrays. m_in/v_in/master_in hold the N workers' shards back to back,
// worker r's shard at [a_r, b_r).
// ---------------------------------------------------------------------------
template <class S>
void sharded_step(int mode, int64_t n, int64_t N, const void* param_in,
                  const void* const* grads, const void* master_in, const S* m_in,
                  const S* v_in, void* param_out, void* master_out, S* m_out,
                  S* v_out, int64_t t, double lr, double b1, double b2, double eps,
                  double wd, const uint8_t* decay, const OptSel& o = kAdam) {
  const StepConsts<S> c = step_consts<S>(lr, b1, b2, eps, wd, t);
  // Start the all-gather target from the old parameters; every element is
  // overwritten below by the worker that owns it.
  const size_t pbytes = mode == MODE_F64 ? 8 : (mode == MODE_F32 ? 4 : 2);
  std::memcpy(param_out, param_in, (size_t)n * pbytes);
  for (int64_t r = 0; r < N; ++r) {
    int64_t a, b;
    split_bounds(n, N, r, &a, &b);
    const int64_t len = b - a;
    // (1) this worker's reduce-scatter output
    std::vector<S> gbar = reduce_scatter_mean<S>(grads, N, a, b, 0, mode);
    // this worker's own state arrays, the size of its shard
    std::vector<S> w(len), m(len), v(len);
    std::vector<uint8_t> dec;
    for (int64_t j = 0; j < len; ++j) {
      w[j] = load_master<S>(param_in, master_in, a + j, mode);
      m[j] = m_in[a + j];
      v[j] = v_in[a + j];
    }
    if (decay) dec.assign(decay + a, decay + b);
    // (2) Adam on the shard only
    opt_update<S>(w.data(), gbar.data(), m.data(), v.data(), len, c,
                  decay ? dec.data() : nullptr, (S)wd, o, t, lr, wd);
    // (3) all-gather: the shard lands in every worker's full vector; with one
    // shared vector that is one write per element.
#if ORACLE_MUTANT == 3
    if (r > 0) continue;  // planted: no all-gather of the other workers' chunks
#endif
    for (int64_t j = 0; j < len; ++j) {
      store_param<S>(param_out, a + j, w[j], mode);
      if (is_mixed(mode)) ((float*)master_out)[a + j] = (float)w[j];
      m_out[a + j] = m[j];
      v_out[a + j] = v[j];
    }
  }
}

// ---------------------------------------------------------------------------
// Shard-free reference: ordinary Adam over the whole vector driven by the
// averaged gradient ("ZeRO-Sharded Adam Step", section "Requirements", first item).
// ---------------------------------------------------------------------------
template <class S>
void full_step(int mode, int64_t n, int64_t N, const void* param_in,
               const void* const* grads, const void* master_in, const S* m_in,
               const S* v_in, void* param_out, void* master_out, S* m_out,
               S* v_out, int64_t t, double lr, double b1, double b2, double eps,
               double wd, const uint8_t* decay, const OptSel& o = kAdam) {
  const StepConsts<S> c = step_consts<S>(lr, b1, b2, eps, wd, t);
  std::vector<S> gbar((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    S s = load_grad<S>(grads[0], i, mode);
    for (int64_t k = 1; k < N; ++k) s = s + load_grad<S>(grads[k], i, mode);
    gbar[(size_t)i] = s / (S)N;
  }
  std::vector<S> w((size_t)n), m(m_in, m_in + n), v(v_in, v_in + n);
  for (int64_t i = 0; i < n; ++i) w[(size_t)i] = load_master<S>(param_in, master_in, i, mode);
  opt_update<S>(w.data(), gbar.data(), m.data(), v.data(), n, c, decay, (S)wd, o, t, lr, wd);
  for (int64_t i = 0; i < n; ++i) {
    store_param<S>(param_out, i, w[(size_t)i], mode);
    if (is_mixed(mode)) ((float*)master_out)[i] = (float)w[(size_t)i];
    m_out[i] = m[(size_t)i];
    v_out[i] = v[(size_t)i];
  }
}

// ---------------------------------------------------------------------------
// One worker's share (ZeRO stage 2 seen from rank r; "Data parallelism and
// ZeRO stages 1 to 3", section "2. Principles", stage 2): rank r holds only
// its chunk [a_r, b_r) of master, m and v, receives from every worker k the
// chunk g_k[a_r:b_r) (a length-c_r buffer), and writes its updated chunk into
// the full gathered parameter vector. Elements outside [a_r, b_r) are copied
// unchanged from param_in.
// ---------------------------------------------------------------------------
template <class S>
void rank_step(int mode, int64_t n, int64_t N, int64_t r, const void* param_in,
               const void* const* chunk_grads, const S* master_in, const S* m_in,
               const S* v_in, void* param_out, S* master_out, S* m_out, S* v_out,
               int64_t t, double lr, double b1, double b2, double eps, double wd,
               const uint8_t* decay, const OptSel& o = kAdam) {
  const StepConsts<S> c = step_consts<S>(lr, b1, b2, eps, wd, t);
  int64_t a, b;
  split_bounds(n, N, r, &a, &b);
  const int64_t len = b - a;
  const size_t pbytes = mode == MODE_F64 ? 8 : (mode == MODE_F32 ? 4 : 2);
  std::memcpy(param_out, param_in, (size_t)n * pbytes);
  std::vector<S> gbar = reduce_scatter_mean<S>(chunk_grads, N, a, b, a, mode);
  std::vector<S> w(master_in, master_in + len), m(m_in, m_in + len), v(v_in, v_in + len);
  std::vector<uint8_t> dec;
  if (decay) dec.assign(decay + a, decay + b);
  opt_update<S>(w.data(), gbar.data(), m.data(), v.data(), len, c,
                decay ? dec.data() : nullptr, (S)wd, o, t, lr, wd);
  for (int64_t j = 0; j < len; ++j) {
    store_param<S>(param_out, a + j, w[(size_t)j], mode);
    master_out[j] = w[(size_t)j];
    m_out[j] = m[(size_t)j];
    v_out[j] = v[(size_t)j];
  }
}

// ---------------------------------------------------------------------------
// Squared norm of one shard's mean gradient, summed in index order in double.
// "Data parallelism and ZeRO stages 1 to 3", section "Going further" names
// sharded global-norm clipping: a sum over ranks of each chunk's squared norm,
// taken before the update.
// ---------------------------------------------------------------------------
template <class S>
double shard_sumsq(const std::vector<S>& g) {
  double acc = 0.0;
  for (const S x : g) {
    const double d = (double)x;
#if ORACLE_MUTANT == 16
    acc = acc + (d < 0 ? -d : d);  // planted: a 1-norm instead of squares
#else
    acc = acc + d * d;
#endif
  }
  return acc;
}

// The reduce-scatter mean of every shard in the call's range, materialised
// (stage 1 keeps the averaged gradient: "2. Principles", "Your emulation's
// bookkeeping"). Full mode (r < 0): all N shards, mean_out holds n values and
// *sumsq_out the sum over shards, in rank order, of each shard's squared norm
// (the all-reduce). Rank mode: worker r's shard from chunk gradients; mean_out
// holds c_r values and *sumsq_out that shard's squared norm alone.
template <class S>
void mean_grad(int mode, int64_t n, int64_t N, int64_t r, const void* const* grads,
               S* mean_out, double* sumsq_out) {
  double total = 0.0;
  const int64_t r0 = r < 0 ? 0 : r, r1 = r < 0 ? N : r + 1;
  for (int64_t k = r0; k < r1; ++k) {
    int64_t a, b;
    split_bounds(n, N, k, &a, &b);
    const int64_t base = r < 0 ? 0 : a;  // chunk buffers start at the shard
    std::vector<S> gbar = reduce_scatter_mean<S>(grads, N, a, b, base, mode);
    for (int64_t j = a; j < b; ++j) mean_out[j - base] = gbar[(size_t)(j - a)];
    total = total + shard_sumsq<S>(gbar);
  }
  if (sumsq_out) *sumsq_out = total;
}

// The clipping factor from the global squared norm, as torch's
// clip_grad_norm_ (the production equivalent the openlearn page names)
// defines it: min(1, max_norm / (norm + 1e-6)), in double, where the clamp at
// 1 lets a NaN through (a NaN norm makes every clipped gradient NaN).
double clip_factor(double sumsq, double max_norm) {
#if ORACLE_MUTANT == 15
  return max_norm / (std::sqrt(sumsq) + 1e-6);  // planted: no clamp at 1
#else
  const double c = max_norm / (std::sqrt(sumsq) + 1e-6);
#if ORACLE_MUTANT != 20  // planted (20): a NaN factor clamped to 1
  if (std::isnan(c)) return c;
#endif
  return c < 1.0 ? c : 1.0;
#endif
}

// Adam driven by a materialised mean gradient: every shard in the call's range
// steps with its own state, the mean gradient optionally scaled by the clipping
// factor (rounded once to S) before the moments.
template <class S>
void step_from_mean(int mode, int64_t n, int64_t N, int64_t r, const void* param_in,
                    const S* mean, const void* master_in, const S* m_in, const S* v_in,
                    void* param_out, void* master_out, S* m_out, S* v_out, int64_t t,
                    double lr, double b1, double b2, double eps, double wd,
                    const uint8_t* decay, const double* clip_sumsq, double max_norm,
                    const OptSel& o = kAdam) {
  const StepConsts<S> c = step_consts<S>(lr, b1, b2, eps, wd, t);
  const bool clip = clip_sumsq != nullptr;
  const S coef = clip ? (S)clip_factor(*clip_sumsq, max_norm) : (S)1;
  const size_t pbytes = mode == MODE_F64 ? 8 : (mode == MODE_F32 ? 4 : 2);
  std::memcpy(param_out, param_in, (size_t)n * pbytes);
  const int64_t r0 = r < 0 ? 0 : r, r1 = r < 0 ? N : r + 1;
  for (int64_t k = r0; k < r1; ++k) {
    int64_t a, b;
    split_bounds(n, N, k, &a, &b);
    const int64_t len = b - a;
    const int64_t base = r < 0 ? 0 : a;  // index of element a in mean/states
    std::vector<S> g(len), w(len), m(len), v(len);
    std::vector<uint8_t> dec;
    for (int64_t j = 0; j < len; ++j) {
      g[j] = mean[a - base + j];
      if (clip) g[j] = g[j] * coef;
      if (r < 0) w[j] = load_master<S>(param_in, master_in, a + j, mode);
      else w[j] = ((const S*)master_in)[j];
      m[j] = m_in[a - base + j];
      v[j] = v_in[a - base + j];
    }
    if (decay) dec.assign(decay + a, decay + b);
    opt_update<S>(w.data(), g.data(), m.data(), v.data(), len, c,
                  decay ? dec.data() : nullptr, (S)wd, o, t, lr, wd);
    for (int64_t j = 0; j < len; ++j) {
      store_param<S>(param_out, a + j, w[(size_t)j], mode);
      if (r >= 0) ((S*)master_out)[j] = w[(size_t)j];
      else if (is_mixed(mode)) ((float*)master_out)[a + j] = (float)w[(size_t)j];
      m_out[a - base + j] = m[(size_t)j];
      v_out[a - base + j] = v[(size_t)j];
    }
  }
}

}  // namespace

extern "C" {

int orc_mutant(void) { return ORACLE_MUTANT; }

// np.array_split bounds of shard r.
void orc_split_bounds(int64_t n, int64_t N, int64_t r, int64_t* a, int64_t* b) {
  split_bounds(n, N, r, a, b);
}

// Owner of index i, by the closed form of "ZeRO One: Sharding the Optimizer",
// section "Synchronizing Parameters": with q = floor(n/N) and rho = n mod N,
// indices below (q+1)*rho belong to i/(q+1), the rest to (i-rho)/q.
int64_t orc_owner(int64_t n, int64_t N, int64_t i) {
  const int64_t q = n / N, rho = n % N;
  if (i < (q + 1) * rho) return i / (q + 1);
  return (i - rho) / q;
}

// bf16 rounding of each of len floats.
void orc_bf16_round(const float* x, uint16_t* out, int64_t len) {
  for (int64_t i = 0; i < len; ++i) out[i] = bf16_round(x[i]);
}

// fp16 rounding of each of len floats, and the exact widening back.
void orc_fp16_round(const float* x, uint16_t* out, int64_t len) {
  for (int64_t i = 0; i < len; ++i) out[i] = fp16_round(x[i]);
}
void orc_fp16_widen(const uint16_t* h, float* out, int64_t len) {
  for (int64_t i = 0; i < len; ++i) out[i] = fp16_widen(h[i]);
}

// init_states ("ZeRO-Sharded Adam Step", section "What to implement"): m and v
// of zeros; in mixed mode the fp32 master is the exact widening of the bf16
// parameters. len elements (full n, or one shard).
void orc_init_states(int mode, int64_t len, const void* param, void* master,
                     void* m, void* v) {
  const size_t s = mode == MODE_F64 ? 8 : 4;
  std::memset(m, 0, (size_t)len * s);
  std::memset(v, 0, (size_t)len * s);
  if (is_mixed(mode) && master) {
    for (int64_t i = 0; i < len; ++i)
      ((float*)master)[i] = mode == MODE_MIXED_F16 ? fp16_widen(((const uint16_t*)param)[i])
                                                   : bf16_widen(((const uint16_t*)param)[i]);
  }
}

// The sharded step (all N workers). Returns 0, or -1 on a bad argument.
int orc_zero_step(int mode, int64_t n, int64_t N, const void* param_in,
                  const void* const* grads, const void* master_in, const void* m_in,
                  const void* v_in, void* param_out, void* master_out, void* m_out,
                  void* v_out, int64_t t, double lr, double b1, double b2,
                  double eps, double wd, const uint8_t* decay) {
  if (n < 0 || N < 1 || t < 1) return -1;
  if (mode == MODE_F64)
    sharded_step<double>(mode, n, N, param_in, grads, master_in, (const double*)m_in,
                         (const double*)v_in, param_out, master_out, (double*)m_out,
                         (double*)v_out, t, lr, b1, b2, eps, wd, decay);
  else if (mode == MODE_F32 || is_mixed(mode))
    sharded_step<float>(mode, n, N, param_in, grads, master_in, (const float*)m_in,
                        (const float*)v_in, param_out, master_out, (float*)m_out,
                        (float*)v_out, t, lr, b1, b2, eps, wd, decay);
  else
    return -1;
  return 0;
}

// The shard-free reference (plain Adam on the full vector, mean gradient).
int orc_full_step(int mode, int64_t n, int64_t N, const void* param_in,
                  const void* const* grads, const void* master_in, const void* m_in,
                  const void* v_in, void* param_out, void* master_out, void* m_out,
                  void* v_out, int64_t t, double lr, double b1, double b2,
                  double eps, double wd, const uint8_t* decay) {
  if (n < 0 || N < 1 || t < 1) return -1;
  if (mode == MODE_F64)
    full_step<double>(mode, n, N, param_in, grads, master_in, (const double*)m_in,
                      (const double*)v_in, param_out, master_out, (double*)m_out,
                      (double*)v_out, t, lr, b1, b2, eps, wd, decay);
  else if (mode == MODE_F32 || is_mixed(mode))
    full_step<float>(mode, n, N, param_in, grads, master_in, (const float*)m_in,
                     (const float*)v_in, param_out, master_out, (float*)m_out,
                     (float*)v_out, t, lr, b1, b2, eps, wd, decay);
  else
    return -1;
  return 0;
}

// One worker's share: chunk gradients of length c_r, shard-local states.
// decay (nullable) is indexed by the global parameter index.
int orc_rank_step(int mode, int64_t n, int64_t N, int64_t r, const void* param_in,
                  const void* const* chunk_grads, const void* master_in,
                  const void* m_in, const void* v_in, void* param_out,
                  void* master_out, void* m_out, void* v_out, int64_t t, double lr,
                  double b1, double b2, double eps, double wd, const uint8_t* decay) {
  if (n < 0 || N < 1 || r < 0 || r >= N || t < 1) return -1;
  if (mode == MODE_F64)
    rank_step<double>(mode, n, N, r, param_in, chunk_grads, (const double*)master_in,
                      (const double*)m_in, (const double*)v_in, param_out,
                      (double*)master_out, (double*)m_out, (double*)v_out, t, lr, b1,
                      b2, eps, wd, decay);
  else if (mode == MODE_F32 || is_mixed(mode))
    rank_step<float>(mode, n, N, r, param_in, chunk_grads, (const float*)master_in,
                     (const float*)m_in, (const float*)v_in, param_out,
                     (float*)master_out, (float*)m_out, (float*)v_out, t, lr, b1, b2,
                     eps, wd, decay);
  else
    return -1;
  return 0;
}

// Materialised reduce-scatter mean (and the squared norm, if sumsq_out).
// rank < 0: full mode; else rank mode with chunk gradients.
int orc_mean_grad(int mode, int64_t n, int64_t N, int64_t rank, const void* const* grads,
                  void* mean_out, double* sumsq_out) {
  if (n < 0 || N < 1 || rank >= N) return -1;
  if (mode == MODE_F64)
    mean_grad<double>(mode, n, N, rank, grads, (double*)mean_out, sumsq_out);
  else if (mode == MODE_F32 || is_mixed(mode))
    mean_grad<float>(mode, n, N, rank, grads, (float*)mean_out, sumsq_out);
  else
    return -1;
  return 0;
}

// The step from a materialised mean gradient; clip_sumsq (nullable) is the
// global squared norm that sets the clipping factor.
int orc_step_mean(int mode, int64_t n, int64_t N, int64_t rank, const void* param_in,
                  const void* mean, const void* master_in, const void* m_in, const void* v_in,
                  void* param_out, void* master_out, void* m_out, void* v_out, int64_t t,
                  double lr, double b1, double b2, double eps, double wd, const uint8_t* decay,
                  const double* clip_sumsq, double max_norm) {
  if (n < 0 || N < 1 || rank >= N || t < 1) return -1;
  if (mode == MODE_F64)
    step_from_mean<double>(mode, n, N, rank, param_in, (const double*)mean, master_in,
                           (const double*)m_in, (const double*)v_in, param_out, master_out,
                           (double*)m_out, (double*)v_out, t, lr, b1, b2, eps, wd, decay,
                           clip_sumsq, max_norm);
  else if (mode == MODE_F32 || is_mixed(mode))
    step_from_mean<float>(mode, n, N, rank, param_in, (const float*)mean, master_in,
                          (const float*)m_in, (const float*)v_in, param_out, master_out,
                          (float*)m_out, (float*)v_out, t, lr, b1, b2, eps, wd, decay,
                          clip_sumsq, max_norm);
  else
    return -1;
  return 0;
}

// The clipping factor for a squared norm (for pins).
double orc_clip_factor(double sumsq, double max_norm) { return clip_factor(sumsq, max_norm); }

// Momentum SGD in every call form: form 0 the sharded step (all workers),
// 1 the shard-free reference, 2 worker `rank`'s share (chunk gradients,
// shard-local master and buffer). The momentum buffer is buf_in/buf_out; the
// master follows the conventions of the Adam entry points.
int orc_sgd_step(int form, int mode, int64_t n, int64_t N, int64_t rank, const void* param_in,
                 const void* const* grads, const void* master_in, const void* buf_in,
                 void* param_out, void* master_out, void* buf_out, int64_t t, double lr,
                 double wd, double momentum, double dampening, int nesterov,
                 const uint8_t* decay) {
  if (n < 0 || N < 1 || t < 1 || form < 0 || form > 2) return -1;
  if (form == 2 && (rank < 0 || rank >= N)) return -1;
  const OptSel o = {1, momentum, dampening, nesterov};
  int64_t len = n;
  if (form == 2) {
    int64_t a, b;
    split_bounds(n, N, rank, &a, &b);
    len = b - a;
  }
  const size_t sb = mode == MODE_F64 ? 8 : 4;
  std::vector<unsigned char> vin((size_t)len * sb, 0), vout((size_t)len * sb, 0);  // unused by SGD
  if (mode == MODE_F64) {
    typedef double S;
    if (form == 0)
      sharded_step<S>(mode, n, N, param_in, grads, master_in, (const S*)buf_in, (const S*)vin.data(),
                      param_out, master_out, (S*)buf_out, (S*)vout.data(), t, lr, 0.9, 0.9, 1.0,
                      wd, decay, o);
    else if (form == 1)
      full_step<S>(mode, n, N, param_in, grads, master_in, (const S*)buf_in, (const S*)vin.data(),
                   param_out, master_out, (S*)buf_out, (S*)vout.data(), t, lr, 0.9, 0.9, 1.0, wd,
                   decay, o);
    else
      rank_step<S>(mode, n, N, rank, param_in, grads, (const S*)master_in, (const S*)buf_in,
                   (const S*)vin.data(), param_out, (S*)master_out, (S*)buf_out, (S*)vout.data(),
                   t, lr, 0.9, 0.9, 1.0, wd, decay, o);
  } else if (mode == MODE_F32 || is_mixed(mode)) {
    typedef float S;
    if (form == 0)
      sharded_step<S>(mode, n, N, param_in, grads, master_in, (const S*)buf_in, (const S*)vin.data(),
                      param_out, master_out, (S*)buf_out, (S*)vout.data(), t, lr, 0.9, 0.9, 1.0,
                      wd, decay, o);
    else if (form == 1)
      full_step<S>(mode, n, N, param_in, grads, master_in, (const S*)buf_in, (const S*)vin.data(),
                   param_out, master_out, (S*)buf_out, (S*)vout.data(), t, lr, 0.9, 0.9, 1.0, wd,
                   decay, o);
    else
      rank_step<S>(mode, n, N, rank, param_in, grads, (const S*)master_in, (const S*)buf_in,
                   (const S*)vin.data(), param_out, (S*)master_out, (S*)buf_out, (S*)vout.data(),
                   t, lr, 0.9, 0.9, 1.0, wd, decay, o);
  } else {
    return -1;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Memory per rank, in bytes: out[0] params, out[1] grads, out[2] optimizer.
//
// convention 0, the closed forms of "Data Parallelism & ZeRO" (section "ZeRO,
// stage by stage"), "Data parallelism and ZeRO optimization" (sections
// "Memory Consumption Analysis", "ZeRO-1/2/3") and "ZeRO One: Sharding the
// Optimizer" (section "Training Memory Requirements"): P bytes per parameter,
// G per gradient, K optimizer bytes per parameter; rank r's chunk has c_r
// elements.
//   stage 0 (no sharding): P n, G n, K n
//   stage 1: P n, G n, K c_r
//   stage 2: P n, G c_r, K c_r
//   stage 3: P c_r, G c_r, K c_r
//
// convention 1, the bookkeeping of "Data parallelism and ZeRO stages 1 to 3",
// section "2. Principles" (its paragraph on the emulation's bookkeeping) and the byte table
// of section "3. Worked example by hand", with bw bytes per value (P is used):
//   one process (stage 0): params bw n, grads bw n, optimizer 2 bw n
//   stage 1: bw n, bw n + bw c_r (the chunk's gradient), 2 bw c_r + bw c_r (master)
//   stage 2: bw n, bw c_r, 3 bw c_r
//   stage 3: bw c_r, bw c_r, 2 bw c_r (the chunk is the parameter storage)
// Returns 0, or -1 on a bad argument.
// ---------------------------------------------------------------------------
int orc_memory_bytes(int64_t n, int64_t N, int64_t r, int stage, int64_t P,
                     int64_t G, int64_t K, int convention, int64_t* out) {
  if (n < 1 || N < 1 || r < 0 || r >= N || stage < 0 || stage > 3) return -1;
  int64_t a, b;
  split_bounds(n, N, r, &a, &b);
  const int64_t c = b - a;
  if (convention == 0) {
    const bool shard_opt = stage >= 1, shard_grad = stage >= 2, shard_param = stage >= 3;
    out[0] = P * (shard_param ? c : n);
#if ORACLE_MUTANT == 13
    out[1] = G * n;  // planted: stage 2 keeping the full gradients
#else
    out[1] = G * (shard_grad ? c : n);
#endif
    out[2] = K * (shard_opt ? c : n);
    return 0;
  }
  if (convention == 1) {
    const int64_t bw = P;
    if (stage == 0) { out[0] = bw * n; out[1] = bw * n; out[2] = 2 * bw * n; }
    else if (stage == 1) { out[0] = bw * n; out[1] = bw * n + bw * c; out[2] = 3 * bw * c; }
    else if (stage == 2) {
      out[0] = bw * n;
#if ORACLE_MUTANT == 13
      out[1] = bw * n;  // planted: stage 2 keeping the full gradients
#else
      out[1] = bw * c;
#endif
      out[2] = 3 * bw * c;
    }
    else { out[0] = bw * c; out[1] = bw * c; out[2] = 2 * bw * c; }
    return 0;
  }
  return -1;
}

// The smallest stage whose memory need (convention 0, rank 0, plus the
// activations) is below the memory available ("Data parallelism and ZeRO
// optimization", section "When to Use Each ZeRO Stage"); -1 if none is.
int orc_min_stage(int64_t n, int64_t N, int64_t P, int64_t G, int64_t K, int64_t act,
                  int64_t avail) {
  for (int stage = 0; stage <= 3; ++stage) {
    int64_t out[3];
    if (orc_memory_bytes(n, N, 0, stage, P, G, K, 0, out) != 0) return -2;
    if (out[0] + out[1] + out[2] + act < avail) return stage;
  }
  return -1;
}

}  // extern "C"
