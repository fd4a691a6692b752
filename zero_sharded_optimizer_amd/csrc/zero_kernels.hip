// gfx950 kernels of the fused ZeRO-sharded Adam step.
//
// One launch performs the three phases of "ZeRO-Sharded Adam Step" (section
// "The step") for every element it owns, in registers:
//   1. reduce-scatter mean: the N workers' gradients at this element, summed in
//      rank order from worker 0, then divided by N;
//   2. Adam (with optional decoupled decay) on the element's master, m and v;
//   3. all-gather: the updated value is stored into the gathered parameter
//      buffer (bf16 in mixed precision, in place otherwise).
// Because all logical workers share one HBM, the shard of an element only says
// which worker "owns" it; the arithmetic of every element is the same
// ("Data parallelism and ZeRO stages 1 to 3", section "2. Principles": the
// chunked update equals the single-process update entry by entry). So the
// kernel streams the flat index space: each byte of every input is read from
// HBM once and each output byte written once. No LDS, no atomics, no MFMA:
// there is no contraction and no reuse, so the design is all about keeping
// enough 16-byte loads in flight per CU.
//
// Layout: thread i of the grid handles 16-byte groups i, i + G, i + 2G, ... of
// the gradient arrays (G = grid size in threads). A group is 2 fp64, 4 fp32 or
// 8 bf16 gradient elements; the matching state words are 16 (fp64, fp32) or
// 32 (mixed) bytes. Any len % VEC leftover elements are done one by one by the
// first threads of the grid.
//
// Floating point: compiled with -ffp-contract=off (and the pragma below) so
// no multiply-add is fused, with IEEE division and square root, and with
// denormals kept; every operation is one round-to-nearest-even operation, in
// the same order as the host-side definition of the step.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "zero_launch.h"

#pragma clang fp contract(off)

namespace {

constexpr int kBlock = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int CAP>
struct GradSet {
  const void* p[CAP];
};

template <class S>
struct Consts {
  S beta1, beta2, omb1, omb2, bias1, bias2, lr, eps, decay, nw;
};

// ---------------------------------------------------------------------------
// Per-mode traits: element types and 16-byte group packing.
//   S: state / compute type; G: gradient element; P: gathered parameter
//   element; VEC: elements per 16-byte gradient group.
// ---------------------------------------------------------------------------
struct ModeF64 {
  typedef double S;
  typedef double G;
  typedef double P;
  static constexpr int VEC = 2;
};
struct ModeF32 {
  typedef float S;
  typedef float G;
  typedef float P;
  static constexpr int VEC = 4;
};
struct ModeMixed {
  typedef float S;
  typedef uint16_t G;
  typedef uint16_t P;
  static constexpr int VEC = 8;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Round to nearest, ties to even; NaN becomes the quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Raw 16-byte gradient group and its widening into S.
template <class M>
struct GradRaw;
template <>
struct GradRaw<ModeF64> {
  f64x2 r;
  __device__ __forceinline__ void load(const void* base, int64_t g) {
    r = reinterpret_cast<const f64x2*>(base)[g];
  }
  __device__ __forceinline__ void widen(double (&s)[2]) const { s[0] = r.x; s[1] = r.y; }
  __device__ __forceinline__ void add(double (&s)[2]) const {
    s[0] = s[0] + r.x;
    s[1] = s[1] + r.y;
  }
};
template <>
struct GradRaw<ModeF32> {
  f32x4 r;
  __device__ __forceinline__ void load(const void* base, int64_t g) {
    r = reinterpret_cast<const f32x4*>(base)[g];
  }
  __device__ __forceinline__ void widen(float (&s)[4]) const {
    s[0] = r.x; s[1] = r.y; s[2] = r.z; s[3] = r.w;
  }
  __device__ __forceinline__ void add(float (&s)[4]) const {
    s[0] = s[0] + r.x;
    s[1] = s[1] + r.y;
    s[2] = s[2] + r.z;
    s[3] = s[3] + r.w;
  }
};
template <>
struct GradRaw<ModeMixed> {
  u32x4 r;
  __device__ __forceinline__ void load(const void* base, int64_t g) {
    r = reinterpret_cast<const u32x4*>(base)[g];
  }
  // element 2q is the low half of word q, element 2q+1 the high half
  __device__ __forceinline__ float elem(int e) const {
    const uint32_t w = r[e >> 1];
    return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  }
  __device__ __forceinline__ void widen(float (&s)[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = elem(e);
  }
  __device__ __forceinline__ void add(float (&s)[8]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = s[e] + elem(e);
  }
};

// State group (VEC elements of S) load / store.
template <class M>
struct StateIO;
template <>
struct StateIO<ModeF64> {
  __device__ __forceinline__ static void load(const double* p, int64_t g, double (&x)[2]) {
    const f64x2 r = reinterpret_cast<const f64x2*>(p)[g];
    x[0] = r.x; x[1] = r.y;
  }
  __device__ __forceinline__ static void store(double* p, int64_t g, const double (&x)[2]) {
    f64x2 r;
    r.x = x[0]; r.y = x[1];
    reinterpret_cast<f64x2*>(p)[g] = r;
  }
};
template <>
struct StateIO<ModeF32> {
  __device__ __forceinline__ static void load(const float* p, int64_t g, float (&x)[4]) {
    const f32x4 r = reinterpret_cast<const f32x4*>(p)[g];
    x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
  }
  __device__ __forceinline__ static void store(float* p, int64_t g, const float (&x)[4]) {
    f32x4 r;
    r.x = x[0]; r.y = x[1]; r.z = x[2]; r.w = x[3];
    reinterpret_cast<f32x4*>(p)[g] = r;
  }
};
template <>
struct StateIO<ModeMixed> {
  __device__ __forceinline__ static void load(const float* p, int64_t g, float (&x)[8]) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[2 * g];
    const f32x4 b = reinterpret_cast<const f32x4*>(p)[2 * g + 1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, int64_t g, const float (&x)[8]) {
    f32x4 a, b;
    a.x = x[0]; a.y = x[1]; a.z = x[2]; a.w = x[3];
    b.x = x[4]; b.y = x[5]; b.z = x[6]; b.w = x[7];
    reinterpret_cast<f32x4*>(p)[2 * g] = a;
    reinterpret_cast<f32x4*>(p)[2 * g + 1] = b;
  }
};

// Gathered-parameter write-back of a group, 16-byte aligned destination.
template <class M>
struct OutIO;
template <>
struct OutIO<ModeF64> {
  __device__ __forceinline__ static void store_vec(double* p, int64_t g, const double (&x)[2]) {
    StateIO<ModeF64>::store(p, g, x);
  }
  __device__ __forceinline__ static double conv(double x) { return x; }
};
template <>
struct OutIO<ModeF32> {
  __device__ __forceinline__ static void store_vec(float* p, int64_t g, const float (&x)[4]) {
    StateIO<ModeF32>::store(p, g, x);
  }
  __device__ __forceinline__ static float conv(float x) { return x; }
};
template <>
struct OutIO<ModeMixed> {
  __device__ __forceinline__ static void store_vec(uint16_t* p, int64_t g, const float (&x)[8]) {
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = f32_to_bf16(x[2 * q]) | (f32_to_bf16(x[2 * q + 1]) << 16);
    reinterpret_cast<u32x4*>(p)[g] = r;
  }
  __device__ __forceinline__ static uint16_t conv(float x) { return (uint16_t)f32_to_bf16(x); }
};

__device__ __forceinline__ float sqrt_rn(float x) { return __builtin_sqrtf(x); }
__device__ __forceinline__ double sqrt_rn(double x) { return __builtin_sqrt(x); }

__device__ __forceinline__ double grad_elem(const double* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float grad_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float grad_elem(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// Steps 2-3 for one element: the moments, bias correction, optional decoupled
// decay, and the update of the master value w, in the defined order.
template <class S>
__device__ __forceinline__ void adam_element(S s, S& w, S& m, S& v, bool decay,
                                             const Consts<S>& c) {
  const S gb = s / c.nw;
  const S b1m = c.beta1 * m;
  const S g1 = c.omb1 * gb;
  const S m_new = b1m + g1;
  const S gsq = gb * gb;
  const S b2v = c.beta2 * v;
  const S g2 = c.omb2 * gsq;
  const S v_new = b2v + g2;
  const S mh = m_new / c.bias1;
  const S vh = v_new / c.bias2;
  const S den = sqrt_rn(vh) + c.eps;
  S ww = w;
  if (decay) ww = ww * c.decay;
  const S ratio = mh / den;
  const S upd = c.lr * ratio;
  w = ww - upd;
  m = m_new;
  v = v_new;
}

// Decay flags of elements j .. j+VEC-1 (bit e of the result is element j+e).
template <int VEC>
__device__ __forceinline__ uint32_t decay_bits(const uint32_t* __restrict__ mask,
                                               int64_t bit0) {
  const int64_t word = bit0 >> 5;
  const int sh = (int)(bit0 & 31);
  uint64_t bits = mask[word];
  if (sh + VEC > 32) bits |= (uint64_t)mask[word + 1] << 32;
  return (uint32_t)(bits >> sh) & ((1u << VEC) - 1u);
}

// The fused step. NFIX > 0: exactly NFIX workers (all gradient loads of a group
// issued before the first add); NFIX == 0: any N <= CAP, loaded in batches of 8.
template <class M, int NFIX, int CAP>
__global__ void __launch_bounds__(kBlock)
    zero_step_kernel(GradSet<CAP> gs, int nw, typename M::S* __restrict__ w,
                     typename M::S* __restrict__ m, typename M::S* __restrict__ v,
                     typename M::P* __restrict__ out, int out_vec, int64_t len,
                     Consts<typename M::S> c, const uint32_t* __restrict__ mask,
                     int64_t mask_off, int decay_kind) {
  typedef typename M::S S;
  constexpr int VEC = M::VEC;
  const int64_t ngroups = len / VEC;
  const int64_t tid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  const int N = NFIX > 0 ? NFIX : nw;

  for (int64_t g = tid; g < ngroups; g += stride) {
    // 1. reduce-scatter mean, rank order
    S s[VEC];
    if constexpr (NFIX > 0) {
      GradRaw<M> raw[NFIX];
#pragma unroll
      for (int k = 0; k < NFIX; ++k) raw[k].load(gs.p[k], g);
      raw[0].widen(s);
#pragma unroll
      for (int k = 1; k < NFIX; ++k) raw[k].add(s);
    } else {
      {
        GradRaw<M> r0;
        r0.load(gs.p[0], g);
        r0.widen(s);
      }
      for (int k0 = 1; k0 < N; k0 += 8) {
        GradRaw<M> raw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (k0 + j < N) raw[j].load(gs.p[k0 + j], g);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (k0 + j < N) raw[j].add(s);
      }
    }
    // 2. Adam on the element's own state
    S wv[VEC], mv[VEC], vv[VEC];
    StateIO<M>::load(w, g, wv);
    StateIO<M>::load(m, g, mv);
    StateIO<M>::load(v, g, vv);
    uint32_t dbits = 0;
    if (decay_kind == 1) dbits = (1u << VEC) - 1u;
    else if (decay_kind == 2) dbits = decay_bits<VEC>(mask, mask_off + g * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) adam_element<S>(s[e], wv[e], mv[e], vv[e], (dbits >> e) & 1u, c);
    StateIO<M>::store(m, g, mv);
    StateIO<M>::store(v, g, vv);
    // 3. all-gather write-back
    if (out == nullptr) {
      StateIO<M>::store(w, g, wv);
    } else {
      StateIO<M>::store(w, g, wv);
      if (out_vec) {
        OutIO<M>::store_vec(out, g, wv);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) out[g * VEC + e] = OutIO<M>::conv(wv[e]);
      }
    }
  }

  // leftover elements, one per thread
  const int64_t i = ngroups * VEC + tid;
  if (i < len) {
    typedef typename M::G G;
    S s = grad_elem(reinterpret_cast<const G*>(gs.p[0]), i);
    for (int k = 1; k < N; ++k) s = s + grad_elem(reinterpret_cast<const G*>(gs.p[k]), i);
    S wi = w[i], mi = m[i], vi = v[i];
    bool dec = decay_kind == 1;
    if (decay_kind == 2) {
      const int64_t b = mask_off + i;
      dec = (mask[b >> 5] >> (b & 31)) & 1u;
    }
    adam_element<S>(s, wi, mi, vi, dec, c);
    w[i] = wi;
    m[i] = mi;
    v[i] = vi;
    if (out != nullptr) out[i] = OutIO<M>::conv(wi);
  }
}

// init_states: m = v = 0; master from the gathered parameters when asked.
template <class M>
__global__ void __launch_bounds__(kBlock)
    zero_init_kernel(const typename M::P* __restrict__ param, typename M::S* __restrict__ master,
                     typename M::S* __restrict__ m, typename M::S* __restrict__ v, int64_t len) {
  typedef typename M::S S;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < len; i += stride) {
    m[i] = S(0);
    v[i] = S(0);
    if (master != nullptr) {
      if constexpr (sizeof(typename M::P) == 2)
        master[i] = bf16_to_f32(param[i]);
      else
        master[i] = param[i];
    }
  }
}

int device_cus() {
  // one query per device; the count is the same for every launch on it
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

template <class S>
Consts<S> round_consts(const zlaunch::StepArgs& a) {
  Consts<S> c;
  c.beta1 = (S)a.beta1;
  c.beta2 = (S)a.beta2;
  c.omb1 = (S)a.one_minus_beta1;
  c.omb2 = (S)a.one_minus_beta2;
  c.bias1 = (S)a.bias1;
  c.bias2 = (S)a.bias2;
  c.lr = (S)a.lr;
  c.eps = (S)a.eps;
  c.decay = (S)a.decay_factor;
  c.nw = (S)a.n_workers_value;
  return c;
}

template <class M, int NFIX, int CAP>
void launch_mode_n(const zlaunch::StepArgs& a, hipStream_t st, int blocks) {
  typedef typename M::S S;
  typedef typename M::P P;
  GradSet<CAP> gs;
  for (int k = 0; k < CAP; ++k) gs.p[k] = k < a.n_workers ? a.grads[k] : nullptr;
  const int out_vec = a.out != nullptr && (reinterpret_cast<uintptr_t>(a.out) % 16 == 0);
  hipLaunchKernelGGL((zero_step_kernel<M, NFIX, CAP>), dim3(blocks), dim3(kBlock), 0, st, gs,
                     a.n_workers, static_cast<S*>(a.w), static_cast<S*>(a.m),
                     static_cast<S*>(a.v), static_cast<P*>(a.out), out_vec, a.len,
                     round_consts<S>(a), a.mask, a.mask_bit_offset, a.decay_kind);
}

template <class M>
void launch_mode(const zlaunch::StepArgs& a, hipStream_t st) {
  const int64_t ngroups = a.len / M::VEC;
  int64_t want = (ngroups + kBlock - 1) / kBlock;
  const int64_t cap = (int64_t)device_cus() * 8;
  int blocks = (int)(want < 1 ? 1 : (want > cap ? cap : want));
  switch (a.n_workers) {
    case 1: launch_mode_n<M, 1, 1>(a, st, blocks); break;
    case 2: launch_mode_n<M, 2, 2>(a, st, blocks); break;
    case 4: launch_mode_n<M, 4, 4>(a, st, blocks); break;
    case 8: launch_mode_n<M, 8, 8>(a, st, blocks); break;
    default:
      if (a.n_workers <= 64) launch_mode_n<M, 0, 64>(a, st, blocks);
      else launch_mode_n<M, 0, zlaunch::kMaxWorkers>(a, st, blocks);
      break;
  }
}

template <class M>
void launch_init_mode(const zlaunch::InitArgs& a, hipStream_t st) {
  typedef typename M::S S;
  typedef typename M::P P;
  int64_t want = (a.len + kBlock - 1) / kBlock;
  const int64_t cap = (int64_t)device_cus() * 8;
  int blocks = (int)(want < 1 ? 1 : (want > cap ? cap : want));
  hipLaunchKernelGGL((zero_init_kernel<M>), dim3(blocks), dim3(kBlock), 0, st,
                     static_cast<const P*>(a.param), static_cast<S*>(a.master),
                     static_cast<S*>(a.m), static_cast<S*>(a.v), a.len);
}

}  // namespace

namespace zlaunch {

const char* launch_step(const StepArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the check below is this launch's
  switch (a.mode) {
    case 0: launch_mode<ModeF64>(a, st); break;
    case 1: launch_mode<ModeF32>(a, st); break;
    case 2: launch_mode<ModeMixed>(a, st); break;
    default: return "unknown mode";
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? nullptr : hipGetErrorString(e);
}

const char* launch_init(const InitArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  switch (a.mode) {
    case 0: launch_init_mode<ModeF64>(a, st); break;
    case 1: launch_init_mode<ModeF32>(a, st); break;
    case 2: launch_init_mode<ModeMixed>(a, st); break;
    default: return "unknown mode";
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? nullptr : hipGetErrorString(e);
}

}  // namespace zlaunch
