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
// ("Data parallelism and ZeRO stages 1 to 3", section "2. Principles": an
// elementwise optimizer on a chunk reproduces the unsharded result for those
// elements). So the
// kernel streams the flat index space: each byte of every input is read from
// HBM once and each output byte written once. No atomics, no MFMA and no use of
// LDS (on some shapes a dynamic LDS allocation that no thread touches caps the
// blocks resident on a CU): there is no contraction and no reuse, so the design
// is all about the amount of wide loads in flight per CU. Too few starve the
// memory system; on this chip, too many slow it down.
//
// Layout: a group is the elements of one gradient stream that one thread
// loads at once: 2 fp64, 4 fp32 (16 bytes) or 4 bf16 (8 bytes); the matching
// state words of each state array are 16 bytes. Block b owns a tile of consecutive
// groups (see the launch shape below). The len % VEC leftover elements are done
// one by one by the first threads of block 0.
//
// Floating point: compiled with -ffp-contract=off (and the pragma below) so
// no multiply-add is fused, with IEEE division and square root, and with
// denormals kept; every operation is one round-to-nearest-even operation, in
// the same order as the host-side definition of the step.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "zero_launch.h"

#pragma clang fp contract(off)

namespace {

// Cache policy and launch shape. The step touches every byte once, so loads
// and stores carry the nontemporal hint (stream through the caches without
// keeping the lines). The grid is not persistent: block b owns one tile of
// BLOCK * C consecutive groups, and blocks retire and start in address order,
// so the window of in-flight requests sweeps each stream front to back. Within
// the tile a thread takes C groups, BLOCK or 64 groups apart (WC below), so
// every load instruction of a wave covers 512 B or 1 KiB of one stream. A
// thread either issues all its loads before it adds any, or one stream at a
// time (ISSUE below). Measured on MI355X, the tiled grid beats a grid-stride
// persistent loop by about 25 % on the many-stream mix of the step.
#ifndef ZERO_STEP_NT_LOAD
#define ZERO_STEP_NT_LOAD 1
#endif
#ifndef ZERO_STEP_NT_STORE
#define ZERO_STEP_NT_STORE 1
#endif
// Any-N path (N not 1, 2, 4 or 8): gradient loads issued per batch (4, 8 and
// 16 measured the same on MI355X).
constexpr int kWideBatch = 8;
// Launch shapes per mode: BLOCK threads, C groups per thread, ISSUE, WC, and
// CU_BLOCKS; overridable at build time for tuning. ISSUE 0: a thread issues its
// gradient loads, folds them, then loads its state words; 1: the state loads
// go out together with the gradient loads, before the thread waits on any; 2:
// every load waits for the one before it (one stream in flight per wave; the
// many small blocks provide the parallelism). WC 1: the C groups of a thread
// are 64 groups apart, so each wave covers C * 64 consecutive groups; 0: BLOCK
// groups apart. CU_BLOCKS > 0: at most that many blocks reside on a CU at once
// (a dynamic LDS allocation the kernel never touches enforces it), which sets
// the loads in flight chip-wide (0: as many as registers allow). The fp32 and
// mixed modes have a bulk shape (serial issue under a cap), used from ROUNDS
// full rounds of resident blocks up, and a wide shape below that (a bucket of
// a few MiB); F32W is the fp32 shape for any N (not 1, 2, 4 or 8). Chosen by
// interleaved A/B runs on MI355X (same process, same buffers; placement moves
// every shape by several percent between processes):
//   mixed, N = 8:      bulk 64 x 2, ISSUE 2, 16 blocks per CU (4 waves per
//                      SIMD, 1 KiB of one stream in flight per wave): 2-4 %
//                      over the same shape at its register-bound 5 waves,
//                      10-12 % over 8 waves; 14, 17, 18 and 20 blocks lose
//                      0-1.5 %, 12 blocks (3 waves) 10 %, 8 blocks 25 %.
//                      Against the wide 512 x 2 with ISSUE 1: 2-9 % on the
//                      10^9-element rank share (0.77-0.79 of 8 TB/s against
//                      0.70-0.78). 64 x 1, 64 x 4, 128 x 2 and 256 x 2 lose
//                      1-3 %, 128 x 2 and 256 x 1 under the same 4-wave cap
//                      4-5 %. Bulk from 6 rounds: below 4 rounds (buckets of
//                      up to 4 M elements) the wide shape is 2-10 % faster,
//                      from 4 to 8 rounds the two are within 1 %;
//   fp32, N = 8:       bulk 64 x 2, ISSUE 2, 12 blocks per CU (3 waves per
//                      SIMD, 2 KiB in flight per wave): 5-13 % over the wide
//                      512 x 2, ISSUE 1, strided groups (0.79-0.80 of 8 TB/s
//                      against 0.70-0.76 on 320 M elements); 10, 11, 13, 14,
//                      16 and 20 blocks lose 1-5 %, 64 x 1 and 64 x 4 2-6 %.
//                      Bulk from 8 rounds: below 4 rounds the wide shape is
//                      2-13 % faster, from 4 to 8 rounds 1-4 % either way;
//   fp32, N = 64:      128 x 8, WC, ISSUE 0: 3 % over 512 x 2 (314 registers,
//                      one wave per SIMD, 64 loads of 1 KiB in flight per wave);
//                      ISSUE 2 shapes lose 2-10 % with or without a cap;
//   fp64 (1 M params): 256 x 1; launch-bound, every shape within noise.
// Tile order: running tile b on block b beat giving each XCD a contiguous
// share of the tiles by 1-7 %.
#ifndef ZERO_F64_BLOCK
#define ZERO_F64_BLOCK 256
#endif
#ifndef ZERO_F64_GROUPS
#define ZERO_F64_GROUPS 1
#endif
#ifndef ZERO_F64_ISSUE
#define ZERO_F64_ISSUE 0
#endif
#ifndef ZERO_F64_WC
#define ZERO_F64_WC 0
#endif
#ifndef ZERO_F32_BLOCK
#define ZERO_F32_BLOCK 64
#endif
#ifndef ZERO_F32_GROUPS
#define ZERO_F32_GROUPS 2
#endif
#ifndef ZERO_F32_ISSUE
#define ZERO_F32_ISSUE 2
#endif
#ifndef ZERO_F32_WC
#define ZERO_F32_WC 1
#endif
#ifndef ZERO_F32_CU_BLOCKS
#define ZERO_F32_CU_BLOCKS 12
#endif
#ifndef ZERO_F32_ROUNDS
#define ZERO_F32_ROUNDS 8
#endif
#ifndef ZERO_F32_WIDE_BLOCK
#define ZERO_F32_WIDE_BLOCK 512
#endif
#ifndef ZERO_F32_WIDE_GROUPS
#define ZERO_F32_WIDE_GROUPS 2
#endif
#ifndef ZERO_F32_WIDE_ISSUE
#define ZERO_F32_WIDE_ISSUE 1
#endif
#ifndef ZERO_F32_WIDE_WC
#define ZERO_F32_WIDE_WC 0
#endif
#ifndef ZERO_F32W_BLOCK
#define ZERO_F32W_BLOCK 128
#endif
#ifndef ZERO_F32W_GROUPS
#define ZERO_F32W_GROUPS 8
#endif
#ifndef ZERO_F32W_ISSUE
#define ZERO_F32W_ISSUE 0
#endif
#ifndef ZERO_F32W_WC
#define ZERO_F32W_WC 1
#endif
#ifndef ZERO_MIX_BLOCK
#define ZERO_MIX_BLOCK 64
#endif
#ifndef ZERO_MIX_GROUPS
#define ZERO_MIX_GROUPS 2
#endif
#ifndef ZERO_MIX_ISSUE
#define ZERO_MIX_ISSUE 2
#endif
#ifndef ZERO_MIX_WC
#define ZERO_MIX_WC 1
#endif
#ifndef ZERO_MIX_CU_BLOCKS
#define ZERO_MIX_CU_BLOCKS 16
#endif
#ifndef ZERO_MIX_ROUNDS
#define ZERO_MIX_ROUNDS 6
#endif
#ifndef ZERO_MIX_WIDE_BLOCK
#define ZERO_MIX_WIDE_BLOCK 512
#endif
#ifndef ZERO_MIX_WIDE_GROUPS
#define ZERO_MIX_WIDE_GROUPS 2
#endif
#ifndef ZERO_MIX_WIDE_ISSUE
#define ZERO_MIX_WIDE_ISSUE 1
#endif
#ifndef ZERO_MIX_WIDE_WC
#define ZERO_MIX_WIDE_WC 1
#endif
#ifndef ZERO_MIXMEAN_CU_BLOCKS
#define ZERO_MIXMEAN_CU_BLOCKS 12
#endif
#ifndef ZERO_MIXMEAN_ROUNDS
#define ZERO_MIXMEAN_ROUNDS 8
#endif

constexpr int kInitBlock = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <class T>
__device__ __forceinline__ T ld_stream(const T* p) {
#if ZERO_STEP_NT_LOAD
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
template <class T>
__device__ __forceinline__ void st_stream(T* p, T v) {
#if ZERO_STEP_NT_STORE
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// A zero that exists only once `word` (a value just loaded) has arrived, and
// once the previous token `prev` has: adding it to the next load's index makes
// that load wait for this one, in hardware (the asm reads the loaded register,
// so the load must have returned) and in the compiler (the next address depends
// on the asm's result, so no load can be moved above it). Used by the issue
// mode that keeps one load in flight per wave.
__device__ __forceinline__ uint32_t after(uint32_t word, uint32_t prev) {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z) : "v"(word), "v"(prev));
  return z;
}
__device__ __forceinline__ uint32_t first_word(float x) { return __float_as_uint(x); }
__device__ __forceinline__ uint32_t first_word(double x) {
  return (uint32_t)__double_as_longlong(x);
}
// A token that exists only once every element of x has been computed. Chaining
// the next gradient load on the running sums (not on the raw loaded word) makes
// each group's add happen as its load arrives, so the raw groups are not kept
// in registers until the end of the fold.
template <class T, int V>
__device__ __forceinline__ uint32_t after_all(const T (&x)[V], uint32_t prev) {
  uint32_t t = prev;
#pragma unroll
  for (int e = 0; e < V; ++e) t = after(first_word(x[e]), t);
  return t;
}

template <int CAP>
struct GradSet {
  const void* p[CAP];
};

template <class S>
struct Consts {
  S beta1, beta2, omb1, omb2, bias1, bias2, lr, eps, decay, nw;
  // momentum SGD
  S wd, mom, omd;
  int has_mom, nesterov, first;
};

// ---------------------------------------------------------------------------
// Per-mode traits: element types and group packing.
//   S: state / compute type; G: gradient element; P: gathered parameter
//   element; VEC: elements per gradient group.
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
// Mixed precision uses 8-byte gradient groups (4 bf16), so that each thread's
// fp32 state words are one 16-byte vector and every state access of a wave is
// lane-interleaved like the gradient loads. (16-byte groups of 8 bf16 put 32
// contiguous state bytes on each lane; on MI355X that measured 4 % slower and
// wrote 5 % more than the bytes it stores.)
struct ModeMixed {
  typedef float S;
  typedef uint16_t G;
  typedef uint16_t P;
  static constexpr int VEC = 4;
};

// fp16 mixed precision: fp16 gradients and gathered parameters (bit patterns),
// fp32 master, m and v; the same 8-byte gradient groups as bf16.
struct ModeMixedF16 {
  typedef float S;
  typedef _Float16 G;
  typedef uint16_t P;
  static constexpr int VEC = 4;
};

// The step driven by a materialised fp32 mean gradient in mixed precision:
// fp32 "gradient" groups, fp32 state, bf16 (or fp16) write-back.
struct ModeMixedMean {
  typedef float S;
  typedef float G;
  typedef uint16_t P;
  static constexpr int VEC = 4;
};
struct ModeMixedF16Mean {
  typedef float S;
  typedef float G;
  typedef uint16_t P;
  static constexpr int VEC = 4;
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

// fp16 <-> fp32 by the hardware conversions: widening is exact; narrowing
// rounds to nearest even, keeps fp16 subnormals and overflows to infinity. NaN
// becomes the quiet NaN 0x7E00.
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_f16(float x) {
  if (x != x) return 0x7E00u;
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Raw gradient group (16 or 8 bytes) and its widening into S.
template <class M>
struct GradRaw;
template <>
struct GradRaw<ModeF64> {
  f64x2 r;
  __device__ __forceinline__ uint32_t word0() const { return first_word(r.x); }
  __device__ __forceinline__ void load(const void* base, int64_t g) {
    r = ld_stream(reinterpret_cast<const f64x2*>(base) + g);
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
  __device__ __forceinline__ uint32_t word0() const { return first_word(r.x); }
  __device__ __forceinline__ void load(const void* base, int64_t g) {
    r = ld_stream(reinterpret_cast<const f32x4*>(base) + g);
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
  u32x2 r;
  __device__ __forceinline__ uint32_t word0() const { return r.x; }
  __device__ __forceinline__ void load(const void* base, int64_t g) {
    r = ld_stream(reinterpret_cast<const u32x2*>(base) + g);
  }
  __device__ __forceinline__ float elem(int e) const {
    const uint32_t w = r[e >> 1];
    return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  }
  __device__ __forceinline__ void widen(float (&s)[4]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = elem(e);
  }
  __device__ __forceinline__ void add(float (&s)[4]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = s[e] + elem(e);
  }
};

template <>
struct GradRaw<ModeMixedF16> {
  u32x2 r;
  __device__ __forceinline__ uint32_t word0() const { return r.x; }
  __device__ __forceinline__ void load(const void* base, int64_t g) {
    r = ld_stream(reinterpret_cast<const u32x2*>(base) + g);
  }
  __device__ __forceinline__ float elem(int e) const {
    const uint32_t w = r[e >> 1];
    return f16_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
  __device__ __forceinline__ void widen(float (&s)[4]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = elem(e);
  }
  __device__ __forceinline__ void add(float (&s)[4]) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = s[e] + elem(e);
  }
};

template <>
struct GradRaw<ModeMixedMean> : GradRaw<ModeF32> {};
template <>
struct GradRaw<ModeMixedF16Mean> : GradRaw<ModeF32> {};

// State group (VEC elements of S) load / store.
template <class M>
struct StateIO;
template <>
struct StateIO<ModeF64> {
  __device__ __forceinline__ static void load(const double* p, int64_t g, double (&x)[2]) {
    const f64x2 r = ld_stream(reinterpret_cast<const f64x2*>(p) + g);
    x[0] = r.x; x[1] = r.y;
  }
  __device__ __forceinline__ static void store(double* p, int64_t g, const double (&x)[2]) {
    f64x2 r;
    r.x = x[0]; r.y = x[1];
    st_stream(reinterpret_cast<f64x2*>(p) + g, r);
  }
};
template <>
struct StateIO<ModeF32> {
  __device__ __forceinline__ static void load(const float* p, int64_t g, float (&x)[4]) {
    const f32x4 r = ld_stream(reinterpret_cast<const f32x4*>(p) + g);
    x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
  }
  __device__ __forceinline__ static void store(float* p, int64_t g, const float (&x)[4]) {
    f32x4 r;
    r.x = x[0]; r.y = x[1]; r.z = x[2]; r.w = x[3];
    st_stream(reinterpret_cast<f32x4*>(p) + g, r);
  }
};
template <>
struct StateIO<ModeMixed> : StateIO<ModeF32> {};
template <>
struct StateIO<ModeMixedMean> : StateIO<ModeF32> {};
template <>
struct StateIO<ModeMixedF16> : StateIO<ModeF32> {};
template <>
struct StateIO<ModeMixedF16Mean> : StateIO<ModeF32> {};

// Gathered-parameter write-back of a group to a destination aligned to kAlign.
template <class M>
struct OutIO;
template <>
struct OutIO<ModeF64> {
  static constexpr int kAlign = 16;
  __device__ __forceinline__ static void store_vec(double* p, int64_t g, const double (&x)[2]) {
    StateIO<ModeF64>::store(p, g, x);
  }
  __device__ __forceinline__ static double conv(double x) { return x; }
};
template <>
struct OutIO<ModeF32> {
  static constexpr int kAlign = 16;
  __device__ __forceinline__ static void store_vec(float* p, int64_t g, const float (&x)[4]) {
    StateIO<ModeF32>::store(p, g, x);
  }
  __device__ __forceinline__ static float conv(float x) { return x; }
};
template <>
struct OutIO<ModeMixed> {
  static constexpr int kAlign = 8;
  __device__ __forceinline__ static void store_vec(uint16_t* p, int64_t g, const float (&x)[4]) {
    u32x2 r;
    r.x = f32_to_bf16(x[0]) | (f32_to_bf16(x[1]) << 16);
    r.y = f32_to_bf16(x[2]) | (f32_to_bf16(x[3]) << 16);
    st_stream(reinterpret_cast<u32x2*>(p) + g, r);
  }
  __device__ __forceinline__ static uint16_t conv(float x) { return (uint16_t)f32_to_bf16(x); }
};

template <>
struct OutIO<ModeMixedF16> {
  static constexpr int kAlign = 8;
  __device__ __forceinline__ static void store_vec(uint16_t* p, int64_t g, const float (&x)[4]) {
    u32x2 r;
    r.x = f32_to_f16(x[0]) | (f32_to_f16(x[1]) << 16);
    r.y = f32_to_f16(x[2]) | (f32_to_f16(x[3]) << 16);
    st_stream(reinterpret_cast<u32x2*>(p) + g, r);
  }
  __device__ __forceinline__ static uint16_t conv(float x) { return (uint16_t)f32_to_f16(x); }
};

template <>
struct OutIO<ModeMixedMean> : OutIO<ModeMixed> {};
template <>
struct OutIO<ModeMixedF16Mean> : OutIO<ModeMixedF16> {};

__device__ __forceinline__ float sqrt_rn(float x) { return __builtin_sqrtf(x); }
__device__ __forceinline__ double sqrt_rn(double x) { return __builtin_sqrt(x); }

__device__ __forceinline__ double grad_elem(const double* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float grad_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float grad_elem(const _Float16* p, int64_t i) { return (float)p[i]; }
__device__ __forceinline__ float grad_elem(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// The global-norm clipping factor min(1, max_norm / (sqrt(sumsq) + 1e-6)), in
// double (the definition torch's clip_grad_norm_ uses), rounded once to S. A NaN
// norm gives a NaN factor, as torch's clamp does, so every clipped element
// becomes NaN rather than taking an unclipped step.
template <class S>
__device__ __forceinline__ S clip_coef(const double* __restrict__ sumsq, double max_norm) {
  const double nrm = __builtin_sqrt(*sumsq);
  const double cf = max_norm / (nrm + 1e-6);
  return (S)((cf < 1.0 || cf != cf) ? cf : 1.0);
}

// Steps 2-3 for one element: the moments, bias correction, optional decoupled
// decay, and the update of the master value w, in the defined order.
template <class S>
__device__ __forceinline__ void adam_element(S s, S& w, S& m, S& v, bool decay,
                                             const Consts<S>& c, bool clip, S coef) {
  S gb = s / c.nw;
  if (clip) gb = gb * coef;
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

// Momentum SGD for one element, in the defined order (coupled decay, buffer
// set to the first step's d, optional dampening and Nesterov).
template <class S>
__device__ __forceinline__ void sgd_element(S s, S& w, S& buf, bool decay, const Consts<S>& c,
                                            bool clip, S coef) {
  S d = s / c.nw;
  if (clip) d = d * coef;
  if (decay) {
    const S dw = c.wd * w;
    d = d + dw;
  }
  if (c.has_mom) {
    S b;
    if (c.first) {
      b = d;
    } else {
      const S kept = c.mom * buf;
      const S added = c.omd * d;
      b = kept + added;
    }
    buf = b;
    if (c.nesterov) {
      const S nb = c.mom * b;
      d = d + nb;
    } else {
      d = b;
    }
  }
  const S step = c.lr * d;
  w = w - step;
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

// Loads the state words of a thread's live groups.
template <class M, int C, int OPT, bool GUARD>
__device__ __forceinline__ void load_states(typename M::S* __restrict__ w,
                                            typename M::S* __restrict__ m,
                                            typename M::S* __restrict__ v, int64_t g0, int block,
                                            const bool* live, bool use_m,
                                            typename M::S (*wv)[M::VEC],
                                            typename M::S (*mv)[M::VEC],
                                            typename M::S (*vv)[M::VEC]) {
#pragma unroll
  for (int u = 0; u < C; ++u) {
    if (GUARD && !live[u]) continue;
    const int64_t g = g0 + (int64_t)u * block;
    StateIO<M>::load(w, g, wv[u]);
    if (use_m) StateIO<M>::load(m, g, mv[u]);
    if (OPT == 0) StateIO<M>::load(v, g, vv[u]);
  }
}

// The C groups of one thread. ISSUE 0 or 1: the gradient loads of all groups
// are issued first (with the state loads too when ISSUE is 1), then the
// gradients are folded in rank order, then each group is updated and stored.
// ISSUE 2: every load is issued alone, after the previous one has returned:
// worker 0's group, then worker 1's, ... (each added as it arrives), then the
// master, m and v words. One load is in flight per wave, and the many waves of
// a small-block launch provide the parallelism; the arithmetic and its order
// are the same in every mode. GUARD: some of the thread's groups may lie past
// the end (only in the last block of the grid); otherwise no load is
// predicated.
template <class M, int NFIX, int CAP, int GS, int C, int OPT, int ISSUE, bool MEAN, bool GUARD>
__device__ __forceinline__ void step_groups(
    const GradSet<CAP>& gs, int N, typename M::S* __restrict__ w, typename M::S* __restrict__ m,
    typename M::S* __restrict__ v, typename M::P* __restrict__ out, int out_vec,
    typename M::S* __restrict__ mean_out, int64_t g0, int64_t ngroups,
    const Consts<typename M::S>& c, const uint32_t* __restrict__ mask, int64_t mask_off,
    int decay_kind, bool clip, typename M::S coef) {
  typedef typename M::S S;
  constexpr int VEC = M::VEC;
  bool live[C];
#pragma unroll
  for (int u = 0; u < C; ++u) live[u] = !GUARD || g0 + (int64_t)u * GS < ngroups;
  const bool use_m = OPT == 0 || c.has_mom;

  S s[C][VEC];
  S wv[C][VEC], mv[C][VEC], vv[C][VEC];
  constexpr bool PRE = ISSUE == 1;
  if constexpr (ISSUE == 2) {
    // each load's index carries the token of the load before it
    uint32_t tok = 0;
    {
      GradRaw<M> raw[C];
#pragma unroll
      for (int u = 0; u < C; ++u)
        if (live[u]) raw[u].load(gs.p[0], g0 + (int64_t)u * GS + tok);
#pragma unroll
      for (int u = 0; u < C; ++u) {
        raw[u].widen(s[u]);
        tok = after_all(s[u], tok);
      }
    }
    constexpr int kUnroll = NFIX > 0 ? NFIX : 1;
#pragma unroll kUnroll
    for (int k = 1; k < N; ++k) {
      GradRaw<M> raw[C];
#pragma unroll
      for (int u = 0; u < C; ++u)
        if (live[u]) raw[u].load(gs.p[k], g0 + (int64_t)u * GS + tok);
#pragma unroll
      for (int u = 0; u < C; ++u) {
        raw[u].add(s[u]);
        tok = after_all(s[u], tok);
      }
    }
#pragma unroll
    for (int u = 0; u < C; ++u)
      if (live[u]) StateIO<M>::load(w, g0 + (int64_t)u * GS + tok, wv[u]);
#pragma unroll
    for (int u = 0; u < C; ++u) tok = after(first_word(wv[u][0]), tok);
    if (use_m) {
#pragma unroll
      for (int u = 0; u < C; ++u)
        if (live[u]) StateIO<M>::load(m, g0 + (int64_t)u * GS + tok, mv[u]);
#pragma unroll
      for (int u = 0; u < C; ++u) tok = after(first_word(mv[u][0]), tok);
    }
    if constexpr (OPT == 0) {
#pragma unroll
      for (int u = 0; u < C; ++u)
        if (live[u]) StateIO<M>::load(v, g0 + (int64_t)u * GS + tok, vv[u]);
    }
  } else if constexpr (NFIX > 0) {
    GradRaw<M> raw[C][NFIX];
#pragma unroll
    for (int u = 0; u < C; ++u)
#pragma unroll
      for (int k = 0; k < NFIX; ++k)
        if (live[u]) raw[u][k].load(gs.p[k], g0 + (int64_t)u * GS);
    if constexpr (PRE)
      load_states<M, C, OPT, GUARD>(w, m, v, g0, GS, live, use_m, wv, mv, vv);
#pragma unroll
    for (int u = 0; u < C; ++u) {
      raw[u][0].widen(s[u]);
#pragma unroll
      for (int k = 1; k < NFIX; ++k) raw[u][k].add(s[u]);
    }
  } else {
    if constexpr (PRE)
      load_states<M, C, OPT, GUARD>(w, m, v, g0, GS, live, use_m, wv, mv, vv);
#pragma unroll
    for (int u = 0; u < C; ++u) {
      GradRaw<M> r0;
      if (live[u]) r0.load(gs.p[0], g0 + (int64_t)u * GS);
      r0.widen(s[u]);
    }
    constexpr int B = kWideBatch;
    for (int k0 = 1; k0 < N; k0 += B) {
      GradRaw<M> raw[C][B];
#pragma unroll
      for (int u = 0; u < C; ++u)
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (k0 + j < N && live[u]) raw[u][j].load(gs.p[k0 + j], g0 + (int64_t)u * GS);
#pragma unroll
      for (int u = 0; u < C; ++u)
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (k0 + j < N) raw[u][j].add(s[u]);
    }
  }

#pragma unroll
  for (int u = 0; u < C; ++u) {
    if (!live[u]) continue;
    const int64_t g = g0 + (int64_t)u * GS;
    if constexpr (ISSUE == 0) {
      StateIO<M>::load(w, g, wv[u]);
      if (use_m) StateIO<M>::load(m, g, mv[u]);
      if (OPT == 0) StateIO<M>::load(v, g, vv[u]);
    }
    if constexpr (MEAN) {  // the averaged gradient, as the update below forms it
      S gb[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) gb[e] = s[u][e] / c.nw;
      StateIO<M>::store(mean_out, g, gb);
    }
    uint32_t dbits = 0;
    if (decay_kind == 1) dbits = (1u << VEC) - 1u;
    else if (decay_kind == 2) dbits = decay_bits<VEC>(mask, mask_off + g * VEC);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if constexpr (OPT == 0)
        adam_element<S>(s[u][e], wv[u][e], mv[u][e], vv[u][e], (dbits >> e) & 1u, c, clip, coef);
      else
        sgd_element<S>(s[u][e], wv[u][e], mv[u][e], (dbits >> e) & 1u, c, clip, coef);
    }
    if (use_m) StateIO<M>::store(m, g, mv[u]);
    if (OPT == 0) StateIO<M>::store(v, g, vv[u]);
    StateIO<M>::store(w, g, wv[u]);
    if (out != nullptr) {
      if (out_vec) {
        OutIO<M>::store_vec(out, g, wv[u]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) out[g * VEC + e] = OutIO<M>::conv(wv[u][e]);
      }
    }
  }
}

// The fused step. NFIX > 0: exactly NFIX workers; NFIX == 0: any N <= CAP,
// loaded in batches of 8 workers. Each thread handles C groups of one tile.
template <class M, int NFIX, int CAP, int BLOCK, int C, int OPT, int ISSUE, bool WC, bool MEAN>
__global__ void __launch_bounds__(BLOCK)
    zero_step_kernel(GradSet<CAP> gs, int nw, typename M::S* __restrict__ w,
                     typename M::S* __restrict__ m, typename M::S* __restrict__ v,
                     typename M::P* __restrict__ out, int out_vec,
                     typename M::S* __restrict__ mean_out, int64_t len,
                     Consts<typename M::S> c, const uint32_t* __restrict__ mask,
                     int64_t mask_off, int decay_kind, const double* __restrict__ clip_sumsq,
                     double max_norm, const zlaunch::DynScalars* __restrict__ dyn) {
  typedef typename M::S S;
  constexpr int VEC = M::VEC;
  if (dyn != nullptr) {  // step-dependent scalars from device memory, rounded as on the host
    c.bias1 = (S)dyn->bias1;
    c.bias2 = (S)dyn->bias2;
    c.first = dyn->t == 1;
  }
  const int64_t ngroups = len / VEC;
  constexpr int GS = WC ? 64 : BLOCK;
  const int64_t g0 = WC ? (int64_t)blockIdx.x * (BLOCK * C) + (threadIdx.x / 64) * (64 * C) +
                              (threadIdx.x % 64)
                        : (int64_t)blockIdx.x * (BLOCK * C) + threadIdx.x;
  const bool clip = clip_sumsq != nullptr;
  const S coef = clip ? clip_coef<S>(clip_sumsq, max_norm) : S(1);
  const int N = NFIX > 0 ? NFIX : nw;
  if (g0 + (int64_t)(C - 1) * GS < ngroups)
    step_groups<M, NFIX, CAP, GS, C, OPT, ISSUE, MEAN, false>(gs, N, w, m, v, out, out_vec,
                                                               mean_out, g0, ngroups, c, mask,
                                                               mask_off, decay_kind, clip, coef);
  else if (g0 < ngroups)
    step_groups<M, NFIX, CAP, GS, C, OPT, ISSUE, MEAN, true>(gs, N, w, m, v, out, out_vec,
                                                              mean_out, g0, ngroups, c, mask,
                                                              mask_off, decay_kind, clip, coef);

  // leftover elements (fewer than VEC), one per thread of block 0
  const int64_t i = ngroups * VEC + threadIdx.x;
  if (blockIdx.x == 0 && i < len) {
    typedef typename M::G G;
    S sum = grad_elem(reinterpret_cast<const G*>(gs.p[0]), i);
    for (int k = 1; k < N; ++k) sum = sum + grad_elem(reinterpret_cast<const G*>(gs.p[k]), i);
    if constexpr (MEAN) mean_out[i] = sum / c.nw;
    bool dec = decay_kind == 1;
    if (decay_kind == 2) {
      const int64_t bit = mask_off + i;
      dec = (mask[bit >> 5] >> (bit & 31)) & 1u;
    }
    S wi = w[i];
    if constexpr (OPT == 0) {
      S mi = m[i], vi = v[i];
      adam_element<S>(sum, wi, mi, vi, dec, c, clip, coef);
      m[i] = mi;
      v[i] = vi;
    } else {
      S bi = c.has_mom ? m[i] : S(0);
      sgd_element<S>(sum, wi, bi, dec, c, clip, coef);
      if (c.has_mom) m[i] = bi;
    }
    w[i] = wi;
    if (out != nullptr) out[i] = OutIO<M>::conv(wi);
  }
}

// Deterministic block sum of one double per thread: a butterfly inside each
// wave, then the waves' totals in wave order. The same inputs in the same
// threads give the same bits on every run.
template <int BLOCK>
__device__ __forceinline__ double block_sum(double x) {
  static_assert(BLOCK % 64 == 0, "whole waves");
  __shared__ double wave_tot[BLOCK / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = x + __shfl_xor(x, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) wave_tot[wave] = x;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
    t = wave_tot[0];
#pragma unroll
    for (int k = 1; k < BLOCK / 64; ++k) t = t + wave_tot[k];
  }
  return t;  // meaningful in thread 0
}

// Reduce-scatter mean, materialised: mean[g] for every group of the call's
// range (the same rank-order fold and division as the step, stored in S), and,
// if partials != nullptr, each block's sum of the squares of its means in
// double (squares of fp32 means are exact in double).
template <class M, int NFIX, int CAP, int BLOCK, int C>
__global__ void __launch_bounds__(BLOCK)
    zero_mean_kernel(GradSet<CAP> gs, int nw, typename M::S* __restrict__ mean, int64_t len,
                     typename M::S nws, double* __restrict__ partials) {
  typedef typename M::S S;
  constexpr int VEC = M::VEC;
  const int64_t ngroups = len / VEC;
  const int64_t g0 = (int64_t)blockIdx.x * (BLOCK * C) + threadIdx.x;
  const int N = NFIX > 0 ? NFIX : nw;
  bool live[C];
#pragma unroll
  for (int u = 0; u < C; ++u) live[u] = g0 + (int64_t)u * BLOCK < ngroups;

  S s[C][VEC];
  if constexpr (NFIX > 0) {
    GradRaw<M> raw[C][NFIX];
#pragma unroll
    for (int u = 0; u < C; ++u)
#pragma unroll
      for (int k = 0; k < NFIX; ++k)
        if (live[u]) raw[u][k].load(gs.p[k], g0 + (int64_t)u * BLOCK);
#pragma unroll
    for (int u = 0; u < C; ++u) {
      raw[u][0].widen(s[u]);
#pragma unroll
      for (int k = 1; k < NFIX; ++k) raw[u][k].add(s[u]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < C; ++u) {
      GradRaw<M> r0;
      if (live[u]) r0.load(gs.p[0], g0 + (int64_t)u * BLOCK);
      r0.widen(s[u]);
    }
    constexpr int B = kWideBatch;
    for (int k0 = 1; k0 < N; k0 += B) {
      GradRaw<M> raw[C][B];
#pragma unroll
      for (int u = 0; u < C; ++u)
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (k0 + j < N && live[u]) raw[u][j].load(gs.p[k0 + j], g0 + (int64_t)u * BLOCK);
#pragma unroll
      for (int u = 0; u < C; ++u)
#pragma unroll
        for (int j = 0; j < B; ++j)
          if (k0 + j < N) raw[u][j].add(s[u]);
    }
  }
  double sq = 0.0;
#pragma unroll
  for (int u = 0; u < C; ++u) {
    if (!live[u]) continue;
    S gb[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      gb[e] = s[u][e] / nws;
      const double d = (double)gb[e];
      sq = sq + d * d;
    }
    StateIO<M>::store(mean, g0 + (int64_t)u * BLOCK, gb);
  }
  // leftover elements, one per thread of block 0
  const int64_t i = ngroups * VEC + threadIdx.x;
  if (blockIdx.x == 0 && i < len) {
    typedef typename M::G G;
    S sum = grad_elem(reinterpret_cast<const G*>(gs.p[0]), i);
    for (int k = 1; k < N; ++k) sum = sum + grad_elem(reinterpret_cast<const G*>(gs.p[k]), i);
    const S gb = sum / nws;
    mean[i] = gb;
    const double d = (double)gb;
    sq = sq + d * d;
  }
  if (partials != nullptr) {
    const double t = block_sum<BLOCK>(sq);
    if (threadIdx.x == 0) partials[blockIdx.x] = t;
  }
}

// Sum of the block partials, in a fixed order: thread t adds partials t,
// t + 1024, ... in order, then the block sum.
constexpr int kFinalBlock = 1024;
__global__ void __launch_bounds__(kFinalBlock)
    zero_sumsq_finalize(const double* __restrict__ partials, int64_t count,
                        double* __restrict__ out) {
  double x = 0.0;
  for (int64_t k = threadIdx.x; k < count; k += kFinalBlock) x = x + partials[k];
  const double t = block_sum<kFinalBlock>(x);
  if (threadIdx.x == 0) *out = t;
}

// init_states: m = v = 0; master from the gathered parameters when asked.
template <class M>
__global__ void __launch_bounds__(kInitBlock)
    zero_init_kernel(const typename M::P* __restrict__ param, typename M::S* __restrict__ master,
                     typename M::S* __restrict__ m, typename M::S* __restrict__ v, int64_t len) {
  typedef typename M::S S;
  const int64_t stride = (int64_t)gridDim.x * kInitBlock;
  for (int64_t i = (int64_t)blockIdx.x * kInitBlock + threadIdx.x; i < len; i += stride) {
    m[i] = S(0);
    if (v != nullptr) v[i] = S(0);
    if (master != nullptr) {
      if constexpr (std::is_same_v<M, ModeMixedF16>)
        master[i] = f16_to_f32(param[i]);
      else if constexpr (sizeof(typename M::P) == 2)
        master[i] = bf16_to_f32(param[i]);
      else
        master[i] = param[i];
    }
  }
}

int device_cus() {
  // one query per device; the count is the same for every launch on it. Atomic
  // so that threads launching at once may fill the cache together (each stores
  // the same value).
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
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
  c.wd = (S)a.weight_decay;
  c.mom = (S)a.momentum;
  c.omd = (S)a.one_minus_dampening;
  c.has_mom = a.momentum != 0.0;
  c.nesterov = a.nesterov;
  c.first = a.first;
  return c;
}

// A launch shape: BLOCK threads, C groups per thread, ISSUE, WC, CU_BLOCKS (as
// in the shape table at the top of this file).
template <int BLOCK_, int C_, int ISSUE_, bool WC_, int CU_BLOCKS_ = 0>
struct LaunchShape {
  static constexpr int BLOCK = BLOCK_, C = C_, ISSUE = ISSUE_, CU_BLOCKS = CU_BLOCKS_;
  static constexpr bool WC = WC_;
};
// Per mode: the bulk shape, used when the launch has at least ROUNDS full
// rounds of resident blocks (ROUNDS * CU_BLOCKS blocks per CU), and the wide
// shape below that. A serial-issue bulk shape keeps few loads in flight per
// wave and relies on many resident waves over many rounds: on a launch that
// fills the chip only once or twice, the chain of dependent loads of each
// wave is the critical path, and the wide shape (every load of a thread in
// flight at once) is faster. A mode with no bulk shape has ROUNDS = 0 and the
// same shape twice.
template <class M>
struct Shape;
template <>
struct Shape<ModeF64> {
  typedef LaunchShape<ZERO_F64_BLOCK, ZERO_F64_GROUPS, ZERO_F64_ISSUE, ZERO_F64_WC> Bulk;
  typedef Bulk Wide;
  static constexpr int ROUNDS = 0;
};
template <>
struct Shape<ModeF32> {
  typedef LaunchShape<ZERO_F32_BLOCK, ZERO_F32_GROUPS, ZERO_F32_ISSUE, ZERO_F32_WC,
                      ZERO_F32_CU_BLOCKS>
      Bulk;
  typedef LaunchShape<ZERO_F32_WIDE_BLOCK, ZERO_F32_WIDE_GROUPS, ZERO_F32_WIDE_ISSUE,
                      ZERO_F32_WIDE_WC>
      Wide;
  static constexpr int ROUNDS = ZERO_F32_ROUNDS;
};
template <>
struct Shape<ModeMixed> {
  typedef LaunchShape<ZERO_MIX_BLOCK, ZERO_MIX_GROUPS, ZERO_MIX_ISSUE, ZERO_MIX_WC,
                      ZERO_MIX_CU_BLOCKS>
      Bulk;
  typedef LaunchShape<ZERO_MIX_WIDE_BLOCK, ZERO_MIX_WIDE_GROUPS, ZERO_MIX_WIDE_ISSUE,
                      ZERO_MIX_WIDE_WC>
      Wide;
  static constexpr int ROUNDS = ZERO_MIX_ROUNDS;
};
template <>
struct Shape<ModeMixedF16> : Shape<ModeMixed> {};
// the step kernel's shapes for NFIX fixed workers (0: any N)
template <class M, int NFIX>
struct StepShape : Shape<M> {};
template <>
struct StepShape<ModeF32, 0> {
  typedef LaunchShape<ZERO_F32W_BLOCK, ZERO_F32W_GROUPS, ZERO_F32W_ISSUE, ZERO_F32W_WC> Bulk;
  typedef Bulk Wide;
  static constexpr int ROUNDS = 0;
};

// LDS bytes per CU of the current device (one query per device, as device_cus).
int device_lds_per_cu() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int lds = cached[dev].load(std::memory_order_relaxed);
  if (lds == 0) {
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        lds <= 0)
      lds = -1;
    cached[dev].store(lds, std::memory_order_relaxed);
  }
  return lds > 0 ? lds : 0;
}

// Dynamic LDS bytes that let at most `cu_blocks` blocks of a launch reside on
// one CU at a time (0: no cap). The step kernel does not touch LDS: the
// allocation only limits how many blocks the hardware places on a CU, and so
// how many loads are in flight chip-wide. Whole 512-byte granules; no cap if
// the device does not report its LDS size or the bytes would pass the
// per-block limit.
size_t occupancy_cap_lds(int cu_blocks) {
  if (cu_blocks <= 0) return 0;
  const int lds = device_lds_per_cu();
  if (lds <= 0) return 0;
  int bytes = lds / cu_blocks;
  bytes -= bytes % 512;
  if (bytes <= 0 || bytes > 65536 || (int64_t)bytes * (cu_blocks + 1) <= lds) return 0;
  return (size_t)bytes;
}

// Launches the step in the shape (BLOCK, C, ISSUE, WC): one tile of BLOCK * C
// groups per block, and at least one block for the leftover elements; at most
// CU_BLOCKS blocks per CU at a time when CU_BLOCKS > 0.
template <class M, int NFIX, int CAP, int BLOCK, int C, int ISSUE, bool WC, bool MEAN,
          int CU_BLOCKS>
void launch_shaped(const zlaunch::StepArgs& a, hipStream_t st, const GradSet<CAP>& gs,
                   int out_vec) {
  typedef typename M::S S;
  typedef typename M::P P;
  const int64_t ngroups = a.len / M::VEC;
  const int64_t per_block = (int64_t)BLOCK * C;
  int64_t blocks = (ngroups + per_block - 1) / per_block;
  if (blocks < 1) blocks = 1;
  const size_t lds = occupancy_cap_lds(CU_BLOCKS);
  if (a.optimizer == 0)
    hipLaunchKernelGGL((zero_step_kernel<M, NFIX, CAP, BLOCK, C, 0, ISSUE, WC, MEAN>),
                       dim3((unsigned)blocks), dim3(BLOCK), lds, st, gs, a.n_workers,
                       static_cast<S*>(a.w), static_cast<S*>(a.m), static_cast<S*>(a.v),
                       static_cast<P*>(a.out), out_vec, static_cast<S*>(a.mean_out), a.len,
                       round_consts<S>(a), a.mask, a.mask_bit_offset, a.decay_kind,
                       a.clip_sumsq, a.max_norm, static_cast<const zlaunch::DynScalars*>(a.dyn));
  else
    hipLaunchKernelGGL((zero_step_kernel<M, NFIX, CAP, BLOCK, C, 1, ISSUE, WC, MEAN>),
                       dim3((unsigned)blocks), dim3(BLOCK), lds, st, gs, a.n_workers,
                       static_cast<S*>(a.w), static_cast<S*>(a.m), static_cast<S*>(a.v),
                       static_cast<P*>(a.out), out_vec, static_cast<S*>(a.mean_out), a.len,
                       round_consts<S>(a), a.mask, a.mask_bit_offset, a.decay_kind,
                       a.clip_sumsq, a.max_norm, static_cast<const zlaunch::DynScalars*>(a.dyn));
}

// Small launches (a bucket of a few MiB) take 256 x 1 tiles when the mode's
// own shape would give fewer than two blocks per CU: the launch then spreads
// over every CU instead of a quarter of them (1 MiB fp32 bucket, 8 workers:
// 4.3 us against 5.8-6.3 us on MI355X). The arithmetic is the same.
#ifndef ZERO_SMALL_BLOCK
#define ZERO_SMALL_BLOCK 256
#endif
#ifndef ZERO_SMALL_ISSUE
#define ZERO_SMALL_ISSUE 0
#endif
constexpr int kSmallBlock = ZERO_SMALL_BLOCK;
constexpr int kSmallIssue = ZERO_SMALL_ISSUE;

// The wide shape W, or 256 x 1 tiles when W would give fewer than two blocks
// per CU.
template <class M, int NFIX, int CAP, bool MEAN, class W>
void launch_wide(const zlaunch::StepArgs& a, hipStream_t st, const GradSet<CAP>& gs,
                 int out_vec) {
  if constexpr (W::BLOCK * W::C > kSmallBlock) {
    const int64_t per_block = (int64_t)W::BLOCK * W::C;
    const int64_t blocks = (a.len / M::VEC + per_block - 1) / per_block;
    if (blocks < 2 * (int64_t)device_cus()) {
      launch_shaped<M, NFIX, CAP, kSmallBlock, 1, kSmallIssue, false, MEAN, 0>(a, st, gs,
                                                                                out_vec);
      return;
    }
  }
  launch_shaped<M, NFIX, CAP, W::BLOCK, W::C, W::ISSUE, W::WC, MEAN, W::CU_BLOCKS>(a, st, gs,
                                                                                    out_vec);
}

template <class M, int NFIX, int CAP, bool MEAN>
void launch_mode_nm(const zlaunch::StepArgs& a, hipStream_t st) {
  typedef StepShape<M, NFIX> SH;
  typedef typename SH::Bulk B;
  GradSet<CAP> gs;
  for (int k = 0; k < CAP; ++k) gs.p[k] = k < a.n_workers ? a.grads[k] : nullptr;
  const int out_vec =
      a.out != nullptr && (reinterpret_cast<uintptr_t>(a.out) % OutIO<M>::kAlign == 0);
  if constexpr (SH::ROUNDS > 0) {
    const int64_t per_block = (int64_t)B::BLOCK * B::C;
    const int64_t blocks = (a.len / M::VEC + per_block - 1) / per_block;
    if (blocks >= (int64_t)SH::ROUNDS * B::CU_BLOCKS * device_cus()) {
      launch_shaped<M, NFIX, CAP, B::BLOCK, B::C, B::ISSUE, B::WC, MEAN, B::CU_BLOCKS>(a, st, gs,
                                                                                      out_vec);
      return;
    }
  }
  launch_wide<M, NFIX, CAP, MEAN, typename SH::Wide>(a, st, gs, out_vec);
}

// The step, with the averaged gradient also stored when a.mean_out is set (the
// step from a materialised mean never stores it again).
template <class M, int NFIX, int CAP>
void launch_mode_n(const zlaunch::StepArgs& a, hipStream_t st) {
  if (a.mean_out != nullptr) launch_mode_nm<M, NFIX, CAP, true>(a, st);
  else launch_mode_nm<M, NFIX, CAP, false>(a, st);
}

template <class M>
void launch_mode(const zlaunch::StepArgs& a, hipStream_t st) {
  switch (a.n_workers) {
    case 1: launch_mode_n<M, 1, 1>(a, st); break;
    case 2: launch_mode_n<M, 2, 2>(a, st); break;
    case 4: launch_mode_n<M, 4, 4>(a, st); break;
    case 8: launch_mode_n<M, 8, 8>(a, st); break;
    default:
      if (a.n_workers <= 64) launch_mode_n<M, 0, 64>(a, st);
      else launch_mode_n<M, 0, zlaunch::kMaxWorkers>(a, st);
      break;
  }
}

// The step from a materialised fp32 mean reads only 16-byte groups, as the
// fp32 step does, and takes the fp32 step's residency cap and rounds.
template <>
struct Shape<ModeMixedMean> {
  typedef LaunchShape<ZERO_MIX_BLOCK, ZERO_MIX_GROUPS, ZERO_MIX_ISSUE, ZERO_MIX_WC,
                      ZERO_MIXMEAN_CU_BLOCKS>
      Bulk;
  typedef Shape<ModeMixed>::Wide Wide;
  static constexpr int ROUNDS = ZERO_MIXMEAN_ROUNDS;
};
template <>
struct Shape<ModeMixedF16Mean> : Shape<ModeMixedMean> {};

// The materialised mean's own launch shape (its block count is the number of
// partial sums of the squared norm, which the workspace queries and the
// library's static scratch are sized by): 512 x 2 groups, 256 x 1 in fp64.
template <class M>
struct MeanShape {
  static constexpr int BLOCK = 512, C = 2;
};
template <>
struct MeanShape<ModeF64> {
  static constexpr int BLOCK = 256, C = 1;
};

template <class M>
int64_t mean_blocks(int64_t len) {
  const int64_t per_block = (int64_t)MeanShape<M>::BLOCK * MeanShape<M>::C;
  const int64_t b = (len / M::VEC + per_block - 1) / per_block;
  return b < 1 ? 1 : b;
}

template <class M, int NFIX, int CAP>
void launch_mean_n(const zlaunch::MeanArgs& a, hipStream_t st) {
  typedef typename M::S S;
  constexpr int BLOCK = MeanShape<M>::BLOCK, C = MeanShape<M>::C;
  const int64_t blocks = mean_blocks<M>(a.len);
  GradSet<CAP> gs;
  for (int k = 0; k < CAP; ++k) gs.p[k] = k < a.n_workers ? a.grads[k] : nullptr;
  hipLaunchKernelGGL((zero_mean_kernel<M, NFIX, CAP, BLOCK, C>), dim3((unsigned)blocks),
                     dim3(BLOCK), 0, st, gs, a.n_workers, static_cast<S*>(a.mean), a.len,
                     (S)a.n_workers_value, a.partials);
}

template <class M>
void launch_mean_mode(const zlaunch::MeanArgs& a, hipStream_t st) {
  switch (a.n_workers) {
    case 1: launch_mean_n<M, 1, 1>(a, st); break;
    case 2: launch_mean_n<M, 2, 2>(a, st); break;
    case 4: launch_mean_n<M, 4, 4>(a, st); break;
    case 8: launch_mean_n<M, 8, 8>(a, st); break;
    default:
      if (a.n_workers <= 64) launch_mean_n<M, 0, 64>(a, st);
      else launch_mean_n<M, 0, zlaunch::kMaxWorkers>(a, st);
      break;
  }
}

template <class M>
void launch_init_mode(const zlaunch::InitArgs& a, hipStream_t st) {
  typedef typename M::S S;
  typedef typename M::P P;
  int64_t want = (a.len + kInitBlock - 1) / kInitBlock;
  const int64_t cap = (int64_t)device_cus() * 8;
  int blocks = (int)(want < 1 ? 1 : (want > cap ? cap : want));
  hipLaunchKernelGGL((zero_init_kernel<M>), dim3(blocks), dim3(kInitBlock), 0, st,
                     static_cast<const P*>(a.param), static_cast<S*>(a.master),
                     static_cast<S*>(a.m), static_cast<S*>(a.v), a.len);
}

}  // namespace

// Library-owned scratch for callers that cannot allocate device memory: the
// squared norm's per-block partial sums of zero_mean_grad_noalloc. Each GPU the
// library runs on holds its own copy until the process ends. In host code the
// name is only a stand-in for the device symbol: its device address is looked
// up once per device (scratch_address) and that address is what kernels get.
static __device__ __align__(256) double scratch[zlaunch::kScratchDoubles];

namespace zlaunch {

const char* scratch_address(void* stream, double** out) {
  // The device the stream belongs to (the null stream: the current device).
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                                   : hipGetDevice(&dev);
  if (e != hipSuccess) return hipGetErrorString(e);
  constexpr int kMaxDevices = 64;
  if (dev < 0 || dev >= kMaxDevices) return "device ordinal outside the scratch table";
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // with that device current, once per device
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hipGetErrorString(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hipGetErrorString(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hipGetErrorString(e);
    if (back != hipSuccess) return hipGetErrorString(back);
    if (p == nullptr) return "hipGetSymbolAddress returned NULL for the scratch array";
    addr[dev] = p;
  }
  *out = static_cast<double*>(addr[dev]);
  return nullptr;
}

const char* launch_step(const StepArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the check below is this launch's
  switch (a.mode) {
    case 0: launch_mode<ModeF64>(a, st); break;
    case 1: launch_mode<ModeF32>(a, st); break;
    case 2: launch_mode<ModeMixed>(a, st); break;
    case 3: launch_mode<ModeMixedF16>(a, st); break;
    default: return "unknown mode";
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? nullptr : hipGetErrorString(e);
}

const char* launch_step_mean(const StepArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (a.mean_out != nullptr) return "the step from a materialised mean stores no mean";
  switch (a.mode) {
    case 0: launch_mode_nm<ModeF64, 1, 1, false>(a, st); break;
    case 1: launch_mode_nm<ModeF32, 1, 1, false>(a, st); break;
    case 2: launch_mode_nm<ModeMixedMean, 1, 1, false>(a, st); break;
    case 3: launch_mode_nm<ModeMixedF16Mean, 1, 1, false>(a, st); break;
    default: return "unknown mode";
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? nullptr : hipGetErrorString(e);
}

int64_t mean_partials(int mode, int64_t len) {
  switch (mode) {
    case 0: return mean_blocks<ModeF64>(len);
    case 1: return mean_blocks<ModeF32>(len);
    case 3: return mean_blocks<ModeMixedF16>(len);
    default: return mean_blocks<ModeMixed>(len);
  }
}

const char* launch_mean(const MeanArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  switch (a.mode) {
    case 0: launch_mean_mode<ModeF64>(a, st); break;
    case 1: launch_mean_mode<ModeF32>(a, st); break;
    case 2: launch_mean_mode<ModeMixed>(a, st); break;
    case 3: launch_mean_mode<ModeMixedF16>(a, st); break;
    default: return "unknown mode";
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? nullptr : hipGetErrorString(e);
}

const char* launch_sumsq_finalize(const double* partials, int64_t count, double* out,
                                  void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(zero_sumsq_finalize, dim3(1), dim3(kFinalBlock), 0, st, partials, count,
                     out);
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
    case 3: launch_init_mode<ModeMixedF16>(a, st); break;
    default: return "unknown mode";
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? nullptr : hipGetErrorString(e);
}

}  // namespace zlaunch
