// Streaming ceiling kernels, used to measure what the memory system delivers
// for a given mix of streams; not part of the optimizer's interface.
//
// zceil_streams reads nin streams and writes nout streams, group by group, with
// the fused step's access pattern and no floating-point arithmetic: each group
// index g reads 8 or 16 bytes of every input stream (as the step reads a bf16 or
// an fp32/fp64 group), folds them with XOR so that no load is dead, and writes
// 8 or 16 bytes of the result to every output stream. The launch shapes are
// those the step uses (BLOCK threads, C groups per thread, BLOCK or 64 groups
// apart), all loads of a thread are issued before any is used, and loads and
// stores carry the nontemporal hint. With one input and one output it is a
// copy; with the step's own streams it is the step without its arithmetic.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxIn = 16;       // streams held in registers all at once
constexpr int kMaxWideIn = 128;  // streams loaded in batches of kBatch
constexpr int kBatch = 8;
constexpr int kMaxOut = 4;
constexpr int kShapes = 7;  // shape 0: 512 x 2, 512 apart; 1: 512 x 2, 64 apart;
                            // 2: 256 x 4, 64 apart; 3: 256 x 1; 4: 128 x 8, 64 apart;
                            // 5: 64 x 2, 64 apart, one stream in flight per wave;
                            // 6: shape 5 with at most 16 blocks per CU

struct Streams {
  const void* in[kMaxWideIn];
  void* out[kMaxOut];
  uint32_t in_wide[kMaxWideIn / 32];  // bit i: input i is read 16 bytes per group, else 8
};

__device__ __forceinline__ u32x4 load_group(const Streams& s, int i, int64_t g) {
  if ((s.in_wide[i / 32] >> (i % 32)) & 1u)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s.in[i]) + g);
  const u32x2 h = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(s.in[i]) + g);
  return u32x4{h.x, h.y, 0u, 0u};
}

template <int NOUT>
__device__ __forceinline__ void store_group(const Streams& s, uint32_t out_wide, int64_t g,
                                            u32x4 acc) {
#pragma unroll
  for (int o = 0; o < NOUT; ++o) {
    if ((out_wide >> o) & 1u)
      __builtin_nontemporal_store(acc, reinterpret_cast<u32x4*>(s.out[o]) + g);
    else
      __builtin_nontemporal_store(u32x2{acc.x, acc.y}, reinterpret_cast<u32x2*>(s.out[o]) + g);
  }
}

// NIN > 0: exactly NIN inputs, all loads of a thread issued before any is used.
// NIN == 0: nin inputs in batches of kBatch (the step's any-N loop).
template <int NIN, int NOUT, int BLOCK, int C, bool WC>
__global__ void __launch_bounds__(BLOCK)
    ceiling_kernel(Streams s, int nin, uint32_t out_wide, int64_t ngroups) {
  constexpr int GS = WC ? 64 : BLOCK;
  const int64_t g0 = WC ? (int64_t)blockIdx.x * (BLOCK * C) + (threadIdx.x / 64) * (64 * C) +
                              (threadIdx.x % 64)
                        : (int64_t)blockIdx.x * (BLOCK * C) + threadIdx.x;
  u32x4 acc[C];
  if constexpr (NIN > 0) {
    u32x4 r[C][NIN];
#pragma unroll
    for (int u = 0; u < C; ++u) {
      const int64_t g = g0 + (int64_t)u * GS;
      if (g >= ngroups) continue;
#pragma unroll
      for (int i = 0; i < NIN; ++i) r[u][i] = load_group(s, i, g);
    }
#pragma unroll
    for (int u = 0; u < C; ++u) {
      acc[u] = r[u][0];
#pragma unroll
      for (int i = 1; i < NIN; ++i) acc[u] ^= r[u][i];
    }
  } else {
#pragma unroll
    for (int u = 0; u < C; ++u) acc[u] = u32x4{0u, 0u, 0u, 0u};
    for (int k0 = 0; k0 < nin; k0 += kBatch) {
      u32x4 r[C][kBatch];
#pragma unroll
      for (int u = 0; u < C; ++u) {
        const int64_t g = g0 + (int64_t)u * GS;
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          if (g < ngroups && k0 + j < nin) r[u][j] = load_group(s, k0 + j, g);
      }
#pragma unroll
      for (int u = 0; u < C; ++u)
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
          if (k0 + j < nin) acc[u] ^= r[u][j];
    }
  }
#pragma unroll
  for (int u = 0; u < C; ++u) {
    const int64_t g = g0 + (int64_t)u * GS;
    if (g < ngroups) store_group<NOUT>(s, out_wide, g, acc[u]);
  }
}

// A zero that exists only once `word` (just loaded) and the previous token have
// arrived; adding it to the next load's index makes that load wait for this one.
__device__ __forceinline__ uint32_t after(uint32_t word, uint32_t prev) {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z) : "v"(word), "v"(prev));
  return z;
}

// Shape 5, the fused step's issue mode for the mixed precisions: 64 threads x 2
// groups 64 apart; the inputs are loaded one stream at a time, each stream's two
// loads waiting for the previous stream's to return.
template <int NOUT>
__global__ void __launch_bounds__(64)
    ceiling_serial_kernel(Streams s, int nin, uint32_t out_wide, int64_t ngroups) {
  constexpr int C = 2;
  const int64_t g0 = (int64_t)blockIdx.x * (64 * C) + threadIdx.x;
  u32x4 acc[C];
#pragma unroll
  for (int u = 0; u < C; ++u) acc[u] = u32x4{0u, 0u, 0u, 0u};
  uint32_t tok = 0;
  for (int i = 0; i < nin; ++i) {
    u32x4 r[C];
#pragma unroll
    for (int u = 0; u < C; ++u) {
      const int64_t g = g0 + (int64_t)u * 64;
      r[u] = g < ngroups ? load_group(s, i, g + tok) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < C; ++u) {
      tok = after(r[u].x, tok);
      acc[u] ^= r[u];
    }
  }
#pragma unroll
  for (int u = 0; u < C; ++u) {
    const int64_t g = g0 + (int64_t)u * 64;
    if (g < ngroups) store_group<NOUT>(s, out_wide, g, acc[u]);
  }
}

// Dynamic LDS bytes that let at most `cu_blocks` blocks reside on a CU at once
// (the kernel never touches LDS; 0 if the device does not report its LDS size).
size_t cap_lds(int cu_blocks) {
  int dev = 0, lds = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
          hipSuccess ||
      lds <= 0)
    return 0;
  int bytes = lds / cu_blocks;
  bytes -= bytes % 512;
  if (bytes <= 0 || bytes > 65536 || (int64_t)bytes * (cu_blocks + 1) <= lds) return 0;
  return (size_t)bytes;
}

template <int NOUT>
hipError_t launch_serial(const Streams& s, int nin, uint32_t ow, int64_t ngroups, size_t lds,
                         hipStream_t st) {
  const int64_t blocks = (ngroups + 127) / 128;
  hipLaunchKernelGGL((ceiling_serial_kernel<NOUT>), dim3((unsigned)blocks), dim3(64), lds, st, s,
                     nin, ow, ngroups);
  return hipGetLastError();
}

hipError_t launch_serial_out(int nout, const Streams& s, int nin, uint32_t ow, int64_t ng,
                             size_t lds, hipStream_t st) {
  switch (nout) {
    case 1: return launch_serial<1>(s, nin, ow, ng, lds, st);
    case 2: return launch_serial<2>(s, nin, ow, ng, lds, st);
    case 3: return launch_serial<3>(s, nin, ow, ng, lds, st);
    default: return launch_serial<4>(s, nin, ow, ng, lds, st);
  }
}

template <int NIN, int NOUT, int BLOCK, int C, bool WC>
hipError_t launch(const Streams& s, int nin, uint32_t out_wide, int64_t ngroups, hipStream_t st) {
  const int64_t per_block = (int64_t)BLOCK * C;
  const int64_t blocks = (ngroups + per_block - 1) / per_block;
  hipLaunchKernelGGL((ceiling_kernel<NIN, NOUT, BLOCK, C, WC>), dim3((unsigned)blocks),
                     dim3(BLOCK), 0, st, s, nin, out_wide, ngroups);
  return hipGetLastError();
}

// shape 4 (8 groups per thread) holds too many registers for all-at-once
// loads, so it always takes the batched kernel
template <int NIN, int NOUT>
hipError_t launch_shape(int shape, const Streams& s, int nin, uint32_t ow, int64_t ng,
                        hipStream_t st) {
  switch (shape) {
    case 0: return launch<NIN, NOUT, 512, 2, false>(s, nin, ow, ng, st);
    case 1: return launch<NIN, NOUT, 512, 2, true>(s, nin, ow, ng, st);
    case 2: return launch<NIN, NOUT, 256, 4, true>(s, nin, ow, ng, st);
    case 3: return launch<NIN, NOUT, 256, 1, false>(s, nin, ow, ng, st);
    default: return launch<0, NOUT, 128, 8, true>(s, nin, ow, ng, st);
  }
}

template <int NIN>
hipError_t launch_out(int nout, int shape, const Streams& s, int nin, uint32_t ow, int64_t ng,
                      hipStream_t st) {
  switch (nout) {
    case 1: return launch_shape<NIN, 1>(shape, s, nin, ow, ng, st);
    case 2: return launch_shape<NIN, 2>(shape, s, nin, ow, ng, st);
    case 3: return launch_shape<NIN, 3>(shape, s, nin, ow, ng, st);
    default: return launch_shape<NIN, 4>(shape, s, nin, ow, ng, st);
  }
}

// NIN = nin for nin <= kMaxIn, else 0 (batched)
template <int NIN>
hipError_t launch_in(int nin, int nout, int shape, const Streams& s, uint32_t ow, int64_t ng,
                     hipStream_t st) {
  if constexpr (NIN > kMaxIn) {
    return launch_out<0>(nout, shape, s, nin, ow, ng, st);
  } else {
    if (nin == NIN) return launch_out<NIN>(nout, shape, s, nin, ow, ng, st);
    return launch_in<NIN + 1>(nin, nout, shape, s, ow, ng, st);
  }
}

}  // namespace

extern "C" {

// Reads in[0..nin) and writes out[0..nout) over ngroups groups; in_width[i] and
// out_width[o] are the bytes per group of each stream (8 or 16), so stream i
// holds ngroups * in_width[i] bytes. Device pointers, aligned to their width;
// 1 <= nin <= 128, 1 <= nout <= 4, ngroups >= 0; shape selects the launch
// shape: 0 = 512 threads x 2 groups 512 apart, 1 = 512 x 2 groups 64 apart,
// 2 = 256 x 4 groups 64 apart, 3 = 256 x 1, 4 = 128 x 8 groups 64 apart,
// 5 = 64 x 2 groups 64 apart with one input stream in flight per wave, 6 = shape 5
// with at most 16 blocks resident per CU (the fused step's mixed-precision
// launch). Up to 16
// inputs (shapes 0-3) are loaded all at once; more, or shape 4, in batches of
// 8. Launches on `stream` (a
// hipStream_t, or NULL) and returns at once. Returns 0, -1 for an invalid
// argument (nothing launched), or -3 for a HIP launch error.
int zceil_streams(const void* const* in, const int32_t* in_width, int32_t nin, void* const* out,
                  const int32_t* out_width, int32_t nout, int64_t ngroups, int32_t shape,
                  void* stream) {
  if (in == nullptr || in_width == nullptr || out == nullptr || out_width == nullptr) return -1;
  if (nin < 1 || nin > kMaxWideIn || nout < 1 || nout > kMaxOut || ngroups < 0) return -1;
  if (shape < 0 || shape >= kShapes) return -1;
  if (ngroups == 0) return 0;
  if (ngroups > (int64_t)0x7FFFFFFF * 256) return -1;
  if (shape >= 5 && ngroups > (int64_t)0x7FFFFFFF) return -1;  // 64-thread blocks
  Streams s{};
  uint32_t ow = 0;
  for (int i = 0; i < nin; ++i) {
    if (in[i] == nullptr || (in_width[i] != 8 && in_width[i] != 16)) return -1;
    if (reinterpret_cast<uintptr_t>(in[i]) % in_width[i] != 0) return -1;
    s.in[i] = in[i];
    if (in_width[i] == 16) s.in_wide[i / 32] |= 1u << (i % 32);
  }
  for (int o = 0; o < nout; ++o) {
    if (out[o] == nullptr || (out_width[o] != 8 && out_width[o] != 16)) return -1;
    if (reinterpret_cast<uintptr_t>(out[o]) % out_width[o] != 0) return -1;
    s.out[o] = out[o];
    if (out_width[o] == 16) ow |= 1u << o;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = shape >= 5 ? launch_serial_out(nout, s, nin, ow, ngroups,
                                                      shape == 6 ? cap_lds(16) : 0, st)
                                  : launch_in<1>(nin, nout, shape, s, ow, ngroups, st);
  return e == hipSuccess ? 0 : -3;
}

}  // extern "C"
