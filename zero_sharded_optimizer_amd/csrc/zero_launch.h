// Interface between the host-side ABI layer (zero_abi.cpp: validation, shard
// bounds, step scalars) and the gfx950 kernels (zero_kernels.hip). Plain C++,
// no HIP types, so the ABI layer builds with the host compiler alone.
#pragma once

#include <cstdint>

namespace zlaunch {

constexpr int kMaxWorkers = 256;

// Largest element count one launch covers; the host layer enqueues a longer
// call as consecutive launches on offset views. It is a multiple of every
// kernel's tile (at most 4096 elements), so each piece but the last is whole
// tiles, and in every launch shape blocks x threads stays below the 2^32
// work-items one dispatch can describe.
constexpr int64_t kLaunchElems = INT64_C(1) << 32;

// Everything one fused step launch needs. All pointers are device addresses
// that the ABI layer has validated (alignment, extents, no overlap of written
// ranges).
struct StepArgs {
  int mode;        // 0 fp64, 1 fp32, 2 mixed bf16/fp32, 3 mixed fp16/fp32
  int n_workers;   // 1..kMaxWorkers
  const void* grads[kMaxWorkers];  // rank order; element j of worker k at grads[k][j]
  void* w;         // master values (S): the parameter itself when updated in place
  void* m;         // S
  void* v;         // S
  void* out;       // gathered parameter slot (P) written from w, or nullptr (in place)
  void* mean_out;  // the averaged gradient (S) of each element, or nullptr (not stored)
  int64_t len;     // elements this launch updates, at most kLaunchElems
  const uint32_t* mask;     // decay bitmask or nullptr
  int64_t mask_bit_offset;  // bit index of element 0
  int decay_kind;  // 0 no decay, 1 every element, 2 per the bitmask
  // Step scalars in double; the launch rounds each once to S.
  double beta1, beta2, one_minus_beta1, one_minus_beta2, bias1, bias2, lr, eps,
      decay_factor, n_workers_value;
  // Global-norm clipping: device pointer to the squared norm, or nullptr.
  const double* clip_sumsq;
  double max_norm;
  // Optimizer: 0 Adam/AdamW, 1 momentum SGD (momentum, 1-dampening, weight
  // decay in double; nesterov; first = t == 1).
  int optimizer;
  double momentum, one_minus_dampening, weight_decay;
  int nesterov, first;
  // Device copy of the step-dependent scalars (DynScalars), or nullptr. When
  // set, the kernel takes bias1, bias2 and first from it instead of the
  // values above, so a captured launch can be replayed for later steps.
  const void* dyn;
};

// Layout of the device step scalars (zero_step_scalars in zero_adam.h).
struct DynScalars {
  double bias1, bias2;  // 1 - beta1^t, 1 - beta2^t, formed in double
  int64_t t;            // the 1-based step number
};

// The materialised reduce-scatter mean of one launch's range.
struct MeanArgs {
  int mode;
  int n_workers;
  const void* grads[kMaxWorkers];
  void* mean;            // len elements of S
  int64_t len;           // at most kLaunchElems
  double n_workers_value;
  double* partials;      // mean_partials(mode, len) per-block sums of the squared
                         // mean, or nullptr when no norm is wanted
};

struct InitArgs {
  int mode;
  const void* param;  // source of the master copy (P), or nullptr
  void* master;       // S or nullptr
  void* m;
  void* v;
  int64_t len;
};

// Each returns nullptr on success, or the HIP runtime's error string.
const char* launch_step(const StepArgs& a, void* stream);
const char* launch_init(const InitArgs& a, void* stream);
// The step with grads = {mean}, one "worker" (the mean is already divided).
const char* launch_step_mean(const StepArgs& a, void* stream);
const char* launch_mean(const MeanArgs& a, void* stream);
// Number of per-block partial sums launch_mean writes for a range of len.
int64_t mean_partials(int mode, int64_t len);
// *out = the sum of partials[0 .. count), in a fixed order.
const char* launch_sumsq_finalize(const double* partials, int64_t count, double* out,
                                  void* stream);
// Makes later work on `stream` wait for `event` (a hipEvent_t) to complete.
const char* stream_wait(void* stream, void* event);

// Size, in doubles, of the library's static device scratch (16 MiB per GPU):
// the largest count of block partial sums zero_mean_grad_noalloc accepts.
constexpr int64_t kScratchDoubles = INT64_C(1) << 21;
// *out = the device address of the scratch on the device `stream` belongs to
// (looked up once per device). Returns nullptr on success, else the error.
const char* scratch_address(void* stream, double** out);

}  // namespace zlaunch
