// fbob_launch.hpp - internal interface between the C ABI (fbob_api.hip) and the
// kernel translation units.  Sizes are already validated; pointers are device
// pointers; all launches go to `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Kernel variants.  The shipped library (built without FBOB_TUNING) launches one
// fixed variant per problem class, compiles no other and reads no environment.  A
// measurement build (-DFBOB_TUNING=1, libfbob_tuning.so) also compiles the
// alternatives that were measured against it and lets an environment variable
// FBOB_TUNE_<KERNEL> pick one at each launch (0 = the shipped variant).
#ifndef FBOB_TUNING
#define FBOB_TUNING 0
#endif
#if FBOB_TUNING
#include <stdlib.h>
#endif

namespace fbob {

#if FBOB_TUNING
inline int tune_choice(const char* name) {
  const char* v = getenv(name);
  return v ? atoi(v) : 0;
}
#endif

struct Problem {
  int B, Hq, Hkv, N, d;
  float tau;
  int causal;
  bool bf16;  // storage type of the seven inputs (else fp32)
};

struct FwdArgs {
  const void *Q, *K, *V, *dO;  // dO may be NULL: then D is not written
  float *O, *L, *D;
};

struct Pass1Args {
  const void *Q, *K, *V, *dO, *UQ, *UK, *UV;
  const float *O, *L, *D;
  float *dQt, *ddOt, *alpha, *E;
};

struct Pass2Args {
  const void *Q, *K, *V, *dO, *UQ, *UK, *UV;
  const float *L, *D, *alpha, *E;
  float *dKt, *dVt;
};

// First-order backward: the row pass writes dQ and D, the column pass reads D.
struct GradArgs {
  const void *Q, *K, *V, *dO;
  const float *O, *L;
  float *dQ, *dK, *dV, *D;
};

hipError_t launch_forward(const Problem& p, const FwdArgs& a, hipStream_t s);
hipError_t launch_pass1(const Problem& p, const Pass1Args& a, hipStream_t s);
hipError_t launch_pass2(const Problem& p, const Pass2Args& a, hipStream_t s);
hipError_t launch_grad_dq(const Problem& p, const GradArgs& a, hipStream_t s);
hipError_t launch_grad_dkv(const Problem& p, const GradArgs& a, hipStream_t s);

}  // namespace fbob
