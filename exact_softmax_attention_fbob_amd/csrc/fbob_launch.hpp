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
  // bf16 at d = 64: Pass 1 sums alpha and E' in fp32 from the unrounded products
  bool fp32_row_sums = false;
};

struct FwdArgs {
  const void *Q, *K, *V, *dO;  // dO may be NULL: then D is not written
  float *O, *L, *D;
  // Split key sweep (small grids): part[s][B Hq][N][d] holds split s's unnormalised O,
  // part_ml[s][B Hq][N][2] its reference maximum (log2 units) and row sum.
  float *part = nullptr, *part_ml = nullptr;
  int nsplit = 1;
};

struct Pass1Args {
  const void *Q, *K, *V, *dO, *UQ, *UK, *UV;
  const float *O, *L, *D;
  float *dQt, *ddOt, *alpha, *E;
  // Split key sweep (small grids): part_acc[s][B Hq][N][4][d] holds the four
  // accumulators (B, X, Omega, ddO~') of split s, part_rs[s][B Hq][N][2] its alpha
  // and (where it is summed over keys) E' partial sums; split s covers the s-th of
  // nsplit equal shares of a work-group's key stages.
  float *part_acc = nullptr, *part_rs = nullptr;
  int nsplit = 1;
};

struct Pass2Args {
  const void *Q, *K, *V, *dO, *UQ, *UK, *UV;
  const float *L, *D, *alpha, *E;
  float *dKt, *dVt;
  // Split row sweep (small grids): part[s][B Hkv][N][2][d] holds tau dK~ and dV~ of
  // split s, which covers the s-th of nsplit equal shares of a work-group's row steps.
  float* part = nullptr;
  int nsplit = 1;
};

// How a BoB call spreads small problems over the GPU: each Pass 1 row tile's key
// sweep in s1 parts, each Pass 2 column tile's row sweep in s2 parts (1 = no
// split), and the device workspace the partial sums need.
struct SplitPlan {
  int s1 = 1, s2 = 1;
  // With s1 > 1 (s2 > 1): the first full1 flattened query heads (full2 key/value heads),
  // whole rounds of work-groups, run unsplit and only the rest split; 0 splits every head.
  int64_t full1 = 0, full2 = 0;
  int64_t bytes1 = 0, bytes2 = 0;  // Pass 1 / Pass 2 partials (the two reuse one buffer)
  int64_t bytes() const { return bytes1 > bytes2 ? bytes1 : bytes2; }
};
SplitPlan split_plan(const Problem& p);
// Pass 1 in s1 parts + reduction, then Pass 2 in s2 parts + reduction, on `s`.
hipError_t launch_bob_split(const Problem& p, const Pass1Args& a1, const Pass2Args& a2,
                            const SplitPlan& plan, void* workspace, hipStream_t s);

// First-order backward: the row pass writes dQ and D, the column pass reads D.
struct GradArgs {
  const void *Q, *K, *V, *dO;
  const float *O, *L;
  float *dQ, *dK, *dV, *D;
  // Split sweeps (small grids): the row pass writes part[s][B Hq][N][d] (tau dQ of
  // split s), the column pass part[s][B Hkv][N][2][d] (tau dK, dV); split s covers the
  // s-th of nsplit equal shares of a work-group's key stages or row steps.
  float* part = nullptr;
  int nsplit = 1;
};

hipError_t launch_forward(const Problem& p, const FwdArgs& a, hipStream_t s);
// Split form (a.part, a.part_ml, a.nsplit set; bf16 only), its plan (parts, workspace
// bytes; 1 / 0 = no split) and the split forward with its reduction.
hipError_t launch_forward_split(const Problem& p, const FwdArgs& a, hipStream_t s);
struct FwdPlan {
  int s = 1;
  int64_t bytes = 0;
};
FwdPlan fwd_split_plan(const Problem& p);
hipError_t launch_forward_split_all(const Problem& p, const FwdArgs& a, const FwdPlan& plan,
                                    void* workspace, hipStream_t s);
hipError_t launch_pass1(const Problem& p, const Pass1Args& a, hipStream_t s);
// The partial-sum forms (a.nsplit > 1) of the default Pass 1 / Pass 2 variants.
hipError_t launch_pass1_split(const Problem& p, const Pass1Args& a, hipStream_t s);
hipError_t launch_pass2_split(const Problem& p, const Pass2Args& a, hipStream_t s);
hipError_t launch_pass2(const Problem& p, const Pass2Args& a, hipStream_t s);
hipError_t launch_grad_dq(const Problem& p, const GradArgs& a, hipStream_t s);
hipError_t launch_grad_dkv(const Problem& p, const GradArgs& a, hipStream_t s);
// Split forms (a.part, a.nsplit set; bf16 only) and the plan that picks them: the row
// pass in s1 parts, the column pass in s2 (1 = no split), one workspace of bytes().
hipError_t launch_grad_dq_split(const Problem& p, const GradArgs& a, hipStream_t s);
hipError_t launch_grad_dkv_split(const Problem& p, const GradArgs& a, hipStream_t s);
struct GradPlan {
  int s1 = 1, s2 = 1;
  int64_t bytes1 = 0, bytes2 = 0;  // the two passes reuse one buffer
  int64_t bytes() const { return bytes1 > bytes2 ? bytes1 : bytes2; }
};
GradPlan grad_split_plan(const Problem& p);
hipError_t launch_backward_split(const Problem& p, const GradArgs& a, const GradPlan& plan,
                                 void* workspace, hipStream_t s);

}  // namespace fbob
