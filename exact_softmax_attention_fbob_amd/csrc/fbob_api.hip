// fbob_api.hip - the C ABI declared in include/fbob.h: argument validation,
// dispatch on (dtype, d, causal) and kernel launch.  Validation happens before
// any HIP call so that every error path is testable on a host without a GPU.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fbob.h"
#include "fbob_launch.hpp"

// Static scratch of fbob_bob_noalloc: the split schedule's fp32 partial sums, for
// callers that cannot allocate.  Each device the library runs on holds its own
// copy until the process ends.  In host code this name is only a stand-in for the
// symbol: kernels get the device address looked up once per device
// (scratch_address below), never the name itself.
static __device__ __align__(256) char scratch[FBOB_SCRATCH_BYTES];

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlap(const Range& x, const Range& y) { return x.lo < y.hi && y.lo < x.hi; }

struct Checked {
  int status;
  fbob::Problem p;
  bool empty;
};

// Shared size/dtype checks.  int32 per-head indexing: N * d must fit in int32 and
// every work-group index must fit in int32.
Checked check_sizes(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                    float tau, int causal) {
  Checked c{FBOB_OK, {}, false};
  if (dtype != FBOB_DTYPE_F32 && dtype != FBOB_DTYPE_BF16) return {FBOB_ERR_INVALID_ARG, {}, false};
  if (B < 0 || Hq < 0 || Hkv < 0 || N < 0 || d < 0) return {FBOB_ERR_INVALID_ARG, {}, false};
  if (!(tau > 0.f) || !isfinite(tau)) return {FBOB_ERR_INVALID_ARG, {}, false};
  if (d != 64 && d != 128) return {FBOB_ERR_UNSUPPORTED, {}, false};
  if (B == 0 || Hq == 0 || N == 0) {
    if (Hkv < 0 || (Hkv == 0 && Hq != 0)) return {FBOB_ERR_INVALID_ARG, {}, false};
    c.empty = true;
  } else {
    if (Hkv == 0 || Hq % Hkv != 0) return {FBOB_ERR_INVALID_ARG, {}, false};
  }
  if (N > (int64_t)INT32_MAX / d) return {FBOB_ERR_UNSUPPORTED, {}, false};
  if (B * Hq > (int64_t)INT32_MAX / 64 || (N / 64 + 1) * B * Hq > (int64_t)INT32_MAX)
    return {FBOB_ERR_UNSUPPORTED, {}, false};
  c.p.B = (int)B;
  c.p.Hq = (int)Hq;
  c.p.Hkv = (int)(Hkv == 0 ? 1 : Hkv);
  c.p.N = (int)N;
  c.p.d = (int)d;
  c.p.tau = tau;
  c.p.causal = causal ? 1 : 0;
  c.p.bf16 = dtype == FBOB_DTYPE_BF16;
  return c;
}

// Pointer checks: non-NULL, 16-byte aligned, outputs disjoint from every other
// buffer.  `ins`/`outs` carry (pointer, byte size).
int check_ptrs(const void* const* ins, const int64_t* in_bytes, int n_in, void* const* outs,
               const int64_t* out_bytes, int n_out) {
  for (int k = 0; k < n_in; ++k)
    if (ins[k] == nullptr) return FBOB_ERR_INVALID_ARG;
  for (int k = 0; k < n_out; ++k)
    if (outs[k] == nullptr) return FBOB_ERR_INVALID_ARG;
  for (int k = 0; k < n_in; ++k)
    if (reinterpret_cast<uintptr_t>(ins[k]) % 16) return FBOB_ERR_ALIGNMENT;
  for (int k = 0; k < n_out; ++k)
    if (reinterpret_cast<uintptr_t>(outs[k]) % 16) return FBOB_ERR_ALIGNMENT;
  for (int k = 0; k < n_out; ++k) {
    const Range o = span(outs[k], out_bytes[k]);
    for (int m = 0; m < n_in; ++m)
      if (overlap(o, span(ins[m], in_bytes[m]))) return FBOB_ERR_ALIAS;
    for (int m = k + 1; m < n_out; ++m)
      if (overlap(o, span(outs[m], out_bytes[m]))) return FBOB_ERR_ALIAS;
  }
  return FBOB_OK;
}

// HIP error behind the calling thread's last FBOB_ERR_HIP (fbob_hip_error_string).
thread_local hipError_t g_last_hip_error = hipSuccess;

int finish(hipError_t e) {
  if (e == hipSuccess) return FBOB_OK;
  g_last_hip_error = e;
  return FBOB_ERR_HIP;
}

// Called after validation, right before an entry point's launches: takes any error
// still pending on the calling thread from earlier HIP calls (the caller's or another
// library's), so that the hipGetLastError after each launch reports that launch only.
void clear_pending() { (void)hipGetLastError(); }

// Pointer checks shared by the BoB entry points: the ten inputs, the six outputs
// and, when it will be used, the workspace of ws_bytes as a seventh output.
int check_bob_ptrs(const Checked& c, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                   const void* Q, const void* K, const void* V, const void* dO, const void* UQ,
                   const void* UK, const void* UV, const float* O, const float* L,
                   const float* D, float* dQt, float* dKt, float* dVt, float* ddOt,
                   float* alpha, float* E, void* workspace, int64_t ws_bytes) {
  const int64_t es = c.p.bf16 ? 2 : 4;
  const int64_t qb = B * Hq * N * d * es, kb = B * Hkv * N * d * es;
  const int64_t ob = B * Hq * N * d * 4, kob = B * Hkv * N * d * 4, rb = B * Hq * N * 4;
  const void* ins[] = {Q, K, V, dO, UQ, UK, UV, O, L, D};
  const int64_t inb[] = {qb, kb, kb, qb, qb, kb, kb, ob, rb, rb};
  void* outs[] = {dQt, dKt, dVt, ddOt, alpha, E, workspace};
  const int64_t outb[] = {ob, kob, kob, ob, rb, rb, ws_bytes};
  return check_ptrs(ins, inb, 10, outs, outb, workspace != nullptr ? 7 : 6);
}

// Both passes on one stream, split when a workspace is given.
int run_bob(const Checked& c, const fbob::SplitPlan& plan, fbob::Pass1Args a1,
            fbob::Pass2Args a2, void* workspace, hipStream_t s) {
  clear_pending();
  if (workspace != nullptr) return finish(fbob::launch_bob_split(c.p, a1, a2, plan, workspace, s));
  const int st = finish(fbob::launch_pass1(c.p, a1, s));
  if (st != FBOB_OK) return st;
  return finish(fbob::launch_pass2(c.p, a2, s));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_address[kMaxDevices] = {};

// Device address of `scratch` on the current device, which must be the stream's:
// looked up with hipGetSymbolAddress on the first call on each device, then cached.
int scratch_address(hipStream_t s, void** out) {
  int dev = -1;
  if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess) return finish(e);
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    if (const hipError_t e = hipStreamGetDevice(s, &sdev); e != hipSuccess) return finish(e);
    if (sdev != dev) return FBOB_ERR_INVALID_ARG;
  }
  if (dev < 0 || dev >= kMaxDevices) return FBOB_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_address[dev] == nullptr) {
    void* addr = nullptr;
    if (const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)); e != hipSuccess)
      return finish(e);
    if (addr == nullptr) return FBOB_ERR_HIP;
    g_scratch_address[dev] = addr;
  }
  *out = g_scratch_address[dev];
  return FBOB_OK;
}

}  // namespace

extern "C" {

int fbob_version(void) { return FBOB_VERSION; }

const char* fbob_hip_error_string(void) {
  return g_last_hip_error == hipSuccess ? "no HIP error" : hipGetErrorName(g_last_hip_error);
}

const char* fbob_strerror(int status) {
  switch (status) {
    case FBOB_OK: return "ok";
    case FBOB_ERR_INVALID_ARG: return "invalid argument";
    case FBOB_ERR_UNSUPPORTED: return "unsupported size or head dimension";
    case FBOB_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case FBOB_ERR_ALIAS: return "output buffer overlaps another buffer";
    case FBOB_ERR_HIP: return "HIP launch error";
    case FBOB_ERR_SCRATCH: return "problem needs more than the static scratch (FBOB_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int fbob_forward(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float tau,
                 int causal, const void* Q, const void* K, const void* V, const void* dO,
                 float* O, float* L, float* D, void* stream) {
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  if (c.empty) return FBOB_OK;
  const int64_t es = c.p.bf16 ? 2 : 4;
  const int64_t qb = B * Hq * N * d * es, kb = B * Hkv * N * d * es;
  const int64_t ob = B * Hq * N * d * 4, rb = B * Hq * N * 4;
  // dO and D are both given (backward row state) or both NULL (forward only).
  if ((dO == nullptr) != (D == nullptr)) return FBOB_ERR_INVALID_ARG;
  const bool with_d = dO != nullptr;
  const void* ins[] = {Q, K, V, dO};
  const int64_t inb[] = {qb, kb, kb, qb};
  void* outs[] = {O, L, D};
  const int64_t outb[] = {ob, rb, rb};
  const int st = check_ptrs(ins, inb, with_d ? 4 : 3, outs, outb, with_d ? 3 : 2);
  if (st != FBOB_OK) return st;
  fbob::FwdArgs a{Q, K, V, dO, O, L, D};
  clear_pending();
  return finish(fbob::launch_forward(c.p, a, static_cast<hipStream_t>(stream)));
}

int fbob_forward_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                int64_t d, float tau, int causal, int64_t* bytes) {
  if (bytes == nullptr) return FBOB_ERR_INVALID_ARG;
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  *bytes = c.empty ? 0 : fbob::fwd_split_plan(c.p).bytes;
  return FBOB_OK;
}

int fbob_forward_ws(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                    float tau, int causal, const void* Q, const void* K, const void* V,
                    const void* dO, float* O, float* L, float* D, void* workspace,
                    int64_t workspace_bytes, void* stream) {
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  if (workspace_bytes < 0) return FBOB_ERR_INVALID_ARG;
  if (c.empty) return FBOB_OK;
  if ((dO == nullptr) != (D == nullptr)) return FBOB_ERR_INVALID_ARG;
  const fbob::FwdPlan plan = fbob::fwd_split_plan(c.p);
  // the split schedule only with a workspace that holds its partial states
  const bool split = plan.bytes > 0 && workspace != nullptr && workspace_bytes >= plan.bytes;
  const bool with_d = dO != nullptr;
  const int64_t es = c.p.bf16 ? 2 : 4;
  const int64_t qb = B * Hq * N * d * es, kb = B * Hkv * N * d * es;
  const int64_t ob = B * Hq * N * d * 4, rb = B * Hq * N * 4;
  const void* ins[] = {Q, K, V, dO};
  const int64_t inb[] = {qb, kb, kb, qb};
  void* outs[] = {O, L, with_d ? D : nullptr, split ? workspace : nullptr};
  const int64_t outb[] = {ob, rb, rb, plan.bytes};
  void* outs_c[4];
  int64_t outb_c[4];
  int n_out = 0;
  for (int i = 0; i < 4; ++i)
    if (outs[i] != nullptr || i < 2) {
      outs_c[n_out] = outs[i];
      outb_c[n_out++] = outb[i];
    }
  const int st = check_ptrs(ins, inb, with_d ? 4 : 3, outs_c, outb_c, n_out);
  if (st != FBOB_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  fbob::FwdArgs a{Q, K, V, dO, O, L, D};
  clear_pending();
  if (split) return finish(fbob::launch_forward_split_all(c.p, a, plan, workspace, s));
  return finish(fbob::launch_forward(c.p, a, s));
}

int fbob_bob_pass1(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float tau,
                   int causal, const void* Q, const void* K, const void* V, const void* dO,
                   const void* UQ, const void* UK, const void* UV, const float* O, const float* L,
                   const float* D, float* dQt, float* ddOt, float* alpha, float* E, void* stream) {
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  if (c.empty) return FBOB_OK;
  const int64_t es = c.p.bf16 ? 2 : 4;
  const int64_t qb = B * Hq * N * d * es, kb = B * Hkv * N * d * es;
  const int64_t ob = B * Hq * N * d * 4, rb = B * Hq * N * 4;
  const void* ins[] = {Q, K, V, dO, UQ, UK, UV, O, L, D};
  const int64_t inb[] = {qb, kb, kb, qb, qb, kb, kb, ob, rb, rb};
  void* outs[] = {dQt, ddOt, alpha, E};
  const int64_t outb[] = {ob, ob, rb, rb};
  const int st = check_ptrs(ins, inb, 10, outs, outb, 4);
  if (st != FBOB_OK) return st;
  fbob::Pass1Args a{Q, K, V, dO, UQ, UK, UV, O, L, D, dQt, ddOt, alpha, E};
  clear_pending();
  return finish(fbob::launch_pass1(c.p, a, static_cast<hipStream_t>(stream)));
}

int fbob_bob_pass2(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float tau,
                   int causal, const void* Q, const void* K, const void* V, const void* dO,
                   const void* UQ, const void* UK, const void* UV, const float* L, const float* D,
                   const float* alpha, const float* E, float* dKt, float* dVt, void* stream) {
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  if (c.empty) return FBOB_OK;
  const int64_t es = c.p.bf16 ? 2 : 4;
  const int64_t qb = B * Hq * N * d * es, kb = B * Hkv * N * d * es;
  const int64_t kob = B * Hkv * N * d * 4, rb = B * Hq * N * 4;
  const void* ins[] = {Q, K, V, dO, UQ, UK, UV, L, D, alpha, E};
  const int64_t inb[] = {qb, kb, kb, qb, qb, kb, kb, rb, rb, rb, rb};
  void* outs[] = {dKt, dVt};
  const int64_t outb[] = {kob, kob};
  const int st = check_ptrs(ins, inb, 11, outs, outb, 2);
  if (st != FBOB_OK) return st;
  fbob::Pass2Args a{Q, K, V, dO, UQ, UK, UV, L, D, alpha, E, dKt, dVt};
  clear_pending();
  return finish(fbob::launch_pass2(c.p, a, static_cast<hipStream_t>(stream)));
}

int fbob_backward(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float tau,
                  int causal, const void* Q, const void* K, const void* V, const void* dO,
                  const float* O, const float* L, float* dQ, float* dK, float* dV, float* D,
                  void* stream) {
  return fbob_backward_ws(dtype, B, Hq, Hkv, N, d, tau, causal, Q, K, V, dO, O, L, dQ, dK, dV,
                          D, nullptr, 0, stream);
}

int fbob_backward_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                 int64_t d, float tau, int causal, int64_t* bytes) {
  if (bytes == nullptr) return FBOB_ERR_INVALID_ARG;
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  *bytes = c.empty ? 0 : fbob::grad_split_plan(c.p).bytes();
  return FBOB_OK;
}

int fbob_backward_ws(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                     float tau, int causal, const void* Q, const void* K, const void* V,
                     const void* dO, const float* O, const float* L, float* dQ, float* dK,
                     float* dV, float* D, void* workspace, int64_t workspace_bytes,
                     void* stream) {
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  if (workspace_bytes < 0) return FBOB_ERR_INVALID_ARG;
  if (c.empty) return FBOB_OK;
  const fbob::GradPlan plan = fbob::grad_split_plan(c.p);
  // the split schedule only with a workspace that holds its partial sums
  const bool split = plan.bytes() > 0 && workspace != nullptr && workspace_bytes >= plan.bytes();
  const int64_t es = c.p.bf16 ? 2 : 4;
  const int64_t qb = B * Hq * N * d * es, kb = B * Hkv * N * d * es;
  const int64_t ob = B * Hq * N * d * 4, kob = B * Hkv * N * d * 4, rb = B * Hq * N * 4;
  const void* ins[] = {Q, K, V, dO, O, L};
  const int64_t inb[] = {qb, kb, kb, qb, ob, rb};
  void* outs[] = {dQ, dK, dV, D, split ? workspace : nullptr};
  const int64_t outb[] = {ob, kob, kob, rb, plan.bytes()};
  const int st = check_ptrs(ins, inb, 6, outs, outb, split ? 5 : 4);
  if (st != FBOB_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  fbob::GradArgs a{Q, K, V, dO, O, L, dQ, dK, dV, D};
  clear_pending();
  if (split) return finish(fbob::launch_backward_split(c.p, a, plan, workspace, s));
  const int st1 = finish(fbob::launch_grad_dq(c.p, a, s));
  if (st1 != FBOB_OK) return st1;
  return finish(fbob::launch_grad_dkv(c.p, a, s));
}

int fbob_bob_workspace_size(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                            float tau, int causal, int64_t* bytes) {
  if (bytes == nullptr) return FBOB_ERR_INVALID_ARG;
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  *bytes = c.empty ? 0 : fbob::split_plan(c.p).bytes();
  return FBOB_OK;
}

int fbob_bob_ws(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float tau,
                int causal, const void* Q, const void* K, const void* V, const void* dO,
                const void* UQ, const void* UK, const void* UV, const float* O, const float* L,
                const float* D, float* dQt, float* dKt, float* dVt, float* ddOt, float* alpha,
                float* E, void* workspace, int64_t workspace_bytes, void* stream) {
  return fbob_bob_ex(dtype, B, Hq, Hkv, N, d, tau, causal, 0, Q, K, V, dO, UQ, UK, UV, O, L, D,
                     dQt, dKt, dVt, ddOt, alpha, E, workspace, workspace_bytes, stream);
}

int fbob_bob_ex(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float tau,
                int causal, int flags, const void* Q, const void* K, const void* V,
                const void* dO, const void* UQ, const void* UK, const void* UV, const float* O,
                const float* L, const float* D, float* dQt, float* dKt, float* dVt,
                float* ddOt, float* alpha, float* E, void* workspace, int64_t workspace_bytes,
                void* stream) {
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  if (workspace_bytes < 0 || (flags & ~FBOB_FLAG_FP32_ROW_SUMS) != 0) return FBOB_ERR_INVALID_ARG;
  if (c.empty) return FBOB_OK;
  // only the bf16 d = 64 kernels round the products their row sums are formed from
  c.p.fp32_row_sums = (flags & FBOB_FLAG_FP32_ROW_SUMS) && c.p.bf16 && c.p.d == 64;
  const fbob::SplitPlan plan = fbob::split_plan(c.p);
  // The split schedule runs only with a workspace that holds its partial sums;
  // otherwise this is fbob_bob.
  const bool split = plan.bytes() > 0 && workspace != nullptr && workspace_bytes >= plan.bytes();
  void* ws = split ? workspace : nullptr;
  const int st = check_bob_ptrs(c, B, Hq, Hkv, N, d, Q, K, V, dO, UQ, UK, UV, O, L, D, dQt,
                                dKt, dVt, ddOt, alpha, E, ws, plan.bytes());
  if (st != FBOB_OK) return st;
  return run_bob(c, plan, fbob::Pass1Args{Q, K, V, dO, UQ, UK, UV, O, L, D, dQt, ddOt, alpha, E},
                 fbob::Pass2Args{Q, K, V, dO, UQ, UK, UV, L, D, alpha, E, dKt, dVt}, ws,
                 static_cast<hipStream_t>(stream));
}

int fbob_bob_noalloc(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                     float tau, int causal, const void* Q, const void* K, const void* V,
                     const void* dO, const void* UQ, const void* UK, const void* UV,
                     const float* O, const float* L, const float* D, float* dQt, float* dKt,
                     float* dVt, float* ddOt, float* alpha, float* E, void* stream) {
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  if (c.empty) return FBOB_OK;
  const int st = check_bob_ptrs(c, B, Hq, Hkv, N, d, Q, K, V, dO, UQ, UK, UV, O, L, D, dQt,
                                dKt, dVt, ddOt, alpha, E, nullptr, 0);
  if (st != FBOB_OK) return st;
  const fbob::SplitPlan plan = fbob::split_plan(c.p);
  if (plan.bytes() > FBOB_SCRATCH_BYTES) return FBOB_ERR_SCRATCH;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (plan.bytes() > 0) {
    // Every partial a split launch reads is written earlier in the same call, so
    // the scratch needs no clearing.
    const int sa = scratch_address(s, &ws);
    if (sa != FBOB_OK) return sa;
  }
  return run_bob(c, plan, fbob::Pass1Args{Q, K, V, dO, UQ, UK, UV, O, L, D, dQt, ddOt, alpha, E},
                 fbob::Pass2Args{Q, K, V, dO, UQ, UK, UV, L, D, alpha, E, dKt, dVt}, ws, s);
}

int fbob_bob(int dtype, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float tau,
             int causal, const void* Q, const void* K, const void* V, const void* dO,
             const void* UQ, const void* UK, const void* UV, const float* O, const float* L,
             const float* D, float* dQt, float* dKt, float* dVt, float* ddOt, float* alpha,
             float* E, void* stream) {
  Checked c = check_sizes(dtype, B, Hq, Hkv, N, d, tau, causal);
  if (c.status != FBOB_OK) return c.status;
  if (c.empty) return FBOB_OK;
  const int st = check_bob_ptrs(c, B, Hq, Hkv, N, d, Q, K, V, dO, UQ, UK, UV, O, L, D, dQt,
                                dKt, dVt, ddOt, alpha, E, nullptr, 0);
  if (st != FBOB_OK) return st;
  return run_bob(c, fbob::SplitPlan{},
                 fbob::Pass1Args{Q, K, V, dO, UQ, UK, UV, O, L, D, dQt, ddOt, alpha, E},
                 fbob::Pass2Args{Q, K, V, dO, UQ, UK, UV, L, D, alpha, E, dKt, dVt}, nullptr,
                 static_cast<hipStream_t>(stream));
}

}  // extern "C"
