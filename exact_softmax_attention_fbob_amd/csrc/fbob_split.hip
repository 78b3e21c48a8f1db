// fbob_split.hip - BoB on problems too small to fill the GPU: split sweeps.
//
// A Pass 1 work-group owns 128 query rows and a Pass 2 work-group 256 (d = 64) or
// 128 (d = 128) keys, and one such work-group runs per CU.  When a problem has
// fewer tiles than about two rounds of the 256 CUs, whole rounds are left partly
// idle (B=1 H=12 N=4096 d=64: 384 Pass 1 work-groups, 1.5 rounds; 192 Pass 2
// work-groups, a quarter of the CUs idle).  The split form divides each row tile's
// key sweep (Pass 1) or each column tile's row sweep (Pass 2) into s parts run by
// consecutive work-groups, each writing fp32 partial sums to a workspace, and a
// short reduction adds the parts in a fixed order (deterministic) and applies what
// the single-sweep epilogue does:
//   Pass 1 (FlashBoB notes, "关键设计" 1, the affine correction, through R = X + D B):
//     ddO~ = ddO~' - alpha o,  dQ~ = tau (Omega - alpha X - E' B),  E = E' - alpha D,
//     with E' = <dO, ddO~> where the split kernel forms alpha by MFMA (d = 64 with the
//     default row sums), else the sum of the parts' E' (fp32 row sums; d = 128);
//   Pass 2: dK~ = sum of tau dK~ parts,  dV~ = sum of dV~ parts.
// When a pass's work-groups fill at least one whole round of the CUs, the heads of the
// whole rounds run unsplit (a launch over that head range) and only the rest split, so
// that the last, partly idle round is filled while only the rest's partial sums are
// written (a third of them for Pass 1 at B=1 H=12 N=4096).
// Every output is still written exactly once, with no atomics.  With the causal mask
// at d = 64 a Pass 2 work-group sweeps two column tiles, p and n - 1 - p, whose row
// steps together are the same for every pair, and causal Pass 1 pairs its row tiles
// n - 1 - p and p; the split cuts each pair's joint sweep into equal parts.  At d = 128
// the tiles are single (longest first) and each tile's own sweep is cut.
#include <algorithm>

#include "fbob_device.hpp"
#include "fbob_launch.hpp"

namespace fbob {
namespace {

constexpr int kCUs = 256;  // MI355X; only the split heuristic depends on it

// Rows of both reductions: one thread per 4 consecutive d values of one row (the
// D / 4 threads of a row are consecutive lanes of one wave).  EDOT: E' as <dO, ddO~>.
template <typename T, int D, bool EDOT>
__global__ __launch_bounds__(256) void reduce_pass1_kernel(Pass1Args a, int64_t rows, int nsplit,
                                                           float tau) {
  constexpr int kChunks = D / 4;
  static_assert(kChunks <= 64 && (kChunks & (kChunks - 1)) == 0, "a row's threads in one wave");
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / kChunks;  // flat (b, h, i)
  // Whole rows leave together, so the row reduction below only reads live lanes.
  if (row >= rows) return;
  const int d0 = 4 * (int)(idx % kChunks);
  f32x4 B = splat4(0.f), X = B, W = B, O = B;
  float al = 0.f, es = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const int64_t prow = (int64_t)s * rows + row;
    const float* pa = a.part_acc + prow * 4 * D;
    B += *reinterpret_cast<const f32x4*>(pa + d0);
    X += *reinterpret_cast<const f32x4*>(pa + D + d0);
    W += *reinterpret_cast<const f32x4*>(pa + 2 * D + d0);
    O += *reinterpret_cast<const f32x4*>(pa + 3 * D + d0);
    al += a.part_rs[2 * prow];
    es += a.part_rs[2 * prow + 1];
  }
  const int64_t ro = row * D + d0;
  const f32x4 o = *reinterpret_cast<const f32x4*>(a.O + ro);
  const f32x4 ddo = O - al * o;
  float ed = es;
  if constexpr (EDOT) {  // E' = <dO, ddO~> of this row
    const T* dO = reinterpret_cast<const T*>(a.dO) + ro;
    float dot = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) dot = __builtin_fmaf((float)dO[q], ddo[q], dot);
#pragma unroll
    for (int m = kChunks / 2; m >= 1; m /= 2) dot += __shfl_xor(dot, m);
    ed = dot;
  }
  *reinterpret_cast<f32x4*>(a.ddOt + ro) = ddo;
  *reinterpret_cast<f32x4*>(a.dQt + ro) = tau * (W - al * X - ed * B);
  if (d0 == 0) {
    a.alpha[row] = al;
    a.E[row] = ed - al * a.D[row];
  }
}

template <int D>
__global__ __launch_bounds__(256) void reduce_pass2_kernel(Pass2Args a, int64_t rows, int nsplit) {
  constexpr int kChunks = D / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / kChunks;  // flat (b, key/value head, j)
  if (row >= rows) return;
  const int d0 = 4 * (int)(idx % kChunks);
  f32x4 k = splat4(0.f), v = k;
  for (int s = 0; s < nsplit; ++s) {
    const float* pp = a.part + ((int64_t)s * rows + row) * 2 * D;
    k += *reinterpret_cast<const f32x4*>(pp + d0);
    v += *reinterpret_cast<const f32x4*>(pp + D + d0);
  }
  *reinterpret_cast<f32x4*>(a.dKt + row * D + d0) = k;
  *reinterpret_cast<f32x4*>(a.dVt + row * D + d0) = v;
}

// First backward, row pass: dQ = the sum of the parts' tau dQ (one thread per 4
// consecutive d values of one row).
template <int D>
__global__ __launch_bounds__(256) void reduce_dq_kernel(GradArgs a, int64_t rows, int nsplit) {
  constexpr int kChunks = D / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / kChunks;  // flat (b, h, i)
  if (row >= rows) return;
  const int d0 = 4 * (int)(idx % kChunks);
  f32x4 q = splat4(0.f);
  for (int s = 0; s < nsplit; ++s)
    q += *reinterpret_cast<const f32x4*>(a.part + ((int64_t)s * rows + row) * D + d0);
  *reinterpret_cast<f32x4*>(a.dQ + row * D + d0) = q;
}

// Parts s in {1, 2, 4, 8} for `units` work-groups whose full sweep takes `sweep_us`
// and has `stages` stages (at least two per part), with `part_bytes` of partial sums
// per part.  Estimated time: the rounds of work-groups over the CUs, each 1/s of a
// sweep, plus writing the partial sums and reading them back in the reduction
// (~5 TB/s each way) and the reduction's launch; a split is taken only if the
// estimate is at least 5 % below the unsplit one.  (Calibrated on B=1 H=12 N=4096
// d=64: Pass 1 290 us unsplit, 242 + 21 us in two parts; Pass 2 198 us unsplit,
// 186 + 20 us in four.)
int choose_parts(int64_t units, int64_t stages, double sweep_us, double part_bytes) {
  auto est = [&](int s) {
    const double rounds = (double)((units * s + kCUs - 1) / kCUs);
    const double extra = s > 1 ? 2.0 * s * part_bytes / 5.0e6 + 5.0 : 0.0;
    return rounds * sweep_us / s + extra;
  };
  int best = 1;
  for (int s = 2; s <= 8; s *= 2) {
    if (stages < 2 * s) break;
    if (est(s) < est(best)) best = s;
  }
  return est(best) <= 0.95 * est(1) ? best : 1;
}

}  // namespace

namespace {

// How one pass splits: every head's work-groups in s parts (full = 0), or the first
// `full` heads, whole rounds of work-groups, unsplit and only the rest in s parts.
struct PassSplit {
  int s = 1;
  int64_t full = 0;
};

// per_head work-groups (tiles or tile pairs) for each of `heads` heads, each sweeping
// `stages` stages in sweep_us, with head_bytes of partial sums per head and part;
// whole(f) tells whether the first f heads form a problem of their own.  Leaving the
// heads of whole rounds unsplit takes the same rounds of sweep time as splitting every
// head and writes only the rest's partial sums (B=1 H=12 N=4096, Pass 1: 8 heads whole,
// 4 in two parts, a third of the partials); it is taken where the estimate is lower.
template <typename Whole>
PassSplit plan_pass(int64_t per_head, int64_t heads, int64_t stages, double sweep_us,
                    double head_bytes, Whole whole) {
  PassSplit r;
  const int64_t units = per_head * heads;
  r.s = choose_parts(units, stages, sweep_us, heads * head_bytes);
  if (units < kCUs || per_head > kCUs) return r;
  const int64_t per_round = kCUs / per_head;  // heads per round of work-groups
  const int64_t full = units / kCUs * per_round;
  const int64_t rest = heads - full;
  if (rest <= 0 || !whole(full)) return r;
  const int s_rest = choose_parts(rest * per_head, stages, sweep_us, rest * head_bytes);
  if (s_rest == 1) return r;
  const auto est = [&](int64_t u, int s, double bytes) {
    const double rounds = (double)((u * s + kCUs - 1) / kCUs);
    return rounds * sweep_us / s + (s > 1 ? 2.0 * s * bytes / 5.0e6 + 5.0 : 0.0);
  };
  const double uniform = est(units, r.s, heads * head_bytes);
  const double partial =
      (double)(full / per_round) * sweep_us + est(rest * per_head, s_rest, rest * head_bytes);
  if (partial < uniform && (r.s > 1 || partial <= 0.95 * est(units, 1, 0.0))) {
    r.s = s_rest;
    r.full = full;
  }
  return r;
}

}  // namespace

SplitPlan split_plan(const Problem& p) {
  SplitPlan plan;
  // The split forms exist for the shipped bf16 variants.  With the causal mask the tiles
  // of both passes are paired at d = 64 (every pair the same work) and single at d = 128,
  // where the tiles' lengths vary; there the model takes the mean tile.
  if (!p.bf16 || (p.d == 64 && !tau_is_pow2(p.tau))) return plan;
  const bool fold = p.causal && p.d == 64;
  const int64_t heads_q = (int64_t)p.B * p.Hq, heads_kv = (int64_t)p.B * p.Hkv;
  const int64_t group = p.Hq / p.Hkv;
  const int64_t stages = (p.N + 63) / 64;  // 64-key / 64-row stages in both passes
  const int col_tile = p.d == 64 ? 256 : 128;
  const int64_t col_tiles = (p.N + col_tile - 1) / col_tile;
  // Pass 2 work-groups and the row steps of each: one column tile sweeping every row
  // of the group's query heads, or (causal, d = 64) a pair of tiles p and n - 1 - p
  // sweeping the rows from each tile's first key on, 2 n_stages - 4 (n - 1) steps per
  // query head for every pair.
  int64_t per_head2 = col_tiles;
  int64_t steps2 = stages * group;
  if (fold) {
    per_head2 = (col_tiles + 1) / 2;
    steps2 = (col_tiles > 1 ? 2 * stages - 4 * (col_tiles - 1) : stages) * group;
  } else if (p.causal) {  // tile c sweeps the rows from its first key on
    steps2 = std::max<int64_t>(1, (stages + 1) / 2) * group;
  }
  // Measured sweep times of one work-group per key (Pass 1) or row step of 64 rows
  // (Pass 2): ~35 and ~74 ns per key, ~3.1 and ~3.7 us per row step at d = 64 / 128.
  const double sweep2 = (p.d == 64 ? 3.1 : 3.7) * steps2;
  const double head_bytes2 = (double)p.N * 2 * p.d * 4;  // one key/value head, one part
  // a leading range of key/value heads is a problem of its own in one batch, or when
  // it holds whole batches
  // Single causal tiles (d = 128) of unequal length already balance over the CUs when
  // dispatched longest first; they split only while they do not fill one round
  // (B=1 H=12 N=4096 split anyway measured 36 % slower, H=4 1.75x faster).
  const bool single = p.causal && !fold;
  PassSplit s2;
  if (!single || per_head2 * heads_kv < kCUs)
    s2 = plan_pass(per_head2, heads_kv, steps2, sweep2, head_bytes2,
                   [&](int64_t f) { return p.B == 1 || f % p.Hkv == 0; });
  plan.s2 = s2.s;
  plan.full2 = s2.full;
  if (plan.s2 > 1) plan.bytes2 = (int64_t)plan.s2 * (heads_kv - s2.full) * p.N * 2 * p.d * 4;
  // Pass 1 work-groups and their 64-key stages: one row tile of 128 rows sweeping
  // every key, or (causal, d = 64) row tiles n - 1 - p and p, 2 (n + 1) stages for
  // every pair when N is a multiple of 128 (the keys up to each tile's last row).
  const int64_t row_tiles = (p.N + 127) / 128;
  int64_t per_head1 = row_tiles;
  int64_t stages1 = stages;
  if (fold) {
    per_head1 = (row_tiles + 1) / 2;
    stages1 = row_tiles > 1 ? stages + 2 : stages;
  } else if (p.causal) {  // tile r sweeps the keys up to its last row
    stages1 = std::max<int64_t>(1, (stages + 1) / 2);
  }
  const double sweep1 = (p.d == 64 ? 0.035 : 0.074) * 64 * stages1;
  const double head_bytes1 = (double)p.N * (4 * p.d + 2) * 4;  // one query head, one part
  // a leading range of query heads must end on a group of query heads (one batch) or
  // on a batch boundary
  PassSplit s1;
  if (!single || per_head1 * heads_q < kCUs)
    s1 = plan_pass(per_head1, heads_q, stages1, sweep1, head_bytes1, [&](int64_t f) {
      return p.B == 1 ? f % group == 0 : f % p.Hq == 0;
    });
  plan.s1 = s1.s;
  plan.full1 = s1.full;
  if (plan.s1 > 1)
    plan.bytes1 = (int64_t)plan.s1 * (heads_q - s1.full) * p.N * (4 * p.d + 2) * 4;
  return plan;
}

namespace {

// The query heads [h0, h0 + n) of a problem (whole groups of one batch, or whole
// batches) as a problem of their own, with every pointer moved to head h0.
void head_range(const Problem& p, const Pass1Args& a, int64_t h0, int64_t n, Problem* sp,
                Pass1Args* sa) {
  const int64_t group = p.Hq / p.Hkv;
  *sp = p;
  if (p.B == 1) {
    sp->Hq = (int)n;
    sp->Hkv = (int)(n / group);
  } else {
    sp->B = (int)(n / p.Hq);
  }
  const int64_t es = p.bf16 ? 2 : 4;
  const int64_t q = h0 * p.N * p.d, kv = h0 / group * p.N * p.d, r = h0 * p.N;
  auto in = [&](const void* x, int64_t off) {
    return static_cast<const void*>(static_cast<const char*>(x) + off * es);
  };
  *sa = a;
  sa->Q = in(a.Q, q);
  sa->dO = in(a.dO, q);
  sa->UQ = in(a.UQ, q);
  sa->K = in(a.K, kv);
  sa->V = in(a.V, kv);
  sa->UK = in(a.UK, kv);
  sa->UV = in(a.UV, kv);
  sa->O = a.O + q;
  sa->L = a.L + r;
  sa->D = a.D + r;
  sa->dQt = a.dQt + q;
  sa->ddOt = a.ddOt + q;
  sa->alpha = a.alpha + r;
  sa->E = a.E + r;
}

// The key/value heads [h0, h0 + n) of a problem (any range of one batch, or whole
// batches) with their query heads, as a problem of their own.
void kv_head_range(const Problem& p, const Pass2Args& a, int64_t h0, int64_t n, Problem* sp,
                   Pass2Args* sa) {
  const int64_t group = p.Hq / p.Hkv;
  *sp = p;
  if (p.B == 1) {
    sp->Hkv = (int)n;
    sp->Hq = (int)(n * group);
  } else {
    sp->B = (int)(n / p.Hkv);
  }
  const int64_t es = p.bf16 ? 2 : 4;
  const int64_t kv = h0 * p.N * p.d, q = h0 * group * p.N * p.d, r = h0 * group * p.N;
  auto in = [&](const void* x, int64_t off) {
    return static_cast<const void*>(static_cast<const char*>(x) + off * es);
  };
  *sa = a;
  sa->Q = in(a.Q, q);
  sa->dO = in(a.dO, q);
  sa->UQ = in(a.UQ, q);
  sa->K = in(a.K, kv);
  sa->V = in(a.V, kv);
  sa->UK = in(a.UK, kv);
  sa->UV = in(a.UV, kv);
  sa->L = a.L + r;
  sa->D = a.D + r;
  sa->alpha = a.alpha + r;
  sa->E = a.E + r;
  sa->dKt = a.dKt + kv;
  sa->dVt = a.dVt + kv;
}

}  // namespace

hipError_t launch_bob_split(const Problem& p, const Pass1Args& a1_in, const Pass2Args& a2_in,
                            const SplitPlan& plan, void* workspace, hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  if (plan.s1 > 1) {
    Problem p1 = p;
    Pass1Args a1 = a1_in;
    if (plan.full1 > 0) {  // leading heads unsplit, the rest split below
      Problem pf;
      Pass1Args af;
      head_range(p, a1_in, 0, plan.full1, &pf, &af);
      const hipError_t e = launch_pass1(pf, af, s);
      if (e != hipSuccess) return e;
      head_range(p, a1_in, plan.full1, (int64_t)p.B * p.Hq - plan.full1, &p1, &a1);
    }
    const int64_t rows = (int64_t)p1.B * p1.Hq * p1.N;
    a1.part_acc = reinterpret_cast<float*>(ws);
    a1.part_rs = a1.part_acc + (int64_t)plan.s1 * rows * 4 * p.d;
    a1.nsplit = plan.s1;
    hipError_t e = launch_pass1_split(p1, a1, s);
    if (e != hipSuccess) return e;
    const int64_t threads = rows * (p1.d / 4);
    const dim3 grid((unsigned)((threads + 255) / 256));
    // split_plan admits bf16 inputs only; the d = 64 split kernel forms alpha by MFMA
    // (E' from ddO~) unless fp32 row sums are asked for, the d = 128 one as lane sums
    // (E' summed over the parts)
    if (p1.d == 64 && !p1.fp32_row_sums)
      hipLaunchKernelGGL((reduce_pass1_kernel<__bf16, 64, true>), grid, dim3(256), 0, s, a1,
                         rows, plan.s1, p1.tau);
    else if (p1.d == 64)
      hipLaunchKernelGGL((reduce_pass1_kernel<__bf16, 64, false>), grid, dim3(256), 0, s, a1,
                         rows, plan.s1, p1.tau);
    else
      hipLaunchKernelGGL((reduce_pass1_kernel<__bf16, 128, false>), grid, dim3(256), 0, s, a1,
                         rows, plan.s1, p1.tau);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const hipError_t e = launch_pass1(p, a1_in, s);
    if (e != hipSuccess) return e;
  }
  if (plan.s2 > 1) {
    Problem p2 = p;
    Pass2Args a2 = a2_in;
    if (plan.full2 > 0) {  // leading key/value heads unsplit, the rest split below
      Problem pf;
      Pass2Args af;
      kv_head_range(p, a2_in, 0, plan.full2, &pf, &af);
      const hipError_t e = launch_pass2(pf, af, s);
      if (e != hipSuccess) return e;
      kv_head_range(p, a2_in, plan.full2, (int64_t)p.B * p.Hkv - plan.full2, &p2, &a2);
    }
    const int64_t rows = (int64_t)p2.B * p2.Hkv * p2.N;
    a2.part = reinterpret_cast<float*>(ws);  // Pass 1's partials are consumed by now
    a2.nsplit = plan.s2;
    hipError_t e = launch_pass2_split(p2, a2, s);
    if (e != hipSuccess) return e;
    const int64_t threads = rows * (p2.d / 4);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (p2.d == 64)
      hipLaunchKernelGGL(reduce_pass2_kernel<64>, grid, dim3(256), 0, s, a2, rows, plan.s2);
    else
      hipLaunchKernelGGL(reduce_pass2_kernel<128>, grid, dim3(256), 0, s, a2, rows, plan.s2);
    return hipGetLastError();
  }
  return launch_pass2(p, a2_in, s);
}

// The first backward's passes split like the BoB's (uniform parts): the row pass owns
// 256 query rows per work-group (128-key stages at d = 64, 64 at d = 128), the column
// pass 256 keys (d = 64, 64-row steps) or 128 (d = 128, 32-row steps).  With the causal
// mask (tiles single, longest first) and at d = 128 a pass splits only while its tiles
// do not fill one round of the CUs.
GradPlan grad_split_plan(const Problem& p) {
  GradPlan plan;
  if (!p.bf16) return plan;
  const int64_t heads_q = (int64_t)p.B * p.Hq, heads_kv = (int64_t)p.B * p.Hkv;
  const int64_t group = p.Hq / p.Hkv;
  const int row_tile = 256, bc = p.d == 64 ? 128 : 64;
  const int col_tile = p.d == 64 ? 256 : 128, brs = p.d == 64 ? 64 : 32;
  const int64_t row_tiles = (p.N + row_tile - 1) / row_tile;
  const int64_t col_tiles = (p.N + col_tile - 1) / col_tile;
  int64_t stages1 = (p.N + bc - 1) / bc;
  int64_t steps2 = (p.N + brs - 1) / brs * group;
  if (p.causal) {  // the mean tile
    stages1 = std::max<int64_t>(1, (stages1 + 1) / 2);
    steps2 = std::max<int64_t>(1, (steps2 + 1) / 2);
  }
  const int64_t units1 = row_tiles * heads_q, units2 = col_tiles * heads_kv;
  // sweep times per 32 keys (row pass) or 32 rows (column pass) of one work-group, from
  // the passes at B=1 H=12 N=16384 d=64 (1.08 ms and 1.45 ms for 3 rounds): ~0.7 and
  // ~0.94 us, about twice that at d = 128
  const double sweep1 = (p.d == 64 ? 0.7 : 1.4) * bc / 32.0 * stages1;
  const double sweep2 = (p.d == 64 ? 0.94 : 1.9) * brs / 32.0 * steps2;
  // Causal tiles, and every tile at d = 128, split only while a pass's tiles do not fill
  // one round (d = 128, B=1 H=20 N=4096: 320 and 640 tiles, split anyway 705 -> 758 us;
  // at d = 64 splits past one round still gained 5-12 %).
  const bool round_only = p.causal || p.d == 128;
  if (!round_only || units1 < kCUs) {
    plan.s1 = choose_parts(units1, stages1, sweep1, (double)heads_q * p.N * p.d * 4);
    if (plan.s1 > 1) plan.bytes1 = (int64_t)plan.s1 * heads_q * p.N * p.d * 4;
  }
  if (!round_only || units2 < kCUs) {
    plan.s2 = choose_parts(units2, steps2, sweep2, (double)heads_kv * p.N * 2 * p.d * 4);
    if (plan.s2 > 1) plan.bytes2 = (int64_t)plan.s2 * heads_kv * p.N * 2 * p.d * 4;
  }
  return plan;
}

hipError_t launch_backward_split(const Problem& p, const GradArgs& a_in, const GradPlan& plan,
                                 void* workspace, hipStream_t s) {
  float* ws = static_cast<float*>(workspace);
  if (plan.s1 > 1) {
    GradArgs a = a_in;
    a.part = ws;
    a.nsplit = plan.s1;
    hipError_t e = launch_grad_dq_split(p, a, s);
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)p.B * p.Hq * p.N;
    const dim3 grid((unsigned)((rows * (p.d / 4) + 255) / 256));
    if (p.d == 64)
      hipLaunchKernelGGL(reduce_dq_kernel<64>, grid, dim3(256), 0, s, a, rows, plan.s1);
    else
      hipLaunchKernelGGL(reduce_dq_kernel<128>, grid, dim3(256), 0, s, a, rows, plan.s1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const hipError_t e = launch_grad_dq(p, a_in, s);
    if (e != hipSuccess) return e;
  }
  if (plan.s2 > 1) {  // after the row pass (it reads D, and reuses the workspace)
    GradArgs a = a_in;
    a.part = ws;
    a.nsplit = plan.s2;
    hipError_t e = launch_grad_dkv_split(p, a, s);
    if (e != hipSuccess) return e;
    Pass2Args r{};  // the BoB's Pass 2 reduction: the same part layout
    r.part = ws;
    r.dKt = a_in.dK;
    r.dVt = a_in.dV;
    const int64_t rows = (int64_t)p.B * p.Hkv * p.N;
    const dim3 grid((unsigned)((rows * (p.d / 4) + 255) / 256));
    if (p.d == 64)
      hipLaunchKernelGGL(reduce_pass2_kernel<64>, grid, dim3(256), 0, s, r, rows, plan.s2);
    else
      hipLaunchKernelGGL(reduce_pass2_kernel<128>, grid, dim3(256), 0, s, r, rows, plan.s2);
    return hipGetLastError();
  }
  return launch_grad_dkv(p, a_in, s);
}

}  // namespace fbob
