// fbob_pass2.hip - BoB Pass 2 (column-resident).
//
// FlashBoB notes, "关键设计" item 2 (second pass) and item 3 (grouped heads).
// For each key position j it streams every query row i, rebuilding from the
// stored row state (L, D) and the Pass 1 row scalars (alpha, E)
//   P = exp(tau Q K^T - L),  dP = dO V^T,  F = tau (U_Q K^T + Q U_K^T),  G = dO U_V^T
//   dS  = P o (dP - D)
//   dS~ = P o (dP~ - E),  dP~ = F o (dP - D) - alpha dP + G   (adjoint of P)
//   ddP = P o (F - alpha)                                     (adjoint of dP)
// and accumulates
//   dK~_j = tau sum_i (dS~_ij Q_i + dS_ij U_Q,i),   dV~_j = sum_i ddP_ij dO_i,
// summing all query heads of a key/value group on chip, then writes dK~ and dV~
// exactly once, with no atomics.
//
// With t = dP - D, u = F - alpha and g' = G - E - alpha D, the adjoints are
//   dS = P t,   ddP = P u,   dS~ = P (u t + g'),
// and t, u, g' come straight out of the MFMAs by seeding their accumulators with
// the row scalars -D, -alpha and -(E + alpha D); tau is folded into the resident
// K and U_K operands of the F tile (when tau is not a power of two, and always at
// d = 128, the operands stay unscaled, the F - alpha accumulator is seeded with
// -alpha / tau and scaled by tau on the VALU).  That leaves five VALU operations
// plus one exp per score element.
//
// Schedule: one work-group = NW waves; each wave owns 16 NJ key positions whose
// K, tau K, tau U_K, V, U_V operand fragments and the two fp32 accumulators stay
// in registers.  Q, dO, U_Q row tiles (BRS rows) plus the four derived row scalars
// are staged through LDS (double-buffered).  Scores are computed with the query
// index on the MFMA row axis, so a lane owns one key and four consecutive rows
// per block; those C registers are directly the B operand of the contractions
// over rows, whose A operand (Q^T, U_Q^T, dO^T) comes from transposed LDS reads.
#include <type_traits>

#include "fbob_device.hpp"
#include "fbob_launch.hpp"

namespace fbob {
namespace {

// SCHED: 0 leaves instruction order to the compiler, 1 fences the phases and
// column blocks; 3 raises the wave priority over the contraction MFMAs, 4 also over
// the score MFMAs (no fences otherwise).
// SPLIT: the work-group sweeps one part of its row steps and writes tau dK~ and dV~
// of that part to a.part; a reduction kernel adds the parts.  With the causal pairing
// the two tiles' row steps form one sequence, cut into equal parts (a part may end in
// the first tile and start the second), so all parts stay equally long.
template <typename T, int D, int NW, int NJ, int BRS, int SCHED, int TM, bool DIRECT, bool CAUSAL,
          bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) void pass2_kernel(Pass2Args a, int Hkv, int group, int N,
                                                        float tau, int n_col_tiles, int total) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr bool FENCE = SCHED == 1;
  constexpr bool kPrioOut = SCHED >= 3;
  constexpr bool kPrioScore = SCHED >= 4;
  constexpr int kThreads = NW * 64;
  constexpr int kCW = 16 * NJ;                      // keys per wave
  constexpr int kBCw = NW * kCW;                    // keys per work-group
  constexpr int kTB = BRS * Tile<T, D>::kRowBytes;  // bytes per staged tile
  constexpr int kDC = D / 32;
  constexpr int kDB = D / 16;
  constexpr int kScal = 4 * BRS * 4;                // -L log2e, -D, -alpha, -(E + alpha D)
  constexpr int kStage = 3 * kTB + kScal;
  __shared__ __attribute__((aligned(16))) char lds[2][kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int logical = xcd_remap(blockIdx.x, total);
  // Causal (d = 64): a work-group takes column tiles p and n - 1 - p, so every
  // work-group sweeps the same number of row chunks (the first has the most);
  // key/value heads stay in consecutive work-groups.
  constexpr bool kFold = CAUSAL && D < 128;
  const int n_units = kFold ? (n_col_tiles + 1) / 2 : n_col_tiles;
  // SPLIT: the parts of one column tile are consecutive work-groups (one XCD).
  const int split = SPLIT ? logical % a.nsplit : 0;
  const int lt = SPLIT ? logical / a.nsplit : logical;
  const int bhk = lt / n_units, unit = lt % n_units;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int Hq = Hkv * group;
  const int64_t kv_off = (int64_t)bhk * N * D;
  const T* Kh = reinterpret_cast<const T*>(a.K) + kv_off;
  const T* Vh = reinterpret_cast<const T*>(a.V) + kv_off;
  const T* UKh = reinterpret_cast<const T*>(a.UK) + kv_off;
  const T* UVh = reinterpret_cast<const T*>(a.UV) + kv_off;

  const int n_tiles_here = kFold && unit != n_col_tiles - 1 - unit ? 2 : 1;
  // Row steps (query head of the group, 64-row chunk) of column tile ct; causal rows
  // start at the chunk holding the tile's first key.
  auto first_row = [&](int ct) { return CAUSAL ? (ct * kBCw / BRS) * BRS : 0; };
  auto steps_of = [&](int ct) { return (N - first_row(ct) + BRS - 1) / BRS * group; };
  // SPLIT: this part's share [part_lo, part_hi) of the work-group's steps, counted
  // over its tiles in order.
  int steps0 = 0, part_lo = 0, part_hi = 0;
  if constexpr (SPLIT) {
    steps0 = steps_of(unit);
    const int all_steps = steps0 + (n_tiles_here == 2 ? steps_of(n_col_tiles - 1 - unit) : 0);
    const int per_part = (all_steps + a.nsplit - 1) / a.nsplit;
    part_lo = min(all_steps, split * per_part);
    part_hi = min(all_steps, part_lo + per_part);
  }
#pragma unroll 1
  for (int tile = 0; tile < n_tiles_here; ++tile) {
    const int ct = tile == 0 ? unit : n_col_tiles - 1 - unit;
    const int jw0 = ct * kBCw + w * kCW;
    // tkf / tukf hold tau K / tau U_K, or K / U_K unscaled under kTauValu; kf (K for
    // the score tile) is a separate copy only under kTauScaled.
    constexpr bool kKcopy = TM == kTauScaled;
    F kf[kKcopy ? NJ : 1][kDC], tkf[NJ][kDC], tukf[NJ][kDC], vf[NJ][kDC], uvf[NJ][kDC];
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
      for (int dc = 0; dc < kDC; ++dc) {
        const int j = jw0 + 16 * jb + r, col = 32 * dc + 8 * g;
        const F k0 = global_frag(Kh, j, N, D, col);
        const F uk0 = global_frag(UKh, j, N, D, col);
        if constexpr (kKcopy) kf[jb][dc] = k0;
        tkf[jb][dc] = TM == kTauValu ? k0 : scale_frag<T>(k0, tau);
        tukf[jb][dc] = TM == kTauValu ? uk0 : scale_frag<T>(uk0, tau);
        vf[jb][dc] = global_frag(Vh, j, N, D, col);
        uvf[jb][dc] = global_frag(UVh, j, N, D, col);
      }

    f32x4 accK[NJ][kDB], accV[NJ][kDB];
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        accK[jb][db] = splat4(0.f);
        accV[jb][db] = accK[jb][db];
      }
    const float c1 = TM == kTauPow2 ? kLog2e : tau * kLog2e;
    // Under kTauValu the F - alpha tile accumulates F / tau - alpha / tau and is scaled
    // by tau afterwards, so its seed is -alpha / tau.
    const float inv_tau = TM == kTauValu ? 1.f / tau : 1.f;
    const LdsLane<T, D> rd(r, g);

    const int i_begin = first_row(ct);
    const int nrc = (N - i_begin + BRS - 1) / BRS;
    const int nsteps = nrc * group;

    const int64_t q_head = (int64_t)N * D * (int64_t)sizeof(T);  // bytes per query head
    const int64_t q0 = ((int64_t)b * Hq + (int64_t)hk * group) * N * D;
    const T* const q_bases[3] = {reinterpret_cast<const T*>(a.Q) + q0,
                                 reinterpret_cast<const T*>(a.dO) + q0,
                                 reinterpret_cast<const T*>(a.UQ) + q0};
    // Q, dO, U_Q tiles: registers + ds_write (MultiStager) or direct global -> LDS.
    using RegStager = MultiStager<T, D, BRS, 3, kThreads>;
    using DirStager = DirectStager<T, D, BRS, 3, NW, !CAUSAL>;
    typename std::conditional<DIRECT, DirStager, RegStager>::type st;
    if constexpr (DIRECT) st.init(q_bases, w, lane);
    else st.init(q_bases, tid);
    // Row scalars: thread tid < BRS stages row tid of the chunk.
    const int64_t s0 = ((int64_t)b * Hq + (int64_t)hk * group) * N;
    f32x4 scal = splat4(0.f);
    // Steps run in order: the next one to load is query head ld_hq, row chunk ld_rc
    // (advanced by one chunk per load rather than divided out of the step index).
    int ld_hq = 0, ld_rc = 0, nxt_i0 = 0;
    // Issue the loads of the next step (tiles go straight into `buf` when DIRECT).
    auto load_step = [&](char* buf) {
      const int hq = ld_hq;
      const int i0 = i_begin + ld_rc * BRS;
      nxt_i0 = i0;
      if (++ld_rc == nrc) {
        ld_rc = 0;
        ++ld_hq;
      }
      if constexpr (DIRECT) st.load(buf, i0, N, hq * q_head);
      else st.load(i0, N, hq * q_head);
      // The raw values stay in registers until store_step: deriving the seeds here
      // would make this wave wait for every load it has in flight (the tiles'
      // included) before it computes the current stage.
      if (tid < BRS) {
        const int64_t ri = s0 + (int64_t)hq * N + min(i0 + tid, N - 1);
        scal = f32x4{a.L[ri], a.D[ri], a.alpha[ri], a.E[ri]};
      }
    };
    // (DIRECT: the caller has waited for every load of the step.)
    auto store_step = [&](char* buf) {
      if constexpr (!DIRECT) st.store(buf);
      if (tid < BRS) {
        const float L = scal[0], Dv = scal[1], al = scal[2], Ev = scal[3];
        const f32x4 seed = {-L * kLog2e, -Dv, -al * inv_tau, -(Ev + al * Dv)};
        float* sp = reinterpret_cast<float*>(buf + 3 * kTB);
#pragma unroll
        for (int m = 0; m < 4; ++m) sp[m * BRS + tid] = seed[m];
      }
    };

    // 32 rows of a staged tile (sub-chunk sc): scores, elementwise, contractions.
    auto chunk = [&](const char* buf, int i0, int sc) {
      const char* Qt = buf;
      const char* dOt = buf + kTB;
      const char* UQt = buf + 2 * kTB;
      const float* sp = reinterpret_cast<const float*>(buf + 3 * kTB);
      const int ic = i0 + 32 * sc;
      const bool edge = (ic + 32 > N) || (CAUSAL && ic < jw0 + kCW - 1);
      F dsB[NJ], ddpB[NJ], dstB[NJ];  // filled half by half: elements 4 ib .. 4 ib + 3
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const int rr = 32 * sc + 16 * ib + 4 * g;  // first of this lane's 4 rows in the tile
        const f32x4 nL = *reinterpret_cast<const f32x4*>(sp + rr);
        const f32x4 nD = *reinterpret_cast<const f32x4*>(sp + BRS + rr);
        const f32x4 nA = *reinterpret_cast<const f32x4*>(sp + 2 * BRS + rr);
        const f32x4 nG = *reinterpret_cast<const f32x4*>(sp + 3 * BRS + rr);
        f32x4 s[NJ], t[NJ], u[NJ], gp[NJ];
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
          s[jb] = splat4(0.f);
          t[jb] = nD;
          u[jb] = nA;
          gp[jb] = nG;
        }
        if constexpr (kPrioScore) FBOB_PRIO_HIGH();
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc) {
          const F qa = rd.row(Qt, 2 * sc + ib, dc);
          const F doa = rd.row(dOt, 2 * sc + ib, dc);
          const F uqa = rd.row(UQt, 2 * sc + ib, dc);
#pragma unroll
          for (int jb = 0; jb < NJ; ++jb) {
            s[jb] = E::mma(qa, kKcopy ? kf[kKcopy ? jb : 0][dc] : tkf[jb][dc], s[jb]);
            u[jb] = E::mma(uqa, tkf[jb][dc], u[jb]);
            u[jb] = E::mma(qa, tukf[jb][dc], u[jb]);
            t[jb] = E::mma(doa, vf[jb][dc], t[jb]);
            gp[jb] = E::mma(doa, uvf[jb][dc], gp[jb]);
          }
        }
        if constexpr (kPrioScore) FBOB_PRIO_LOW();
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
          if constexpr (TM == kTauValu) u[jb] = tau * u[jb];
          f32x4 p;
#pragma unroll
          for (int q = 0; q < 4; ++q) p[q] = fast_exp2(__builtin_fmaf(s[jb][q], c1, nL[q]));
          if (edge) {
            const int j = jw0 + 16 * jb + r;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int i = ic + 16 * ib + 4 * g + q;
              if (i >= N || (CAUSAL && j > i)) p[q] = 0.f;
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            dsB[jb][4 * ib + q] = (T)(p[q] * t[jb][q]);
            ddpB[jb][4 * ib + q] = (T)(p[q] * u[jb][q]);
            dstB[jb][4 * ib + q] = (T)(p[q] * __builtin_fmaf(u[jb][q], t[jb][q], gp[jb][q]));
          }
        }
      }
      if constexpr (FENCE) FBOB_SCHED_FENCE();
      if constexpr (kPrioOut) FBOB_PRIO_HIGH();
      const char* Qs = Qt + 32 * sc * Tile<T, D>::kRowBytes;
      const char* dOs = dOt + 32 * sc * Tile<T, D>::kRowBytes;
      const char* UQs = UQt + 32 * sc * Tile<T, D>::kRowBytes;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        if constexpr (FENCE) FBOB_SCHED_FENCE();
        const F qt = rd.tr(Qs, db);
        const F uqt = rd.tr(UQs, db);
        const F dot = rd.tr(dOs, db);
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
          accK[jb][db] = E::mma(qt, dstB[jb], accK[jb][db]);
          accK[jb][db] = E::mma(uqt, dsB[jb], accK[jb][db]);
          accV[jb][db] = E::mma(dot, ddpB[jb], accV[jb][db]);
        }
      }
      if constexpr (kPrioOut) FBOB_PRIO_LOW();
    };

    // This work-group's row steps of the tile (all of them unless SPLIT).
    int step_lo = 0, step_hi = nsteps;
    if constexpr (SPLIT) {
      const int base = tile == 0 ? 0 : steps0;
      step_lo = min(nsteps, max(0, part_lo - base));
      step_hi = min(nsteps, max(0, part_hi - base));
    }
    // An empty range (a part that does not reach this tile, or the empty last part
    // when the steps do not divide evenly) stages nothing, and its part of the sums
    // is written as zeros: step nsteps would address the query head after the group.
    // Uniform per work-group, so the barriers below stay uniform too.
    if (step_lo < step_hi) {
    ld_hq = step_lo / nrc;
    ld_rc = step_lo - ld_hq * nrc;
    load_step(lds[0]);
    if constexpr (DIRECT) wait_all_memory();
    store_step(lds[0]);
    __syncthreads();

    int cur_i0 = nxt_i0;  // first row of the step staged in `cur`
    auto step = [&](int t, char* cur, char* nxt) {
      const int i0 = cur_i0;
      const bool more = t + 1 < step_hi;
      if (more) load_step(nxt);
#pragma unroll
      for (int sc = 0; sc < BRS / 32; ++sc) {
        const bool active = !CAUSAL || i0 + 32 * sc + 31 >= jw0;
        if (active) chunk(cur, i0, sc);
      }
      // Unconditional, so that the compiler sees every load of the step complete
      // at the barrier (on the last step nothing is outstanding).
      if constexpr (DIRECT) wait_all_memory();
      if (more) store_step(nxt);
      __syncthreads();
      cur_i0 = nxt_i0;
    };
#pragma unroll 1
    for (int t = step_lo; t < step_hi; t += 2) {
      step(t, lds[0], lds[1]);
      if (t + 1 < step_hi) step(t + 1, lds[1], lds[0]);
    }
    }  // step_lo < step_hi

    // ---- single exclusive write of dK~ and dV~ ----
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
      const int j = jw0 + 16 * jb + r;
      if (SPLIT && j < N) {
        const int64_t heads = (int64_t)gridDim.x / ((int64_t)n_units * a.nsplit);
        float* pp = a.part + (((int64_t)split * heads + bhk) * N + j) * 2 * D;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int d0 = 16 * db + 4 * g;
          *reinterpret_cast<f32x4*>(pp + d0) = tau * accK[jb][db];
          *reinterpret_cast<f32x4*>(pp + D + d0) = accV[jb][db];
        }
      }
      if (!SPLIT && j < N) {
        const int64_t ro = kv_off + (int64_t)j * D;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int d0 = 16 * db + 4 * g;
          *reinterpret_cast<f32x4*>(a.dKt + ro + d0) = tau * accK[jb][db];
          *reinterpret_cast<f32x4*>(a.dVt + ro + d0) = accV[jb][db];
        }
      }
    }
  }
}

template <typename T, int D, int NW, int NJ, int BRS, int SCHED, int TM, bool DIRECT = false>
hipError_t launch_t(const Problem& p, const Pass2Args& a, hipStream_t s) {
  constexpr int kBCw = NW * 16 * NJ;
  const int n_col_tiles = (p.N + kBCw - 1) / kBCw;
  // causal d = 64: column tiles paired per work-group (see the kernel)
  const int n_units = p.causal && D < 128 ? (n_col_tiles + 1) / 2 : n_col_tiles;
  const int total = n_units * p.B * p.Hkv;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((pass2_kernel<T, D, NW, NJ, BRS, SCHED, TM, DIRECT, true>), dim3(total), dim3(NW * 64),
                       0, s, a, p.Hkv, group, p.N, p.tau, n_col_tiles, total);
  else
    hipLaunchKernelGGL((pass2_kernel<T, D, NW, NJ, BRS, SCHED, TM, DIRECT, false>), dim3(total), dim3(NW * 64),
                       0, s, a, p.Hkv, group, p.N, p.tau, n_col_tiles, total);
  return hipGetLastError();
}

template <typename T, int D, int NW, int NJ, int BRS, int SCHED, int TM, bool DIRECT>
hipError_t launch_split_t(const Problem& p, const Pass2Args& a, hipStream_t s) {
  constexpr int kBCw = NW * 16 * NJ;
  const int n_col_tiles = (p.N + kBCw - 1) / kBCw;
  const int n_units = p.causal && D < 128 ? (n_col_tiles + 1) / 2 : n_col_tiles;
  const int total = n_units * p.B * p.Hkv * a.nsplit;
  if (p.causal) {
    hipLaunchKernelGGL((pass2_kernel<T, D, NW, NJ, BRS, SCHED, TM, DIRECT, true, true>),
                       dim3(total), dim3(NW * 64), 0, s, a, p.Hkv, p.Hq / p.Hkv, p.N, p.tau,
                       n_col_tiles, total);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((pass2_kernel<T, D, NW, NJ, BRS, SCHED, TM, DIRECT, false, true>),
                     dim3(total), dim3(NW * 64), 0, s, a, p.Hkv, p.Hq / p.Hkv, p.N, p.tau,
                     n_col_tiles, total);
  return hipGetLastError();
}

}  // namespace

// The shipped bf16 variants of launch_pass2 below (d = 64 with tau a power of two, with
// or without the causal mask; d = 128 without it), in split form; split_plan admits no
// other problem.
hipError_t launch_pass2_split(const Problem& p, const Pass2Args& a, hipStream_t s) {
  if (p.d == 64) return launch_split_t<__bf16, 64, 8, 2, 64, 4, kTauPow2, true>(p, a, s);
  return launch_split_t<__bf16, 128, 8, 1, 64, false, kTauValu, true>(p, a, s);
}

hipError_t launch_pass2(const Problem& p, const Pass2Args& a, hipStream_t s) {
  if (p.bf16) {
    if (p.d == 64) {
      if (tau_is_pow2(p.tau)) {
#if FBOB_TUNING
        const int cfg = tune_choice("FBOB_TUNE_P2");
        if (cfg == 1) return launch_t<__bf16, 64, 8, 2, 64, false, kTauPow2, false>(p, a, s);
        if (cfg == 2) return launch_t<__bf16, 64, 8, 2, 64, true, kTauPow2, true>(p, a, s);
        if (cfg == 3) return launch_t<__bf16, 64, 8, 1, 64, true, kTauPow2, false>(p, a, s);
        if (cfg == 4) return launch_t<__bf16, 64, 8, 2, 64, 3, kTauPow2, true>(p, a, s);
        if (cfg == 5) return launch_t<__bf16, 64, 8, 2, 64, 0, kTauPow2, true>(p, a, s);
#endif
        return launch_t<__bf16, 64, 8, 2, 64, 4, kTauPow2, true>(p, a, s);
      }
      return launch_t<__bf16, 64, 8, 2, 64, false, kTauValu, true>(p, a, s);
    }
    // d = 128: unscaled operands (kTauValu) for two waves per SIMD, 64-row stages.
    // Alternatives: 1 with scheduling fences, 2 the one-wave-per-SIMD layout with
    // tau-scaled operand copies, 3 32-row stages.
#if FBOB_TUNING
    const int cfg = tune_choice("FBOB_TUNE_P2_D128");
    if (cfg == 1) return launch_t<__bf16, 128, 8, 1, 64, true, kTauValu, true>(p, a, s);
    if (cfg == 2) return launch_t<__bf16, 128, 4, 1, 32, true, kTauScaled>(p, a, s);
    if (cfg == 3) return launch_t<__bf16, 128, 8, 1, 32, true, kTauValu, true>(p, a, s);
#endif
    return launch_t<__bf16, 128, 8, 1, 64, false, kTauValu, true>(p, a, s);
  }
  if (p.d == 64) return launch_t<float, 64, 4, 1, 32, true, kTauScaled>(p, a, s);
  return launch_t<float, 128, 4, 1, 32, true, kTauValu>(p, a, s);
}

}  // namespace fbob
