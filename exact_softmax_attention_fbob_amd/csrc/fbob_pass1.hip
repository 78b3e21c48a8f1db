// fbob_pass1.hip - BoB Pass 1 (row-resident).
//
// FlashBoB notes, "关键设计" item 2 (first pass) with the affine decomposition of
// item 1.  For each query row i it streams every key tile j and accumulates
//   alpha_i  = sum_j P_ij F_ij                       F = tau (U_Q K^T + Q U_K^T)
//   B_i      = sum_j P_ij K_j
//   X_i      = sum_j dS_ij K_j                       dS = P o (dP - D), dP = dO V^T
//   Omega_i  = sum_j P_ij dP~'_ij K_j + dS_ij U_K,j  dP~' = F o (dP - D) + G, G = dO U_V^T
//   ddO~'_i  = sum_j P_ij F_ij V_j + P_ij U_V,j
// with P = exp(tau Q K^T - L) rebuilt from the stored log-partition L.  The
// printed correction dQ~ = tau (Omega - alpha R - E B), with R = sum_j P dP K and
// E = E' - alpha D, E'_i = sum_j P_ij dP~'_ij, is applied through R = X + D B:
//   dQ~ = tau (Omega - alpha X - E' B),  ddO~ = ddO~' - alpha O,  E = E' - alpha D.
// Expanding dP~' gives
//   E'_i = sum_j P F dP + P G - alpha_i D_i = <dO_i, ddO~'_i> - alpha_i <dO_i, O_i>
//        = <dO_i, ddO~_i>,
// so where alpha is an MFMA row sum (d = 64) E' is that dot product of the corrected
// row, formed once at the end instead of summed over the keys.  dQ~, ddO~, alpha and E
// are written exactly once per row.
//
// Schedule: one work-group = NW waves; each wave owns 16 query rows whose Q,
// tau Q, tau U_Q and dO operand fragments and the fp32 accumulators stay in
// registers for the whole sweep.  K, V, U_K, U_V tiles of BC keys (64 by default,
// processed as 32-key halves) are staged through LDS (double-buffered, one barrier
// per stage).  The four score-shaped
// tiles are computed transposed (key index on the MFMA row axis, query row on the
// column axis): their C registers are directly the B operand of the contractions
// over keys, whose A operand (K^T, V^T, U_K^T, U_V^T) comes from transposed LDS
// reads, and the outputs are accumulated transposed so that every row scalar is
// lane-local.  Row scalars enter as MFMA accumulator seeds (the dP tile starts at
// -D, giving dP - D directly), tau is folded into the resident operands of the F
// tile, and the row sum alpha is an MFMA contraction with a ones operand, which
// leaves seven VALU operations plus one exp per score element (E' comes from the
// identity above).  At d = 128 (twice
// the accumulators) the register budget of two waves per SIMD is met by keeping the
// operands unscaled (tau applied to the F tile on the VALU), taking alpha and E' as
// lane-local fp32 sums, and keeping one LDS offset per access pattern.  The d = 64
// kernels take the same lane sums when the caller asks for fp32 row sums (the VSUM
// form below): alpha then carries no bf16 rounding of P F, and E' is summed over the
// keys, since the identity above holds for the rounded products only with the MFMA alpha.
#include <type_traits>

#include "fbob_device.hpp"
#include "fbob_launch.hpp"

namespace fbob {
namespace {

// SCHED: 0 leaves instruction order to the compiler, 1 fences each phase and
// column block (sched_barrier), 2 double-buffers the LDS fragments one step ahead
// of the MFMAs that use them, with the order pinned by sched_group_barrier; 3 is 2
// with raised wave priority over the contraction MFMAs, 4 also over the score
// MFMAs.
// VSUM: the row sums alpha and E' as lane-local fp32 sums of the unrounded products
// (the d = 128 and multi-row-block layouts always do this).
// SPLIT: the work-group sweeps one part of its key stages and writes its raw
// accumulators and row sums to a.part_acc / a.part_rs; a reduction kernel adds the
// parts and applies the correction.  With the causal pairing the two row tiles' key
// stages form one sequence, cut into equal parts (a part may end in the first tile and
// start the second).
template <typename T, int D, int NW, int NI, int SCHED, int TM, int BC, bool DIRECT, bool CAUSAL,
          bool VSUM = false, bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) void pass1_kernel(Pass1Args a, int Hq, int group, int N,
                                                        float tau, int n_row_tiles, int total) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr bool FENCE = SCHED == 1;
  constexpr bool kPipe = SCHED >= 2;
  constexpr bool kPrioOut = SCHED >= 3;
  constexpr bool kPrioScore = SCHED >= 4;
  constexpr int kThreads = NW * 64;
  constexpr int kRW = 16 * NI;                       // query rows per wave
  constexpr int kBR = NW * kRW;                      // query rows per work-group
  constexpr int kBC = BC;                            // keys per LDS stage
  constexpr int kTB = kBC * Tile<T, D>::kRowBytes;   // bytes per staged tile
  constexpr int kDC = D / 32;
  constexpr int kDB = D / 16;
  __shared__ __attribute__((aligned(16))) char lds[2][4 * kTB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r = lane & 15, g = lane >> 4;
  const int logical = xcd_remap(blockIdx.x, total);
  // Causal (d = 64): a work-group takes row tiles n - 1 - p and p, so every
  // work-group sweeps the same number of key tiles; heads stay in consecutive
  // work-groups (their K/V tiles shared in one L2).  At d = 128 the pairing loop
  // does not fit the register budget: one tile per work-group, the longest
  // dispatched first.
  constexpr bool kFold = CAUSAL && D < 128;
  const int n_units = kFold ? (n_row_tiles + 1) / 2 : n_row_tiles;
  // SPLIT: the parts of one row tile are consecutive work-groups (one XCD).
  const int split = SPLIT ? logical % a.nsplit : 0;
  const int lt = SPLIT ? logical / a.nsplit : logical;
  const int bh = lt / n_units;
  const int unit = lt % n_units;
  const int b = bh / Hq, h = bh % Hq, hk = h / group;
  const int64_t q_off = (int64_t)bh * N * D;
  const int64_t kv_off = ((int64_t)b * (Hq / group) + hk) * N * D;
  const T* Qh = reinterpret_cast<const T*>(a.Q) + q_off;
  const T* dOh = reinterpret_cast<const T*>(a.dO) + q_off;
  const T* UQh = reinterpret_cast<const T*>(a.UQ) + q_off;
  const T* const kv_bases[4] = {reinterpret_cast<const T*>(a.K) + kv_off,
                                reinterpret_cast<const T*>(a.V) + kv_off,
                                reinterpret_cast<const T*>(a.UK) + kv_off,
                                reinterpret_cast<const T*>(a.UV) + kv_off};

  // Key stages of row tile rt (causal: up to its last row) and, under SPLIT, this
  // part's share [part_lo, part_hi) of the work-group's stages, counted over its tiles
  // in the order they run.
  auto key_end = [&](int rt) { return CAUSAL ? min(N, rt * kBR + kBR) : N; };
  auto stages_of = [&](int rt) { return (key_end(rt) + kBC - 1) / kBC; };
  const int rt_first = CAUSAL ? n_row_tiles - 1 - unit : unit;
  const bool two_tiles = kFold && unit != n_row_tiles - 1 - unit;
  int stages0 = 0, part_lo = 0, part_hi = 0;
  if constexpr (SPLIT) {
    stages0 = stages_of(rt_first);
    const int all = stages0 + (two_tiles ? stages_of(unit) : 0);
    const int per = (all + a.nsplit - 1) / a.nsplit;
    part_lo = min(all, split * per);
    part_hi = min(all, part_lo + per);
  }

  auto run_tile = [&](const int rt, const int tile) {
    // ---- resident row operands (B operand of the transposed score tiles) ----
    const int iw0 = rt * kBR + w * kRW;
    // tqf / tuqf hold tau Q / tau U_Q, or Q / U_Q unscaled under kTauValu; qf (Q for
    // the score tile) is a separate copy only under kTauScaled.
    constexpr bool kQcopy = TM == kTauScaled;
    F qf[kQcopy ? NI : 1][kDC], tqf[NI][kDC], tuqf[NI][kDC], dof[NI][kDC];
    float nl2[NI], dv[NI];
#pragma unroll
    for (int ib = 0; ib < NI; ++ib) {
      const int i = iw0 + 16 * ib + r;
#pragma unroll
      for (int dc = 0; dc < kDC; ++dc) {
        const F q0 = global_frag(Qh, i, N, D, 32 * dc + 8 * g);
        const F uq0 = global_frag(UQh, i, N, D, 32 * dc + 8 * g);
        if constexpr (kQcopy) qf[ib][dc] = q0;
        tqf[ib][dc] = TM == kTauValu ? q0 : scale_frag<T>(q0, tau);
        tuqf[ib][dc] = TM == kTauValu ? uq0 : scale_frag<T>(uq0, tau);
        dof[ib][dc] = global_frag(dOh, i, N, D, 32 * dc + 8 * g);
      }
      nl2[ib] = i < N ? -a.L[(int64_t)bh * N + i] * kLog2e : 0.f;
      dv[ib] = i < N ? a.D[(int64_t)bh * N + i] : 0.f;
    }
    // The row sum alpha = sum_j P F by MFMA: an operand of ones in rows 0..7 makes C
    // rows 0..7 hold it, so lane (r, g) holds alpha of row r for g < 2.
    const F onesA = r < 8 ? ones_frag<T>() : zero_frag<T>();
    // At d = 128 the register of the ones operand is worth more than the VALU adds:
    // there alpha and E' are lane-local fp32 partial sums (keys 4 g + q of row r),
    // reduced over the four lanes of a row at the end.
    constexpr bool kVsum = D >= 128 || NI >= 2 || VSUM;
    // With alpha summed from the same bf16-rounded P F that feed ddO~', E' is taken
    // as <dO_i, ddO~_i> at the end (the rounding of P F cancels in ddO~' - alpha o and
    // thus in E'); with an fp32 alpha it would not, so E' is summed over the keys.
    constexpr bool kEdot = !kVsum;
    float asum[NI], esum[NI];

    f32x4 accB[NI][kDB], accX[NI][kDB], accW[NI][kDB], accO[NI][kDB];
    f32x4 accAE[NI];
#pragma unroll
    for (int ib = 0; ib < NI; ++ib) {
      accAE[ib] = splat4(0.f);
      asum[ib] = 0.f;
      esum[ib] = 0.f;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        accB[ib][db] = splat4(0.f);
        accX[ib][db] = accB[ib][db];
        accW[ib][db] = accB[ib][db];
        accO[ib][db] = accB[ib][db];
      }
    }
    const float c1 = TM == kTauPow2 ? kLog2e : tau * kLog2e;
    // At d = 128 the lane keeps one LDS offset per access pattern (XOR form).
    const LdsLane<T, D, (D >= 128 || NI >= 2)> rd(r, g);

    int jbeg = 0, jend = key_end(rt);  // jbeg a multiple of kBC
    if constexpr (SPLIT) {
      const int base = tile == 0 ? 0 : stages0, full = stages_of(rt);
      jbeg = min(full, max(0, part_lo - base)) * kBC;
      jend = min(jend, min(full, max(0, part_hi - base)) * kBC);
    }
    const int ntc = max(jend - jbeg + kBC - 1, 0) / kBC;

    // Operand fragments of one 32-key tile for the contractions over keys.
    struct Frags {
      F p[NI], ds[NI], pf[NI], pw[NI];
    };

    // Scores and elementwise work of one 32-key tile, one 16-key block at a time;
    // the K, V, U_K, U_V fragments of a block serve every row block of the wave.
    // The bounds / causal test runs only on edge tiles (a wave-uniform branch
    // around the P values).
    // `edge_tag` is a bool (runtime test) or std::true_type / std::false_type (the
    // test resolved at compile time: a separate straight-line copy).
    auto score_body = [&](const char* Kt, int j0, Frags& fr, auto edge_tag) {
      const bool edge = edge_tag;
      const char* Vt = Kt + kTB;
      const char* UKt = Kt + 2 * kTB;
      const char* UVt = Kt + 3 * kTB;
      const auto rx = rd.fresh();
      // kPipe: the four fragments of (jb, dc) step it + 1 are read while step it's
      // MFMAs run (two register slots, alternating).
      constexpr int kSteps = 2 * kDC;
      F pk[2], pv[2], puk[2], puv[2];
      auto rowload = [&](int it, int sl) {
        pk[sl] = rx.row(Kt, it / kDC, it % kDC);
        pv[sl] = rx.row(Vt, it / kDC, it % kDC);
        puk[sl] = rx.row(UKt, it / kDC, it % kDC);
        puv[sl] = rx.row(UVt, it / kDC, it % kDC);
      };
      if constexpr (kPipe) {
        rowload(0, 0);
        FBOB_SGB(kSgDsRead, 4);
      }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        f32x4 s[NI], t[NI], f[NI], gg[NI];
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) {
          s[ib] = splat4(0.f);
          t[ib] = splat4(-dv[ib]);
          f[ib] = splat4(0.f);
          gg[ib] = splat4(0.f);
        }
        if constexpr (kPrioScore) FBOB_PRIO_HIGH();
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc) {
          const int it = jb * kDC + dc, sl = it & 1;
          F kf, vf, ukf, uvf;
          if constexpr (kPipe) {
            if (it + 1 < kSteps) {
              rowload(it + 1, sl ^ 1);
              FBOB_SGB(kSgDsRead, 4);
            }
            kf = pk[sl];
            vf = pv[sl];
            ukf = puk[sl];
            uvf = puv[sl];
          } else {
            kf = rx.row(Kt, jb, dc);
            vf = rx.row(Vt, jb, dc);
            ukf = rx.row(UKt, jb, dc);
            uvf = rx.row(UVt, jb, dc);
          }
#pragma unroll
          for (int ib = 0; ib < NI; ++ib) {
            s[ib] = E::mma(kf, kQcopy ? qf[kQcopy ? ib : 0][dc] : tqf[ib][dc], s[ib]);
            f[ib] = E::mma(kf, tuqf[ib][dc], f[ib]);
            f[ib] = E::mma(ukf, tqf[ib][dc], f[ib]);
            t[ib] = E::mma(vf, dof[ib][dc], t[ib]);
            gg[ib] = E::mma(uvf, dof[ib][dc], gg[ib]);
          }
          if constexpr (kPipe) FBOB_SGB(kSgMfma, 5 * NI);
        }
        if constexpr (kPrioScore) FBOB_PRIO_LOW();
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) {
          if constexpr (TM == kTauValu) f[ib] = tau * f[ib];
          f32x4 p;
#pragma unroll
          for (int q = 0; q < 4; ++q) p[q] = fast_exp2(__builtin_fmaf(s[ib][q], c1, nl2[ib]));
          if (edge) {
            const int i = iw0 + 16 * ib + r;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int j = j0 + 16 * jb + 4 * g + q;
              if (j >= N || (CAUSAL && j > i)) p[q] = 0.f;
            }
          }
          // elements 4 jb .. 4 jb + 3 of the fragments
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float pf = p[q] * f[ib][q];
            const float pw = p[q] * __builtin_fmaf(f[ib][q], t[ib][q], gg[ib][q]);
            fr.p[ib][4 * jb + q] = (T)p[q];
            fr.ds[ib][4 * jb + q] = (T)(p[q] * t[ib][q]);
            fr.pf[ib][4 * jb + q] = (T)pf;
            fr.pw[ib][4 * jb + q] = (T)pw;
            if constexpr (kVsum) {
              asum[ib] += pf;
              esum[ib] += pw;
            }
          }
        }
      }
    };
    // Under kPipe the bounds / causal test is compiled into a separate copy of the
    // tile body that only edge tiles take, so the pinned schedule spans one
    // straight-line region; otherwise it is a wave-uniform branch inside the body.
    auto score_phase = [&](const char* Kt, int j0, Frags& fr) {
      const bool edge = (j0 + 32 > N) || (CAUSAL && j0 + 31 > iw0);
      if constexpr (kPipe) {
        if (edge) score_body(Kt, j0, fr, std::true_type{});
        else score_body(Kt, j0, fr, std::false_type{});
      } else {
        score_body(Kt, j0, fr, edge);
      }
    };

    // Contractions over the tile's keys (transposed outputs) and the row sums.
    auto output_phase = [&](const char* Kt, const Frags& fr) {
      const char* Vt = Kt + kTB;
      const char* UKt = Kt + 2 * kTB;
      const char* UVt = Kt + 3 * kTB;
      if constexpr (FENCE) FBOB_SCHED_FENCE();
      if constexpr (kPrioOut) FBOB_PRIO_HIGH();
      const auto rx = rd.fresh();
      if constexpr (!kVsum) {
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) accAE[ib] = E::mma(onesA, fr.pf[ib], accAE[ib]);
        if constexpr (kPipe) FBOB_SGB(kSgMfma, NI);
      }
      // kPipe: the transposed fragments of column block db + 1 are read while
      // block db's MFMAs run (two register slots; each read is two instructions).
      F tk[2], tuk[2], tv[2], tuv[2];
      auto trload = [&](int db, int sl) {
        tk[sl] = rx.tr(Kt, db);
        tuk[sl] = rx.tr(UKt, db);
        tv[sl] = rx.tr(Vt, db);
        tuv[sl] = rx.tr(UVt, db);
      };
      if constexpr (kPipe) {
        trload(0, 0);
        FBOB_SGB(kSgDsRead, 8);
      }
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        if constexpr (FENCE) FBOB_SCHED_FENCE();
        F kt, ukt, vt, uvt;
        if constexpr (kPipe) {
          const int sl = db & 1;
          if (db + 1 < kDB) {
            trload(db + 1, sl ^ 1);
            FBOB_SGB(kSgDsRead, 8);
          }
          kt = tk[sl];
          ukt = tuk[sl];
          vt = tv[sl];
          uvt = tuv[sl];
        } else {
          kt = rx.tr(Kt, db);
          ukt = rx.tr(UKt, db);
          vt = rx.tr(Vt, db);
          uvt = rx.tr(UVt, db);
        }
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) {
          accB[ib][db] = E::mma(kt, fr.p[ib], accB[ib][db]);
          accX[ib][db] = E::mma(kt, fr.ds[ib], accX[ib][db]);
          accW[ib][db] = E::mma(kt, fr.pw[ib], accW[ib][db]);
          accW[ib][db] = E::mma(ukt, fr.ds[ib], accW[ib][db]);
          accO[ib][db] = E::mma(vt, fr.pf[ib], accO[ib][db]);
          accO[ib][db] = E::mma(uvt, fr.p[ib], accO[ib][db]);
        }
        if constexpr (kPipe) FBOB_SGB(kSgMfma, 6 * NI);
      }
      if constexpr (kPrioOut) FBOB_PRIO_LOW();
    };

    // Staging: registers + ds_write (MultiStager) or direct global -> LDS.
    using RegStager = MultiStager<T, D, kBC, 4, kThreads>;
    using DirStager = DirectStager<T, D, kBC, 4, NW, false, (D >= 128)>;
    typename std::conditional<DIRECT, DirStager, RegStager>::type st;
    auto stage_init = [&]() {
      if constexpr (DIRECT) st.init(kv_bases, w, lane);
      else st.init(kv_bases, tid);
    };
    // Issue the loads of the tile at key j0 (into `buf` when DIRECT).
    auto stage_load = [&](char* buf, int j0) {
      if constexpr (DIRECT) st.load(buf, j0, N);
      else st.load(j0, N);
    };
    // Make the staged tile visible in `buf` (the barrier follows).
    auto stage_commit = [&](char* buf) {
      if constexpr (DIRECT) wait_all_memory();
      else st.store(buf);
    };
    stage_init();
    stage_load(lds[0], jbeg);  // rows are clamped to N - 1 (an empty range computes nothing)
    stage_commit(lds[0]);
    __syncthreads();

    auto active_tile = [&](int j0) { return !CAUSAL || j0 <= iw0 + kRW - 1; };
    // Both 32-key halves of a stage (BC = 64) or the single one (BC = 32).
    auto compute_stage = [&](const char* cur, int j0) {
#pragma unroll
      for (int hs = 0; hs < kBC / 32; ++hs) {
        const int js = j0 + 32 * hs;
        if (!CAUSAL || js <= iw0 + kRW - 1) {
          Frags fr;
          score_phase(cur + 32 * hs * Tile<T, D>::kRowBytes, js, fr);
          output_phase(cur + 32 * hs * Tile<T, D>::kRowBytes, fr);
        }
      }
    };

    // One pipeline step: prefetch tile t+1, compute tile t from `cur`, publish
    // tile t+1 in `nxt`, barrier.  Unrolled by two so that both LDS buffers are
    // compile-time addresses.
    auto step = [&](int t, char* cur, char* nxt) {
      const int j0 = jbeg + t * kBC;
      const bool more = t + 1 < ntc;
      if (more) stage_load(nxt, j0 + kBC);
      if (active_tile(j0)) compute_stage(cur, j0);
      if (more) stage_commit(nxt);
      __syncthreads();
    };
#pragma unroll 1
    for (int t = 0; t < ntc; t += 2) {
      step(t, lds[0], lds[1]);
      if (t + 1 < ntc) step(t + 1, lds[1], lds[0]);
    }

    // ---- row correction and the single write of each row output ----
    // E' = E + alpha D equals <dO_i, ddO~_i> exactly (ddO~ = ddO~' - alpha o, and the
    // sum over keys of P dP~' expands to the same products); with kEdot it is formed
    // from the corrected ddO~ row here, otherwise it is the lane sums' total.
#pragma unroll
    for (int ib = 0; ib < NI; ++ib) {
      const int i = iw0 + 16 * ib + r;
      // F carries tau through the scaled resident operands.
      const float al = kVsum ? group_sum(asum[ib]) : __shfl(accAE[ib][0], r);
      const float esum_row = kEdot ? 0.f : group_sum(esum[ib]);
      if constexpr (SPLIT) {
        if (i < N) {
          const int64_t heads = (int64_t)gridDim.x / ((int64_t)n_units * a.nsplit);
          const int64_t prow = ((int64_t)split * heads + bh) * N + i;
          float* pa = a.part_acc + prow * 4 * D;
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            const int d0 = 16 * db + 4 * g;
            *reinterpret_cast<f32x4*>(pa + d0) = accB[ib][db];
            *reinterpret_cast<f32x4*>(pa + D + d0) = accX[ib][db];
            *reinterpret_cast<f32x4*>(pa + 2 * D + d0) = accW[ib][db];
            *reinterpret_cast<f32x4*>(pa + 3 * D + d0) = accO[ib][db];
          }
          if (g == 0) {  // E' of this part when it is summed over keys (else unused)
            a.part_rs[2 * prow] = al;
            a.part_rs[2 * prow + 1] = esum_row;
          }
        }
        continue;
      }
      const int64_t ro = q_off + (int64_t)i * D;
      float dot = 0.f;  // this lane's part of <dO_i, ddO~_i>
      if (i < N) {
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int d0 = 16 * db + 4 * g;
          const f32x4 o = *reinterpret_cast<const f32x4*>(a.O + ro + d0);
          accO[ib][db] -= al * o;  // ddO~
          if constexpr (kEdot) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              dot = __builtin_fmaf((float)dOh[(int64_t)i * D + d0 + q], accO[ib][db][q], dot);
          }
        }
      }
      // (the four lanes of row i share the branch above)
      const float edeg = kEdot ? group_sum(dot) : esum_row;
      if (i < N) {
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const int d0 = 16 * db + 4 * g;
          *reinterpret_cast<f32x4*>(a.ddOt + ro + d0) = accO[ib][db];
          *reinterpret_cast<f32x4*>(a.dQt + ro + d0) =
              tau * (accW[ib][db] - al * accX[ib][db] - edeg * accB[ib][db]);
        }
        if (g == 0) {
          a.alpha[(int64_t)bh * N + i] = al;
          a.E[(int64_t)bh * N + i] = edeg - al * dv[ib];
        }
      }
    }
  };
  if constexpr (kFold) {
#pragma unroll 1
    for (int tile = 0; tile < (two_tiles ? 2 : 1); ++tile)
      run_tile(tile == 0 ? rt_first : unit, tile);
  } else {
    run_tile(rt_first, 0);
  }
}

template <typename T, int D, int NW, int NI, int SCHED, int TM, int BC = 32, bool DIRECT = false,
          bool VSUM = false>
hipError_t launch_t(const Problem& p, const Pass1Args& a, hipStream_t s) {
  constexpr int kBR = NW * 16 * NI;
  const int n_row_tiles = (p.N + kBR - 1) / kBR;
  // causal d = 64: row tiles paired per work-group (see the kernel)
  const int n_units = p.causal && D < 128 ? (n_row_tiles + 1) / 2 : n_row_tiles;
  const int total = n_units * p.B * p.Hq;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((pass1_kernel<T, D, NW, NI, SCHED, TM, BC, DIRECT, true, VSUM>), dim3(total), dim3(NW * 64), 0, s,
                       a, p.Hq, group, p.N, p.tau, n_row_tiles, total);
  else
    hipLaunchKernelGGL((pass1_kernel<T, D, NW, NI, SCHED, TM, BC, DIRECT, false, VSUM>), dim3(total), dim3(NW * 64), 0,
                       s, a, p.Hq, group, p.N, p.tau, n_row_tiles, total);
  return hipGetLastError();
}

template <typename T, int D, int NW, int NI, int SCHED, int TM, int BC, bool DIRECT,
          bool VSUM = false>
hipError_t launch_split_t(const Problem& p, const Pass1Args& a, hipStream_t s) {
  constexpr int kBR = NW * 16 * NI;
  const int n_row_tiles = (p.N + kBR - 1) / kBR;
  const int n_units = p.causal && D < 128 ? (n_row_tiles + 1) / 2 : n_row_tiles;
  const int total = n_units * p.B * p.Hq * a.nsplit;
  if (p.causal) {
    hipLaunchKernelGGL((pass1_kernel<T, D, NW, NI, SCHED, TM, BC, DIRECT, true, VSUM, true>),
                       dim3(total), dim3(NW * 64), 0, s, a, p.Hq, p.Hq / p.Hkv, p.N, p.tau,
                       n_row_tiles, total);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((pass1_kernel<T, D, NW, NI, SCHED, TM, BC, DIRECT, false, VSUM, true>),
                     dim3(total), dim3(NW * 64), 0, s, a, p.Hq, p.Hq / p.Hkv, p.N, p.tau,
                     n_row_tiles, total);
  return hipGetLastError();
}

}  // namespace

// The shipped bf16 variants of launch_pass1 below (d = 64 with tau a power of two, with
// either row-sum form; d = 128), with or without the causal mask, in split form;
// split_plan admits no other problem.
hipError_t launch_pass1_split(const Problem& p, const Pass1Args& a, hipStream_t s) {
  if (p.d == 64 && p.fp32_row_sums)
    return launch_split_t<__bf16, 64, 8, 1, 3, kTauPow2, 64, true, true>(p, a, s);
  if (p.d == 64) return launch_split_t<__bf16, 64, 8, 1, 3, kTauPow2, 64, true>(p, a, s);
  return launch_split_t<__bf16, 128, 8, 1, true, kTauValu, 32, true>(p, a, s);
}

hipError_t launch_pass1(const Problem& p, const Pass1Args& a, hipStream_t s) {
  if (p.bf16) {
    if (p.d == 64) {
      // fp32 row sums on request: the same layouts with alpha and E' as lane sums
      if (p.fp32_row_sums) {
        if (tau_is_pow2(p.tau)) return launch_t<__bf16, 64, 8, 1, 3, kTauPow2, 64, true, true>(p, a, s);
        return launch_t<__bf16, 64, 8, 1, true, kTauValu, 64, true, true>(p, a, s);
      }
      if (tau_is_pow2(p.tau)) {
#if FBOB_TUNING
        const int cfg = tune_choice("FBOB_TUNE_P1");
        if (cfg == 1) return launch_t<__bf16, 64, 8, 1, 1, kTauPow2, 64, true>(p, a, s);
        if (cfg == 2) return launch_t<__bf16, 64, 8, 1, 1, kTauPow2, 32, true>(p, a, s);
        if (cfg == 3) return launch_t<__bf16, 64, 8, 1, 1, kTauPow2, 32, false>(p, a, s);
        if (cfg == 4) return launch_t<__bf16, 64, 8, 1, 0, kTauPow2, 64, true>(p, a, s);
        if (cfg == 5) return launch_t<__bf16, 64, 8, 1, 2, kTauPow2, 64, true>(p, a, s);
        if (cfg == 6) return launch_t<__bf16, 64, 8, 1, 4, kTauPow2, 64, true>(p, a, s);
        // one wave per SIMD with 32 query rows (K/V fragments shared by two row
        // blocks), compiler order, pinned order, pinned order + priority
        if (cfg == 7) return launch_t<__bf16, 64, 4, 2, 0, kTauPow2, 64, true>(p, a, s);
        if (cfg == 8) return launch_t<__bf16, 64, 4, 2, 2, kTauPow2, 64, true>(p, a, s);
        if (cfg == 9) return launch_t<__bf16, 64, 4, 2, 3, kTauPow2, 64, true>(p, a, s);
#endif
        return launch_t<__bf16, 64, 8, 1, 3, kTauPow2, 64, true>(p, a, s);
      }
      return launch_t<__bf16, 64, 8, 1, true, kTauValu, 64, true>(p, a, s);
    }
    // d = 128: two waves per SIMD need the unscaled operands (kTauValu), the VALU row
    // sums and the XOR-form LDS offsets to fit 256 registers; 32-key stages (64-key
    // stages spill).  Alternatives: 1 no scheduling fences, 2 the one-wave-per-SIMD
    // layout with tau-scaled operand copies.
#if FBOB_TUNING
    const int cfg = tune_choice("FBOB_TUNE_P1_D128");
    if (cfg == 1) return launch_t<__bf16, 128, 8, 1, false, kTauValu, 32, true>(p, a, s);
    if (cfg == 2) return launch_t<__bf16, 128, 4, 1, true, kTauScaled>(p, a, s);
#endif
    return launch_t<__bf16, 128, 8, 1, true, kTauValu, 32, true>(p, a, s);
  }
  if (p.d == 64) return launch_t<float, 64, 4, 1, true, kTauScaled>(p, a, s);
  return launch_t<float, 128, 4, 1, true, kTauValu>(p, a, s);
}

}  // namespace fbob
