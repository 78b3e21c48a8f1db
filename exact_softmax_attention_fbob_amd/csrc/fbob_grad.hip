// fbob_grad.hip - first-order attention backward (dQ, dK, dV) in two passes.
//
// FlashAttention blog ("FlashAttention 的反向传播设计"), section 一 for the
// gradients of one head,
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = tau dS K,  dK = tau dS^T Q,
// with D_i = dO_i . O_i, and section 二 for rebuilding P = exp(tau Q K^T - L)
// on chip from the stored log-partition L instead of keeping P.  The work is
// split like the two BoB passes of the FlashBoB notes ("关键设计" 2): a
// row-resident pass writes dQ (and D) and a column-resident pass writes dK and
// dV, summing the query heads of a key/value group on chip, so every output is
// written exactly once and no atomics are needed.  D is the row scalar that the
// BoB passes take, so this call also produces their complete row state.
//
// Both kernels reuse the layouts of the BoB passes: score tiles computed with
// the contracted index on the MFMA row axis so that their C registers are the B
// operand of the following contraction, dP - D obtained by seeding the dP
// accumulator with -D, staged tiles read back with the swizzled LDS readers, and
// the wave priority raised while a wave issues its contraction MFMAs (the other
// wave of the SIMD fills the gaps with its exp and elementwise work).

#include <type_traits>

#include "fbob_device.hpp"
#include "fbob_launch.hpp"

namespace fbob {
namespace {

// ---------------------------------------------------------------------------
// Row pass: each wave owns 16 NI query rows (Q and dO operand fragments in
// registers), streams K and V tiles of BC keys through LDS (every fragment read
// serves the NI row blocks) and accumulates dS K transposed (lane (r, g) holds
// columns 16 db + 4 g .. +3 of its row).  D_i is formed from the resident dO
// fragments and the fp32 O rows first.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int BC, bool DIRECT, bool CAUSAL, int NI = 1,
          bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) void grad_dq_kernel(GradArgs a, int Hq, int group, int N,
                                                          float tau, int n_row_tiles, int total) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int kThreads = NW * 64;
  constexpr int kRW = 16 * NI;  // query rows per wave
  constexpr int kBR = NW * kRW;
  constexpr int kTB = BC * Tile<T, D>::kRowBytes;
  constexpr int kDC = D / 32;
  constexpr int kDB = D / 16;
  __shared__ __attribute__((aligned(16))) char lds[2][2 * kTB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int logical = xcd_remap(blockIdx.x, total);
  // SPLIT: the parts of one row tile are consecutive work-groups (one XCD).
  const int split = SPLIT ? logical % a.nsplit : 0;
  const int lt = SPLIT ? logical / a.nsplit : logical;
  const int bh = lt / n_row_tiles;
  // Causal: the last row tiles see the most keys, so they are dispatched first.
  const int rt = CAUSAL ? n_row_tiles - 1 - lt % n_row_tiles : lt % n_row_tiles;
  const int b = bh / Hq, h = bh % Hq, hk = h / group;
  const int64_t q_off = (int64_t)bh * N * D;
  const int64_t kv_off = ((int64_t)b * (Hq / group) + hk) * N * D;
  const T* Qh = reinterpret_cast<const T*>(a.Q) + q_off;
  const T* dOh = reinterpret_cast<const T*>(a.dO) + q_off;
  const T* const kv_bases[2] = {reinterpret_cast<const T*>(a.K) + kv_off,
                                reinterpret_cast<const T*>(a.V) + kv_off};

  const int iw0 = rt * kBR + w * kRW;
  // this lane's query row in row block ib: iw0 + 16 ib + r
  F qf[NI][kDC], dof[NI][kDC];
  float dv[NI], nl2[NI];
#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
    const int i = iw0 + 16 * ib + r;
    float dpart = 0.f;
#pragma unroll
    for (int dc = 0; dc < kDC; ++dc) {
      const int col = 32 * dc + 8 * g;
      qf[ib][dc] = global_frag(Qh, i, N, D, col);
      dof[ib][dc] = global_frag(dOh, i, N, D, col);
      if (i < N) {
        const f32x4* op = reinterpret_cast<const f32x4*>(a.O + q_off + (int64_t)i * D + col);
        const f32x4 o0 = op[0], o1 = op[1];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dpart += (float)dof[ib][dc][q] * o0[q] + (float)dof[ib][dc][4 + q] * o1[q];
      }
    }
    dv[ib] = group_sum(dpart);  // D_i: the 4 lanes of row r hold 8 columns each
    nl2[ib] = i < N ? -a.L[(int64_t)bh * N + i] * kLog2e : 0.f;
    if (i < N && g == 0 && split == 0) a.D[(int64_t)bh * N + i] = dv[ib];
  }

  f32x4 accX[NI][kDB];
#pragma unroll
  for (int ib = 0; ib < NI; ++ib)
#pragma unroll
    for (int db = 0; db < kDB; ++db) accX[ib][db] = splat4(0.f);
  const float c1 = tau * kLog2e;
  const LdsLane<T, D> rd(r, g);

  const int jend = CAUSAL ? min(N, rt * kBR + kBR) : N;
  const int ntc = (jend + BC - 1) / BC;
  // this work-group's key stages [t_lo, t_hi): all of them, or its part's share
  int t_lo = 0, t_hi = ntc;
  if constexpr (SPLIT) {
    const int per = (ntc + a.nsplit - 1) / a.nsplit;
    t_lo = min(ntc, split * per);
    t_hi = min(ntc, t_lo + per);
  }

  // 32 keys at j0 from the staged K tile Kt (V tile follows it).
  auto half = [&](const char* Kt, int j0) {
    const char* Vt = Kt + kTB;
    const bool edge = (j0 + 32 > N) || (CAUSAL && j0 + 31 > iw0);
    F ds[NI];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      f32x4 s[NI], t[NI];
#pragma unroll
      for (int ib = 0; ib < NI; ++ib) {
        s[ib] = splat4(0.f);
        t[ib] = splat4(-dv[ib]);
      }
#pragma unroll
      for (int dc = 0; dc < kDC; ++dc) {
        const F kf = rd.row(Kt, jb, dc), vf = rd.row(Vt, jb, dc);
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) {
          s[ib] = E::mma(kf, qf[ib][dc], s[ib]);
          t[ib] = E::mma(vf, dof[ib][dc], t[ib]);
        }
      }
#pragma unroll
      for (int ib = 0; ib < NI; ++ib) {
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
#pragma unroll
        for (int q = 0; q < 4; ++q) ds[ib][4 * jb + q] = (T)(p[q] * t[ib][q]);
      }
    }
    FBOB_PRIO_HIGH();
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const F kt = rd.tr(Kt, db);
#pragma unroll
      for (int ib = 0; ib < NI; ++ib) accX[ib][db] = E::mma(kt, ds[ib], accX[ib][db]);
    }
    FBOB_PRIO_LOW();
  };

  using RegStager = MultiStager<T, D, BC, 2, kThreads>;
  using DirStager = DirectStager<T, D, BC, 2, NW, true>;
  typename std::conditional<DIRECT, DirStager, RegStager>::type st;
  if constexpr (DIRECT) st.init(kv_bases, w, lane);
  else st.init(kv_bases, tid);
  auto stage_load = [&](char* buf, int j0) {
    if constexpr (DIRECT) st.load(buf, j0, N);
    else st.load(j0, N);
  };
  auto stage_commit = [&](char* buf) {
    if constexpr (DIRECT) wait_all_memory();
    else st.store(buf);
  };
  if (!SPLIT || t_lo < t_hi) {  // (an empty part stages nothing)
    stage_load(lds[0], t_lo * BC);
    stage_commit(lds[0]);
  }
  __syncthreads();

  auto step = [&](int t, char* cur, char* nxt) {
    const int j0 = t * BC;
    const bool more = t + 1 < t_hi;
    if (more) stage_load(nxt, j0 + BC);
#pragma unroll
    for (int hs = 0; hs < BC / 32; ++hs) {
      const int js = j0 + 32 * hs;
      if (!CAUSAL || js <= iw0 + kRW - 1) half(cur + 32 * hs * Tile<T, D>::kRowBytes, js);
    }
    if (more) stage_commit(nxt);
    __syncthreads();
  };
#pragma unroll 1
  for (int t = t_lo; t < t_hi; t += 2) {
    step(t, lds[0], lds[1]);
    if (t + 1 < t_hi) step(t + 1, lds[1], lds[0]);
  }

#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
    const int i = iw0 + 16 * ib + r;
    if (SPLIT && i < N) {  // this part's tau dQ (zeros for an empty part)
      const int64_t heads = (int64_t)gridDim.x / ((int64_t)n_row_tiles * a.nsplit);
      float* pp = a.part + (((int64_t)split * heads + bh) * N + i) * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        *reinterpret_cast<f32x4*>(pp + 16 * db + 4 * g) = tau * accX[ib][db];
    } else if (i < N) {
      const int64_t ro = q_off + (int64_t)i * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        *reinterpret_cast<f32x4*>(a.dQ + ro + 16 * db + 4 * g) = tau * accX[ib][db];
    }
  }
}

// ---------------------------------------------------------------------------
// Column pass: each wave owns 16 NJ keys (K and V fragments in registers),
// streams row tiles of Q and dO (BRS rows) plus the row scalars -L log2 e and
// -D through LDS for every query head of the group, and accumulates
// dK^T += Q^T dS and dV^T += dO^T P with the score C registers as B operands.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int NJ, int BRS, bool DIRECT, bool CAUSAL,
          bool SPLIT = false>
__global__ __launch_bounds__(NW * 64) void grad_dkv_kernel(GradArgs a, int Hkv, int group, int N,
                                                           float tau, int n_col_tiles, int total) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int kThreads = NW * 64;
  constexpr int kCW = 16 * NJ;
  constexpr int kBCw = NW * kCW;
  constexpr int kTB = BRS * Tile<T, D>::kRowBytes;
  constexpr int kDC = D / 32;
  constexpr int kDB = D / 16;
  constexpr int kStage = 2 * kTB + 2 * BRS * 4;
  static_assert(kThreads >= BRS, "one thread per staged row scalar");
  __shared__ __attribute__((aligned(16))) char lds[2][kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int logical = xcd_remap(blockIdx.x, total);
  // SPLIT: the parts of one column tile are consecutive work-groups (one XCD).
  const int split = SPLIT ? logical % a.nsplit : 0;
  const int lt = SPLIT ? logical / a.nsplit : logical;
  const int bhk = lt / n_col_tiles, ct = lt % n_col_tiles;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int Hq = Hkv * group;
  const int64_t kv_off = (int64_t)bhk * N * D;
  const T* Kh = reinterpret_cast<const T*>(a.K) + kv_off;
  const T* Vh = reinterpret_cast<const T*>(a.V) + kv_off;

  const int jw0 = ct * kBCw + w * kCW;
  F kf[NJ][kDC], vf[NJ][kDC];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
    for (int dc = 0; dc < kDC; ++dc) {
      const int j = jw0 + 16 * jb + r, col = 32 * dc + 8 * g;
      kf[jb][dc] = global_frag(Kh, j, N, D, col);
      vf[jb][dc] = global_frag(Vh, j, N, D, col);
    }
  f32x4 accK[NJ][kDB], accV[NJ][kDB];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      accK[jb][db] = splat4(0.f);
      accV[jb][db] = accK[jb][db];
    }
  const float c1 = tau * kLog2e;
  const LdsLane<T, D> rd(r, g);

  const int i_begin = CAUSAL ? (ct * kBCw / BRS) * BRS : 0;
  const int nrc = (N - i_begin + BRS - 1) / BRS;
  const int nsteps = nrc * group;
  // this work-group's steps [t_lo, t_hi): all of them, or its part's share
  int t_lo = 0, t_hi = nsteps;
  if constexpr (SPLIT) {
    const int per = (nsteps + a.nsplit - 1) / a.nsplit;
    t_lo = min(nsteps, split * per);
    t_hi = min(nsteps, t_lo + per);
  }
  const int64_t q_head = (int64_t)N * D * (int64_t)sizeof(T);
  const int64_t q0 = ((int64_t)b * Hq + (int64_t)hk * group) * N * D;
  const T* const q_bases[2] = {reinterpret_cast<const T*>(a.Q) + q0,
                               reinterpret_cast<const T*>(a.dO) + q0};
  using RegStager = MultiStager<T, D, BRS, 2, kThreads>;
  using DirStager = DirectStager<T, D, BRS, 2, NW, true>;
  typename std::conditional<DIRECT, DirStager, RegStager>::type st;
  if constexpr (DIRECT) st.init(q_bases, w, lane);
  else st.init(q_bases, tid);
  const int64_t s0 = ((int64_t)b * Hq + (int64_t)hk * group) * N;
  float sl = 0.f, sd = 0.f;
  // The raw L and D stay in registers until store_step: deriving the seeds here
  // would make this wave wait for every load it has in flight (the tiles'
  // included) before it computes the current stage.
  // Steps run in order: the next one to load is query head ld_hq, row chunk ld_rc
  // (advanced by one chunk per load rather than divided out of the step index).
  int ld_hq = 0, ld_rc = 0, nxt_i0 = 0;
  if constexpr (SPLIT) {  // the part's first step (one division, before the sweep)
    ld_hq = t_lo / nrc;
    ld_rc = t_lo - ld_hq * nrc;
  }
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
    if (tid < BRS) {
      const int64_t ri = s0 + (int64_t)hq * N + min(i0 + tid, N - 1);
      sl = a.L[ri];
      sd = a.D[ri];
    }
  };
  // (DIRECT: the caller has waited for every load of the step.)
  auto store_step = [&](char* buf) {
    if constexpr (!DIRECT) st.store(buf);
    if (tid < BRS) {
      float* sp = reinterpret_cast<float*>(buf + 2 * kTB);
      sp[tid] = -sl * kLog2e;
      sp[BRS + tid] = -sd;
    }
  };

  auto chunk = [&](const char* buf, int i0, int sc) {
    const char* Qt = buf;
    const char* dOt = buf + kTB;
    const float* sp = reinterpret_cast<const float*>(buf + 2 * kTB);
    const int ic = i0 + 32 * sc;
    const bool edge = (ic + 32 > N) || (CAUSAL && ic < jw0 + kCW - 1);
    F pB[NJ], dsB[NJ];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const int rr = 32 * sc + 16 * ib + 4 * g;
      const f32x4 nL = *reinterpret_cast<const f32x4*>(sp + rr);
      const f32x4 nD = *reinterpret_cast<const f32x4*>(sp + BRS + rr);
      f32x4 s[NJ], t[NJ];
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        s[jb] = splat4(0.f);
        t[jb] = nD;
      }
#pragma unroll
      for (int dc = 0; dc < kDC; ++dc) {
        const F qa = rd.row(Qt, 2 * sc + ib, dc);
        const F doa = rd.row(dOt, 2 * sc + ib, dc);
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
          s[jb] = E::mma(qa, kf[jb][dc], s[jb]);
          t[jb] = E::mma(doa, vf[jb][dc], t[jb]);
        }
      }
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
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
          pB[jb][4 * ib + q] = (T)p[q];
          dsB[jb][4 * ib + q] = (T)(p[q] * t[jb][q]);
        }
      }
    }
    FBOB_PRIO_HIGH();
    const char* Qs = Qt + 32 * sc * Tile<T, D>::kRowBytes;
    const char* dOs = dOt + 32 * sc * Tile<T, D>::kRowBytes;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const F qt = rd.tr(Qs, db);
      const F dot = rd.tr(dOs, db);
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        accK[jb][db] = E::mma(qt, dsB[jb], accK[jb][db]);
        accV[jb][db] = E::mma(dot, pB[jb], accV[jb][db]);
      }
    }
    FBOB_PRIO_LOW();
  };

  if (!SPLIT || t_lo < t_hi) {  // (an empty part stages nothing)
    load_step(lds[0]);
    if constexpr (DIRECT) wait_all_memory();
    store_step(lds[0]);
  }
  __syncthreads();
  int cur_i0 = nxt_i0;
  auto step = [&](int t, char* cur, char* nxt) {
    const int i0 = cur_i0;
    const bool more = t + 1 < t_hi;
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
  for (int t = t_lo; t < t_hi; t += 2) {
    step(t, lds[0], lds[1]);
    if (t + 1 < t_hi) step(t + 1, lds[1], lds[0]);
  }

#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int j = jw0 + 16 * jb + r;
    if (SPLIT && j < N) {  // this part's tau dK, dV (zeros for an empty part)
      const int64_t heads = (int64_t)gridDim.x / ((int64_t)n_col_tiles * a.nsplit);
      float* pp = a.part + (((int64_t)split * heads + bhk) * N + j) * 2 * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int d0 = 16 * db + 4 * g;
        *reinterpret_cast<f32x4*>(pp + d0) = tau * accK[jb][db];
        *reinterpret_cast<f32x4*>(pp + D + d0) = accV[jb][db];
      }
    } else if (j < N) {
      const int64_t ro = kv_off + (int64_t)j * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int d0 = 16 * db + 4 * g;
        *reinterpret_cast<f32x4*>(a.dK + ro + d0) = tau * accK[jb][db];
        *reinterpret_cast<f32x4*>(a.dV + ro + d0) = accV[jb][db];
      }
    }
  }
}

template <typename T, int D, int NW, int BC, bool DIRECT, int NI = 1>
hipError_t launch_dq(const Problem& p, const GradArgs& a, hipStream_t s) {
  constexpr int kBR = NW * 16 * NI;
  const int n_row_tiles = (p.N + kBR - 1) / kBR;
  const int total = n_row_tiles * p.B * p.Hq;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((grad_dq_kernel<T, D, NW, BC, DIRECT, true, NI>), dim3(total), dim3(NW * 64), 0, s,
                       a, p.Hq, group, p.N, p.tau, n_row_tiles, total);
  else
    hipLaunchKernelGGL((grad_dq_kernel<T, D, NW, BC, DIRECT, false, NI>), dim3(total), dim3(NW * 64), 0,
                       s, a, p.Hq, group, p.N, p.tau, n_row_tiles, total);
  return hipGetLastError();
}

template <typename T, int D, int NW, int NJ, int BRS, bool DIRECT>
hipError_t launch_dkv(const Problem& p, const GradArgs& a, hipStream_t s) {
  constexpr int kBCw = NW * 16 * NJ;
  const int n_col_tiles = (p.N + kBCw - 1) / kBCw;
  const int total = n_col_tiles * p.B * p.Hkv;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((grad_dkv_kernel<T, D, NW, NJ, BRS, DIRECT, true>), dim3(total),
                       dim3(NW * 64), 0, s, a, p.Hkv, group, p.N, p.tau, n_col_tiles, total);
  else
    hipLaunchKernelGGL((grad_dkv_kernel<T, D, NW, NJ, BRS, DIRECT, false>), dim3(total),
                       dim3(NW * 64), 0, s, a, p.Hkv, group, p.N, p.tau, n_col_tiles, total);
  return hipGetLastError();
}

template <typename T, int D, int NW, int BC, bool DIRECT, int NI>
hipError_t launch_dq_split(const Problem& p, const GradArgs& a, hipStream_t s) {
  constexpr int kBR = NW * 16 * NI;
  const int n_row_tiles = (p.N + kBR - 1) / kBR;
  const int total = n_row_tiles * p.B * p.Hq * a.nsplit;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((grad_dq_kernel<T, D, NW, BC, DIRECT, true, NI, true>), dim3(total),
                       dim3(NW * 64), 0, s, a, p.Hq, group, p.N, p.tau, n_row_tiles, total);
  else
    hipLaunchKernelGGL((grad_dq_kernel<T, D, NW, BC, DIRECT, false, NI, true>), dim3(total),
                       dim3(NW * 64), 0, s, a, p.Hq, group, p.N, p.tau, n_row_tiles, total);
  return hipGetLastError();
}

template <typename T, int D, int NW, int NJ, int BRS, bool DIRECT>
hipError_t launch_dkv_split(const Problem& p, const GradArgs& a, hipStream_t s) {
  constexpr int kBCw = NW * 16 * NJ;
  const int n_col_tiles = (p.N + kBCw - 1) / kBCw;
  const int total = n_col_tiles * p.B * p.Hkv * a.nsplit;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((grad_dkv_kernel<T, D, NW, NJ, BRS, DIRECT, true, true>), dim3(total),
                       dim3(NW * 64), 0, s, a, p.Hkv, group, p.N, p.tau, n_col_tiles, total);
  else
    hipLaunchKernelGGL((grad_dkv_kernel<T, D, NW, NJ, BRS, DIRECT, false, true>), dim3(total),
                       dim3(NW * 64), 0, s, a, p.Hkv, group, p.N, p.tau, n_col_tiles, total);
  return hipGetLastError();
}

}  // namespace

// The shipped bf16 layouts of the two passes below, in split form (bf16 only).
hipError_t launch_grad_dq_split(const Problem& p, const GradArgs& a, hipStream_t s) {
  if (p.d == 64) return launch_dq_split<__bf16, 64, 8, 128, true, 2>(p, a, s);
  return launch_dq_split<__bf16, 128, 8, 64, true, 2>(p, a, s);
}

hipError_t launch_grad_dkv_split(const Problem& p, const GradArgs& a, hipStream_t s) {
  if (p.d == 64) return launch_dkv_split<__bf16, 64, 8, 2, 64, true>(p, a, s);
  return launch_dkv_split<__bf16, 128, 8, 1, 32, true>(p, a, s);
}

hipError_t launch_grad_dq(const Problem& p, const GradArgs& a, hipStream_t s) {
  if (p.bf16) {
    // 32 query rows per wave (~3-5 % faster than 16 on the whole backward); 1
    // selects 16 rows per wave, 2 the other stage size.
#if FBOB_TUNING
    const int cfg = tune_choice(p.d == 64 ? "FBOB_TUNE_DQ" : "FBOB_TUNE_DQ_D128");
#endif
    if (p.d == 64) {
#if FBOB_TUNING
      if (cfg == 1) return launch_dq<__bf16, 64, 8, 64, true, 1>(p, a, s);
      if (cfg == 2) return launch_dq<__bf16, 64, 8, 64, true, 2>(p, a, s);
      // four-wave work-groups: three per CU at 64-key stages, two at 128
      if (cfg == 3) return launch_dq<__bf16, 64, 4, 64, true, 2>(p, a, s);
      if (cfg == 4) return launch_dq<__bf16, 64, 4, 128, true, 2>(p, a, s);
#endif
      return launch_dq<__bf16, 64, 8, 128, true, 2>(p, a, s);
    }
#if FBOB_TUNING
    if (cfg == 1) return launch_dq<__bf16, 128, 8, 32, true, 1>(p, a, s);
    if (cfg == 2) return launch_dq<__bf16, 128, 8, 32, true, 2>(p, a, s);
#endif
    return launch_dq<__bf16, 128, 8, 64, true, 2>(p, a, s);
  }
  if (p.d == 64) return launch_dq<float, 64, 4, 32, false>(p, a, s);
  return launch_dq<float, 128, 4, 32, false>(p, a, s);
}

hipError_t launch_grad_dkv(const Problem& p, const GradArgs& a, hipStream_t s) {
  if (p.bf16) {
#if FBOB_TUNING
    // four-wave work-groups (two or three per CU, by registers)
    if (p.d == 64 && tune_choice("FBOB_TUNE_DKV") == 1)
      return launch_dkv<__bf16, 64, 4, 2, 64, true>(p, a, s);
#endif
    if (p.d == 64) return launch_dkv<__bf16, 64, 8, 2, 64, true>(p, a, s);
    return launch_dkv<__bf16, 128, 8, 1, 32, true>(p, a, s);
  }
  if (p.d == 64) return launch_dkv<float, 64, 4, 1, 32, false>(p, a, s);
  return launch_dkv<float, 128, 4, 1, 32, false>(p, a, s);
}

}  // namespace fbob
