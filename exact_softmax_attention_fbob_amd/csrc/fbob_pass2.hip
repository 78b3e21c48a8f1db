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
// Schedule: one work-group = 4 waves; each wave owns 16*NJ key positions whose
// K, V, U_K, U_V operand fragments and the two fp32 accumulators stay in
// registers.  Q, dO, U_Q row tiles of 32 rows plus their four row scalars are
// staged through LDS (double-buffered).  Scores are computed with the query index
// on the MFMA row axis, so a lane owns one key and four consecutive rows per
// block; those C registers are directly the B operand of the contractions over
// rows, whose A operand (Q^T, U_Q^T, dO^T) comes from transposed LDS reads.
#include "fbob_device.hpp"
#include "fbob_launch.hpp"

namespace fbob {
namespace {

constexpr int kThreads = 256;
constexpr int kBRs = 32;  // rows per LDS stage

template <typename T, int D, int NJ, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void pass2_kernel(Pass2Args a, int Hkv, int group, int N,
                                                         float tau, int n_col_tiles, int total) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int kColsW = 16 * NJ;
  constexpr int kBCw = 4 * kColsW;
  constexpr int kTB = kBRs * Tile<T, D>::kRowBytes;
  constexpr int kDC = D / 32;
  constexpr int kDB = D / 16;
  constexpr int kScal = 4 * kBRs * 4;  // L, D, alpha, E for the stage rows (bytes)
  __shared__ __attribute__((aligned(16))) char lds[2][3 * kTB + kScal];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int logical = xcd_remap(blockIdx.x, total);
  const int bhk = logical / n_col_tiles, ct = logical % n_col_tiles;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int Hq = Hkv * group;
  const int64_t kv_off = (int64_t)bhk * N * D;
  const T* Kh = reinterpret_cast<const T*>(a.K) + kv_off;
  const T* Vh = reinterpret_cast<const T*>(a.V) + kv_off;
  const T* UKh = reinterpret_cast<const T*>(a.UK) + kv_off;
  const T* UVh = reinterpret_cast<const T*>(a.UV) + kv_off;

  const int jw0 = ct * kBCw + w * kColsW;
  F kf[NJ][kDC], vf[NJ][kDC], ukf[NJ][kDC], uvf[NJ][kDC];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
    for (int dc = 0; dc < kDC; ++dc) {
      const int j = jw0 + 16 * jb + r, col = 32 * dc + 8 * g;
      kf[jb][dc] = global_frag(Kh, j, N, D, col);
      vf[jb][dc] = global_frag(Vh, j, N, D, col);
      ukf[jb][dc] = global_frag(UKh, j, N, D, col);
      uvf[jb][dc] = global_frag(UVh, j, N, D, col);
    }

  f32x4 accK[NJ][kDB], accV[NJ][kDB];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      accK[jb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      accV[jb][db] = accK[jb][db];
    }
  const float c1 = tau * kLog2e;

  // Row chunks: causal rows start at the work-group's first key.
  const int i_begin = CAUSAL ? (ct * kBCw / kBRs) * kBRs : 0;
  const int nrc = (N - i_begin + kBRs - 1) / kBRs;
  const int nsteps = nrc * group;  // (query head of the group, row chunk)

  Stager<T, D, kBRs, kThreads> sq, sdo, suq;
  const T* const Qg = reinterpret_cast<const T*>(a.Q);
  const T* const dOg = reinterpret_cast<const T*>(a.dO);
  const T* const UQg = reinterpret_cast<const T*>(a.UQ);
  // Row scalar streamed by this thread (tid < 4 * kBRs): L, D, alpha or E.
  const int which = tid / kBRs;
  const float* const scal_src = which == 0 ? a.L : which == 1 ? a.D : which == 2 ? a.alpha : a.E;
  float sc_v = 0.f;
  auto load_step = [&](int step) {
    const int hq = hk * group + step / nrc;
    const int i0 = i_begin + (step % nrc) * kBRs;
    const int64_t q_off = ((int64_t)b * Hq + hq) * N * D;
    sq.load(Qg + q_off, i0, N, tid);
    sdo.load(dOg + q_off, i0, N, tid);
    suq.load(UQg + q_off, i0, N, tid);
    if (tid < 4 * kBRs) {
      const int i = i0 + tid % kBRs;
      sc_v = i < N ? scal_src[((int64_t)b * Hq + hq) * N + i] : 0.f;
    }
  };
  auto store_step = [&](char* buf) {
    sq.store(buf, tid);
    sdo.store(buf + kTB, tid);
    suq.store(buf + 2 * kTB, tid);
    if (tid < 4 * kBRs) reinterpret_cast<float*>(buf + 3 * kTB)[tid] = sc_v;
  };

  load_step(0);
  store_step(lds[0]);
  __syncthreads();

  for (int t = 0; t < nsteps; ++t) {
    const int i0 = i_begin + (t % nrc) * kBRs;
    const bool more = t + 1 < nsteps;
    if (more) load_step(t + 1);
    const char* Qt = lds[t & 1];
    const char* dOt = Qt + kTB;
    const char* UQt = Qt + 2 * kTB;
    const float* sc = reinterpret_cast<const float*>(Qt + 3 * kTB);
    const bool active = !CAUSAL || i0 + kBRs - 1 >= jw0;
    if (active) {
      // ---- score-shaped tiles: [row block ib][key block jb] ----
      f32x4 s[2][NJ], dp[2][NJ], f[2][NJ], gg[2][NJ];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
          s[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[ib][jb] = s[ib][jb];
          f[ib][jb] = s[ib][jb];
          gg[ib][jb] = s[ib][jb];
        }
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc) {
          const int row = 16 * ib + r, col = 32 * dc + 8 * g;
          const F qa = lds_frag_row<T, D>(Qt, row, col);
          const F doa = lds_frag_row<T, D>(dOt, row, col);
          const F uqa = lds_frag_row<T, D>(UQt, row, col);
#pragma unroll
          for (int jb = 0; jb < NJ; ++jb) {
            s[ib][jb] = E::mma(qa, kf[jb][dc], s[ib][jb]);
            f[ib][jb] = E::mma(uqa, kf[jb][dc], f[ib][jb]);
            f[ib][jb] = E::mma(qa, ukf[jb][dc], f[ib][jb]);
            dp[ib][jb] = E::mma(doa, vf[jb][dc], dp[ib][jb]);
            gg[ib][jb] = E::mma(doa, uvf[jb][dc], gg[ib][jb]);
          }
        }
      // ---- elementwise with per-row scalars (rows 16 ib + 4 g + q) ----
      const bool edge = (i0 + kBRs > N) || (CAUSAL && i0 < jw0 + kColsW - 1);
      F dstB[NJ], dsB[NJ], ddpB[NJ];
      f32x4 vdst[NJ][2], vds[NJ][2], vddp[NJ][2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const int rr = 16 * ib + 4 * g;
        const f32x4 Lr = *reinterpret_cast<const f32x4*>(sc + rr) * kLog2e;
        const f32x4 Dr = *reinterpret_cast<const f32x4*>(sc + kBRs + rr);
        const f32x4 Ar = *reinterpret_cast<const f32x4*>(sc + 2 * kBRs + rr);
        const f32x4 Er = *reinterpret_cast<const f32x4*>(sc + 3 * kBRs + rr);
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float p = fast_exp2(s[ib][jb][q] * c1 - Lr[q]);
            if (edge) {
              const int i = i0 + rr + q, j = jw0 + 16 * jb + r;
              if (i >= N || (CAUSAL && j > i)) p = 0.f;
            }
            const float dpv = dp[ib][jb][q];
            const float tv = dpv - Dr[q];
            const float fv = f[ib][jb][q] * tau;
            const float dpt = fv * tv - Ar[q] * dpv + gg[ib][jb][q];
            vds[jb][ib][q] = p * tv;
            vdst[jb][ib][q] = p * (dpt - Er[q]);
            vddp[jb][ib][q] = p * (fv - Ar[q]);
          }
      }
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) {
        dstB[jb] = E::from_f32(vdst[jb][0], vdst[jb][1]);
        dsB[jb] = E::from_f32(vds[jb][0], vds[jb][1]);
        ddpB[jb] = E::from_f32(vddp[jb][0], vddp[jb][1]);
      }
      // ---- contractions over the stage's 32 rows (transposed outputs) ----
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const F qt = lds_frag_tr<T, D>(Qt, 0, 16 * db, r, g);
        const F uqt = lds_frag_tr<T, D>(UQt, 0, 16 * db, r, g);
        const F dot = lds_frag_tr<T, D>(dOt, 0, 16 * db, r, g);
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
          accK[jb][db] = E::mma(qt, dstB[jb], accK[jb][db]);
          accK[jb][db] = E::mma(uqt, dsB[jb], accK[jb][db]);
          accV[jb][db] = E::mma(dot, ddpB[jb], accV[jb][db]);
        }
      }
    }
    if (more) store_step(lds[(t + 1) & 1]);
    __syncthreads();
  }

  // ---- single exclusive write of dK~ and dV~ ----
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int j = jw0 + 16 * jb + r;
    if (j < N) {
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

template <typename T, int D, int NJ>
hipError_t launch_t(const Problem& p, const Pass2Args& a, hipStream_t s) {
  constexpr int kBCw = 4 * 16 * NJ;
  const int n_col_tiles = (p.N + kBCw - 1) / kBCw;
  const int total = n_col_tiles * p.B * p.Hkv;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((pass2_kernel<T, D, NJ, true>), dim3(total), dim3(kThreads), 0, s, a, p.Hkv,
                       group, p.N, p.tau, n_col_tiles, total);
  else
    hipLaunchKernelGGL((pass2_kernel<T, D, NJ, false>), dim3(total), dim3(kThreads), 0, s, a,
                       p.Hkv, group, p.N, p.tau, n_col_tiles, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pass2(const Problem& p, const Pass2Args& a, hipStream_t s) {
  if (p.bf16) {
    if (p.d == 64) return launch_t<__bf16, 64, 2>(p, a, s);
    return launch_t<__bf16, 128, 1>(p, a, s);
  }
  if (p.d == 64) return launch_t<float, 64, 1>(p, a, s);
  return launch_t<float, 128, 1>(p, a, s);
}

}  // namespace fbob
