// fbob_pass1.hip - BoB Pass 1 (row-resident).
//
// FlashBoB notes, "关键设计" item 2 (first pass) with the affine decomposition of
// item 1.  For each query row i it streams every key tile j and accumulates
//   alpha_i  = sum_j P_ij F_ij                       F = tau (U_Q K^T + Q U_K^T)
//   E'_i     = sum_j P_ij dP~'_ij                    dP~' = F o (dP - D) + G, G = dO U_V^T
//   B_i      = sum_j P_ij K_j
//   R_i      = sum_j P_ij dP_ij K_j                  dP = dO V^T
//   Omega_i  = sum_j P_ij dP~'_ij K_j + dS_ij U_K,j  dS = P o (dP - D)
//   ddO~'_i  = sum_j P_ij F_ij V_j + P_ij U_V,j
// with P = exp(tau Q K^T - L) rebuilt from the stored log-partition L, then
// applies the row correction once:
//   E = E' - alpha D,  ddO~ = ddO~' - alpha O,  dQ~ = tau (Omega - alpha R - E B)
// and writes dQ~, ddO~, alpha and E exactly once per row.
//
// Schedule: one work-group = 4 waves; each wave owns 16*NI query rows whose Q,
// dO, U_Q operand fragments and four fp32 accumulators stay in registers for the
// whole sweep.  K, V, U_K, U_V tiles of 32 keys are staged through LDS
// (double-buffered, one barrier per tile).  The five score-shaped tiles are
// computed transposed (key index on the MFMA row axis), so each lane holds one
// query row: alpha and E' are per-lane partial sums reduced across the four lane
// groups once at the end, and the P-shaped tiles are directly the B operand of
// the output contractions, whose A operand (K^T, V^T, ...) comes from transposed
// LDS reads.  The outputs are accumulated transposed (d on the row axis), so the
// row corrections are lane-local.
#include "fbob_device.hpp"
#include "fbob_launch.hpp"

namespace fbob {
namespace {

constexpr int kThreads = 256;
constexpr int kBC = 32;

template <typename T, int D, int NI, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void pass1_kernel(Pass1Args a, int Hq, int group, int N,
                                                         float tau, int n_row_tiles, int total) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int kRowsW = 16 * NI;
  constexpr int kBR = 4 * kRowsW;
  constexpr int kTB = kBC * Tile<T, D>::kRowBytes;
  constexpr int kDC = D / 32;
  constexpr int kDB = D / 16;
  __shared__ __attribute__((aligned(16))) char lds[2][4 * kTB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int logical = xcd_remap(blockIdx.x, total);
  const int bh = logical / n_row_tiles, rt = logical % n_row_tiles;
  const int b = bh / Hq, h = bh % Hq, hk = h / group;
  const int64_t q_off = (int64_t)bh * N * D;
  const int64_t kv_off = ((int64_t)b * (Hq / group) + hk) * N * D;
  const T* Qh = reinterpret_cast<const T*>(a.Q) + q_off;
  const T* dOh = reinterpret_cast<const T*>(a.dO) + q_off;
  const T* UQh = reinterpret_cast<const T*>(a.UQ) + q_off;
  const T* Kh = reinterpret_cast<const T*>(a.K) + kv_off;
  const T* Vh = reinterpret_cast<const T*>(a.V) + kv_off;
  const T* UKh = reinterpret_cast<const T*>(a.UK) + kv_off;
  const T* UVh = reinterpret_cast<const T*>(a.UV) + kv_off;

  const int iw0 = rt * kBR + w * kRowsW;
  F qf[NI][kDC], dof[NI][kDC], uqf[NI][kDC];
  float l2[NI], dv[NI];
#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
    const int i = iw0 + 16 * ib + r;
#pragma unroll
    for (int dc = 0; dc < kDC; ++dc) {
      qf[ib][dc] = global_frag(Qh, i, N, D, 32 * dc + 8 * g);
      dof[ib][dc] = global_frag(dOh, i, N, D, 32 * dc + 8 * g);
      uqf[ib][dc] = global_frag(UQh, i, N, D, 32 * dc + 8 * g);
    }
    l2[ib] = i < N ? a.L[(int64_t)bh * N + i] * kLog2e : 0.f;
    dv[ib] = i < N ? a.D[(int64_t)bh * N + i] : 0.f;
  }

  f32x4 accB[NI][kDB], accR[NI][kDB], accW[NI][kDB], accO[NI][kDB];
  float alp[NI], edg[NI];
#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
    alp[ib] = 0.f;
    edg[ib] = 0.f;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      accB[ib][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      accR[ib][db] = accB[ib][db];
      accW[ib][db] = accB[ib][db];
      accO[ib][db] = accB[ib][db];
    }
  }
  const float c1 = tau * kLog2e;

  int jend = N;
  if (CAUSAL) jend = min(N, rt * kBR + kBR);
  const int ntc = (jend + kBC - 1) / kBC;

  Stager<T, D, kBC, kThreads> sk, sv, suk, suv;
  sk.load(Kh, 0, N, tid);
  sv.load(Vh, 0, N, tid);
  suk.load(UKh, 0, N, tid);
  suv.load(UVh, 0, N, tid);
  sk.store(lds[0], tid);
  sv.store(lds[0] + kTB, tid);
  suk.store(lds[0] + 2 * kTB, tid);
  suv.store(lds[0] + 3 * kTB, tid);
  __syncthreads();

  for (int t = 0; t < ntc; ++t) {
    const int j0 = t * kBC;
    const bool more = t + 1 < ntc;
    if (more) {
      sk.load(Kh, j0 + kBC, N, tid);
      sv.load(Vh, j0 + kBC, N, tid);
      suk.load(UKh, j0 + kBC, N, tid);
      suv.load(UVh, j0 + kBC, N, tid);
    }
    const char* Kt = lds[t & 1];
    const char* Vt = Kt + kTB;
    const char* UKt = Kt + 2 * kTB;
    const char* UVt = Kt + 3 * kTB;
    const bool active = !CAUSAL || j0 <= iw0 + kRowsW - 1;
    if (active) {
      // ---- score-shaped tiles, transposed: [key block jb][row block ib] ----
      f32x4 s[2][NI], dp[2][NI], f[2][NI], gg[2][NI];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) {
          s[jb][ib] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[jb][ib] = s[jb][ib];
          f[jb][ib] = s[jb][ib];
          gg[jb][ib] = s[jb][ib];
        }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc) {
          const int row = 16 * jb + r, col = 32 * dc + 8 * g;
          const F kf = lds_frag_row<T, D>(Kt, row, col);
          const F vf = lds_frag_row<T, D>(Vt, row, col);
          const F ukf = lds_frag_row<T, D>(UKt, row, col);
          const F uvf = lds_frag_row<T, D>(UVt, row, col);
#pragma unroll
          for (int ib = 0; ib < NI; ++ib) {
            s[jb][ib] = E::mma(kf, qf[ib][dc], s[jb][ib]);
            f[jb][ib] = E::mma(kf, uqf[ib][dc], f[jb][ib]);
            f[jb][ib] = E::mma(ukf, qf[ib][dc], f[jb][ib]);
            dp[jb][ib] = E::mma(vf, dof[ib][dc], dp[jb][ib]);
            gg[jb][ib] = E::mma(uvf, dof[ib][dc], gg[jb][ib]);
          }
        }
      // ---- elementwise: P, dS, P o F, P o dP~', P o dP; row partial sums ----
      const bool edge = (j0 + kBC > N) || (CAUSAL && j0 + kBC - 1 > iw0);
      F pB[NI], pdpB[NI], pdtB[NI], dsB[NI], pfB[NI];
#pragma unroll
      for (int ib = 0; ib < NI; ++ib) {
        const int i = iw0 + 16 * ib + r;
        f32x4 vp[2], vpdp[2], vpdt[2], vds[2], vpf[2];
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float p = fast_exp2(s[jb][ib][q] * c1 - l2[ib]);
            if (edge) {
              const int j = j0 + 16 * jb + 4 * g + q;
              if (j >= N || (CAUSAL && j > i)) p = 0.f;
            }
            const float dpv = dp[jb][ib][q];
            const float tv = dpv - dv[ib];
            const float fv = f[jb][ib][q] * tau;
            const float dpt = fv * tv + gg[jb][ib][q];
            const float pf = p * fv;
            const float pdt = p * dpt;
            alp[ib] += pf;
            edg[ib] += pdt;
            vp[jb][q] = p;
            vpdp[jb][q] = p * dpv;
            vpdt[jb][q] = pdt;
            vds[jb][q] = p * tv;
            vpf[jb][q] = pf;
          }
        pB[ib] = E::from_f32(vp[0], vp[1]);
        pdpB[ib] = E::from_f32(vpdp[0], vpdp[1]);
        pdtB[ib] = E::from_f32(vpdt[0], vpdt[1]);
        dsB[ib] = E::from_f32(vds[0], vds[1]);
        pfB[ib] = E::from_f32(vpf[0], vpf[1]);
      }
      // ---- output contractions over the tile's 32 keys (transposed outputs) ----
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const F kt = lds_frag_tr<T, D>(Kt, 0, 16 * db, r, g);
        const F ukt = lds_frag_tr<T, D>(UKt, 0, 16 * db, r, g);
        const F vt = lds_frag_tr<T, D>(Vt, 0, 16 * db, r, g);
        const F uvt = lds_frag_tr<T, D>(UVt, 0, 16 * db, r, g);
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) {
          accB[ib][db] = E::mma(kt, pB[ib], accB[ib][db]);
          accR[ib][db] = E::mma(kt, pdpB[ib], accR[ib][db]);
          accW[ib][db] = E::mma(kt, pdtB[ib], accW[ib][db]);
          accW[ib][db] = E::mma(ukt, dsB[ib], accW[ib][db]);
          accO[ib][db] = E::mma(vt, pfB[ib], accO[ib][db]);
          accO[ib][db] = E::mma(uvt, pB[ib], accO[ib][db]);
        }
      }
    }
    if (more) {
      char* nb = lds[(t + 1) & 1];
      sk.store(nb, tid);
      sv.store(nb + kTB, tid);
      suk.store(nb + 2 * kTB, tid);
      suv.store(nb + 3 * kTB, tid);
    }
    __syncthreads();
  }

  // ---- affine row correction and the single write of each row output ----
#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
    const int i = iw0 + 16 * ib + r;
    const float al = group_sum(alp[ib]);
    const float ev = group_sum(edg[ib]) - al * dv[ib];
    if (i < N) {
      const int64_t ro = q_off + (int64_t)i * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int d0 = 16 * db + 4 * g;
        const f32x4 o = *reinterpret_cast<const f32x4*>(a.O + ro + d0);
        const f32x4 ddo = accO[ib][db] - al * o;
        const f32x4 dq = tau * (accW[ib][db] - al * accR[ib][db] - ev * accB[ib][db]);
        *reinterpret_cast<f32x4*>(a.ddOt + ro + d0) = ddo;
        *reinterpret_cast<f32x4*>(a.dQt + ro + d0) = dq;
      }
      if (g == 0) {
        a.alpha[(int64_t)bh * N + i] = al;
        a.E[(int64_t)bh * N + i] = ev;
      }
    }
  }
}

template <typename T, int D, int NI>
hipError_t launch_t(const Problem& p, const Pass1Args& a, hipStream_t s) {
  constexpr int kBR = 4 * 16 * NI;
  const int n_row_tiles = (p.N + kBR - 1) / kBR;
  const int total = n_row_tiles * p.B * p.Hq;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((pass1_kernel<T, D, NI, true>), dim3(total), dim3(kThreads), 0, s, a, p.Hq,
                       group, p.N, p.tau, n_row_tiles, total);
  else
    hipLaunchKernelGGL((pass1_kernel<T, D, NI, false>), dim3(total), dim3(kThreads), 0, s, a, p.Hq,
                       group, p.N, p.tau, n_row_tiles, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pass1(const Problem& p, const Pass1Args& a, hipStream_t s) {
  if (p.bf16) {
    if (p.d == 64) return launch_t<__bf16, 64, 2>(p, a, s);
    return launch_t<__bf16, 128, 1>(p, a, s);
  }
  if (p.d == 64) return launch_t<float, 64, 1>(p, a, s);
  return launch_t<float, 128, 1>(p, a, s);
}

}  // namespace fbob
