// fbob_forward.hip - forward pass with the row state BoB recomputes from.
//
// Computes, per query head, O = softmax_row(tau Q K^T) V, the natural-log
// log-sum-exp L of each scaled score row and D_i = dO_i . O_i from the fp32 O.
// FlashAttention blog ("FlashAttention 的反向传播设计"), sections 一 and 二: the
// forward keeps only per-row statistics; FlashBoB notes, "关键设计" 1: D_i.
//
// Schedule: one work-group = 4 waves, each wave owns 16*NI query rows that stay
// in registers (Q as MFMA operand, O as fp32 accumulator).  K and V column tiles
// of 32 keys are staged through LDS, double-buffered.  Scores are computed
// transposed (S^T = K Q^T), so a lane owns one query row and 8 keys of the tile;
// the row maximum needs one cross-group reduction per tile, the row sum is kept
// per lane and reduced once at the end (online softmax with exp2).
#include "fbob_device.hpp"
#include "fbob_launch.hpp"

namespace fbob {
namespace {

constexpr int kThreads = 256;
constexpr int kBC = 32;  // keys per LDS stage

template <typename T, int D, int NI, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdArgs a, int Hq, int group, int N,
                                                       float tau, int n_row_tiles, int total) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int kRowsW = 16 * NI;
  constexpr int kBR = 4 * kRowsW;
  constexpr int kTB = kBC * Tile<T, D>::kRowBytes;  // bytes per staged tile
  constexpr int kDC = D / 32;                        // 32-wide d chunks
  constexpr int kDB = D / 16;                        // 16-wide d blocks
  __shared__ __attribute__((aligned(16))) char lds[2][2 * kTB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int logical = xcd_remap(blockIdx.x, total);
  const int bh = logical / n_row_tiles, rt = logical % n_row_tiles;
  const int b = bh / Hq, h = bh % Hq, hk = h / group;
  const int64_t q_off = (int64_t)bh * N * D;
  const int64_t kv_off = ((int64_t)b * (Hq / group) + hk) * N * D;
  const T* Qh = reinterpret_cast<const T*>(a.Q) + q_off;
  const T* Kh = reinterpret_cast<const T*>(a.K) + kv_off;
  const T* Vh = reinterpret_cast<const T*>(a.V) + kv_off;
  const T* dOh = reinterpret_cast<const T*>(a.dO) + q_off;

  const int iw0 = rt * kBR + w * kRowsW;
  F qf[NI][kDC];
#pragma unroll
  for (int ib = 0; ib < NI; ++ib)
#pragma unroll
    for (int dc = 0; dc < kDC; ++dc) qf[ib][dc] = global_frag(Qh, iw0 + 16 * ib + r, N, D, 32 * dc + 8 * g);

  f32x4 acc[NI][kDB];
  float m[NI], l[NI];
#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
    m[ib] = -INFINITY;
    l[ib] = 0.f;
#pragma unroll
    for (int db = 0; db < kDB; ++db) acc[ib][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c1 = tau * kLog2e;

  int jend = N;
  if (CAUSAL) jend = min(N, rt * kBR + kBR);
  const int ntc = (jend + kBC - 1) / kBC;

  Stager<T, D, kBC, kThreads> sk, sv;
  sk.load(Kh, 0, N, tid);
  sv.load(Vh, 0, N, tid);
  sk.store(lds[0], tid);
  sv.store(lds[0] + kTB, tid);
  __syncthreads();

  for (int t = 0; t < ntc; ++t) {
    const int j0 = t * kBC;
    const bool more = t + 1 < ntc;
    if (more) {
      sk.load(Kh, j0 + kBC, N, tid);
      sv.load(Vh, j0 + kBC, N, tid);
    }
    const char* Kt = lds[t & 1];
    const char* Vt = Kt + kTB;
    const bool active = !CAUSAL || j0 <= iw0 + kRowsW - 1;
    if (active) {
      f32x4 s[2][NI];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) s[jb][ib] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc) {
          const F kf = lds_frag_row<T, D>(Kt, 16 * jb + r, 32 * dc + 8 * g);
#pragma unroll
          for (int ib = 0; ib < NI; ++ib) s[jb][ib] = E::mma(kf, qf[ib][dc], s[jb][ib]);
        }
      const bool edge = (j0 + kBC > N) || (CAUSAL && j0 + kBC - 1 > iw0);
      F pf[NI];
#pragma unroll
      for (int ib = 0; ib < NI; ++ib) {
        const int i = iw0 + 16 * ib + r;
        float mt = -INFINITY;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float x = s[jb][ib][q] * c1;
            if (edge) {
              const int j = j0 + 16 * jb + 4 * g + q;
              if (j >= N || (CAUSAL && j > i)) x = -INFINITY;
            }
            s[jb][ib][q] = x;
            mt = fmaxf(mt, x);
          }
        mt = group_max(mt);
        const float mn = fmaxf(m[ib], mt);
        const float sc = fast_exp2(m[ib] - mn);
        m[ib] = mn;
        float ls = 0.f;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float p = fast_exp2(s[jb][ib][q] - mn);
            s[jb][ib][q] = p;
            ls += p;
          }
        l[ib] = l[ib] * sc + ls;
#pragma unroll
        for (int db = 0; db < kDB; ++db) acc[ib][db] *= sc;
        pf[ib] = E::from_f32(s[0][ib], s[1][ib]);
      }
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const F vt = lds_frag_tr<T, D>(Vt, 0, 16 * db, r, g);
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) acc[ib][db] = E::mma(vt, pf[ib], acc[ib][db]);
      }
    }
    if (more) {
      sk.store(lds[(t + 1) & 1], tid);
      sv.store(lds[(t + 1) & 1] + kTB, tid);
    }
    __syncthreads();
  }

  // Epilogue: O = acc / l, L = ln(sum) + max, D = dO . O (fp32 O).
#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
    const int i = iw0 + 16 * ib + r;
    const float lsum = group_sum(l[ib]);
    const float inv = 1.f / lsum;
    float dpart = 0.f;
    if (i < N) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int d0 = 16 * db + 4 * g;
        const f32x4 o = acc[ib][db] * inv;
        *reinterpret_cast<f32x4*>(a.O + q_off + (int64_t)i * D + d0) = o;
#pragma unroll
        for (int q = 0; q < 4; ++q) dpart += (float)dOh[(int64_t)i * D + d0 + q] * o[q];
      }
    }
    const float dsum = group_sum(dpart);
    if (i < N && g == 0) {
      a.L[(int64_t)bh * N + i] = (m[ib] + __log2f(lsum)) * kLn2;
      a.D[(int64_t)bh * N + i] = dsum;
    }
  }
}

template <typename T, int D, int NI>
hipError_t launch_t(const Problem& p, const FwdArgs& a, hipStream_t s) {
  constexpr int kBR = 4 * 16 * NI;
  const int n_row_tiles = (p.N + kBR - 1) / kBR;
  const int total = n_row_tiles * p.B * p.Hq;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((fwd_kernel<T, D, NI, true>), dim3(total), dim3(kThreads), 0, s, a, p.Hq,
                       group, p.N, p.tau, n_row_tiles, total);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, NI, false>), dim3(total), dim3(kThreads), 0, s, a, p.Hq,
                       group, p.N, p.tau, n_row_tiles, total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const Problem& p, const FwdArgs& a, hipStream_t s) {
  if (p.bf16) {
    if (p.d == 64) return launch_t<__bf16, 64, 2>(p, a, s);
    return launch_t<__bf16, 128, 2>(p, a, s);
  }
  if (p.d == 64) return launch_t<float, 64, 1>(p, a, s);
  return launch_t<float, 128, 1>(p, a, s);
}

}  // namespace fbob
