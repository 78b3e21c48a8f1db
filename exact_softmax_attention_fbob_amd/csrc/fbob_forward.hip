// fbob_forward.hip - forward pass with the row state BoB recomputes from.
//
// Computes, per query head, O = softmax_row(tau Q K^T) V, the natural-log
// log-sum-exp L of each scaled score row and D_i = dO_i . O_i from the fp32 O.
// FlashAttention blog ("FlashAttention 的反向传播设计"), sections 一 and 二: the
// forward keeps only per-row statistics; FlashBoB notes, "关键设计" 1: D_i.
//
// Schedule: one work-group = NW waves, each wave owns 16 NI query rows (Q as MFMA
// operand, O as fp32 accumulator in registers); every K and V fragment read from
// LDS serves the NI row blocks of the wave.  K and V tiles of BC keys are
// staged straight into LDS (double-buffered).  Scores are computed transposed
// (S^T = K Q^T), so a lane owns one query row and 8 keys per 32-key block.
// Online softmax in base 2 with a lazy running maximum: the weights are
// exp2(x - m) for a per-row reference m that is raised only when a row's new
// maximum exceeds it by more than kSlack (weights then stay <= 2^kSlack), so the
// accumulator rescale is rare.  The row sum of the weights is an MFMA contraction
// with a ones operand over the same bf16 weights that multiply V.

#include <algorithm>
#include <type_traits>

#include "fbob_device.hpp"
#include "fbob_launch.hpp"

namespace fbob {
namespace {

constexpr float kSlack = 8.0f;  // log2 headroom before the reference max is raised

// PRIO: raise the wave priority while the P V contraction MFMAs issue.
// NI: 16-row blocks per wave.
// Waves per SIMD the compiler must allow: the bf16 d = 64 kernel with tau not a power of
// two (tau applied in the exp2 argument) left alone takes 130 registers, i.e. three waves
// per SIMD and one eight-wave work-group per CU; held to four it fits 126 with no spill
// (8 % faster).
template <typename T, int D, int NW, int BC, bool TP2, bool CAUSAL>
constexpr int fwd_waves_per_simd() {
  return D < 128 && sizeof(T) == 2 && !TP2 ? 4 : 1;
}

template <typename T, int D, int NW, int BC, bool TP2, bool CAUSAL, bool PRIO = false, int NI = 1,
          bool SPLIT = false>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_simd<T, D, NW, BC, TP2, CAUSAL>()))) void fwd_kernel(FwdArgs a, int Hq, int group, int N,
                                                      float tau, int n_row_tiles, int total) {
  using E = Elem<T>;
  using F = typename E::frag;
  constexpr int kRW = 16 * NI;                     // query rows per wave
  constexpr int kBR = NW * kRW;
  constexpr int kTB = BC * Tile<T, D>::kRowBytes;  // bytes per staged tile
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
  // Causal rows near the end see the most keys: dispatch them first so the
  // shortest tiles fill the tail of the grid.
  const int rt = CAUSAL ? n_row_tiles - 1 - lt % n_row_tiles : lt % n_row_tiles;
  const int b = bh / Hq, h = bh % Hq, hk = h / group;
  const int64_t q_off = (int64_t)bh * N * D;
  const int64_t kv_off = ((int64_t)b * (Hq / group) + hk) * N * D;
  const T* Qh = reinterpret_cast<const T*>(a.Q) + q_off;
  const T* const kv_bases[2] = {reinterpret_cast<const T*>(a.K) + kv_off,
                                reinterpret_cast<const T*>(a.V) + kv_off};

  const int iw0 = rt * kBR + w * kRW;
  // this lane's query row in row block ib: iw0 + 16 ib + r
  // With TP2 (tau an exact power of two) the score operand is tau Q (exact).
  F qf[NI][kDC];
#pragma unroll
  for (int ib = 0; ib < NI; ++ib)
#pragma unroll
    for (int dc = 0; dc < kDC; ++dc) {
      const F q0 = global_frag(Qh, iw0 + 16 * ib + r, N, D, 32 * dc + 8 * g);
      qf[ib][dc] = TP2 ? scale_frag<T>(q0, tau) : q0;
    }
  const float c1 = TP2 ? kLog2e : tau * kLog2e;
  const F ones = ones_frag<T>();

  f32x4 acc[NI][kDB], accL[NI];  // accL: row sum of the weights (every q holds it)
  float m[NI];                   // reference maximum of this lane's row (log2 units)
  float thr[NI];                 // (m + kSlack) / c1: the raw score that forces a rescale
#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
#pragma unroll
    for (int db = 0; db < kDB; ++db) acc[ib][db] = splat4(0.f);
    accL[ib] = splat4(0.f);
    // A part may hold no key of a row (causal, keys past its diagonal): a finite floor
    // keeps its weights exp2(-inf - m) at 0 instead of NaN, and the first valid key of
    // the row still raises the reference (the unsplit sweep always starts at key 0).
    m[ib] = SPLIT ? -1.0e30f : -INFINITY;
    thr[ib] = -INFINITY;
  }
  const LdsLane<T, D> rd(r, g);

  int jend = N;
  if (CAUSAL) jend = min(N, rt * kBR + kBR);
  const int ntc = (jend + BC - 1) / BC;
  // this work-group's key stages [t_lo, t_hi): all of them, or its part's share
  int t_lo = 0, t_hi = ntc;
  if constexpr (SPLIT) {
    const int per = (ntc + a.nsplit - 1) / a.nsplit;
    t_lo = min(ntc, split * per);
    t_hi = min(ntc, t_lo + per);
  }

  // 32 keys of a staged tile.
  auto block32 = [&](const char* Kt, const char* Vt, int j0) {
    const bool edge = (j0 + 32 > N) || (CAUSAL && j0 + 31 > iw0);
    // Raw scores; the row maximum is taken before scaling (c1 > 0 commutes with
    // max), so each weight costs one FMA and one exp2.
    f32x4 s[NI][2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
      for (int ib = 0; ib < NI; ++ib) s[ib][jb] = splat4(0.f);
#pragma unroll
      for (int dc = 0; dc < kDC; ++dc) {
        const F kf = rd.row(Kt, jb, dc);
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) s[ib][jb] = E::mma(kf, qf[ib][dc], s[ib][jb]);
      }
      if (edge) {
#pragma unroll
        for (int ib = 0; ib < NI; ++ib)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = j0 + 16 * jb + 4 * g + q;
            if (j >= N || (CAUSAL && j > iw0 + 16 * ib + r)) s[ib][jb][q] = -INFINITY;
          }
      }
    }
    // This lane's maximum over its 8 keys of the block; m is shared by the four
    // lanes of a row, so a lane above m + kSlack is enough to trigger the rescale,
    // and the row maximum across lanes is only formed when it happens.
    // (raw scores: c1 > 0, so the test against thr = (m + kSlack) / c1 needs no
    // scaling; every row's first block holds a valid key, so m is finite after it)
    float ml[NI];
    bool raise = false;
#pragma unroll
    for (int ib = 0; ib < NI; ++ib) {
      ml[ib] = max8(s[ib][0], s[ib][1]);
      raise |= ml[ib] > thr[ib];
    }
    // Raise the reference only when the new maximum would push a weight above
    // 2^kSlack (always on the first block, where m = -inf).  Every row block of the
    // wave is brought up to its current maximum then (never lowered).
    if (__any(raise)) {
#pragma unroll
      for (int ib = 0; ib < NI; ++ib) {
        const float mn = fmaxf(m[ib], group_max(ml[ib]) * c1);
        const float sc = fast_exp2(m[ib] - mn);
#pragma unroll
        for (int db = 0; db < kDB; ++db) acc[ib][db] *= sc;
        accL[ib] *= sc;
        m[ib] = mn;
        thr[ib] = (mn + kSlack) / c1;
      }
    }
    F pB[NI];
#pragma unroll
    for (int ib = 0; ib < NI; ++ib) {
      const float nm = -m[ib];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          pB[ib][4 * jb + q] = (T)fast_exp2(__builtin_fmaf(s[ib][jb][q], c1, nm));
    }
    if constexpr (PRIO) FBOB_PRIO_HIGH();
#pragma unroll
    for (int ib = 0; ib < NI; ++ib) accL[ib] = E::mma(ones, pB[ib], accL[ib]);
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const F vt = rd.tr(Vt, db);
#pragma unroll
      for (int ib = 0; ib < NI; ++ib) acc[ib][db] = E::mma(vt, pB[ib], acc[ib][db]);
    }
    if constexpr (PRIO) FBOB_PRIO_LOW();
  };

  DirectStager<T, D, BC, 2, NW> st;
  st.init(kv_bases, w, lane);
  if (!SPLIT || t_lo < t_hi) st.load(lds[0], t_lo * BC, N);  // (an empty part stages nothing)
  wait_all_memory();
  __syncthreads();

  // Causal: a 32-key block past the wave's last row is masked whole.  Skipping it
  // saves little (the stage barrier waits for the wave with the most keys anyway),
  // and at d = 64 the branch around the block costs 44 registers, i.e. half the
  // occupancy (one work-group per CU instead of two), so there it is computed and
  // masked (its weights are exactly 0).
  constexpr bool kSkipMasked = CAUSAL && !(D < 128 && std::is_same<T, __bf16>::value);
  auto step = [&](int t, char* cur, char* nxt) {
    const int j0 = t * BC;
    const bool more = t + 1 < t_hi;
    if (more) st.load(nxt, j0 + BC, N);
#pragma unroll
    for (int hs = 0; hs < BC / 32; ++hs) {
      const int js = j0 + 32 * hs;
      if (!kSkipMasked || js <= iw0 + kRW - 1)
        block32(cur + 32 * hs * Tile<T, D>::kRowBytes,
                cur + kTB + 32 * hs * Tile<T, D>::kRowBytes, js);
    }
    if (more) wait_all_memory();
    __syncthreads();
  };
#pragma unroll 1
  for (int t = t_lo; t < t_hi; t += 2) {
    step(t, lds[0], lds[1]);
    if (t + 1 < t_hi) step(t + 1, lds[1], lds[0]);
  }

  if constexpr (SPLIT) {
    // this part's unnormalised O, its row sum and reference maximum (log2 units); the
    // reduction rescales the parts to their common maximum
    const int64_t heads = (int64_t)gridDim.x / ((int64_t)n_row_tiles * a.nsplit);
#pragma unroll
    for (int ib = 0; ib < NI; ++ib) {
      const int i = iw0 + 16 * ib + r;
      if (i < N) {
        const int64_t prow = ((int64_t)split * heads + bh) * N + i;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
          *reinterpret_cast<f32x4*>(a.part + prow * D + 16 * db + 4 * g) = acc[ib][db];
        if (g == 0) {
          a.part_ml[2 * prow] = m[ib];
          a.part_ml[2 * prow + 1] = accL[ib][0];
        }
      }
    }
    return;
  }

  // Epilogue: O = acc / l, L = (m + log2 l) ln 2, and D = dO . O (fp32 O) when
  // dO is given (a uniform branch).
  const bool with_d = a.dO != nullptr;
#pragma unroll
  for (int ib = 0; ib < NI; ++ib) {
    const int i = iw0 + 16 * ib + r;
    const float lsum = accL[ib][0];
    const float inv = 1.f / lsum;
    float dpart = 0.f;
    if (i < N) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const int d0 = 16 * db + 4 * g;
        const f32x4 o = acc[ib][db] * inv;
        *reinterpret_cast<f32x4*>(a.O + q_off + (int64_t)i * D + d0) = o;
        if (with_d) {
          const T* dOh = reinterpret_cast<const T*>(a.dO) + q_off;
#pragma unroll
          for (int q = 0; q < 4; ++q) dpart += (float)dOh[(int64_t)i * D + d0 + q] * o[q];
        }
      }
    }
    const float dsum = group_sum(dpart);
    if (i < N && g == 0) {
      a.L[(int64_t)bh * N + i] = (m[ib] + __log2f(lsum)) * kLn2;
      if (with_d) a.D[(int64_t)bh * N + i] = dsum;
    }
  }
}

template <typename T, int D, int NW, int BC, bool TP2, bool PRIO = false, int NI = 1>
hipError_t launch_t(const Problem& p, const FwdArgs& a, hipStream_t s) {
  constexpr int kBR = NW * 16 * NI;
  const int n_row_tiles = (p.N + kBR - 1) / kBR;
  const int total = n_row_tiles * p.B * p.Hq;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, BC, TP2, true, PRIO, NI>), dim3(total), dim3(NW * 64), 0, s, a,
                       p.Hq, group, p.N, p.tau, n_row_tiles, total);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, BC, TP2, false, PRIO, NI>), dim3(total), dim3(NW * 64), 0, s, a,
                       p.Hq, group, p.N, p.tau, n_row_tiles, total);
  return hipGetLastError();
}

template <typename T, int D, int NW, int BC, bool TP2, bool PRIO, int NI>
hipError_t launch_split_t(const Problem& p, const FwdArgs& a, hipStream_t s) {
  constexpr int kBR = NW * 16 * NI;
  const int n_row_tiles = (p.N + kBR - 1) / kBR;
  const int total = n_row_tiles * p.B * p.Hq * a.nsplit;
  const int group = p.Hq / p.Hkv;
  if (p.causal)
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, BC, TP2, true, PRIO, NI, true>), dim3(total),
                       dim3(NW * 64), 0, s, a, p.Hq, group, p.N, p.tau, n_row_tiles, total);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, BC, TP2, false, PRIO, NI, true>), dim3(total),
                       dim3(NW * 64), 0, s, a, p.Hq, group, p.N, p.tau, n_row_tiles, total);
  return hipGetLastError();
}

}  // namespace

// The shipped bf16 layouts of launch_forward below, in split form (bf16 only).
hipError_t launch_forward_split(const Problem& p, const FwdArgs& a, hipStream_t s) {
  if (p.d == 64) {
    if (tau_is_pow2(p.tau)) return launch_split_t<__bf16, 64, 8, 128, true, true, 2>(p, a, s);
    return launch_split_t<__bf16, 64, 8, 128, false, false, 2>(p, a, s);
  }
  return launch_split_t<__bf16, 128, 8, 64, false, false, 2>(p, a, s);
}

hipError_t launch_forward(const Problem& p, const FwdArgs& a, hipStream_t s) {
  if (p.bf16) {
    // bf16 defaults: 32 query rows per wave (each K / V fragment read from LDS
    // serves two row blocks), measured ~12 % faster than 16 at d = 64 and ~7 % at
    // d = 128.
    if (p.d == 64) {
      if (tau_is_pow2(p.tau)) {
        // 128-key stages and raised wave priority over the P V MFMAs; 1 selects 16
        // rows per wave, 2 64-key stages, 3 the plain instruction order.
#if FBOB_TUNING
        const int cfg = tune_choice("FBOB_TUNE_FWD");
        if (cfg == 1) return launch_t<__bf16, 64, 8, 64, true, true, 1>(p, a, s);
        if (cfg == 2) return launch_t<__bf16, 64, 8, 64, true, true, 2>(p, a, s);
        if (cfg == 3) return launch_t<__bf16, 64, 8, 128, true, false, 2>(p, a, s);
#endif
        return launch_t<__bf16, 64, 8, 128, true, true, 2>(p, a, s);
      }
      return launch_t<__bf16, 64, 8, 128, false, false, 2>(p, a, s);
    }
    // d = 128: 64-key stages; 1 and 2 select 16 rows per wave with 32-key stages
    // and 8 or 4 waves per work-group, 3 16 rows per wave with 64-key stages, 4
    // raised priority over the P V MFMAs, 5 128-key stages.
#if FBOB_TUNING
    const int cfg = tune_choice("FBOB_TUNE_FWD_D128");
    if (cfg == 1) return launch_t<__bf16, 128, 8, 32, false>(p, a, s);
    if (cfg == 2) return launch_t<__bf16, 128, 4, 32, false>(p, a, s);
    if (cfg == 3) return launch_t<__bf16, 128, 8, 64, false>(p, a, s);
    if (cfg == 4) return launch_t<__bf16, 128, 8, 64, false, true, 2>(p, a, s);
    if (cfg == 5) return launch_t<__bf16, 128, 8, 128, false, false, 2>(p, a, s);
#endif
    return launch_t<__bf16, 128, 8, 64, false, false, 2>(p, a, s);
  }
  if (p.d == 64) return launch_t<float, 64, 4, 32, false>(p, a, s);
  return launch_t<float, 128, 4, 32, false>(p, a, s);
}

namespace {

// Merge of the split forward: each part holds, per row, an unnormalised O_s, its
// row sum l_s and reference maximum m_s (log2 units).  With M = max_s m_s the row's
// sum is l = sum_s l_s 2^(m_s - M) and O = sum_s O_s 2^(m_s - M) / l, L = (M + log2 l)
// ln 2 -- the merge of online-softmax partial states (FlashAttention blog, section 一:
// the softmax of a concatenation from the blocks' maxima and sums).  D / 4 lanes per
// row, 4 columns each; D_i = dO_i . O_i is summed over the row's lanes.  NS parts as a
// template argument: every part's loads issue together (one memory round trip for the
// row states, one for the O parts).
template <int D, int NS>
__global__ __launch_bounds__(256) void fwd_reduce_kernel(FwdArgs a, int64_t rows) {
  constexpr int kLanes = D / 4;
  const int64_t row = (int64_t)blockIdx.x * (256 / kLanes) + threadIdx.x / kLanes;
  const int c = (threadIdx.x % kLanes) * 4;
  const bool ok = row < rows;
  f32x4 o = splat4(0.f);
  float M = -INFINITY, l = 0.f;
  if (ok) {
    float2 ml[NS];
    f32x4 op[NS];
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      const int64_t pr = sp * rows + row;
      ml[sp] = *reinterpret_cast<const float2*>(a.part_ml + 2 * pr);
      op[sp] = *reinterpret_cast<const f32x4*>(a.part + pr * D + c);
    }
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) M = fmaxf(M, ml[sp].x);
#pragma unroll
    for (int sp = 0; sp < NS; ++sp) {
      const float w = exp2f(ml[sp].x - M);  // 0 for a part with no key of the row
      l += w * ml[sp].y;
      o += w * op[sp];
    }
    o *= 1.f / l;
    *reinterpret_cast<f32x4*>(a.O + row * D + c) = o;
  }
  float dpart = 0.f;
  if (ok && a.dO != nullptr) {
    const __bf16* dOr = reinterpret_cast<const __bf16*>(a.dO) + row * D + c;
#pragma unroll
    for (int q = 0; q < 4; ++q) dpart += (float)dOr[q] * o[q];
  }
#pragma unroll
  for (int off = kLanes / 2; off > 0; off >>= 1) dpart += __shfl_xor(dpart, off);
  if (ok && c == 0) {
    a.L[row] = (M + __log2f(l)) * kLn2;
    if (a.dO != nullptr) a.D[row] = dpart;
  }
}

constexpr int kMaxFwdParts = 16;

template <int D, int NS = 2>
hipError_t launch_fwd_reduce(const FwdArgs& a, int64_t rows, dim3 grid, hipStream_t s) {
  if constexpr (NS > kMaxFwdParts) {
    return hipErrorInvalidValue;
  } else {
    if (a.nsplit != NS) return launch_fwd_reduce<D, NS + 1>(a, rows, grid, s);
    hipLaunchKernelGGL((fwd_reduce_kernel<D, NS>), grid, dim3(256), 0, s, a, rows);
    return hipGetLastError();
  }
}

}  // namespace

// Parts per row tile for the split forward (bf16 only), considered while the row tiles
// (256 rows each) are fewer than the resident work-group slots (two per CU at d = 64,
// one at d = 128, register-limited), with at most 16 parts of at least four key stages
// (of the mean causal sweep).  Unequal causal tiles: enough parts to fill the slots.
// Equal (unmasked) tiles: a cost estimate -- whole rounds of the 256 CUs (a second
// resident work-group adds no throughput at d = 64) times the part's stages at the
// measured stage time of a lone work-group (2.2 us per 128 keys at d = 64, 1.87 us per
// 64 keys at d = 128), plus the partial states written and re-read by the merge
// (2 s (d + 2) fp32 per row at 5 TB/s) and 5 us of launch and prologue -- and a split
// only where it is at most 0.9 of the unsplit estimate.
FwdPlan fwd_split_plan(const Problem& p) {
  FwdPlan f;
  if (!p.bf16) return f;
  constexpr int64_t kCUs = 256;
  const int64_t slots = (p.d == 64 ? 2 : 1) * kCUs;
  const int64_t bc = p.d == 64 ? 128 : 64;
  const int64_t tiles = (int64_t)((p.N + 255) / 256) * p.B * p.Hq;
  if (tiles >= slots) return f;
  int64_t stages = (p.N + bc - 1) / bc;
  if (p.causal) stages = (stages + 1) / 2;
  const int64_t cap = std::min<int64_t>(stages / 4, kMaxFwdParts);
  const int64_t rows = (int64_t)p.B * p.Hq * p.N;
  int64_t sp = 1;
  if (p.causal) {
    sp = std::min<int64_t>((slots + tiles - 1) / tiles, cap);
  } else {
    const double t_stage = p.d == 64 ? 2.2 : 1.87;  // us
    const double unsplit = (double)((tiles + kCUs - 1) / kCUs) * stages * t_stage;
    double best = 0.9 * unsplit;
    for (int64_t k = 2; k <= cap; ++k) {
      const double rounds = (double)((tiles * k + kCUs - 1) / kCUs);
      const double merge = 2.0 * k * rows * (p.d + 2) * 4 / 5.0e6;  // bytes / (B/us)
      const double t = rounds * ((stages + k - 1) / k) * t_stage + merge + 5.0;
      if (t < best) {
        best = t;
        sp = k;
      }
    }
  }
  if (sp < 2) return f;
  f.s = (int)sp;
  f.bytes = sp * rows * (p.d + 2) * 4;
  return f;
}

hipError_t launch_forward_split_all(const Problem& p, const FwdArgs& a0, const FwdPlan& plan,
                                    void* workspace, hipStream_t s) {
  FwdArgs a = a0;
  const int64_t rows = (int64_t)p.B * p.Hq * p.N;
  a.nsplit = plan.s;
  a.part = static_cast<float*>(workspace);
  a.part_ml = a.part + (int64_t)plan.s * rows * p.d;
  hipError_t e = launch_forward_split(p, a, s);
  if (e != hipSuccess) return e;
  const int per = 256 / (p.d / 4);
  const dim3 grid((unsigned)((rows + per - 1) / per));
  if (p.d == 64) return launch_fwd_reduce<64>(a, rows, grid, s);
  return launch_fwd_reduce<128>(a, rows, grid, s);
}

}  // namespace fbob
