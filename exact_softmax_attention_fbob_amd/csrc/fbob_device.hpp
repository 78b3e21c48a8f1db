// fbob_device.hpp - gfx950 device primitives shared by the forward, Pass 1 and
// Pass 2 kernels: MFMA fragments, LDS tile layout, tile staging, lane reductions.
//
// Wavefront layout used everywhere (64 lanes, lane = 16 g + r, r in [0,16),
// g in [0,4)), for a 16x16 output block of a 16x16xK MFMA:
//   A operand  lane (r, g) holds A[row r][k(g, e)], e = 0..7
//   B operand  lane (r, g) holds B[k(g, e)][col r]
//   C/D        lane (r, g) holds C[row 4 g + q][col r], q = 0..3
// Only the pairing of (g, e) between A and B matters for the product, so any
// bijection k(g, e) works as long as both operands use the same one.  The score
// tiles are computed transposed (keys/rows that are contracted later along the
// C "row" axis) so that the C registers of two adjacent 16-row blocks are directly
// the 8-element B operand of the next contraction, with
//   k(g, e) = 16 (e / 4) + 4 g + (e % 4).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace fbob {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Keeps the machine scheduler from hoisting loads across phases of a tile (it
// otherwise front-loads every LDS fragment and runs out of registers).
#define FBOB_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
constexpr float kLn2 = 0.6931471805599453f;

// Instruction groups for __builtin_amdgcn_sched_group_barrier: the scheduler
// fills the groups in the order they are declared (one pipeline per region), so a
// sequence of (LDS read, n) and (MFMA, m) groups fixes how far fragment loads run
// ahead of the MFMAs that consume them.
constexpr int kSgMfma = 0x008;
constexpr int kSgDsRead = 0x100;
#define FBOB_SGB(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

// Wave priority around an MFMA-dense block: while one wave of a SIMD issues its
// MFMAs at raised priority the matrix pipe stays fed, and the other wave's VALU
// work fills the issue cycles in between.  The scheduling fences keep the block's
// instructions between the two priority changes.
#define FBOB_PRIO_HIGH()               \
  do {                                 \
    __builtin_amdgcn_sched_barrier(0); \
    __builtin_amdgcn_s_setprio(1);     \
    __builtin_amdgcn_sched_barrier(0); \
  } while (0)
#define FBOB_PRIO_LOW()                \
  do {                                 \
    __builtin_amdgcn_sched_barrier(0); \
    __builtin_amdgcn_s_setprio(0);     \
    __builtin_amdgcn_sched_barrier(0); \
  } while (0)

// ---------------------------------------------------------------------------
// Element traits: storage type of the seven inputs.
// ---------------------------------------------------------------------------
template <typename T> struct Elem;

template <> struct Elem<__bf16> {
  using frag = bf16x8;  // 8 operand elements per lane
  static __device__ __forceinline__ frag from_f32(const f32x4 lo, const f32x4 hi) {
    frag o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[q] = (__bf16)lo[q];
      o[4 + q] = (__bf16)hi[q];
    }
    return o;
  }
  // C += A * B for one 16x16x32 block (bf16 inputs, fp32 accumulate).
  static __device__ __forceinline__ f32x4 mma(const frag a, const frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Elem<float> {
  using frag = f32x8;
  static __device__ __forceinline__ frag from_f32(const f32x4 lo, const f32x4 hi) {
    frag o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[q] = lo[q];
      o[4 + q] = hi[q];
    }
    return o;
  }
  // Same contraction as the bf16 block: eight fp32 16x16x4 MFMAs, the e-th one
  // pairing element e of every lane (k index g within that MFMA).
  static __device__ __forceinline__ f32x4 mma(const frag a, const frag b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
  }
};

// ---------------------------------------------------------------------------
// LDS tile: R rows x D columns of T, row-major, 16-byte chunks XOR-swizzled
// within a row so that the three access patterns of the kernels are free of
// bank conflicts on gfx950:
//   (a) b128 fragment reads: 16 consecutive rows at one logical chunk;
//   (b) transposed b64 reads: 4 rows x 32 bytes per 16-lane group;
//   (c) b128 staging writes of consecutive chunks.
// 128-byte rows (bf16, d = 64): the XOR mask is an invertible map of row bits
// 1..3, (r2) | (r2 ^ r3) << 1 | (r1) << 2, chosen by measuring
// SQ_LDS_BANK_CONFLICT for all 168 such maps on the three patterns (zero on
// each); 256-byte and longer rows use a 16-valued mask of row bits 0..3, also
// measured conflict-free on the three patterns.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct Tile {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per row
  static_assert(kChunks >= 8, "swizzle needs at least 8 chunks per row");
  static __device__ __forceinline__ int swz(int row) {
    if constexpr (kRowBytes == 128)
      return ((row >> 2) & 1) | ((((row >> 2) ^ (row >> 3)) & 1) << 1) | (((row >> 1) & 1) << 2);
    else
      return ((row >> 1) & 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 1) |
             ((((row >> 1) ^ (row >> 2)) & 1) << 2) | ((row & 1) << 3);
  }
  // byte offset of chunk c of row `row`
  static __device__ __forceinline__ int chunk_off(int row, int c) {
    return row * kRowBytes + ((c ^ swz(row)) << 4);
  }
  // byte offset of element (row, col)
  static __device__ __forceinline__ int elem_off(int row, int col) {
    constexpr int per_chunk = 16 / (int)sizeof(T);
    return chunk_off(row, col / per_chunk) + (col % per_chunk) * (int)sizeof(T);
  }
};

// fp32 operand fragments from an LDS tile (bf16 tiles are read through LdsLane
// below, with precomputed offsets and the gfx950 transposing read).
// Row-major: 8 consecutive elements (row, col .. col+7), col a multiple of 8.
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag lds_frag_row(const char* tile, int row, int col) {
  static_assert(sizeof(T) == 4, "bf16 tiles are read through LdsLane");
  const f32x4 lo = *reinterpret_cast<const f32x4*>(tile + Tile<T, D>::chunk_off(row, col >> 2));
  const f32x4 hi = *reinterpret_cast<const f32x4*>(tile + Tile<T, D>::chunk_off(row, (col >> 2) + 1));
  return Elem<T>::from_f32(lo, hi);
}

// Transposed, for a contraction over tile rows: lane (r, g) gets
// X[row0 + k(g, e)][col0 + r], k(g, e) = 16 (e / 4) + 4 g + (e % 4).
template <typename T, int D>
__device__ __forceinline__ typename Elem<T>::frag lds_frag_tr(const char* tile, int row0, int col0,
                                                              int r, int g) {
  static_assert(sizeof(T) == 4, "bf16 tiles are read through LdsLane");
  typename Elem<T>::frag o;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int row = row0 + 16 * (e >> 2) + 4 * g + (e & 3);
    o[e] = *reinterpret_cast<const float*>(tile + Tile<T, D>::elem_off(row, col0 + r));
  }
  return o;
}

// Operand fragment straight from global memory: 8 consecutive elements of one
// row, or zeros when the row is past the end.
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag global_frag(const T* base, int row, int nrows,
                                                              int ld, int col) {
  using F = typename Elem<T>::frag;
  F o;
  if (row < nrows) {
    if constexpr (sizeof(T) == 2) {
      o = *reinterpret_cast<const F*>(base + (int64_t)row * ld + col);
    } else {
      const f32x4* p = reinterpret_cast<const f32x4*>(base + (int64_t)row * ld + col);
      o = Elem<T>::from_f32(p[0], p[1]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (T)0.0f;
  }
  return o;
}

// ---------------------------------------------------------------------------
// Staging of NT same-shaped tiles (ROWS rows each) in one pass: the NT * ROWS *
// chunks 16-byte chunks are spread evenly over the work-group.  Rows past the
// end are clamped to the last row (finite data; every consumer gives them zero
// weight), so the loads need no predication.  The tiles are stored back to back
// in LDS, kTileBytes apart.
// ---------------------------------------------------------------------------
template <typename T, int D, int ROWS, int NT, int NTHREADS>
struct MultiStager {
  static constexpr int kRB = Tile<T, D>::kRowBytes;
  static constexpr int kChunks = Tile<T, D>::kChunks;
  static constexpr int kPerTensor = ROWS * kChunks;
  static constexpr int kTotal = NT * kPerTensor;
  static_assert(kTotal % NTHREADS == 0, "staged chunks must divide evenly over threads");
  static constexpr int kPer = kTotal / NTHREADS;
  static constexpr int kTileBytes = ROWS * kRB;
  const char* src[kPer];  // tensor base + chunk column, per owned chunk
  int row[kPer];          // row within the tile
  int lds_off[kPer];      // tensor tile offset + swizzled chunk offset
  u32x4 v[kPer];

  // `bases` are the NT tensor bases (element pointers of the current head).
  __device__ __forceinline__ void init(const T* const (&bases)[NT], int tid) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int idx = tid + k * NTHREADS;
      const int tensor = idx / kPerTensor, rem = idx % kPerTensor;
      row[k] = rem / kChunks;
      const int c = rem % kChunks;
      const T* base = bases[0];
#pragma unroll
      for (int m = 1; m < NT; ++m)
        if (tensor == m) base = bases[m];
      src[k] = reinterpret_cast<const char*>(base) + c * 16;
      lds_off[k] = tensor * kTileBytes + Tile<T, D>::chunk_off(row[k], c);
    }
  }
  // Retarget the chunks to new tensor bases (same layout), e.g. another head.
  __device__ __forceinline__ void rebase(const T* const (&bases)[NT], int tid) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int idx = tid + k * NTHREADS;
      const int tensor = idx / kPerTensor, c = (idx % kPerTensor) % kChunks;
      const T* base = bases[0];
#pragma unroll
      for (int m = 1; m < NT; ++m)
        if (tensor == m) base = bases[m];
      src[k] = reinterpret_cast<const char*>(base) + c * 16;
    }
  }
  // `byte_off` shifts every tensor by the same amount (another head of the same
  // shape); rows are clamped to nrows - 1.
  __device__ __forceinline__ void load(int row0, int nrows, int64_t byte_off = 0) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int gr = min(row0 + row[k], nrows - 1);
      v[k] = *reinterpret_cast<const u32x4*>(src[k] + byte_off + (int64_t)gr * kRB);
    }
  }
  __device__ __forceinline__ void store(char* tiles) const {
#pragma unroll
    for (int k = 0; k < kPer; ++k) *reinterpret_cast<u32x4*>(tiles + lds_off[k]) = v[k];
  }
};

// ---------------------------------------------------------------------------
// Direct global -> LDS staging (gfx950 global_load_lds_dwordx4): each
// instruction moves 64 lanes x 16 bytes into 1 KiB of consecutive LDS (lane l at
// byte 16 l), i.e. kRowsPerInst whole rows.  The XOR swizzle is applied on the
// global side: the lane at physical chunk p of tile row `row` fetches logical
// chunk p ^ swz(row).  No VGPRs hold the data and no ds_write is issued; the
// caller waits on vmcnt before the barrier that publishes the tile.  Rows past
// the end are clamped to the last row (finite data, given zero weight).
//
// Per lane only one 32-bit offset per instruction is kept (row within the 1 KiB
// block times the row pitch plus the swizzled chunk); tensor bases, block rows
// and LDS offsets are wave-uniform.  A stage that lies wholly inside the tensor
// is addressed as uniform base + lane offset; only a stage that crosses the end
// takes the per-lane clamp.  With RFL the uniform part is read from the first lane
// into scalar registers before the lane offset is added: the compiler otherwise
// keeps base + lane offset as a 64-bit per-lane address for the whole sweep (two
// registers per instruction instead of one), which pushed the d = 128 row pass into
// spills (a reload at every stage, ~3.6 % of its time).
// ---------------------------------------------------------------------------

// A wave-uniform pointer, taken from the first lane.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

template <typename T, int D, int ROWS, int NT, int NW, bool ASM_DMA = false, bool RFL = false>
struct DirectStager {
  static constexpr int kRB = Tile<T, D>::kRowBytes;
  static constexpr int kChunks = Tile<T, D>::kChunks;
  static constexpr int kRowsPerInst = 64 / kChunks;
  static_assert(kRowsPerInst >= 1 && 64 % kChunks == 0, "rows must tile a 1 KiB block");
  static constexpr int kInstPerTensor = ROWS / kRowsPerInst;
  static constexpr int kInst = NT * kInstPerTensor;
  static_assert(kInst % NW == 0, "staging instructions must divide evenly over waves");
  static constexpr int kPer = kInst / NW;  // instructions per wave
  static constexpr int kTileBytes = ROWS * kRB;
  const char* base[kPer];  // tensor base of instruction k (wave-uniform)
  int row_blk[kPer];       // first tile row of instruction k's block (wave-uniform)
  int lds_off[kPer];       // LDS offset of instruction k's 1 KiB block (wave-uniform)
  uint32_t voff[kPer];     // per lane: lrow * kRB + 16 * (swizzled chunk)
  int lrow;                // per lane: row within the block

  // w must be wave-uniform.
  __device__ __forceinline__ void init(const T* const (&bases)[NT], int w, int lane) {
    lrow = lane / kChunks;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int ii = k * NW + w;
      const int tensor = ii / kInstPerTensor, rg = ii % kInstPerTensor;
      row_blk[k] = rg * kRowsPerInst;
      const int c = (lane % kChunks) ^ Tile<T, D>::swz(row_blk[k] + lrow);
      voff[k] = (uint32_t)(lrow * kRB + c * 16);
      const T* b = bases[0];
#pragma unroll
      for (int m = 1; m < NT; ++m)
        if (tensor == m) b = bases[m];
      base[k] = reinterpret_cast<const char*>(b);
      lds_off[k] = tensor * kTileBytes + rg * 1024;
    }
  }
  // One 16-byte-per-lane global -> LDS transfer into the 1 KiB block at `lds`.
  __device__ __forceinline__ static void dma(const char* gp, char* lds) {
    typedef __attribute__((address_space(3))) void lds_void;
    typedef __attribute__((address_space(1))) void glb_void;
    if constexpr (ASM_DMA) {
      // The same instruction written out.  The compiler does not track it, so it
      // neither holds each transposing LDS read (which it cannot prove disjoint from
      // the transfer) until the transfer lands, nor orders other memory accesses
      // around it (no memory clobber).  That is sound under the staging discipline
      // every caller follows: the transfer targets the buffer that no wave reads
      // before the next barrier, the caller's s_waitcnt(0) precedes that barrier,
      // and the barrier (a fence) keeps later reads of the buffer after it; volatile
      // asm is never moved across the waitcnt or the barrier.  The instruction
      // writes no VGPR and reads its address at issue.  M0 (the LDS address) is set
      // by the compiler for the operand, one wait state before the load.
      const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)lds;
      asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gp), "{m0}"(m0));
    } else {
      __builtin_amdgcn_global_load_lds((glb_void*)gp, (lds_void*)lds, 16, 0, 0);
    }
  }
  __device__ __forceinline__ void load(char* tiles, int row0, int nrows, int64_t byte_off = 0) const {
    if (row0 + ROWS <= nrows) {  // wave-uniform: the whole stage lies inside the tensor
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const char* ub = base[k] + byte_off + (int64_t)(row0 + row_blk[k]) * kRB;
        dma((RFL ? uniform_ptr(ub) : ub) + voff[k], tiles + lds_off[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        // rows past the end read the last row: shift this lane's row back
        const int rb = row0 + row_blk[k];
        const int shift = max(rb + lrow - (nrows - 1), 0);
        const char* gp = base[k] + byte_off + ((int64_t)rb - shift) * kRB + voff[k];
        dma(gp, tiles + lds_off[k]);
      }
    }
  }
};

// Wait for every outstanding memory operation of this wave (used before the
// barrier that publishes tiles written by global_load_lds).
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// ---------------------------------------------------------------------------
// Per-lane LDS fragment reader for 32-row staged tiles.  The swizzled byte
// offsets that depend only on the lane are computed once; a read is then a
// tile base plus a compile-time constant plus one of these registers.
//   row(tile, rb, dc): A/B operand rows 16 rb + r, columns 32 dc + 8 g .. +7
//   tr(tile, db):      transposed operand, lane (r, g) gets X[k(g, e)][16 db + r]
// With XOR set (bf16 only) the lane keeps a single offset per pattern: the chunk
// index enters the swizzle by XOR on bits that no other part of the offset uses,
// so the offset of column block dc (db) is the dc = 0 (db = 0) offset XOR
// dc << 6 (db << 5).  `fresh()` returns a copy whose offsets the compiler cannot
// treat as loop invariants, so the XORs are formed once per use site inside the
// loop instead of being hoisted into a table of registers.
// ---------------------------------------------------------------------------
template <typename T, int D, bool XOR = false>
struct LdsLane {
  static constexpr int kRB = Tile<T, D>::kRowBytes;
  static constexpr int kDC = D / 32, kDB = D / 16;
  static constexpr bool kXor = XOR && sizeof(T) == 2;
  int ro[kXor ? 1 : kDC];
  int to[kXor ? 1 : kDB];
  int r, g;

  __device__ __forceinline__ LdsLane(int r_, int g_) : r(r_), g(g_) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int dc = 0; dc < (kXor ? 1 : kDC); ++dc) ro[dc] = Tile<T, D>::chunk_off(r, 4 * dc + g);
      const int b = r >> 2, c = r & 3;
#pragma unroll
      for (int db = 0; db < (kXor ? 1 : kDB); ++db)
        to[db] = Tile<T, D>::elem_off(4 * g + b, 16 * db + 4 * c);
    }
  }
  __device__ __forceinline__ LdsLane fresh() const {
    LdsLane o = *this;
    if constexpr (kXor) {
      asm volatile("" : "+v"(o.ro[0]));
      asm volatile("" : "+v"(o.to[0]));
    }
    return o;
  }
  __device__ __forceinline__ int row_off(int dc) const {
    if constexpr (kXor) return ro[0] ^ (dc << 6);
    else return ro[dc];
  }
  __device__ __forceinline__ int tr_off(int db) const {
    if constexpr (kXor) return to[0] ^ (db << 5);
    else return to[db];
  }
  __device__ __forceinline__ typename Elem<T>::frag row(const char* tile, int rb, int dc) const {
    using F = typename Elem<T>::frag;
    if constexpr (sizeof(T) == 2) {
      return *reinterpret_cast<const F*>(tile + rb * 16 * kRB + row_off(dc));
    } else {
      return lds_frag_row<T, D>(tile, 16 * rb + r, 32 * dc + 8 * g);
    }
  }
  __device__ __forceinline__ typename Elem<T>::frag tr(const char* tile, int db) const {
    if constexpr (sizeof(T) == 2) {
      // gfx950 transposing LDS read: in each 16-lane group, lane (4 b + c)
      // addresses 4 elements of row b at columns 4 c .. 4 c + 3 and receives
      // column r of the 4 addressed rows.
      typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
      const uintptr_t base = reinterpret_cast<uintptr_t>(tile) + tr_off(db);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 16 * kRB));
      typename Elem<T>::frag o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[q] = lo[q];
        o[4 + q] = hi[q];
      }
      return o;
    } else {
      return lds_frag_tr<T, D>(tile, 0, 16 * db, r, g);
    }
  }
};

// How tau reaches the two score-shaped tiles that carry it, S = tau Q K^T and
// F = tau (U_Q K^T + Q U_K^T), in the BoB passes:
//   kTauScaled  the resident operands hold X and tau X (tau X rounded to T); S uses
//               X with the exp2 scale tau log2 e, F uses the scaled copies;
//   kTauPow2    tau is a power of two, so tau X is exact and serves both tiles
//               (exp2 scale log2 e) and X itself is not kept;
//   kTauValu    the resident operands stay unscaled (one operand set fewer in
//               registers); S uses the exp2 scale tau log2 e and the F tile is
//               multiplied by tau on the VALU (one multiply per element).
enum TauMode { kTauScaled = 0, kTauPow2 = 1, kTauValu = 2 };

// Operand fragment scaled by s (fp32 product, rounded back to T).  Exact for
// bf16 when s is a power of two.
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag scale_frag(typename Elem<T>::frag f, float s) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (T)((float)f[e] * s);
  return f;
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::frag zero_frag() {
  typename Elem<T>::frag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (T)0.0f;
  return f;
}

template <typename T>
__device__ __forceinline__ typename Elem<T>::frag ones_frag() {
  typename Elem<T>::frag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (T)1.0f;
  return f;
}

__device__ __forceinline__ f32x4 splat4(float x) { return f32x4{x, x, x, x}; }

// True when tau is an exact power of two, so that tau * x is exact in bf16.
inline bool tau_is_pow2(float tau) {
  int e = 0;
  return tau > 0.f && frexpf(tau, &e) == 0.5f;
}

// Sum over the four 16-lane groups (lanes r, r+16, r+32, r+48).
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of the eight values of two score fragments.  The IEEE-2019 maximum
// (NaN-propagating) maps to gfx950's three-input v_maximum3_f32, four
// instructions for eight values; fmaxf would first canonicalize every MFMA result
// with a move of its own.
__device__ __forceinline__ float max8(const f32x4& a, const f32x4& b) {
  const float m0 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a[0], a[1]), a[2]);
  const float m1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a[3], b[0]), b[1]);
  const float m2 = __builtin_elementwise_maximum(b[2], b[3]);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(m0, m1), m2);
}

// Work-group index remapped so that consecutive logical blocks run on the same
// XCD (the dispatcher hands block b to XCD b % 8): blocks of one head then share
// that XCD's L2 for the streamed operand tiles.  Bijective for any `total`.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, rem = total % kXcd;
  const int xcd = bid % kXcd, slot = bid / kXcd;
  return (xcd < rem) ? xcd * (q + 1) + slot : rem * (q + 1) + (xcd - rem) * q + slot;
}

}  // namespace fbob
