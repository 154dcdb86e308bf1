// Grouped-GEMM building blocks for gfx950: LDS tiles, operand loaders, MFMA main loop.
//
// Every GEMM of the layer is C[M][N] = sum_k A[m][k] * B[n][k] over one expert.
// Both operands are staged in LDS "K-contiguous": tile row = one m (or n), 128
// bytes of K per row (64 bf16 or 32 fp32), 16-byte chunks XOR-swizzled so that
// the MFMA fragment reads (32 consecutive rows, one chunk) and the transposing
// stores (rows 8 apart) are both free of bank conflicts.
//
// Operands arrive in one of two global layouts:
//  * K-contiguous rows (x, dy, h, dGU rows; W1/W2 in the forward), possibly
//    gathered through the schedule's permutation -- KLoader;
//  * MN-contiguous (W2/W1 in the backward data-gradient GEMMs; token-major
//    operands of the weight-gradient GEMMs, where K runs over routed rows) --
//    MNLoader, which loads an 8x8 (bf16) / 4x4 (fp32) block per thread and
//    transposes it in registers before the LDS store.
//
// MFMA: v_mfma_f32_32x32x16_bf16 (bf16) or 4 x v_mfma_f32_32x32x2_f32 (fp32).
// Lane l supplies row (l % 32) of A / column (l % 32) of B and the 16-byte
// K-chunk (l / 32) of a chunk pair; both operands use the same K assignment, so
// any assignment is a valid dot product. Accumulator register r of lane l
// holds C[8*(r/4) + 4*(l/32) + r%4][l % 32] of the 32x32 block.
#pragma once
#include "common.h"

namespace mok {

constexpr int kThreads = 256;  // 4 waves per GEMM workgroup
constexpr int kRowBytes = 128; // bytes of K per LDS tile row

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static __device__ __forceinline__ void run(f32x16_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x16_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// K-contiguous operand: ROWS tile rows, each a pointer to K-contiguous data
// (nullptr = zero row). Thread t owns 16-byte vectors t + v*256 of the tile.
// ---------------------------------------------------------------------------
template <typename T, int ROWS>
struct KLoader {
  static constexpr int VE = Elem<T>::VE;
  static constexpr int BKE = kRowBytes / (int)sizeof(T);  // K elements per tile
  static constexpr int NV = ROWS * 8 / kThreads;
  static_assert(NV >= 1 && ROWS * 8 % kThreads == 0, "tile rows must be a multiple of 32");
  const T* ptr[NV];

  // rowptr(row) -> const T* (start of the row's K range) or nullptr
  template <class F> __device__ __forceinline__ void init(int tid, F rowptr) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int idx = tid + v * kThreads;
      const T* p = rowptr(idx >> 3);
      ptr[v] = p ? p + (idx & 7) * VE : nullptr;
    }
  }
  __device__ __forceinline__ void load(int kt, uint4 (&r)[NV]) const {
#pragma unroll
    for (int v = 0; v < NV; ++v) r[v] = ptr[v] ? ldg16(ptr[v] + (int64_t)kt * BKE) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(int tid, const uint4 (&r)[NV], char* lds) const {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int idx = tid + v * kThreads;
      *reinterpret_cast<uint4*>(lds + lds_off(idx >> 3, idx & 7)) = r[v];
    }
  }
};

// ---------------------------------------------------------------------------
// MN-contiguous operand: element (k, mn) read through a functor
// src(k, mn0) -> uint4 holding elements mn0 .. mn0+VE-1 at row k (zeros past
// the end of K). Blocks of VE (k) x VE (mn) per thread, transposed in registers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// v[q] holds 8 consecutive mn at k = q; o[j] receives 8 consecutive k at mn = j.
__device__ __forceinline__ void transpose8x8_b16(const uint4 (&v)[8], uint4 (&o)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = word(v[2 * d], j >> 1), y = word(v[2 * d + 1], j >> 1);
      w[d] = (j & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
    }
    o[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}
__device__ __forceinline__ void transpose4x4_b32(const uint4 (&v)[4], uint4 (&o)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = make_uint4(word(v[0], j), word(v[1], j), word(v[2], j), word(v[3], j));
}

template <typename T, int ROWS>
struct MNLoader {
  static constexpr int VE = Elem<T>::VE;
  static constexpr int BKE = kRowBytes / (int)sizeof(T);
  static constexpr int KB = BKE / VE;   // 8 k-blocks per tile
  static constexpr int MB = ROWS / VE;  // mn-blocks per tile
  static constexpr int NBLK = MB * KB;
  static constexpr int NB = (NBLK + kThreads - 1) / kThreads;

  template <class S> __device__ __forceinline__ void load(int tid, int kt, const S& src, uint4 (&r)[NB][VE]) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = tid + i * kThreads;
      if (NBLK % kThreads == 0 || b < NBLK) {
        const int mnb = b % MB, kb = b / MB;
#pragma unroll
        for (int q = 0; q < VE; ++q) r[i][q] = src(kt * BKE + kb * VE + q, mnb * VE);
      }
    }
  }
  __device__ __forceinline__ void store(int tid, const uint4 (&r)[NB][VE], char* lds) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = tid + i * kThreads;
      if (NBLK % kThreads == 0 || b < NBLK) {
        const int mnb = b % MB, kb = b / MB;
        uint4 o[VE];
        if constexpr (VE == 8)
          transpose8x8_b16(r[i], o);
        else
          transpose4x4_b32(r[i], o);
#pragma unroll
        for (int j = 0; j < VE; ++j) *reinterpret_cast<uint4*>(lds + lds_off(mnb * VE + j, kb)) = o[j];
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Wave tiling and the MFMA step over one LDS K-tile.
// ---------------------------------------------------------------------------
template <int BM_, int BN_, int WM_, int WN_>
struct Tiling {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN;        // waves per workgroup
  static constexpr int NT = 64 * NW;        // threads per workgroup
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static constexpr int LDS_A = BM * kRowBytes, LDS_B = BN * kRowBytes;
  static constexpr int LDS_STAGE = LDS_A + LDS_B;
  static constexpr int LDS_BYTES = 2 * LDS_STAGE;
};

template <typename T, class Tl>
__device__ __forceinline__ void mma_tile(const char* sA, const char* sB, int wm, int wn, int lane,
                                         f32x16_t (&acc)[Tl::FM][Tl::FN]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = ks * 2 + (lane >> 5);
    uint4 a[Tl::FM], b[Tl::FN];
#pragma unroll
    for (int fm = 0; fm < Tl::FM; ++fm)
      a[fm] = *reinterpret_cast<const uint4*>(sA + lds_off(wm * Tl::WTM + fm * 32 + (lane & 31), ch));
#pragma unroll
    for (int fn = 0; fn < Tl::FN; ++fn)
      b[fn] = *reinterpret_cast<const uint4*>(sB + lds_off(wn * Tl::WTN + fn * 32 + (lane & 31), ch));
#pragma unroll
    for (int fm = 0; fm < Tl::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < Tl::FN; ++fn) Mma<T>::run(acc[fm][fn], a[fm], b[fn]);
  }
}

template <class Tl>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[Tl::FM][Tl::FN]) {
#pragma unroll
  for (int fm = 0; fm < Tl::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < Tl::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;
}

// Row (within the workgroup tile) of accumulator register r of block fm.
template <class Tl>
__device__ __forceinline__ int acc_row(int wm, int fm, int r, int lane) {
  return wm * Tl::WTM + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
template <class Tl>
__device__ __forceinline__ int acc_col(int wn, int fn, int lane) {
  return wn * Tl::WTN + fn * 32 + (lane & 31);
}

// Double-buffered main loop. LA/LB are "stagers": objects with
//   load(kt) (global -> registers) and store(stage_ptr) (registers -> LDS).
template <typename T, class Tl, class SA, class SB>
__device__ __forceinline__ void main_loop(SA& la, SB& lb, int KT, char* smem, int wm, int wn, int lane,
                                          f32x16_t (&acc)[Tl::FM][Tl::FN]) {
  zero_acc<Tl>(acc);
  if (KT <= 0) return;
  la.load(0);
  lb.load(0);
  la.store(smem);
  lb.store(smem + Tl::LDS_A);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    char* cur = smem + (kt & 1) * Tl::LDS_STAGE;
    char* nxt = smem + ((kt + 1) & 1) * Tl::LDS_STAGE;
    const bool more = kt + 1 < KT;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
    mma_tile<T, Tl>(cur, cur + Tl::LDS_A, wm, wn, lane, acc);
    if (more) {
      la.store(nxt);
      lb.store(nxt + Tl::LDS_A);
    }
    __syncthreads();
  }
}

// Stager adaptors binding a loader to its row/element source.
template <typename T, int ROWS>
struct KStager {
  KLoader<T, ROWS> L;
  uint4 r[KLoader<T, ROWS>::NV];
  int tid;
  __device__ __forceinline__ void load(int kt) { L.load(kt, r); }
  __device__ __forceinline__ void store(char* lds) const { L.store(tid, r, lds); }
};
template <typename T, int ROWS, class S>
struct MNStager {
  MNLoader<T, ROWS> L;
  uint4 r[MNLoader<T, ROWS>::NB][MNLoader<T, ROWS>::VE];
  S src;
  int tid;
  __device__ __forceinline__ void load(int kt) { L.load(tid, kt, src, r); }
  __device__ __forceinline__ void store(char* lds) const { L.store(tid, r, lds); }
};

}  // namespace mok

namespace mok {

// Schedule view passed to the row GEMMs by value.
struct Sched {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* tile_start;
  const int32_t* perm;
  int E;
  int BM;
  Guard guard;
};

// Persistent walk over the tiles of a row GEMM (M = routed rows of one
// schedule tile, N split into NTN tiles). The logical tile order is
// expert-major: expert e, then N-tile n, then M-tile m, so workgroups that run
// together share the expert's weight panel (over m) and its gathered token
// rows (over n). The logical range is split into 8 contiguous parts, one per
// XCD (workgroup b runs on XCD b % 8), so each XCD's L2 sees few experts
// (fewer parts when the grid has fewer than 8 workgroups).
// The number of tiles is read on the device (s_ts = tile_start in LDS).
struct RowTile {
  int e, m, n, row0, nrows;
};

// wg / nwg: this workgroup's index and the number of workgroups walking the tiles (the
// grid of a kernel of its own, or of a fused persistent kernel).
template <class F>
__device__ __forceinline__ void for_each_row_tile(const Sched& sc, const int* s_ts, int NTN, int wg, int nwg,
                                                  F&& body) {
  const int64_t total = (int64_t)s_ts[sc.E] * NTN;
  const int P = min(8, nwg);  // partitions (XCDs that have workgroups)
  const int xcd = wg % P;
  const int nx = (nwg - xcd + P - 1) / P;
  const int li = wg / P;
  const int64_t lo = total * xcd / P, hi = total * (xcd + 1) / P;
  for (int64_t L = lo + li; L < hi; L += nx) {
    // e = last expert with s_ts[e] * NTN <= L
    int a = 0, b = sc.E;  // invariant: s_ts[a]*NTN <= L < s_ts[b]*NTN
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if ((int64_t)s_ts[mid] * NTN <= L) a = mid; else b = mid;
    }
    const int e = a;
    const int Me = s_ts[e + 1] - s_ts[e];
    const int rel = (int)(L - (int64_t)s_ts[e] * NTN);
    RowTile t;  // wave-uniform values: keep them in scalar registers
    t.e = __builtin_amdgcn_readfirstlane(e);
    t.n = __builtin_amdgcn_readfirstlane(rel / Me);
    t.m = __builtin_amdgcn_readfirstlane(rel - t.n * Me);
    t.row0 = __builtin_amdgcn_readfirstlane(sc.offsets[t.e] + t.m * sc.BM);
    t.nrows = __builtin_amdgcn_readfirstlane(min(sc.BM, sc.counts[t.e] - t.m * sc.BM));
    body(t);
  }
}

// Load tile_start[0..E] into LDS (called once per persistent kernel). When the
// schedule check fails every entry is 0: the tile walk then visits no tile and the
// kernel exits having written nothing.
__device__ __forceinline__ void load_tile_start(const Sched& sc, int* s_ts) {
  const bool bad = guard_fail(sc.guard);
  for (int i = threadIdx.x; i <= sc.E; i += blockDim.x) s_ts[i] = bad ? 0 : sc.tile_start[i];
  __syncthreads();
}

}  // namespace mok

namespace mok {

// Epilogue staging: each wave copies one (or a pair of) 32x32 accumulator
// block(s) through its own LDS patch and hands them back with every lane
// owning 16 consecutive columns of one row, so global accesses are 16-byte
// vectors. Call after main_loop (its final barrier frees smem). A wave only
// touches its own patch and a wave's LDS operations execute in issue order, so
// there is no workgroup barrier inside; a caller that shares LDS results across
// waves afterwards (or reuses smem) synchronises itself.
//   f(row, col, g, u): row/col are workgroup-tile coordinates of the first of
//   the lane's 16 columns; g[16] = block fn values; u[16] = block fn+1 values
//   when PAIR (the SwiGLU up half), otherwise unused.
constexpr int kPatchLd = 68;  // floats per patch row: 64 columns + 4 pad

template <class Tl, bool PAIR, class F>
__device__ __forceinline__ void epilogue16(f32x16_t (&acc)[Tl::FM][Tl::FN], char* smem, int wave, int wm, int wn,
                                           int lane, F&& f) {
  float* patch = reinterpret_cast<float*>(smem) + wave * (32 * kPatchLd);
  constexpr int STEP = PAIR ? 2 : 1;
#pragma unroll
  for (int fm = 0; fm < Tl::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < Tl::FN; fn += STEP) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        patch[row * kPatchLd + (lane & 31)] = acc[fm][fn][r];
        if constexpr (PAIR) patch[row * kPatchLd + 32 + (lane & 31)] = acc[fm][fn + 1][r];
      }
      const int row = lane >> 1, c0 = (lane & 1) * 16;
      float g[16], u[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = *reinterpret_cast<const float4*>(patch + row * kPatchLd + c0 + 4 * q);
        g[4 * q] = a.x; g[4 * q + 1] = a.y; g[4 * q + 2] = a.z; g[4 * q + 3] = a.w;
        if constexpr (PAIR) {
          const float4 b = *reinterpret_cast<const float4*>(patch + row * kPatchLd + 32 + c0 + 4 * q);
          u[4 * q] = b.x; u[4 * q + 1] = b.y; u[4 * q + 2] = b.z; u[4 * q + 3] = b.w;
        }
      }
      f(wm * Tl::WTM + fm * 32 + row, wn * Tl::WTN + fn * 32 + c0, g, u);
    }
}

// 16 values -> two 16-byte vectors of T at p (8 bf16 each) or four (fp32).
template <typename T>
__device__ __forceinline__ void store16(T* p, const float (&v)[16]);
template <>
__device__ __forceinline__ void store16<bf16>(bf16* p, const float (&v)[16]) {
  float a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { a[i] = v[i]; b[i] = v[8 + i]; }
  stg16(p, pack(a, (bf16*)nullptr));
  stg16(p + 8, pack(b, (bf16*)nullptr));
}
template <>
__device__ __forceinline__ void store16<float>(float* p, const float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) stg16(p + 4 * q, make_uint4(__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                                                          __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])));
}

// 16 consecutive elements of T at p -> floats.
template <typename T>
__device__ __forceinline__ void load16(const T* p, float (&v)[16]);
template <>
__device__ __forceinline__ void load16<bf16>(const bf16* p, float (&v)[16]) {
  float a[8], b[8];
  unpack(ldg16(p), a, (bf16*)nullptr);
  unpack(ldg16(p + 8), b, (bf16*)nullptr);
#pragma unroll
  for (int i = 0; i < 8; ++i) { v[i] = a[i]; v[8 + i] = b[i]; }
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 w = ldg16(p + 4 * q);
    v[4 * q] = __uint_as_float(w.x); v[4 * q + 1] = __uint_as_float(w.y);
    v[4 * q + 2] = __uint_as_float(w.z); v[4 * q + 3] = __uint_as_float(w.w);
  }
}

}  // namespace mok
