// Backward grouped expert GEMMs, fp32 path (bf16 runs on the direct-to-LDS
// core in gemm2.hip).
//
// dH: pull reverse-combine -- dY rows gathered through the schedule's
//   permutation into LDS -- times W2[e] (MN-contiguous, transposed in
//   registers). The epilogue fuses the SwiGLU backward and the gate gradient
//   (router-weight gradients fused into the SwiGLU backward, SonicMoE-style:
//   dothoosh.com MoK page, "Technical details of the MoK mechanism"):
//     g'_partial(row, 32-column block) = sum over the block's columns of dA * h
//     dh = g * dA;  da = dh*u*sig(a)*(1 + a*(1 - sig(a)));  du = dh*silu(a)
//   Partials are summed in a fixed order -- 16 columns sequentially per lane,
//   the two halves of each 32-column block, then the blocks in ascending column
//   order in the router-backward kernel -- independent of the tile shape, the
//   wave layout and the grid; no float atomics.
// dX: push reverse-dispatch -- q = dGU . W1[e] written to the (token, slot)
//   partial row perm[row]; reduced per token in slot order afterwards.
// dW2[e] = sum_r (g*dY)_r^T h_r and dW1[e] = sum_r dGU_r^T x_r: K runs over the
//   expert's routed rows (ragged tail zero-padded); one workgroup per output
//   tile, XCD-grouped by expert; zero-token experts write zeros.
#include "gemm.h"
#include "kernels.h"

namespace mok {

constexpr int kMaxEb = 1024;

template <typename T>
struct DhArgs {
  Sched sc;
  const T* dy;
  const T* w2;
  const T* au;
  const T* h;
  const float* gate;
  T* dgu;
  float* dgp;
  int H, I, k, R;
};

template <typename T>
struct DxArgs {
  Sched sc;
  const T* dgu;
  const T* w1;
  T* part;
  int H, I;
};

// Row-major matrix read in the MN-contiguous orientation: element (k, mn) at base[k*ld + mn].
template <typename T>
struct DenseMN {
  const T* base;
  int64_t ld;
  __device__ __forceinline__ uint4 operator()(int k, int mn) const { return ldg16(base + (int64_t)k * ld + mn); }
};

template <typename T, class Tl>
__global__ __launch_bounds__(256) void dh_kernel(DhArgs<T> a) {
  __shared__ __align__(16) char smem[Tl::LDS_BYTES];
  __shared__ int s_ts[kMaxEb + 1];
  __shared__ int s_slot[Tl::BM];
  constexpr int BKE = kRowBytes / (int)sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int I2 = 2 * a.I;
  load_tile_start(a.sc, s_ts);
  for_each_row_tile(a.sc, s_ts, a.I / Tl::BN, blockIdx.x, gridDim.x, [&](const RowTile& t) {
    __syncthreads();
    for (int i = tid; i < Tl::BM; i += kThreads) s_slot[i] = i < t.nrows ? a.sc.perm[t.row0 + i] : -1;
    __syncthreads();
    KStager<T, Tl::BM> sa;
    sa.tid = tid;
    sa.L.init(tid, [&](int row) -> const T* {
      const int s = s_slot[row];
      return s >= 0 ? a.dy + (int64_t)(s / a.k) * a.H : nullptr;
    });
    MNStager<T, Tl::BN, DenseMN<T>> sb;
    sb.tid = tid;
    sb.src = DenseMN<T>{a.w2 + (int64_t)t.e * a.H * a.I + t.n * Tl::BN, a.I};
    f32x16_t acc[Tl::FM][Tl::FN];
    main_loop<T, Tl>(sa, sb, a.H / BKE, smem, wm, wn, lane, acc);
    epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane, [&](int row, int col, const float (&dA)[16], const float (&)[16]) {
      const bool ok = row < t.nrows;
      float part = 0.0f;
      if (ok) {
        const int64_t R = t.row0 + row;
        const int c = t.n * Tl::BN + col;
        const float g = a.gate[s_slot[row]];
        float av[16], uv[16], hv[16], da[16], du[16];
        load16<T>(a.au + R * I2 + c, av);
        load16<T>(a.au + R * I2 + a.I + c, uv);
        load16<T>(a.h + R * a.I + c, hv);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          part = __builtin_fmaf(dA[i], hv[i], part);
          const float dh = g * dA[i];
          const float sg = 1.0f / (1.0f + expf(-av[i]));
          da[i] = dh * uv[i] * sg * (1.0f + av[i] * (1.0f - sg));
          du[i] = dh * av[i] * sg;
        }
        store16<T>(a.dgu + R * I2 + c, da);
        store16<T>(a.dgu + R * I2 + a.I + c, du);
      }
      // the 32-column block's sum: columns 0-15 (even lane) + columns 16-31 (odd lane)
      const float other = __shfl_xor(part, 1);
      const float blk = (lane & 1) ? other + part : part + other;
      // one partial per 32-column block of I: the sum over blocks (router_bwd, ascending)
      // does not depend on the tile shape, the wave layout or the grid
      if ((lane & 1) == 0 && row < t.nrows) a.dgp[(int64_t)((t.n * Tl::BN + col) >> 5) * a.R + t.row0 + row] = blk;
    });
  });
}

template <typename T, class Tl>
__global__ __launch_bounds__(256) void dx_kernel(DxArgs<T> a) {
  __shared__ __align__(16) char smem[Tl::LDS_BYTES];
  __shared__ int s_ts[kMaxEb + 1];
  __shared__ int s_slot[Tl::BM];
  constexpr int BKE = kRowBytes / (int)sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int I2 = 2 * a.I;
  load_tile_start(a.sc, s_ts);
  for_each_row_tile(a.sc, s_ts, a.H / Tl::BN, blockIdx.x, gridDim.x, [&](const RowTile& t) {
    __syncthreads();
    for (int i = tid; i < Tl::BM; i += kThreads) s_slot[i] = i < t.nrows ? a.sc.perm[t.row0 + i] : -1;
    __syncthreads();
    KStager<T, Tl::BM> sa;
    sa.tid = tid;
    sa.L.init(tid, [&](int row) -> const T* {
      return s_slot[row] >= 0 ? a.dgu + (int64_t)(t.row0 + row) * I2 : nullptr;
    });
    MNStager<T, Tl::BN, DenseMN<T>> sb;
    sb.tid = tid;
    sb.src = DenseMN<T>{a.w1 + (int64_t)t.e * I2 * a.H + t.n * Tl::BN, a.H};
    f32x16_t acc[Tl::FM][Tl::FN];
    main_loop<T, Tl>(sa, sb, I2 / BKE, smem, wm, wn, lane, acc);
    epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane, [&](int row, int col, const float (&g)[16], const float (&)[16]) {
      if (row < t.nrows) store16<T>(a.part + (int64_t)s_slot[row] * a.H + t.n * Tl::BN + col, g);
    });
  });
}

// ---------------------------------------------------------------------------
// Weight gradients: K = the expert's routed rows [offsets[e], offsets[e] + counts[e]).
// ---------------------------------------------------------------------------
template <typename T, typename TO>
struct DwArgs {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const T* tok;        // token-indexed operand (dY for dW2, x for dW1), [T][H]
  const float* gate;   // dW2 only: scales the dY rows
  const T* rows;       // routed-row operand (h for dW2 [R][I], dGU for dW1 [R][2I])
  TO* out;
  int H, I, k;
  Guard guard;
};

// (g*dY)[row] or dY[row] / x[row] read through the permutation (token-major operand).
template <typename T, bool SCALE>
struct TokSrc {
  const int32_t* perm;
  const float* gate;
  const T* base;  // already offset by the tile's first column
  int64_t ld;
  int seg0, cnt, k;
  __device__ __forceinline__ uint4 operator()(int kk, int mn) const {
    if (kk >= cnt) return make_uint4(0, 0, 0, 0);
    const int s = perm[seg0 + kk];
    const uint4 v = ldg16(base + (int64_t)(s / k) * ld + mn);
    if constexpr (!SCALE) {
      return v;
    } else {
      const float g = gate[s];
      float f[Elem<T>::VE];
      unpack(v, f, (T*)nullptr);
#pragma unroll
      for (int q = 0; q < Elem<T>::VE; ++q) f[q] = g * f[q];
      return pack(f, (T*)nullptr);
    }
  }
};

template <typename T>
struct RowSrc {
  const T* base;  // routed row seg0, first column of the tile
  int64_t ld;
  int cnt;
  __device__ __forceinline__ uint4 operator()(int kk, int mn) const {
    return kk < cnt ? ldg16(base + (int64_t)kk * ld + mn) : make_uint4(0, 0, 0, 0);
  }
};

// DW2: C[m = h][n = i] over expert rows; A = g*dY (token operand), B = h (row operand).
// DW1: C[m = c][n = h] over expert rows; A = dGU (row operand), B = x (token operand).
template <typename T, typename TO, class Tl, bool IS_DW2>
__global__ __launch_bounds__(256) void dw_kernel(DwArgs<T, TO> a) {
  __shared__ __align__(16) char smem[Tl::LDS_BYTES];
  constexpr int BKE = kRowBytes / (int)sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int M = IS_DW2 ? a.H : 2 * a.I;
  const int N = IS_DW2 ? a.I : a.H;
  const int MT = M / Tl::BM, NT = N / Tl::BN;
  if (guard_fail(a.guard)) return;
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const int e = L / (MT * NT);
  const int rem = L - e * MT * NT;
  const int mt = rem / NT, nt = rem - mt * NT;
  const int seg0 = a.offsets[e], cnt = a.counts[e];
  const int KT = (cnt + BKE - 1) / BKE;
  f32x16_t acc[Tl::FM][Tl::FN];
  if constexpr (IS_DW2) {
    MNStager<T, Tl::BM, TokSrc<T, true>> sa;
    sa.tid = tid;
    sa.src = TokSrc<T, true>{a.perm, a.gate, a.tok + mt * Tl::BM, a.H, seg0, cnt, a.k};
    MNStager<T, Tl::BN, RowSrc<T>> sb;
    sb.tid = tid;
    sb.src = RowSrc<T>{a.rows + (int64_t)seg0 * a.I + nt * Tl::BN, a.I, cnt};
    main_loop<T, Tl>(sa, sb, KT, smem, wm, wn, lane, acc);
  } else {
    MNStager<T, Tl::BM, RowSrc<T>> sa;
    sa.tid = tid;
    sa.src = RowSrc<T>{a.rows + (int64_t)seg0 * 2 * a.I + mt * Tl::BM, 2 * a.I, cnt};
    MNStager<T, Tl::BN, TokSrc<T, false>> sb;
    sb.tid = tid;
    sb.src = TokSrc<T, false>{a.perm, nullptr, a.tok + nt * Tl::BN, a.H, seg0, cnt, a.k};
    main_loop<T, Tl>(sa, sb, KT, smem, wm, wn, lane, acc);
  }
  TO* out = a.out + ((int64_t)e * M + mt * Tl::BM) * N + nt * Tl::BN;
  epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane, [&](int row, int col, const float (&g)[16], const float (&)[16]) {
    store16<TO>(out + (int64_t)row * N + col, g);
  });
}

// ---------------------------------------------------------------------------
template <int BM, int BN>
using RowTilingB = Tiling<BM, BN, (BM == 128 ? 2 : 1), (BM == 128 ? 2 : 4)>;
using DwTiling = Tiling<128, 128, 2, 2>;

template <class Tl>
static int persistent_grid_b(const Ctx& c, int ntn) {
  const int lds = Tl::LDS_BYTES + 4 * (kMaxEb + 1) + 4 * Tl::BM * (1 + Tl::BN / 32);
  const int occ = std::max(1, std::min(2, (160 * 1024) / lds));
  int g = c.grid > 0 ? c.grid : c.num_cu * occ;
  const int64_t upper = (int64_t)c.max_tiles * ntn;
  if (g > upper) g = (int)std::max<int64_t>(upper, 1);
  return g;
}

static Sched sched_of_b(const Ctx& c) { return Sched{c.counts, c.offsets, c.tile_start, c.perm, c.E, c.BM, c.guard}; }

template <typename T, int BM, int BN>
static hipError_t dh_t(const Ctx& c, const void* dy, const void* w2, const void* au, const void* h, const float* gate,
                       void* dgu, float* dgp) {
  using Tl = RowTilingB<BM, BN>;
  DhArgs<T> a{sched_of_b(c), (const T*)dy, (const T*)w2, (const T*)au, (const T*)h, gate, (T*)dgu, dgp,
              c.H, c.I, c.k, c.R};
  hipLaunchKernelGGL((dh_kernel<T, Tl>), dim3(persistent_grid_b<Tl>(c, c.I / BN)), dim3(kThreads), 0, c.s, a);
  return hipGetLastError();
}

template <typename T, int BM, int BN>
static hipError_t dx_t(const Ctx& c, const void* dgu, const void* w1, void* part) {
  using Tl = RowTilingB<BM, BN>;
  DxArgs<T> a{sched_of_b(c), (const T*)dgu, (const T*)w1, (T*)part, c.H, c.I};
  hipLaunchKernelGGL((dx_kernel<T, Tl>), dim3(persistent_grid_b<Tl>(c, c.H / BN)), dim3(kThreads), 0, c.s, a);
  return hipGetLastError();
}

#define MOK_BM_SWITCH(CALL_32, CALL_64, CALL_128) \
  switch (c.BM) {                                 \
    case 32: return CALL_32;                      \
    case 64: return CALL_64;                      \
    case 128: return CALL_128;                    \
  }                                               \
  return hipErrorInvalidValue;

template <typename T, int BN>
static hipError_t dh_bn(const Ctx& c, const void* dy, const void* w2, const void* au, const void* h, const float* gate,
                        void* dgu, float* dgp) {
  MOK_BM_SWITCH((dh_t<T, 32, BN>(c, dy, w2, au, h, gate, dgu, dgp)), (dh_t<T, 64, BN>(c, dy, w2, au, h, gate, dgu, dgp)),
                (dh_t<T, 128, BN>(c, dy, w2, au, h, gate, dgu, dgp)))
}

template <typename T, int BN>
static hipError_t dx_bn(const Ctx& c, const void* dgu, const void* w1, void* part) {
  MOK_BM_SWITCH((dx_t<T, 32, BN>(c, dgu, w1, part)), (dx_t<T, 64, BN>(c, dgu, w1, part)),
                (dx_t<T, 128, BN>(c, dgu, w1, part)))
}

hipError_t launch_dh(const Ctx& c, const void* dy, const void* w2, const void* au, const void* h, const float* gate,
                     void* dgu, float* dgp) {
  if (c.R == 0) return hipSuccess;
  if (c.act != MOK_F32) return launch_dh_bf16(c, dy, w2, au, h, gate, dgu, dgp);
  return bn_rows(c.I) == 256 ? dh_bn<float, 256>(c, dy, w2, au, h, gate, dgu, dgp)
                             : dh_bn<float, 128>(c, dy, w2, au, h, gate, dgu, dgp);
}

hipError_t launch_dx(const Ctx& c, const void* dgu, const void* w1, void* part) {
  if (c.R == 0) return hipSuccess;
  if (c.act != MOK_F32) return launch_dx_bf16(c, dgu, w1, part);
  return bn_rows(c.H) == 256 ? dx_bn<float, 256>(c, dgu, w1, part) : dx_bn<float, 128>(c, dgu, w1, part);
}

template <typename T, typename TO, bool IS_DW2>
static hipError_t dw_t(const Ctx& c, const T* tok, const float* gate, const T* rows, void* out) {
  using Tl = DwTiling;
  DwArgs<T, TO> a{c.counts, c.offsets, c.perm, tok, gate, rows, (TO*)out, c.H, c.I, c.k, c.guard};
  const int M = IS_DW2 ? c.H : 2 * c.I, N = IS_DW2 ? c.I : c.H;
  const int64_t blocks = (int64_t)c.E * (M / Tl::BM) * (N / Tl::BN);
  hipLaunchKernelGGL((dw_kernel<T, TO, Tl, IS_DW2>), dim3((unsigned)blocks), dim3(kThreads), 0, c.s, a);
  return hipGetLastError();
}

// fp32 weight gradients (bf16 runs on the direct-to-LDS core over pre-gathered rows)
hipError_t launch_dw2(const Ctx& c, const void* dy, const float* gate, const void* h, void* dw2) {
  return dw_t<float, float, true>(c, (const float*)dy, gate, (const float*)h, dw2);
}

hipError_t launch_dw1(const Ctx& c, const void* dgu, const void* x, void* dw1) {
  return dw_t<float, float, false>(c, (const float*)x, nullptr, (const float*)dgu, dw1);
}

}  // namespace mok
