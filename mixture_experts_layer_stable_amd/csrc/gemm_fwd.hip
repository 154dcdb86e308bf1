// Forward grouped expert GEMMs, fp32 path (bf16 runs on the direct-to-LDS
// core in gemm2.hip).
//
// FC1 + SwiGLU: pull dispatch -- the A tile is gathered straight from x through
// the schedule's permutation (token = perm[row] / k) into LDS; B is the
// expert's W1 with gate and up rows interleaved per 32-column block so that
// one wave holds matching gate/up accumulators and applies
// h = silu(a) * u in registers (SwiGLU expert FFN, dothoosh.com MoK page,
// "Technical details of the MoK mechanism").
// FC2: o = h . W2[e]^T, written as partial row perm[row] = t*k+j (push
// combine: each (token, slot) gets its own landing row; the combine kernel
// reduces them in slot order).
#include "gemm.h"
#include "kernels.h"

namespace mok {

constexpr int kMaxE = 1024;

template <typename T>
struct Fc1Args {
  Sched sc;
  const T* x;
  const T* w1;
  T* au;
  T* h;
  int H, I, k;
};

template <typename T>
struct Fc2Args {
  Sched sc;
  const T* h;
  const T* w2;
  T* part;
  int H, I;
};

template <typename T, class Tl>
__global__ __launch_bounds__(256) void fc1_kernel(Fc1Args<T> a) {
  static_assert(Tl::FN % 2 == 0, "FC1 pairs gate/up blocks");
  __shared__ __align__(16) char smem[Tl::LDS_BYTES];
  __shared__ int s_ts[kMaxE + 1];
  __shared__ int s_slot[Tl::BM];
  constexpr int BKE = kRowBytes / (int)sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int I2 = 2 * a.I;
  load_tile_start(a.sc, s_ts);
  for_each_row_tile(a.sc, s_ts, a.I / (Tl::BN / 2), blockIdx.x, gridDim.x, [&](const RowTile& t) {
    __syncthreads();
    for (int i = tid; i < Tl::BM; i += kThreads) s_slot[i] = i < t.nrows ? a.sc.perm[t.row0 + i] : -1;
    __syncthreads();
    KStager<T, Tl::BM> sa;
    sa.tid = tid;
    sa.L.init(tid, [&](int row) -> const T* {
      const int s = s_slot[row];
      return s >= 0 ? a.x + (int64_t)(s / a.k) * a.H : nullptr;
    });
    const int cbase = t.n * (Tl::BN / 2);
    KStager<T, Tl::BN> sb;
    sb.tid = tid;
    sb.L.init(tid, [&](int j) -> const T* {
      const int wj = j / Tl::WTN, fn = (j % Tl::WTN) >> 5;
      const int c = cbase + wj * (Tl::WTN / 2) + (fn >> 1) * 32 + (j & 31);
      return a.w1 + ((int64_t)t.e * I2 + ((fn & 1) ? a.I + c : c)) * a.H;
    });
    f32x16_t acc[Tl::FM][Tl::FN];
    main_loop<T, Tl>(sa, sb, a.H / BKE, smem, wm, wn, lane, acc);
    epilogue16<Tl, true>(acc, smem, wave, wm, wn, lane, [&](int row, int col, const float (&g)[16], const float (&u)[16]) {
      if (row >= t.nrows) return;
      const int64_t R = t.row0 + row;
      // tile column of a gate block -> gate column of W1: blocks alternate gate/up per wave
      const int wj = col / Tl::WTN, cw = col % Tl::WTN;
      const int c = cbase + wj * (Tl::WTN / 2) + (cw >> 6) * 32 + (cw & 31);
      float hv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) hv[i] = g[i] / (1.0f + expf(-g[i])) * u[i];
      store16<T>(a.au + R * I2 + c, g);
      store16<T>(a.au + R * I2 + a.I + c, u);
      store16<T>(a.h + R * a.I + c, hv);
    });
  });
}

template <typename T, class Tl>
__global__ __launch_bounds__(256) void fc2_kernel(Fc2Args<T> a) {
  __shared__ __align__(16) char smem[Tl::LDS_BYTES];
  __shared__ int s_ts[kMaxE + 1];
  __shared__ int s_slot[Tl::BM];
  constexpr int BKE = kRowBytes / (int)sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  load_tile_start(a.sc, s_ts);
  for_each_row_tile(a.sc, s_ts, a.H / Tl::BN, blockIdx.x, gridDim.x, [&](const RowTile& t) {
    __syncthreads();
    for (int i = tid; i < Tl::BM; i += kThreads) s_slot[i] = i < t.nrows ? a.sc.perm[t.row0 + i] : -1;
    __syncthreads();
    KStager<T, Tl::BM> sa;
    sa.tid = tid;
    sa.L.init(tid, [&](int row) -> const T* {
      return s_slot[row] >= 0 ? a.h + (int64_t)(t.row0 + row) * a.I : nullptr;
    });
    KStager<T, Tl::BN> sb;
    sb.tid = tid;
    sb.L.init(tid, [&](int j) -> const T* { return a.w2 + ((int64_t)t.e * a.H + t.n * Tl::BN + j) * a.I; });
    f32x16_t acc[Tl::FM][Tl::FN];
    main_loop<T, Tl>(sa, sb, a.I / BKE, smem, wm, wn, lane, acc);
    epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane, [&](int row, int col, const float (&g)[16], const float (&)[16]) {
      if (row < t.nrows) store16<T>(a.part + (int64_t)s_slot[row] * a.H + t.n * Tl::BN + col, g);
    });
  });
}

// Wave layout per schedule tile height: 2x2 waves for 128-row tiles, 1x4 below.
template <int BM, int BN>
using RowTiling = Tiling<BM, BN, (BM == 128 ? 2 : 1), (BM == 128 ? 2 : 4)>;

template <class Tl>
static int persistent_grid(const Ctx& c, int ntn) {
  const int lds = Tl::LDS_BYTES + 4 * (kMaxE + 1) + 4 * Tl::BM;
  const int occ = std::max(1, std::min(2, (160 * 1024) / lds));
  int g = c.grid > 0 ? c.grid : c.num_cu * occ;
  const int64_t upper = (int64_t)c.max_tiles * ntn;
  if (g > upper) g = (int)std::max<int64_t>(upper, 1);
  return g;
}

static Sched sched_of(const Ctx& c) { return Sched{c.counts, c.offsets, c.tile_start, c.perm, c.E, c.BM, c.guard}; }

template <typename T, int BM>
static hipError_t fc1_bm(const Ctx& c, const void* x, const void* w1, void* au, void* h) {
  using Tl = RowTiling<BM, 256>;
  Fc1Args<T> a{sched_of(c), (const T*)x, (const T*)w1, (T*)au, (T*)h, c.H, c.I, c.k};
  const int g = persistent_grid<Tl>(c, c.I / (Tl::BN / 2));
  hipLaunchKernelGGL((fc1_kernel<T, Tl>), dim3(g), dim3(kThreads), 0, c.s, a);
  return hipGetLastError();
}

template <typename T, int BM, int BN>
static hipError_t fc2_t(const Ctx& c, const void* h, const void* w2, void* part) {
  using Tl = RowTiling<BM, BN>;
  Fc2Args<T> a{sched_of(c), (const T*)h, (const T*)w2, (T*)part, c.H, c.I};
  const int g = persistent_grid<Tl>(c, c.H / Tl::BN);
  hipLaunchKernelGGL((fc2_kernel<T, Tl>), dim3(g), dim3(kThreads), 0, c.s, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t fc1_t(const Ctx& c, const void* x, const void* w1, void* au, void* h) {
  switch (c.BM) {
    case 32: return fc1_bm<T, 32>(c, x, w1, au, h);
    case 64: return fc1_bm<T, 64>(c, x, w1, au, h);
    case 128: return fc1_bm<T, 128>(c, x, w1, au, h);
  }
  return hipErrorInvalidValue;
}

template <typename T, int BN>
static hipError_t fc2_bn(const Ctx& c, const void* h, const void* w2, void* part) {
  switch (c.BM) {
    case 32: return fc2_t<T, 32, BN>(c, h, w2, part);
    case 64: return fc2_t<T, 64, BN>(c, h, w2, part);
    case 128: return fc2_t<T, 128, BN>(c, h, w2, part);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fc1(const Ctx& c, const void* x, const void* w1, void* au, void* h) {
  if (c.R == 0) return hipSuccess;
  return c.act == MOK_F32 ? fc1_t<float>(c, x, w1, au, h) : launch_fc1_bf16(c, x, w1, au, h);
}

hipError_t launch_fc2(const Ctx& c, const void* h, const void* w2, void* part) {
  if (c.R == 0) return hipSuccess;
  if (c.act != MOK_F32) return launch_fc2_bf16(c, h, w2, part);
  return bn_rows(c.H) == 256 ? fc2_bn<float, 256>(c, h, w2, part) : fc2_bn<float, 128>(c, h, w2, part);
}

}  // namespace mok
