// bf16 grouped expert GEMMs on the direct-to-LDS core (gemm2.h).
//
// Row GEMMs (M = routed rows of one schedule tile, persistent, XCD-partitioned,
// expert-major tile walk):
//   fc1  pull dispatch: A = x rows gathered through perm; B = W1[e] rows with
//        gate/up interleaved per 32-column block; SwiGLU epilogue (h = silu(a)*u).
//   fc2  A = h rows; B = W2[e] rows; o written to the (token, slot) partial row.
//   dh   pull reverse-combine: A = dY rows gathered through perm; B = W2[e] read
//        transposed (MN-contiguous); epilogue: SwiGLU backward + gate-gradient
//        partials (router-weight gradients fused into the SwiGLU backward,
//        dothoosh.com MoK page, "Technical details of the MoK mechanism").
//   dx   push reverse-dispatch: A = dGU rows; B = W1[e] read transposed; q
//        written to the (token, slot) partial row.
// Weight gradients (one workgroup per output tile, XCD-grouped by expert):
//   dw2  dW2[e] = sum over e's routed rows of dO_r^T h_r, dO = g*dY gathered.
//   dw1  dW1[e] = sum over e's routed rows of dGU_r^T x_r, x gathered.
//   Both operands are token-major rows (MN-contiguous, K = routed rows),
//   K-tail rows read from a zero block.
#include "gemm2.h"
#include "kernels.h"

namespace mok {

__device__ uint4 g_zero_1k[64] = {};

constexpr int kMaxE2 = 1024;
constexpr int kRowStages = 3;
constexpr int kDwStages = 4;

// Row GEMM wave layouts. 512-wide tiles (dh, dx, whose weights are read transposed
// in 1 KB k-rows): 8 waves side by side (BM x 64 wave tiles, 32-element K-tiles), so
// each LDS byte written by the DMA feeds twice the MFMA work of a 256-wide tile and
// fragment reads per MFMA drop by a quarter. fc1/fc2 keep 256-wide tiles with 64-element
// K-tiles: their weight rows are K-contiguous, and 32-element K-tiles would fetch them
// 64 bytes at a time. 256/128-wide: 8 waves (2 x 4, 64x64 wave tiles) for 64/128-row
// tiles, 4 waves for 32-row tiles.
template <int BM, int BN>
using RowTiling2 = Tiling<BM, BN, (BN == 512 || BM == 32 ? 1 : 2), (BN == 512 ? 8 : 4)>;

struct RowArgs {
  Sched sc;
  const bf16* a;     // fc1: x; fc2: h; dh: dy; dx: dgu
  const bf16* w;     // fc1: w1; fc2: w2; dh: w2; dx: w1
  bf16* out0;        // fc1: au; fc2/dx: part; dh: dgu
  bf16* out1;        // fc1: h
  const bf16* au;    // dh
  const bf16* h;     // dh
  const float* gate; // dh
  float* dgp;        // dh
  int H, I, k, R;
};

enum RowKind { FC1 = 0, FC2 = 1, DH = 2, DX = 3 };

template <int KIND, class Tl>
__global__ __launch_bounds__(Tl::NT) void row_gemm2_kernel(RowArgs a) {
  constexpr bool K32 = Tl::BN == 512;  // 32-element K-tiles
  using OA = typename std::conditional<K32, OpK32<Tl::BM, Tl::FM, Tl::NW>, OpK<Tl::BM, Tl::FM, Tl::NW>>::type;
  constexpr bool B_MN = KIND == DH || KIND == DX;
  using OBK = typename std::conditional<K32, OpK32<Tl::BN, Tl::FN, Tl::NW>, OpK<Tl::BN, Tl::FN, Tl::NW>>::type;
  using OB = typename std::conditional<B_MN, OpMN<Tl::BN, OA::BK, Tl::FN, Tl::NW>, OBK>::type;
  constexpr int SB = OA::BYTES + OB::BYTES;
  // a fourth ring stage where it fits (32-row tiles: their short per-K-tile work leaves the
  // DMA latency exposed with only two K-tiles in flight)
  constexpr int STAGES = 4 * SB + 8 * 1024 <= 160 * 1024 ? 4 : kRowStages;
  __shared__ __align__(1024) char smem[STAGES * SB];
  __shared__ int s_ts[kMaxE2 + 1];
  __shared__ int s_slot[Tl::BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int I2 = 2 * a.I;
  // N of the GEMM and its tile count; K
  const int N = KIND == FC1 ? I2 : (KIND == FC2 || KIND == DX ? a.H : a.I);
  const int K = KIND == FC1 || KIND == DH ? a.H : (KIND == FC2 ? a.I : I2);
  load_tile_start(a.sc, s_ts);
  for_each_row_tile(a.sc, s_ts, N / Tl::BN, [&](const RowTile& t) {
    __syncthreads();
    for (int i = tid; i < Tl::BM; i += Tl::NT) s_slot[i] = i < t.nrows ? a.sc.perm[t.row0 + i] : -1;
    __syncthreads();
    const auto frow_a = [&](int f) { return wm * Tl::WTM + f * 32; };
    const auto frow_b = [&](int f) { return wn * Tl::WTN + f * 32; };
    OA oa;
    if constexpr (KIND == FC1 || KIND == DH) {
      // gathered token rows; padding rows re-read row 0 (finite; their outputs are dropped)
      oa.init(a.a, [&](int row) -> uint32_t {
        return (uint32_t)(s_slot[row < t.nrows ? row : 0] / a.k) * (uint32_t)(2 * a.H);
      }, frow_a, wave, lane);
    } else {
      oa.init(a.a + (int64_t)t.row0 * K, [&](int row) -> uint32_t {
        return (uint32_t)(row < t.nrows ? row : 0) * (uint32_t)(2 * K);
      }, frow_a, wave, lane);
    }
    OB ob;
    if constexpr (B_MN) {
      // dh: W2[e] [H][I], k = h, columns i; dx: W1[e] [2I][H], k = c, columns h
      const bf16* base = KIND == DH ? a.w + (int64_t)t.e * a.H * a.I + t.n * Tl::BN
                                    : a.w + (int64_t)t.e * I2 * a.H + t.n * Tl::BN;
      ob.init(base, 2 * (int64_t)(KIND == DH ? a.I : a.H), K, frow_b, wave, lane);
    } else if constexpr (KIND == FC1) {
      const int cbase = t.n * (Tl::BN / 2);
      ob.init(a.w + (int64_t)t.e * I2 * a.H, [&](int j) -> uint32_t {
        const int wj = j / Tl::WTN, fn = (j % Tl::WTN) >> 5;
        const int c = cbase + wj * (Tl::WTN / 2) + (fn >> 1) * 32 + (j & 31);
        return (uint32_t)((fn & 1) ? a.I + c : c) * (uint32_t)(2 * a.H);
      }, frow_b, wave, lane);
    } else {
      ob.init(a.w + ((int64_t)t.e * a.H + t.n * Tl::BN) * a.I,
              [&](int j) -> uint32_t { return (uint32_t)j * (uint32_t)(2 * a.I); }, frow_b, wave, lane);
    }
    f32x16_t acc[Tl::FM][Tl::FN];
    main_loop2<Tl, STAGES>(oa, ob, K / OA::BK, smem, wave, wm, wn, lane, acc);

    if constexpr (KIND == FC1) {
      const int cbase = t.n * (Tl::BN / 2);
      epilogue16<Tl, true>(acc, smem, wave, wm, wn, lane,
                           [&](int row, int col, const float (&g)[16], const float (&u)[16]) {
        if (row >= t.nrows) return;
        const int64_t R = t.row0 + row;
        const int wj = col / Tl::WTN, cw = col % Tl::WTN;
        const int c = cbase + wj * (Tl::WTN / 2) + (cw >> 6) * 32 + (cw & 31);
        float hv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) hv[i] = g[i] / (1.0f + expf(-g[i])) * u[i];
        store16<bf16>(a.out0 + R * I2 + c, g);
        store16<bf16>(a.out0 + R * I2 + a.I + c, u);
        store16<bf16>(a.out1 + R * a.I + c, hv);
      });
    } else if constexpr (KIND == FC2 || KIND == DX) {
      epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane,
                            [&](int row, int col, const float (&g)[16], const float (&)[16]) {
        if (row < t.nrows) store16<bf16>(a.out0 + (int64_t)s_slot[row] * a.H + t.n * Tl::BN + col, g);
      });
    } else {  // DH
      epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane,
                            [&](int row, int col, const float (&dA)[16], const float (&)[16]) {
        float part = 0.0f;
        if (row < t.nrows) {
          const int64_t R = t.row0 + row;
          const int c = t.n * Tl::BN + col;
          const float g = a.gate[s_slot[row]];
          float av[16], uv[16], hv[16], da[16], du[16];
          load16<bf16>(a.au + R * I2 + c, av);
          load16<bf16>(a.au + R * I2 + a.I + c, uv);
          load16<bf16>(a.h + R * a.I + c, hv);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            part = __builtin_fmaf(dA[i], hv[i], part);
            const float dh = g * dA[i];
            const float sg = 1.0f / (1.0f + expf(-av[i]));
            da[i] = dh * uv[i] * sg * (1.0f + av[i] * (1.0f - sg));
            du[i] = dh * av[i] * sg;
          }
          store16<bf16>(a.out0 + R * I2 + c, da);
          store16<bf16>(a.out0 + R * I2 + a.I + c, du);
        }
        const float other = __shfl_xor(part, 1);
        const float blk = (lane & 1) ? other + part : part + other;
        // one partial per 32-column block of I: the sum over blocks (router_bwd, ascending)
        // does not depend on the tile shape, the wave layout or the grid
        if ((lane & 1) == 0 && row < t.nrows)
          a.dgp[(int64_t)((t.n * Tl::BN + col) >> 5) * a.R + t.row0 + row] = blk;
      });
    }
  });
}

struct DwArgs2 {
  const int32_t* counts;
  const int32_t* offsets;
  const bf16* arows;  // dw2: dO rows [R][H]; dw1: dGU rows [R][2I]
  const bf16* brows;  // dw2: h rows [R][I];  dw1: x rows [R][H]
  void* out;
  int M, N;           // dw2: H, I; dw1: 2I, H
  int lda, ldb;       // elements per routed row of arows / brows
  Guard guard;
};

template <class Tl, typename TO>
__global__ __launch_bounds__(Tl::NT) void dw_gemm2_kernel(DwArgs2 a) {
  using OA = OpMN<Tl::BM, 32, Tl::FM, Tl::NW>;
  using OB = OpMN<Tl::BN, 32, Tl::FN, Tl::NW>;
  __shared__ __align__(1024) char smem[kDwStages * (OA::BYTES + OB::BYTES)];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int MT = a.M / Tl::BM, NT = a.N / Tl::BN;
  if (guard_fail(a.guard)) return;
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const int e = L / (MT * NT);
  const int rem = L - e * MT * NT;
  const int mt = rem / NT, nt = rem - mt * NT;
  const int seg0 = a.offsets[e], cnt = a.counts[e];
  OA oa;
  oa.init(a.arows + (int64_t)seg0 * a.lda + mt * Tl::BM, 2 * (int64_t)a.lda, cnt,
          [&](int f) { return wm * Tl::WTM + f * 32; }, wave, lane);
  OB ob;
  ob.init(a.brows + (int64_t)seg0 * a.ldb + nt * Tl::BN, 2 * (int64_t)a.ldb, cnt,
          [&](int f) { return wn * Tl::WTN + f * 32; }, wave, lane);
  f32x16_t acc[Tl::FM][Tl::FN];
  main_loop2<Tl, kDwStages>(oa, ob, (cnt + 31) / 32, smem, wave, wm, wn, lane, acc);
  TO* out = reinterpret_cast<TO*>(a.out) + ((int64_t)e * a.M + mt * Tl::BM) * a.N + nt * Tl::BN;
  epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane, [&](int row, int col, const float (&g)[16], const float (&)[16]) {
    store16<TO>(out + (int64_t)row * a.N + col, g);
  });
}

// Weight gradients with bf16 output, persistent and pipelined across output tiles:
// the ring prologue of the next tile is issued before this tile's epilogue, so the
// epilogue's stores drain while the next tile's first K-tiles load. The workgroup
// walks a contiguous range of the tile list (e, mt, nt), one range per XCD.
// When the per-wave patches fit in one ring stage they use the stage that the next
// tile's prologue leaves free (stage STAGES-1); otherwise they follow the ring.
template <class Tl>
__global__ __launch_bounds__(Tl::NT) void dw_gemm2_pipe_kernel(DwArgs2 a, int E) {
  using OA = OpMN<Tl::BM, 32, Tl::FM, Tl::NW>;
  using OB = OpMN<Tl::BN, 32, Tl::FN, Tl::NW>;
  constexpr int STAGES = 3;
  constexpr int SB = OA::BYTES + OB::BYTES;
  constexpr int PATCH = kBf16PatchBytes;
  constexpr bool IN_RING = Tl::NW * PATCH <= SB;
  constexpr int EXTRA = Tl::FM * Tl::FN * 2;  // global stores per lane in epilogue_bf16
  __shared__ __align__(1024) char smem[STAGES * SB + (IN_RING ? 0 : Tl::NW * PATCH)];
  __shared__ int s_u[kMaxE2 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  char* patch = smem + (IN_RING ? (STAGES - 1) * SB : STAGES * SB) + wave * PATCH;
  const int MT = a.M / Tl::BM, NT = a.N / Tl::BN;
  const int P = min(8, (int)gridDim.x);
  const int xcd = blockIdx.x % P;
  const int nx = ((int)gridDim.x - xcd + P - 1) / P;
  const int li = blockIdx.x / P;
  if (guard_fail(a.guard)) return;
  int64_t lo, hi;
  dw_balanced_part(E, (int64_t)MT * NT, [&](int e) { return (a.counts[e] + 31) / 32; }, s_u, P, xcd, lo, hi);
  int64_t L = lo + li;
  if (L >= hi) return;
  OA oa;
  OB ob;
  int e = 0, mt = 0, nt = 0, KT = 0;
  const auto setup = [&](int64_t l) {
    e = __builtin_amdgcn_readfirstlane((int)(l / (MT * NT)));
    const int rem = (int)(l - (int64_t)e * MT * NT);
    mt = __builtin_amdgcn_readfirstlane(rem / NT);
    nt = __builtin_amdgcn_readfirstlane(rem - mt * NT);
    const int seg0 = __builtin_amdgcn_readfirstlane(a.offsets[e]);
    const int cnt = __builtin_amdgcn_readfirstlane(a.counts[e]);
    oa.init(a.arows + (int64_t)seg0 * a.lda + mt * Tl::BM, 2 * (int64_t)a.lda, cnt,
            [&](int f) { return wm * Tl::WTM + f * 32; }, wave, lane);
    ob.init(a.brows + (int64_t)seg0 * a.ldb + nt * Tl::BN, 2 * (int64_t)a.ldb, cnt,
            [&](int f) { return wn * Tl::WTN + f * 32; }, wave, lane);
    KT = (cnt + 31) / 32;
  };
  setup(L);
  ring_prologue<STAGES>(oa, ob, KT, smem, wave);
  bool first = true;
  for (;;) {
    f32x16_t acc[Tl::FM][Tl::FN];
    if (first)
      ring_loop<Tl, STAGES, 0>(oa, ob, KT, smem, wave, lane, acc);
    else
      ring_loop<Tl, STAGES, EXTRA>(oa, ob, KT, smem, wave, lane, acc);
    bf16* out = reinterpret_cast<bf16*>(a.out) + ((int64_t)e * a.M + mt * Tl::BM) * a.N + nt * Tl::BN;
    const int64_t Ln = L + nx;
    if (Ln < hi) {
      setup(Ln);
      ring_prologue<STAGES>(oa, ob, KT, smem, wave);
    }
    epilogue_bf16<Tl>(acc, patch, wm, wn, lane,
                      [&](int row, int col, const uint4& v) { stg16_nt(out + (int64_t)row * a.N + col, v); });
    if (Ln >= hi) break;
    L = Ln;
    first = false;
  }
}

// ---------------------------------------------------------------------------
static Sched sched_of2(const Ctx& c) { return Sched{c.counts, c.offsets, c.tile_start, c.perm, c.E, c.BM, c.guard}; }

template <int KIND, int BM, int BN>
static hipError_t row_launch(const Ctx& c, const RowArgs& a, int N) {
  using Tl = RowTiling2<BM, BN>;
  int g = c.grid > 0 ? c.grid : c.num_cu;
  const int64_t upper = (int64_t)c.max_tiles * (N / BN);
  if (g > upper) g = (int)std::max<int64_t>(upper, 1);
  hipLaunchKernelGGL((row_gemm2_kernel<KIND, Tl>), dim3(g), dim3(Tl::NT), 0, c.s, a);
  return hipGetLastError();
}

template <int KIND, int BN>
static hipError_t row_bm(const Ctx& c, const RowArgs& a, int N) {
  if constexpr (BN == 512) {
    return row_launch<KIND, 128, 512>(c, a, N);  // chosen only for 128-row tiles
  } else {
    switch (c.BM) {
      case 32: return row_launch<KIND, 32, BN>(c, a, N);
      case 64: return row_launch<KIND, 64, BN>(c, a, N);
      case 128: return row_launch<KIND, 128, BN>(c, a, N);
    }
    return hipErrorInvalidValue;
  }
}

static RowArgs row_args(const Ctx& c) {
  RowArgs a{};
  a.sc = sched_of2(c);
  a.H = c.H;
  a.I = c.I;
  a.k = c.k;
  a.R = c.R;
  return a;
}

hipError_t launch_fc1_bf16(const Ctx& c, const void* x, const void* w1, void* au, void* h) {
  RowArgs a = row_args(c);
  a.a = (const bf16*)x;
  a.w = (const bf16*)w1;
  a.out0 = (bf16*)au;
  a.out1 = (bf16*)h;
  return row_bm<FC1, 256>(c, a, 2 * c.I);
}

hipError_t launch_fc2_bf16(const Ctx& c, const void* h, const void* w2, void* part) {
  RowArgs a = row_args(c);
  a.a = (const bf16*)h;
  a.w = (const bf16*)w2;
  a.out0 = (bf16*)part;
  return bn_rows(c.H) == 256 ? row_bm<FC2, 256>(c, a, c.H) : row_bm<FC2, 128>(c, a, c.H);
}

hipError_t launch_dh_bf16(const Ctx& c, const void* dy, const void* w2, const void* au, const void* h,
                          const float* gate, void* dgu, float* dgp) {
  RowArgs a = row_args(c);
  a.a = (const bf16*)dy;
  a.w = (const bf16*)w2;
  a.out0 = (bf16*)dgu;
  a.au = (const bf16*)au;
  a.h = (const bf16*)h;
  a.gate = gate;
  a.dgp = dgp;
  switch (bn_rows_bf16(c.I, c.BM)) {
    case 512: return row_bm<DH, 512>(c, a, c.I);
    case 256: return row_bm<DH, 256>(c, a, c.I);
  }
  return row_bm<DH, 128>(c, a, c.I);
}

hipError_t launch_dx_bf16(const Ctx& c, const void* dgu, const void* w1, void* part) {
  RowArgs a = row_args(c);
  a.a = (const bf16*)dgu;
  a.w = (const bf16*)w1;
  a.out0 = (bf16*)part;
  switch (bn_rows_bf16(c.H, c.BM)) {
    case 512: return row_bm<DX, 512>(c, a, c.H);
    case 256: return row_bm<DX, 256>(c, a, c.H);
  }
  return row_bm<DX, 128>(c, a, c.H);
}

template <class Tl>
static hipError_t dw_launch(const Ctx& c, const DwArgs2& a) {
  const int64_t blocks = (int64_t)c.E * (a.M / Tl::BM) * (a.N / Tl::BN);
  if (c.wgrad_f32)
    hipLaunchKernelGGL((dw_gemm2_kernel<Tl, float>), dim3((unsigned)blocks), dim3(Tl::NT), 0, c.s, a);
  else
    hipLaunchKernelGGL((dw_gemm2_kernel<Tl, bf16>), dim3((unsigned)blocks), dim3(Tl::NT), 0, c.s, a);
  return hipGetLastError();
}

static hipError_t dw_any2(const Ctx& c, const DwArgs2& a) {
  if (!c.wgrad_f32 && a.M % 256 == 0 && a.N % 256 == 0) {
    using Tl = Tiling<256, 256, 2, 4>;
    const int64_t tiles = (int64_t)c.E * (a.M / 256) * (a.N / 256);
    const int g = (int)std::min<int64_t>(c.grid > 0 ? c.grid : c.num_cu, std::max<int64_t>(tiles, 1));
    hipLaunchKernelGGL((dw_gemm2_pipe_kernel<Tl>), dim3(g), dim3(Tl::NT), 0, c.s, a, c.E);
    return hipGetLastError();
  }
  if (a.M % 256 == 0 && a.N % 256 == 0) return dw_launch<Tiling<256, 256, 2, 4>>(c, a);
  return dw_launch<Tiling<128, 128, 2, 2>>(c, a);
}

hipError_t launch_dw2_bf16(const Ctx& c, const void* dos, const void* h, void* dw2) {
  DwArgs2 a{c.counts, c.offsets, (const bf16*)dos, (const bf16*)h, dw2, c.H, c.I, c.H, c.I, c.guard};
  return dw_any2(c, a);
}

hipError_t launch_dw1_bf16(const Ctx& c, const void* dgu, const void* xs, void* dw1) {
  DwArgs2 a{c.counts, c.offsets, (const bf16*)dgu, (const bf16*)xs, dw1, 2 * c.I, c.H, 2 * c.I, c.H, c.guard};
  return dw_any2(c, a);
}

}  // namespace mok
