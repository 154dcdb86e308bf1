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
#include "elementwise.h"
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

// LDS of a row GEMM: the DMA ring (STAGES stages of A and B K-tiles)
template <int KIND, class Tl>
struct RowGemm {
  static constexpr bool K32 = Tl::BN == 512;  // 32-element K-tiles
  using OA = typename std::conditional<K32, OpK32<Tl::BM, Tl::FM, Tl::NW>, OpK<Tl::BM, Tl::FM, Tl::NW>>::type;
  static constexpr bool B_MN = KIND == DH || KIND == DX;
  using OBK = typename std::conditional<K32, OpK32<Tl::BN, Tl::FN, Tl::NW>, OpK<Tl::BN, Tl::FN, Tl::NW>>::type;
  using OB = typename std::conditional<B_MN, OpMN<Tl::BN, OA::BK, Tl::FN, Tl::NW>, OBK>::type;
  static constexpr int SB = OA::BYTES + OB::BYTES;
  // a fourth ring stage where it fits (32-row tiles: their short per-K-tile work leaves the
  // DMA latency exposed with only two K-tiles in flight)
  static constexpr int STAGES = 4 * SB + 8 * 1024 <= 160 * 1024 ? 4 : kRowStages;
  static constexpr int SMEM = STAGES * SB;
};

// One row GEMM over the schedule's tiles, walked by workgroup wg of nwg. smem: RowGemm::SMEM
// bytes (1 KB aligned); s_ts: E + 1 ints; s_slot: BM ints.
template <int KIND, class Tl>
__device__ __forceinline__ void row_gemm2_body(const RowArgs& a, char* smem, int* s_ts, int* s_slot, int wg, int nwg) {
  using G = RowGemm<KIND, Tl>;
  using OA = typename G::OA;
  using OB = typename G::OB;
  constexpr bool B_MN = G::B_MN;
  constexpr int STAGES = G::STAGES;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int I2 = 2 * a.I;
  // N of the GEMM and its tile count; K
  const int N = KIND == FC1 ? I2 : (KIND == FC2 || KIND == DX ? a.H : a.I);
  const int K = KIND == FC1 || KIND == DH ? a.H : (KIND == FC2 ? a.I : I2);
  load_tile_start(a.sc, s_ts);
  for_each_row_tile(a.sc, s_ts, N / Tl::BN, wg, nwg, [&](const RowTile& t) {
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

template <int KIND, class Tl>
__global__ __launch_bounds__(Tl::NT) void row_gemm2_kernel(RowArgs a) {
  __shared__ __align__(1024) char smem[RowGemm<KIND, Tl>::SMEM];
  __shared__ int s_ts[kMaxE2 + 1];
  __shared__ int s_slot[Tl::BM];
  row_gemm2_body<KIND, Tl>(a, smem, s_ts, s_slot, blockIdx.x, gridDim.x);
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

// LDS of one weight-gradient tile (4-deep ring of MN-contiguous K-tiles)
template <class Tl>
struct DwGemm {
  using OA = OpMN<Tl::BM, 32, Tl::FM, Tl::NW>;
  using OB = OpMN<Tl::BN, 32, Tl::FN, Tl::NW>;
  static constexpr int SMEM = kDwStages * (OA::BYTES + OB::BYTES);
};

// Output tile L (expert-major, then M-tile, N-tile) of a weight-gradient GEMM.
template <class Tl, typename TO>
__device__ __forceinline__ void dw_gemm2_body(const DwArgs2& a, char* smem, int L) {
  using OA = typename DwGemm<Tl>::OA;
  using OB = typename DwGemm<Tl>::OB;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int MT = a.M / Tl::BM, NT = a.N / Tl::BN;
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

template <class Tl, typename TO>
__global__ __launch_bounds__(Tl::NT) void dw_gemm2_kernel(DwArgs2 a) {
  __shared__ __align__(1024) char smem[DwGemm<Tl>::SMEM];
  if (guard_fail(a.guard)) return;
  dw_gemm2_body<Tl, TO>(a, smem, xcd_logical(blockIdx.x, gridDim.x));
}

// Weight gradients with bf16 output, persistent and pipelined across output tiles:
// the ring prologue of the next tile is issued before this tile's epilogue, so the
// epilogue's stores drain while the next tile's first K-tiles load.
// When the per-wave patches fit in one ring stage they use the stage that the next
// tile's prologue leaves free (stage STAGES-1); otherwise they follow the ring.
//
// Q = false (large launches): the workgroup walks a contiguous range of the tile list
// (e, mt, nt), one range per XCD, split by work (dw_balanced_part).
// Q = true (launches of a few tiles per workgroup, where one expert with many rows makes
// tiles several times longer than the others): the tiles are listed longest K first and
// dealt round-robin to P parts (list position p goes to part p % P); a part's tiles go
// out one at a time from its queue line in the schedule header, in list order, each
// workgroup's first one by its index. A workgroup claims its next tile three K-tiles
// before the end of the current one, so the claim's latency hides behind the last
// K-tiles and the next tile's prologue still precedes this tile's epilogue. Greedy
// longest-first assignment keeps a hot expert's tiles from queueing behind one another
// (2048 tokens, experts 8x the mean: in a model of the walk, the busiest workgroup's
// K-tiles 59 -> 36 for dW1, 41 -> 36 for dW2). The last workgroup of a part to stop
// claiming zeroes the part's line for the next launch. Which workgroup computes a tile
// never changes its bits.
template <class Tl, bool Q>
__global__ __launch_bounds__(Tl::NT) void dw_gemm2_pipe_kernel(DwArgs2 a, int E) {
  using OA = OpMN<Tl::BM, 32, Tl::FM, Tl::NW>;
  using OB = OpMN<Tl::BN, 32, Tl::FN, Tl::NW>;
  constexpr int STAGES = 3;
  constexpr int SB = OA::BYTES + OB::BYTES;
  constexpr int PATCH = kBf16PatchBytes;
  constexpr bool IN_RING = Tl::NW * PATCH <= SB;
  constexpr int EXTRA = Tl::FM * Tl::FN * 2;  // global stores per lane in epilogue_bf16
  static_assert(!Q || STAGES * SB >= 4 * kDwQueueMaxE, "the ring holds the order scratch");
  __shared__ __align__(1024) char smem[STAGES * SB + (IN_RING ? 0 : Tl::NW * PATCH)];
  __shared__ int s_u[kMaxE2 + 1];
  __shared__ int s_next;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  char* patch = smem + (IN_RING ? (STAGES - 1) * SB : STAGES * SB) + wave * PATCH;
  const int MT = a.M / Tl::BM, NT = a.N / Tl::BN;
  const int64_t TPE = (int64_t)MT * NT;
  const int P = min(8, (int)gridDim.x);
  const int xcd = blockIdx.x % P;
  const int nx = ((int)gridDim.x - xcd + P - 1) / P;
  const int li = blockIdx.x / P;
  if (guard_fail(a.guard)) return;
  const auto kt_of = [&](int e) { return (a.counts[e] + 31) / 32; };
  int32_t* qline = nullptr;
  int64_t L, hi;
  if constexpr (Q) {
    dw_lpt_order(E, kt_of, reinterpret_cast<int*>(smem), s_u);
    qline = dw_queue_line(a.guard.hdr, xcd);
    hi = ((int64_t)E * TPE - xcd + P - 1) / P;  // this part's tiles: list positions xcd + P q, q < hi
    L = li;
    if (L >= hi) {
      dw_queue_leave(qline, nx);
      return;
    }
  } else {
    int64_t lo;
    dw_balanced_part(E, TPE, kt_of, s_u, P, xcd, lo, hi);
    L = lo + li;
    if (L >= hi) return;
  }
  OA oa;
  OB ob;
  int e = 0, mt = 0, nt = 0, KT = 0;
  const auto setup = [&](int64_t l) {
    int rem;
    if constexpr (Q) {
      const int64_t pos = xcd + (int64_t)P * l;
      const int i = (int)(pos / TPE);
      e = __builtin_amdgcn_readfirstlane(s_u[i]);
      rem = (int)(pos - (int64_t)i * TPE);
    } else {
      e = __builtin_amdgcn_readfirstlane((int)(l / TPE));
      rem = (int)(l - (int64_t)e * TPE);
    }
    dw_tile_order(rem, MT, NT, mt, nt);
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
    int claim = 0;  // lane 0 of wave 0: the part's next queue index
    const int kc = KT > 3 ? KT - 3 : 0;
    const auto hook = [&](int kt) {
      if (Q && kt == kc && tid == 0) claim = dw_queue_claim(qline);
    };
    if (Q && KT == 0 && tid == 0) claim = dw_queue_claim(qline);
    if (first)
      ring_loop<Tl, STAGES, 0, true>(oa, ob, KT, smem, wave, lane, acc, hook);
    else
      ring_loop<Tl, STAGES, EXTRA, true>(oa, ob, KT, smem, wave, lane, acc, hook);
    bf16* out = reinterpret_cast<bf16*>(a.out) + ((int64_t)e * a.M + mt * Tl::BM) * a.N + nt * Tl::BN;
    int64_t Ln;
    if constexpr (Q) {
      asm volatile("" : "+v"(claim));  // the claim is read here, after the K-loop
      if (tid == 0) s_next = claim;
      __syncthreads();
      Ln = nx + (int64_t)__builtin_amdgcn_readfirstlane(s_next);
    } else {
      Ln = L + nx;
    }
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
  if constexpr (Q) dw_queue_leave(qline, nx);
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

// Persistent weight-gradient launch: one workgroup per CU for 256 x 256 tiles, two for
// 128 x 128 tiles (whose 76 KB of LDS let two share a CU).
template <class Tl>
static hipError_t dw_pipe_launch(const Ctx& c, const DwArgs2& a) {
  const int64_t tiles = (int64_t)c.E * (a.M / Tl::BM) * (a.N / Tl::BN);
  const int per_cu = Tl::BM == 128 ? 2 : 1;
  const int g = (int)std::min<int64_t>(c.grid > 0 ? c.grid : per_cu * c.num_cu, std::max<int64_t>(tiles, 1));
  // tile queues for the 128 x 128 launches (a few tiles per workgroup), with a schedule
  // header to hold them
  if constexpr (Tl::BM == 128) {
    if (c.E <= kDwQueueMaxE && a.guard.hdr != nullptr) {
      hipLaunchKernelGGL((dw_gemm2_pipe_kernel<Tl, true>), dim3(g), dim3(Tl::NT), 0, c.s, a, c.E);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((dw_gemm2_pipe_kernel<Tl, false>), dim3(g), dim3(Tl::NT), 0, c.s, a, c.E);
  return hipGetLastError();
}

static hipError_t dw_any2(const Ctx& c, const DwArgs2& a) {
  if (!c.wgrad_f32 && a.M % 256 == 0 && a.N % 256 == 0) {
    // 256 x 256 tiles when they give at least eight waves over the CUs, else 128 x 128
    // tiles: four times as many, so a hot expert's long K is spread over four times the
    // workgroups (2048 tokens, Zipf routing: dW1 0.040 -> 0.038 ms, dW2 0.036 -> 0.027;
    // near-uniform: 0.031 -> 0.028, 0.025 -> 0.021). Every output element is summed over
    // all of K by one wave in the same order under either tiling: the bits do not change.
    if ((int64_t)c.E * (a.M / 256) * (a.N / 256) >= 8 * (int64_t)c.num_cu)
      return dw_pipe_launch<Tiling<256, 256, 2, 4>>(c, a);
    return dw_pipe_launch<Tiling<128, 128, 2, 2>>(c, a);
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

// ---------------------------------------------------------------------------
// Fused persistent kernels: the stages of the forward (or backward) pass in one launch,
// one workgroup per compute unit, separated by a grid barrier instead of kernel
// boundaries -- the pages' single megakernel for the layer (aikraft.ru MoK article,
// section 01), on one GPU. Every stage is the body of the separate kernel with the same
// tiling and summation order, so the outputs are the separate path's bits (tested); the
// weight gradients use 128 x 128 tiles, whose per-element sums are the same as the 256 x
// 256 tiles' (every output element is summed by one wave over all of K, in order).
// The grid is one workgroup per compute unit, all resident at once unless another kernel
// holds compute units during the launch; the waits are bounded for that case: after
// kFusedSpinLimit polls a workgroup records MOK_ERR_HIP in the schedule header's status
// word and goes on, so every wave exits.
//
// The barrier is hierarchical over the XCDs, because making a stage's results visible
// to the other XCDs means writing back the XCD's L2, and one write-back per workgroup
// (a release on every arrival) stalls the workgroups still working on the stage. Each
// wave first waits for its own stores (acknowledged by its XCD's L2); the workgroup then
// counts itself in its XCC's arrival line; the last of an XCC writes that XCC's L2 back
// (a release fence at agent scope) and counts the XCC in the global line; the last XCC
// stores the new generation into every XCC's release line, which that XCC's workgroups
// poll with relaxed loads (an acquire on every poll would invalidate the L2 under the
// workgroups still working); one acquire fence follows the wait. Which XCC a workgroup
// runs on is read from the hardware (HW_REG_XCC_ID); a start barrier counts the
// workgroups of each XCC once per launch.
constexpr uint32_t kFusedSpinLimit = 1u << 22;
constexpr int kFusedThreads = 256;
constexpr int kFusedMinLds = 81 * 1024;  // more than half a CU's 160 KB: one workgroup per CU

struct FusedSync {
  int32_t* hdr;
  int nwg, xcc, members, nxcc, mask, gen;  // mask: the XCCs that hold workgroups
};

__device__ __forceinline__ int32_t* sync_line(int32_t* hdr, int i) { return hdr + i * kSyncLine; }

__device__ __forceinline__ int hw_xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return (int)(v & (kSyncXcc - 1));
}

// Polls *p until it reaches `target`; false after kFusedSpinLimit polls (status recorded).
__device__ __forceinline__ bool sync_wait(int32_t* hdr, const int32_t* p, int target) {
  uint32_t spins = 0;
  while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kFusedSpinLimit) {
      hdr[kHdrStatus] = MOK_ERR_HIP;
      return false;
    }
  }
  return true;
}

// Start barrier: every workgroup counts itself on its XCC's line and polls the sum of
// the XCC counts until it reaches the grid size; the counts are then final. No data is
// published here (the stages' inputs come from earlier launches), so no fences.
__device__ __forceinline__ bool fused_start(FusedSync& fs, int32_t* hdr) {
  __shared__ int s_v[4];
  fs.hdr = hdr;
  fs.nwg = gridDim.x;
  fs.gen = 0;
  if (threadIdx.x == 0) {
    const int x = hw_xcc_id();
    __hip_atomic_fetch_add(sync_line(hdr, kSyncArrive + x) + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int cnt[kSyncXcc];
    bool ok = false;
    for (uint32_t spins = 0; spins <= kFusedSpinLimit; ++spins) {
      int sum = 0;
#pragma unroll
      for (int y = 0; y < kSyncXcc; ++y) {
        cnt[y] = __hip_atomic_load(sync_line(hdr, kSyncArrive + y) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sum += cnt[y];
      }
      if (sum >= fs.nwg) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (!ok) hdr[kHdrStatus] = MOK_ERR_HIP;
    int n = 0, mask = 0, mine = 0;
#pragma unroll
    for (int y = 0; y < kSyncXcc; ++y) {
      n += cnt[y] > 0;
      mask |= (cnt[y] > 0) << y;
      mine = y == x ? cnt[y] : mine;
    }
    s_v[0] = x;
    s_v[1] = mine;
    s_v[2] = ok ? n : 0;
    s_v[3] = mask;
  }
  __syncthreads();
  fs.xcc = s_v[0];
  fs.members = s_v[1];
  fs.nxcc = s_v[2];
  fs.mask = s_v[3];
  return fs.nxcc > 0;
}

__device__ __forceinline__ bool fused_barrier(FusedSync& fs) {
  __shared__ int s_ok;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have reached the XCD's L2
  __syncthreads();
  ++fs.gen;
  if (threadIdx.x == 0) {
    int32_t* hdr = fs.hdr;
    int32_t* l1 = sync_line(hdr, 1);
    const int old = __hip_atomic_fetch_add(sync_line(hdr, kSyncArrive + fs.xcc), 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    if (old == fs.gen * fs.members - 1) {  // last on this XCC: publish the XCC's L2
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const int oldx = __hip_atomic_fetch_add(l1 + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (oldx == fs.gen * fs.nxcc - 1) {  // last XCC: release every XCC
        for (int y = 0; y < kSyncXcc; ++y)
          if (fs.mask >> y & 1)
            __hip_atomic_store(sync_line(hdr, kSyncRelease + y), fs.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    s_ok = sync_wait(hdr, sync_line(hdr, kSyncRelease + fs.xcc), fs.gen);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return s_ok != 0;
}

// Work items [0, n) handed out one at a time by an atomic counter (queue line q), so that
// workgroups that finished their share of the stage's GEMM tiles early take more of the
// rest. Each item is done whole by one workgroup, so the results do not depend on which
// one takes it. The next item is claimed while this one runs. body(i) must end with the
// workgroup's threads done with shared memory it used.
template <class F>
__device__ __forceinline__ void queue_items(const FusedSync& fs, int q, int64_t n, F&& body) {
  __shared__ int s_item;
  int32_t* ctr = sync_line(fs.hdr, kSyncQueue + q);
  __syncthreads();
  if (threadIdx.x == 0) s_item = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  int64_t i = s_item;
  while (i < n) {
    int next = 0;
    if (threadIdx.x == 0) next = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    body(i);
    __syncthreads();
    if (threadIdx.x == 0) s_item = next;
    __syncthreads();
    i = s_item;
  }
}

// The last workgroup to leave zeroes the barrier lines for the next launch (kernel
// completion publishes them): exits are counted per XCC, then per grid. Every other
// workgroup counts its exit after its last poll, so nothing reads the lines once the
// count is complete. The counts are relaxed: a fence here would write back and
// invalidate the L2 under workgroups still in the last stage.
__device__ __forceinline__ void fused_exit(const FusedSync& fs) {
  __syncthreads();
  if (threadIdx.x == 0 && fs.nxcc > 0) {
    const int old = __hip_atomic_fetch_add(sync_line(fs.hdr, kSyncArrive + fs.xcc) + 2, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    if (old == fs.members - 1 &&
        __hip_atomic_fetch_add(sync_line(fs.hdr, 1) + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == fs.nxcc - 1)
      sync_zero(fs.hdr);
  }
}

struct FwdFusedArgs {
  RowArgs fc1, fc2;
  const bf16* part;
  const float* gate;
  bf16* y;
  int64_t T;
  int H, k;
};

template <int BNH>
__global__ __launch_bounds__(kFusedThreads) void forward_fused_kernel(FwdFusedArgs a) {
  using T1 = RowTiling2<32, 256>;
  using T2 = RowTiling2<32, BNH>;
  static_assert(T1::NT == kFusedThreads && T2::NT == kFusedThreads, "one block size for every stage");
  constexpr int SMEM = RowGemm<FC1, T1>::SMEM > RowGemm<FC2, T2>::SMEM ? RowGemm<FC1, T1>::SMEM
                                                                       : RowGemm<FC2, T2>::SMEM;
  __shared__ __align__(1024) char smem[SMEM < kFusedMinLds ? kFusedMinLds : SMEM];
  __shared__ int s_ts[kMaxE2 + 1];
  __shared__ int s_slot[32];
  if (guard_fail(a.fc1.sc.guard)) return;  // uniform over the grid: no workgroup reaches a barrier
  const int wg = blockIdx.x, nwg = gridDim.x;
  FusedSync fs;
  if (fused_start(fs, a.fc1.sc.guard.hdr)) {
  row_gemm2_body<FC1, T1>(a.fc1, smem, s_ts, s_slot, wg, nwg);
  if (fused_barrier(fs)) {
    row_gemm2_body<FC2, T2>(a.fc2, smem, s_ts, s_slot, wg, nwg);
    if (fused_barrier(fs)) {
      const int64_t n = a.T * (a.H / 8);
      for (int64_t g = (int64_t)wg * kFusedThreads + threadIdx.x; g < n; g += (int64_t)nwg * kFusedThreads)
        combine_body(a.part, a.gate, a.y, a.T, a.H, a.k, g);
    }
  }
  }
  fused_exit(fs);
}

struct BwdFusedArgs {
  RowArgs dh, dx;
  DwArgs2 dw2, dw1;
  const bf16* x;
  const bf16* dy;
  const int32_t* idx;
  const int32_t* perm;
  const int32_t* inv;
  const int32_t* offsets;
  const float* gate;
  const bf16* wr;
  const float* dgp;
  float* dgate;
  float* dz;
  bf16* xs;
  bf16* dos;
  const bf16* bpart;
  bf16* dxo;
  bf16* dwr;
  int64_t T;
  int H, I, E, k, R;
};

// dgate and dz for a chunk of tokens per workgroup, chunks spread over the grid: the
// workgroup loads the chunk's d-gate partials (k slots x I/32 blocks per token) into LDS
// at once, then each slot sums its partials in ascending block order (as
// router_gsum_body) and each token forms dz from its slots (as router_dz_body).
__device__ __forceinline__ void router_bwd_stage(const BwdFusedArgs& a, float* red, int wg, int nwg) {
  const int tid = threadIdx.x;
  const int nb = dgate_parts(a.I), kn = a.k * nb;
  const int tpc = kn >= kFusedThreads ? 1 : kFusedThreads / kn;  // tokens per chunk
  float* gp = red + tpc * kn;                                     // the chunk's g' values
  const int64_t chunks = (a.T + tpc - 1) / tpc;
  for (int64_t c = wg; c < chunks; c += nwg) {
    const int64_t t0 = c * tpc;
    const int nt = (int)min<int64_t>(tpc, a.T - t0);
    __syncthreads();
    for (int v = tid; v < nt * kn; v += kFusedThreads) {
      const int tt = v / kn, rem = v - tt * kn, j = rem / nb, n = rem - j * nb;
      const int r = a.inv[(t0 + tt) * a.k + j];
      red[v] = a.dgp[(int64_t)n * a.R + r];
    }
    __syncthreads();
    for (int q = tid; q < nt * a.k; q += kFusedThreads) {
      float v = 0.0f;
      for (int n = 0; n < nb; ++n) v += red[q * nb + n];
      gp[q] = v;
      a.dgate[t0 * a.k + q] = v;
    }
    __syncthreads();
    for (int tt = tid; tt < nt; tt += kFusedThreads) {
      const int64_t s0 = (t0 + tt) * a.k;
      router_dz_token(a.gate + s0, gp + tt * a.k, a.dz + s0, a.k);
    }
  }
}

template <int BNH, int BNI>
__global__ __launch_bounds__(kFusedThreads) void backward_fused_kernel(BwdFusedArgs a) {
  using TH = RowTiling2<32, BNI>;  // dh: N = I
  using TX = RowTiling2<32, BNH>;  // dx: N = H
  using TW = Tiling<128, 128, 2, 2>;
  static_assert(TH::NT == kFusedThreads && TX::NT == kFusedThreads && TW::NT == kFusedThreads, "block size");
  constexpr int S1 = RowGemm<DH, TH>::SMEM > RowGemm<DX, TX>::SMEM ? RowGemm<DH, TH>::SMEM : RowGemm<DX, TX>::SMEM;
  constexpr int SMEM = S1 > DwGemm<TW>::SMEM ? S1 : DwGemm<TW>::SMEM;
  static_assert(SMEM >= 64 * 33 * 4 && SMEM >= 32 * 65 * 4, "dWr reduction fits");
  static_assert(SMEM >= (kFusedMaxSlotParts + kFusedThreads) * 4, "router chunk fits");
  __shared__ __align__(1024) char smem[SMEM < kFusedMinLds ? kFusedMinLds : SMEM];
  __shared__ int s_ts[kMaxE2 + 1];
  __shared__ int s_slot[32];
  if (guard_fail(a.dh.sc.guard)) return;
  const int wg = blockIdx.x, nwg = gridDim.x, tid = threadIdx.x;
  const int64_t stride = (int64_t)nwg * kFusedThreads, g0 = (int64_t)wg * kFusedThreads + tid;
  FusedSync fs;
  if (fused_start(fs, a.dh.sc.guard.hdr)) {
  // S1: dH GEMM (SwiGLU backward, d-gate partials); token rows in routed order for dW
  row_gemm2_body<DH, TH>(a.dh, smem, s_ts, s_slot, wg, nwg);
  {
    constexpr int PER = 8;  // 16-byte vectors per thread and item
    const int64_t ng = (int64_t)a.R * (a.H / 8);
    queue_items(fs, 0, (ng + PER * kFusedThreads - 1) / (PER * kFusedThreads), [&](int64_t it) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int64_t g = (it * PER + u) * kFusedThreads + tid;
        gather_rows_body(a.dy, a.perm, a.gate, a.dos, a.R, a.H, a.k, g);
        gather_rows_body(a.x, a.perm, nullptr, a.xs, a.R, a.H, a.k, g);
      }
    });
  }
  if (fused_barrier(fs)) {
    // S2: router backward per token
    router_bwd_stage(a, reinterpret_cast<float*>(smem), wg, nwg);
    if (fused_barrier(fs)) {
      // S3: dX partials, weight gradients, dWr
      row_gemm2_body<DX, TX>(a.dx, smem, s_ts, s_slot, wg, nwg);
      // weight-gradient tiles, then the dWr items, from one queue
      const int n2 = a.E * (a.H / 128) * (a.I / 128), n1 = a.E * (2 * a.I / 128) * (a.H / 128);
      const bool small_h = a.H <= 2048;
      const int nvb = small_h ? (a.H / 8 + 3) / 4 : (a.H / 8 + 7) / 8;
      const int nr = a.dwr != nullptr ? a.E * nvb : 0;
      float* red = reinterpret_cast<float*>(smem);
      queue_items(fs, 1, (int64_t)n2 + n1 + nr, [&](int64_t it) {
        const int L = (int)it;
        if (L < n2) {
          dw_gemm2_body<TW, bf16>(a.dw2, smem, L);
        } else if (L < n2 + n1) {
          dw_gemm2_body<TW, bf16>(a.dw1, smem, L - n2);
        } else if (small_h) {
          dwr_body<bf16, bf16, 4, 64>(a.dz, a.x, a.offsets, a.perm, a.dwr, a.E, a.H, a.k, L - n2 - n1, red);
        } else {
          dwr_body<bf16, bf16, 8, 32>(a.dz, a.x, a.offsets, a.perm, a.dwr, a.E, a.H, a.k, L - n2 - n1, red);
        }
      });
      if (fused_barrier(fs)) {
        // S4: dX = slot-order sum of the partials + router term
        const int64_t n = a.T * (a.H / 8);
        for (int64_t g = g0; g < n; g += stride)
          dx_reduce_body(a.bpart, a.dz, a.idx, a.wr, a.dxo, a.T, a.H, a.k, g);
      }
    }
  }
  }
  fused_exit(fs);
}

static int fused_grid(const Ctx& c) { return c.grid > 0 && c.grid < c.num_cu ? c.grid : c.num_cu; }

// An ordinary launch: with one workgroup per compute unit (the LDS of one fills a CU) and
// the stream's earlier kernels finished, every workgroup is resident at once. (A
// cooperative launch guarantees that too, and costs about 20 us more per launch.)
template <class K, class A>
static hipError_t launch_coop(K kernel, const Ctx& c, A& args) {
  hipLaunchKernelGGL(kernel, dim3(fused_grid(c)), dim3(kFusedThreads), 0, c.s, args);
  return hipGetLastError();
}

hipError_t launch_forward_fused(const Ctx& c, const void* x, const void* w1, const void* w2, void* au, void* h,
                                void* part, const float* gate, void* y) {
  if (c.BM != 32 || c.act != MOK_BF16 || c.E > kMaxE2) return hipErrorInvalidValue;
  FwdFusedArgs a{};
  a.fc1 = row_args(c);
  a.fc1.a = (const bf16*)x;
  a.fc1.w = (const bf16*)w1;
  a.fc1.out0 = (bf16*)au;
  a.fc1.out1 = (bf16*)h;
  a.fc2 = row_args(c);
  a.fc2.a = (const bf16*)h;
  a.fc2.w = (const bf16*)w2;
  a.fc2.out0 = (bf16*)part;
  a.part = (const bf16*)part;
  a.gate = gate;
  a.y = (bf16*)y;
  a.T = c.T;
  a.H = c.H;
  a.k = c.k;
  return bn_rows(c.H) == 256 ? launch_coop(forward_fused_kernel<256>, c, a)
                             : launch_coop(forward_fused_kernel<128>, c, a);
}

hipError_t launch_backward_fused(const Ctx& c, const void* x, const int32_t* idx, const float* gate, const void* w1,
                                 const void* w2, const void* wr, const void* au, const void* h, const void* dy,
                                 void* dgu, void* bpart, float* dgp, float* dz, void* xs, void* dos, void* dx,
                                 void* dw1, void* dw2, float* dgate, void* dwr) {
  if (c.BM != 32 || c.act != MOK_BF16 || c.wgrad_f32 || c.E > kMaxE2) return hipErrorInvalidValue;
  BwdFusedArgs a{};
  a.dh = row_args(c);
  a.dh.a = (const bf16*)dy;
  a.dh.w = (const bf16*)w2;
  a.dh.out0 = (bf16*)dgu;
  a.dh.au = (const bf16*)au;
  a.dh.h = (const bf16*)h;
  a.dh.gate = gate;
  a.dh.dgp = dgp;
  a.dx = row_args(c);
  a.dx.a = (const bf16*)dgu;
  a.dx.w = (const bf16*)w1;
  a.dx.out0 = (bf16*)bpart;
  a.dw2 = DwArgs2{c.counts, c.offsets, (const bf16*)dos, (const bf16*)h, dw2, c.H, c.I, c.H, c.I, c.guard};
  a.dw1 = DwArgs2{c.counts, c.offsets, (const bf16*)dgu, (const bf16*)xs, dw1, 2 * c.I, c.H, 2 * c.I, c.H, c.guard};
  a.x = (const bf16*)x;
  a.dy = (const bf16*)dy;
  a.idx = idx;
  a.perm = c.perm;
  a.inv = c.inv;
  a.offsets = c.offsets;
  a.gate = gate;
  a.wr = (const bf16*)wr;
  a.dgp = dgp;
  a.dgate = dgate;
  a.dz = dz;
  a.xs = (bf16*)xs;
  a.dos = (bf16*)dos;
  a.bpart = (const bf16*)bpart;
  a.dxo = (bf16*)dx;
  a.dwr = (bf16*)dwr;
  a.T = c.T;
  a.H = c.H;
  a.I = c.I;
  a.E = c.E;
  a.k = c.k;
  a.R = c.R;
  const bool h256 = bn_rows(c.H) == 256, i256 = bn_rows(c.I) == 256;
  if (h256 && i256) return launch_coop(backward_fused_kernel<256, 256>, c, a);
  if (h256) return launch_coop(backward_fused_kernel<256, 128>, c, a);
  if (i256) return launch_coop(backward_fused_kernel<128, 256>, c, a);
  return launch_coop(backward_fused_kernel<128, 128>, c, a);
}

}  // namespace mok
