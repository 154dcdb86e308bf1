// MX grouped expert GEMMs: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 x E4M3 (MXFP8)
// or E2M1 x E2M1 (MXFP4) operands, one E8M0 scale per 32 K-elements of every row of A
// and B, fp32 accumulation (expert GEMMs in MXFP8, dothoosh.com MoK page, "Technical
// details of the MoK mechanism"; MXFP4 as the narrower format of aikraft.ru MoK
// article, section 03). The template parameter F picks the element format (MxFmt).
//
// Every operand is K-contiguous in HBM (the weights are pre-quantised in the
// orientation each GEMM reads; the token-axis operands of the weight gradients are
// quantised transposed), so one operand type serves all six GEMMs: the direct-to-
// LDS K-contiguous tile of the bf16 core (OpK: 128-byte tile rows, here 128 E4M3
// elements per K-tile) plus the rows' scale dwords (4 scale bytes = the 4 blocks of
// the K-tile), DMA'd into the same ring stage.
//
// Operand lane layout of the 32x32x64 instruction (E4M3): lane l (half h = l/32)
// holds row l%32, bytes 0..15 = k 16h..16h+15 and bytes 16..31 = k 32+16h..32+16h+15
// of the 64-k step; the scale of row i for k-block q (k 32q..32q+31) comes from lane
// i + 32q, byte `opsel` of its scale operand. In a 128-byte tile row the 64-k step ks
// is chunks 4ks..4ks+3, so lane half h reads chunks 4ks+h and 4ks+2+h (OpK::frag
// positions 2ks and 2ks+1) and scale byte 2ks+h of the row's dword (shifted down by
// 8h, opsel 2ks).
//
// E2M1 (pinned by an in-bounds probe against a CPU model with per-block scales): lane l
// (half h) holds row l%32's k-block h (k 32h..32h+31) as 16 bytes, two codes per byte;
// the scale of row i for k-block q again comes from lane i + 32q. A 128-byte tile row is
// 256 elements (4 steps of 64); step ks is chunks 2ks and 2ks+1, lane half h reads chunk
// 2ks+h (OpK::frag position ks), and its scale byte 2ks+h of the K-tile's 8 is byte
// 2(ks%2)+h of scale dword ks/2 (shifted down by 8h, opsel 2(ks%2)).
#include "gemm2.h"
#include "kernels.h"
#include "mx.h"

namespace mok {

typedef int v8i32_t __attribute__((ext_vector_type(8)));

constexpr int kMaxEx = 1024;
constexpr int kMxStages = 3;

// One-dword-per-lane DMA: lane l's 4 bytes land at LDS base + 4*l.
__device__ __forceinline__ void dma4_sv(const char* sbase, uint32_t voff, char* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(l), "v"(voff), "s"(sbase) : "memory", "m0");
}

// Scale dwords of ROWS tile rows per K-tile: SD per row (one per 128 elements of the
// K-tile). Wave w loads rows [w*RPW, (w+1)*RPW) with lanes 0..RPW-1 (SD DMA
// instructions per wave per stage, RPW >= 8 so each always has active lanes). The
// dwords of 128-element slab j sit j * kstride bytes after slab 0's: 4 for row-major
// scales; the matrix's rows * 4 for K-tile-major ones, whose dwords for consecutive
// rows are contiguous (one 128-byte request per 32 rows instead of one per row).
template <int ROWS, int NF, int NW, int SD = 1>
struct OpScale {
  static constexpr int RPW = ROWS / NW;
  static_assert(ROWS % NW == 0 && RPW >= 8 && RPW <= 64, "scale rows per wave");
  static constexpr int BYTES = SD * ROWS * 4;
  const char* sbase;
  uint32_t voff;
  uint32_t kstride;
  uint32_t foff[NF];
  bool active;

  // rowoff(row) -> byte offset of the row's K-tile-0 scale dword from sbase_ (< 2 GiB)
  template <class F, class G>
  __device__ __forceinline__ void init(const void* sbase_, F rowoff, G frow, int wave, int lane,
                                       uint32_t kstride_ = 4) {
    sbase = reinterpret_cast<const char*>(sbase_);
    kstride = kstride_;
    active = lane < RPW;
    voff = rowoff(wave * RPW + (active ? lane : 0));
#pragma unroll
    for (int f = 0; f < NF; ++f) foff[f] = 4u * (uint32_t)(frow(f) + (lane & 31));
  }
  __device__ __forceinline__ void issue(int kt, char* stage, int wave) const {
#pragma unroll
    for (int d = 0; d < SD; ++d) {
      const char* b = uniform_ptr(sbase + (int64_t)(SD * kt + d) * kstride);
      if (active) dma4_sv(b, voff, stage + d * ROWS * 4 + wave * RPW * 4);
    }
  }
  __device__ __forceinline__ uint32_t get(const char* stage, int f, int lane, int d = 0) const {
    return *reinterpret_cast<const uint32_t*>(stage + d * ROWS * 4 + foff[f]) >> (8 * (lane >> 5));
  }
};

__device__ __forceinline__ v8i32_t join8(const uint4& lo, const uint4& hi) {
  v8i32_t v;
  v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
  v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
  return v;
}

// One 64-k step of the K-tile in `cur`. E4M3: 32 bytes per lane (frag positions 2KS,
// 2KS+1), opsel = byte 2*KS of scale dword 0. E2M1: 16 bytes per lane (frag position KS;
// the instruction reads the low 4 dwords), opsel = byte 2*(KS%2) of scale dword KS/2.
// TR: operands (and their scales) swapped, giving transposed blocks with the same bits.
template <int F, int KS, bool TR, class Tl, class OA, class OB>
__device__ __forceinline__ void mx_kstep(const OA& oa, const OB& ob, const char* ca, const char* cb,
                                         const uint32_t (&xa)[MxFmt<F>::SD][Tl::FM],
                                         const uint32_t (&xb)[MxFmt<F>::SD][Tl::FN], f32x16_t (&acc)[Tl::FM][Tl::FN]) {
  constexpr int FMT = F == 0 ? 0 : 4;  // cbsz / blgp: E4M3 or E2M1
  constexpr int D = F == 0 ? 0 : KS / 2, OP = F == 0 ? 2 * KS : 2 * (KS % 2);
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  v8i32_t a[Tl::FM], b[Tl::FN];
#pragma unroll
  for (int fm = 0; fm < Tl::FM; ++fm)
    a[fm] = F == 0 ? join8(oa.frag(ca, fm, 2 * KS), oa.frag(ca, fm, 2 * KS + 1)) : join8(oa.frag(ca, fm, KS), z);
#pragma unroll
  for (int fn = 0; fn < Tl::FN; ++fn)
    b[fn] = F == 0 ? join8(ob.frag(cb, fn, 2 * KS), ob.frag(cb, fn, 2 * KS + 1)) : join8(ob.frag(cb, fn, KS), z);
#pragma unroll
  for (int fm = 0; fm < Tl::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < Tl::FN; ++fn)
      if constexpr (TR)
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[fn], a[fm], acc[fm][fn], FMT, FMT, OP,
                                                                      (int)xb[D][fn], OP, (int)xa[D][fm]);
      else
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[fm], b[fn], acc[fm][fn], FMT, FMT, OP,
                                                                      (int)xa[D][fm], OP, (int)xb[D][fn]);
}

// STAGES-deep ring as in the bf16 core; a stage holds A rows, B rows, A scales, B scales.
// Split like the bf16 core's ring_prologue / ring_loop: the prologue issues the first
// STAGES-1 K-tiles; the loop's waits for those K-tiles may leave EXTRA younger global
// stores per lane outstanding (a persistent kernel's previous epilogue), while any later
// K-tile, issued after those stores, covers them (vector memory completes in order).
template <int STAGES, class OA, class OB, class SA, class SB>
__device__ __forceinline__ void mx_ring_prologue(const OA& oa, const OB& ob, const SA& sa, const SB& sb, int KT,
                                                 char* smem, int wave) {
  constexpr int OFF_B = OA::BYTES, OFF_SA = OA::BYTES + OB::BYTES, OFF_SB = OFF_SA + SA::BYTES;
  constexpr int STG = OFF_SB + SB::BYTES;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    if (s < KT) {
      char* st = smem + s * STG;
      oa.issue(s, st, wave);
      ob.issue(s, st + OFF_B, wave);
      sa.issue(s, st + OFF_SA, wave);
      sb.issue(s, st + OFF_SB, wave);
    }
  }
}

// hook(kt) runs after K-tile kt's MMAs and refill DMAs are issued (as in ring_loop).
template <int F, class Tl, int STAGES, int EXTRA, bool TR = false, class OA, class OB, class SA, class SB,
          class HK = NoKtHook>
__device__ __forceinline__ void mx_ring_loop(const OA& oa, const OB& ob, const SA& sa, const SB& sb, int KT,
                                             char* smem, int wave, int lane, f32x16_t (&acc)[Tl::FM][Tl::FN],
                                             HK hook = HK{}) {
  static_assert(STAGES == 3, "the waits are written for 3 stages");
  constexpr int SD = MxFmt<F>::SD;
  constexpr int OFF_B = OA::BYTES, OFF_SA = OA::BYTES + OB::BYTES, OFF_SB = OFF_SA + SA::BYTES;
  constexpr int STG = OFF_SB + SB::BYTES;
  constexpr int NI = OA::NI + OB::NI + 2 * SD;
  zero_acc<Tl>(acc);
  for (int kt = 0; kt < KT; ++kt) {
    const bool pro = kt < STAGES - 1;  // issued by mx_ring_prologue, before any EXTRA stores
    if (kt + 1 < KT) wait_vmcnt_extra<NI, EXTRA>(pro); else wait_vmcnt_extra<0, EXTRA>(pro);
    ring_barrier();
    // refill with K-tile nk in two bursts, as in the bf16 core: A rows and both
    // scale rows now, the B rows between the two 64-k steps
    const int nk = kt + STAGES - 1;
    char* st = smem + (nk % STAGES) * STG;
    if (nk < KT) {
      oa.issue(nk, st, wave);
      sa.issue(nk, st + OFF_SA, wave);
      sb.issue(nk, st + OFF_SB, wave);
    }
    const char* cur = smem + (kt % STAGES) * STG;
    uint32_t xa[SD][Tl::FM], xb[SD][Tl::FN];
#pragma unroll
    for (int d = 0; d < SD; ++d) {
#pragma unroll
      for (int fm = 0; fm < Tl::FM; ++fm) xa[d][fm] = sa.get(cur + OFF_SA, fm, lane, d);
#pragma unroll
      for (int fn = 0; fn < Tl::FN; ++fn) xb[d][fn] = sb.get(cur + OFF_SB, fn, lane, d);
    }
    mx_kstep<F, 0, TR, Tl>(oa, ob, cur, cur + OFF_B, xa, xb, acc);
    if constexpr (F == 0) {
      if (nk < KT) ob.issue(nk, st + OFF_B, wave);
      mx_kstep<F, 1, TR, Tl>(oa, ob, cur, cur + OFF_B, xa, xb, acc);
    } else {
      mx_kstep<F, 1, TR, Tl>(oa, ob, cur, cur + OFF_B, xa, xb, acc);
      if (nk < KT) ob.issue(nk, st + OFF_B, wave);
      mx_kstep<F, 2, TR, Tl>(oa, ob, cur, cur + OFF_B, xa, xb, acc);
      mx_kstep<F, 3, TR, Tl>(oa, ob, cur, cur + OFF_B, xa, xb, acc);
    }
    hook(kt);
  }
  __syncthreads();
}

template <int F, class Tl, int STAGES, class OA, class OB, class SA, class SB>
__device__ __forceinline__ void main_loop_mx(const OA& oa, const OB& ob, const SA& sa, const SB& sb, int KT,
                                             char* smem, int wave, int lane, f32x16_t (&acc)[Tl::FM][Tl::FN]) {
  mx_ring_prologue<STAGES>(oa, ob, sa, sb, KT, smem, wave);
  mx_ring_loop<F, Tl, STAGES, 0>(oa, ob, sa, sb, KT, smem, wave, lane, acc);
}

template <int BM, int BN>
using RowTilingMx = Tiling<BM, BN, (BM == 32 ? 1 : 2), 4>;

struct MxRowArgs {
  Sched sc;
  const uint8_t* aq;  // fc1: x; fc2: h; dh: dy; dx: dgu  (E4M3 rows)
  const uint8_t* as;  // their scales
  const uint8_t* wq;  // fc1: w1q; fc2: w2q; dh: w2tq; dx: w1tq
  const uint8_t* ws;
  bf16* out0;         // fc1: au; fc2/dx: part; dh: dgu (bf16)
  bf16* out1;         // fc1: h
  uint8_t* oq;        // fc1: h quantised along I; dh: dgu quantised along 2I
  uint8_t* os;
  const bf16* au;     // dh
  const bf16* h;      // dh
  const float* gate;  // dh
  float* dgp;         // dh
  int H, I, k, R, T;  // T = tokens of the micro-batch (R = T * k)
};

enum MxKind { MFC1 = 0, MFC2 = 1, MDH = 2, MDX = 3 };

template <int KIND, class Tl, int F>
__global__ __launch_bounds__(Tl::NT) void row_gemm_mx_kernel(MxRowArgs a) {
  using Fm = MxFmt<F>;
  using OA = OpK<Tl::BM, Tl::FM, Tl::NW>;
  using OB = OpK<Tl::BN, Tl::FN, Tl::NW>;
  using SA = OpScale<Tl::BM, Tl::FM, Tl::NW, Fm::SD>;
  using SB = OpScale<Tl::BN, Tl::FN, Tl::NW, Fm::SD>;
  constexpr int STG = OA::BYTES + OB::BYTES + SA::BYTES + SB::BYTES;
  __shared__ __align__(1024) char smem[kMxStages * STG];
  __shared__ int s_ts[kMaxEx + 1];
  __shared__ int s_slot[Tl::BM];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int I2 = 2 * a.I;
  const int N = KIND == MFC1 ? I2 : (KIND == MFC2 || KIND == MDX ? a.H : a.I);
  const int K = KIND == MFC1 || KIND == MDH ? a.H : (KIND == MFC2 ? a.I : I2);
  const int KB = K / 32;                       // scale bytes per row
  const uint32_t KQ = (uint32_t)Fm::bytes(K);  // element bytes per row
  load_tile_start(a.sc, s_ts);
  for_each_row_tile(a.sc, s_ts, N / Tl::BN, blockIdx.x, gridDim.x, [&](const RowTile& t) {
    __syncthreads();
    for (int i = tid; i < Tl::BM; i += Tl::NT) s_slot[i] = i < t.nrows ? a.sc.perm[t.row0 + i] : -1;
    __syncthreads();
    const auto frow_a = [&](int f) { return wm * Tl::WTM + f * 32; };
    const auto frow_b = [&](int f) { return wn * Tl::WTN + f * 32; };
    OA oa;
    SA sa;
    if constexpr (KIND == MFC1 || KIND == MDH) {
      // pull dispatch / reverse-combine: token rows gathered through perm (padding rows re-read row 0)
      const auto tok = [&](int row) { return (uint32_t)(s_slot[row < t.nrows ? row : 0] / a.k); };
      oa.init(a.aq, [&](int row) -> uint32_t { return tok(row) * KQ; }, frow_a, wave, lane);
      sa.init(a.as, [&](int row) -> uint32_t { return tok(row) * 4u; }, frow_a, wave, lane, (uint32_t)a.T * 4u);
    } else {
      const auto rr = [&](int row) { return (uint32_t)(row < t.nrows ? row : 0); };
      oa.init(a.aq + (int64_t)t.row0 * KQ, [&](int row) -> uint32_t { return rr(row) * KQ; }, frow_a, wave, lane);
      sa.init(a.as + (int64_t)t.row0 * 4, [&](int row) -> uint32_t { return rr(row) * 4u; }, frow_a, wave, lane,
              (uint32_t)a.R * 4u);
    }
    OB ob;
    SB sb;
    if constexpr (KIND == MFC1) {
      // W1 rows with gate/up interleaved per 32-column block of the tile
      const int cbase = t.n * (Tl::BN / 2);
      const auto wrow = [&](int j) -> uint32_t {
        const int wj = j / Tl::WTN, fn = (j % Tl::WTN) >> 5;
        const int c = cbase + wj * (Tl::WTN / 2) + (fn >> 1) * 32 + (j & 31);
        return (uint32_t)((fn & 1) ? a.I + c : c);
      };
      ob.init(a.wq + (int64_t)t.e * I2 * KQ, [&](int j) -> uint32_t { return wrow(j) * KQ; }, frow_b, wave, lane);
      sb.init(a.ws + (int64_t)t.e * I2 * KB, [&](int j) -> uint32_t { return wrow(j) * 4u; }, frow_b, wave, lane,
              (uint32_t)I2 * 4u);
    } else {
      // weight rows n*BN + j of expert e's [N][K] matrix
      const int64_t r0 = (int64_t)t.e * N + (int64_t)t.n * Tl::BN;
      ob.init(a.wq + r0 * KQ, [&](int j) -> uint32_t { return (uint32_t)j * KQ; }, frow_b, wave, lane);
      sb.init(a.ws + (int64_t)t.e * N * KB + (int64_t)t.n * Tl::BN * 4, [&](int j) -> uint32_t { return (uint32_t)j * 4u; },
              frow_b, wave, lane, (uint32_t)N * 4u);
    }
    f32x16_t acc[Tl::FM][Tl::FN];
    main_loop_mx<F, Tl, kMxStages>(oa, ob, sa, sb, K / Fm::KTILE, smem, wave, lane, acc);

    if constexpr (KIND == MFC1) {
      const int cbase = t.n * (Tl::BN / 2);
      epilogue16<Tl, true>(acc, smem, wave, wm, wn, lane,
                           [&](int row, int col, const float (&g)[16], const float (&u)[16]) {
        if (row >= t.nrows) return;  // both lanes of a pair share the row
        const int64_t R = t.row0 + row;
        const int wj = col / Tl::WTN, cw = col % Tl::WTN;
        const int c = cbase + wj * (Tl::WTN / 2) + (cw >> 6) * 32 + (cw & 31);
        float hv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) hv[i] = g[i] / (1.0f + expf(-g[i])) * u[i];
        round16_bf16(hv);
        store16<bf16>(a.out0 + R * I2 + c, g);
        store16<bf16>(a.out0 + R * I2 + a.I + c, u);
        store16<bf16>(a.out1 + R * a.I + c, hv);
        const uint32_t sbyte = Fm::quant_store16(hv, a.oq, R * a.I + c);
        if ((lane & 1) == 0) a.os[(int64_t)(c >> 7) * a.R * 4 + R * 4 + ((c >> 5) & 3)] = (uint8_t)sbyte;
      });
    } else if constexpr (KIND == MFC2 || KIND == MDX) {
      epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane,
                            [&](int row, int col, const float (&g)[16], const float (&)[16]) {
        if (row < t.nrows) store16<bf16>(a.out0 + (int64_t)s_slot[row] * a.H + t.n * Tl::BN + col, g);
      });
    } else {  // MDH
      epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane,
                            [&](int row, int col, const float (&dA)[16], const float (&)[16]) {
        float part = 0.0f;
        if (row < t.nrows) {  // both lanes of a pair share the row
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
          round16_bf16(da);
          round16_bf16(du);
          store16<bf16>(a.out0 + R * I2 + c, da);
          store16<bf16>(a.out0 + R * I2 + a.I + c, du);
          const uint32_t s1 = Fm::quant_store16(da, a.oq, R * I2 + c);
          const uint32_t s2 = Fm::quant_store16(du, a.oq, R * I2 + a.I + c);
          if ((lane & 1) == 0) {
            const int c2 = a.I + c;
            a.os[(int64_t)(c >> 7) * a.R * 4 + R * 4 + ((c >> 5) & 3)] = (uint8_t)s1;
            a.os[(int64_t)(c2 >> 7) * a.R * 4 + R * 4 + ((c2 >> 5) & 3)] = (uint8_t)s2;
          }
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

// Weight gradients: out[e] [M][N] = sum over k in e's padded segment of A[m][k] B[n][k],
// A [M][kld] and B [N][kld] elements with K-tile-major scales [kld/128][M][4], [kld/128][N][4]; e's segment is
// columns pofs[e] .. pofs[e+1] (a multiple of the K-tile; empty -> zeros written).
struct MxDwArgs {
  const int32_t* pofs;
  const uint8_t *aq, *as, *bq, *bs;
  void* out;
  int M, N;
  int64_t kld;
  Guard guard;
};

template <class Tl, typename TO, int F>
__global__ __launch_bounds__(Tl::NT) void dw_mx_kernel(MxDwArgs a) {
  using Fm = MxFmt<F>;
  using OA = OpK<Tl::BM, Tl::FM, Tl::NW>;
  using OB = OpK<Tl::BN, Tl::FN, Tl::NW>;
  using SA = OpScale<Tl::BM, Tl::FM, Tl::NW, Fm::SD>;
  using SB = OpScale<Tl::BN, Tl::FN, Tl::NW, Fm::SD>;
  __shared__ __align__(1024) char smem[kMxStages * (OA::BYTES + OB::BYTES + SA::BYTES + SB::BYTES)];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  const int MT = a.M / Tl::BM, NT = a.N / Tl::BN;
  if (guard_fail(a.guard)) return;
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const int e = L / (MT * NT);
  const int rem = L - e * MT * NT;
  const int mt = rem / NT, nt = rem - mt * NT;
  const int64_t k0 = a.pofs[e];
  const int KT = (int)((a.pofs[e + 1] - k0) / Fm::KTILE);
  const int64_t ldq = Fm::bytes(a.kld), k0q = Fm::bytes(k0);
  const auto frow_a = [&](int f) { return wm * Tl::WTM + f * 32; };
  const auto frow_b = [&](int f) { return wn * Tl::WTN + f * 32; };
  OA oa;
  SA sa;
  OB ob;
  SB sb;
  oa.init(a.aq + (int64_t)mt * Tl::BM * ldq + k0q, [&](int r) -> uint32_t { return (uint32_t)(r * ldq); },
          frow_a, wave, lane);
  sa.init(a.as + (k0 / 128) * a.M * 4 + (int64_t)mt * Tl::BM * 4, [&](int r) -> uint32_t { return (uint32_t)r * 4u; },
          frow_a, wave, lane, (uint32_t)a.M * 4u);
  ob.init(a.bq + (int64_t)nt * Tl::BN * ldq + k0q, [&](int r) -> uint32_t { return (uint32_t)(r * ldq); },
          frow_b, wave, lane);
  sb.init(a.bs + (k0 / 128) * a.N * 4 + (int64_t)nt * Tl::BN * 4, [&](int r) -> uint32_t { return (uint32_t)r * 4u; },
          frow_b, wave, lane, (uint32_t)a.N * 4u);
  f32x16_t acc[Tl::FM][Tl::FN];
  main_loop_mx<F, Tl, kMxStages>(oa, ob, sa, sb, KT, smem, wave, lane, acc);
  TO* out = reinterpret_cast<TO*>(a.out) + ((int64_t)e * a.M + mt * Tl::BM) * a.N + nt * Tl::BN;
  epilogue16<Tl, false>(acc, smem, wave, wm, wn, lane, [&](int row, int col, const float (&g)[16], const float (&)[16]) {
    store16<TO>(out + (int64_t)row * a.N + col, g);
  });
}

// Persistent form of dw_mx_kernel for bf16 gradients (the same tiles and arithmetic):
// the next tile's first K-tiles are issued before this tile's epilogue, whose stores
// then drain under the next K-loop. The epilogue's per-wave patches use the ring stage
// that this prologue leaves free. Q = false: a workgroup walks tiles L = lo + li,
// lo + li + nx, ... of its XCD's contiguous part of the (expert, M-tile, N-tile) range
// (hundreds of tiles per workgroup at the streamed Kimi-K2 shape, where a hot expert's
// tile is a small share of a workgroup's work). Q = true (launches of a few tiles per
// workgroup): longest-K-first tile queues, as in the bf16 weight-gradient kernel.
template <class Tl, int F, bool Q>
__global__ __launch_bounds__(Tl::NT) void dw_mx_pipe_kernel(MxDwArgs a, int E) {
  using Fm = MxFmt<F>;
  using OA = OpK<Tl::BM, Tl::FM, Tl::NW>;
  using OB = OpK<Tl::BN, Tl::FN, Tl::NW>;
  using SA = OpScale<Tl::BM, Tl::FM, Tl::NW, Fm::SD>;
  using SB = OpScale<Tl::BN, Tl::FN, Tl::NW, Fm::SD>;
  constexpr int STAGES = kMxStages;
  constexpr int STG = OA::BYTES + OB::BYTES + SA::BYTES + SB::BYTES;
  constexpr int EXTRA = Tl::FM * Tl::FN * 2;  // global stores per lane in epilogue_bf16
  static_assert(Tl::NW * kBf16PatchBytes <= STG, "epilogue patches fit in one ring stage");
  __shared__ __align__(1024) char smem[STAGES * STG];
  __shared__ int s_u[kMaxEx + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Tl::WN, wn = wave % Tl::WN;
  char* patch = smem + (STAGES - 1) * STG + wave * kBf16PatchBytes;
  const int MT = a.M / Tl::BM, NT = a.N / Tl::BN;
  const int P = min(8, (int)gridDim.x);
  const int xcd = blockIdx.x % P;
  const int nx = ((int)gridDim.x - xcd + P - 1) / P;
  const int li = blockIdx.x / P;
  const int64_t TPE = (int64_t)MT * NT;
  if (guard_fail(a.guard)) return;
  const auto kt_of = [&](int e) { return (a.pofs[e + 1] - a.pofs[e]) / Fm::KTILE; };
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
  const auto frow_a = [&](int f) { return wm * Tl::WTM + f * 32; };
  const auto frow_b = [&](int f) { return wn * Tl::WTN + f * 32; };
  OA oa;
  OB ob;
  SA sa;
  SB sb;
  int e = 0, mt = 0, nt = 0, KT = 0;
  const int64_t ldq = Fm::bytes(a.kld);
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
    const int64_t k0 = __builtin_amdgcn_readfirstlane(a.pofs[e]);
    KT = __builtin_amdgcn_readfirstlane((int)((a.pofs[e + 1] - k0) / Fm::KTILE));
    oa.init(a.aq + (int64_t)mt * Tl::BM * ldq + Fm::bytes(k0), [&](int r) -> uint32_t { return (uint32_t)(r * ldq); },
            frow_a, wave, lane);
    sa.init(a.as + (k0 / 128) * a.M * 4 + (int64_t)mt * Tl::BM * 4, [&](int r) -> uint32_t { return (uint32_t)r * 4u; },
            frow_a, wave, lane, (uint32_t)a.M * 4u);
    ob.init(a.bq + (int64_t)nt * Tl::BN * ldq + Fm::bytes(k0), [&](int r) -> uint32_t { return (uint32_t)(r * ldq); },
            frow_b, wave, lane);
    sb.init(a.bs + (k0 / 128) * a.N * 4 + (int64_t)nt * Tl::BN * 4, [&](int r) -> uint32_t { return (uint32_t)r * 4u; },
            frow_b, wave, lane, (uint32_t)a.N * 4u);
  };
  setup(L);
  mx_ring_prologue<STAGES>(oa, ob, sa, sb, KT, smem, wave);
  bool first = true;
  for (;;) {
    f32x16_t acc[Tl::FM][Tl::FN];
    int claim = 0;  // lane 0 of wave 0: the part's next queue index
    const int kc = KT > 2 ? KT - 2 : 0;  // K-tiles of 128 (256) rows: two hide the claim
    const auto hook = [&](int kt) {
      if (Q && kt == kc && tid == 0) claim = dw_queue_claim(qline);
    };
    if (Q && KT == 0 && tid == 0) claim = dw_queue_claim(qline);
    if (first)
      mx_ring_loop<F, Tl, STAGES, 0, true>(oa, ob, sa, sb, KT, smem, wave, lane, acc, hook);
    else
      mx_ring_loop<F, Tl, STAGES, EXTRA, true>(oa, ob, sa, sb, KT, smem, wave, lane, acc, hook);
    bf16* out = reinterpret_cast<bf16*>(a.out) + ((int64_t)e * a.M + mt * Tl::BM) * a.N + nt * Tl::BN;
    int64_t Ln;
    if constexpr (Q) {
      __shared__ int s_next;
      asm volatile("" : "+v"(claim));  // the claim is read here, after the K-loop
      if (tid == 0) s_next = claim;
      __syncthreads();
      Ln = nx + (int64_t)__builtin_amdgcn_readfirstlane(s_next);
    } else {
      Ln = L + nx;
    }
    if (Ln < hi) {
      setup(Ln);
      mx_ring_prologue<STAGES>(oa, ob, sa, sb, KT, smem, wave);
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
static Sched sched_of_mx(const Ctx& c) { return Sched{c.counts, c.offsets, c.tile_start, c.perm, c.E, c.BM, c.guard}; }

template <int KIND, int BM, int BN>
static hipError_t row_launch_mx(const Ctx& c, const MxRowArgs& a, int N) {
  using Tl = RowTilingMx<BM, BN>;
  int g = c.grid > 0 ? c.grid : c.num_cu;
  const int64_t upper = (int64_t)c.max_tiles * (N / BN);
  if (g > upper) g = (int)std::max<int64_t>(upper, 1);
  if (c.mx4)
    hipLaunchKernelGGL((row_gemm_mx_kernel<KIND, Tl, 1>), dim3(g), dim3(Tl::NT), 0, c.s, a);
  else
    hipLaunchKernelGGL((row_gemm_mx_kernel<KIND, Tl, 0>), dim3(g), dim3(Tl::NT), 0, c.s, a);
  return hipGetLastError();
}

template <int KIND, int BN>
static hipError_t row_bm_mx(const Ctx& c, const MxRowArgs& a, int N) {
  switch (c.BM) {
    case 32: return row_launch_mx<KIND, 32, BN>(c, a, N);
    case 64: return row_launch_mx<KIND, 64, BN>(c, a, N);
    case 128: return row_launch_mx<KIND, 128, BN>(c, a, N);
  }
  return hipErrorInvalidValue;
}

static MxRowArgs mx_args(const Ctx& c) {
  MxRowArgs a{};
  a.sc = sched_of_mx(c);
  a.H = c.H;
  a.I = c.I;
  a.k = c.k;
  a.R = c.R;
  a.T = (int)c.T;
  return a;
}

hipError_t launch_fc1_mx(const Ctx& c, const void* xq, const void* xs, const void* w1q, const void* w1s, void* au,
                         void* h, void* hq, void* hs) {
  MxRowArgs a = mx_args(c);
  a.aq = (const uint8_t*)xq;
  a.as = (const uint8_t*)xs;
  a.wq = (const uint8_t*)w1q;
  a.ws = (const uint8_t*)w1s;
  a.out0 = (bf16*)au;
  a.out1 = (bf16*)h;
  a.oq = (uint8_t*)hq;
  a.os = (uint8_t*)hs;
  return row_bm_mx<MFC1, 256>(c, a, 2 * c.I);
}

hipError_t launch_fc2_mx(const Ctx& c, const void* hq, const void* hs, const void* w2q, const void* w2s, void* part) {
  MxRowArgs a = mx_args(c);
  a.aq = (const uint8_t*)hq;
  a.as = (const uint8_t*)hs;
  a.wq = (const uint8_t*)w2q;
  a.ws = (const uint8_t*)w2s;
  a.out0 = (bf16*)part;
  return bn_rows(c.H) == 256 ? row_bm_mx<MFC2, 256>(c, a, c.H) : row_bm_mx<MFC2, 128>(c, a, c.H);
}

hipError_t launch_dh_mx(const Ctx& c, const void* dyq, const void* dys, const void* w2tq, const void* w2ts,
                        const void* au, const void* h, const float* gate, void* dgu, void* dguq, void* dgus,
                        float* dgp) {
  MxRowArgs a = mx_args(c);
  a.aq = (const uint8_t*)dyq;
  a.as = (const uint8_t*)dys;
  a.wq = (const uint8_t*)w2tq;
  a.ws = (const uint8_t*)w2ts;
  a.out0 = (bf16*)dgu;
  a.oq = (uint8_t*)dguq;
  a.os = (uint8_t*)dgus;
  a.au = (const bf16*)au;
  a.h = (const bf16*)h;
  a.gate = gate;
  a.dgp = dgp;
  return bn_rows(c.I) == 256 ? row_bm_mx<MDH, 256>(c, a, c.I) : row_bm_mx<MDH, 128>(c, a, c.I);
}

hipError_t launch_dx_mx(const Ctx& c, const void* dguq, const void* dgus, const void* w1tq, const void* w1ts,
                        void* part) {
  MxRowArgs a = mx_args(c);
  a.aq = (const uint8_t*)dguq;
  a.as = (const uint8_t*)dgus;
  a.wq = (const uint8_t*)w1tq;
  a.ws = (const uint8_t*)w1ts;
  a.out0 = (bf16*)part;
  return bn_rows(c.H) == 256 ? row_bm_mx<MDX, 256>(c, a, c.H) : row_bm_mx<MDX, 128>(c, a, c.H);
}

template <class Tl>
static hipError_t dw_launch_mx(const Ctx& c, const MxDwArgs& a) {
  const int64_t blocks = (int64_t)c.E * (a.M / Tl::BM) * (a.N / Tl::BN);
  if (blocks == 0) return hipSuccess;
  if (!c.wgrad_f32) {
    const int g = (int)std::min<int64_t>(c.grid > 0 ? c.grid : c.num_cu, blocks);
    // tile queues when the launch has a few tiles per workgroup
    const bool q = blocks <= 16 * (int64_t)g && c.E <= kDwQueueMaxE && a.guard.hdr != nullptr;
    if (c.mx4) {
      if (q)
        hipLaunchKernelGGL((dw_mx_pipe_kernel<Tl, 1, true>), dim3(g), dim3(Tl::NT), 0, c.s, a, c.E);
      else
        hipLaunchKernelGGL((dw_mx_pipe_kernel<Tl, 1, false>), dim3(g), dim3(Tl::NT), 0, c.s, a, c.E);
    } else {
      if (q)
        hipLaunchKernelGGL((dw_mx_pipe_kernel<Tl, 0, true>), dim3(g), dim3(Tl::NT), 0, c.s, a, c.E);
      else
        hipLaunchKernelGGL((dw_mx_pipe_kernel<Tl, 0, false>), dim3(g), dim3(Tl::NT), 0, c.s, a, c.E);
    }
    return hipGetLastError();
  }
  if (c.mx4)
    hipLaunchKernelGGL((dw_mx_kernel<Tl, float, 1>), dim3((unsigned)blocks), dim3(Tl::NT), 0, c.s, a);
  else
    hipLaunchKernelGGL((dw_mx_kernel<Tl, float, 0>), dim3((unsigned)blocks), dim3(Tl::NT), 0, c.s, a);
  return hipGetLastError();
}

hipError_t launch_dw_mx(const Ctx& c, const int32_t* pofs, const void* aq, const void* as, const void* bq,
                        const void* bs, void* out, int M, int N, int64_t kld) {
  MxDwArgs a{pofs, (const uint8_t*)aq, (const uint8_t*)as, (const uint8_t*)bq, (const uint8_t*)bs, out, M, N, kld,
              c.guard};
  if (N % 256 == 0) return dw_launch_mx<Tiling<128, 256, 2, 4>>(c, a);
  return dw_launch_mx<Tiling<128, 128, 2, 2>>(c, a);
}

}  // namespace mok
