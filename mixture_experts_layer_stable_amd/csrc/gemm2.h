// bf16 grouped-GEMM core for gfx950 with direct global->LDS loads.
//
// Both operands of every K-tile are fetched by global_load_lds_dwordx4 (each
// lane's 16 bytes land at LDS base + 16*lane, 1 KB per wave instruction) into
// a ring of STAGES LDS buffers, so STAGES-1 K-tiles are in flight while one is
// multiplied, without staging registers. One barrier per K-tile.
//
// LDS layouts (a 16-byte chunk is never split):
//  * OpK  -- K-contiguous rows (token rows gathered through the schedule,
//    weight rows): tile row = one m/n, 128 bytes (64 bf16) of K, chunk
//    c stored at position c ^ ((row ^ row>>3) & 7). MFMA fragment = one
//    ds_read_b128 (8 consecutive k of one row).
//  * OpMN -- MN-contiguous rows (W1/W2 read transposed, token-major operands
//    of the weight gradients): tile row = one k, ROWS bf16 of m/n, chunk c
//    stored at c ^ 4*(k & 3). MFMA fragment = two ds_read_b64_tr_b16: a group
//    of 16 lanes addressing rows kb + i/4, columns mnb + 4*(i%4) receives in
//    lane l the 4 values (kb + q, mnb + l), q = 0..3.
// Both deliver lane L the 8 consecutive k of k-half L/32 at row/column L%32,
// which is what v_mfma_f32_32x32x16_bf16 consumes for A and for B.
#pragma once
#include <type_traits>
#include "gemm.h"

namespace mok {

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_t;

// 1 KB of zeros: the source of K-tail rows of the weight-gradient GEMMs.
extern __device__ uint4 g_zero_1k[64];

// The DMA is issued through inline asm so that the compiler does not treat it
// as a pending write to every LDS location (it would otherwise wait for all
// outstanding loads, vmcnt(0), before each LDS read and collapse the ring to
// one stage). Completion is tracked explicitly with wait_vmcnt below; loads
// complete in issue order, so compiler-managed waits on later loads stay valid.
__device__ __forceinline__ void dma16(const void* src, char* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(l), "v"(src) : "memory", "m0");
}

// s_waitcnt with vmcnt <= N (N < 64), no wait on the other counters.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fences of __syncthreads (which would
// drain every outstanding load). Inside the K-loop the only LDS writes are this
// core's DMAs, and every wave waits for its own (wait_vmcnt) before arriving;
// LDS reads of the previous stage were consumed by MFMAs before arrival.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ int swz_k(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int swz_mn(int k) { return 4 * (k & 3); }

// DMA with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit offset:
// advancing along K only changes the scalar base.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ void dma16_sv(const char* sbase, uint32_t voff, char* lds_wave_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(l), "v"(voff), "s"(sbase) : "memory", "m0");
}

__device__ __forceinline__ uint4 tr_pair(const char* a0, const char* a1) {
  const v4i16_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)a0);
  const v4i16_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)a1);
  const uint2 u0 = __builtin_bit_cast(uint2, r0), u1 = __builtin_bit_cast(uint2, r1);
  return make_uint4(u0.x, u0.y, u1.x, u1.y);
}

// ---------------------------------------------------------------------------
// K-contiguous operand, ROWS rows x 64 bf16 per stage; this wave reads NF
// fragments (32-row blocks) per k-step. Sources are sbase + per-lane 32-bit
// byte offsets (row offset + chunk), sbase advancing 128 bytes per K-tile.
// ---------------------------------------------------------------------------
template <int ROWS, int NF, int NW>
struct OpK {
  static constexpr int BK = 64;
  static constexpr int BYTES = ROWS * 128;
  static constexpr int NI = ROWS / (8 * NW);  // DMA instructions per wave per stage (8 rows each)
  static_assert(ROWS % (8 * NW) == 0, "rows");
  const char* sbase;
  uint32_t voff[NI];
  uint32_t foff[NF][4];

  // rowoff(row) -> byte offset of the row's K start from sbase_ (< 4 GiB);
  // frow(f) -> first tile row of fragment f of this wave.
  template <class F, class G>
  __device__ __forceinline__ void init(const void* sbase_, F rowoff, G frow, int wave, int lane) {
    sbase = reinterpret_cast<const char*>(sbase_);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = 8 * (wave + NW * j) + (lane >> 3);
      voff[j] = rowoff(row) + 16u * (uint32_t)((lane & 7) ^ swz_k(row));
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int row = frow(f) + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) foff[f][ks] = row * 128 + 16 * ((2 * ks + (lane >> 5)) ^ swz_k(row));
    }
  }
  __device__ __forceinline__ void issue(int kt, char* stage, int wave) const {
    const char* b = uniform_ptr(sbase + (int64_t)kt * 128);
#pragma unroll
    for (int j = 0; j < NI; ++j) dma16_sv(b, voff[j], stage + (wave + NW * j) * 1024);
  }
  __device__ __forceinline__ uint4 frag(const char* stage, int f, int ks) const {
    return *reinterpret_cast<const uint4*>(stage + foff[f][ks]);
  }
};

// ---------------------------------------------------------------------------
// K-contiguous operand with 32-element K-tiles: tile row = 64 bytes (4 chunks),
// chunk c stored at position c ^ ((row >> 2) & 3), so the 16 rows a quarter-wave
// reads (one chunk each) fall on 16 distinct 16-byte bank groups. One DMA
// instruction fills 16 rows; lane l fetches the chunk that belongs at its slot.
// ---------------------------------------------------------------------------
template <int ROWS, int NF, int NW>
struct OpK32 {
  static constexpr int BK = 32;
  static constexpr int BYTES = ROWS * 64;
  static constexpr int NI = ROWS / (16 * NW);
  static_assert(ROWS % (16 * NW) == 0, "rows");
  const char* sbase;
  uint32_t voff[NI];
  uint32_t foff[NF][2];

  template <class F, class G>
  __device__ __forceinline__ void init(const void* sbase_, F rowoff, G frow, int wave, int lane) {
    sbase = reinterpret_cast<const char*>(sbase_);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = 16 * (wave + NW * j) + (lane >> 2);
      voff[j] = rowoff(row) + 16u * (uint32_t)((lane & 3) ^ ((row >> 2) & 3));
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int row = frow(f) + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) foff[f][ks] = row * 64 + 16 * ((2 * ks + (lane >> 5)) ^ ((row >> 2) & 3));
    }
  }
  __device__ __forceinline__ void issue(int kt, char* stage, int wave) const {
    const char* b = uniform_ptr(sbase + (int64_t)kt * 64);
#pragma unroll
    for (int j = 0; j < NI; ++j) dma16_sv(b, voff[j], stage + (wave + NW * j) * 1024);
  }
  __device__ __forceinline__ uint4 frag(const char* stage, int f, int ks) const {
    return *reinterpret_cast<const uint4*>(stage + foff[f][ks]);
  }
};

// ---------------------------------------------------------------------------
// MN-contiguous operand, BK k-rows x ROWS bf16 per stage. Row k of the whole
// operand starts at sbase + k * ld (bytes); rows k >= cnt read zeros (only the
// last K-tile checks). NF fragments per k-step for this wave.
// ---------------------------------------------------------------------------
template <int ROWS, int BK_, int NF, int NW>
struct OpMN {
  static constexpr int BK = BK_;
  static constexpr int PITCH = ROWS * 2;
  static constexpr int BYTES = BK * PITCH;
  static constexpr int NI = BYTES / (1024 * NW);  // per wave per stage
  static_assert(BYTES % (1024 * NW) == 0 && PITCH <= 1024, "tile");
  const char* sbase;
  int64_t ld;
  int cnt;
  uint32_t voff[NI];   // krow * ld + swizzled column chunk
  uint32_t foff[NF];   // fragment (mb, ks = 0, first read) offset in the stage

  template <class G>
  __device__ __forceinline__ void init(const void* base_, int64_t ld_bytes, int cnt_, G fcol, int wave, int lane) {
    sbase = reinterpret_cast<const char*>(base_);
    ld = ld_bytes;
    cnt = cnt_;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int o = (wave + NW * j) * 1024 + 16 * lane;  // byte position in the stage
      const int kr = o / PITCH;
      voff[j] = (uint32_t)(kr * ld_bytes) + 16u * (uint32_t)(((o % PITCH) >> 4) ^ swz_mn(kr));
    }
    const int g = lane >> 4, i = lane & 15;
    const int k0 = 8 * (g >> 1) + (i >> 2);  // k-row of the first read at ks = 0; k0 & 3 = (i >> 2) & 3
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int mn = fcol(f) + 16 * (g & 1) + 4 * (i & 3);
      foff[f] = k0 * PITCH + 16 * ((mn >> 3) ^ swz_mn(k0)) + 2 * (mn & 7);
    }
  }
  __device__ __forceinline__ void issue(int kt, char* stage, int wave) const {
    const int k0 = kt * BK;
    if (k0 + BK <= cnt) {
      const char* b = uniform_ptr(sbase + (int64_t)k0 * ld);
#pragma unroll
      for (int j = 0; j < NI; ++j) dma16_sv(b, voff[j], stage + (wave + NW * j) * 1024);
    } else {
      // tail K-tile: rows past cnt read the zero block at the same column chunk;
      // addresses derive from the 32-bit offsets (no 64-bit per-lane state kept)
      const char* b = sbase + (int64_t)k0 * ld;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int o = (wave + NW * j) * 1024 + 16 * (threadIdx.x & 63);
        const int kr = o / PITCH;
        const char* p = k0 + kr < cnt ? b + voff[j]
                                      : reinterpret_cast<const char*>(g_zero_1k) + (voff[j] - (uint32_t)(kr * ld));
        dma16(p, stage + (wave + NW * j) * 1024);
      }
    }
  }
  // k-step ks: rows 16ks + {k0, k0+4} relative to the first read
  __device__ __forceinline__ uint4 frag(const char* stage, int f, int ks) const {
    const char* a = stage + foff[f] + ks * 16 * PITCH;
    return tr_pair(a, a + 4 * PITCH);
  }
};

// ---------------------------------------------------------------------------
// Main loop: STAGES-deep ring; at K-tile kt wait for this wave's DMA of kt,
// barrier (tile kt visible to all; everyone finished kt-1), refill the stage
// of kt-1 with kt+STAGES-1, multiply kt.
// ---------------------------------------------------------------------------
template <int STAGES, int NI>
__device__ __forceinline__ void wait_tiles_behind(int behind) {
  // behind = number of K-tiles issued after the one we need (0 .. STAGES-2)
  if constexpr (STAGES >= 4) {
    if (behind >= 2) { wait_vmcnt<2 * NI>(); return; }
  }
  if constexpr (STAGES >= 3) {
    if (behind >= 1) { wait_vmcnt<NI>(); return; }
  }
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// One K-tile of MFMAs from stage `cur`, fragments of 16-k step ks+1 read while
// the MFMAs of ks run. The DMAs that refill the ring with K-tile nk (when `more`)
// are not issued in one burst after the barrier: A's go out at the top of the
// first 16-k step and B's (the larger share in every kernel here) at the top of
// step KS/2, so the memory system sees two smaller bursts per K-tile. Measured
// on the Kimi-K2-shaped layer, this is 2-5% faster than one burst for the row
// GEMMs; issuing most of the bytes in the first half gains nothing.
// ---------------------------------------------------------------------------

// TR: accumulate the transposed blocks (MFMA operands swapped: the same products summed
// over the same k, so the same bits), for the epilogue_bf16 layout below.
template <class Tl, bool TR = false, class OA, class OB>
__device__ __forceinline__ void ktile_mma(const OA& oa, const OB& ob, const char* cur, bool more, int nk, char* st,
                                          int wave, f32x16_t (&acc)[Tl::FM][Tl::FN]) {
  constexpr int KS = OA::BK / 16;
  uint4 a[2][Tl::FM], b[2][Tl::FN];
#pragma unroll
  for (int fm = 0; fm < Tl::FM; ++fm) a[0][fm] = oa.frag(cur, fm, 0);
#pragma unroll
  for (int fn = 0; fn < Tl::FN; ++fn) b[0][fn] = ob.frag(cur + OA::BYTES, fn, 0);
  static_for<0, KS>([&](auto kc) {
    constexpr int ks = decltype(kc)::value, c = ks & 1;
    if constexpr (ks == 0)
      if (more) oa.issue(nk, st, wave);
    if constexpr (ks == KS / 2)
      if (more) ob.issue(nk, st + OA::BYTES, wave);
    if constexpr (ks + 1 < KS) {
#pragma unroll
      for (int fm = 0; fm < Tl::FM; ++fm) a[c ^ 1][fm] = oa.frag(cur, fm, ks + 1);
#pragma unroll
      for (int fn = 0; fn < Tl::FN; ++fn) b[c ^ 1][fn] = ob.frag(cur + OA::BYTES, fn, ks + 1);
    }
#pragma unroll
    for (int fm = 0; fm < Tl::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < Tl::FN; ++fn) {
        if constexpr (TR)
          Mma<bf16>::run(acc[fm][fn], b[c][fn], a[c][fm]);
        else
          Mma<bf16>::run(acc[fm][fn], a[c][fm], b[c][fn]);
      }
  });
}

template <class Tl, int STAGES, class OA, class OB>
__device__ __forceinline__ void main_loop2(const OA& oa, const OB& ob, int KT, char* smem, int wave, int wm, int wn,
                                           int lane, f32x16_t (&acc)[Tl::FM][Tl::FN]) {
  static_assert(OA::BK == OB::BK, "operands disagree on the K-tile");
  constexpr int SB = OA::BYTES + OB::BYTES;
  constexpr int NI = OA::NI + OB::NI;
  zero_acc<Tl>(acc);
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    if (s < KT) {
      oa.issue(s, smem + s * SB, wave);
      ob.issue(s, smem + s * SB + OA::BYTES, wave);
    }
  }
  for (int kt = 0; kt < KT; ++kt) {
    const int ahead = KT - 1 - kt;
    wait_tiles_behind<STAGES, NI>(ahead < STAGES - 2 ? ahead : STAGES - 2);
    ring_barrier();
    const int nk = kt + STAGES - 1;
    ktile_mma<Tl>(oa, ob, smem + (kt % STAGES) * SB, nk < KT, nk, smem + (nk % STAGES) * SB, wave, acc);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Split form of main_loop2 for kernels that pipeline across output tiles: the
// prologue (first STAGES-1 K-tiles) of tile i+1 is issued before tile i's
// epilogue, whose EXTRA global stores per wave are then younger than the prologue
// DMAs. Vector-memory operations complete in issue order, so a wait for a prologue
// tile may leave those stores outstanding; a wait for any later tile covers them.
// ---------------------------------------------------------------------------
template <int STAGES, class OA, class OB>
__device__ __forceinline__ void ring_prologue(const OA& oa, const OB& ob, int KT, char* smem, int wave) {
  constexpr int SB = OA::BYTES + OB::BYTES;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    if (s < KT) {
      oa.issue(s, smem + s * SB, wave);
      ob.issue(s, smem + s * SB + OA::BYTES, wave);
    }
  }
}

template <int N, int EXTRA>
__device__ __forceinline__ void wait_vmcnt_extra(bool prologue_tile) {
  if (prologue_tile) wait_vmcnt<N + EXTRA>(); else wait_vmcnt<N>();
}

struct NoKtHook {
  __device__ void operator()(int) const {}
};

// hook(kt) runs after K-tile kt's MMAs and refill DMAs are issued. A vector-memory
// operation it issues only makes the later vmcnt waits cover more (completion is in
// issue order), never less.
template <class Tl, int STAGES, int EXTRA, bool TR = false, class OA, class OB, class HK = NoKtHook>
__device__ __forceinline__ void ring_loop(const OA& oa, const OB& ob, int KT, char* smem, int wave, int lane,
                                          f32x16_t (&acc)[Tl::FM][Tl::FN], HK hook = HK{}) {
  static_assert(STAGES == 3, "ring_loop waits are written for 3 stages");
  constexpr int SB = OA::BYTES + OB::BYTES;
  constexpr int NI = OA::NI + OB::NI;
  zero_acc<Tl>(acc);
  for (int kt = 0; kt < KT; ++kt) {
    const bool pro = kt < STAGES - 1;  // issued by ring_prologue, before the stores
    if (kt + 1 < KT) wait_vmcnt_extra<NI, EXTRA>(pro); else wait_vmcnt_extra<0, EXTRA>(pro);
    ring_barrier();
    const int nk = kt + STAGES - 1;
    ktile_mma<Tl, TR>(oa, ob, smem + (kt % STAGES) * SB, nk < KT, nk, smem + (nk % STAGES) * SB, wave, acc);
    hook(kt);
  }
  __syncthreads();
}

// 16-byte store marked non-temporal: the weight gradients are written once and not read
// again by the step, so they should not displace operand lines from the caches (the
// weight-gradient GEMMs' stores, measured: dW2 5.62 -> 5.21 ms at the Kimi-K2 shape).
__device__ __forceinline__ void stg16_nt(void* p, const uint4& v) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// Work-balanced split of a weight-gradient GEMM's tile range over the XCDs. Tiles are
// ordered (expert, M-tile, N-tile); each of the TPE tiles of expert e costs
// kt(e) + kDwTileCost units (its K-tiles plus an epilogue's worth), so an expert with
// eight times the mean rows weighs eight times as much. Part x of P holds the tiles whose
// cumulative cost starts in [x W / P, (x+1) W / P): contiguous, disjoint, covering every
// tile, and a function of the counts only (which workgroup computes a tile never changes
// its bits). s_u (E + 1 ints of LDS) receives the exclusive prefix of kt(e) + kDwTileCost.
constexpr int kDwTileCost = 4;

template <class F>
__device__ __forceinline__ void dw_balanced_part(int E, int64_t TPE, F kt, int* s_u, int P, int x, int64_t& lo,
                                                 int64_t& hi) {
  const int nt = blockDim.x, t = threadIdx.x;
  const int per = (E + nt - 1) / nt;  // experts summed by this thread
  const int e0 = min(E, t * per), e1 = min(E, e0 + per);
  int sum = 0;
  for (int e = e0; e < e1; ++e) sum += kt(e) + kDwTileCost;
  s_u[E] = 0;
  __syncthreads();
  if (e1 > e0) s_u[e0] = sum;  // chunk totals at the chunk starts
  __syncthreads();
  if (t == 0) {  // fixed-order scan of the chunk totals
    int run = 0;
    for (int c = 0; c * per < E; ++c) {
      const int v = s_u[c * per];
      s_u[c * per] = run;
      run += v;
    }
    s_u[E] = run;
  }
  __syncthreads();
  if (e1 > e0) {
    int run = s_u[e0];
    for (int e = e0; e < e1; ++e) {
      const int u = kt(e) + kDwTileCost;
      s_u[e] = run;
      run += u;
    }
  }
  __syncthreads();
  const int64_t W = TPE * s_u[E];
  const auto tile_at = [&](int64_t w) -> int64_t {  // first tile whose cost starts at or after w
    int a = 0, b = E;                               // TPE * s_u[a] <= w < TPE * s_u[b] (or b = E)
    while (b - a > 1) {
      const int m = (a + b) >> 1;
      if (TPE * s_u[m] <= w) a = m; else b = m;
    }
    if (TPE * s_u[a + 1] <= w) return (int64_t)E * TPE;
    const int64_t u = s_u[a + 1] - s_u[a];
    const int64_t i = (w - TPE * s_u[a] + u - 1) / u;
    return (int64_t)a * TPE + min(i, TPE);
  };
  const int64_t l = tile_at(W * x / P);
  const int64_t h = x + 1 == P ? (int64_t)E * TPE : tile_at(W * (x + 1) / P);
  // wave-uniform: keep them in scalar registers
  lo = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)l >> 32)) << 32) |
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)l));
  hi = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)h >> 32)) << 32) |
                 (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)h));
}

// Order of an expert's output tiles in the persistent weight-gradient walk: blocks of
// kDwBandGroup row bands, column-major inside a block, so the 32 tiles an XCD works on at
// once share 4 row bands of A and 8 column bands of B (about 2 MB at the Kimi-K2 shape,
// which the XCD's 4 MB L2 keeps); B is then fetched once per block instead of once per
// row band (dW1 HBM reads 26.2 -> 8.5 GB per launch at the Kimi-K2 shape, same time;
// 8-band blocks read 5.3 GB but ran 3.5 % slower). Which tile a workgroup takes never
// changes its bits. The MX weight gradients (128 x 256 tiles) use the same walk (streamed
// Kimi-K2 step: MXFP8 dW1 8.66 -> 8.16 ms, bit-identical).
constexpr int kDwBandGroup = 4;

__device__ __forceinline__ void dw_tile_order(int rem, int MT, int NT, int& mt, int& nt) {
  const int b = rem / (kDwBandGroup * NT), gm = min(kDwBandGroup, MT - b * kDwBandGroup);
  const int r = rem - b * kDwBandGroup * NT, c = r / gm;
  nt = __builtin_amdgcn_readfirstlane(c);
  mt = __builtin_amdgcn_readfirstlane(b * kDwBandGroup + (r - c * gm));
}

// Longest-K-first order of the experts for the weight-gradient tile queues: s_ord[i] is
// the expert with the i-th largest K-tile count (ties by expert index), a fixed function
// of the counts. s_kt is scratch for E ints. One rank per expert, E / blockDim passes over
// E counts: meant for E <= kDwQueueMaxE.
constexpr int kDwQueueMaxE = 256;

template <class F>
__device__ __forceinline__ void dw_lpt_order(int E, F kt, int* s_kt, int* s_ord) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_kt[e] = kt(e);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int v = s_kt[e];
    int r = 0;
    for (int f = 0; f < E; ++f) {
      const int w = s_kt[f];
      r += (w > v) | ((w == v) & (f < e));
    }
    s_ord[r] = e;
  }
  __syncthreads();
}

// Weight-gradient tile queue of part p (a line of the schedule header, zero at rest):
// claim returns the part's next queue index; a workgroup that will claim no more calls
// leave, and the part's last one zeroes the line for the next launch (no claim of this
// launch can follow: every member has had its last claim answered).
__device__ __forceinline__ int32_t* dw_queue_line(int32_t* hdr, int p) { return hdr + (kSyncDw + p) * kSyncLine; }

__device__ __forceinline__ int dw_queue_claim(int32_t* line) {
  return __hip_atomic_fetch_add(line, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void dw_queue_leave(int32_t* line, int members) {
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(line + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1) {
    __hip_atomic_store(line, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(line + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// bf16 epilogue through a per-wave LDS patch, from transposed accumulator blocks
// (ktile_mma with TR): a lane holds 16 column values of one tile row, lane%32 being the
// row and registers 4g..4g+3 the columns 8g + 4(lane/32) .. +3. One conversion packs two
// neighbouring columns, and four columns go into the 32-row x 64-column patch of a block
// pair in one 8-byte write; with a row pitch of 34 dwords the 32 rows that a half-wave
// writes fall on distinct bank pairs. The patch is read back (two 8-byte reads: odd rows
// start 8-byte aligned) so that every store instruction writes 8 whole rows of 128
// contiguous bytes (lane: row = 8i + lane/8, 16-byte chunk lane%8). FM*FN*2 global
// stores per lane, as store(row, col, v) with v the 8 bf16 at tile (row, col .. col+7).
// The patch (kBf16PatchBytes) lies outside any ring stage still in use; a wave's LDS
// operations run in issue order.
constexpr int kBf16PatchPitch = 34;  // dwords
constexpr int kBf16PatchBytes = 32 * kBf16PatchPitch * 4;

template <class Tl, class F>
__device__ __forceinline__ void epilogue_bf16(f32x16_t (&acc)[Tl::FM][Tl::FN], char* patch, int wm, int wn, int lane,
                                              F&& store) {
  static_assert(Tl::FN % 2 == 0, "blocks are stored in horizontal pairs");
  constexpr int P = kBf16PatchPitch;
  const int m = lane & 31, h = lane >> 5;
  uint32_t* pw = reinterpret_cast<uint32_t*>(patch);
#pragma unroll
  for (int fm = 0; fm < Tl::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < Tl::FN; fn += 2) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 v;
          v.x = bf16x2_rne(acc[fm][fn + hb][4 * g], acc[fm][fn + hb][4 * g + 1]);
          v.y = bf16x2_rne(acc[fm][fn + hb][4 * g + 2], acc[fm][fn + hb][4 * g + 3]);
          *reinterpret_cast<uint2*>(pw + m * P + 16 * hb + 4 * g + 2 * h) = v;
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * i + (lane >> 3), c = (lane & 7) * 8;
        const uint2 lo = *reinterpret_cast<const uint2*>(pw + row * P + c / 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(pw + row * P + c / 2 + 2);
        store(wm * Tl::WTM + fm * 32 + row, wn * Tl::WTN + fn * 32 + c, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
    }
}

}  // namespace mok
