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

// ---------------------------------------------------------------------------
// K-contiguous operand, ROWS rows x 64 bf16 per stage.
// ---------------------------------------------------------------------------
template <int ROWS>
struct OpK {
  static constexpr int BK = 64;
  static constexpr int BYTES = ROWS * 128;
  static constexpr int NI = ROWS / 32;  // DMA instructions per wave per stage (8 rows each)
  static_assert(ROWS % 32 == 0, "rows");
  const char* src[NI];

  // rowptr(row) -> const bf16* at K offset 0; must be readable for the whole K range.
  template <class F> __device__ __forceinline__ void init(int wave, int lane, F rowptr) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = 8 * (wave + 4 * j) + (lane >> 3);
      src[j] = reinterpret_cast<const char*>(rowptr(row)) + 16 * ((lane & 7) ^ swz_k(row));
    }
  }
  __device__ __forceinline__ void issue(int kt, char* stage, int wave) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) dma16(src[j] + (int64_t)kt * 128, stage + (wave + 4 * j) * 1024);
  }
  __device__ __forceinline__ uint4 frag(const char* stage, int row0, int ks, int lane) const {
    const int row = row0 + (lane & 31);
    return *reinterpret_cast<const uint4*>(stage + row * 128 + 16 * ((2 * ks + (lane >> 5)) ^ swz_k(row)));
  }
};

// ---------------------------------------------------------------------------
// MN-contiguous operand, BK k-rows x ROWS bf16 per stage. Row k of the whole
// operand starts at base + (k0 + k) * ld (bytes); rows k >= cnt read zeros.
// ---------------------------------------------------------------------------
template <int ROWS, int BK_>
struct OpMN {
  static constexpr int BK = BK_;
  static constexpr int PITCH = ROWS * 2;
  static constexpr int BYTES = BK * PITCH;
  static constexpr int NI = BYTES / 4096;      // per wave per stage
  static constexpr int RPI = 1024 / PITCH;     // k-rows per DMA instruction
  static_assert(BYTES % 4096 == 0 && PITCH <= 1024, "tile");
  const char* base;  // byte address of row 0 at this lane's column chunk (before swizzle)
  int64_t ld;
  int cnt;
  int krow[NI];
  int colb[NI];

  __device__ __forceinline__ void init(const void* base_, int64_t ld_bytes, int cnt_, int wave, int lane) {
    base = reinterpret_cast<const char*>(base_);
    ld = ld_bytes;
    cnt = cnt_;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int o = (wave + 4 * j) * 1024 + 16 * lane;  // byte position in the stage
      krow[j] = o / PITCH;
      colb[j] = 16 * (((o % PITCH) >> 4) ^ swz_mn(krow[j]));
    }
  }
  __device__ __forceinline__ void issue(int kt, char* stage, int wave) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int k = kt * BK + krow[j];
      const char* p = k < cnt ? base + (int64_t)k * ld + colb[j] : reinterpret_cast<const char*>(g_zero_1k) + colb[j];
      dma16(p, stage + (wave + 4 * j) * 1024);
    }
  }
  // fragment for columns mb .. mb+31 and k-step ks (16 k) of the stage
  __device__ __forceinline__ uint4 frag(const char* stage, int mb, int ks, int lane) const {
    const int g = lane >> 4, i = lane & 15;
    const int mn = mb + 16 * (g & 1) + 4 * (i & 3);
    const int k0 = 16 * ks + 8 * (g >> 1) + (i >> 2);
    const int k1 = k0 + 4;
    const char* a0 = stage + k0 * PITCH + 16 * ((mn >> 3) ^ swz_mn(k0)) + 2 * (mn & 7);
    const char* a1 = stage + k1 * PITCH + 16 * ((mn >> 3) ^ swz_mn(k1)) + 2 * (mn & 7);
    const v4i16_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)a0);
    const v4i16_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t)a1);
    uint4 v;
    v.x = (uint16_t)r0[0] | ((uint32_t)(uint16_t)r0[1] << 16);
    v.y = (uint16_t)r0[2] | ((uint32_t)(uint16_t)r0[3] << 16);
    v.z = (uint16_t)r1[0] | ((uint32_t)(uint16_t)r1[1] << 16);
    v.w = (uint16_t)r1[2] | ((uint32_t)(uint16_t)r1[3] << 16);
    return v;
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

template <class Tl, int STAGES, class OA, class OB>
__device__ __forceinline__ void main_loop2(const OA& oa, const OB& ob, int KT, char* smem, int wave, int wm, int wn,
                                           int lane, f32x16_t (&acc)[Tl::FM][Tl::FN]) {
  static_assert(OA::BK == OB::BK, "operands disagree on the K-tile");
  constexpr int SB = OA::BYTES + OB::BYTES;
  constexpr int NI = OA::NI + OB::NI;
  constexpr int KS = OA::BK / 16;  // 16-k MFMA steps per K-tile
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
    if (nk < KT) {
      char* st = smem + (nk % STAGES) * SB;
      oa.issue(nk, st, wave);
      ob.issue(nk, st + OA::BYTES, wave);
    }
    const char* cur = smem + (kt % STAGES) * SB;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 a[Tl::FM], b[Tl::FN];
#pragma unroll
      for (int fm = 0; fm < Tl::FM; ++fm) a[fm] = oa.frag(cur, wm * Tl::WTM + fm * 32, ks, lane);
#pragma unroll
      for (int fn = 0; fn < Tl::FN; ++fn) b[fn] = ob.frag(cur + OA::BYTES, wn * Tl::WTN + fn * 32, ks, lane);
#pragma unroll
      for (int fm = 0; fm < Tl::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Tl::FN; ++fn) Mma<bf16>::run(acc[fm][fn], a[fm], b[fn]);
    }
  }
  __syncthreads();
}

}  // namespace mok
