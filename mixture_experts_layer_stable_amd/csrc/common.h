// Shared device helpers for the gfx950 kernels of libmok.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "../../include/mok.h"

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

namespace mok {

// bf16 values live in memory as uint16_t bit patterns.
typedef uint16_t bf16;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> two bf16 packed in one dword (lo in bits 0..15), round to nearest
// even, by the hardware conversion (v_cvt_pk_bf16_f32). For finite values and
// infinities it gives the same bits as f32_to_bf16; NaN inputs do not occur here.
typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_hw_t));
}

// Element traits: storage type T, elements per 16-byte vector, load/store of one element as float.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VE = 4;
  static __device__ __forceinline__ float get(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void put(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16> {
  static constexpr int VE = 8;
  static __device__ __forceinline__ float get(const bf16* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void put(bf16* p, int64_t i, float v) { p[i] = (bf16)f32_to_bf16(v); }
};

// Unpack a 16-byte vector into floats / pack floats into one.
__device__ __forceinline__ void unpack(const uint4& v, float (&f)[8], bf16*) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void unpack(const uint4& v, float (&f)[4], float*) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ uint4 pack(const float (&f)[8], bf16*) {
  uint4 r;
  r.x = bf16x2_rne(f[0], f[1]);
  r.y = bf16x2_rne(f[2], f[3]);
  r.z = bf16x2_rne(f[4], f[5]);
  r.w = bf16x2_rne(f[6], f[7]);
  return r;
}
__device__ __forceinline__ uint4 pack(const float (&f)[4], float*) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = I .. N-1.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stg16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Schedule header check. mok_schedule_build writes, at the start of the schedule
// buffer, the hash of the descriptor it was built for (word 1) and a status word
// (word 4). A kernel that consumes the schedule (or runs as part of a call that
// does) compares the hash with the one of its own descriptor first: on a mismatch
// every workgroup leaves MOK_ERR_SCHEDULE_MISMATCH in the status word (all write
// the same value) and exits before touching anything else, so a table built for
// another problem never indexes memory. The test is uniform over the workgroup.
// hdr == nullptr: no schedule involved (weight quantisation), never fails.
constexpr int kHdrHash = 1, kHdrStatus = 4;

// Grid-barrier words of the fused kernels, after the 64-byte header in 128-byte lines
// (32 int32 each; line 0 is the header's), so that the atomics of different XCCs do not
// queue on one line: line 1 counts the XCCs that have left (word 1) and the XCC
// arrivals at the barriers (word 2); line 2 + x counts the arrivals (word 0), the
// workgroups (1) and the exits (2) of XCC x; line 18 + x holds the release generation
// of XCC x; line 34 + q is work queue q (the next item to hand out); line 38 + p is the
// weight-gradient tile queue of part p (word 0: tiles handed out, word 1: workgroups that
// have stopped claiming). mok_schedule_build zeroes them; the last workgroup to leave a
// fused kernel zeroes them again, and the last workgroup of a part to stop claiming
// zeroes that part's queue line.
constexpr int kSyncLine = 32, kSyncXcc = 16, kSyncQueues = 4, kSyncDwParts = 8;
constexpr int kSyncArrive = 2, kSyncRelease = 2 + kSyncXcc, kSyncQueue = 2 + 2 * kSyncXcc;
constexpr int kSyncDw = kSyncQueue + kSyncQueues;
constexpr int kSyncLines = kSyncDw + kSyncDwParts;
constexpr size_t kSchedHeaderBytes = (size_t)kSyncLines * kSyncLine * 4;

__device__ __forceinline__ void sync_zero(int32_t* hdr) {
  int32_t* l1 = hdr + kSyncLine;
  l1[0] = l1[1] = l1[2] = 0;
  for (int x = 0; x < kSyncXcc; ++x) {
    int32_t* la = hdr + (kSyncArrive + x) * kSyncLine;
    la[0] = la[1] = la[2] = 0;
    hdr[(kSyncRelease + x) * kSyncLine] = 0;
  }
  for (int q = 0; q < kSyncQueues; ++q) hdr[(kSyncQueue + q) * kSyncLine] = 0;
  for (int p = 0; p < kSyncDwParts; ++p) hdr[(kSyncDw + p) * kSyncLine] = hdr[(kSyncDw + p) * kSyncLine + 1] = 0;
}

struct Guard {
  int32_t* hdr;
  uint32_t expect;
};

__device__ __forceinline__ bool guard_fail(const Guard& g) {
  if (g.hdr == nullptr) return false;
  if ((uint32_t)g.hdr[kHdrHash] == g.expect) return false;
  if (threadIdx.x == 0) g.hdr[kHdrStatus] = MOK_ERR_SCHEDULE_MISMATCH;
  return true;
}

// Logical workgroup index with consecutive indices on one XCD: the dispatcher
// places workgroup b on XCD b % 8, so b -> (b % 8) * ceil(G/8) + b / 8 gives
// each XCD a contiguous range (G need not be a multiple of 8).
__device__ __forceinline__ int xcd_logical(int b, int G) {
  const int per = (G + 7) / 8;
  const int x = b % 8, i = b / 8;
  const int full = G % 8 == 0 ? 8 : G % 8;  // XCDs that receive `per` workgroups
  return x < full ? x * per + i : full * per + (x - full) * (per - 1) + i;
}

}  // namespace mok
