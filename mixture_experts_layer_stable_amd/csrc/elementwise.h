// Bodies of the bandwidth-bound kernels (elementwise.hip), shared with the fused
// forward/backward kernels (gemm2.hip). Each body handles one work item -- a 16-byte
// vector of a row, a routed row, a token, or one (expert, column block) of dWr -- so the
// same arithmetic runs in a kernel of its own and as a stage of a persistent kernel.
#pragma once
#include "common.h"

namespace mok {

// y_t = sum_{j=0..k-1} g_tj * partial[t*k+j], item gid = t * (H/VE) + vector
template <typename T>
__device__ __forceinline__ void combine_body(const T* __restrict__ part, const float* __restrict__ gate,
                                             T* __restrict__ y, int64_t T_, int H, int k, int64_t gid) {
  constexpr int VE = Elem<T>::VE;
  const int vpr = H / VE;
  if (gid >= T_ * vpr) return;
  const int64_t t = gid / vpr;
  const int h0 = (int)(gid - t * vpr) * VE;
  float acc[VE];
#pragma unroll
  for (int q = 0; q < VE; ++q) acc[q] = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int64_t s = t * k + j;
    const float g = gate[s];
    float f[VE];
    unpack(ldg16(part + s * H + h0), f, (T*)nullptr);
#pragma unroll
    for (int q = 0; q < VE; ++q) acc[q] = __builtin_fmaf(g, f[q], acc[q]);
  }
  stg16(y + t * H + h0, pack(acc, (T*)nullptr));
}

// g'_s for the slot of routed row r: the d-gate partials of r's 32-column blocks of I,
// summed in ascending block order (threads of a wave read consecutive rows: coalesced).
__device__ __forceinline__ void router_gsum_body(const float* __restrict__ dgp, const int32_t* __restrict__ perm,
                                                 float* __restrict__ dgate, int R, int nb, int r) {
  if (r >= R) return;
  float v = 0.0f;
  for (int n = 0; n < nb; ++n) v += dgp[(int64_t)n * R + r];
  dgate[perm[r]] = v;
}

// dz_j = g_j * (g'_j - sum_i g_i g'_i) over one token's k slots, the sum in slot order.
__device__ __forceinline__ void router_dz_token(const float* g, const float* gp, float* dz, int k) {
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s = __builtin_fmaf(g[j], gp[j], s);
  for (int j = 0; j < k; ++j) dz[j] = g[j] * (gp[j] - s);
}

__device__ __forceinline__ void router_dz_body(const float* __restrict__ dgate, const float* __restrict__ gate,
                                               float* __restrict__ dz, int64_t T_, int k, int64_t t) {
  if (t >= T_) return;
  router_dz_token(gate + t * k, dgate + t * k, dz + t * k, k);
}

// dx_t = sum_j q[t*k+j] + sum_j dz_tj * wr[idx_tj], item gid = t * (H/VE) + vector
template <typename T>
__device__ __forceinline__ void dx_reduce_body(const T* __restrict__ part, const float* __restrict__ dz,
                                               const int32_t* __restrict__ idx, const T* __restrict__ wr,
                                               T* __restrict__ dx, int64_t T_, int H, int k, int64_t gid) {
  constexpr int VE = Elem<T>::VE;
  const int vpr = H / VE;
  if (gid >= T_ * vpr) return;
  const int64_t t = gid / vpr;
  const int h0 = (int)(gid - t * vpr) * VE;
  float acc[VE];
#pragma unroll
  for (int q = 0; q < VE; ++q) acc[q] = 0.0f;
  for (int j = 0; j < k; ++j) {
    float f[VE];
    unpack(ldg16(part + (t * k + j) * H + h0), f, (T*)nullptr);
#pragma unroll
    for (int q = 0; q < VE; ++q) acc[q] += f[q];
  }
  if (wr != nullptr) {
    for (int j = 0; j < k; ++j) {
      const float d = dz[t * k + j];
      float f[VE];
      unpack(ldg16(wr + (int64_t)idx[t * k + j] * H + h0), f, (T*)nullptr);
#pragma unroll
      for (int q = 0; q < VE; ++q) acc[q] = __builtin_fmaf(d, f[q], acc[q]);
    }
  }
  stg16(dx + t * H + h0, pack(acc, (T*)nullptr));
}

// dWr[e] = sum over e's routed rows r of dz[perm[r]] * x[token of r]. Work item
// = (expert, block of kDwrVec 16-byte column vectors) run by kDwrVec * kDwrLanes threads:
// thread (row lane l, vector v) sums rows l, l + LANES, l + 2*LANES, ... of the expert in
// ascending order; then the LANES row-lane sums of each column are added in ascending lane
// order. The order depends only on H (which picks the shape) and the expert's row count,
// not on the grid; a hot expert's rows are spread over LANES threads per column. Shapes:
// 64 lanes x 4 vectors for H <= 2048 (2048 tokens, Zipf: 18 -> 13 us), 32 lanes x 8
// vectors (whole 128-byte row pieces) above (Kimi-K2 shape: 0.33 ms, against 0.56 with
// 64 x 4). red: kDwrLanes x (kDwrVec * VE + 1) floats of LDS.
// xs (nullptr: not written): routed-order copy of the x rows, xs[r] = x[perm[r] / k], for the
// dW1 GEMM; every (row, vector) of x is read by exactly one thread here.
template <typename T, typename TO, int kDwrVec, int kDwrLanes>
__device__ __forceinline__ void dwr_body(const float* __restrict__ dz, const T* __restrict__ x,
                                         const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
                                         TO* __restrict__ dwr, int E, int H, int k, int item, float* red,
                                         T* __restrict__ xs = nullptr) {
  constexpr int VE = Elem<T>::VE;
  constexpr int COLS = kDwrVec * VE;
  const int vpr = H / VE;
  const int nvb = (vpr + kDwrVec - 1) / kDwrVec;
  const int e = item / nvb, vb = item % nvb;
  const int tv = threadIdx.x % kDwrVec, rl = threadIdx.x / kDwrVec;
  const int v = vb * kDwrVec + tv;
  float acc[VE];
#pragma unroll
  for (int q = 0; q < VE; ++q) acc[q] = 0.0f;
  if (v < vpr) {
    const int r1 = offsets[e + 1];
    if (xs == nullptr) {
      for (int r = offsets[e] + rl; r < r1; r += kDwrLanes) {
        const int s = perm[r];
        const float d = dz[s];
        float f[VE];
        unpack(ldg16(x + (int64_t)(s / k) * H + v * VE), f, (T*)nullptr);
#pragma unroll
        for (int q = 0; q < VE; ++q) acc[q] = __builtin_fmaf(d, f[q], acc[q]);
      }
    } else {
      // rows in groups of 4: the group's loads go out before its copies are stored, so a
      // load waits behind the previous group's stores only (vmcnt counts both in order)
      constexpr int G = 4;
      for (int r = offsets[e] + rl; r < r1; r += G * kDwrLanes) {
        uint4 raw[G];
        float d[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int rr = r + g * kDwrLanes;
          const int s = rr < r1 ? perm[rr] : 0;
          d[g] = rr < r1 ? dz[s] : 0.0f;
          raw[g] = rr < r1 ? ldg16(x + (int64_t)(s / k) * H + v * VE) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const int rr = r + g * kDwrLanes;
          if (rr < r1) {
            typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
            const u32x4_t w = {raw[g].x, raw[g].y, raw[g].z, raw[g].w};
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(xs + (int64_t)rr * H + v * VE));
            float f[VE];
            unpack(raw[g], f, (T*)nullptr);
#pragma unroll
            for (int q = 0; q < VE; ++q) acc[q] = __builtin_fmaf(d[g], f[q], acc[q]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < VE; ++q) red[rl * (COLS + 1) + tv * VE + q] = acc[q];
  __syncthreads();
  if (threadIdx.x < COLS) {
    const int col = (int)threadIdx.x;
    float sum = 0.0f;
#pragma unroll 8
    for (int l = 0; l < kDwrLanes; ++l) sum += red[l * (COLS + 1) + col];
    if (vb * kDwrVec + col / VE < vpr) Elem<TO>::put(dwr + (int64_t)e * H, (int64_t)vb * COLS + col, sum);
  }
  __syncthreads();
}

// dst[r] = src[perm[r] / k] (* gate[perm[r]], rounded to bf16): token rows in routed order,
// item gid = r * (H/8) + vector.
__device__ __forceinline__ void gather_rows_body(const bf16* __restrict__ src, const int32_t* __restrict__ perm,
                                                 const float* __restrict__ gate, bf16* __restrict__ dst, int R, int H,
                                                 int k, int64_t gid) {
  const int vpr = H / 8;
  if (gid >= (int64_t)R * vpr) return;
  const int r = (int)(gid / vpr);
  const int h0 = (int)(gid - (int64_t)r * vpr) * 8;
  const int s = perm[r];
  uint4 v = ldg16(src + (int64_t)(s / k) * H + h0);
  if (gate != nullptr) {
    const float g = gate[s];
    float f[8];
    unpack(v, f, (bf16*)nullptr);
#pragma unroll
    for (int q = 0; q < 8; ++q) f[q] = g * f[q];
    v = pack(f, (bf16*)nullptr);
  }
  stg16(dst + (int64_t)r * H + h0, v);
}

}  // namespace mok
