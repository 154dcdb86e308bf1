// Bandwidth-bound kernels of the layer step, all with fixed summation orders.
//
//  combine     y_t = sum_{j=0..k-1} g_tj * partial[t*k+j]            (push combine)
//  router_bwd  g'_s = sum over the 32-column blocks of I (ascending) of the d-gate partials
//              (one thread per routed row), then per token
//              dz_tj = g_tj * (g'_tj - sum_i g_ti g'_ti)   (softmax over the top k)
//  dx_reduce   dx_t = sum_j q[t*k+j] + sum_j dz_tj * wr[idx_tj]  (push reverse-dispatch)
//  dwr         dWr[e] = sum over e's routed rows (ascending slot) of dz_s * x_t
// Each thread owns one 16-byte vector of a row; loops over j / rows run in
// ascending order with fp32 fused multiply-adds.
#include "kernels.h"

namespace mok {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(Guard gd, const T* __restrict__ part,
                                                      const float* __restrict__ gate, T* __restrict__ y, int64_t T_,
                                                      int H, int k) {
  constexpr int VE = Elem<T>::VE;
  const int vpr = H / VE;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (guard_fail(gd) || gid >= T_ * vpr) return;
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
__global__ __launch_bounds__(256) void router_gsum_kernel(Guard gd, const float* __restrict__ dgp,
                                                          const int32_t* __restrict__ perm,
                                                          float* __restrict__ dgate, int R, int nb) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (guard_fail(gd) || r >= R) return;
  float v = 0.0f;
  for (int n = 0; n < nb; ++n) v += dgp[(int64_t)n * R + r];
  dgate[perm[r]] = v;
}

// dz_tj = g_tj * (g'_tj - sum_i g_ti g'_ti), the sum in slot order.
__global__ __launch_bounds__(256) void router_dz_kernel(Guard gd, const float* __restrict__ dgate,
                                                        const float* __restrict__ gate, float* __restrict__ dz,
                                                        int64_t T_, int k) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (guard_fail(gd) || t >= T_) return;
  float s = 0.0f;
  for (int j = 0; j < k; ++j) s = __builtin_fmaf(gate[t * k + j], dgate[t * k + j], s);
  for (int j = 0; j < k; ++j) dz[t * k + j] = gate[t * k + j] * (dgate[t * k + j] - s);
}

template <typename T>
__global__ __launch_bounds__(256) void dx_reduce_kernel(Guard gd, const T* __restrict__ part,
                                                        const float* __restrict__ dz, const int32_t* __restrict__ idx,
                                                        const T* __restrict__ wr, T* __restrict__ dx, int64_t T_, int H,
                                                        int k) {
  constexpr int VE = Elem<T>::VE;
  const int vpr = H / VE;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (guard_fail(gd) || gid >= T_ * vpr) return;
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

// dWr[e] = sum over e's routed rows r of dz[perm[r]] * x[token of r]. Workgroup =
// (expert, block of kDwrVec 16-byte column vectors): thread (row lane l, vector v) sums
// rows l, l + LANES, l + 2*LANES, ... of the expert in ascending order; then the LANES
// row-lane sums of each column are added in ascending lane order. The order depends only
// on H (which picks the shape) and the expert's row count, not on the grid; a hot
// expert's rows are spread over LANES threads per column. Shapes: 64 lanes x 4 vectors
// for H <= 2048 (2048 tokens, Zipf: 18 -> 13 us), 32 lanes x 8 vectors (whole 128-byte
// row pieces) above (Kimi-K2 shape: 0.33 ms, against 0.56 with 64 x 4).
template <typename T, typename TO, int kDwrVec, int kDwrLanes>
__global__ __launch_bounds__(kDwrVec * kDwrLanes) void dwr_kernel(Guard gd, const float* __restrict__ dz,
                                                                  const T* __restrict__ x,
                                                                  const int32_t* __restrict__ offsets,
                                                                  const int32_t* __restrict__ perm,
                                                                  TO* __restrict__ dwr, int E, int H, int k) {
  constexpr int VE = Elem<T>::VE;
  constexpr int COLS = kDwrVec * VE;
  __shared__ float red[kDwrLanes][COLS + 1];
  if (guard_fail(gd)) return;
  const int vpr = H / VE;
  const int nvb = (vpr + kDwrVec - 1) / kDwrVec;
  const int e = (int)(blockIdx.x / nvb), vb = (int)(blockIdx.x % nvb);
  const int tv = threadIdx.x % kDwrVec, rl = threadIdx.x / kDwrVec;
  const int v = vb * kDwrVec + tv;
  float acc[VE];
#pragma unroll
  for (int q = 0; q < VE; ++q) acc[q] = 0.0f;
  if (v < vpr) {
    const int r1 = offsets[e + 1];
    for (int r = offsets[e] + rl; r < r1; r += kDwrLanes) {
      const int s = perm[r];
      const float d = dz[s];
      float f[VE];
      unpack(ldg16(x + (int64_t)(s / k) * H + v * VE), f, (T*)nullptr);
#pragma unroll
      for (int q = 0; q < VE; ++q) acc[q] = __builtin_fmaf(d, f[q], acc[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < VE; ++q) red[rl][tv * VE + q] = acc[q];
  __syncthreads();
  if (threadIdx.x < COLS) {
    const int col = (int)threadIdx.x;
    float sum = 0.0f;
#pragma unroll 8
    for (int l = 0; l < kDwrLanes; ++l) sum += red[l][col];
    if (vb * kDwrVec + col / VE < vpr) Elem<TO>::put(dwr + (int64_t)e * H, (int64_t)vb * COLS + col, sum);
  }
}

// dst[r] = src[perm[r] / k] (* gate[perm[r]], rounded to bf16): token rows in routed order.
__global__ __launch_bounds__(256) void gather_rows_kernel(Guard gd, const bf16* __restrict__ src,
                                                          const int32_t* __restrict__ perm,
                                                          const float* __restrict__ gate, bf16* __restrict__ dst, int R,
                                                          int H, int k) {
  const int vpr = H / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (guard_fail(gd) || gid >= (int64_t)R * vpr) return;
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

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_gather_rows(const Ctx& c, const void* src, const float* gate, void* dst) {
  if (c.R == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks_for((int64_t)c.R * (c.H / 8))), dim3(256), 0, c.s,
                     c.guard, (const bf16*)src, c.perm, gate, (bf16*)dst, c.R, c.H, c.k);
  return hipGetLastError();
}

hipError_t launch_combine(const Ctx& c, const void* part, const float* gate, void* y) {
  if (c.T == 0) return hipSuccess;
  if (c.act == MOK_F32) {
    const int64_t n = c.T * (c.H / 4);
    hipLaunchKernelGGL(combine_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, c.s, c.guard,
                       (const float*)part, gate, (float*)y, c.T, c.H, c.k);
  } else {
    const int64_t n = c.T * (c.H / 8);
    hipLaunchKernelGGL(combine_kernel<bf16>, dim3(blocks_for(n)), dim3(256), 0, c.s, c.guard,
                       (const bf16*)part, gate, (bf16*)y, c.T, c.H, c.k);
  }
  return hipGetLastError();
}

hipError_t launch_router_bwd(const Ctx& c, const float* dgp, const float* gate, float* dgate, float* dz) {
  if (c.T == 0) return hipSuccess;
  hipLaunchKernelGGL(router_gsum_kernel, dim3(blocks_for(c.R)), dim3(256), 0, c.s, c.guard, dgp, c.perm, dgate, c.R,
                     dgate_parts(c.I));
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(router_dz_kernel, dim3(blocks_for(c.T)), dim3(256), 0, c.s, c.guard, dgate, gate, dz, c.T, c.k);
  return hipGetLastError();
}

hipError_t launch_dx_reduce(const Ctx& c, const void* part, const float* dz, const int32_t* idx, const void* wr,
                            void* dx) {
  if (c.T == 0) return hipSuccess;
  if (c.act == MOK_F32) {
    hipLaunchKernelGGL(dx_reduce_kernel<float>, dim3(blocks_for(c.T * (c.H / 4))), dim3(256), 0, c.s,
                       c.guard, (const float*)part, dz, idx, (const float*)wr, (float*)dx, c.T, c.H, c.k);
  } else {
    hipLaunchKernelGGL(dx_reduce_kernel<bf16>, dim3(blocks_for(c.T * (c.H / 8))), dim3(256), 0, c.s,
                       c.guard, (const bf16*)part, dz, idx, (const bf16*)wr, (bf16*)dx, c.T, c.H, c.k);
  }
  return hipGetLastError();
}

template <int VEC, int LANES>
static hipError_t launch_dwr_shape(const Ctx& c, const float* dz, const void* x, void* dwr) {
  const int ve = c.act == MOK_F32 ? 4 : 8;
  const int64_t nvb = ((int64_t)(c.H / ve) + VEC - 1) / VEC;
  const dim3 grid((unsigned)(c.E * nvb)), block(VEC * LANES);
  if (c.E * nvb == 0) return hipSuccess;
  if (c.act == MOK_F32) {
    hipLaunchKernelGGL((dwr_kernel<float, float, VEC, LANES>), grid, block, 0, c.s, c.guard, dz, (const float*)x, c.offsets,
                       c.perm, (float*)dwr, c.E, c.H, c.k);
  } else if (c.wgrad_f32) {
    hipLaunchKernelGGL((dwr_kernel<bf16, float, VEC, LANES>), grid, block, 0, c.s, c.guard, dz, (const bf16*)x, c.offsets,
                       c.perm, (float*)dwr, c.E, c.H, c.k);
  } else {
    hipLaunchKernelGGL((dwr_kernel<bf16, bf16, VEC, LANES>), grid, block, 0, c.s, c.guard, dz, (const bf16*)x, c.offsets,
                       c.perm, (bf16*)dwr, c.E, c.H, c.k);
  }
  return hipGetLastError();
}

hipError_t launch_dwr(const Ctx& c, const float* dz, const void* x, void* dwr) {
  return c.H <= 2048 ? launch_dwr_shape<4, 64>(c, dz, x, dwr) : launch_dwr_shape<8, 32>(c, dz, x, dwr);
}

}  // namespace mok
