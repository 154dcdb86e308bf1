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
#include "elementwise.h"
#include "kernels.h"

namespace mok {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(Guard gd, const T* __restrict__ part,
                                                      const float* __restrict__ gate, T* __restrict__ y, int64_t T_,
                                                      int H, int k) {
  if (guard_fail(gd)) return;
  combine_body(part, gate, y, T_, H, k, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

__global__ __launch_bounds__(256) void router_gsum_kernel(Guard gd, const float* __restrict__ dgp,
                                                          const int32_t* __restrict__ perm,
                                                          float* __restrict__ dgate, int R, int nb) {
  if (guard_fail(gd)) return;
  router_gsum_body(dgp, perm, dgate, R, nb, blockIdx.x * blockDim.x + threadIdx.x);
}

__global__ __launch_bounds__(256) void router_dz_kernel(Guard gd, const float* __restrict__ dgate,
                                                        const float* __restrict__ gate, float* __restrict__ dz,
                                                        int64_t T_, int k) {
  if (guard_fail(gd)) return;
  router_dz_body(dgate, gate, dz, T_, k, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

template <typename T>
__global__ __launch_bounds__(256) void dx_reduce_kernel(Guard gd, const T* __restrict__ part,
                                                        const float* __restrict__ dz, const int32_t* __restrict__ idx,
                                                        const T* __restrict__ wr, T* __restrict__ dx, int64_t T_, int H,
                                                        int k) {
  if (guard_fail(gd)) return;
  dx_reduce_body(part, dz, idx, wr, dx, T_, H, k, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

template <typename T, typename TO, int kDwrVec, int kDwrLanes>
__global__ __launch_bounds__(kDwrVec * kDwrLanes) void dwr_kernel(Guard gd, const float* __restrict__ dz,
                                                                  const T* __restrict__ x,
                                                                  const int32_t* __restrict__ offsets,
                                                                  const int32_t* __restrict__ perm,
                                                                  TO* __restrict__ dwr, int E, int H, int k,
                                                                  T* __restrict__ xs) {
  __shared__ float red[kDwrLanes * (kDwrVec * Elem<T>::VE + 1)];
  if (guard_fail(gd)) return;
  dwr_body<T, TO, kDwrVec, kDwrLanes>(dz, x, offsets, perm, dwr, E, H, k, (int)blockIdx.x, red, xs);
}

__global__ __launch_bounds__(256) void gather_rows_kernel(Guard gd, const bf16* __restrict__ src,
                                                          const int32_t* __restrict__ perm,
                                                          const float* __restrict__ gate, bf16* __restrict__ dst, int R,
                                                          int H, int k) {
  if (guard_fail(gd)) return;
  gather_rows_body(src, perm, gate, dst, R, H, k, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
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
static hipError_t launch_dwr_shape(const Ctx& c, const float* dz, const void* x, void* dwr, void* xs) {
  const int ve = c.act == MOK_F32 ? 4 : 8;
  const int64_t nvb = ((int64_t)(c.H / ve) + VEC - 1) / VEC;
  const dim3 grid((unsigned)(c.E * nvb)), block(VEC * LANES);
  if (c.E * nvb == 0) return hipSuccess;
  if (c.act == MOK_F32) {
    hipLaunchKernelGGL((dwr_kernel<float, float, VEC, LANES>), grid, block, 0, c.s, c.guard, dz, (const float*)x, c.offsets,
                       c.perm, (float*)dwr, c.E, c.H, c.k, (float*)nullptr);
  } else if (c.wgrad_f32) {
    hipLaunchKernelGGL((dwr_kernel<bf16, float, VEC, LANES>), grid, block, 0, c.s, c.guard, dz, (const bf16*)x, c.offsets,
                       c.perm, (float*)dwr, c.E, c.H, c.k, (bf16*)xs);
  } else {
    hipLaunchKernelGGL((dwr_kernel<bf16, bf16, VEC, LANES>), grid, block, 0, c.s, c.guard, dz, (const bf16*)x, c.offsets,
                       c.perm, (bf16*)dwr, c.E, c.H, c.k, (bf16*)xs);
  }
  return hipGetLastError();
}

hipError_t launch_dwr(const Ctx& c, const float* dz, const void* x, void* dwr, void* xs) {
  return c.H <= 2048 ? launch_dwr_shape<4, 64>(c, dz, x, dwr, xs) : launch_dwr_shape<8, 32>(c, dz, x, dwr, xs);
}

}  // namespace mok
