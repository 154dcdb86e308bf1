// Router: logits, top-k selection and gates in one kernel.
//
// Top-k gating (kwkr.cn MoK explainer, section 4.1). The routing decision is an
// integer result that has to be reproducible bit for bit, so the logit of each
// (token, expert) is a fixed-order fp32 fused-multiply-add chain over h
// ascending, computed on the vector ALU (an MFMA would sum in an unspecified
// internal order). Independent chains are interleaved across registers and
// lanes; no single chain is reordered.
//
// Two workgroup layouts, both with every chain a sequential fp32 FMA over h:
//  * large batches (route_lds_kernel): 256 threads, TT = 4*TPT tokens x all E
//    experts; lane l of wave w owns tokens w*TPT.. and experts l + 64*q; 16-h chunks
//    of x and Wr are staged in LDS as fp32, so each bf16 value is unpacked once per
//    workgroup; after the H loop every wave holds complete logit rows for its tokens.
//  * small batches (route_kernel): 64*EPT threads, thread e owns expert e (its Wr row
//    streams through registers) for TT = 8..32 tokens whose x rows are wave-uniform
//    (scalar loads feeding the FMA's scalar operand), so a 2048-token batch still
//    spreads over every compute unit; logits go through LDS once before selection.
// Selection: k rounds of a wave arg-max with butterfly shuffles.
#include "kernels.h"

namespace mok {

constexpr int kRouteHC = 16;  // h values per LDS chunk (LDS layout)
constexpr int kNoExpert = 0x7FFFFFFF;

// Strict total order of candidates: larger value first; equal values
// (-0 == +0) by lower expert; NaN below every number; "no candidate" last.
__device__ __forceinline__ bool better(float a, int ea, float b, int eb) {
  if (eb == kNoExpert) return ea != kNoExpert;
  if (ea == kNoExpert) return false;
  const bool na = a != a, nb = b != b;
  if (na || nb) return (!na && nb) || (na && nb && ea < eb);
  return a > b || (a == b && ea < eb);
}

template <typename T, int TPT, int EPT>
__global__ __launch_bounds__(256) void route_lds_kernel(const T* __restrict__ x, const T* __restrict__ wr,
                                                    const float* __restrict__ bias, int32_t* __restrict__ idx,
                                                    float* __restrict__ gate, float* __restrict__ logits, int64_t Tn,
                                                    int H, int E, int k) {
  constexpr int TT = 4 * TPT;
  constexpr int EC = 64 * EPT;
  constexpr int VE = Elem<T>::VE;
  constexpr int VPR = kRouteHC / VE;  // 16-byte vectors per row chunk
  __shared__ float sx[TT][kRouteHC];
  __shared__ float sw[kRouteHC][EC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TT;

  float acc[TPT][EPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int q = 0; q < EPT; ++q) acc[i][q] = 0.0f;

  for (int h0 = 0; h0 < H; h0 += kRouteHC) {
    for (int i = tid; i < TT * VPR; i += 256) {
      const int t = i / VPR, vv = i % VPR;
      const int64_t tok = t0 + t;
      float f[VE];
      if (tok < Tn) {
        unpack(ldg16(x + tok * H + h0 + vv * VE), f, (T*)nullptr);
      } else {
#pragma unroll
        for (int q = 0; q < VE; ++q) f[q] = 0.0f;
      }
#pragma unroll
      for (int q = 0; q < VE; ++q) sx[t][vv * VE + q] = f[q];
    }
    for (int i = tid; i < EC * VPR; i += 256) {
      const int e = i / VPR, vv = i % VPR;
      float f[VE];
      if (e < E) {
        unpack(ldg16(wr + (int64_t)e * H + h0 + vv * VE), f, (T*)nullptr);
      } else {
#pragma unroll
        for (int q = 0; q < VE; ++q) f[q] = 0.0f;
      }
#pragma unroll
      for (int q = 0; q < VE; ++q) sw[vv * VE + q][e] = f[q];
    }
    __syncthreads();
#pragma unroll 4
    for (int hh = 0; hh < kRouteHC; ++hh) {
      float xv[TPT], wv[EPT];
#pragma unroll
      for (int i = 0; i < TPT; ++i) xv[i] = sx[wave * TPT + i][hh];
#pragma unroll
      for (int q = 0; q < EPT; ++q) wv[q] = sw[hh][lane + 64 * q];
#pragma unroll
      for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int q = 0; q < EPT; ++q) acc[i][q] = __builtin_fmaf(xv[i], wv[q], acc[i][q]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int64_t tok = t0 + wave * TPT + i;
    if (tok < Tn) {  // uniform across the wave
      float v[EPT];
#pragma unroll
      for (int q = 0; q < EPT; ++q) {
        const int e = lane + 64 * q;
        v[q] = acc[i][q];
        if (bias != nullptr && e < E) v[q] = v[q] + bias[e];
        if (logits != nullptr && e < E) logits[tok * E + e] = v[q];
      }
      // k rounds of wave arg-max; lane j keeps slot j's expert and exp(z_j - z_0)
      uint32_t taken = 0;
      float z0 = 0.0f, s = 0.0f, my_ex = 0.0f;
      int my_e = 0;
#pragma unroll 1
      for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int be = kNoExpert;
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
          const int e = lane + 64 * q;
          if (e < E && !((taken >> q) & 1u) && better(v[q], e, bv, be)) {
            bv = v[q];
            be = e;
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const float ov = __shfl_xor(bv, off);
          const int oe = __shfl_xor(be, off);
          if (better(ov, oe, bv, be)) {
            bv = ov;
            be = oe;
          }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (j == 0) z0 = bv;
        const float ex = expf(bv - z0);  // softmax over the selected logits, summed in slot order
        s = s + ex;
        if (lane == j) {
          my_e = be;
          my_ex = ex;
        }
      }
      if (lane < k) {
        idx[tok * k + lane] = my_e;
        gate[tok * k + lane] = my_ex / s;
      }
    }
  }
}

template <typename T, int TT, int EPT>
__global__ __launch_bounds__(1024) void route_kernel(const T* __restrict__ x, const T* __restrict__ wr,
                                                     const float* __restrict__ bias, int32_t* __restrict__ idx,
                                                     float* __restrict__ gate, float* __restrict__ logits,
                                                     int64_t Tn, int H, int E, int k) {
  constexpr int VE = Elem<T>::VE;
  constexpr int EC = 64 * EPT;
  __shared__ float sz[TT][EC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int e = tid;
  const T* wrow = wr + (int64_t)(e < E ? e : 0) * H;
  // rows past the end re-read the last token; their results are dropped
  const T* xr = x + min(t0, Tn - 1) * (int64_t)H;
  const int nt = (int)min<int64_t>(TT, Tn - t0);

  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.0f;
#pragma unroll 2
  for (int h0 = 0; h0 < H; h0 += VE) {
    float w[VE];
    unpack(ldg16(wrow + h0), w, (T*)nullptr);
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      float xv[VE];
      unpack(ldg16(xr + (int64_t)(i < nt ? i : 0) * H + h0), xv, (T*)nullptr);
#pragma unroll
      for (int j = 0; j < VE; ++j) acc[i] = __builtin_fmaf(xv[j], w[j], acc[i]);
    }
  }
  const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const float v = bias != nullptr ? acc[i] + b : acc[i];
    sz[i][e] = v;
    if (logits != nullptr && e < E && i < nt) logits[(t0 + i) * E + e] = v;
  }
  __syncthreads();

  for (int i = wave; i < nt; i += EPT) {
    const int64_t tok = t0 + i;
    float v[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) v[q] = sz[i][lane + 64 * q];
    // k rounds of wave arg-max; lane j keeps slot j's expert and exp(z_j - z_0)
    uint32_t taken = 0;
    float z0 = 0.0f, s = 0.0f, my_ex = 0.0f;
    int my_e = 0;
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
      float bv = 0.0f;
      int be = kNoExpert;
#pragma unroll
      for (int q = 0; q < EPT; ++q) {
        const int ee = lane + 64 * q;
        if (ee < E && !((taken >> q) & 1u) && better(v[q], ee, bv, be)) {
          bv = v[q];
          be = ee;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (better(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (j == 0) z0 = bv;
      const float ex = expf(bv - z0);  // softmax over the selected logits, summed in slot order
      s = s + ex;
      if (lane == j) {
        my_e = be;
        my_ex = ex;
      }
    }
    if (lane < k) {
      idx[tok * k + lane] = my_e;
      gate[tok * k + lane] = my_ex / s;
    }
  }
}

template <typename T, int TT, int EPT>
static hipError_t launch_route_t(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx,
                                 float* gate, float* logits) {
  const int64_t blocks = (c.T + TT - 1) / TT;
  hipLaunchKernelGGL((route_kernel<T, TT, EPT>), dim3((unsigned)blocks), dim3(64 * EPT), 0, c.s, (const T*)x,
                     (const T*)wr, bias, idx, gate, logits, c.T, c.H, c.E, c.k);
  return hipGetLastError();
}

template <typename T, int TPT, int EPT>
static hipError_t launch_route_lds(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx,
                                   float* gate, float* logits) {
  const int64_t blocks = (c.T + 4 * TPT - 1) / (4 * TPT);
  hipLaunchKernelGGL((route_lds_kernel<T, TPT, EPT>), dim3((unsigned)blocks), dim3(256), 0, c.s, (const T*)x,
                     (const T*)wr, bias, idx, gate, logits, c.T, c.H, c.E, c.k);
  return hipGetLastError();
}

// Layout choice: the LDS layout once 32-token workgroups give at least two per
// compute unit; otherwise the register layout with the largest of 32/16/8 tokens
// per workgroup that still gives two per compute unit (each reads all of Wr).
template <typename T, int EPT>
static hipError_t route_tt(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx, float* gate,
                           float* logits) {
  int cus = 256;
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  constexpr int TPT = EPT <= 8 ? 8 : 4;
  if (c.T >= 4LL * TPT * 2 * cus) return launch_route_lds<T, TPT, EPT>(c, x, wr, bias, idx, gate, logits);
  if (c.T >= 16LL * 2 * cus) return launch_route_t<T, 16, EPT>(c, x, wr, bias, idx, gate, logits);
  return launch_route_t<T, 8, EPT>(c, x, wr, bias, idx, gate, logits);
}

template <typename T>
static hipError_t route_dispatch(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx,
                                 float* gate, float* logits) {
  const int ept = (c.E + 63) / 64;
  switch (ept) {
#define MOK_ROUTE_CASE(N) \
  case N:                 \
    return route_tt<T, N>(c, x, wr, bias, idx, gate, logits);
    MOK_ROUTE_CASE(1)
    MOK_ROUTE_CASE(2)
    MOK_ROUTE_CASE(3)
    MOK_ROUTE_CASE(4)
    MOK_ROUTE_CASE(5)
    MOK_ROUTE_CASE(6)
    MOK_ROUTE_CASE(7)
    MOK_ROUTE_CASE(8)
    MOK_ROUTE_CASE(9)
    MOK_ROUTE_CASE(10)
    MOK_ROUTE_CASE(11)
    MOK_ROUTE_CASE(12)
    MOK_ROUTE_CASE(13)
    MOK_ROUTE_CASE(14)
    MOK_ROUTE_CASE(15)
    MOK_ROUTE_CASE(16)
#undef MOK_ROUTE_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_route(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx, float* gate,
                        float* logits) {
  if (c.T == 0) return hipSuccess;
  return c.act == MOK_F32 ? route_dispatch<float>(c, x, wr, bias, idx, gate, logits)
                          : route_dispatch<bf16>(c, x, wr, bias, idx, gate, logits);
}

}  // namespace mok
