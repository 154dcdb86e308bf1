// Router: logits, top-k selection and gates in one kernel.
//
// Top-k gating (kwkr.cn MoK explainer, section 4.1). The routing decision is an
// integer result that has to be reproducible bit for bit, so the logit of each
// (token, expert) is a fixed-order fp32 fused-multiply-add chain over h
// ascending, computed on the vector ALU (an MFMA would sum in an unspecified
// internal order). Independent chains are interleaved across registers and
// lanes; no single chain is reordered.
//
// Workgroup: 64*EPT threads, thread e owns expert e for TT = 4, 8, 16 or 32 tokens, so
// even a 2048-token micro-batch spreads over every compute unit (two workgroups each). Each thread streams
// its Wr row through registers one 64-h chunk ahead of use (cover for L2 latency);
// 64-h chunks of the TT x rows are unpacked to fp32 in LDS once per workgroup
// (double-buffered) and read by every lane at the same address (a broadcast). Every
// logit is a sequential fp32 FMA chain over h. Logits go through LDS once; then
// selection: k rounds of a wave arg-max with butterfly shuffles.
#include "kernels.h"

namespace mok {

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

// FULLX (small H, 4-token workgroups): the workgroup's x rows are unpacked into LDS for
// all of H at once (one load latency instead of one per chunk), each thread keeps its Wr
// row PD = 4 (bf16) or 2 (fp32) chunks ahead in registers, there is no barrier inside the
// h loop, and the 4 chains of a lane alternate instruction by instruction. Every chain is the same
// sequence of FMAs as in the chunked form. Measured at 2048 tokens, H = 1024, E = 32:
// 45 -> 37 us with the first three changes.
constexpr int kRouteFullXMaxH = 2048;

template <typename T, int TT, int EPT, bool FULLX = false>
__global__ __launch_bounds__(FULLX ? 64 * EPT : 1024) void route_kernel(const T* __restrict__ x, const T* __restrict__ wr,
                                                     const float* __restrict__ bias, int32_t* __restrict__ idx,
                                                     float* __restrict__ gate, float* __restrict__ logits,
                                                     int64_t Tn, int H, int E, int k) {
  constexpr int VE = Elem<T>::VE;
  constexpr int EC = 64 * EPT;
  constexpr int HC = 64;  // h per LDS chunk
  __shared__ __align__(16) float sx[FULLX ? 1 : 2][FULLX ? 1 : TT][HC];
  __shared__ __align__(16) float sxf[FULLX ? TT : 1][FULLX ? kRouteFullXMaxH : 4];
  __shared__ float sz[TT][EC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int nt = (int)min<int64_t>(TT, Tn - t0);
  const int e = tid;
  const T* wrow = wr + (int64_t)(e < E ? e : 0) * H;

  // x chunk -> fp32 in LDS, unpacked once per workgroup (rows past the end re-read the
  // last token; their results are dropped)
  const auto stage = [&](int h0, int buf) {
    for (int i = tid; i < TT * (HC / VE); i += EC) {
      const int t = i / (HC / VE), v = i % (HC / VE);
      const int64_t tok = t0 + (t < nt ? t : nt - 1);
      float f[VE];
      unpack(ldg16(x + tok * H + h0 + v * VE), f, (T*)nullptr);
#pragma unroll
      for (int q = 0; q < VE; q += 4)
        *reinterpret_cast<float4*>(&sx[buf][t][v * VE + q]) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
    }
  };
  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.0f;
  const int nc = H / HC;
  constexpr int NV = HC / VE;  // 16-byte Wr vectors per chunk
  if constexpr (FULLX) {
    for (int i = tid; i < TT * (H / VE); i += EC) {
      const int t = i / (H / VE), v = i % (H / VE);
      const int64_t tok = t0 + (t < nt ? t : nt - 1);
      float f[VE];
      unpack(ldg16(x + tok * H + v * VE), f, (T*)nullptr);
#pragma unroll
      for (int q = 0; q < VE; q += 4)
        *reinterpret_cast<float4*>(&sxf[t][v * VE + q]) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
    }
    constexpr int PD = sizeof(T) == 2 ? 4 : 2;  // fp32 rows: 2 chunks = 128 registers
    uint4 wb[PD][NV];
#pragma unroll
    for (int j = 0; j < PD - 1; ++j)
      if (j < nc) {
#pragma unroll
        for (int v = 0; v < NV; ++v) wb[j][v] = ldg16(wrow + j * HC + v * VE);
      }
    __syncthreads();
    for (int c0 = 0; c0 < nc; c0 += PD) {
      static_for<0, PD>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int c = c0 + j;
        if (c < nc) {
          if (c + PD - 1 < nc) {
#pragma unroll
            for (int v = 0; v < NV; ++v) wb[(j + PD - 1) % PD][v] = ldg16(wrow + (c + PD - 1) * HC + v * VE);
          }
          // the TT chains alternate FMA by FMA (each still runs over h in ascending order)
#pragma unroll
          for (int hv = 0; hv < HC; hv += VE) {
            float w[VE];
            unpack(wb[j][hv / VE], w, (T*)nullptr);
#pragma unroll
            for (int q = 0; q < VE; q += 4) {
              float4 xv[TT];
#pragma unroll
              for (int i = 0; i < TT; ++i) xv[i] = *reinterpret_cast<const float4*>(&sxf[i][c * HC + hv + q]);
#pragma unroll
              for (int i = 0; i < TT; ++i) acc[i] = __builtin_fmaf(xv[i].x, w[q], acc[i]);
#pragma unroll
              for (int i = 0; i < TT; ++i) acc[i] = __builtin_fmaf(xv[i].y, w[q + 1], acc[i]);
#pragma unroll
              for (int i = 0; i < TT; ++i) acc[i] = __builtin_fmaf(xv[i].z, w[q + 2], acc[i]);
#pragma unroll
              for (int i = 0; i < TT; ++i) acc[i] = __builtin_fmaf(xv[i].w, w[q + 3], acc[i]);
            }
          }
        }
      });
    }
  } else {
  // this thread's Wr chunk in registers, loaded one chunk ahead (L2 latency cover)
  uint4 wv[NV], wn[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) wv[v] = ldg16(wrow + v * VE);
  stage(0, 0);
  __syncthreads();
  for (int c = 0; c < nc; ++c) {
    const int buf = c & 1;
    if (c + 1 < nc) {
      stage((c + 1) * HC, buf ^ 1);
#pragma unroll
      for (int v = 0; v < NV; ++v) wn[v] = ldg16(wrow + (c + 1) * HC + v * VE);
    }
#pragma unroll
    for (int hv = 0; hv < HC; hv += VE) {
      float w[VE];
      unpack(wv[hv / VE], w, (T*)nullptr);
#pragma unroll
      for (int i = 0; i < TT; ++i) {
#pragma unroll
        for (int q = 0; q < VE; q += 4) {
          const float4 xv = *reinterpret_cast<const float4*>(&sx[buf][i][hv + q]);  // same address in every lane
          acc[i] = __builtin_fmaf(xv.x, w[q], acc[i]);
          acc[i] = __builtin_fmaf(xv.y, w[q + 1], acc[i]);
          acc[i] = __builtin_fmaf(xv.z, w[q + 2], acc[i]);
          acc[i] = __builtin_fmaf(xv.w, w[q + 3], acc[i]);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) wv[v] = wn[v];
    __syncthreads();
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

// Few experts (E <= 32, H <= kRouteFullXMaxH): with one thread per expert a wave would
// leave 64 - E lanes idle and a 2048-token batch would give half a wave per SIMD. Here a
// one-wave workgroup holds G = 64 / EP tokens x EP experts (EP = E rounded up to a power
// of two, at least 8): lane (g, e) runs the chains of expert e for the TT tokens
// g, g + G, ... of the workgroup, so every lane has work and a 2048-token, 32-expert batch
// gives one wave per SIMD. The x rows are unpacked to fp32 in LDS for all of H (row pitch
// H + 4 floats, so the G rows a wave reads at once fall on different banks); each lane keeps
// its Wr row PD chunks ahead in registers. Every logit is the same sequential FMA chain
// over h as in route_kernel; selection runs on EP-lane segments of the wave (butterfly
// offsets below EP stay inside a segment), with the same order of candidates.
template <typename T, int EP, int TT>
__global__ __launch_bounds__(64) void route_few_kernel(const T* __restrict__ x, const T* __restrict__ wr,
                                                       const float* __restrict__ bias, int32_t* __restrict__ idx,
                                                       float* __restrict__ gate, float* __restrict__ logits,
                                                       int64_t Tn, int H, int E, int k) {
  constexpr int G = 64 / EP;
  constexpr int VE = Elem<T>::VE;
  constexpr int HC = 64;
  constexpr int NV = HC / VE;
  constexpr int PD = sizeof(T) == 2 ? 4 : 2;
  extern __shared__ __align__(16) float sxf[];  // [TT * G][H + 4]
  const int lane = threadIdx.x, g = lane / EP, e = lane % EP;
  const int XP = H + 4;
  const int64_t t0 = (int64_t)blockIdx.x * (TT * G);
  const int nt = (int)min<int64_t>(TT * G, Tn - t0);
  const T* wrow = wr + (int64_t)(e < E ? e : 0) * H;
  for (int i = lane; i < TT * G * (H / VE); i += 64) {
    const int r = i / (H / VE), v = i % (H / VE);
    const int64_t tok = t0 + (r < nt ? r : nt - 1);  // rows past the end re-read the last token
    float f[VE];
    unpack(ldg16(x + tok * H + v * VE), f, (T*)nullptr);
#pragma unroll
    for (int q = 0; q < VE; q += 4)
      *reinterpret_cast<float4*>(&sxf[r * XP + v * VE + q]) = make_float4(f[q], f[q + 1], f[q + 2], f[q + 3]);
  }
  const int nc = H / HC;
  uint4 wb[PD][NV];
#pragma unroll
  for (int j = 0; j < PD - 1; ++j)
    if (j < nc) {
#pragma unroll
      for (int v = 0; v < NV; ++v) wb[j][v] = ldg16(wrow + j * HC + v * VE);
    }
  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.0f;
  __syncthreads();
  for (int c0 = 0; c0 < nc; c0 += PD) {
    static_for<0, PD>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int c = c0 + j;
      if (c < nc) {
        if (c + PD - 1 < nc) {
#pragma unroll
          for (int v = 0; v < NV; ++v) wb[(j + PD - 1) % PD][v] = ldg16(wrow + (c + PD - 1) * HC + v * VE);
        }
#pragma unroll
        for (int hv = 0; hv < HC; hv += VE) {
          float w[VE];
          unpack(wb[j][hv / VE], w, (T*)nullptr);
#pragma unroll
          for (int q = 0; q < VE; q += 4) {
            float4 xv[TT];
#pragma unroll
            for (int i = 0; i < TT; ++i)
              xv[i] = *reinterpret_cast<const float4*>(&sxf[(g + G * i) * XP + c * HC + hv + q]);
#pragma unroll
            for (int i = 0; i < TT; ++i) acc[i] = __builtin_fmaf(xv[i].x, w[q], acc[i]);
#pragma unroll
            for (int i = 0; i < TT; ++i) acc[i] = __builtin_fmaf(xv[i].y, w[q + 1], acc[i]);
#pragma unroll
            for (int i = 0; i < TT; ++i) acc[i] = __builtin_fmaf(xv[i].z, w[q + 2], acc[i]);
#pragma unroll
            for (int i = 0; i < TT; ++i) acc[i] = __builtin_fmaf(xv[i].w, w[q + 3], acc[i]);
          }
        }
      }
    });
  }
  const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const int r = g + G * i;  // token row of this chain in the workgroup
    const float v = bias != nullptr ? acc[i] + b : acc[i];
    if (logits != nullptr && e < E && r < nt) logits[(t0 + r) * E + e] = v;
    // k rounds of segment arg-max; lane j of the segment keeps slot j's expert and exp(z_j - z_0)
    bool taken = false;
    float z0 = 0.0f, s = 0.0f, my_ex = 0.0f;
    int my_e = 0;
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
      float bv = 0.0f;
      int be = kNoExpert;
      if (e < E && !taken) {
        bv = v;
        be = e;
      }
#pragma unroll
      for (int off = EP / 2; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (better(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      if (be == e) taken = true;
      if (j == 0) z0 = bv;
      const float ex = expf(bv - z0);  // softmax over the selected logits, summed in slot order
      s = s + ex;
      if (e == j) {
        my_e = be;
        my_ex = ex;
      }
    }
    if (e < k && r < nt) {
      idx[(t0 + r) * k + e] = my_e;
      gate[(t0 + r) * k + e] = my_ex / s;
    }
  }
}

constexpr size_t kRouteFewMaxLds = 64 * 1024;

// Chains per lane of route_few_kernel: one while that leaves at most four waves per CU,
// else two; 0 when the x rows do not fit the LDS.
template <int EP>
static int route_few_tt(const Ctx& c) {
  constexpr int G = 64 / EP;
  const int cus = c.num_cu > 0 ? c.num_cu : 256;
  const int tt = c.T <= 4LL * G * cus ? 1 : 2;
  return (size_t)tt * G * (c.H + 4) * 4 <= kRouteFewMaxLds ? tt : 0;
}

template <typename T, int EP>
static hipError_t launch_route_few(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx,
                                   float* gate, float* logits) {
  constexpr int G = 64 / EP;
  if (route_few_tt<EP>(c) == 1) {
    const size_t lds = (size_t)G * (c.H + 4) * 4;
    hipLaunchKernelGGL((route_few_kernel<T, EP, 1>), dim3((unsigned)((c.T + G - 1) / G)), dim3(64), lds, c.s,
                       (const T*)x, (const T*)wr, bias, idx, gate, logits, c.T, c.H, c.E, c.k);
  } else {
    const size_t lds = (size_t)2 * G * (c.H + 4) * 4;
    hipLaunchKernelGGL((route_few_kernel<T, EP, 2>), dim3((unsigned)((c.T + 2 * G - 1) / (2 * G))), dim3(64), lds,
                       c.s, (const T*)x, (const T*)wr, bias, idx, gate, logits, c.T, c.H, c.E, c.k);
  }
  return hipGetLastError();
}

template <typename T, int TT, int EPT>
static hipError_t launch_route_t(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx,
                                 float* gate, float* logits) {
  const int64_t blocks = (c.T + TT - 1) / TT;
  if constexpr (TT == 4 && EPT <= 2) {
    if (c.H <= kRouteFullXMaxH) {
      hipLaunchKernelGGL((route_kernel<T, TT, EPT, true>), dim3((unsigned)blocks), dim3(64 * EPT), 0, c.s,
                         (const T*)x, (const T*)wr, bias, idx, gate, logits, c.T, c.H, c.E, c.k);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((route_kernel<T, TT, EPT>), dim3((unsigned)blocks), dim3(64 * EPT), 0, c.s, (const T*)x,
                     (const T*)wr, bias, idx, gate, logits, c.T, c.H, c.E, c.k);
  return hipGetLastError();
}

// Tokens per workgroup: the largest of 32/16/8/4 that still gives at least two
// workgroups per compute unit (each workgroup streams all of Wr once; at 2048 tokens
// 4 beats 8 by a fifth, 2 loses to 4).
template <typename T, int EPT>
static hipError_t route_tt(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx, float* gate,
                           float* logits) {
  const int cus = c.num_cu > 0 ? c.num_cu : 256;
  if (c.T >= 32LL * 2 * cus) return launch_route_t<T, 32, EPT>(c, x, wr, bias, idx, gate, logits);
  if (c.T >= 16LL * 2 * cus) return launch_route_t<T, 16, EPT>(c, x, wr, bias, idx, gate, logits);
  if (c.T >= 8LL * 2 * cus) return launch_route_t<T, 8, EPT>(c, x, wr, bias, idx, gate, logits);
  return launch_route_t<T, 4, EPT>(c, x, wr, bias, idx, gate, logits);
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

static int route_few_ep(const Ctx& c) {
  if (c.E > 32 || c.H > kRouteFullXMaxH) return 0;
  const int ep = c.E <= 8 ? 8 : (c.E <= 16 ? 16 : 32);
  const int tt = ep == 8 ? route_few_tt<8>(c) : (ep == 16 ? route_few_tt<16>(c) : route_few_tt<32>(c));
  return tt > 0 ? ep : 0;
}

template <typename T>
static hipError_t route_few(const Ctx& c, int ep, const void* x, const void* wr, const float* bias, int32_t* idx,
                            float* gate, float* logits) {
  if (ep == 8) return launch_route_few<T, 8>(c, x, wr, bias, idx, gate, logits);
  if (ep == 16) return launch_route_few<T, 16>(c, x, wr, bias, idx, gate, logits);
  return launch_route_few<T, 32>(c, x, wr, bias, idx, gate, logits);
}

hipError_t launch_route(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx, float* gate,
                        float* logits) {
  if (c.T == 0) return hipSuccess;
  if (const int ep = route_few_ep(c))
    return c.act == MOK_F32 ? route_few<float>(c, ep, x, wr, bias, idx, gate, logits)
                            : route_few<bf16>(c, ep, x, wr, bias, idx, gate, logits);
  return c.act == MOK_F32 ? route_dispatch<float>(c, x, wr, bias, idx, gate, logits)
                          : route_dispatch<bf16>(c, x, wr, bias, idx, gate, logits);
}

}  // namespace mok
