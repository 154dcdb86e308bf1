// MX quantisers (MXFP8 and MXFP4 elements, template parameter F of MxFmt) and the
// deferred weight-gradient bookkeeping (HBM-bound kernels).
//
//  quant_rows   blocks of 32 along each row: x and dY rows (K = H of fc1 / dh) and the
//               forward weight orientations W1 (rows along H) and W2 (rows along I).
//  quant_cols   blocks of 32 along the row axis, written transposed (feature-major,
//               K = rows contiguous): W2^T and W1^T for dh / dx, and the token-axis
//               operands of the weight-gradient GEMMs (dO, h, dGU, x over each
//               expert's routed rows of the whole step).
//  flush_table  per expert: rows over all stashed micro-batches, and the K offset of its
//               segment in the token-axis operands (segments padded to a whole K-tile,
//               128 rows for MXFP8 and 256 for MXFP4, with zero rows, i.e. all-zero
//               blocks, which add nothing).
//  rowmap       padded segment row -> stash row (micro-batch m's routed row r is stash
//               row m*R + r); -1 for padding.
//  dwr_stash    dWr[e] = sum over e's rows of the step (micro-batch then slot order) of
//               dz_s * x_t: 8 fixed chunks of consecutive rows summed row by row, then the
//               chunk sums in ascending order.
#include "gemm.h"
#include "kernels.h"
#include "mx.h"

namespace mok {

static unsigned nblk(int64_t n, int b = 256) { return (unsigned)((n + b - 1) / b); }

// nvec = (rows * F) / 16 sixteen-element vectors; F % 32 == 0, so vector pairs
// (2j, 2j+1) are exactly the 32-element blocks and block b's scale is s[b].
// Scale byte of block b (32 features) of row r: row-major (kmaj_rows = 0) at
// r * F/32 + b; K-tile-major (kmaj_rows > 0 = rows per matrix) at
// [z][b/4][r % kmaj_rows][b % 4] with z = r / kmaj_rows.
template <int FM>
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(Guard gd, const bf16* __restrict__ src, int64_t nvec,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ s, int F,
                                                            int64_t kmaj_rows) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (guard_fail(gd) || v >= nvec) return;  // nvec and blockDim are even: a pair leaves together
  float f[16];
  load16<bf16>(src + v * 16, f);
  const uint32_t sb = MxFmt<FM>::quant_store16(f, q, v * 16);
  if ((v & 1) == 0) {
    int64_t i = v >> 1;
    if (kmaj_rows > 0) {
      const int64_t nb = F / 32, row = i / nb, b = i - row * nb, z = row / kmaj_rows, r = row - z * kmaj_rows;
      i = z * kmaj_rows * nb + (b >> 2) * kmaj_rows * 4 + r * 4 + (b & 3);
    }
    s[i] = (uint8_t)sb;
  }
}

hipError_t launch_mx_quant_rows(const Ctx& c, const void* src, int64_t rows, int F, void* q, void* s,
                                int64_t kmaj_rows) {
  const int64_t nvec = rows * (F / 16);
  if (nvec == 0) return hipSuccess;
  if (c.mx4)
    hipLaunchKernelGGL(mx_quant_rows_kernel<1>, dim3(nblk(nvec)), dim3(256), 0, c.s, c.guard, (const bf16*)src, nvec,
                       (uint8_t*)q, (uint8_t*)s, F, kmaj_rows);
  else
    hipLaunchKernelGGL(mx_quant_rows_kernel<0>, dim3(nblk(nvec)), dim3(256), 0, c.s, c.guard, (const bf16*)src, nvec,
                       (uint8_t*)q, (uint8_t*)s, F, kmaj_rows);
  return hipGetLastError();
}

// Transposing quantiser. Matrix z = blockIdx.z; logical row r in [0, K) reads
// physical row rowmap[r] (rowmap != nullptr; < 0 = zero row) or r of
// src + z * src_mat, ld elements per physical row; feature f in [0, F).
// Writes element q[(z*F + f) * out_ld + r] (out_ld in elements) and the scale of block
// b = r/32 K-tile-major,
// s[z*F*(out_ld/32) + (b/4)*F*4 + f*4 + b%4]: each 128-row K-tile's scale dwords of
// consecutive features are contiguous.
// Workgroup: 128 logical rows x 64 features. Wave w quantises features 16w .. 16w+15;
// lane l takes feature 16w + l/4 and row block l%4, so the 4 lanes of a feature write
// its 128 consecutive output bytes (and 4 consecutive scale bytes) together. In LDS (row
// pitch 65 floats), the rows of row blocks 2 and 3 are stored rotated by 16 columns: the
// 64 lanes of a column read (16 features x 4 row blocks) then start on 64 different
// 4-byte banks modulo 256 bytes (and cover each bank of a 128-byte window twice). Row
// blocks at or past *kdev (when given) are skipped.
struct ColQuantArgs {
  const bf16* src;
  int64_t src_mat, ld;
  const int32_t* rowmap;
  const int32_t* kdev;
  int F;
  int64_t out_ld;
  uint8_t* q;
  uint8_t* s;
  Guard guard;
};

template <int FM>
__global__ __launch_bounds__(256) void mx_quant_cols_kernel(ColQuantArgs a) {
  // The 128-row x 64-feature tile as raw bf16 (16.5 KB, so eight workgroups share a CU),
  // row pitch 66 elements (33 dwords): with rows 64..127 rotated by 16 columns, the column
  // reads of a wave below fall on distinct banks.
  constexpr int TP = 66;
  __shared__ __align__(16) uint16_t tile[128 * TP];
  const int r0 = blockIdx.x * 128, f0 = blockIdx.y * 64, z = blockIdx.z;
  if (guard_fail(a.guard) || (a.kdev != nullptr && r0 >= *a.kdev)) return;
  const bf16* src = a.src + (int64_t)z * a.src_mat;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = threadIdx.x + 256 * i;  // 128 rows x 8 vectors of 8 features
    const int row = v >> 3, c8 = (v & 7) * 8;
    const int r = r0 + row;
    const int64_t p = a.rowmap != nullptr ? (int64_t)a.rowmap[r] : (int64_t)r;
    const uint4 raw = p >= 0 ? ldg16(src + p * a.ld + f0 + c8) : make_uint4(0u, 0u, 0u, 0u);
    const int pc = (c8 + 16 * ((row >> 6) & 1)) & 63;
    uint32_t* t32 = reinterpret_cast<uint32_t*>(tile + row * TP + pc);
    t32[0] = raw.x;
    t32[1] = raw.y;
    t32[2] = raw.z;
    t32[3] = raw.w;
  }
  const auto at = [&](int row, int col) { return __uint_as_float((uint32_t)tile[row * TP + col] << 16); };
  __syncthreads();
  const int f = 16 * (threadIdx.x >> 6) + ((threadIdx.x & 63) >> 2), b = threadIdx.x & 3;
  const int pf = (f + 16 * (b >> 1)) & 63;  // rows 32b .. 32b+31 all carry the same rotation
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(at(32 * b + i, pf)));
  const int64_t orow = (int64_t)z * a.F + f0 + f;
  uint32_t sb;
  if constexpr (FM == 0) {
    sb = mx_scale_byte(m);
    const float inv = mx_inv_scale(sb);
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = 32 * b + 4 * j;
      w[j] = mx_pack4(at(i, pf), at(i + 1, pf), at(i + 2, pf), at(i + 3, pf), inv);
    }
    uint8_t* qo = a.q + orow * a.out_ld + r0 + 32 * b;
    stg16(qo, make_uint4(w[0], w[1], w[2], w[3]));
    stg16(qo + 16, make_uint4(w[4], w[5], w[6], w[7]));
  } else {
    sb = mx4_scale_byte(m);
    const float inv = mx_inv_scale(sb);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i >> 3] |= e2m1_code(at(32 * b + i, pf) * inv) << (4 * (i & 7));
    stg16(a.q + orow * (a.out_ld / 2) + (r0 + 32 * b) / 2, make_uint4(w[0], w[1], w[2], w[3]));
  }
  const int64_t kb = r0 / 32 + b;
  a.s[(int64_t)z * a.F * (a.out_ld / 32) + (kb >> 2) * a.F * 4 + (int64_t)(f0 + f) * 4 + (kb & 3)] = (uint8_t)sb;
}

hipError_t launch_mx_quant_cols(const Ctx& c, const void* src, int64_t src_mat, int64_t ld, const int32_t* rowmap,
                                const int32_t* kdev, int K, int F, int mats, int64_t out_ld, void* q, void* s) {
  if (K == 0 || F == 0 || mats == 0) return hipSuccess;
  ColQuantArgs a{(const bf16*)src, src_mat, ld, rowmap, kdev, F, out_ld, (uint8_t*)q, (uint8_t*)s, c.guard};
  if (c.mx4)
    hipLaunchKernelGGL(mx_quant_cols_kernel<1>, dim3(K / 128, F / 64, mats), dim3(256), 0, c.s, a);
  else
    hipLaunchKernelGGL(mx_quant_cols_kernel<0>, dim3(K / 128, F / 64, mats), dim3(256), 0, c.s, a);
  return hipGetLastError();
}

// One workgroup of 1024 threads (E <= 1024). counts is [M][E].
__global__ __launch_bounds__(1024) void mx_flush_table_kernel(Guard gd, const int32_t* __restrict__ counts, int M,
                                                              int E, int kt, int32_t* __restrict__ gcnt,
                                                              int32_t* __restrict__ pofs) {
  __shared__ int sc[1024];
  if (guard_fail(gd)) return;
  const int e = threadIdx.x;
  int c = 0;
  if (e < E)
    for (int m = 0; m < M; ++m) c += counts[(int64_t)m * E + e];
  const int p = (c + kt - 1) / kt * kt;
  sc[e] = p;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan
    const int v = e >= d ? sc[e - d] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) {
    gcnt[e] = c;
    pofs[e] = sc[e] - p;
  }
  if (e == E - 1) pofs[E] = sc[e];
}

// offsets is [M][E+1]; one thread per padded row p < kmax.
__global__ __launch_bounds__(256) void mx_rowmap_kernel(Guard gd, const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ offsets, int M, int E, int R,
                                                        const int32_t* __restrict__ gcnt,
                                                        const int32_t* __restrict__ pofs, int64_t kmax,
                                                        int32_t* __restrict__ rowmap) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (guard_fail(gd) || p >= kmax || p >= pofs[E]) return;
  int lo = 0, hi = E;  // pofs[lo] <= p < pofs[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pofs[mid] <= p) lo = mid; else hi = mid;
  }
  const int e = lo;
  int j = (int)(p - pofs[e]);
  int out = -1;
  if (j < gcnt[e]) {
    for (int m = 0; m < M; ++m) {
      const int cm = counts[(int64_t)m * E + e];
      if (j < cm) {
        out = m * R + offsets[(int64_t)m * (E + 1) + e] + j;
        break;
      }
      j -= cm;
    }
  }
  rowmap[p] = out;
}

hipError_t launch_mx_flush_table(const Ctx& c, const int32_t* counts, const int32_t* offsets, int M, int32_t* gcnt,
                                 int32_t* pofs, int64_t kmax, int32_t* rowmap) {
  hipLaunchKernelGGL(mx_flush_table_kernel, dim3(1), dim3(1024), 0, c.s, c.guard, counts, M, c.E, c.mx4 ? 256 : 128,
                     gcnt, pofs);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(mx_rowmap_kernel, dim3(nblk(kmax)), dim3(256), 0, c.s, c.guard, counts, offsets, M, c.E, c.R, gcnt, pofs,
                     kmax, rowmap);
  return hipGetLastError();
}

// dz and perm are [M][R] (micro-batch m's slot-indexed dz and its schedule perm);
// xs is [M*R][H] (micro-batch m's x rows in routed order at rows m*R ..).
// dWr[e] = sum over kDwrChunks consecutive chunks of e's rows (chunk c = rows
// [c*n/kDwrChunks, (c+1)*n/kDwrChunks) in step order), each summed row by row with fp32
// fused multiply-adds, the chunk sums added in ascending order: a hot expert's rows are
// spread over kDwrChunks threads per column.
constexpr int kDwrChunks = 8;

__global__ __launch_bounds__(256) void dwr_stash_part_kernel(Guard gd, const float* __restrict__ dz,
                                                             const int32_t* __restrict__ perm,
                                                             const bf16* __restrict__ xs,
                                                             const int32_t* __restrict__ gcnt,
                                                             const int32_t* __restrict__ pofs,
                                                             const int32_t* __restrict__ rowmap,
                                                             float* __restrict__ part, int E, int H, int R) {
  const int vpr = H / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (guard_fail(gd) || gid >= (int64_t)E * kDwrChunks * vpr) return;
  const int h0 = (int)(gid % vpr) * 8;
  const int64_t ec = gid / vpr;
  const int c = (int)(ec % kDwrChunks), e = (int)(ec / kDwrChunks);
  const int n = gcnt[e];
  const int j0 = (int)((int64_t)c * n / kDwrChunks), j1 = (int)((int64_t)(c + 1) * n / kDwrChunks);
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  const int32_t* rm = rowmap + pofs[e];
  for (int j = j0; j < j1; ++j) {
    const int row = rm[j];
    const int m = row / R;
    const float d = dz[(int64_t)m * R + perm[row]];
    float f[8];
    unpack(ldg16(xs + (int64_t)row * H + h0), f, (bf16*)nullptr);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = __builtin_fmaf(d, f[q], acc[q]);
  }
  float* o = part + ((int64_t)e * kDwrChunks + c) * H + h0;
  *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

template <typename TO>
__global__ __launch_bounds__(256) void dwr_stash_sum_kernel(Guard gd, const float* __restrict__ part,
                                                            TO* __restrict__ dwr, int E, int H) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (guard_fail(gd) || gid >= (int64_t)E * H) return;
  const int64_t e = gid / H, h = gid % H;
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kDwrChunks; ++c) s += part[(e * kDwrChunks + c) * H + h];
  Elem<TO>::put(dwr, gid, s);
}

hipError_t launch_dwr_stash(const Ctx& c, const float* dz, const int32_t* perm, const void* xs, const int32_t* gcnt,
                            const int32_t* pofs, const int32_t* rowmap, float* part, void* dwr) {
  const int64_t n = (int64_t)c.E * kDwrChunks * (c.H / 8);
  hipLaunchKernelGGL(dwr_stash_part_kernel, dim3(nblk(n)), dim3(256), 0, c.s, c.guard, dz, perm, (const bf16*)xs, gcnt, pofs,
                     rowmap, part, c.E, c.H, c.R);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int64_t m = (int64_t)c.E * c.H;
  if (c.wgrad_f32)
    hipLaunchKernelGGL((dwr_stash_sum_kernel<float>), dim3(nblk(m)), dim3(256), 0, c.s, c.guard, part, (float*)dwr, c.E, c.H);
  else
    hipLaunchKernelGGL((dwr_stash_sum_kernel<bf16>), dim3(nblk(m)), dim3(256), 0, c.s, c.guard, part, (bf16*)dwr, c.E, c.H);
  return hipGetLastError();
}

size_t dwr_stash_part_bytes(int E, int H) { return (size_t)E * kDwrChunks * H * sizeof(float); }

}  // namespace mok
