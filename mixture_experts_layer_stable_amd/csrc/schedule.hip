// The single schedule table (dothoosh.com MoK page, "Technical details of the
// MoK mechanism": one schedule drives dispatch, combine, reverse-combine and
// reverse-dispatch).
//
// A stable counting sort of the R = T*k flat slots by expert, done without
// atomics so that it is exact and independent of scheduling:
//   1. count:  one wave per expert scans idx and counts its slots;
//   2. scan:   one workgroup forms exclusive offsets and per-expert tile starts
//              and writes the tile list (expert, first row, rows);
//   3. rank:   one wave per expert scans idx again in ascending slot order; a
//              slot's row is offsets[e] + number of earlier slots of e
//              (ballot + popcount), giving perm (row -> slot) and inv.
// The scan step also stamps the header (descriptor hash, tile height, tile
// capacity, status MOK_OK) that the forward and backward kernels check.
#include "kernels.h"

namespace mok {

struct Stamp {
  int32_t* hdr;
  uint32_t hash;
  int tile_m, max_tiles;
};

__device__ __forceinline__ void stamp_header(const Stamp& st) {
  st.hdr[0] = 0x4D4F4B53;
  st.hdr[kHdrHash] = (int32_t)st.hash;
  st.hdr[2] = st.tile_m;
  st.hdr[3] = st.max_tiles;
  st.hdr[kHdrStatus] = MOK_OK;
}

__global__ __launch_bounds__(64) void sched_count_kernel(const int32_t* __restrict__ idx, int R,
                                                         int32_t* __restrict__ counts) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int n4 = R >> 2;
  const int4* v4 = reinterpret_cast<const int4*>(idx);
  int cnt = 0;
  for (int i = lane; i < n4; i += 64) {
    const int4 q = v4[i];
    cnt += (q.x == e) + (q.y == e) + (q.z == e) + (q.w == e);
  }
  for (int i = (n4 << 2) + lane; i < R; i += 64) cnt += idx[i] == e;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
  if (lane == 0) counts[e] = cnt;
}

// Block-wide exclusive scan of one int per thread (1024 threads); returns the
// exclusive prefix and writes the total to *total.
__device__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = s_wave[w];
      s_wave[w] = acc;
      acc += t;
    }
    s_wave[nw] = acc;
  }
  __syncthreads();
  const int ex = s_wave[wave] + inc - v;
  *total = s_wave[nw];
  __syncthreads();
  return ex;
}

__global__ __launch_bounds__(1024) void sched_scan_kernel(const int32_t* __restrict__ counts, int E, int R, int BM,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tile_start,
                                                          int32_t* __restrict__ num_tiles, int4* __restrict__ tiles,
                                                          Stamp st) {
  __shared__ int s_wave[17];
  const int e = threadIdx.x;
  const int c = e < E ? counts[e] : 0;
  const int nt = (c + BM - 1) / BM;
  int tot_c, tot_t;
  const int off = block_exclusive_scan(c, s_wave, &tot_c);
  const int ts = block_exclusive_scan(nt, s_wave, &tot_t);
  if (e < E) {
    offsets[e] = off;
    tile_start[e] = ts;
    for (int m = 0; m < nt; ++m) tiles[ts + m] = make_int4(e, off + m * BM, min(BM, c - m * BM), 0);
  }
  if (e == 0) {
    offsets[E] = R;
    tile_start[E] = tot_t;
    *num_tiles = tot_t;
    stamp_header(st);
  }
}

__global__ __launch_bounds__(64) void sched_rank_kernel(const int32_t* __restrict__ idx, int R,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int e = blockIdx.x, lane = threadIdx.x;
  const int base = offsets[e];
  const uint64_t lt = (1ull << lane) - 1ull;
  const int n4 = R >> 2;
  const int4* v4 = reinterpret_cast<const int4*>(idx);
  int running = 0;
  for (int i0 = 0; i0 < n4; i0 += 64) {
    const int i = i0 + lane;
    int4 q = make_int4(-1, -1, -1, -1);
    if (i < n4) q = v4[i];
    const bool m0 = q.x == e, m1 = q.y == e, m2 = q.z == e, m3 = q.w == e;
    const uint64_t b0 = __ballot(m0), b1 = __ballot(m1), b2 = __ballot(m2), b3 = __ballot(m3);
    int r = running + __popcll(b0 & lt) + __popcll(b1 & lt) + __popcll(b2 & lt) + __popcll(b3 & lt);
    const int s = i << 2;
    if (m0) { perm[base + r] = s;     inv[s] = base + r;     ++r; }
    if (m1) { perm[base + r] = s + 1; inv[s + 1] = base + r; ++r; }
    if (m2) { perm[base + r] = s + 2; inv[s + 2] = base + r; ++r; }
    if (m3) { perm[base + r] = s + 3; inv[s + 3] = base + r; }
    running += __popcll(b0) + __popcll(b1) + __popcll(b2) + __popcll(b3);
  }
  for (int i0 = n4 << 2; i0 < R; i0 += 64) {
    const int s = i0 + lane;
    const bool m = s < R && idx[s] == e;
    const uint64_t b = __ballot(m);
    if (m) {
      const int r = running + __popcll(b & lt);
      perm[base + r] = s;
      inv[s] = base + r;
    }
    running += __popcll(b);
  }
}

// Tiny batches (R * E <= 2^14): the three steps in one workgroup of 16 waves, with idx
// staged in LDS; wave w counts and then ranks experts w, w + 16, ... as the per-expert
// waves above do (ranks by ascending slot), so every output is the same; two launches
// fewer. Measured: 64 tokens x 8 experts 11-14 -> 6 us; at 4096 routed rows x 32 experts
// the one workgroup takes 33 us against 19 us for the three kernels, hence the bound.
constexpr int kSchedFusedMaxR = 16384;

__global__ __launch_bounds__(1024) void sched_fused_kernel(const int32_t* __restrict__ idx, int R, int E, int BM,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ tile_start,
                                                           int32_t* __restrict__ num_tiles, int4* __restrict__ tiles,
                                                           int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                           Stamp st) {
  __shared__ int s_idx[kSchedFusedMaxR];
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1024];
  __shared__ int s_wave[17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < R; i += 1024) s_idx[i] = idx[i];
  __syncthreads();
  for (int e = wave; e < E; e += 16) {
    int cnt = 0;
    for (int i = lane; i < R; i += 64) cnt += s_idx[i] == e;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off);
    if (lane == 0) s_cnt[e] = cnt;
  }
  __syncthreads();
  const int e = tid;
  const int c = e < E ? s_cnt[e] : 0;
  const int nt = (c + BM - 1) / BM;
  int tot_c, tot_t;
  const int off = block_exclusive_scan(c, s_wave, &tot_c);
  const int ts = block_exclusive_scan(nt, s_wave, &tot_t);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    s_off[e] = off;
    tile_start[e] = ts;
    for (int m = 0; m < nt; ++m) tiles[ts + m] = make_int4(e, off + m * BM, min(BM, c - m * BM), 0);
  }
  if (e == 0) {
    offsets[E] = R;
    tile_start[E] = tot_t;
    *num_tiles = tot_t;
    stamp_header(st);
  }
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int ex = wave; ex < E; ex += 16) {
    const int base = s_off[ex];
    int running = 0;
    for (int i0 = 0; i0 < R; i0 += 64) {
      const int sl = i0 + lane;
      const bool m = sl < R && s_idx[sl] == ex;
      const uint64_t b = __ballot(m);
      if (m) {
        const int r = running + __popcll(b & lt);
        perm[base + r] = sl;
        inv[sl] = base + r;
      }
      running += __popcll(b);
    }
  }
}

hipError_t launch_schedule(const Ctx& c, const int32_t* idx) {
  const Stamp st{c.guard.hdr, c.guard.expect, c.BM, c.max_tiles};
  if (c.R <= kSchedFusedMaxR && c.E <= 1024 && (int64_t)c.R * c.E <= (int64_t)1 << 14) {
    hipLaunchKernelGGL(sched_fused_kernel, dim3(1), dim3(1024), 0, c.s, idx, c.R, c.E, c.BM, c.counts, c.offsets,
                       c.tile_start, c.num_tiles, c.tiles, c.perm, c.inv, st);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(sched_count_kernel, dim3(c.E), dim3(64), 0, c.s, idx, c.R, c.counts);
  hipLaunchKernelGGL(sched_scan_kernel, dim3(1), dim3(1024), 0, c.s, c.counts, c.E, c.R, c.BM, c.offsets,
                     c.tile_start, c.num_tiles, c.tiles, st);
  if (c.R > 0) hipLaunchKernelGGL(sched_rank_kernel, dim3(c.E), dim3(64), 0, c.s, idx, c.R, c.offsets, c.perm, c.inv);
  return hipGetLastError();
}

// Copy of one micro-batch's counts, offsets and perm into the weight-gradient stash.
// With a failed schedule check the stash gets zero counts and offsets, so that a later
// flush treats the micro-batch as empty instead of reading through stale rows.
__global__ __launch_bounds__(256) void stash_sched_kernel(Guard gd, const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ perm, int E, int R,
                                                          int32_t* __restrict__ st_counts,
                                                          int32_t* __restrict__ st_offsets,
                                                          int32_t* __restrict__ st_perm) {
  const bool bad = guard_fail(gd);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < E) st_counts[i] = bad ? 0 : counts[i];
  if (i <= E) st_offsets[i] = bad ? 0 : offsets[i];
  if (!bad && i < R) st_perm[i] = perm[i];
}

hipError_t launch_stash_sched(const Ctx& c, int32_t* counts, int32_t* offsets, int32_t* perm) {
  const int64_t n = std::max<int64_t>(c.R, (int64_t)c.E + 1);
  hipLaunchKernelGGL(stash_sched_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, c.s, c.guard, c.counts,
                     c.offsets, c.perm, c.E, c.R, counts, offsets, perm);
  return hipGetLastError();
}

}  // namespace mok
