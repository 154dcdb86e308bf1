// The single schedule table (dothoosh.com MoK page, "Technical details of the
// MoK mechanism": one schedule drives dispatch, combine, reverse-combine and
// reverse-dispatch).
//
// A stable counting sort of the R = T*k flat slots by expert, with work O(R + E)
// and no atomics on global memory, so it is exact and independent of scheduling:
//   1. hist:    block b (sched_block(R) consecutive slots) counts its slots per expert
//               (integer LDS counters) -> hist[e][b];
//   2. scan:    one workgroup sums each expert's block counts (counts), forms the
//               exclusive offsets and per-expert tile starts, writes the tile list
//               (expert, first row, rows) and turns hist[e][b] into the first row of
//               expert e's slots from block b (offsets[e] + earlier blocks' counts);
//   3. scatter: block b again; each of 16 waves takes 1/16 of its slots, its
//               per-expert bases come from hist and the earlier waves' counts, and
//               inside a group of 64 slots a lane's rank among equal experts is the
//               number of lower lanes holding the same expert. Row of slot s =
//               base + rank, so rows follow ascending slot order within each expert:
//               perm (row -> slot) and inv.
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
  sync_zero(st.hdr);
}

constexpr int kSchedWaves = 16;  // waves of the scatter block

__global__ __launch_bounds__(1024) void sched_hist_kernel(const int32_t* __restrict__ idx, int R, int E, int nb,
                                                          int blk, int32_t* __restrict__ hist) {
  __shared__ int s_h[1024];
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_h[e] = 0;
  __syncthreads();
  const int s0 = b * blk, s1 = min(R, s0 + blk);
  for (int s = s0 + (int)threadIdx.x; s < s1; s += blockDim.x) atomicAdd(&s_h[idx[s]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(int64_t)e * nb + b] = s_h[e];
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

__global__ __launch_bounds__(1024) void sched_scan_kernel(int32_t* __restrict__ hist, int nb, int E, int R, int BM,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tile_start,
                                                          int32_t* __restrict__ num_tiles, int4* __restrict__ tiles,
                                                          Stamp st) {
  __shared__ int s_wave[17];
  const int e = threadIdx.x;
  int c = 0;
  if (e < E)
    for (int b = 0; b < nb; ++b) c += hist[(int64_t)e * nb + b];
  const int nt = (c + BM - 1) / BM;
  int tot_c, tot_t;
  const int off = block_exclusive_scan(c, s_wave, &tot_c);
  const int ts = block_exclusive_scan(nt, s_wave, &tot_t);
  if (e < E) {
    counts[e] = c;
    offsets[e] = off;
    tile_start[e] = ts;
    for (int m = 0; m < nt; ++m) tiles[ts + m] = make_int4(e, off + m * BM, min(BM, c - m * BM), 0);
    int run = off;  // first row of e's slots from each block, blocks ascending
    for (int b = 0; b < nb; ++b) {
      const int64_t i = (int64_t)e * nb + b;
      const int h = hist[i];
      hist[i] = run;
      run += h;
    }
  }
  if (e == 0) {
    offsets[E] = R;
    tile_start[E] = tot_t;
    *num_tiles = tot_t;
    stamp_header(st);
  }
}

__global__ __launch_bounds__(1024) void sched_scatter_kernel(const int32_t* __restrict__ idx, int R, int E, int nb,
                                                             int blk, const int32_t* __restrict__ base,
                                                             int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int PER_WAVE = blk / kSchedWaves;  // a multiple of 64
  __shared__ int s_w[kSchedWaves][1024];  // per-wave counts, then per-wave next row per expert
  const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kSchedWaves * E; i += blockDim.x) s_w[i / E][i % E] = 0;
  __syncthreads();
  const int w0 = b * blk + wave * PER_WAVE;
  for (int s = w0 + lane; s < min(R, w0 + PER_WAVE); s += 64) atomicAdd(&s_w[wave][idx[s]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = base[(int64_t)e * nb + b];
    for (int w = 0; w < kSchedWaves; ++w) {
      const int t = s_w[w][e];
      s_w[w][e] = run;
      run += t;
    }
  }
  __syncthreads();
  for (int g = 0; g < PER_WAVE; g += 64) {
    const int s = w0 + g + lane;
    const int v = s < R ? idx[s] : -1;
    int rank = 0, cnt = 0;
    for (int j = 0; j < 64; ++j) {
      const int vj = __builtin_amdgcn_readlane(v, j);
      const int eq = vj == v;
      cnt += eq;
      rank += eq & (j < lane);
    }
    if (v >= 0) {
      const int row = s_w[wave][v] + rank;
      perm[row] = s;
      inv[s] = row;
    }
    // the last lane of each expert in this group moves that expert's next row on
    if (v >= 0 && rank == cnt - 1) s_w[wave][v] += cnt;
  }
}

// Tiny batches (R * E <= 2^14): count, scan and rank in one workgroup of 16 waves, with
// idx staged in LDS; wave w counts and then ranks experts w, w + 16, ... by a ballot scan
// in ascending slot order, so every output equals the three-kernel path's; two launches
// fewer (64 tokens x 8 experts: 11-14 -> 6 us).
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
  const int blk = sched_block(c.R);
  const int nb = (c.R + blk - 1) / blk;
  hipLaunchKernelGGL(sched_hist_kernel, dim3(nb), dim3(1024), 0, c.s, idx, c.R, c.E, nb, blk, c.hist);
  hipLaunchKernelGGL(sched_scan_kernel, dim3(1), dim3(1024), 0, c.s, c.hist, nb, c.E, c.R, c.BM, c.counts, c.offsets,
                     c.tile_start, c.num_tiles, c.tiles, st);
  hipLaunchKernelGGL(sched_scatter_kernel, dim3(nb), dim3(1024), 0, c.s, idx, c.R, c.E, nb, blk, c.hist, c.perm,
                     c.inv);
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
