// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once
#include "common.h"

namespace mok {

// Everything a launch needs to know about the problem and the schedule.
struct Ctx {
  int64_t T;
  int H, E, k, I;
  int R;           // T*k routed rows
  int act;         // MOK_F32 / MOK_BF16
  bool wgrad_f32;  // weight gradients written as fp32
  int BM;          // schedule tile rows
  int max_tiles;
  int num_cu;
  int grid;        // persistent GEMM grid
  int gemm;        // expert-GEMM dtype (mok_dtype)
  bool mx4;        // MX GEMMs with E2M1 elements (MOK_MXFP4)
  hipStream_t s;
  Guard guard;     // schedule header check (every kernel of forward/backward)
  // schedule table (device)
  int32_t* counts;
  int32_t* offsets;
  int32_t* tile_start;
  int32_t* num_tiles;
  int32_t* perm;
  int32_t* inv;
  int4* tiles;
  int32_t* hist;   // schedule build scratch: per-(expert, slot block) counts, then bases
};

hipError_t launch_route(const Ctx& c, const void* x, const void* wr, const float* bias, int32_t* idx, float* gate,
                        float* logits);
// builds the table and stamps the header (hash c.guard.expect, status MOK_OK)
hipError_t launch_schedule(const Ctx& c, const int32_t* idx);
// stash copy of a micro-batch's counts, offsets (E+1) and perm (R); zero counts and
// offsets (nothing else) when the schedule check fails
hipError_t launch_stash_sched(const Ctx& c, int32_t* counts, int32_t* offsets, int32_t* perm);

hipError_t launch_fc1(const Ctx& c, const void* x, const void* w1, void* au, void* h);
hipError_t launch_fc2(const Ctx& c, const void* h, const void* w2, void* part);
hipError_t launch_combine(const Ctx& c, const void* part, const float* gate, void* y);

hipError_t launch_dh(const Ctx& c, const void* dy, const void* w2, const void* au, const void* h, const float* gate,
                     void* dgu, float* dgp);
hipError_t launch_router_bwd(const Ctx& c, const float* dgp, const float* gate, float* dgate, float* dz);
hipError_t launch_dx(const Ctx& c, const void* dgu, const void* w1, void* part);
hipError_t launch_dx_reduce(const Ctx& c, const void* part, const float* dz, const int32_t* idx, const void* wr,
                            void* dx);
hipError_t launch_dw2(const Ctx& c, const void* dy, const float* gate, const void* h, void* dw2);
hipError_t launch_dw1(const Ctx& c, const void* dgu, const void* x, void* dw1);
// xs (bf16 only; nullptr: not written): the routed-order copy of the x rows for dW1
hipError_t launch_dwr(const Ctx& c, const float* dz, const void* x, void* dwr, void* xs);

// bf16 grouped GEMMs on the direct-to-LDS core
hipError_t launch_fc1_bf16(const Ctx& c, const void* x, const void* w1, void* au, void* h);
hipError_t launch_fc2_bf16(const Ctx& c, const void* h, const void* w2, void* part);
hipError_t launch_dh_bf16(const Ctx& c, const void* dy, const void* w2, const void* au, const void* h,
                          const float* gate, void* dgu, float* dgp);
hipError_t launch_dx_bf16(const Ctx& c, const void* dgu, const void* w1, void* part);
hipError_t launch_dw2_bf16(const Ctx& c, const void* dos, const void* h, void* dw2);
hipError_t launch_dw1_bf16(const Ctx& c, const void* dgu, const void* xs, void* dw1);
// dst[r] = src[perm[r] / k] (times gate[perm[r]] when gate != nullptr), bf16 rows of H
hipError_t launch_gather_rows(const Ctx& c, const void* src, const float* gate, void* dst);

// MXFP8: quantisers (E4M3 elements + E8M0 scale bytes per 32 along K)
// rows x F bf16 -> q [rows][F] and scales of the 32-blocks along each row: s [rows][F/32]
// when kmaj_rows = 0, else per matrix of kmaj_rows rows K-tile-major [F/128][kmaj_rows][4]
hipError_t launch_mx_quant_rows(const Ctx& c, const void* src, int64_t rows, int F, void* q, void* s,
                                int64_t kmaj_rows = 0);
// transposed, blocks along rows: q [mats][F][out_ld], s K-tile-major [mats][out_ld/128][F][4]; logical
// row r of matrix z reads physical row rowmap[r] (or r) of src + z*src_mat (ld elements
// per row); K logical rows (multiple of 128), row blocks at or past *kdev skipped
hipError_t launch_mx_quant_cols(const Ctx& c, const void* src, int64_t src_mat, int64_t ld, const int32_t* rowmap,
                                const int32_t* kdev, int K, int F, int mats, int64_t out_ld, void* q, void* s);
// per-expert rows over M stashed micro-batches, 128-padded segment offsets, row map
hipError_t launch_mx_flush_table(const Ctx& c, const int32_t* counts, const int32_t* offsets, int M, int32_t* gcnt,
                                 int32_t* pofs, int64_t kmax, int32_t* rowmap);
hipError_t launch_dwr_stash(const Ctx& c, const float* dz, const int32_t* perm, const void* xs, const int32_t* gcnt,
                            const int32_t* pofs, const int32_t* rowmap, float* part, void* dwr);
size_t dwr_stash_part_bytes(int E, int H);  // fp32 chunk partials of launch_dwr_stash
// MXFP8 grouped GEMMs
hipError_t launch_fc1_mx(const Ctx& c, const void* xq, const void* xs, const void* w1q, const void* w1s, void* au,
                         void* h, void* hq, void* hs);
hipError_t launch_fc2_mx(const Ctx& c, const void* hq, const void* hs, const void* w2q, const void* w2s, void* part);
hipError_t launch_dh_mx(const Ctx& c, const void* dyq, const void* dys, const void* w2tq, const void* w2ts,
                        const void* au, const void* h, const float* gate, void* dgu, void* dguq, void* dgus,
                        float* dgp);
hipError_t launch_dx_mx(const Ctx& c, const void* dguq, const void* dgus, const void* w1tq, const void* w1ts,
                        void* part);
hipError_t launch_dw_mx(const Ctx& c, const int32_t* pofs, const void* aq, const void* as, const void* bq,
                        const void* bs, void* out, int M, int N, int64_t kld);

// Slots per histogram / scatter block of the schedule build (1024 up to 65536 routed rows
// so that a few thousand rows still spread over several workgroups, 4096 above); shared
// by the schedule's scratch sizing and its launches.
inline int sched_block(int64_t R) { return R <= 65536 ? 1024 : 4096; }

// Fused forward (fc1 -> fc2 -> combine) and backward (dh + row gathers -> router backward ->
// dx + weight gradients + dWr -> dx reduction): one cooperative persistent launch each,
// stages separated by a grid barrier. bf16, 32-row schedule tiles.
hipError_t launch_forward_fused(const Ctx& c, const void* x, const void* w1, const void* w2, void* au, void* h,
                                void* part, const float* gate, void* y);
hipError_t launch_backward_fused(const Ctx& c, const void* x, const int32_t* idx, const float* gate, const void* w1,
                                 const void* w2, const void* wr, const void* au, const void* h, const void* dy,
                                 void* dgu, void* bpart, float* dgp, float* dz, void* xs, void* dos, void* dx,
                                 void* dw1, void* dw2, float* dgate, void* dwr);

// Tile widths (N) of the row GEMMs; shared by workspace sizing and launches.
inline int bn_fc1(int I) { return I % 128 == 0 ? 256 : 128; }
inline int bn_rows(int N) { return N % 256 == 0 ? 256 : 128; }
// bf16 dh/dx GEMMs: 512-wide tiles (8 waves side by side) for 128-row tiles when N allows
inline int bn_rows_bf16(int N, int BM) { return (BM == 128 && N % 512 == 0) ? 512 : bn_rows(N); }
// d-gate partials per routed row: one per 32-column block of I (summed in ascending
// block order by router_bwd, so the bits do not depend on the GEMM's tiling)
__host__ __device__ inline int dgate_parts(int I) { return I / 32; }
// The fused backward keeps one token's d-gate partials (k * I/32 floats) in LDS.
constexpr int kFusedMaxSlotParts = 2048;

}  // namespace mok
