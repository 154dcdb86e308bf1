/*
 * mok.h -- C ABI of libmok.so: one GPU's share of a deterministic
 * Mixture-of-Experts layer step (forward and backward) on AMD MI355X (gfx950).
 *
 * The layer follows the Mixture-of-Kittens pages:
 *  - "Cursor Mixture-of-Kittens cuts MoE training latency by 5.8x"
 *    (dothoosh.com), section "Technical details of the MoK mechanism":
 *    pull dispatch and push combine in the forward pass, pull reverse-combine
 *    and push reverse-dispatch in the backward pass, all four driven by one
 *    schedule table; BF16 and MXFP8; router-weight gradients fused into the
 *    SwiGLU backward; grouped expert GEMMs sized for at least two full waves of
 *    the machine; no token dropping.
 *  - kwkr.cn MoK explainer, section 4.1 (top-k gating) and section 2
 *    (determinism: the same inputs give the same bits).
 *  - aikraft.ru MoK article, section 04 (pull dispatch; the CPU kept off the
 *    critical path).
 *
 * On one GPU "dispatch" is a gather of token rows through the schedule's
 * permutation straight into the GEMM's LDS tiles, and "combine" writes one
 * partial row per (token, slot) that a second pass reduces in slot order.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - T tokens, hidden size H, E experts, top-k routing (k slots per token),
 *    expert intermediate size I.  R = T*k routed rows.  Flat slot s = t*k + j.
 *  - All arrays are row-major, device memory, 16-byte aligned, owned by the
 *    caller.  A pointer to an array of zero elements (T = 0) may be NULL.
 *    The library never allocates, frees or synchronises; every call only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = default stream) and
 *    returns.  Nothing is read back to the host.
 *  - Activation dtype `act` (MOK_F32 or MOK_BF16) is the storage type of
 *    x, y, dy, dx, the router weight wr, the expert weights and every saved or
 *    intermediate activation.  All arithmetic accumulates in fp32.
 *  - Expert-GEMM dtype `gemm`: equal to `act`, or MOK_MXFP8 (with act = MOK_BF16):
 *    every operand of the six expert GEMMs is then quantised to MXFP8 along that
 *    GEMM's K (OCP Microscaling v1.0: FP8 E4M3 elements, round to nearest even,
 *    saturating at +-448; one E8M0 scale 2^s per 32 elements, s = floor(log2 of
 *    the block's largest magnitude) - 8 clamped to [-127, 127], stored as the byte
 *    s + 127; an all-zero block has s = -127).  Quantised:
 *      fc1  x rows and W1 rows along H;     fc2  h rows and W2 rows along I;
 *      dh   dY rows and W2^T rows along H;  dx   dGU rows and W1^T rows along 2I;
 *      dW2  dO = g*dY and h along routed rows;  dW1  dGU and x along routed rows,
 *    the routed rows of one expert in blocks of 32 from its first row of the
 *    whole step (all micro-batches, in token order), the last block zero-padded.
 *    Quantiser inputs are the stored bf16 values; outputs are stored as with bf16.
 *    MOK_MXFP4 (with act = MOK_BF16; the narrower expert GEMMs of aikraft.ru MoK
 *    article, section 03): the same quantisation points and scales with FP4 E2M1
 *    elements (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives; round to
 *    nearest even, saturating at +-6; s = floor(log2 amax) - 2), two elements per
 *    byte with the even element in the low nibble (sign bit 3, exponent bits 2..1,
 *    mantissa bit 0).  Needs H and I multiples of 256.
 *  - Layouts: x, y, dy, dx [T][H]; wr [E][H]; w1 [E][2I][H] (rows 0..I-1 are
 *    the SwiGLU gate projection, rows I..2I-1 the up projection); w2 [E][H][I];
 *    idx [T][k] int32; gate, dgate, logits [T][k] / [T][E] fp32.
 *  - Errors: arguments (pointers, alignment, descriptor, buffer sizes) are
 *    checked before anything is enqueued and a status is returned; nothing is
 *    thrown across the ABI.  A failed launch returns MOK_ERR_HIP.  Faults inside
 *    kernels surface at the caller's next synchronisation of `stream`.
 *  - Schedule check: mok_schedule_build stamps a header at the start of the
 *    schedule buffer with a hash of the descriptor it was built for (T, H, E, k,
 *    I, act, gemm, the resolved tile height and tile capacity).  Every kernel of
 *    mok_moe_forward / mok_moe_backward compares that hash with the hash of its
 *    own descriptor first; on a mismatch it writes nothing but the header's
 *    status word (MOK_ERR_SCHEDULE_MISMATCH) and exits, so a schedule built for
 *    another problem is never used to index memory.  The caller reads the status
 *    word (mok_schedule_layout.status) after synchronising the stream.
 *  - Determinism: no floating-point atomics are used; every reduction runs in
 *    a fixed order, so repeated calls with the same inputs and descriptor give
 *    bit-identical outputs.
 */
#ifndef MOK_H
#define MOK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mok_status {
  MOK_OK = 0,
  MOK_ERR_NULL = 1,  /* a required pointer is NULL */
  MOK_ERR_ALIGN = 2, /* a pointer is not 16-byte aligned */
  MOK_ERR_SHAPE = 3, /* a size in the descriptor is out of range (see mok_desc) */
  MOK_ERR_DTYPE = 4, /* unsupported dtype combination */
  MOK_ERR_HIP = 5,   /* a HIP call (device query or kernel launch) failed */
  MOK_ERR_WORKSPACE = 6,         /* a caller buffer is smaller than mok_workspace_query asks */
  MOK_ERR_SCHEDULE_MISMATCH = 7  /* the schedule was built for another descriptor (reported
                                    in the schedule header's status word, see above) */
} mok_status;

typedef enum mok_dtype { MOK_F32 = 0, MOK_BF16 = 1, MOK_MXFP8 = 2, MOK_MXFP4 = 3 } mok_dtype;

/* flags */
#define MOK_FLAG_WGRAD_F32 1u   /* dw1, dw2, dwr are written as fp32 instead of `act` */
#define MOK_FLAG_WGRAD_DEFER 2u /* MXFP8 backward: stash this micro-batch's weight-gradient
                                   operands only; dw1, dw2, dwr are not touched (see
                                   mok_moe_backward) */
#define MOK_FLAG_REPLAY 4u      /* forward-activation replay: the forward keeps nothing for the
                                   backward (mok_sizes.saved = 0, `saved` may be NULL; a, u, h
                                   are formed in the forward workspace) and the backward forms
                                   a, u, h again with the forward's own kernels from x (one
                                   more FC1 GEMM, MXFP8: also the x quantiser) before the
                                   dH GEMM; every output is bit-identical to the stored path.
                                   Forward and backward of one step must agree on the flag. */
#define MOK_FLAG_FUSED 8u       /* one persistent launch per pass (the pages' single megakernel,
                                   aikraft.ru MoK article, section 01): mok_moe_forward runs
                                   FC1 -> FC2 -> combine, mok_moe_backward runs dH and the row
                                   gathers -> router backward -> dX, the weight gradients and
                                   dWr -> the dX reduction, as stages of one kernel with one
                                   workgroup per compute unit, separated by grid barriers
                                   whose words live in the schedule buffer. Same arithmetic
                                   and bits as the separate kernels. Requires act = gemm =
                                   MOK_BF16, a 32-row schedule tile (tile_m = 0 picks it with
                                   this flag, or tile_m = 32),
                                   k * I / 32 <= 2048 and no MOK_FLAG_WGRAD_F32: else
                                   MOK_ERR_SHAPE or MOK_ERR_DTYPE. The workgroups must be
                                   resident together: no other kernel may hold compute units
                                   during the launch. A barrier that does not complete within
                                   its bounded wait leaves MOK_ERR_HIP in the schedule
                                   header's status word; rebuild the schedule after that. */

/*
 * Problem descriptor.  Limits: T >= 0; 1 <= k <= min(E, 16); 1 <= E <= 1024;
 * H and I positive multiples of 128; T*k, T*H, T*k*2I and 2I*H below 2^31.
 * act is MOK_F32 or MOK_BF16; gemm equals act, or is MOK_MXFP8 or MOK_MXFP4 with
 * act = MOK_BF16 (anything else: MOK_ERR_DTYPE); MOK_MXFP4 needs H and I multiples
 * of 256 (else MOK_ERR_SHAPE).
 * tile_m: rows per schedule tile (32, 64 or 128); 0 picks the largest tile
 *   that still gives every grouped GEMM at least two full waves of the
 *   GPU's compute units (judged on the FC1 GEMM, as if every row went to one
 *   expert); 32 with MOK_FLAG_FUSED.
 * grid: workgroups of the persistent GEMM kernels; 0 = one wave of the GPU.
 * Micro-batch streaming (MX only; bf16/fp32 need mb_count <= 1): one step is
 *   mb_count micro-batches of T tokens each, forward in any order and backward in
 *   any order, every call naming its micro-batch in mb_index (0 <= mb_index <
 *   mb_count).  ring: number of slots of the forward and backward workspaces
 *   (the fixed ring that the pages' rotating token buffer becomes on one GPU);
 *   micro-batch m uses slot m % ring, so calls for micro-batches in the same slot
 *   must not overlap in time (one stream orders them).  mb_count = 0 and ring = 0
 *   mean 1.  Extra limit for MX: (mb_count*T*k + 256*E) * max(H, 2I) < 2^31
 *   (128*E for MXFP8).
 * The same descriptor must be passed to mok_schedule_build and to the
 * forward/backward calls that use that schedule (mb_index may differ).
 */
typedef struct mok_desc {
  int64_t T;
  int32_t H, E, k, I;
  int32_t act;  /* mok_dtype */
  int32_t gemm; /* mok_dtype */
  uint32_t flags;
  int32_t tile_m;
  int32_t grid;
  int32_t mb_index;
  int32_t mb_count;
  int32_t ring;
  int32_t reserved; /* must be 0 */
} mok_desc;

/* MX expert weights, quantised once per weight update by mok_weights_quantize.
 * Each orientation is K-contiguous for the GEMM that reads it; *q are E4M3 bytes
 * (MXFP8) or E2M1 codes two per byte (MXFP4: the *q shapes below with K halved),
 * *s the E8M0 scale bytes of consecutive 32-element blocks along K, stored
 * K-tile-major: for every 128-element K-tile, the 4 scale bytes of each row, rows
 * consecutive, so a GEMM tile's scales for one K-tile are one contiguous run.
 *   w1q  [E][2I][H],  w1s  [E][H/128][2I][4]    fc1 (K = H)
 *   w2q  [E][H][I],   w2s  [E][I/128][H][4]     fc2 (K = I)
 *   w2tq [E][I][H],   w2ts [E][H/128][I][4]     dh  (W2 transposed, K = H)
 *   w1tq [E][H][2I],  w1ts [E][2I/128][H][4]    dx  (W1 transposed, K = 2I)
 * (row r's scale of K-block b is byte [b/4][r][b%4] of its expert's array). */
typedef struct mok_mx_weights {
  void *w1q, *w1s, *w2q, *w2s, *w2tq, *w2ts, *w1tq, *w1ts;
} mok_mx_weights;

/* Expert weights (device pointers).  w1, w2 in `act`; mx (read only by the
 * forward and backward calls) is required when gemm is MX, else ignored. */
typedef struct mok_weights {
  const void* w1;            /* [E][2I][H] */
  const void* w2;            /* [E][H][I]  */
  const mok_mx_weights* mx;  /* host pointer to the MX orientations, or NULL */
} mok_weights;

/* Sizes in bytes of the caller-owned buffers (worst case over routings). */
typedef struct mok_sizes {
  size_t sched;  /* schedule table (mok_schedule_build)                        */
  size_t saved;  /* forward activations kept for the backward pass (per micro-batch) */
  size_t fwd_ws; /* forward scratch: per-(token,slot) partial rows [R][H]; MXFP8:
                    `ring` slots of partial rows and quantised x and h rows */
  size_t bwd_ws; /* backward scratch: dGU [R][2I], partials [R][H], d-gate parts,
                    and for bf16 the routed-order rows of x and g*dy [R][H] each.
                    MXFP8: `ring` slots of quantised dY and dGU rows, partials and
                    d-gate parts, then the weight-gradient stash of all mb_count
                    micro-batches (routed-order x, g*dy, h, dGU rows, dz, counts)
                    and the token-axis quantised operands of the dW GEMMs. The same
                    bwd_ws must be passed to every backward call of one step. */
} mok_sizes;

/* Byte offsets of the schedule table's parts inside the schedule buffer.
 * (After the header come the grid-barrier words of MOK_FLAG_FUSED and the counters
 * of the weight-gradient tile queues, and after the tiles the build's scratch; none
 * is listed here. Those words are zero between calls; two calls that use one schedule
 * buffer must not overlap in time.)
 *   header int32[16] at offset 0: [0] 0x4D4F4B53, [1] descriptor hash, [2] tile
 *                              height, [3] tile capacity, [4] status (MOK_OK after
 *                              mok_schedule_build; MOK_ERR_SCHEDULE_MISMATCH once a
 *                              forward/backward kernel saw another descriptor's hash)
 *   counts[E] int32            rows routed to each expert
 *   offsets[E+1] int32         exclusive prefix sum of counts; offsets[E] = R
 *   tile_start[E+1] int32      first tile of each expert; tile_start[E] = number of tiles
 *   num_tiles int32            number of valid tiles (also tile_start[E])
 *   perm[R] int32              routed row r -> flat slot t*k+j
 *   inv[R] int32               flat slot -> routed row (inverse of perm)
 *   tiles[max_tiles][4] int32  (expert, first routed row, rows <= tile_m, 0)
 * Rows of one expert are contiguous and in ascending slot order (a stable
 * sort of the slots by expert); tiles list experts in ascending order. */
typedef struct mok_schedule_layout {
  size_t status; /* byte offset of the header's status word */
  size_t counts, offsets, tile_start, num_tiles, perm, inv, tiles;
  int32_t tile_m;
  int32_t max_tiles;
  uint32_t hash; /* descriptor hash stamped into the header */
  int32_t reserved;
} mok_schedule_layout;

/* Layout of the `saved` buffer: au [R][2I] (fp32 accumulators a = x.W1_gate,
 * u = x.W1_up rounded to `act`, routed-row order), then h [R][I]
 * (h = silu(a)*u rounded to `act`).  au_offset/h_offset are byte offsets. */
typedef struct mok_saved_layout {
  size_t au_offset, h_offset;
} mok_saved_layout;

/* MXFP8 workspaces (for inspection): byte offsets of the quantised GEMM operands.
 * Forward slot m % ring starts at m % ring * fwd_slot in fwd_ws: xq [T][H] with scales
 * xs [H/128][T][4], hq [R][I] with hs [I/128][R][4].  Backward slot: dyq [T][H] with dys
 * [H/128][T][4], dguq [R][2I] with dgus [2I/128][R][4].  The weight-gradient stash in
 * bwd_ws holds bf16 rows in routed order, micro-batch m at rows m*R..: st_xs [M*R][H]
 * (x), st_dos [M*R][H] (dO = g*dy), st_h [M*R][I], st_dgu [M*R][2I].  After a flush
 * bwd_ws holds pofs[E+1] int32 (first padded row of each expert's segment, pofs[E] =
 * rows used) and the token-axis operands, feature-major over kmax padded rows:
 * dot [H][kmax] (dO), ht [I][kmax], dgut [2I][kmax], xt [H][kmax], each with
 * scales [kmax/128][F][4] (F = its feature count). */
typedef struct mok_mx_layout {
  size_t fwd_slot, xq, xs, hq, hs;
  size_t bwd_slot, dyq, dys, dguq, dgus;
  size_t st_xs, st_dos, st_h, st_dgu;
  size_t pofs, dot, dots, ht, hts, dgut, dguts, xt, xts;
  int64_t kmax;
} mok_mx_layout;

/* Fill *sizes for descriptor d.  Pure host computation. */
mok_status mok_workspace_query(const mok_desc* d, mok_sizes* sizes);
mok_status mok_schedule_layout_query(const mok_desc* d, mok_schedule_layout* layout);
mok_status mok_saved_layout_query(const mok_desc* d, mok_saved_layout* layout);
/* MOK_ERR_DTYPE unless gemm is MOK_MXFP8 or MOK_MXFP4. */
mok_status mok_mx_layout_query(const mok_desc* d, mok_mx_layout* layout);

/*
 * mok_route -- top-k router gating (kwkr.cn explainer, section 4.1).
 *   z[t][e] = fp32 fused-multiply-add chain over h = 0..H-1 ascending of
 *             x[t][h]*wr[e][h], starting from +0, then + bias[e] (one fp32 add).
 *   idx[t][0..k-1]: the k largest z[t][.] -- larger first, equal values
 *             (-0 == +0) ordered by lower expert index, NaN below everything.
 *   gate[t][j] = exp(z_j - z_0) / sum_i exp(z_i - z_0)  (softmax over the k
 *             selected logits, i.e. the full softmax renormalised over them).
 * x [T][H] and wr [E][H] in `act`; bias [E] fp32 or NULL; idx [T][k] int32 and
 * gate [T][k] fp32 are written; logits [T][E] fp32 is written when non-NULL.
 */
mok_status mok_route(const mok_desc* d, const void* x, const void* wr, const float* bias, int32_t* idx,
                     float* gate, float* logits, void* stream);

/*
 * mok_schedule_build -- the single schedule table shared by dispatch, combine,
 * reverse-combine and reverse-dispatch (dothoosh.com page, "Technical details
 * of the MoK mechanism").  A stable counting sort of the R flat slots by
 * expert: counts, offsets, perm, inv, then the tile list.  Integer-exact and
 * independent of launch order.  idx [T][k] int32 with values in [0, E)
 * (values outside that range are a caller error and give an unspecified
 * schedule); sched has sched_bytes >= mok_sizes.sched bytes (else
 * MOK_ERR_WORKSPACE).  The header is stamped with the descriptor's hash and
 * status MOK_OK.  The number of tiles stays on the device: the GEMM kernels
 * read it there.
 */
mok_status mok_schedule_build(const mok_desc* d, const int32_t* idx, void* sched, size_t sched_bytes, void* stream);

/*
 * mok_moe_forward -- pull dispatch, grouped SwiGLU expert FFN, push combine.
 * For every routed row r (slot s = perm[r] = t*k+j routed to expert e):
 *   a = W1[e][0:I].x_t, u = W1[e][I:2I].x_t  (gathered straight into LDS),
 *   h = silu(a)*u, o = W2[e].h  -> partial row s (rounded to `act`),
 *   y_t = sum_{j=0..k-1} gate[t][j] * partial[t*k+j]   (fp32, slot order).
 * Writes y [T][H], saved (saved_bytes >= mok_sizes.saved, layout
 * mok_saved_layout), uses ws (ws_bytes >= mok_sizes.fwd_ws); smaller buffers give
 * MOK_ERR_WORKSPACE.  sched is the table mok_schedule_build made for the same
 * descriptor (else nothing is written but its status word, see "Schedule check").
 * MXFP8: x rows and h rows are quantised along K inside the call (h in the fc1
 * epilogue, from its bf16 value); w->mx supplies w1q/w1s and w2q/w2s.  Each
 * micro-batch needs its own `saved` buffer until its backward call.
 */
mok_status mok_moe_forward(const mok_desc* d, void* sched, const void* x, const float* gate, const mok_weights* w,
                           void* y, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);

/*
 * mok_moe_forward_noalloc -- mok_moe_forward (same kernels, same results) for callers that
 * cannot allocate device memory (code under stream capture, tight serving loops): the
 * forward workspace is a library-owned device array of MOK_NOALLOC_WS_BYTES (32 MiB) per
 * GPU instead of a caller buffer, so no allocation happens in or for the call.  Returns
 * MOK_ERR_WORKSPACE when mok_sizes.fwd_ws of d exceeds it (e.g. the 2048-token bf16 layer
 * needs 8 MiB and fits; a 16384-token Kimi-K2-shaped one does not).  The array holds only
 * values a call writes before it reads them (nothing must start at zero).  Every call on
 * one GPU shares that GPU's array: calls that may overlap in time on one GPU (other
 * streams, other threads) race and must not be issued; calls ordered on one stream are
 * safe.  sched, x, gate, w, y, saved, saved_bytes and stream as for mok_moe_forward.
 */
#define MOK_NOALLOC_WS_BYTES ((size_t)32 << 20)
mok_status mok_moe_forward_noalloc(const mok_desc* d, void* sched, const void* x, const float* gate,
                                   const mok_weights* w, void* y, void* saved, size_t saved_bytes, void* stream);

/*
 * mok_moe_backward -- gradients of L = <dy, y>.
 *   pull reverse-combine: dy rows gathered through perm into the dH GEMM;
 *   dA = dy_t.W2[e]; the gate gradient g'_s = <dA, h> (= <dy_t, o_s>) is
 *   formed in that GEMM's epilogue (SonicMoE-style fusion, dothoosh.com page,
 *   "Technical details"), one partial per 32-column block of I, summed over
 *   the blocks in ascending order;
 *   dh = g*dA; da = dh*u*sig(a)*(1 + a*(1 - sig(a))); du = dh*silu(a);
 *   dGU = [da, du] (rounded to `act`); push reverse-dispatch:
 *   q_s = dGU.W1[e] (rounded to `act`), dx_t = sum_j q_tj + sum_j dz_tj*wr[idx_tj];
 *   dW1[e] = sum_r dGU_r x_t^T; dW2[e] = sum_r (g*dy_t rounded to act) h_r^T;
 *   dz = g*(g' - sum_i g_i g'_i); dWr[e] = sum_{s routed to e} dz_s x_t.
 * wr and dwr may both be NULL: the router backward is then skipped and dx
 * holds only the expert term.  dgate [T][k] fp32 receives g'.  Every element
 * of dw1 [E][2I][H], dw2 [E][H][I], dwr [E][H] is written (zero for experts
 * without tokens).  ws has mok_sizes.bwd_ws bytes.
 * MX (gemm = MOK_MXFP8 or MOK_MXFP4): dY rows are quantised along H and dGU rows along 2I
 * inside the call (dGU in the dh epilogue); w->mx supplies w2tq/w2ts and
 * w1tq/w1ts.  The weight gradients are deferred: every call copies micro-batch
 * mb_index's routed-order x, dO = g*dy (rounded to bf16), h and dGU rows, its dz
 * and its expert counts into the stash inside ws.  A call without
 * MOK_FLAG_WGRAD_DEFER then computes dW1, dW2 (and dWr when dwr != NULL) over the
 * stashed rows of all mb_count micro-batches -- each expert's rows in micro-batch
 * order, which is token order -- so the result equals that of one call over the
 * whole step; every micro-batch must have been stashed by a call since the
 * previous such call.  With MOK_FLAG_WGRAD_DEFER, dw1/dw2/dwr may be NULL.
 * saved_bytes >= mok_sizes.saved and ws_bytes >= mok_sizes.bwd_ws, else
 * MOK_ERR_WORKSPACE; the schedule check is as for mok_moe_forward.
 */
mok_status mok_moe_backward(const mok_desc* d, void* sched, const void* x, const int32_t* idx, const float* gate,
                            const mok_weights* w, const void* wr, const void* saved, size_t saved_bytes,
                            const void* dy, void* dx, void* dw1, void* dw2, float* dgate, void* dwr, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * Measurement aid.  The caller owns a mok_trace and binds it to the calling
 * thread with mok_trace_bind; the library keeps only that thread-local pointer
 * (no state shared between threads).  While bound, every launch made by this
 * thread's calls of the kernel group `filter` -- one of "route", "schedule",
 * "fc1", "fc2", "combine", "dh", "router_bwd", "dx", "dx_reduce", "gather",
 * "dw2", "dw1", "dwr", and for MXFP8 "quant" (row quantisers and stash
 * copies), "flush" (block table and token-axis quantisers), or "*" for all --
 * is bracketed by hipEventRecord(events[2n]) before and
 * hipEventRecord(events[2n+1]) after it on the launch stream, for
 * n = count, count + 1, ... < capacity (later launches are not bracketed);
 * names[n] receives the group's static name and count is advanced.
 * `events` are caller-created hipEvent_t handles.  The trace never
 * synchronises; elapsed times are read by the caller.
 */
#define MOK_TRACE_MAX 4096
typedef struct mok_trace {
  const char* filter;               /* kernel group or "*" (caller-owned string)  */
  void* const* events;              /* 2 * capacity hipEvent_t handles             */
  int32_t capacity;                 /* 0 .. MOK_TRACE_MAX                          */
  int32_t count;                    /* launches bracketed so far (library-written) */
  const char* names[MOK_TRACE_MAX]; /* group of each bracketed launch              */
} mok_trace;
/* Bind t to the calling thread (NULL unbinds).  MOK_ERR_SHAPE if capacity is out of
 * range, MOK_ERR_NULL if filter or events is NULL. */
mok_status mok_trace_bind(mok_trace* t);
/*
 * mok_weights_quantize -- the MX orientations of bf16 expert weights w1
 * [E][2I][H] and w2 [E][H][I] (see mok_mx_weights for shapes): w1q/w2q quantise
 * rows along their contiguous axis; w2tq[e][i][h] and w1tq[e][h][c] are W2[e][h][i]
 * and W1[e][c][h] quantised in blocks of 32 along h and c respectively and stored
 * transposed.  Requires act = MOK_BF16 and gemm = MOK_MXFP8 or MOK_MXFP4; every pointer in
 * *out non-NULL and 16-byte aligned.  Run once per weight update, outside the
 * layer step.
 */
mok_status mok_weights_quantize(const mok_desc* d, const void* w1, const void* w2, const mok_mx_weights* out,
                                void* stream);

/* Static string naming a status code. */
const char* mok_status_string(mok_status s);

/* Library ABI version (major*100 + minor). */
int32_t mok_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOK_H */
