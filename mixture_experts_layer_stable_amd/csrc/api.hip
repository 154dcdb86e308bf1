// C-ABI entry points of libmok: argument checks, buffer layouts, launches.
#include <cstring>
#include <mutex>

#include "kernels.h"

using namespace mok;

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_size(int act) { return act == MOK_F32 ? 4 : 2; }

int mb_count_of(const mok_desc* d) { return d->mb_count > 0 ? d->mb_count : 1; }
int ring_of(const mok_desc* d) { return d->ring > 0 ? d->ring : 1; }
bool is_mx(const mok_desc* d) { return d->gemm == MOK_MXFP8 || d->gemm == MOK_MXFP4; }
// Quantised element bytes of n MX elements (E4M3: 1 each; E2M1: two per byte).
size_t mxb(const mok_desc* d, int64_t n) { return (size_t)(d->gemm == MOK_MXFP4 ? n / 2 : n); }
bool is_replay(const mok_desc* d) { return (d->flags & MOK_FLAG_REPLAY) != 0; }
bool is_fused(const mok_desc* d) { return (d->flags & MOK_FLAG_FUSED) != 0; }

// The fused persistent kernels run the bf16 path on 32-row tiles only.
mok_status check_fused(const mok_desc* d, const Ctx& c) {
  if (!is_fused(d)) return MOK_OK;
  if (d->act != MOK_BF16 || d->gemm != MOK_BF16 || (d->flags & MOK_FLAG_WGRAD_F32)) return MOK_ERR_DTYPE;
  if (c.BM != 32 || (int64_t)d->k * dgate_parts(d->I) > kFusedMaxSlotParts) return MOK_ERR_SHAPE;
  return MOK_OK;
}

// Rows of the token-axis operands of the MX weight-gradient GEMMs: every expert's rows
// of the step padded to a whole K-tile (128 elements for MXFP8, 256 for MXFP4).
int64_t mx_kmax(const mok_desc* d) {
  const int64_t kt = d->gemm == MOK_MXFP4 ? 256 : 128;
  return ((int64_t)mb_count_of(d) * d->T * d->k + kt * d->E + kt - 1) / kt * kt;
}

mok_status check_desc(const mok_desc* d) {
  if (d == nullptr) return MOK_ERR_NULL;
  if (d->act != MOK_F32 && d->act != MOK_BF16) return MOK_ERR_DTYPE;
  if (d->gemm != d->act && !(is_mx(d) && d->act == MOK_BF16)) return MOK_ERR_DTYPE;
  if ((d->flags & MOK_FLAG_WGRAD_DEFER) && !is_mx(d)) return MOK_ERR_DTYPE;
  if (d->reserved != 0 || d->mb_count < 0 || d->ring < 0 || d->mb_count > 1024 || d->ring > 1024)
    return MOK_ERR_SHAPE;
  if (d->mb_index < 0 || d->mb_index >= mb_count_of(d)) return MOK_ERR_SHAPE;
  if (!is_mx(d) && mb_count_of(d) > 1) return MOK_ERR_SHAPE;
  if (d->T < 0 || d->E < 1 || d->E > 1024 || d->k < 1 || d->k > 16 || d->k > d->E) return MOK_ERR_SHAPE;
  if (d->H <= 0 || d->I <= 0 || d->H % 128 != 0 || d->I % 128 != 0) return MOK_ERR_SHAPE;
  // MXFP4 K-tiles are 256 elements along H, I and 2I
  if (d->gemm == MOK_MXFP4 && (d->H % 256 != 0 || d->I % 256 != 0)) return MOK_ERR_SHAPE;
  if (d->T * (int64_t)d->k >= ((int64_t)1 << 31)) return MOK_ERR_SHAPE;
  // 32-bit byte offsets inside one operand: token rows, routed rows, one expert's weights
  if (d->T * (int64_t)d->H >= ((int64_t)1 << 31)) return MOK_ERR_SHAPE;
  if (d->T * (int64_t)d->k * 2 * d->I >= ((int64_t)1 << 31)) return MOK_ERR_SHAPE;
  if ((int64_t)d->I * 2 * d->H >= ((int64_t)1 << 31)) return MOK_ERR_SHAPE;
  if (d->tile_m != 0 && d->tile_m != 32 && d->tile_m != 64 && d->tile_m != 128) return MOK_ERR_SHAPE;
  if (d->grid < 0) return MOK_ERR_SHAPE;
  // 32-bit offsets inside the token-axis operands of the MXFP8 weight gradients
  if (is_mx(d) && mx_kmax(d) * std::max<int64_t>(d->H, 2LL * d->I) >= ((int64_t)1 << 31)) return MOK_ERR_SHAPE;
  return MOK_OK;
}

// Compute units of the current device, cached per device id.
mok_status device_cus(int* out) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOK_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 64 && cache[dev] > 0) {
    *out = cache[dev];
    return MOK_OK;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return MOK_ERR_HIP;
  if (dev < 64) cache[dev] = cus;
  *out = cus;
  return MOK_OK;
}

// Schedule tile height. The pages' overlap heuristic asks every expert-grouped
// GEMM for at least two full waves of the machine (dothoosh.com MoK page,
// "Technical details of the MoK mechanism"); we take the tallest tile for which
// even a fully concentrated routing gives (R / BM) * (2I / 256) >= 2 * CUs
// tiles in the FC1 GEMM, else the smallest tile. The fused passes are built for 32-row
// tiles and always take them.
int choose_tile_m(int64_t R, int I, int cus, bool fused) {
  if (fused) return 32;
  const int cands[3] = {128, 64, 32};
  for (int bm : cands)
    if ((R / bm) * (int64_t)(2 * I / 256) >= 2LL * cus) return bm;
  return 32;
}

struct Layout {
  int BM = 32, max_tiles = 0;
  size_t counts, offsets, tile_start, num_tiles, perm, inv, tiles, hist, sched;  // header at 0
  size_t au, h, saved;
  size_t fwd_part, fwd;
  size_t fau, fh, bau, bh;  // replay: a|u and h in the forward and the backward workspaces
  size_t dgu, bpart, dgp, dz, xs, dos, bwd;
};

// Buffer layouts. The schedule is sized for the smallest tile height, so its
// size does not depend on the device.
Layout layout_of(const mok_desc* d, int BM) {
  Layout L;
  const int64_t R = d->T * d->k;
  const size_t es = elem_size(d->act);
  L.BM = BM;
  L.max_tiles = (int)(R / BM + std::min<int64_t>(d->E, R));
  const int64_t worst_tiles = R / 32 + std::min<int64_t>(d->E, R);
  size_t o = up(kSchedHeaderBytes);  // header int32[16], then the fused kernels' barrier lines
  L.counts = o; o = up(o + 4 * (size_t)d->E);
  L.offsets = o; o = up(o + 4 * (size_t)(d->E + 1));
  L.tile_start = o; o = up(o + 4 * (size_t)(d->E + 1));
  L.num_tiles = o; o = up(o + 4);
  L.perm = o; o = up(o + 4 * (size_t)R);
  L.inv = o; o = up(o + 4 * (size_t)R);
  L.tiles = o; o = up(o + 16 * (size_t)std::max<int64_t>(worst_tiles, 1));
  L.hist = o; o = up(o + 4 * (size_t)d->E * (size_t)((R + sched_block(R) - 1) / sched_block(R)));  // build scratch
  L.sched = o;
  o = 0;
  L.au = o; o = up(o + es * (size_t)R * 2 * d->I);
  L.h = o; o = up(o + es * (size_t)R * d->I);
  const size_t act_bytes = o;  // a|u then h
  L.saved = is_replay(d) ? 0 : act_bytes;
  L.fwd_part = 0;
  L.fwd = up(es * (size_t)R * d->H);
  L.fau = L.fwd + L.au;
  L.fh = L.fwd + L.h;
  if (is_replay(d)) L.fwd += act_bytes;
  o = 0;
  L.dgu = o; o = up(o + es * (size_t)R * 2 * d->I);
  L.bpart = o; o = up(o + es * (size_t)R * d->H);
  L.dgp = o; o = up(o + 4 * (size_t)R * dgate_parts(d->I));
  L.dz = o; o = up(o + 4 * (size_t)R);
  // bf16: token rows in routed order for the weight-gradient GEMMs (x and g*dy)
  const size_t rows = d->act == MOK_BF16 ? es * (size_t)R * d->H : 0;
  L.xs = o; o = up(o + rows);
  L.dos = o; o = up(o + rows);
  L.bau = o + L.au;
  L.bh = o + L.h;
  if (is_replay(d)) o += act_bytes;
  L.bwd = o;
  return L;
}

// MX buffer layout (quantised rows hold 1 byte per element for MXFP8, half for MXFP4;
// scales 1 byte per 32 elements). Forward ring slot: quantised x rows, quantised h rows, partial
// rows. Backward ring slot: quantised dY and dGU rows, partial rows, d-gate parts.
// Then the stash of all micro-batches (array-major: micro-batch m's part of each
// array at its m-th R rows) and the flush buffers.
struct MxLayout {
  size_t xq, xs, hq, hs, part, rau, rh, fslot, fwd;
  size_t dyq, dys, dguq, dgus, bpart, dgp, bxq, bxs, bhq, bhs, bau, bh, bslot;
  size_t st_counts, st_offsets, st_perm, st_dz, st_xs, st_dos, st_h, st_dgu;
  size_t gcnt, pofs, rowmap, xt, xts, dot, dots, ht, hts, dgut, dguts, dwrp, bwd;
  int64_t kmax;
};

MxLayout mx_layout_of(const mok_desc* d) {
  MxLayout L;
  const int64_t T = d->T, R = d->T * d->k, H = d->H, I = d->I, E = d->E;
  const int64_t M = mb_count_of(d), S = ring_of(d);
  size_t o = 0;
  L.xq = o; o = up(o + mxb(d, T * H));
  L.xs = o; o = up(o + (size_t)(T * H / 32));
  L.hq = o; o = up(o + mxb(d, R * I));
  L.hs = o; o = up(o + (size_t)(R * I / 32));
  L.part = o; o = up(o + (size_t)(2 * R * H));
  // replay: a|u and h of this micro-batch live in the slot instead of `saved`
  const size_t rp = is_replay(d) ? 1 : 0;
  L.rau = o; o = up(o + rp * (size_t)(2 * R * 2 * I));
  L.rh = o; o = up(o + rp * (size_t)(2 * R * I));
  L.fslot = o;
  L.fwd = (size_t)S * L.fslot;
  o = 0;
  L.dyq = o; o = up(o + mxb(d, T * H));
  L.dys = o; o = up(o + (size_t)(T * H / 32));
  L.dguq = o; o = up(o + mxb(d, R * 2 * I));
  L.dgus = o; o = up(o + (size_t)(R * 2 * I / 32));
  L.bpart = o; o = up(o + (size_t)(2 * R * H));
  L.dgp = o; o = up(o + (size_t)(4 * R * dgate_parts(d->I)));
  // replay: the backward forms quantised x, a|u, h (and quantised h) again in its slot
  L.bxq = o; o = up(o + rp * mxb(d, T * H));
  L.bxs = o; o = up(o + rp * (size_t)(T * H / 32));
  L.bhq = o; o = up(o + rp * mxb(d, R * I));
  L.bhs = o; o = up(o + rp * (size_t)(R * I / 32));
  L.bau = o; o = up(o + rp * (size_t)(2 * R * 2 * I));
  L.bh = o; o = up(o + rp * (size_t)(2 * R * I));
  L.bslot = o;
  o = (size_t)S * L.bslot;
  L.st_counts = o; o = up(o + (size_t)(4 * M * E));
  L.st_offsets = o; o = up(o + (size_t)(4 * M * (E + 1)));
  L.st_perm = o; o = up(o + (size_t)(4 * M * R));
  L.st_dz = o; o = up(o + (size_t)(4 * M * R));
  L.st_xs = o; o = up(o + (size_t)(2 * M * R * H));
  L.st_dos = o; o = up(o + (size_t)(2 * M * R * H));
  L.st_h = o; o = up(o + (size_t)(2 * M * R * I));
  L.st_dgu = o; o = up(o + (size_t)(2 * M * R * 2 * I));
  L.kmax = mx_kmax(d);
  const int64_t K = L.kmax;
  L.gcnt = o; o = up(o + (size_t)(4 * E));
  L.pofs = o; o = up(o + (size_t)(4 * (E + 1)));
  L.rowmap = o; o = up(o + (size_t)(4 * K));
  L.xt = o; o = up(o + mxb(d, H * K));
  L.xts = o; o = up(o + (size_t)(H * K / 32));
  L.dot = o; o = up(o + mxb(d, H * K));
  L.dots = o; o = up(o + (size_t)(H * K / 32));
  L.ht = o; o = up(o + mxb(d, I * K));
  L.hts = o; o = up(o + (size_t)(I * K / 32));
  L.dgut = o; o = up(o + mxb(d, 2 * I * K));
  L.dguts = o; o = up(o + (size_t)(2 * I * K / 32));
  L.dwrp = o; o = up(o + dwr_stash_part_bytes((int)E, (int)H));
  L.bwd = o;
  return L;
}

mok_status resolve(const mok_desc* d, Layout* L, int* cus) {
  mok_status st = check_desc(d);
  if (st != MOK_OK) return st;
  st = device_cus(cus);
  if (st != MOK_OK) return st;
  const int bm = d->tile_m ? d->tile_m : choose_tile_m(d->T * d->k, d->I, *cus, is_fused(d));
  *L = layout_of(d, bm);
  return MOK_OK;
}

// FNV-1a over the 32-bit words that fix a schedule's meaning: the problem shape and
// dtypes, the resolved tile height and the tile capacity.
uint32_t desc_hash(const mok_desc* d, const Layout& L) {
  const uint32_t w[10] = {(uint32_t)d->T, (uint32_t)(d->T >> 32), (uint32_t)d->H, (uint32_t)d->E, (uint32_t)d->k,
                          (uint32_t)d->I, (uint32_t)d->act, (uint32_t)d->gemm, (uint32_t)L.BM,
                          (uint32_t)L.max_tiles};
  uint32_t h = 2166136261u;
  for (uint32_t v : w)
    for (int b = 0; b < 4; ++b) {
      h ^= (v >> (8 * b)) & 0xFFu;
      h *= 16777619u;
    }
  return h;
}

mok_status make_ctx(const mok_desc* d, const void* sched, void* stream, Ctx* c) {
  Layout L;
  int cus = 0;
  mok_status st = resolve(d, &L, &cus);
  if (st != MOK_OK) return st;
  char* sb = (char*)sched;
  c->guard = Guard{(int32_t*)sb, desc_hash(d, L)};
  c->T = d->T;
  c->H = d->H;
  c->E = d->E;
  c->k = d->k;
  c->I = d->I;
  c->R = (int)(d->T * d->k);
  c->act = d->act;
  c->wgrad_f32 = (d->flags & MOK_FLAG_WGRAD_F32) != 0;
  c->BM = L.BM;
  c->max_tiles = L.max_tiles;
  c->num_cu = cus;
  c->grid = d->grid;
  c->gemm = d->gemm;
  c->mx4 = d->gemm == MOK_MXFP4;
  c->s = (hipStream_t)stream;
  c->counts = (int32_t*)(sb + L.counts);
  c->offsets = (int32_t*)(sb + L.offsets);
  c->tile_start = (int32_t*)(sb + L.tile_start);
  c->num_tiles = (int32_t*)(sb + L.num_tiles);
  c->perm = (int32_t*)(sb + L.perm);
  c->inv = (int32_t*)(sb + L.inv);
  c->tiles = (int4*)(sb + L.tiles);
  c->hist = (int32_t*)(sb + L.hist);
  return MOK_OK;
}

#define MOK_REQUIRE(p)                   \
  do {                                   \
    if ((p) == nullptr) return MOK_ERR_NULL;  \
    if (!aligned16(p)) return MOK_ERR_ALIGN; \
  } while (0)

// ---- workspace of mok_moe_forward_noalloc: a file-scope device array ----
// In host code `scratch` only names the symbol; its device address (one per GPU, each GPU
// holds its own copy until the process ends) comes from hipGetSymbolAddress, taken once
// per device with that device current and cached here.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

mok_status scratch_ptr(void** out) {
  static std::mutex mu;
  static void* cache[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOK_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOK_ERR_HIP;
    cache[dev] = p;
  }
  *out = cache[dev];
  return MOK_OK;
}

// Buffer sizes passed by the caller against what the descriptor needs.
mok_status need(size_t have, size_t want) { return have >= want ? MOK_OK : MOK_ERR_WORKSPACE; }

// ---- measurement trace (see mok_trace_bind): the calling thread's caller-owned trace ----
thread_local mok_trace* t_trace = nullptr;

bool trace_on(const char* name) {
  const mok_trace* t = t_trace;
  return t != nullptr && t->count >= 0 && t->count < t->capacity &&
         (std::strcmp(t->filter, "*") == 0 || std::strcmp(t->filter, name) == 0);
}

// Launch `call` (a hipError_t expression) bracketed by trace events when traced.
#define MOK_LAUNCH(name, stream, call)                                                          \
  do {                                                                                          \
    const bool tr_ = trace_on(name);                                                            \
    if (tr_ && hipEventRecord((hipEvent_t)t_trace->events[2 * t_trace->count], stream) != hipSuccess) \
      return MOK_ERR_HIP;                                                                       \
    if ((call) != hipSuccess) return MOK_ERR_HIP;                                               \
    if (tr_) {                                                                                  \
      if (hipEventRecord((hipEvent_t)t_trace->events[2 * t_trace->count + 1], stream) != hipSuccess) \
        return MOK_ERR_HIP;                                                                     \
      t_trace->names[t_trace->count] = name;                                                    \
      ++t_trace->count;                                                                         \
    }                                                                                           \
  } while (0)

// MX backward of micro-batch d->mb_index (see mok_moe_backward in mok.h).
mok_status mx_backward(const mok_desc* d, const Ctx& c, const void* x, const int32_t* idx, const float* gate,
                       const mok_weights* w, const void* wr, const void* saved, const void* dy, void* dx, void* dw1,
                       void* dw2, float* dgate, void* dwr, void* ws) {
  const bool flush = (d->flags & MOK_FLAG_WGRAD_DEFER) == 0;
  if (flush) {
    MOK_REQUIRE(dw1);
    MOK_REQUIRE(dw2);
    if (dwr != nullptr && !aligned16(dwr)) return MOK_ERR_ALIGN;
  }
  if (wr != nullptr && !aligned16(wr)) return MOK_ERR_ALIGN;
  MOK_REQUIRE(ws);
  const mok_mx_weights* q = w->mx;
  const bool replay = is_replay(d);
  if (c.R > 0) {
    MOK_REQUIRE(x);
    MOK_REQUIRE(idx);
    MOK_REQUIRE(gate);
    if (!replay) MOK_REQUIRE(saved);
    MOK_REQUIRE(dy);
    MOK_REQUIRE(dx);
    MOK_REQUIRE(dgate);
    if (q == nullptr) return MOK_ERR_NULL;
    MOK_REQUIRE(q->w2tq);
    MOK_REQUIRE(q->w2ts);
    MOK_REQUIRE(q->w1tq);
    MOK_REQUIRE(q->w1ts);
    if (replay) {
      MOK_REQUIRE(q->w1q);
      MOK_REQUIRE(q->w1s);
    }
  }
  const Layout L = layout_of(d, c.BM);
  const MxLayout X = mx_layout_of(d);
  char* wb = (char*)ws;
  char* bs = wb + (size_t)(d->mb_index % ring_of(d)) * X.bslot;
  const char* au = replay ? bs + X.bau : (const char*)saved + L.au;
  const char* hr = replay ? bs + X.bh : (const char*)saved + L.h;
  const int64_t m = d->mb_index, R = c.R, H = c.H, I = c.I, E = c.E;
  float* dz = (float*)(wb + X.st_dz) + m * R;
  char* st_dgu = wb + X.st_dgu + (size_t)(m * R * 2 * I * 2);
  if (c.R > 0) {
    float* dgp = (float*)(bs + X.dgp);
    if (replay) {  // the forward's x quantiser and FC1, again
      MOK_LAUNCH("quant", c.s, launch_mx_quant_rows(c, x, c.T, c.H, bs + X.bxq, bs + X.bxs, c.T));
      MOK_LAUNCH("fc1", c.s, launch_fc1_mx(c, bs + X.bxq, bs + X.bxs, q->w1q, q->w1s, bs + X.bau, bs + X.bh,
                                           bs + X.bhq, bs + X.bhs));
    }
    MOK_LAUNCH("quant", c.s, launch_mx_quant_rows(c, dy, c.T, c.H, bs + X.dyq, bs + X.dys, c.T));
    MOK_LAUNCH("dh", c.s, launch_dh_mx(c, bs + X.dyq, bs + X.dys, q->w2tq, q->w2ts, au, hr, gate, st_dgu,
                                       bs + X.dguq, bs + X.dgus, dgp));
    MOK_LAUNCH("router_bwd", c.s, launch_router_bwd(c, dgp, gate, dgate, dz));
    MOK_LAUNCH("dx", c.s, launch_dx_mx(c, bs + X.dguq, bs + X.dgus, q->w1tq, q->w1ts, bs + X.bpart));
    MOK_LAUNCH("dx_reduce", c.s, launch_dx_reduce(c, bs + X.bpart, dz, idx, wr, dx));
    // stash: routed-order x and dO = g*dy rows, h rows, perm
    MOK_LAUNCH("quant", c.s, launch_gather_rows(c, x, nullptr, wb + X.st_xs + (size_t)(m * R * H * 2)));
    MOK_LAUNCH("quant", c.s, launch_gather_rows(c, dy, gate, wb + X.st_dos + (size_t)(m * R * H * 2)));
    MOK_LAUNCH("quant", c.s, hipMemcpyAsync(wb + X.st_h + (size_t)(m * R * I * 2), hr, (size_t)(R * I * 2),
                                            hipMemcpyDeviceToDevice, c.s));
  }
  MOK_LAUNCH("quant", c.s, launch_stash_sched(c, (int32_t*)(wb + X.st_counts) + m * E,
                                              (int32_t*)(wb + X.st_offsets) + m * (E + 1),
                                              (int32_t*)(wb + X.st_perm) + m * R));
  if (!flush) return MOK_OK;

  // weight gradients over the whole step
  const int M = mb_count_of(d);
  const int64_t K = X.kmax;
  int32_t* gcnt = (int32_t*)(wb + X.gcnt);
  int32_t* pofs = (int32_t*)(wb + X.pofs);
  int32_t* rowmap = (int32_t*)(wb + X.rowmap);
  MOK_LAUNCH("flush", c.s, launch_mx_flush_table(c, (const int32_t*)(wb + X.st_counts),
                                                 (const int32_t*)(wb + X.st_offsets), M, gcnt, pofs, K, rowmap));
  MOK_LAUNCH("flush", c.s, launch_mx_quant_cols(c, wb + X.st_dos, 0, H, rowmap, pofs + E, (int)K, (int)H, 1, K,
                                                wb + X.dot, wb + X.dots));
  MOK_LAUNCH("flush", c.s, launch_mx_quant_cols(c, wb + X.st_h, 0, I, rowmap, pofs + E, (int)K, (int)I, 1, K,
                                                wb + X.ht, wb + X.hts));
  MOK_LAUNCH("dw2", c.s, launch_dw_mx(c, pofs, wb + X.dot, wb + X.dots, wb + X.ht, wb + X.hts, dw2, (int)H, (int)I,
                                      K));
  MOK_LAUNCH("flush", c.s, launch_mx_quant_cols(c, wb + X.st_dgu, 0, 2 * I, rowmap, pofs + E, (int)K, (int)(2 * I), 1,
                                                K, wb + X.dgut, wb + X.dguts));
  MOK_LAUNCH("flush", c.s, launch_mx_quant_cols(c, wb + X.st_xs, 0, H, rowmap, pofs + E, (int)K, (int)H, 1, K,
                                                wb + X.xt, wb + X.xts));
  MOK_LAUNCH("dw1", c.s, launch_dw_mx(c, pofs, wb + X.dgut, wb + X.dguts, wb + X.xt, wb + X.xts, dw1, (int)(2 * I),
                                      (int)H, K));
  if (dwr != nullptr)
    MOK_LAUNCH("dwr", c.s, launch_dwr_stash(c, (const float*)(wb + X.st_dz), (const int32_t*)(wb + X.st_perm),
                                            wb + X.st_xs, gcnt, pofs, rowmap, (float*)(wb + X.dwrp), dwr));
  return MOK_OK;
}

}  // namespace

extern "C" {

mok_status mok_workspace_query(const mok_desc* d, mok_sizes* sizes) {
  mok_status st = check_desc(d);
  if (st != MOK_OK) return st;
  if (sizes == nullptr) return MOK_ERR_NULL;
  const Layout L = layout_of(d, 32);
  sizes->sched = L.sched;
  sizes->saved = L.saved;
  sizes->fwd_ws = L.fwd;
  sizes->bwd_ws = L.bwd;
  if (is_mx(d)) {
    const MxLayout X = mx_layout_of(d);
    sizes->fwd_ws = X.fwd;
    sizes->bwd_ws = X.bwd;
  }
  return MOK_OK;
}

mok_status mok_schedule_layout_query(const mok_desc* d, mok_schedule_layout* out) {
  if (out == nullptr) return MOK_ERR_NULL;
  Layout L;
  int cus = 0;
  mok_status st = resolve(d, &L, &cus);
  if (st != MOK_OK) return st;
  out->status = 4 * kHdrStatus;
  out->hash = desc_hash(d, L);
  out->reserved = 0;
  out->counts = L.counts;
  out->offsets = L.offsets;
  out->tile_start = L.tile_start;
  out->num_tiles = L.num_tiles;
  out->perm = L.perm;
  out->inv = L.inv;
  out->tiles = L.tiles;
  out->tile_m = L.BM;
  out->max_tiles = L.max_tiles;
  return MOK_OK;
}

mok_status mok_saved_layout_query(const mok_desc* d, mok_saved_layout* out) {
  mok_status st = check_desc(d);
  if (st != MOK_OK) return st;
  if (out == nullptr) return MOK_ERR_NULL;
  const Layout L = layout_of(d, 32);
  out->au_offset = L.au;
  out->h_offset = L.h;
  return MOK_OK;
}

mok_status mok_mx_layout_query(const mok_desc* d, mok_mx_layout* out) {
  mok_status st = check_desc(d);
  if (st != MOK_OK) return st;
  if (out == nullptr) return MOK_ERR_NULL;
  if (!is_mx(d)) return MOK_ERR_DTYPE;
  const MxLayout X = mx_layout_of(d);
  *out = mok_mx_layout{X.fslot, X.xq,     X.xs,   X.hq,   X.hs,   X.bslot, X.dyq, X.dys,
                       X.dguq,  X.dgus,   X.st_xs, X.st_dos, X.st_h, X.st_dgu, X.pofs, X.dot,
                       X.dots,  X.ht,     X.hts,  X.dgut, X.dguts, X.xt,    X.xts, X.kmax};
  return MOK_OK;
}

mok_status mok_route(const mok_desc* d, const void* x, const void* wr, const float* bias, int32_t* idx, float* gate,
                     float* logits, void* stream) {
  mok_status st = check_desc(d);
  if (st != MOK_OK) return st;
  if (d->T == 0) return MOK_OK;  // empty arrays may be NULL
  MOK_REQUIRE(x);
  MOK_REQUIRE(wr);
  MOK_REQUIRE(idx);
  MOK_REQUIRE(gate);
  if (logits != nullptr && !aligned16(logits)) return MOK_ERR_ALIGN;
  if (bias != nullptr && ((uintptr_t)bias & 3u)) return MOK_ERR_ALIGN;
  Ctx c{};
  c.T = d->T;
  c.H = d->H;
  c.E = d->E;
  c.k = d->k;
  c.I = d->I;
  c.act = d->act;
  c.s = (hipStream_t)stream;
  st = device_cus(&c.num_cu);
  if (st != MOK_OK) return st;
  MOK_LAUNCH("route", c.s, launch_route(c, x, wr, bias, idx, gate, logits));
  return MOK_OK;
}

mok_status mok_schedule_build(const mok_desc* d, const int32_t* idx, void* sched, size_t sched_bytes, void* stream) {
  MOK_REQUIRE(sched);
  mok_status st = check_desc(d);
  if (st != MOK_OK) return st;
  if ((st = need(sched_bytes, layout_of(d, 32).sched)) != MOK_OK) return st;
  Ctx c;
  st = make_ctx(d, sched, stream, &c);
  if (st != MOK_OK) return st;
  if (c.R > 0) MOK_REQUIRE(idx);
  MOK_LAUNCH("schedule", c.s, launch_schedule(c, idx));
  return MOK_OK;
}

mok_status mok_moe_forward(const mok_desc* d, void* sched, const void* x, const float* gate, const mok_weights* w,
                           void* y, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
  MOK_REQUIRE(sched);
  if (w == nullptr) return MOK_ERR_NULL;
  mok_sizes need_sz;
  mok_status st = mok_workspace_query(d, &need_sz);
  if (st != MOK_OK) return st;
  if ((st = need(saved_bytes, need_sz.saved)) != MOK_OK || (st = need(ws_bytes, need_sz.fwd_ws)) != MOK_OK) return st;
  Ctx c;
  st = make_ctx(d, sched, stream, &c);
  if (st != MOK_OK) return st;
  if (c.R == 0) return MOK_OK;
  MOK_REQUIRE(x);
  MOK_REQUIRE(gate);
  MOK_REQUIRE(y);
  if (!is_replay(d)) MOK_REQUIRE(saved);
  MOK_REQUIRE(ws);
  const Layout L = layout_of(d, c.BM);
  char* au = is_replay(d) ? (char*)ws + L.fau : (char*)saved + L.au;
  char* hr = is_replay(d) ? (char*)ws + L.fh : (char*)saved + L.h;
  if (is_mx(d)) {
    const mok_mx_weights* q = w->mx;
    if (q == nullptr) return MOK_ERR_NULL;
    MOK_REQUIRE(q->w1q);
    MOK_REQUIRE(q->w1s);
    MOK_REQUIRE(q->w2q);
    MOK_REQUIRE(q->w2s);
    const MxLayout X = mx_layout_of(d);
    char* fs = (char*)ws + (size_t)(d->mb_index % ring_of(d)) * X.fslot;
    if (is_replay(d)) {
      au = fs + X.rau;
      hr = fs + X.rh;
    }
    MOK_LAUNCH("quant", c.s, launch_mx_quant_rows(c, x, c.T, c.H, fs + X.xq, fs + X.xs, c.T));
    MOK_LAUNCH("fc1", c.s, launch_fc1_mx(c, fs + X.xq, fs + X.xs, q->w1q, q->w1s, au, hr, fs + X.hq, fs + X.hs));
    MOK_LAUNCH("fc2", c.s, launch_fc2_mx(c, fs + X.hq, fs + X.hs, q->w2q, q->w2s, fs + X.part));
    MOK_LAUNCH("combine", c.s, launch_combine(c, fs + X.part, gate, y));
    return MOK_OK;
  }
  MOK_REQUIRE(w->w1);
  MOK_REQUIRE(w->w2);
  if ((st = check_fused(d, c)) != MOK_OK) return st;
  if (is_fused(d)) {
    MOK_LAUNCH("forward_fused", c.s, launch_forward_fused(c, x, w->w1, w->w2, au, hr, ws, gate, y));
    return MOK_OK;
  }
  MOK_LAUNCH("fc1", c.s, launch_fc1(c, x, w->w1, au, hr));
  MOK_LAUNCH("fc2", c.s, launch_fc2(c, hr, w->w2, ws));
  MOK_LAUNCH("combine", c.s, launch_combine(c, ws, gate, y));
  return MOK_OK;
}

mok_status mok_moe_forward_noalloc(const mok_desc* d, void* sched, const void* x, const float* gate,
                                   const mok_weights* w, void* y, void* saved, size_t saved_bytes, void* stream) {
  mok_sizes sz;
  mok_status st = mok_workspace_query(d, &sz);
  if (st != MOK_OK) return st;
  if (sz.fwd_ws > kScratchBytes) return MOK_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws)) != MOK_OK) return st;
  return mok_moe_forward(d, sched, x, gate, w, y, saved, saved_bytes, ws, kScratchBytes, stream);
}

mok_status mok_moe_backward(const mok_desc* d, void* sched, const void* x, const int32_t* idx, const float* gate,
                            const mok_weights* w, const void* wr, const void* saved, size_t saved_bytes,
                            const void* dy, void* dx, void* dw1, void* dw2, float* dgate, void* dwr, void* ws,
                            size_t ws_bytes, void* stream) {
  MOK_REQUIRE(sched);
  if (w == nullptr) return MOK_ERR_NULL;
  mok_sizes need_sz;
  mok_status st = mok_workspace_query(d, &need_sz);
  if (st != MOK_OK) return st;
  if ((st = need(saved_bytes, need_sz.saved)) != MOK_OK || (st = need(ws_bytes, need_sz.bwd_ws)) != MOK_OK) return st;
  Ctx c;
  st = make_ctx(d, sched, stream, &c);
  if (st != MOK_OK) return st;
  if (is_mx(d)) return mx_backward(d, c, x, idx, gate, w, wr, saved, dy, dx, dw1, dw2, dgate, dwr, ws);
  MOK_REQUIRE(dw1);
  MOK_REQUIRE(dw2);
  if (dwr != nullptr && !aligned16(dwr)) return MOK_ERR_ALIGN;
  if (wr != nullptr && !aligned16(wr)) return MOK_ERR_ALIGN;
  if (c.R > 0) {
    MOK_REQUIRE(x);
    MOK_REQUIRE(idx);
    MOK_REQUIRE(gate);
    MOK_REQUIRE(w->w1);
    MOK_REQUIRE(w->w2);
    if (!is_replay(d)) MOK_REQUIRE(saved);
    MOK_REQUIRE(dy);
    MOK_REQUIRE(dx);
    MOK_REQUIRE(dgate);
    MOK_REQUIRE(ws);
  }
  const Layout L = layout_of(d, c.BM);
  char* wb = (char*)ws;
  const bool replay = is_replay(d);
  char* au = replay ? wb + L.bau : (char*)saved + L.au;
  char* hr = replay ? wb + L.bh : (char*)saved + L.h;
  float* dgp = (float*)(wb + L.dgp);
  float* dz = (float*)(wb + L.dz);
  if ((st = check_fused(d, c)) != MOK_OK) return st;
  if (is_fused(d) && c.R > 0) {
    if (replay) MOK_LAUNCH("fc1", c.s, launch_fc1(c, x, w->w1, au, hr));
    MOK_LAUNCH("backward_fused", c.s, launch_backward_fused(c, x, idx, gate, w->w1, w->w2, wr, au, hr, dy,
                                                            wb + L.dgu, wb + L.bpart, dgp, dz, wb + L.xs,
                                                            wb + L.dos, dx, dw1, dw2, dgate, dwr));
    return MOK_OK;
  }
  if (c.R > 0) {
    if (replay) MOK_LAUNCH("fc1", c.s, launch_fc1(c, x, w->w1, au, hr));  // the forward's FC1, again
    MOK_LAUNCH("dh", c.s, launch_dh(c, dy, w->w2, au, hr, gate, wb + L.dgu, dgp));
    MOK_LAUNCH("router_bwd", c.s, launch_router_bwd(c, dgp, gate, dgate, dz));
    MOK_LAUNCH("dx", c.s, launch_dx(c, wb + L.dgu, w->w1, wb + L.bpart));
    MOK_LAUNCH("dx_reduce", c.s, launch_dx_reduce(c, wb + L.bpart, dz, idx, wr, dx));
  }
  if (c.act == MOK_BF16) {
    // routed-order operands of the weight gradients: dO = bf16(g * dY) rows by a gather; the
    // x rows by the router-weight gradient, which reads each of them once (else a gather)
    MOK_LAUNCH("gather", c.s, launch_gather_rows(c, dy, gate, wb + L.dos));
    if (dwr != nullptr)
      MOK_LAUNCH("dwr", c.s, launch_dwr(c, dz, x, dwr, wb + L.xs));
    else
      MOK_LAUNCH("gather", c.s, launch_gather_rows(c, x, nullptr, wb + L.xs));
    MOK_LAUNCH("dw2", c.s, launch_dw2_bf16(c, wb + L.dos, hr, dw2));
    MOK_LAUNCH("dw1", c.s, launch_dw1_bf16(c, wb + L.dgu, wb + L.xs, dw1));
  } else {
    MOK_LAUNCH("dw2", c.s, launch_dw2(c, dy, gate, hr, dw2));
    MOK_LAUNCH("dw1", c.s, launch_dw1(c, wb + L.dgu, x, dw1));
    if (dwr != nullptr) MOK_LAUNCH("dwr", c.s, launch_dwr(c, dz, x, dwr, nullptr));
  }
  return MOK_OK;
}

mok_status mok_weights_quantize(const mok_desc* d, const void* w1, const void* w2, const mok_mx_weights* out,
                                void* stream) {
  mok_status st = check_desc(d);
  if (st != MOK_OK) return st;
  if (!is_mx(d)) return MOK_ERR_DTYPE;
  if (out == nullptr) return MOK_ERR_NULL;
  MOK_REQUIRE(w1);
  MOK_REQUIRE(w2);
  MOK_REQUIRE(out->w1q);
  MOK_REQUIRE(out->w1s);
  MOK_REQUIRE(out->w2q);
  MOK_REQUIRE(out->w2s);
  MOK_REQUIRE(out->w2tq);
  MOK_REQUIRE(out->w2ts);
  MOK_REQUIRE(out->w1tq);
  MOK_REQUIRE(out->w1ts);
  Ctx c{};
  c.E = d->E;
  c.H = d->H;
  c.I = d->I;
  c.mx4 = d->gemm == MOK_MXFP4;
  c.s = (hipStream_t)stream;
  const int64_t E = d->E, H = d->H, I = d->I;
  MOK_LAUNCH("quant", c.s, launch_mx_quant_rows(c, w1, E * 2 * I, (int)H, out->w1q, out->w1s, 2 * I));
  MOK_LAUNCH("quant", c.s, launch_mx_quant_rows(c, w2, E * H, (int)I, out->w2q, out->w2s, H));
  MOK_LAUNCH("quant", c.s, launch_mx_quant_cols(c, w2, H * I, I, nullptr, nullptr, (int)H, (int)I, (int)E, H,
                                                out->w2tq, out->w2ts));
  MOK_LAUNCH("quant", c.s, launch_mx_quant_cols(c, w1, 2 * I * H, H, nullptr, nullptr, (int)(2 * I), (int)H, (int)E,
                                                2 * I, out->w1tq, out->w1ts));
  return MOK_OK;
}

mok_status mok_trace_bind(mok_trace* t) {
  if (t == nullptr) {
    t_trace = nullptr;
    return MOK_OK;
  }
  if (t->filter == nullptr || t->events == nullptr) return MOK_ERR_NULL;
  if (t->capacity < 0 || t->capacity > MOK_TRACE_MAX || t->count < 0) return MOK_ERR_SHAPE;
  t_trace = t;
  return MOK_OK;
}

const char* mok_status_string(mok_status s) {
  switch (s) {
    case MOK_OK: return "ok";
    case MOK_ERR_NULL: return "required pointer is NULL";
    case MOK_ERR_ALIGN: return "pointer is not 16-byte aligned";
    case MOK_ERR_SHAPE: return "descriptor size out of range";
    case MOK_ERR_DTYPE: return "unsupported dtype combination";
    case MOK_ERR_HIP: return "HIP call failed";
    case MOK_ERR_WORKSPACE: return "caller buffer smaller than the descriptor needs";
    case MOK_ERR_SCHEDULE_MISMATCH: return "schedule built for another descriptor";
  }
  return "unknown status";
}

int32_t mok_version(void) { return 301; }

}  // extern "C"
