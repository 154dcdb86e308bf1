// C-ABI entry points of libmok: argument checks, buffer layouts, launches.
#include <mutex>
#include <string>

#include "kernels.h"

using namespace mok;

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_size(int act) { return act == MOK_F32 ? 4 : 2; }

mok_status check_desc(const mok_desc* d) {
  if (d == nullptr) return MOK_ERR_NULL;
  if (d->act != MOK_F32 && d->act != MOK_BF16) return MOK_ERR_DTYPE;
  if (d->gemm != d->act) return MOK_ERR_DTYPE;
  if (d->T < 0 || d->E < 1 || d->E > 1024 || d->k < 1 || d->k > 16 || d->k > d->E) return MOK_ERR_SHAPE;
  if (d->H <= 0 || d->I <= 0 || d->H % 128 != 0 || d->I % 128 != 0) return MOK_ERR_SHAPE;
  if (d->T * (int64_t)d->k >= ((int64_t)1 << 31)) return MOK_ERR_SHAPE;
  // 32-bit byte offsets inside one operand: token rows, routed rows, one expert's weights
  if (d->T * (int64_t)d->H >= ((int64_t)1 << 31)) return MOK_ERR_SHAPE;
  if (d->T * (int64_t)d->k * 2 * d->I >= ((int64_t)1 << 31)) return MOK_ERR_SHAPE;
  if ((int64_t)d->I * 2 * d->H >= ((int64_t)1 << 31)) return MOK_ERR_SHAPE;
  if (d->tile_m != 0 && d->tile_m != 32 && d->tile_m != 64 && d->tile_m != 128) return MOK_ERR_SHAPE;
  if (d->grid < 0) return MOK_ERR_SHAPE;
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
// tiles in the FC1 GEMM, else the smallest tile.
int choose_tile_m(int64_t R, int I, int cus) {
  const int cands[3] = {128, 64, 32};
  for (int bm : cands)
    if ((R / bm) * (int64_t)(2 * I / 256) >= 2LL * cus) return bm;
  return 32;
}

struct Layout {
  int BM = 32, max_tiles = 0;
  size_t counts, offsets, tile_start, num_tiles, perm, inv, tiles, sched;
  size_t au, h, saved;
  size_t fwd_part, fwd;
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
  size_t o = 0;
  L.counts = o; o = up(o + 4 * (size_t)d->E);
  L.offsets = o; o = up(o + 4 * (size_t)(d->E + 1));
  L.tile_start = o; o = up(o + 4 * (size_t)(d->E + 1));
  L.num_tiles = o; o = up(o + 4);
  L.perm = o; o = up(o + 4 * (size_t)R);
  L.inv = o; o = up(o + 4 * (size_t)R);
  L.tiles = o; o = up(o + 16 * (size_t)std::max<int64_t>(worst_tiles, 1));
  L.sched = o;
  o = 0;
  L.au = o; o = up(o + es * (size_t)R * 2 * d->I);
  L.h = o; o = up(o + es * (size_t)R * d->I);
  L.saved = o;
  L.fwd_part = 0;
  L.fwd = up(es * (size_t)R * d->H);
  o = 0;
  L.dgu = o; o = up(o + es * (size_t)R * 2 * d->I);
  L.bpart = o; o = up(o + es * (size_t)R * d->H);
  L.dgp = o; o = up(o + 4 * (size_t)R * dh_ntiles(d->I));
  L.dz = o; o = up(o + 4 * (size_t)R);
  // bf16: token rows in routed order for the weight-gradient GEMMs (x and g*dy)
  const size_t rows = d->act == MOK_BF16 ? es * (size_t)R * d->H : 0;
  L.xs = o; o = up(o + rows);
  L.dos = o; o = up(o + rows);
  L.bwd = o;
  return L;
}

mok_status resolve(const mok_desc* d, Layout* L, int* cus) {
  mok_status st = check_desc(d);
  if (st != MOK_OK) return st;
  st = device_cus(cus);
  if (st != MOK_OK) return st;
  const int bm = d->tile_m ? d->tile_m : choose_tile_m(d->T * d->k, d->I, *cus);
  *L = layout_of(d, bm);
  return MOK_OK;
}

mok_status make_ctx(const mok_desc* d, const void* sched, void* stream, Ctx* c) {
  Layout L;
  int cus = 0;
  mok_status st = resolve(d, &L, &cus);
  if (st != MOK_OK) return st;
  char* sb = (char*)sched;
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
  c->s = (hipStream_t)stream;
  c->counts = (int32_t*)(sb + L.counts);
  c->offsets = (int32_t*)(sb + L.offsets);
  c->tile_start = (int32_t*)(sb + L.tile_start);
  c->num_tiles = (int32_t*)(sb + L.num_tiles);
  c->perm = (int32_t*)(sb + L.perm);
  c->inv = (int32_t*)(sb + L.inv);
  c->tiles = (int4*)(sb + L.tiles);
  return MOK_OK;
}

#define MOK_REQUIRE(p)                   \
  do {                                   \
    if ((p) == nullptr) return MOK_ERR_NULL;  \
    if (!aligned16(p)) return MOK_ERR_ALIGN; \
  } while (0)

// ---- measurement trace (see mok_trace_set) ----
struct Trace {
  std::string filter;
  void* const* events = nullptr;
  int cap = 0;
  int count = 0;
  const char* names[4096];
};
Trace g_trace;

bool trace_on(const char* name) {
  return g_trace.events != nullptr && g_trace.count < g_trace.cap &&
         (g_trace.filter == "*" || g_trace.filter == name);
}

// Launch `call` (a hipError_t expression) bracketed by trace events when traced.
#define MOK_LAUNCH(name, stream, call)                                                              \
  do {                                                                                              \
    const bool tr_ = trace_on(name);                                                                \
    if (tr_ && hipEventRecord((hipEvent_t)g_trace.events[2 * g_trace.count], stream) != hipSuccess) \
      return MOK_ERR_HIP;                                                                           \
    if ((call) != hipSuccess) return MOK_ERR_HIP;                                                   \
    if (tr_) {                                                                                      \
      if (hipEventRecord((hipEvent_t)g_trace.events[2 * g_trace.count + 1], stream) != hipSuccess)  \
        return MOK_ERR_HIP;                                                                         \
      if (g_trace.count < 4096) g_trace.names[g_trace.count] = name;                                \
      ++g_trace.count;                                                                              \
    }                                                                                               \
  } while (0)

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
  return MOK_OK;
}

mok_status mok_schedule_layout_query(const mok_desc* d, mok_schedule_layout* out) {
  if (out == nullptr) return MOK_ERR_NULL;
  Layout L;
  int cus = 0;
  mok_status st = resolve(d, &L, &cus);
  if (st != MOK_OK) return st;
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
  MOK_LAUNCH("route", c.s, launch_route(c, x, wr, bias, idx, gate, logits));
  return MOK_OK;
}

mok_status mok_schedule_build(const mok_desc* d, const int32_t* idx, void* sched, void* stream) {
  MOK_REQUIRE(sched);
  Ctx c;
  mok_status st = make_ctx(d, sched, stream, &c);
  if (st != MOK_OK) return st;
  if (c.R > 0) MOK_REQUIRE(idx);
  MOK_LAUNCH("schedule", c.s, launch_schedule(c, idx));
  return MOK_OK;
}

mok_status mok_moe_forward(const mok_desc* d, const void* sched, const void* x, const float* gate,
                           const mok_weights* w, void* y, void* saved, void* ws, void* stream) {
  MOK_REQUIRE(sched);
  if (w == nullptr) return MOK_ERR_NULL;
  Ctx c;
  mok_status st = make_ctx(d, sched, stream, &c);
  if (st != MOK_OK) return st;
  if (c.R == 0) return MOK_OK;
  MOK_REQUIRE(x);
  MOK_REQUIRE(gate);
  MOK_REQUIRE(w->w1);
  MOK_REQUIRE(w->w2);
  MOK_REQUIRE(y);
  MOK_REQUIRE(saved);
  MOK_REQUIRE(ws);
  const Layout L = layout_of(d, c.BM);
  char* sv = (char*)saved;
  MOK_LAUNCH("fc1", c.s, launch_fc1(c, x, w->w1, sv + L.au, sv + L.h));
  MOK_LAUNCH("fc2", c.s, launch_fc2(c, sv + L.h, w->w2, ws));
  MOK_LAUNCH("combine", c.s, launch_combine(c, ws, gate, y));
  return MOK_OK;
}

mok_status mok_moe_backward(const mok_desc* d, const void* sched, const void* x, const int32_t* idx,
                            const float* gate, const mok_weights* w, const void* wr, const void* saved,
                            const void* dy, void* dx, void* dw1, void* dw2, float* dgate, void* dwr, void* ws,
                            void* stream) {
  MOK_REQUIRE(sched);
  if (w == nullptr) return MOK_ERR_NULL;
  Ctx c;
  mok_status st = make_ctx(d, sched, stream, &c);
  if (st != MOK_OK) return st;
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
    MOK_REQUIRE(saved);
    MOK_REQUIRE(dy);
    MOK_REQUIRE(dx);
    MOK_REQUIRE(dgate);
    MOK_REQUIRE(ws);
  }
  const Layout L = layout_of(d, c.BM);
  const char* sv = (const char*)saved;
  char* wb = (char*)ws;
  float* dgp = (float*)(wb + L.dgp);
  float* dz = (float*)(wb + L.dz);
  if (c.R > 0) {
    MOK_LAUNCH("dh", c.s, launch_dh(c, dy, w->w2, sv + L.au, sv + L.h, gate, wb + L.dgu, dgp));
    MOK_LAUNCH("router_bwd", c.s, launch_router_bwd(c, dgp, gate, dgate, dz));
    MOK_LAUNCH("dx", c.s, launch_dx(c, wb + L.dgu, w->w1, wb + L.bpart));
    MOK_LAUNCH("dx_reduce", c.s, launch_dx_reduce(c, wb + L.bpart, dz, idx, wr, dx));
  }
  if (c.act == MOK_BF16) {
    MOK_LAUNCH("gather", c.s, launch_gather_rows(c, dy, gate, wb + L.dos));
    MOK_LAUNCH("gather", c.s, launch_gather_rows(c, x, nullptr, wb + L.xs));
    MOK_LAUNCH("dw2", c.s, launch_dw2_bf16(c, wb + L.dos, sv + L.h, dw2));
    MOK_LAUNCH("dw1", c.s, launch_dw1_bf16(c, wb + L.dgu, wb + L.xs, dw1));
  } else {
    MOK_LAUNCH("dw2", c.s, launch_dw2(c, dy, gate, sv + L.h, dw2));
    MOK_LAUNCH("dw1", c.s, launch_dw1(c, wb + L.dgu, x, dw1));
  }
  if (dwr != nullptr) MOK_LAUNCH("dwr", c.s, launch_dwr(c, dz, x, dwr));
  return MOK_OK;
}

mok_status mok_trace_set(const char* name, void* const* events, int32_t capacity) {
  if (name == nullptr) {
    g_trace.events = nullptr;
    g_trace.cap = 0;
    return MOK_OK;
  }
  if (events == nullptr) return MOK_ERR_NULL;
  if (capacity < 0) return MOK_ERR_SHAPE;
  g_trace.filter = name;
  g_trace.events = events;
  g_trace.cap = std::min(capacity, 4096);
  g_trace.count = 0;
  return MOK_OK;
}

int32_t mok_trace_count(void) { return g_trace.count; }

const char* mok_trace_name(int32_t n) { return (n >= 0 && n < g_trace.count && n < 4096) ? g_trace.names[n] : nullptr; }

const char* mok_status_string(mok_status s) {
  switch (s) {
    case MOK_OK: return "ok";
    case MOK_ERR_NULL: return "required pointer is NULL";
    case MOK_ERR_ALIGN: return "pointer is not 16-byte aligned";
    case MOK_ERR_SHAPE: return "descriptor size out of range";
    case MOK_ERR_DTYPE: return "unsupported dtype combination";
    case MOK_ERR_HIP: return "HIP call failed";
  }
  return "unknown status";
}

int32_t mok_version(void) { return 100; }

}  // extern "C"
