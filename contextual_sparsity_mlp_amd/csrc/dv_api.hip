// dv_api.hip - the C ABI of include/dv.h: argument checks, workspace layout,
// grid planning and launches.  Every check runs on the host before anything is
// enqueued, so all error codes can be produced without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cassert>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dv.h"
#include "dv_internal.h"

using namespace dv;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// Bounded in-launch waits: poll limit and a target offset that tests raise to make
// every wait give up (dv_debug_wait_limits).
constexpr uint32_t kDefaultSpins = 1u << 20;
std::atomic<uint32_t> g_wait_spins{kDefaultSpins};
std::atomic<uint32_t> g_wait_extra{0};

// Launch plan of the one-token bf16 sparse step (dv_set_step_path).
std::atomic<int> g_step_path{DV_PATH_AUTO};
constexpr int kAutoStepPath = DV_PATH_TWO_LAUNCH;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int cdiv(int a, int b) { return (a + b - 1) / b; }
size_t esize(dv_dtype t) { return t == DV_FP8 ? 1 : (t == DV_BF16 ? 2 : 4); }
bool valid_dtype(int t) { return t == DV_F32 || t == DV_BF16; }
int wcode(dv_dtype t) { return t == DV_FP8 ? W_FP8 : (t == DV_BF16 ? W_BF16 : W_F32); }
bool valid_act(int a) { return a == DV_ACT_RELU || a == DV_ACT_GELU; }
int act_code(int a) { return a == DV_ACT_GELU ? A_GELU : A_RELU; }

#define CHECK_PTR(p) \
  do { if (!(p)) return fail(DV_EINVAL, "%s: %s is NULL", fn, #p); } while (0)
#define CHECK_ALIGN(p) \
  do { if (!aligned16(p)) return fail(DV_EALIGN, "%s: %s is not 16-byte aligned", fn, #p); } while (0)

// ------------------------------------------------------------------------- //
// device properties                                                         //
// ------------------------------------------------------------------------- //

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// ------------------------------------------------------------------------- //
// phase timing                                                              //
// ------------------------------------------------------------------------- //

struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;     // 2 events per record
  size_t used = 0;                  // events handed out
  struct Rec { int slot; hipEvent_t a, b; };
  std::vector<Rec> recs;
};
TimingState& timing() { static TimingState t; return t; }
constexpr size_t kTimingPairs = 8192;

// Per-call launch counter (the k-th launch of the current entry point).
thread_local int t_slot = 0;

// Event pair of the next launch slot when timing is on (null otherwise); the launch
// hands them to the runtime, which stamps them with the kernel's own start and end.
struct SlotEvents { hipEvent_t a = nullptr, b = nullptr; };
SlotEvents slot_events() {
  TimingState& T = timing();
  SlotEvents ev;
  const int slot = t_slot++;
  if (T.on) {
    std::lock_guard<std::mutex> g(T.mu);
    if (T.used + 2 <= T.pool.size()) {
      ev.a = T.pool[T.used++];
      ev.b = T.pool[T.used++];
      T.recs.push_back({slot, ev.a, ev.b});
    }
  }
  return ev;
}

int axpy_mfma_lds(int tokens);
int launch(int flags, int bt, const PhaseArgs& a, int grid, int lds, void* stream, const char* fn) {
  if (grid <= 0) return DV_OK;
  if (flags & T_AXPY)
    for (int s = 0; s < a.axpy.nseg; ++s) {
      if (a.axpy.seg[s].mfma_nt) flags |= T_MFMA;
      if (a.axpy.seg[s].mfma_nt == 2) flags |= T_MFMA2;
    }
  if (flags & T_MFMA) {
    lds = std::max(lds, axpy_mfma_lds((flags & T_MFMA2) ? 32 : 16));
    // matrix-core launches run the bt-4 kernel instances; at 2 tokens (the look-ahead
    // output row sum) every row sum of the launch is a matrix-core one, so the wave
    // path's token tile does not arise
    bool all = true;
    for (int s = 0; s < a.axpy.nseg; ++s) all = all && a.axpy.seg[s].mfma_nt > 0;
    if (all) bt = 4;
  }
  const SlotEvents ev = slot_events();
  const int err = launch_phase(flags, bt, a, grid, lds, stream, ev.a, ev.b);
  if (err != 0)
    return fail(DV_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString((hipError_t)err));
  return DV_OK;
}

// ------------------------------------------------------------------------- //
// workspace layout                                                          //
// ------------------------------------------------------------------------- //

struct Ws {
  size_t off = 0;
  size_t take(size_t bytes) { size_t o = off; off = align256(off + bytes); return o; }
};

int pick_bt(int batch) { return batch <= 1 ? 1 : (batch == 2 ? 2 : 4); }

// Axpy segment geometry that does not depend on the device.  A batch of at least
// kAxMfmaMinBatch tokens over bf16 rows whose row length is a multiple of 128 runs on
// the matrix cores (128-column slices, 16 tokens per block tile, 32 above 16 tokens);
// otherwise the wave path (pick_bt tokens per block, each row read once per block
// tile).
struct AxGeo { int vec, nslices, nbt, chunks_max, mfma_nt, bt; };
AxGeo ax_geo(int batch, int ncols, long long row_stride, dv_dtype wdt, int cap_rows,
             int mfma_min_batch = kAxMfmaMinBatch) {
  AxGeo g;
  const int full = (wdt == DV_FP8) ? 16 : ((wdt == DV_BF16) ? 8 : 4);
  g.vec = (ncols % full == 0 && row_stride % full == 0) ? full : 1;
  g.mfma_nt = 0;
  if (batch >= mfma_min_batch && wdt == DV_BF16 && ncols % kMfmaCols == 0 && row_stride % 8 == 0)
    g.mfma_nt = batch <= kMfmaRows ? 1 : 2;
  g.nslices = g.mfma_nt ? ncols / kMfmaCols : cdiv(ncols, kAxSliceLanes * g.vec);
  g.bt = g.mfma_nt ? kMfmaRows * g.mfma_nt : pick_bt(batch);
  g.nbt = cdiv(batch, g.bt);
  g.chunks_max = std::max(1, std::min(kMaxChunks, cap_rows));
  return g;
}
size_t ax_partial_floats(int batch, int ncols, const AxGeo& g) {
  (void)batch;
  return (size_t)g.nbt * g.chunks_max * g.bt * ncols;
}
size_t ax_tickets(const AxGeo& g) { return (size_t)g.nbt * g.nslices; }

int attn_nsplit_max(int n_ctx) { return std::max(1, std::min(kMaxSplit, cdiv(n_ctx, 64))); }

// Top-k scratch for one problem (N scores per row, `batch` rows).
struct TopkWs { size_t bits, cand, ccount; int nseg, nwords; };
TopkWs plan_topk_parts(Ws& w, int batch, int N) {
  TopkWs t;
  t.nseg = cdiv(N, kSegElems);
  t.nwords = cdiv(N, 32);
  t.bits = w.take((size_t)batch * t.nwords * 4);
  t.cand = w.take((size_t)batch * t.nseg * kSegElems * 8);
  t.ccount = w.take((size_t)batch * t.nseg * 4);
  return t;
}

// Matrix-core row dots with y in LDS (RowdotTask::mfma_nt 3) split each 128-row unit's
// row length into parts when there are few units: each part stores a partial tile
// (2048 floats) and the last part to finish (per-unit ticket) sums them in part order.
// Parts are chosen so that units x parts stays near kRdItems, so the partials need at
// most (kRdItems + units) tiles.  Sized from a bound on the rows.
constexpr int kRdItems = 1024;
constexpr int kRdUnitRows = kWaves * kMfmaRT * kMfmaRows;   // 128
constexpr int kRdTile = kWaves * kMfmaRT * 4 * 64 * 2;      // partial tile floats (32 tokens)
struct RdWs { size_t partial = 0, tickets = 0; int ticket_words = 0; };
bool rd_lds_path(int batch, int d) {
  return batch >= kMfmaMinBatch && batch <= 2 * kMfmaRows && d % kMfmaCols == 0;
}
int rd_parts(int units, int d) {
  const int max_parts = std::max(1, d / kMfmaCols / 4);      // at least 4 steps a part
  return std::max(1, std::min(cdiv(kRdItems, std::max(units, 1)), max_parts));
}
RdWs plan_rd(Ws& w, int batch, int d, int rows_bound, bool bf16_rows) {
  RdWs p;
  if (!bf16_rows || !rd_lds_path(batch, d)) return p;
  const int units = cdiv(std::max(rows_bound, 1) + kMaxSeg * kMfmaRows, kRdUnitRows);
  p.partial = w.take((size_t)(kRdItems + units) * kRdTile * 4);
  p.ticket_words = units;
  p.tickets = w.take((size_t)p.ticket_words * 4);
  return p;
}

struct PredictWs { size_t z, tickets, partial, total; int nt; RdWs rd; };
PredictWs plan_predict(int batch, int d, int r, int N, dv_dtype wdt) {
  PredictWs p; Ws w;
  const AxGeo g = ax_geo(batch, N, N, wdt, r);
  p.nt = (int)ax_tickets(g);
  p.z = w.take((size_t)batch * r * 4);
  p.tickets = w.take((size_t)p.nt * 4);
  p.partial = w.take(ax_partial_floats(batch, N, g) * 4);
  p.rd = plan_rd(w, batch, d, r, wdt == DV_BF16);
  p.total = w.off;
  return p;
}

// Zero region first: histogram [batch][kHistBins], row tickets [batch], union ticket.
struct SelectWs { size_t zero, hist, rtick, ticket, total; int zero_words; TopkWs t; };
SelectWs plan_select(int batch, int N) {
  SelectWs p; Ws w;
  p.zero = w.off;
  p.hist = p.zero;
  p.rtick = p.hist + (size_t)batch * kHistBins * 4;
  p.ticket = p.rtick + (size_t)batch * 4;
  w.off = align256(p.ticket + 4);
  p.zero_words = (int)((p.ticket + 4 - p.zero) / 4);
  p.t = plan_topk_parts(w, batch, N);
  p.total = w.off;
  return p;
}

struct MlpWs { size_t a, tickets, partial, total; int nt; RdWs rd; };
MlpWs plan_mlp(int batch, int d, int cap, dv_dtype wdt) {
  MlpWs p; Ws w;
  const AxGeo g = ax_geo(batch, d, d, wdt, std::max(cap, 1));
  p.nt = (int)ax_tickets(g);
  p.a = w.take((size_t)batch * std::max(cap, 1) * 4);
  p.tickets = w.take((size_t)p.nt * 4);
  p.partial = w.take(ax_partial_floats(batch, d, g) * 4);
  p.rd = plan_rd(w, batch, d, cap, wdt == DV_BF16);
  p.total = w.off;
  return p;
}

struct MhaWs { size_t q, o, part, tickets, partial, total; int nt_attn, nt_ax; RdWs rd; };
MhaWs plan_mha(int batch, int d, int dh, int n_ctx, int cap, dv_dtype wdt) {
  MhaWs p; Ws w;
  cap = std::max(cap, 1);
  const AxGeo g = ax_geo(batch, d, d, wdt, cap * dh);
  p.nt_attn = batch * cap;
  p.nt_ax = (int)ax_tickets(g);
  p.q = w.take((size_t)batch * cap * dh * 4);
  p.o = w.take((size_t)batch * cap * dh * 4);
  p.part = w.take((size_t)batch * cap * attn_nsplit_max(n_ctx) * (dh + 2) * 4);
  p.tickets = w.take((size_t)(p.nt_attn + p.nt_ax) * 4);
  p.partial = w.take(ax_partial_floats(batch, d, g) * 4);
  p.rd = plan_rd(w, batch, d, cap * dh, wdt == DV_BF16);
  p.total = w.off;
  return p;
}

// Geometry of the one-launch sparse step (StreamTask) for one token: cap_m neuron
// slots, cap_a head slots, n_att keys per head.
struct StreamGeo {
  int n_qi, n_mi, ncm, per_m, nslice, nsplit, n_a, n_items;
  int c_qdone, c_mdone, c_oready, c_stick, nctr, npart;
};
int attn_splits(int n, int base, int other_blocks);
StreamGeo stream_geo(int d, int dh, int n_att, int cap_m, int cap_a) {
  StreamGeo g;
  g.n_qi = cdiv(cap_a * dh, kStreamDotRows);
  g.n_mi = cdiv(cap_m, kStreamDotRows);
  g.per_m = cdiv(std::max(1, cdiv(std::max(cap_m, 1), kStreamChunks)), kStreamDotRows) *
            kStreamDotRows;
  g.ncm = std::max(1, cdiv(cap_m, g.per_m));
  g.nslice = cdiv(d, kStreamSlice);
  g.nsplit = attn_splits(std::max(n_att, 1), std::max(cap_a, 1), 1);
  g.n_a = cap_a * g.nsplit;
  g.n_items = g.n_qi + g.n_mi + g.n_a + g.ncm * g.nslice + g.nslice * cap_a;
  g.c_qdone = kStreamQueues;
  g.c_mdone = g.c_qdone + cap_a;
  g.c_oready = g.c_mdone + g.ncm;
  g.c_stick = g.c_oready + cap_a;
  g.nctr = g.c_stick + g.nslice;
  g.npart = g.ncm + cap_a;
  return g;
}

// Zero region first: all tickets, both score histograms, row and union tickets.
struct LayerWs {
  size_t zero, tickets, hist_m, hist_a, rtick_m, rtick_a, uticket, done;
  size_t a, q, o, part, zm, za, sm, sa;
  size_t p_bm, p_ba, p_wo, total;
  size_t s_ctr = 0, s_atick = 0, s_y = 0, s_partial = 0;   // one-launch sparse step (one token)
  int s_zero_words = 0;                                     // counters + attention tickets
  int t_attn, t_bm, t_ba, t_wo, t_total, zero_words;
  TopkWs tm, ta;
  RdWs rd;
};
LayerWs plan_layer(int batch, int d, int F, int h, int dh, int n_ctx, int r, int cap_m, int cap_a,
                   dv_dtype wdt, dv_dtype pwdt) {
  LayerWs p; Ws w;
  cap_m = std::max(cap_m, 1);
  cap_a = std::max(cap_a, 1);
  const AxGeo g_bm = ax_geo(batch, F, F, pwdt, r);
  const AxGeo g_ba = ax_geo(batch, h, h, pwdt, r);
  const AxGeo g_wo = ax_geo(batch, d, d, wdt, cap_m + cap_a * dh);   // W2 and W^O rows
  // (the look-ahead step's output row sum takes the matrix cores from 2 tokens: room
  // for either geometry)
  const AxGeo g_wo2 = ax_geo(batch, d, d, wdt, cap_m + cap_a * dh, 2);
  p.t_attn = batch * cap_a;
  p.t_bm = (int)ax_tickets(g_bm);
  p.t_ba = (int)ax_tickets(g_ba);
  p.t_wo = (int)std::max(ax_tickets(g_wo), ax_tickets(g_wo2));
  p.t_total = p.t_attn + p.t_bm + p.t_ba + p.t_wo;
  // zero region: tickets | hist_m | hist_a | union tickets (2)
  p.zero = w.off;
  p.tickets = p.zero;
  p.hist_m = p.tickets + (size_t)p.t_total * 4;
  p.hist_a = p.hist_m + (size_t)batch * kHistBins * 4;
  p.rtick_m = p.hist_a + (size_t)batch * kHistBins * 4;
  p.rtick_a = p.rtick_m + (size_t)batch * 4;
  p.uticket = p.rtick_a + (size_t)batch * 4;
  // per head slot, o stored (single-launch path): one counter per 256-byte line
  p.done = align256(p.uticket + 8);
  const size_t done_bytes = (size_t)cap_a * kCtrStride * 4;
  w.off = align256(p.done + done_bytes);
  p.zero_words = (int)((p.done + done_bytes - p.zero) / 4);
  p.a = w.take((size_t)batch * cap_m * 4);
  p.q = w.take((size_t)batch * cap_a * dh * 4);
  p.o = w.take((size_t)batch * cap_a * dh * 4);
  // pieces for n_ctx + 1 attended rows: room for the step with the KV append
  p.part = w.take((size_t)batch * cap_a * attn_nsplit_max(n_ctx + 1) * (dh + 2) * 4);
  p.zm = w.take((size_t)batch * r * 4);
  p.za = w.take((size_t)batch * r * 4);
  p.sm = w.take((size_t)batch * F * 4);
  p.sa = w.take((size_t)batch * h * 4);
  p.p_bm = w.take(ax_partial_floats(batch, F, g_bm) * 4);
  p.p_ba = w.take(ax_partial_floats(batch, h, g_ba) * 4);
  p.p_wo = w.take(std::max(ax_partial_floats(batch, d, g_wo), ax_partial_floats(batch, d, g_wo2)) * 4);
  p.tm = plan_topk_parts(w, batch, F);
  p.ta = plan_topk_parts(w, batch, h);
  // row dots: W1 rows of S_M, W^Q rows of S_A and the two predictor factors
  p.rd = plan_rd(w, batch, d, cap_m + cap_a * dh + 2 * r, wdt == DV_BF16 && pwdt == DV_BF16);
  if (batch == 1) {
    const StreamGeo g = stream_geo(d, dh, n_ctx, cap_m, cap_a);
    p.s_ctr = w.take((size_t)g.nctr * kCtrStride * 4 + (size_t)cap_a * 4);
    p.s_atick = p.s_ctr + (size_t)g.nctr * kCtrStride * 4;
    p.s_zero_words = g.nctr * kCtrStride + cap_a;
    p.s_y = w.take((size_t)d * 4);
    p.s_partial = w.take((size_t)g.npart * d * 4);
  }
  p.total = w.off;
  return p;
}

// ------------------------------------------------------------------------- //
// task builders                                                             //
// ------------------------------------------------------------------------- //

RowList make_list(const int32_t* idx, const int32_t* count, int host_count, int expand, int items) {
  RowList L;
  L.idx = idx; L.count = count; L.host_count = host_count; L.expand = expand; L.items = items;
  return L;
}

// store: the segment's dots go into a KV cache row instead of out (RowdotTask::seg_store).
void add_rowdot(RowdotTask& T, const void* W, long long stride, dv_dtype wdt, RowList L, float* out,
                int out_ld, const float* scale = nullptr, void* store = nullptr) {
  assert(T.nseg < kMaxRowdotSeg);
  T.seg_scale[T.nseg] = scale;
  T.seg_store[T.nseg] = store;
  RowdotSeg& S = T.seg[T.nseg++];
  S.W = W; S.row_stride = stride; S.wdt = wcode(wdt);
  S.rows = L; S.out = out; S.out_ld = out_ld; S.cap = L.host_count * L.expand;
}

// Rowdot blocks: enough waves for every row, at most a few resident blocks per CU.
void finish_rowdot(RowdotTask& T, const float* y, int batch, int d, uint32_t* zero, int nzero,
                   char* ws, const RdWs& rd) {
  T.y = y; T.batch = batch; T.d = d;
  T.bt_lds = std::max(1, std::min(pick_bt(batch), kLdsBudget / (d * 4)));
  int cap = 0;
  for (int s = 0; s < T.nseg; ++s) cap += T.seg[s].cap;
  const int want = std::max(1, cdiv(cap, kWaves));
  // one resident round: LDS holds bt_lds * d floats per block
  const int per_cu = std::max(1, std::min(4, (160 * 1024) / std::max(1, T.bt_lds * d * 4)));
  T.blocks = std::min(want, device_cus() * per_cu);
  T.zero_ptr = zero; T.zero_words = nzero;
  // A batch of tokens over bf16 rows runs on the matrix cores, which read each row
  // once for up to 32 tokens, when the wave-per-row path would stream it more than
  // once (it stages bt_lds tokens of y in LDS at a time).
  bool mfma = batch >= kMfmaMinBatch && batch > T.bt_lds && d % kMfmaCols == 0;
  for (int s = 0; s < T.nseg; ++s) mfma = mfma && T.seg[s].wdt == W_BF16 && !T.seg_store[s];
  T.mfma_nt = 0;
  if (mfma) {
    T.mfma_nt = batch <= kMfmaRows ? 1 : 2;
    int tiles = 0;
    for (int s = 0; s < T.nseg; ++s) tiles += cdiv(T.seg[s].cap, kMfmaRows);
    T.blocks = std::max(1, std::min(cdiv(tiles, kMfmaRT), device_cus() * kMfmaBlocksPerCu));
    T.mfma_parts = 1;
    if (rd.ticket_words > 0 && rd_lds_path(batch, d)) {
      // y staged in LDS: 128-row units, row lengths split into parts when units are few
      const int units = cdiv(tiles, kWaves * kMfmaRT);
      assert(units <= rd.ticket_words);
      T.mfma_nt = batch <= kMfmaRows ? 3 : 4;     // 16 or 32 tokens a block
      T.mfma_parts = rd_parts(units, d);
      T.mfma_partial = reinterpret_cast<float*>(ws + rd.partial);
      T.mfma_tickets = reinterpret_cast<uint32_t*>(ws + rd.tickets);
      T.mfma_ticket_words = units;
      // resident blocks per CU: 4 with 16 tokens (109 registers), 3 with 32 (136)
      const int per_cu_lds = T.mfma_nt == 3 ? kMfmaLdsBlocksPerCu + 1 : kMfmaLdsBlocksPerCu;
      T.blocks = std::max(1, std::min(units * T.mfma_parts, device_cus() * per_cu_lds));
    }
  }
}
// The row-dot launch; row dots split into parts first clear their unit tickets (a
// small launch outside the per-launch timing slots).
int launch_rowdot(int flags, int bt, const PhaseArgs& a1, void* stream, const char* fn);
int rowdot_lds(const RowdotTask& T) {
  if (T.mfma_nt == 3 || T.mfma_nt == 4)     // two steps of y fragments (16 or 32 tokens) + flag
    return (T.mfma_nt - 2) * 2 * 4 * 2 * 64 * 16 + 16;
  if (T.mfma_nt > 0) return kWaves * kMfmaRT * T.mfma_nt * 4 * 64 * 4;
  return T.bt_lds * T.d * 4;
}

// Axpy segment over one row source, or two sources summed into the same columns
// (second source: W2 != nullptr; same stride and dtype, rows after the first's).
void add_axpy2(AxpyTask& T, int batch, const void* W, long long stride, dv_dtype wdt, RowList L,
               const float* coef, int coef_ld, int act, const void* W2, RowList L2,
               const float* coef2, int coef2_ld, int act2, int ncols, float* partial,
               uint32_t* tickets, float* out, int out_ld, const float* add0, const float* add1,
               int add_ld, int accumulate, int target_blocks, const float* scale = nullptr,
               const float* scale2 = nullptr, int mfma_min_batch = kAxMfmaMinBatch) {
  T.seg_scale[T.nseg][0] = scale;
  T.seg_scale[T.nseg][1] = scale2;
  AxpySeg& S = T.seg[T.nseg];
  int cap_rows = L.host_count * L.expand + (W2 ? L2.host_count * L2.expand : 0);
  cap_rows = std::max(1, cap_rows);
  const AxGeo g = ax_geo(batch, ncols, stride, wdt, cap_rows, mfma_min_batch);
  S.W = W; S.row_stride = stride; S.wdt = wcode(wdt);
  S.rows = L; S.coef = coef; S.coef_ld = coef_ld; S.act = act; S.ncols = ncols;
  S.W2 = W2; S.rows2 = L2; S.coef2 = coef2; S.coef2_ld = coef2_ld; S.act2 = act2;
  S.vec = g.vec; S.nslices = g.nslices; S.nbt = g.nbt; S.mfma_nt = g.mfma_nt;
  // About target_blocks blocks for the segment (512-byte row slices need many loads
  // in flight to stream well); at most kMaxChunks chunk partials per slice (a short,
  // fixed-order final sum) and at least one row per row group (a matrix-core block
  // takes 32 rows per wave at a time).
  const int per_chunk = g.nslices * g.nbt;
  int chunks = std::max(1, target_blocks / per_chunk);
  chunks = std::min(chunks, std::max(1, cap_rows / (g.mfma_nt ? kWaves * 32 : kAxGroups)));
  S.nchunks = std::max(1, std::min(chunks, g.chunks_max));
  S.block0 = T.blocks;
  S.partial = partial; S.tickets = tickets; S.hist = nullptr;
  S.out = out; S.out_ld = out_ld; S.add0 = add0; S.add1 = add1; S.add_ld = add_ld;
  S.accumulate = accumulate;
  T.blocks += S.nbt * S.nslices * S.nchunks;
  T.nseg++;
}

void add_axpy(AxpyTask& T, int batch, const void* W, long long stride, dv_dtype wdt, RowList L,
              const float* coef, int coef_ld, int act, int ncols, float* partial, uint32_t* tickets,
              float* out, int out_ld, const float* add0, const float* add1, int add_ld,
              int accumulate, int target_blocks) {
  add_axpy2(T, batch, W, stride, wdt, L, coef, coef_ld, act, nullptr, RowList{}, nullptr, 0, 0,
            ncols, partial, tickets, out, out_ld, add0, add1, add_ld, accumulate, target_blocks);
}

// Blocks that are resident at once for the light launch mixes: measured 8 per CU
// for 256-thread blocks of <= 64 VGPRs, <= 80 SGPRs and <= 20 KB of LDS.
int resident_blocks() { return 8 * device_cus(); }

// Chunk-share skews (AxpyTask::skew) of the row sums without waits: the wave path and
// the matrix-core path.
constexpr int kSkewWave = 32;
constexpr int kSkewMfma = 16;

// Row-sum grid of a launch that runs the segment alone: six blocks per CU.
int default_axpy_blocks() { return 6 * device_cus(); }

// LDS of a row-sum block: row ids and coefficients of a tile, and the row groups'
// column sums (kAxSliceLanes * vec columns per slice; vec 16 for fp8 rows), or the
// histogram of a row sum that builds one.
int axpy_lds(int bt, int vec = 8) {
  return std::max((kAxpyTileRows * (1 + bt) + kAxGroups * bt * kAxSliceLanes * vec) * 4,
                  (16 + kHistBins) * 4);
}
// LDS of a matrix-core row-sum block: row ids and a padded coefficient tile of
// kAxmTile rows for its 16 or 32 tokens, and the wave sums (a launch with T_MFMA takes
// the larger of this and its other tasks' needs).
int axpy_mfma_lds(int tokens) {
  return (kAxmTile + tokens * (kAxmTile + 4) + tokens * (kMfmaCols + 1)) * 4;
}

// Key splits per (token, head) for n keys and `base` (token, head) pairs: splits of
// about 128 keys keep each block's chain of dependent loads short; with few pairs and
// nothing else in the launch, more splits spread the cache over the chip.
int attn_splits(int n, int base, int other_blocks) {
  int ns = std::max(cdiv(n, 128), other_blocks > 0 ? 1 : cdiv(device_cus(), base));
  return std::max(1, std::min(ns, attn_nsplit_max(n)));
}

// n: cache rows attended; kv_cap: rows per (token, head) in K and V (>= n).
void setup_attn(AttnTask& A, const float* q, int q_ld, const void* K, const void* V, dv_dtype kvdt,
                int batch, int h, int n, int kv_cap, int dh, RowList heads, float scale, float* part,
                uint32_t* tickets, float* o, int o_ld, int other_blocks) {
  A.q = q; A.q_ld = q_ld; A.K = K; A.V = V; A.kvdt = (kvdt == DV_BF16) ? W_BF16 : W_F32;
  A.batch = batch; A.h = h; A.n = n; A.cap = kv_cap; A.dh = dh; A.heads = heads; A.scale = scale;
  const int cap = heads.host_count;
  const int ns = attn_splits(n, std::max(1, batch * cap), other_blocks);
  A.nsplit = ns;
  A.per = cdiv(n, ns);
  A.part = part; A.tickets = tickets; A.o = o; A.o_ld = o_ld;
  A.blocks = batch * cap * ns;
}
int attn_lds() { return (128 + 2048 + 16) * 4; }

int hist_lds() { return kHistBins * 4; }
int classify_lds() { return (16 + kLowBins + kResolveWords + kMaxSegs + 1) * 4; }

// One top-k problem over `batch` score rows of N (row stride ld).
TopkProblem make_topk(const float* scores, int ld, int N, int k, int batch, int unite,
                      int32_t* idx, int32_t* count, uint32_t* hist, uint32_t* row_tickets,
                      uint32_t* ticket, char* ws, const TopkWs& t) {
  TopkProblem P{};
  P.scores = scores; P.ld = ld; P.N = N; P.k = k; P.batch = batch;
  P.unite = (unite && batch > 1) ? 1 : 0;
  P.idx = idx; P.count = count; P.hist = hist; P.row_tickets = row_tickets; P.ticket = ticket;
  P.bits = reinterpret_cast<uint32_t*>(ws + t.bits);
  P.nwords = cdiv(N, 32);
  P.cand = reinterpret_cast<uint2*>(ws + t.cand);
  P.ccount = reinterpret_cast<int32_t*>(ws + t.ccount);
  P.nseg = cdiv(N, kSegElems);
  return P;
}
int topk_seg_blocks(const TopkTask& T) {
  int n = 0;
  for (int i = 0; i < T.np; ++i) n += T.p[i].batch * T.p[i].nseg;
  return n;
}

PhaseArgs zero_args() {
  PhaseArgs a;
  memset(&a, 0, sizeof a);
  return a;
}

int launch_rowdot(int flags, int bt, const PhaseArgs& a1, void* stream, const char* fn) {
  const RowdotTask& T = a1.rowdot;
  if ((T.mfma_nt == 3 || T.mfma_nt == 4) && T.mfma_parts > 1) {
    PhaseArgs z = zero_args();
    z.zero.ptr = T.mfma_tickets;
    z.zero.words = T.mfma_ticket_words;
    z.zero.blocks = std::max(1, std::min(cdiv(T.mfma_ticket_words, kThreads * 4), 64));
    const int err = launch_phase(T_ZERO, 1, z, z.zero.blocks, 0, stream);
    if (err != 0)
      return fail(DV_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString((hipError_t)err));
  }
  return launch(flags, bt, a1, T.blocks, rowdot_lds(T), stream, fn);
}

// ------------------------------------------------------------------------- //
// shared validation                                                         //
// ------------------------------------------------------------------------- //

int check_ws(const char* fn, void* ws, size_t ws_bytes, size_t need) {
  if (need > 0 && !ws) return fail(DV_EWORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (ws_bytes < need)
    return fail(DV_EWORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
  if (ws && !aligned16(ws)) return fail(DV_EALIGN, "%s: ws is not 16-byte aligned", fn);
  return DV_OK;
}

int check_d(const char* fn, int d) {
  if (d <= 0) return fail(DV_EINVAL, "%s: d = %d must be positive", fn, d);
  if (d % 8 != 0) return fail(DV_EALIGN, "%s: d = %d must be a multiple of 8", fn, d);
  if (d * 4 > kLdsBudget) return fail(DV_EUNSUPPORTED, "%s: d = %d exceeds %d", fn, d, kLdsBudget / 4);
  return DV_OK;
}

constexpr int kMaxCtx = 1 << 20;

int check_nctx(const char* fn, int n) {
  if (n <= 0) return fail(DV_EINVAL, "%s: n_ctx = %d must be >= 1", fn, n);
  if (n > kMaxCtx) return fail(DV_EUNSUPPORTED, "%s: n_ctx = %d exceeds %d", fn, n, kMaxCtx);
  return DV_OK;
}

int check_dh(const char* fn, int dh) {
  if (dh != 32 && dh != 64 && dh != 128 && dh != 256)
    return fail(DV_EUNSUPPORTED, "%s: dh = %d not in {32, 64, 128, 256}", fn, dh);
  return DV_OK;
}

}  // namespace

// =========================================================================== //
// C ABI                                                                       //
// =========================================================================== //

extern "C" {

const char* dv_last_error(void) { return g_err.c_str(); }

int dv_version(void) { return 104; }

static size_t ws_bytes_for(int op, const dv_shape* s, dv_dtype wdt) {
  const int B = s->batch;
  switch (op) {
    case DV_OP_PREDICT: return plan_predict(B, s->d, s->r, s->N, wdt).total;
    case DV_OP_SELECT_TOPK: return plan_select(B, s->N).total;
    case DV_OP_SPARSE_MLP: return plan_mlp(B, s->d, s->max_count_m, wdt).total;
    case DV_OP_SPARSE_MHA: return plan_mha(B, s->d, s->dh, s->n_ctx, s->max_count_a, wdt).total;
    default:
      // (fp8 weights need no more: their row sums have fewer slices, the predictor
      // factors are bf16 or fp32)
      return plan_layer(B, s->d, s->F, s->h, s->dh, s->n_ctx, s->r, s->max_count_m, s->max_count_a,
                        wdt, wdt).total;
  }
}

size_t dv_workspace_bytes(int op, const dv_shape* s) {
  const char* fn = "dv_workspace_bytes";
  if (!s) { fail(DV_EINVAL, "%s: shape is NULL", fn); return 0; }
  const int B = s->batch;
  if (B <= 0) { fail(DV_EINVAL, "%s: batch = %d", fn, B); return 0; }
  switch (op) {
    case DV_OP_PREDICT:
      if (s->r <= 0 || s->N <= 0 || s->d <= 0) { fail(DV_EINVAL, "%s: bad predict shape", fn); return 0; }
      break;
    case DV_OP_SELECT_TOPK:
      if (s->N <= 0) { fail(DV_EINVAL, "%s: N = %d", fn, s->N); return 0; }
      break;
    case DV_OP_SPARSE_MLP:
      if (s->d <= 0 || s->max_count_m < 0) { fail(DV_EINVAL, "%s: bad mlp shape", fn); return 0; }
      break;
    case DV_OP_SPARSE_MHA:
      if (s->d <= 0 || s->dh <= 0 || s->n_ctx <= 0 || s->max_count_a < 0) {
        fail(DV_EINVAL, "%s: bad mha shape", fn); return 0;
      }
      break;
    case DV_OP_DECODE_LAYER:
      if (s->d <= 0 || s->F <= 0 || s->h <= 0 || s->dh <= 0 || s->n_ctx < 0 || s->r <= 0 ||
          s->max_count_m < 0 || s->max_count_a < 0) {
        fail(DV_EINVAL, "%s: bad layer shape", fn); return 0;
      }
      break;
    default:
      fail(DV_EINVAL, "%s: unknown op %d", fn, op);
      return 0;
  }
  // The layout depends on the weight dtype only through the column split of the
  // axpy tiles; report the larger of the two so one size serves both.
  return std::max(ws_bytes_for(op, s, DV_BF16), ws_bytes_for(op, s, DV_F32));
}

int dv_predict(const float* y, int batch, int d, const void* A, const void* Bm, int r, int N,
               dv_dtype wdt, float* scores, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dv_predict";
  t_slot = 0;
  CHECK_PTR(y); CHECK_PTR(A); CHECK_PTR(Bm); CHECK_PTR(scores);
  if (batch <= 0) return fail(DV_EINVAL, "%s: batch = %d", fn, batch);
  if (r <= 0 || N <= 0) return fail(DV_EINVAL, "%s: r = %d, N = %d", fn, r, N);
  if (wdt == DV_FP8)
    return fail(DV_EUNSUPPORTED, "%s: fp8 weights are taken by dv_decode_layer only", fn);
  if (!valid_dtype(wdt)) return fail(DV_EINVAL, "%s: bad dtype %d", fn, (int)wdt);
  if (int e = check_d(fn, d)) return e;
  CHECK_ALIGN(y); CHECK_ALIGN(A); CHECK_ALIGN(Bm); CHECK_ALIGN(scores);
  const PredictWs P = plan_predict(batch, d, r, N, wdt);
  if (int e = check_ws(fn, ws, ws_bytes, P.total)) return e;
  char* w = static_cast<char*>(ws);
  float* z = reinterpret_cast<float*>(w + P.z);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(w + P.tickets);
  const int bt = pick_bt(batch);

  PhaseArgs a1 = zero_args();
  add_rowdot(a1.rowdot, A, d, wdt, make_list(nullptr, nullptr, r, 1, r), z, r);
  finish_rowdot(a1.rowdot, y, batch, d, tickets, P.nt, w, P.rd);
  if (int e = launch_rowdot(T_ROWDOT, bt, a1, stream, fn)) return e;

  PhaseArgs a2 = zero_args();
  add_axpy(a2.axpy, batch, Bm, N, wdt, make_list(nullptr, nullptr, r, 1, r), z, r, 0, N,
           reinterpret_cast<float*>(w + P.partial), tickets, scores, N, nullptr, nullptr, 0, 0, default_axpy_blocks());
  a2.axpy.batch = batch;
  return launch(T_AXPY, bt, a2, a2.axpy.blocks, axpy_lds(bt), stream, fn);
}

int dv_select_topk(const float* scores, int batch, int N, int k, int union_rows, int32_t* idx,
                   int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dv_select_topk";
  t_slot = 0;
  CHECK_PTR(scores); CHECK_PTR(idx); CHECK_PTR(count);
  if (batch <= 0) return fail(DV_EINVAL, "%s: batch = %d", fn, batch);
  if (N <= 0) return fail(DV_EINVAL, "%s: N = %d", fn, N);
  if (k < 0 || k > N) return fail(DV_EINVAL, "%s: k = %d not in [0, N = %d]", fn, k, N);
  if (N > kMaxSegs * kSegElems)
    return fail(DV_EUNSUPPORTED, "%s: N = %d exceeds %d", fn, N, kMaxSegs * kSegElems);
  CHECK_ALIGN(scores); CHECK_ALIGN(idx); CHECK_ALIGN(count);
  const SelectWs P = plan_select(batch, N);
  if (int e = check_ws(fn, ws, ws_bytes, P.total)) return e;
  char* w = static_cast<char*>(ws);

  PhaseArgs z = zero_args();
  z.zero.ptr = reinterpret_cast<uint32_t*>(w + P.zero);
  z.zero.words = P.zero_words;
  z.zero.blocks = std::max(1, std::min(cdiv(P.zero_words, kThreads * 4), 64));
  if (int e = launch(T_ZERO, 1, z, z.zero.blocks, 0, stream, fn)) return e;

  PhaseArgs a = zero_args();
  a.topk.np = 1;
  a.topk.p[0] = make_topk(scores, N, N, k, batch, union_rows,
                          idx, count, reinterpret_cast<uint32_t*>(w + P.hist),
                          reinterpret_cast<uint32_t*>(w + P.rtick),
                          reinterpret_cast<uint32_t*>(w + P.ticket), w, P.t);
  a.topk.blocks = topk_seg_blocks(a.topk);
  if (int e = launch(T_HIST, 1, a, a.topk.blocks, hist_lds(), stream, fn)) return e;
  return launch(T_CLASSIFY, 1, a, a.topk.blocks, classify_lds(), stream, fn);
}

int dv_sparse_mlp(const float* y, int batch, int d, const void* W1t, const void* W2t, int F,
                  dv_dtype wdt, const int32_t* idx, const int32_t* count, int max_count, float* out,
                  int accumulate, int act, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dv_sparse_mlp";
  t_slot = 0;
  CHECK_PTR(y); CHECK_PTR(W1t); CHECK_PTR(W2t); CHECK_PTR(idx); CHECK_PTR(count); CHECK_PTR(out);
  if (batch <= 0) return fail(DV_EINVAL, "%s: batch = %d", fn, batch);
  if (F <= 0) return fail(DV_EINVAL, "%s: F = %d", fn, F);
  if (max_count < 0 || max_count > F) return fail(DV_EINVAL, "%s: max_count = %d not in [0, F]", fn, max_count);
  if (wdt == DV_FP8)
    return fail(DV_EUNSUPPORTED, "%s: fp8 weights are taken by dv_decode_layer only", fn);
  if (!valid_dtype(wdt)) return fail(DV_EINVAL, "%s: bad dtype %d", fn, (int)wdt);
  if (!valid_act(act)) return fail(DV_EINVAL, "%s: bad activation %d", fn, act);
  if (int e = check_d(fn, d)) return e;
  CHECK_ALIGN(y); CHECK_ALIGN(W1t); CHECK_ALIGN(W2t); CHECK_ALIGN(idx); CHECK_ALIGN(count);
  CHECK_ALIGN(out);
  if (out == y) return fail(DV_EINVAL, "%s: out must not alias y", fn);
  const MlpWs P = plan_mlp(batch, d, max_count, wdt);
  if (int e = check_ws(fn, ws, ws_bytes, P.total)) return e;
  char* w = static_cast<char*>(ws);
  const int cap = std::max(max_count, 1);
  float* hbuf = reinterpret_cast<float*>(w + P.a);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(w + P.tickets);
  const int bt = pick_bt(batch);
  const RowList L = make_list(idx, count, max_count, 1, F);

  PhaseArgs a1 = zero_args();
  add_rowdot(a1.rowdot, W1t, d, wdt, L, hbuf, cap);
  finish_rowdot(a1.rowdot, y, batch, d, tickets, P.nt, w, P.rd);
  if (int e = launch_rowdot(T_ROWDOT, bt, a1, stream, fn)) return e;

  PhaseArgs a2 = zero_args();
  add_axpy(a2.axpy, batch, W2t, d, wdt, L, hbuf, cap, act_code(act), d, reinterpret_cast<float*>(w + P.partial),
           tickets, out, d, nullptr, nullptr, 0, accumulate, default_axpy_blocks());
  a2.axpy.batch = batch;
  return launch(T_AXPY, bt, a2, a2.axpy.blocks, axpy_lds(bt), stream, fn);
}

int dv_sparse_mha(const float* y, int batch, int d, int h, int dh, const void* Wq, const void* Wo,
                  dv_dtype wdt, const void* K, const void* V, int n_ctx, dv_dtype kvdt,
                  const int32_t* heads, const int32_t* count, int max_count, float scale, float* out,
                  int accumulate, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dv_sparse_mha";
  t_slot = 0;
  CHECK_PTR(y); CHECK_PTR(Wq); CHECK_PTR(Wo); CHECK_PTR(K); CHECK_PTR(V); CHECK_PTR(heads);
  CHECK_PTR(count); CHECK_PTR(out);
  if (batch <= 0) return fail(DV_EINVAL, "%s: batch = %d", fn, batch);
  if (h <= 0) return fail(DV_EINVAL, "%s: h = %d", fn, h);
  if (int e = check_nctx(fn, n_ctx)) return e;
  if (max_count < 0 || max_count > h) return fail(DV_EINVAL, "%s: max_count = %d not in [0, h]", fn, max_count);
  if (wdt == DV_FP8)
    return fail(DV_EUNSUPPORTED, "%s: fp8 weights are taken by dv_decode_layer only", fn);
  if (!valid_dtype(wdt) || !valid_dtype(kvdt)) return fail(DV_EINVAL, "%s: bad dtype", fn);
  if (!(scale == scale)) return fail(DV_EINVAL, "%s: scale is NaN", fn);
  if (int e = check_d(fn, d)) return e;
  if (int e = check_dh(fn, dh)) return e;
  CHECK_ALIGN(y); CHECK_ALIGN(Wq); CHECK_ALIGN(Wo); CHECK_ALIGN(K); CHECK_ALIGN(V);
  CHECK_ALIGN(heads); CHECK_ALIGN(count); CHECK_ALIGN(out);
  if (out == y) return fail(DV_EINVAL, "%s: out must not alias y", fn);
  const MhaWs P = plan_mha(batch, d, dh, n_ctx, max_count, wdt);
  if (int e = check_ws(fn, ws, ws_bytes, P.total)) return e;
  char* w = static_cast<char*>(ws);
  const int cap = std::max(max_count, 1);
  float* q = reinterpret_cast<float*>(w + P.q);
  float* o = reinterpret_cast<float*>(w + P.o);
  float* part = reinterpret_cast<float*>(w + P.part);
  uint32_t* t_attn = reinterpret_cast<uint32_t*>(w + P.tickets);
  uint32_t* t_ax = t_attn + P.nt_attn;
  const int bt = pick_bt(batch);
  const RowList L = make_list(heads, count, max_count, dh, h);

  PhaseArgs a1 = zero_args();
  add_rowdot(a1.rowdot, Wq, d, wdt, L, q, cap * dh);
  finish_rowdot(a1.rowdot, y, batch, d, t_attn, P.nt_attn + P.nt_ax, w, P.rd);
  if (int e = launch_rowdot(T_ROWDOT, bt, a1, stream, fn)) return e;

  PhaseArgs a2 = zero_args();
  setup_attn(a2.attn, q, cap * dh, K, V, kvdt, batch, h, n_ctx, n_ctx, dh,
             make_list(heads, count, max_count, 1, h), scale, part, t_attn, o, cap * dh, 0);
  if (max_count > 0) {
    if (int e = launch(T_ATTN, 1, a2, a2.attn.blocks, attn_lds(), stream, fn)) return e;
  }

  PhaseArgs a3 = zero_args();
  add_axpy(a3.axpy, batch, Wo, d, wdt, L, o, cap * dh, 0, d, reinterpret_cast<float*>(w + P.partial),
           t_ax, out, d, nullptr, nullptr, 0, accumulate, default_axpy_blocks());
  a3.axpy.batch = batch;
  return launch(T_AXPY, bt, a3, a3.axpy.blocks, axpy_lds(bt), stream, fn);
}

}  // extern "C"

namespace {

// ------------------------------------------------------------------------- //
// allocation-free scratch                                                   //
// ------------------------------------------------------------------------- //

// The workspace of dv_decode_layer_noalloc: one copy of this array per device, held
// by the loaded library until the process ends.  In host code `scratch` is only a
// stand-in for the symbol; its device address comes from hipGetSymbolAddress, per
// device, and is the only form ever handed to a kernel.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's copy of `scratch` (looked up once per device, with
// that device current); nullptr on failure, with the error text set.
void* scratch_ptr(const char* fn) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    fail(DV_EHIP, "%s: no current HIP device", fn);
    return nullptr;
  }
  std::lock_guard<std::mutex> g(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      fail(DV_EHIP, "%s: scratch lookup failed: %s", fn, hipGetErrorString(e));
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

// dv_decode_layer's body.  use_scratch: the workspace is the library's scratch array
// (ws and ws_bytes are ignored; shapes whose workspace exceeds it are rejected).
int decode_layer_impl(const char* fn, const dv_layer* L, const dv_layer* nx, int batch,
                      const float* y_in, float* y_out, const int32_t* idx_m,
                      const int32_t* count_m, int max_count_m, const int32_t* idx_a,
                      const int32_t* count_a, int max_count_a, int32_t* next_idx_m,
                      int32_t* next_count_m, int32_t* next_idx_a, int32_t* next_count_a,
                      void* ws, size_t ws_bytes, bool use_scratch, void* stream) {
  t_slot = 0;
  CHECK_PTR(L); CHECK_PTR(y_in); CHECK_PTR(y_out);
  CHECK_PTR(idx_m); CHECK_PTR(count_m); CHECK_PTR(idx_a); CHECK_PTR(count_a);
  if (batch <= 0) return fail(DV_EINVAL, "%s: batch = %d", fn, batch);
  const int d = L->d, F = L->F, h = L->h, dh = L->dh, n = L->n_ctx;
  if (F <= 0 || h <= 0) return fail(DV_EINVAL, "%s: F = %d, h = %d", fn, F, h);
  // The full step with the KV append (W^K and W^V given): the current token's k and
  // v go to row n_ctx of every head's cache, and n_ctx + 1 rows are attended.
  const bool append = L->Wk != nullptr || L->Wv != nullptr;
  if (append) {
    CHECK_PTR(L->Wk); CHECK_PTR(L->Wv); CHECK_ALIGN(L->Wk); CHECK_ALIGN(L->Wv);
    if (n < 0) return fail(DV_EINVAL, "%s: n_ctx = %d", fn, n);
  }
  const int n_att = n + (append ? 1 : 0);
  if (int e = check_nctx(fn, n_att)) return e;
  if (L->kv_cap < 0) return fail(DV_EINVAL, "%s: kv_cap = %d", fn, L->kv_cap);
  const int kv_cap = L->kv_cap ? L->kv_cap : n;
  if (kv_cap < n_att)
    return fail(DV_EINVAL, "%s: kv_cap = %d rows cannot hold %d%s", fn, kv_cap, n_att,
                append ? " (the cached rows and the appended one)" : "");
  if (!(valid_dtype(L->wdt) || L->wdt == DV_FP8) || !valid_dtype(L->kvdt))
    return fail(DV_EINVAL, "%s: bad dtype", fn);
  if (!valid_act(L->act)) return fail(DV_EINVAL, "%s: bad activation %d", fn, L->act);
  if (L->wdt == DV_FP8) {
    CHECK_PTR(L->W1s); CHECK_PTR(L->W2s); CHECK_PTR(L->Wqs); CHECK_PTR(L->Wos);
    CHECK_ALIGN(L->W1s); CHECK_ALIGN(L->W2s); CHECK_ALIGN(L->Wqs); CHECK_ALIGN(L->Wos);
    if (append) { CHECK_PTR(L->Wks); CHECK_PTR(L->Wvs); CHECK_ALIGN(L->Wks); CHECK_ALIGN(L->Wvs); }
    if (L->d % 16 != 0) return fail(DV_EALIGN, "%s: fp8 rows need d %% 16 == 0 (d = %d)", fn, L->d);
  }
  if (!(L->scale == L->scale)) return fail(DV_EINVAL, "%s: scale is NaN", fn);
  if (int e = check_d(fn, d)) return e;
  if (int e = check_dh(fn, dh)) return e;
  if (max_count_m < 0 || max_count_m > F) return fail(DV_EINVAL, "%s: max_count_m = %d", fn, max_count_m);
  if (max_count_a < 0 || max_count_a > h) return fail(DV_EINVAL, "%s: max_count_a = %d", fn, max_count_a);
  CHECK_PTR(L->W1t); CHECK_PTR(L->W2t); CHECK_PTR(L->Wq); CHECK_PTR(L->Wo); CHECK_PTR(L->K);
  CHECK_PTR(L->V);
  CHECK_ALIGN(y_in); CHECK_ALIGN(y_out); CHECK_ALIGN(idx_m); CHECK_ALIGN(count_m);
  CHECK_ALIGN(idx_a); CHECK_ALIGN(count_a);
  CHECK_ALIGN(L->W1t); CHECK_ALIGN(L->W2t); CHECK_ALIGN(L->Wq); CHECK_ALIGN(L->Wo);
  CHECK_ALIGN(L->K); CHECK_ALIGN(L->V);
  int r = 1, Fn = 1, hn = 1, km = 0, ka = 0;
  if (nx) {
    CHECK_PTR(next_idx_m); CHECK_PTR(next_count_m); CHECK_PTR(next_idx_a); CHECK_PTR(next_count_a);
    CHECK_PTR(nx->A_M); CHECK_PTR(nx->B_M); CHECK_PTR(nx->A_A); CHECK_PTR(nx->B_A);
    CHECK_ALIGN(next_idx_m); CHECK_ALIGN(next_count_m); CHECK_ALIGN(next_idx_a);
    CHECK_ALIGN(next_count_a);
    CHECK_ALIGN(nx->A_M); CHECK_ALIGN(nx->B_M); CHECK_ALIGN(nx->A_A); CHECK_ALIGN(nx->B_A);
    if (nx->d != d) return fail(DV_EINVAL, "%s: next->d = %d differs from d = %d", fn, nx->d, d);
    if (!valid_dtype(nx->pwdt)) return fail(DV_EINVAL, "%s: bad predictor dtype %d", fn, (int)nx->pwdt);
    r = nx->r; Fn = nx->F; hn = nx->h; km = nx->k_m; ka = nx->k_a;
    if (r <= 0 || Fn <= 0 || hn <= 0) return fail(DV_EINVAL, "%s: next r/F/h", fn);
    if (km < 0 || km > Fn || ka < 0 || ka > hn)
      return fail(DV_EINVAL, "%s: next k_m = %d / k_a = %d out of range", fn, km, ka);
    if (Fn > kMaxSegs * kSegElems)
      return fail(DV_EUNSUPPORTED, "%s: next F = %d exceeds %d", fn, Fn, kMaxSegs * kSegElems);
  }
  const dv_dtype wdt = L->wdt;
  const dv_dtype pwdt = nx ? nx->pwdt : DV_BF16;   // the next layer's predictor factors
  const bool fp8 = wdt == DV_FP8;
  const LayerWs P = plan_layer(batch, d, std::max(F, Fn), std::max(h, hn), dh, n, r, max_count_m,
                               max_count_a, wdt, pwdt);
  if (use_scratch) {
    if (P.total > kScratchBytes)
      return fail(DV_EWORKSPACE, "%s: these shapes need %zu bytes of workspace, more than the "
                  "%zu of the library's scratch (use dv_decode_layer with a workspace)", fn,
                  P.total, kScratchBytes);
    ws = scratch_ptr(fn);
    if (!ws) return DV_EHIP;
    ws_bytes = kScratchBytes;
  }
  if (int e = check_ws(fn, ws, ws_bytes, P.total)) return e;

  char* w = static_cast<char*>(ws);
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
  auto up = [&](size_t off) { return reinterpret_cast<uint32_t*>(w + off); };
  const int cap_m = std::max(max_count_m, 1), cap_a = std::max(max_count_a, 1);
  uint32_t* t_attn = up(P.tickets);
  uint32_t* t_bm = t_attn + P.t_attn;
  uint32_t* t_ba = t_bm + P.t_bm;
  uint32_t* t_wo = t_ba + P.t_ba;
  const int bt = pick_bt(batch);
  const RowList LM = make_list(idx_m, count_m, max_count_m, 1, F);
  const RowList LQ = make_list(idx_a, count_a, max_count_a, dh, h);
  const RowList LH = make_list(idx_a, count_a, max_count_a, 1, h);

  // Without a next layer, one token and bf16 rows: the whole step is one launch whose
  // resident blocks work through one ordered queue (row dots, attention, row sums; see
  // StreamTask), so no launch boundary, prologue or block-end spread sits between its
  // parts.
  const int path = g_step_path.load() == DV_PATH_AUTO ? kAutoStepPath : g_step_path.load();
  if (path == DV_PATH_ONE_LAUNCH && !nx && batch == 1 && wdt == DV_BF16 && !append) {
    const StreamGeo G = stream_geo(d, dh, n_att, max_count_m, max_count_a);
    StreamTask t;
    memset(&t, 0, sizeof t);
    t.W1 = L->W1t; t.W2 = L->W2t; t.Wq = L->Wq; t.Wo = L->Wo;
    t.LM = LM; t.LQ = LQ;
    t.d = d; t.dh = dh; t.act = act_code(L->act);
    t.y = y_in; t.y_out = y_out;
    t.a = fp(P.a); t.q = fp(P.q); t.partial = fp(P.s_partial);
    t.ctr = up(P.s_ctr);
    setup_attn(t.at, fp(P.q), cap_a * dh, L->K, L->V, L->kvdt, 1, h, n_att, kv_cap, dh, LH,
               L->scale, fp(P.part), up(P.s_atick), fp(P.o), cap_a * dh, 1);
    assert(t.at.nsplit == G.nsplit);
    t.c_qdone = G.c_qdone; t.c_mdone = G.c_mdone; t.c_oready = G.c_oready; t.c_stick = G.c_stick;
    t.n_qi = G.n_qi; t.n_mi = G.n_mi; t.n_a = G.n_a;
    t.ncm = G.ncm; t.per_m = G.per_m; t.nslice = G.nslice; t.n_items = G.n_items;
    t.spins = g_wait_spins.load(); t.extra = g_wait_extra.load();
    t.fault = fault_word();
    // LDS: y for the dot items, shared with the row-sum and attention scratch; 64 bytes
    // of block words after it
    t.lds_union = (int)align256((size_t)std::max({d * 4, (2 * kAxpyTileRows +
                                                            kAxGroups * kStreamSlice) * 4,
                                                   attn_lds()}));
    const int lds = t.lds_union + 64;
    const int kvc = L->kvdt == DV_BF16 ? W_BF16 : W_F32;
    const int per_cu = stream_occupancy(kvc, lds);
    t.grid = (per_cu * device_cus()) / 64 * 64;
    // the first round of items (one per block) all dots, plus a quarter round more, so
    // that the heads' W^Q rows are dotted when the attention items are taken
    t.n_mfirst = std::max(0, std::min(G.n_mi, t.grid + t.grid / 4 - G.n_qi));
    if (t.grid >= 64 && t.fault) {
      // y_out is y: the blocks stage y from a copy, so that no block reads an element of y
      // another block has already overwritten
      if (y_in == y_out) {
        float* yc = fp(P.s_y);
        const hipError_t e = hipMemcpyAsync(yc, y_in, (size_t)d * 4, hipMemcpyDeviceToDevice,
                                            static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(DV_EHIP, "%s: copy of y failed: %s", fn, hipGetErrorString(e));
        t.y = yc;
      }
      // the counters start at zero: a small launch clears them
      PhaseArgs z = zero_args();
      z.zero.ptr = up(P.s_ctr);
      z.zero.words = P.s_zero_words;
      z.zero.blocks = std::max(1, std::min(cdiv(P.s_zero_words, kThreads * 4), 64));
      int err = launch_phase(T_ZERO, 1, z, z.zero.blocks, 0, stream);
      if (err == 0) {
        const SlotEvents ev = slot_events();
        err = launch_stream(kvc, t, t.grid, lds, stream, ev.a, ev.b);
      }
      if (err != 0)
        return fail(DV_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString((hipError_t)err));
      return DV_OK;
    }
  }

  // Phase 1: every gathered row dotted with y_in (W1 rows of S_M, W^Q columns of
  // S_A, and the next layer's predictor factors A_M, A_A); clears the counters and
  // histograms the later phases use.
  PhaseArgs a1 = zero_args();
  add_rowdot(a1.rowdot, L->W1t, d, wdt, LM, fp(P.a), cap_m, fp8 ? L->W1s : nullptr);
  add_rowdot(a1.rowdot, L->Wq, d, wdt, LQ, fp(P.q), cap_a * dh, fp8 ? L->Wqs : nullptr);
  if (nx) {
    add_rowdot(a1.rowdot, nx->A_M, d, pwdt, make_list(nullptr, nullptr, r, 1, r), fp(P.zm), r);
    add_rowdot(a1.rowdot, nx->A_A, d, pwdt, make_list(nullptr, nullptr, r, 1, r), fp(P.za), r);
  }
  if (append) {   // every head's k and v, stored at row n of its cache
    const RowList LK = make_list(nullptr, nullptr, h, dh, h);
    const size_t row_n = (size_t)n * dh * esize(L->kvdt);
    add_rowdot(a1.rowdot, L->Wk, d, wdt, LK, nullptr, 0, fp8 ? L->Wks : nullptr,
               static_cast<char*>(L->K) + row_n);
    add_rowdot(a1.rowdot, L->Wv, d, wdt, LK, nullptr, 0, fp8 ? L->Wvs : nullptr,
               static_cast<char*>(L->V) + row_n);
    a1.rowdot.store_ld_b = (long long)h * kv_cap * dh;
    a1.rowdot.store_ld_item = (long long)kv_cap * dh;
    a1.rowdot.store_dt = L->kvdt == DV_BF16 ? W_BF16 : W_F32;
  }
  finish_rowdot(a1.rowdot, y_in, batch, d, up(P.zero), P.zero_words, w, P.rd);
  if (int e = launch_rowdot(T_ROWDOT | (fp8 ? T_FP8 : 0) | (append ? T_KV : 0), bt, a1, stream, fn))
    return e;

  // After the row dots, the rest of the layer: attention over the cache for S_A; one
  // row sum y_out = y_in + sum_{S_M} ReLU(a) W2 rows + sum_{S_A} o W^O rows; and for
  // the next layer its predictor scores (with top-digit histograms) and top-k.
  // (mfma_min_batch 2: the look-ahead step's output row sum, which shares its launch with
  // the top-k only, runs on the matrix cores from 2 tokens: measured at batch 2 82 us
  // against 96 for the wave path; the sparse step without a next layer keeps the wave
  // path there, for its single waiting launch)
  auto add_out = [&](AxpyTask& T, int target, int mfma_min_batch = kAxMfmaMinBatch) {
    add_axpy2(T, batch, L->W2t, d, wdt, LM, fp(P.a), cap_m, act_code(L->act), L->Wo, LQ, fp(P.o),
              cap_a * dh, A_NONE,
              d, fp(P.p_wo), t_wo, y_out, d, y_in, nullptr, d, 0, target,
              fp8 ? L->W2s : nullptr, fp8 ? L->Wos : nullptr, mfma_min_batch);
  };

  // Without a next layer, one launch when its blocks fit one resident round: every
  // row-sum block streams its W2 rows, then takes its W^O rows one head slot at a
  // time: it waits until that slot's o is stored (attention blocks come first in block
  // order; the last key split of each head combines the splits into o and raises the
  // slot's counter) and stages o as the coefficients.  The attention, its combine
  // included, hides under the W2 stream, and a head that finishes late holds back only
  // the blocks whose W^O rows belong to it.  (Combining the splits in each row-sum block
  // instead, as it stages its W^O coefficients, measured 48.3 us against 46.1.)
  // (fp8 rows take it too: with the W^O rows on chunks of their own, no block's chain
  // holds both sources)
  // (Row sums on the matrix cores do not wait inside a launch: batches of tokens
  // over bf16 rows take the two launches below.)
  if (!nx && max_count_a > 0 && ax_geo(batch, d, d, wdt, 1).mfma_nt == 0) {
    PhaseArgs f = zero_args();
    setup_attn(f.attn, fp(P.q), cap_a * dh, L->K, L->V, L->kvdt, batch, h, n_att, kv_cap, dh, LH,
               L->scale,
               fp(P.part), t_attn, fp(P.o), cap_a * dh, 1);
    f.attn.done_ctr = up(P.done);
    f.b_attn = 0;
    f.b_axpy = f.attn.blocks;
    const int wflags = T_ATTN | T_AXPY | T_WAIT | (fp8 ? T_FP8 : 0);
    const int lds = std::max(axpy_lds(bt, fp8 ? 16 : 8), attn_lds());
    const int fit = std::min(resident_blocks(), phase_occupancy(wflags, bt, lds) * device_cus());
    // The grid holds every attention block first; with fewer than two row-sum blocks
    // per CU left beside them, the separate launches below are faster (OPT-175B batch
    // 2: 566 against 180 us per layer).
    const bool room = fit - f.attn.blocks >= 2 * device_cus();
    add_out(f.axpy, std::max(1, fit - f.attn.blocks));
    AxpySeg& S = f.axpy.seg[0];
    S.wait_ctr = up(P.done);
    S.wait_target = (uint32_t)batch + g_wait_extra.load();   // each token's o of the slot
    // When every row-sum block's two shares fit one tile (bf16 rows), the key splits
    // only store their softmax pieces and each block combines the pieces of its heads
    // as it stages its W^O coefficients: a head is ready when its last split is, with
    // no combining round trips after it.
    // The W^O rows also get row chunks of their own (about their share of the row
    // bytes), after the W2 chunks in block order: the W2 blocks are dispatched first and
    // stream at once, the W^O blocks start as the heads complete.
    {
      const int nch = S.nchunks;
      const int c2 = nch >= 2 ? std::max(1, std::min(nch - 1, (int)std::lround(nch * kWoChunkShare)))
                              : 0;
      const int per1 = cdiv(std::max(cap_m, 1), nch - c2);
      const int per2 = cdiv(cap_a * dh, c2 > 0 ? c2 : nch);
      const int tile = c2 > 0 ? std::max(per1, per2) : per1 + per2;
      const int ns_max = cdiv(per2 + dh - 1, dh) + 1;       // slots one share can touch
      const int red_floats = kAxGroups * bt * kAxSliceLanes * S.vec;
      f.axpy.c2 = c2;
      if (f.attn.nsplit > 1 && wdt == DV_BF16 && S.vec == 8 && tile <= kAxpyTileRows &&
          ns_max <= kThreads && 64 + 2 * bt * ns_max * f.attn.nsplit <= red_floats) {
        f.attn.part_only = 1;
        f.axpy.part2 = fp(P.part);
        f.axpy.nsplit2 = f.attn.nsplit;
        S.wait_target = (uint32_t)(batch * f.attn.nsplit) + g_wait_extra.load();
      }
    }
    f.axpy.spins = g_wait_spins.load();
    f.axpy.fault = fault_word();
    f.axpy.batch = batch;
    const int grid = f.attn.blocks + f.axpy.blocks;
    if (room && grid <= fit && f.axpy.fault) return launch(wflags, bt, f, grid, lds, stream, fn);
  }

  // Otherwise two launches: the attention (its last split of each head combines the
  // pieces into o) beside the next layer's predictor scores; then the row sum beside
  // the next layer's top-k, whose last classify block of each row resolves it.  When
  // the predictor's row sums run on the matrix cores (a batch of tokens), the attention
  // gets a launch of its own first: sharing a kernel with them would hold its
  // latency-bound blocks to their register budget (measured at batch 16: 437 us for the
  // shared launch against 283 us for the attention alone).
  const bool attn_alone = nx && max_count_a > 0 && ax_geo(batch, Fn, Fn, pwdt, r).mfma_nt > 0;
  if (attn_alone) {
    PhaseArgs at = zero_args();
    setup_attn(at.attn, fp(P.q), cap_a * dh, L->K, L->V, L->kvdt, batch, h, n_att, kv_cap, dh, LH,
               L->scale, fp(P.part), t_attn, fp(P.o), cap_a * dh, 0);
    if (int e = launch(T_ATTN, 1, at, at.attn.blocks, attn_lds(), stream, fn)) return e;
  }
  PhaseArgs a2 = zero_args();
  if (max_count_a > 0 && !attn_alone)
    setup_attn(a2.attn, fp(P.q), cap_a * dh, L->K, L->V, L->kvdt, batch, h, n_att, kv_cap, dh, LH,
               L->scale,
               fp(P.part), t_attn, fp(P.o), cap_a * dh, nx ? 1 : 0);
  a2.b_attn = 0;
  a2.b_axpy = a2.attn.blocks;
  if (nx) {
    // B_M's row sum fills the resident round beside the attention (measured 31.0 us for
    // the launch against 31.5 with six blocks per CU and 33.9 with four); on the
    // matrix-core path, alone in its launch, few long blocks (at OPT-175B one chunk of
    // all 1000 rows per 128-column slice, no partials): measured at batch 4 / 16 / 32
    // 30 / 39 / 57 us against 35 / 41 / 67 with two chunks and 40 / 48 / 84 with five
    const int bm_blocks = attn_alone ? 2 * device_cus()
                                     : std::max(default_axpy_blocks(), resident_blocks() - a2.attn.blocks - 48);
    // The blocks that finish the scores also build their top-digit histograms, except on
    // the matrix-core path: there a block finishes 16 tokens' scores, one LDS histogram
    // pass each, so the histograms get a launch of their own below.
    add_axpy(a2.axpy, batch, nx->B_M, Fn, pwdt, make_list(nullptr, nullptr, r, 1, r), fp(P.zm), r,
             0, Fn, fp(P.p_bm), t_bm, fp(P.sm), Fn, nullptr, nullptr, 0, 0, bm_blocks);
    a2.axpy.seg[a2.axpy.nseg - 1].hist = attn_alone ? nullptr : up(P.hist_m);
    add_axpy(a2.axpy, batch, nx->B_A, hn, pwdt, make_list(nullptr, nullptr, r, 1, r), fp(P.za), r,
             0, hn, fp(P.p_ba), t_ba, fp(P.sa), hn, nullptr, nullptr, 0, 0, default_axpy_blocks());
    a2.axpy.seg[a2.axpy.nseg - 1].hist = attn_alone ? nullptr : up(P.hist_a);
  }
  a2.axpy.batch = batch;
  a2.axpy.skew = kSkewWave;
  const int flags2 = (a2.attn.blocks ? T_ATTN : 0) | (a2.axpy.nseg ? T_AXPY : 0);
  if (flags2) {
    const int lds2 = std::max((flags2 & T_AXPY) ? axpy_lds(bt) : 0, a2.attn.blocks ? attn_lds() : 0);
    if (int e = launch(flags2, flags2 == T_ATTN ? 1 : bt, a2, a2.attn.blocks + a2.axpy.blocks, lds2,
                       stream, fn))
      return e;
  }
  PhaseArgs a3 = zero_args();
  add_out(a3.axpy, default_axpy_blocks(), nx ? 2 : kAxMfmaMinBatch);
  a3.axpy.batch = batch;
  // chunk shares weighted toward the blocks dispatched first (measured at OPT-175B:
  // look-ahead layer 112.5 -> 109.0 us at batch 1, 969 -> 955 at 16, 1528 -> 1496 at
  // 32; the matrix-core row sum alone, without the top-k blocks, measured slower, so
  // it keeps equal shares)
  a3.axpy.skew = a3.axpy.seg[0].mfma_nt > 0 ? (nx ? kSkewMfma : 0) : kSkewWave;
  int flags3 = T_AXPY | (fp8 ? T_FP8 : 0);
  if (nx) {
    TopkTask& tk = a3.topk;
    tk.np = 2;
    tk.p[0] = make_topk(fp(P.sm), Fn, Fn, km, batch, 1, next_idx_m, next_count_m, up(P.hist_m),
                        up(P.rtick_m), up(P.uticket), w, P.tm);
    tk.p[1] = make_topk(fp(P.sa), hn, hn, ka, batch, 1, next_idx_a, next_count_a, up(P.hist_a),
                        up(P.rtick_a), up(P.uticket) + 1, w, P.ta);
    tk.blocks = topk_seg_blocks(tk);
    flags3 |= T_CLASSIFY;
    a3.b_topk = 0;
    a3.b_axpy = tk.blocks;
  }
  if (nx && attn_alone) {   // the score histograms, a launch of their own (see above)
    PhaseArgs hs = zero_args();
    hs.topk = a3.topk;
    if (int e = launch(T_HIST, 1, hs, hs.topk.blocks, hist_lds(), stream, fn)) return e;
  }
  const int lds3 = std::max(axpy_lds(bt, fp8 ? 16 : 8), nx ? classify_lds() : 0);
  if (int e = launch(flags3, bt, a3, a3.topk.blocks + a3.axpy.blocks, lds3, stream, fn)) return e;
  return DV_OK;
}

}  // namespace

extern "C" {

int dv_decode_layer(const dv_layer* L, const dv_layer* nx, int batch, const float* y_in, float* y_out,
                    const int32_t* idx_m, const int32_t* count_m, int max_count_m,
                    const int32_t* idx_a, const int32_t* count_a, int max_count_a,
                    int32_t* next_idx_m, int32_t* next_count_m, int32_t* next_idx_a,
                    int32_t* next_count_a, void* ws, size_t ws_bytes, void* stream) {
  return decode_layer_impl("dv_decode_layer", L, nx, batch, y_in, y_out, idx_m, count_m,
                           max_count_m, idx_a, count_a, max_count_a, next_idx_m, next_count_m,
                           next_idx_a, next_count_a, ws, ws_bytes, false, stream);
}

int dv_decode_layer_noalloc(const dv_layer* L, const dv_layer* nx, int batch, const float* y_in,
                            float* y_out, const int32_t* idx_m, const int32_t* count_m,
                            int max_count_m, const int32_t* idx_a, const int32_t* count_a,
                            int max_count_a, int32_t* next_idx_m, int32_t* next_count_m,
                            int32_t* next_idx_a, int32_t* next_count_a, void* stream) {
  return decode_layer_impl("dv_decode_layer_noalloc", L, nx, batch, y_in, y_out, idx_m, count_m,
                           max_count_m, idx_a, count_a, max_count_a, next_idx_m, next_count_m,
                           next_idx_a, next_count_a, nullptr, 0, true, stream);
}

size_t dv_noalloc_scratch_bytes(void) { return kScratchBytes; }

int dv_check(void* stream) {
  const char* fn = "dv_check";
  uint32_t v = 0;
  const int e = fault_take(stream, &v);
  if (e != 0) return fail(DV_EHIP, "%s: %s", fn, hipGetErrorString((hipError_t)e));
  if (v) return fail(DV_ETIMEOUT, "%s: a wait inside an earlier launch on this device gave up "
                     "(its blocks were not all resident, or its producers never arrived); "
                     "the outputs that depended on it were written as NaN", fn);
  return DV_OK;
}

int dv_set_step_path(int path) {
  if (path != DV_PATH_AUTO && path != DV_PATH_TWO_LAUNCH && path != DV_PATH_ONE_LAUNCH)
    return fail(DV_EINVAL, "dv_set_step_path: unknown path %d", path);
  g_step_path.store(path);
  return DV_OK;
}

int dv_debug_wait_limits(unsigned spins, unsigned extra) {
  g_wait_spins.store(spins ? spins : kDefaultSpins);
  g_wait_extra.store(extra);
  return DV_OK;
}

int dv_timing_enable(int on) {
  TimingState& T = timing();
  std::lock_guard<std::mutex> g(T.mu);
  if (on && T.pool.empty()) {
    T.pool.resize(2 * kTimingPairs);
    for (auto& e : T.pool) {
      if (hipEventCreate(&e) != hipSuccess) {
        T.pool.clear();
        return fail(DV_EHIP, "dv_timing_enable: hipEventCreate failed");
      }
    }
  }
  T.on = on != 0;
  return DV_OK;
}

int dv_timing_read(float* ms_sum, int* launches, int max_slots, int* n_slots) {
  const char* fn = "dv_timing_read";
  CHECK_PTR(ms_sum); CHECK_PTR(launches); CHECK_PTR(n_slots);
  TimingState& T = timing();
  std::lock_guard<std::mutex> g(T.mu);
  for (int i = 0; i < max_slots; ++i) { ms_sum[i] = 0.f; launches[i] = 0; }
  int filled = 0;
  for (const auto& r : T.recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(DV_EHIP, "%s: event sync failed", fn);
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(DV_EHIP, "%s: elapsed failed", fn);
    if (r.slot < max_slots) {
      ms_sum[r.slot] += ms;
      launches[r.slot] += 1;
      filled = std::max(filled, r.slot + 1);
    }
  }
  T.recs.clear();
  T.used = 0;
  *n_slots = filled;
  return DV_OK;
}

}  // extern "C"
