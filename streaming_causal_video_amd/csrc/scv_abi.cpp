// C ABI of the streaming chunk-attention library: argument validation, the
// cache layout, per-cache constants and kernel launches.  Every entry point
// validates before enqueueing anything and never lets an exception escape.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "scv_internal.h"

struct scv_cache {
  scv::Geometry g;
  scv::Omegas om;
  scv_cache_layout lay;
  char* base;
  // Time position of frame g of stream b is g - pos_off[b]; RoPE refreshes
  // move it forward, cache_init resets it.  Host state, updated in call
  // order (a cache is used by one stream at a time).
  int64_t pos_off[scv::kMaxBatch];
};

namespace {

thread_local std::string g_last_error;

scv_status fail(scv_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates a config and derives geometry + layout.  Returns SCV_OK or an
// error status with the reason in `why`.
scv_status derive(const scv_config* c, scv::Geometry* g, scv_cache_layout* L, std::string* why) {
  if (!c) {
    *why = "config is NULL";
    return SCV_E_INVALID;
  }
  if (c->dtype != SCV_FP32 && c->dtype != SCV_BF16) {
    *why = "dtype must be SCV_FP32 or SCV_BF16";
    return SCV_E_DTYPE;
  }
  const int qk = c->qk_dtype == 0 ? c->dtype : c->qk_dtype;
  if (!(qk == c->dtype || (qk == SCV_FP16 && c->dtype == SCV_BF16))) {
    *why = "qk_dtype must be 0, equal to dtype, or SCV_FP16 with dtype SCV_BF16";
    return SCV_E_DTYPE;
  }
  if (c->head_dim != 64 && c->head_dim != 128) {
    *why = "head_dim must be 64 or 128";
    return SCV_E_DTYPE;
  }
  if (c->batch < 1 || c->batch > scv::kMaxBatch) {
    *why = "batch must be in [1, 64]";
    return SCV_E_INVALID;
  }
  if (c->heads < 1 || c->heads > 65535) {
    *why = "heads must be in [1, 65535]";
    return SCV_E_INVALID;
  }
  const int dt = c->rope_split[0], dh = c->rope_split[1], dw = c->rope_split[2];
  if (dt < 2 || dh < 2 || dw < 2 || (dt | dh | dw) & 1 || dt + dh + dw != c->head_dim) {
    *why = "rope_split must be three even values >= 2 summing to head_dim";
    return SCV_E_INVALID;
  }
  if (!(c->rope_base > 1.0) || !std::isfinite(c->rope_base)) {
    *why = "rope_base must be finite and > 1";
    return SCV_E_INVALID;
  }
  if (c->grid_h < 1 || c->grid_w < 1 || int64_t(c->grid_h) * c->grid_w > (int64_t(1) << 20)) {
    *why = "grid_h, grid_w must be >= 1 with grid_h*grid_w <= 2^20";
    return SCV_E_INVALID;
  }
  if (c->sink_frames < 0 || c->window_frames < 0 || c->chunk_frames < 1 || c->max_query_chunks < 1 ||
      c->max_query_chunks > scv::kMaxQueryChunks) {
    *why = "need sink_frames >= 0, window_frames >= 0, chunk_frames >= 1, 1 <= max_query_chunks <= 8";
    return SCV_E_INVALID;
  }
  const int64_t R = int64_t(c->window_frames) + int64_t(c->max_query_chunks) * c->chunk_frames;
  const int64_t n_slots = c->sink_frames + R;
  if (n_slots > scv::kMaxSlots) {
    *why = "sink_frames + window_frames + max_query_chunks*chunk_frames must be <= 64";
    return SCV_E_INVALID;
  }
  const int64_t P = int64_t(c->grid_h) * c->grid_w;
  if (P * c->chunk_frames * c->max_query_chunks >= (int64_t(1) << 31)) {
    *why = "query rows per call must stay below 2^31";
    return SCV_E_SHAPE;
  }
  g->B = c->batch;
  g->H = c->heads;
  g->D = c->head_dim;
  g->dt = dt;
  g->dh = dh;
  g->dw = dw;
  g->grid_h = c->grid_h;
  g->grid_w = c->grid_w;
  g->P = int32_t(P);
  g->S_f = c->sink_frames;
  g->W = c->window_frames;
  g->C = c->chunk_frames;
  g->k_max = c->max_query_chunks;
  g->R = int32_t(R);
  g->n_slots = int32_t(n_slots);
  g->slot_rows = int64_t(align_up(size_t(P), 8));
  g->rows = n_slots * g->slot_rows;
  g->rows_pad = int64_t(align_up(size_t(g->rows), scv::kKeyTile));
  g->dtype = c->dtype;
  g->qk_dtype = qk;
  g->elem_bytes = c->dtype == SCV_BF16 ? 2 : 4;
  g->base = c->rope_base;

  std::memset(L, 0, sizeof(*L));
  size_t off = 0;
  L->stamps_offset = off;
  off = align_up(off + size_t(g->B) * n_slots * 8, 256);
  L->table_h_offset = off;
  off = align_up(off + size_t(g->grid_h) * (dh / 2) * 8, 256);
  L->table_w_offset = off;
  off = align_up(off + size_t(g->grid_w) * (dw / 2) * 8, 256);
  const size_t kv = size_t(g->B) * g->H * size_t(g->rows_pad) * g->D * g->elem_bytes;
  L->k_offset = off;
  off = align_up(off + kv, 256);
  L->v_offset = off;
  off = align_up(off + kv, 256);
  L->total_bytes = off;
  L->n_slots = n_slots;
  L->ring_frames = R;
  L->slot_rows = g->slot_rows;
  L->rows = g->rows;
  L->rows_pad = g->rows_pad;
  L->elem_bytes = g->elem_bytes;
  return SCV_OK;
}

scv_status check_cache(const scv_cache* c) {
  if (!c) return fail(SCV_E_INVALID, "cache handle is NULL");
  return SCV_OK;
}

scv_status check_times(const scv_cache* c, const int64_t* t0, int32_t n_frames) {
  if (!t0) return fail(SCV_E_INVALID, "t0 is NULL");
  for (int b = 0; b < c->g.B; ++b) {
    if (t0[b] < 0 || t0[b] > scv::kMaxTime - n_frames)
      return fail(SCV_E_RANGE, "t0[" + std::to_string(b) + "] = " + std::to_string(t0[b]) +
                                   " puts a frame outside [0, 2^40)");
  }
  return SCV_OK;
}

// Time positions t0[b] - pos_off[b] .. + n_frames - 1 must stay in [0, 2^40).
scv_status check_positions(const scv_cache* c, const int64_t* t0, int32_t n_frames) {
  for (int b = 0; b < c->g.B; ++b) {
    const int64_t p = t0[b] - c->pos_off[b];
    if (p < 0 || p > scv::kMaxTime - n_frames)
      return fail(SCV_E_RANGE, "stream " + std::to_string(b) + ": frame " + std::to_string(t0[b]) +
                                   " has time position " + std::to_string(p) + " after RoPE refreshes of " +
                                   std::to_string(c->pos_off[b]) + " frames; positions must lie in [0, 2^40)");
  }
  return SCV_OK;
}

scv_status check_ptr(const void* p, const char* name, bool required) {
  if (!p) {
    if (required) return fail(SCV_E_INVALID, std::string(name) + " is NULL");
    return SCV_OK;
  }
  if (!aligned16(p)) return fail(SCV_E_ALIGN, std::string(name) + " is not 16-byte aligned");
  return SCV_OK;
}

scv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SCV_OK;
  return fail(SCV_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Ring frames among t0[b] .. t0[b]+n-1 (frames >= S_f) must fit in the ring.
scv_status check_append_frames(const scv_cache* c, const int64_t* t0, int32_t n_frames) {
  if (n_frames < 1) return fail(SCV_E_SHAPE, "n_frames must be >= 1");
  for (int b = 0; b < c->g.B; ++b) {
    const int64_t lo = t0[b], hi = t0[b] + n_frames;  // [lo, hi)
    const int64_t sink_part = std::max<int64_t>(0, std::min<int64_t>(hi, c->g.S_f) - lo);
    if (n_frames - sink_part > c->g.R)
      return fail(SCV_E_SHAPE, "an append may place at most R = " + std::to_string(c->g.R) + " frames in the ring");
  }
  if (int64_t(n_frames) * c->g.P >= (int64_t(1) << 31)) return fail(SCV_E_SHAPE, "n_frames * P must be < 2^31");
  return SCV_OK;
}

scv::RopeArgs base_rope_args(const scv_cache* c, const int64_t* t0, int32_t n_frames) {
  scv::RopeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.g = c->g;
  a.n_frames = n_frames;
  for (int b = 0; b < c->g.B; ++b) {
    a.t0[b] = t0[b];
    a.pos_off[b] = c->pos_off[b];
  }
  for (int j = 0; j < c->g.dt / 2; ++j) a.omega_t[j] = c->om.t[j];
  a.tab_h = reinterpret_cast<const float2*>(c->base + c->lay.table_h_offset);
  a.tab_w = reinterpret_cast<const float2*>(c->base + c->lay.table_w_offset);
  return a;
}

void set_cache_targets(const scv_cache* c, scv::RopeArgs* a) {
  a->cache_k = c->base + c->lay.k_offset;
  a->cache_v = c->base + c->lay.v_offset;
  a->stamps = reinterpret_cast<int64_t*>(c->base + c->lay.stamps_offset);
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

size_t workspace_bytes(const scv_cache* c, int32_t n_frames, int splits);

// Frames a query chunk starting at frame s_c can see once its history is in
// the cache: the sink frames before its end, and the window + chunk frames.
int64_t seen_frames(const scv_cache* c, int64_t s_c) {
  const int64_t end = s_c + c->g.C;
  const int64_t sink = std::min<int64_t>(c->g.S_f, std::max<int64_t>(end, 0));
  const int64_t lo = std::max<int64_t>(c->g.S_f, s_c - c->g.W);
  return std::min<int64_t>(c->g.n_slots, sink + std::max<int64_t>(0, end - lo));
}

// Key tiles a query chunk starting at frame s_c visits when the cache holds
// every frame the sink and window rules keep for it: the tiles holding a key
// of a visible slot (at least 1, so that every item of the balanced
// schedule owns a unit and gets its output written).
int visited_tiles(const scv_cache* c, int64_t s_c) {
  const scv::Geometry& g = c->g;
  const int64_t end = s_c + g.C;
  uint64_t mask = 0;
  for (int j = 0; j < g.S_f && j < end; ++j) mask |= uint64_t(1) << j;
  const int64_t lo = std::max<int64_t>(std::max<int64_t>(g.S_f, s_c - g.W), std::max<int64_t>(0, end - g.R));
  for (int64_t f = lo; f < end; ++f) mask |= uint64_t(1) << (g.S_f + int(f % g.R));
  const int64_t tiles = g.rows_pad / scv::kKeyTile;
  int64_t count = 0, prev_hi = -1;
  for (int s = 0; s < g.n_slots;) {
    if (!((mask >> s) & 1)) {
      ++s;
      continue;
    }
    int s1 = s;
    while (s1 < g.n_slots && ((mask >> s1) & 1)) ++s1;
    const int64_t r_lo = int64_t(s) * g.slot_rows, r_hi = int64_t(s1 - 1) * g.slot_rows + g.P;
    int64_t t_lo = r_lo / scv::kKeyTile;
    const int64_t t_hi = std::min<int64_t>((r_hi - 1) / scv::kKeyTile, tiles - 1);
    if (t_lo <= prev_hi) t_lo = prev_hi + 1;  // a tile shared by two runs counts once
    if (t_hi >= t_lo) count += t_hi - t_lo + 1;
    prev_hi = std::max(prev_hi, t_hi);
    s = s1;
  }
  return int(std::max<int64_t>(1, count));
}

// The balanced schedule needs the bf16 kernel and unit counts that fit int16.
bool lean_possible(const scv_cache* c) {
  return c->g.dtype == SCV_BF16 && c->g.rows_pad / scv::kKeyTile <= 32767;
}

size_t lean_workspace_bytes(const scv_cache* c, int ctas) {
  const size_t rows = size_t(ctas) * 2 * scv::kAttnRowsBf16;
  return align_up(rows * c->g.D * 4, 256) + align_up(rows * 4, 256);
}

// Units per item of each (stream, chunk) class, class id ch + n_chunks * b:
// visited key tiles from t0, or the steady state for every stream without.
void class_units(const scv_cache* c, const int64_t* t0, int32_t n_frames, int16_t* out) {
  const int nch = (n_frames + c->g.C - 1) / c->g.C;
  const int steady = visited_tiles(c, int64_t(c->g.S_f) + c->g.W + c->g.R);
  for (int b = 0; b < c->g.B; ++b)
    for (int ch = 0; ch < nch; ++ch)
      out[ch + nch * b] = int16_t(t0 ? visited_tiles(c, t0[b] + int64_t(ch) * c->g.C) : steady);
}

// The balanced schedule's work: total units and workgroup count.  The
// workgroups are a multiple k of the compute units (so that equal ranges
// fill whole rounds), with k the smallest that keeps every range no longer
// than the shortest item: a range then touches at most two items, which is
// all the kernel handles.  With rounds (kv_splits = -2), when every item
// has the same length and there are more items than compute units, the
// first F whole rounds of items run instead as whole-item ranges (no
// partials; the compute units of an XCD walk consecutive query tiles of a
// head side by side and share its K/V in L2) and only the items left over
// are cut into equal ranges: on the 720p layer 3.1x instead of 10.7x the
// algorithmic HBM bytes, and the same time within the spread between
// boxes (A/B on four boxes: -1.9% to +1.8%, +0.1% on average).  The
// automatic choice takes whichever cut the model finds cheaper (rounds
// write fewer partials).
constexpr int64_t kMaxLeanRounds = 16;
constexpr double kSegmentCost = 7.0;  // fixed cost of a segment, in tile-times (Q loads, pipeline fill, drain)
struct LeanPlan {
  int64_t units;
  int ctas;
  int v0 = 0;       // whole-item ranges (0: every range is cut equally)
  int64_t u0 = 0;   // units of those items
  int round = 0;    // workgroups per round of whole-item ranges
  double cost = 0;  // modeled time in tile-times, without the merge
};
LeanPlan lean_plan(const scv_cache* c, int32_t n_frames, const int16_t* units, bool rounds = false) {
  const int rows = scv::kAttnRowsBf16;
  const int64_t nq = int64_t(n_frames) * c->g.P;
  const int64_t rows_per_chunk = std::min<int64_t>(int64_t(c->g.C) * c->g.P, nq);
  const int nch = (n_frames + c->g.C - 1) / c->g.C;
  int64_t total = 0, shortest = INT64_MAX, longest = 0, n_items = 0;
  for (int b = 0; b < c->g.B; ++b)
    for (int ch = 0; ch < nch; ++ch) {
      const int64_t rows_ch = std::min<int64_t>(rows_per_chunk, nq - int64_t(ch) * rows_per_chunk);
      const int64_t u = units[ch + nch * b];
      const int64_t items = ((rows_ch + rows - 1) / rows) * c->g.H;
      total += items * u;
      n_items += items;
      shortest = std::min(shortest, u);
      longest = std::max(longest, u);
    }
  const int64_t cus = device_cu_count();
  const int64_t k = std::max<int64_t>(1, (total + cus * shortest - 1) / (cus * shortest));
  LeanPlan p;
  p.units = total;
  p.ctas = k <= kMaxLeanRounds ? int(k * cus) : 0;  // 0: items too short for the balanced schedule
  if (p.ctas > 0) p.cost = double(k) * (std::ceil(double(total) / p.ctas) + 2.0 * kSegmentCost);
  const int64_t full = n_items / cus;
  if (rounds && shortest == longest && full >= 1 && n_items > full * cus) {
    // whole-item rounds, then the left-over items cut equally
    LeanPlan h;
    h.units = total;
    h.v0 = int(full * cus);
    h.u0 = int64_t(h.v0) * shortest;
    h.round = int(cus);
    const int64_t tail = total - h.u0;
    const int64_t kt = std::max<int64_t>(1, (tail + cus * shortest - 1) / (cus * shortest));
    if (kt <= kMaxLeanRounds) {
      // the left-over items go to half as many ranges as there are compute
      // units: each range is twice as long, but the merge reads half the
      // partials, and the compute units left idle let the others clock
      // higher (720p: the same time within 0.1%, HBM traffic 1.00 -> 0.97
      // GB per launch pair)
      const int64_t g = kt * cus / 2;
      h.ctas = int(h.v0 + g);
      h.cost = double(full) * (double(shortest) + kSegmentCost) +
               double(kt) * (std::ceil(double(tail) / g) + 2.0 * kSegmentCost);
      p = h;
    }
  }
  return p;
}

// Schedule for a request: a key split count >= 1 (grid schedule) or -1 (the
// balanced schedule).  kv_splits > 0 is taken as given (capped at 64 and at
// the tile count); kv_splits = -1 asks for the balanced schedule (the fp32
// path runs the grid schedule unsplit).  With kv_splits = 0 a makespan model
// picks the cheapest option whose workspace fits ws_limit.  Grid schedule:
// workgroups of each (stream, chunk) class visit their visible key tiles
// (from t0 when given, else the steady state), split s ways -- a split may
// hold up to all of a class's tiles, at most tiles/s of them; they run in
// rounds over the compute units, each round as long as the longest
// workgroup plus a fixed 3-tile start/drain cost; with splits the fp32
// partials are written and read back by the merge (at ~8.5 MB per
// tile-time, plus 2 tile-times for the extra launch).  Balanced schedule:
// every compute unit runs an equal share of all units plus the fixed cost of
// two segments, then the merge reads back up to two partials per range.
int resolve_splits(const scv_cache* c, const int64_t* t0, int32_t n_frames, int32_t requested, size_t ws_limit) {
  const int tiles = int(c->g.rows_pad / scv::kKeyTile);
  if (requested > 0) return std::max(1, std::min(std::min(requested, tiles), 64));
  int16_t units[scv::kMaxBatch * scv::kMaxQueryChunks];
  LeanPlan plan{0, 0};
  if (lean_possible(c)) {
    class_units(c, t0, n_frames, units);
    plan = lean_plan(c, n_frames, units);
  }
  const bool lean_ok = plan.ctas > 0;
  if (requested == -1) return lean_ok ? -1 : 1;
  if (requested == -2) {
    if (!lean_ok) return 1;
    return lean_plan(c, n_frames, units, true).v0 > 0 ? -2 : -1;
  }
  const int rows = scv::attn_rows_per_workgroup(c->g);
  const int64_t nq = int64_t(n_frames) * c->g.P;
  const int64_t rows_per_chunk = std::min<int64_t>(int64_t(c->g.C) * c->g.P, nq);
  const int n_chunks = (n_frames + c->g.C - 1) / c->g.C;
  const int64_t per_class = ((rows_per_chunk + rows - 1) / rows) * c->g.H;  // workgroups per (stream, chunk)
  const int cus = device_cu_count();
  constexpr int kMaxClasses = scv::kMaxBatch * scv::kMaxQueryChunks;
  int64_t len[kMaxClasses];
  int n_cls = 0;
  for (int b = 0; b < (t0 ? c->g.B : 1); ++b)
    for (int ch = 0; ch < n_chunks; ++ch) {
      const int64_t f = t0 ? seen_frames(c, t0[b] + int64_t(ch) * c->g.C)
                           : std::min<int64_t>(c->g.n_slots, int64_t(c->g.S_f) + c->g.W + c->g.C);
      len[n_cls++] = std::min<int64_t>(tiles, (f * c->g.slot_rows + scv::kKeyTile - 1) / scv::kKeyTile + 1);
    }
  const int64_t class_mult = t0 ? 1 : c->g.B;  // without t0 every stream is one steady-state class
  const double rows_total = double(nq) * c->g.H * c->g.B;
  const double merge_unit = 2.0 * rows_total * (4.0 * c->g.D + 4.0) / 8.5e6;
  double best = 0.0;
  int best_s = 1;
  for (int s = 1; s <= std::min(64, tiles); ++s) {
    if (s > 1 && workspace_bytes(c, n_frames, s) > ws_limit) break;
    const int64_t cap = (tiles + s - 1) / s;
    double work = 0.0, lmax = 0.0;
    for (int i = 0; i < n_cls; ++i) {
      const double per = double(std::min<int64_t>(len[i], cap)) + 3.0;
      work += double(per_class * class_mult * s) * per;
      lmax = std::max(lmax, per);
    }
    const double rounds = std::ceil(work / (double(cus) * lmax) - 1e-9);
    double cost = rounds * lmax;
    if (s > 1) cost += 2.0 + s * merge_unit;
    if (s == 1 || cost < best) {
      best = cost;
      best_s = s;
    }
  }
  if (lean_ok) {
    // the cut ranges' partials are written and read back by the merge
    auto lean_cost = [&](const LeanPlan& p) {
      const double partial_bytes = 4.0 * (p.ctas - p.v0) * rows * (4.0 * c->g.D + 4.0);
      return p.cost + 2.0 + partial_bytes / 8.5e6;
    };
    int lean_s = -1;
    double cost = lean_cost(plan);
    const LeanPlan pr = lean_plan(c, n_frames, units, true);
    if (pr.v0 > 0 && lean_cost(pr) < cost && lean_workspace_bytes(c, pr.ctas) <= ws_limit) {
      lean_s = -2;
      cost = lean_cost(pr);
    }
    // Only a clear win moves off the grid schedule: with every compute unit
    // busy the shader clock drops a few percent (measured ~3% on the 480p
    // layer, which then runs no faster balanced), and the balanced
    // schedule reads more K/V from HBM.
    const int ctas = lean_s == -2 ? pr.ctas : plan.ctas;
    if (cost < 0.95 * best && lean_workspace_bytes(c, ctas) <= ws_limit) return lean_s;
  }
  return best_s;
}

// Workgroups of the balanced schedule (t0 null: the steady state).
int lean_ctas(const scv_cache* c, const int64_t* t0, int32_t n_frames, bool rounds) {
  int16_t units[scv::kMaxBatch * scv::kMaxQueryChunks];
  class_units(c, t0, n_frames, units);
  return lean_plan(c, n_frames, units, rounds).ctas;
}

size_t workspace_bytes(const scv_cache* c, int32_t n_frames, int splits) {
  if (splits < 0) return lean_workspace_bytes(c, lean_ctas(c, nullptr, n_frames, splits == -2));
  if (splits <= 1) return 0;
  const size_t rows = size_t(c->g.B) * c->g.H * size_t(n_frames) * c->g.P;
  return align_up(size_t(splits) * rows * c->g.D * 4, 256) + align_up(size_t(splits) * rows * 4, 256);
}

}  // namespace

extern "C" {

size_t scv_cache_bytes(const scv_config* cfg) {
  try {
    scv::Geometry g;
    scv_cache_layout L;
    std::string why;
    if (derive(cfg, &g, &L, &why) != SCV_OK) {
      g_last_error = why;
      return 0;
    }
    return L.total_bytes;
  } catch (...) {
    g_last_error = "internal error";
    return 0;
  }
}

scv_status scv_cache_layout_of(const scv_config* cfg, scv_cache_layout* out) {
  try {
    if (!out) return fail(SCV_E_INVALID, "out is NULL");
    scv::Geometry g;
    std::string why;
    const scv_status s = derive(cfg, &g, out, &why);
    if (s != SCV_OK) return fail(s, why);
    return SCV_OK;
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_cache_create(const scv_config* cfg, void* dev_buf, size_t bytes, scv_cache** out) {
  try {
    if (!out) return fail(SCV_E_INVALID, "out is NULL");
    *out = nullptr;
    scv::Geometry g;
    scv_cache_layout L;
    std::string why;
    const scv_status s = derive(cfg, &g, &L, &why);
    if (s != SCV_OK) return fail(s, why);
    if (!dev_buf) return fail(SCV_E_INVALID, "dev_buf is NULL");
    if (reinterpret_cast<uintptr_t>(dev_buf) & 255u) return fail(SCV_E_ALIGN, "dev_buf must be 256-byte aligned");
    if (bytes < L.total_bytes)
      return fail(SCV_E_STATE, "cache buffer holds " + std::to_string(bytes) + " bytes, config needs " +
                                   std::to_string(L.total_bytes));
    scv_cache* c = new (std::nothrow) scv_cache;
    if (!c) return fail(SCV_E_INVALID, "out of host memory");
    std::memset(c, 0, sizeof(*c));
    c->g = g;
    c->lay = L;
    c->base = static_cast<char*>(dev_buf);
    // omega_{a,j} = base^(-2j/d_a): one libm pow of the fp64 exponent each.
    for (int j = 0; j < g.dt / 2; ++j) c->om.t[j] = std::pow(g.base, -(2.0 * j) / double(g.dt));
    for (int j = 0; j < g.dh / 2; ++j) c->om.h[j] = std::pow(g.base, -(2.0 * j) / double(g.dh));
    for (int j = 0; j < g.dw / 2; ++j) c->om.w[j] = std::pow(g.base, -(2.0 * j) / double(g.dw));
    *out = c;
    return SCV_OK;
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_cache_destroy(scv_cache* c) {
  delete c;
  return SCV_OK;
}

scv_status scv_cache_init(scv_cache* c, const void* sink_k, const void* sink_v, void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if ((sink_k == nullptr) != (sink_v == nullptr)) return fail(SCV_E_INVALID, "give both sink_k and sink_v or neither");
    if (sink_k && c->g.S_f == 0) return fail(SCV_E_SHAPE, "sink given but sink_frames == 0");
    if ((s = check_ptr(sink_k, "sink_k", false)) != SCV_OK) return s;
    if ((s = check_ptr(sink_v, "sink_v", false)) != SCV_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int b = 0; b < c->g.B; ++b) c->pos_off[b] = 0;
    if ((s = hip_status(scv::launch_cache_reset(c->g, c->base + c->lay.k_offset, c->lay.total_bytes - c->lay.k_offset,
                                                reinterpret_cast<int64_t*>(c->base + c->lay.stamps_offset), st),
                        "cache reset launch")) != SCV_OK)
      return s;
    if ((s = hip_status(scv::launch_rope_tables(c->g, c->om, nullptr, 0, nullptr,
                                                reinterpret_cast<float2*>(c->base + c->lay.table_h_offset),
                                                reinterpret_cast<float2*>(c->base + c->lay.table_w_offset), st),
                        "rope table launch")) != SCV_OK)
      return s;
    if (sink_k) {
      int64_t zeros[scv::kMaxBatch] = {0};
      scv::RopeArgs a = base_rope_args(c, zeros, c->g.S_f);
      set_cache_targets(c, &a);
      a.k_in = sink_k;
      a.v_in = sink_v;
      a.rotate_k = 1;
      if ((s = hip_status(scv::launch_rope_append(a, st), "sink append launch")) != SCV_OK) return s;
    }
    return SCV_OK;
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_rope3d_apply(const scv_cache* c, void* q, void* k, const int64_t* t0, int32_t n_frames, void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if (!q && !k) return fail(SCV_E_INVALID, "q and k are both NULL");
    if ((s = check_ptr(q, "q", false)) != SCV_OK) return s;
    if ((s = check_ptr(k, "k", false)) != SCV_OK) return s;
    if (n_frames < 1 || n_frames > 65535 || int64_t(n_frames) * c->g.P >= (int64_t(1) << 31))
      return fail(SCV_E_SHAPE, "n_frames must be in [1, 65535] with n_frames * P < 2^31");
    if ((s = check_times(c, t0, n_frames)) != SCV_OK) return s;
    if ((s = check_positions(c, t0, n_frames)) != SCV_OK) return s;
    scv::RopeArgs a = base_rope_args(c, t0, n_frames);
    a.q_in = q;
    a.q_out = q;
    a.k_in = k;
    a.k_out = k;
    a.rotate_k = 1;
    return hip_status(scv::launch_rope_append(a, static_cast<hipStream_t>(stream)), "rope3d_apply launch");
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_kv_append_roll(scv_cache* c, const void* k_rot, const void* v, const int64_t* t0, int32_t n_frames,
                              void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if ((s = check_ptr(k_rot, "k_rot", true)) != SCV_OK) return s;
    if ((s = check_ptr(v, "v", true)) != SCV_OK) return s;
    if ((s = check_times(c, t0, n_frames < 1 ? 1 : n_frames)) != SCV_OK) return s;
    if ((s = check_append_frames(c, t0, n_frames)) != SCV_OK) return s;
    scv::RopeArgs a = base_rope_args(c, t0, n_frames);
    set_cache_targets(c, &a);
    a.k_in = k_rot;
    a.v_in = v;
    a.rotate_k = 0;
    return hip_status(scv::launch_rope_append(a, static_cast<hipStream_t>(stream)), "kv_append_roll launch");
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_rope3d_append(scv_cache* c, const void* q, void* q_rot, const void* k, const void* v,
                             const int64_t* t0, int32_t n_frames, void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if ((q == nullptr) != (q_rot == nullptr)) return fail(SCV_E_INVALID, "give both q and q_rot or neither");
    if ((s = check_ptr(q, "q", false)) != SCV_OK) return s;
    if ((s = check_ptr(q_rot, "q_rot", false)) != SCV_OK) return s;
    if ((s = check_ptr(k, "k", true)) != SCV_OK) return s;
    if ((s = check_ptr(v, "v", true)) != SCV_OK) return s;
    if ((s = check_times(c, t0, n_frames < 1 ? 1 : n_frames)) != SCV_OK) return s;
    if ((s = check_append_frames(c, t0, n_frames)) != SCV_OK) return s;
    if ((s = check_positions(c, t0, n_frames)) != SCV_OK) return s;
    scv::RopeArgs a = base_rope_args(c, t0, n_frames);
    set_cache_targets(c, &a);
    a.q_in = q;
    a.q_out = q_rot;
    a.k_in = k;
    a.v_in = v;
    a.rotate_k = 1;
    return hip_status(scv::launch_rope_append(a, static_cast<hipStream_t>(stream)), "rope3d_append launch");
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_rope_refresh(scv_cache* c, const int64_t* delta, void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if (!delta) return fail(SCV_E_INVALID, "delta is NULL");
    bool any = false;
    for (int b = 0; b < c->g.B; ++b) {
      if (delta[b] < 0 || delta[b] >= scv::kMaxTime - c->pos_off[b])
        return fail(SCV_E_RANGE, "delta[" + std::to_string(b) + "] = " + std::to_string(delta[b]) +
                                     " must be >= 0 and keep the stream's offset below 2^40");
      any = any || delta[b] != 0;
    }
    if (!any) return SCV_OK;
    scv::RefreshArgs a;
    std::memset(&a, 0, sizeof(a));
    a.g = c->g;
    a.cache_k = c->base + c->lay.k_offset;
    for (int b = 0; b < c->g.B; ++b) a.delta[b] = delta[b];
    for (int j = 0; j < c->g.dt / 2; ++j) a.omega_t[j] = c->om.t[j];
    if ((s = hip_status(scv::launch_rope_refresh(a, static_cast<hipStream_t>(stream)), "rope_refresh launch")) !=
        SCV_OK)
      return s;
    for (int b = 0; b < c->g.B; ++b) c->pos_off[b] += delta[b];
    return SCV_OK;
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_time_offsets(const scv_cache* c, int64_t* out) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if (!out) return fail(SCV_E_INVALID, "out is NULL");
    for (int b = 0; b < c->g.B; ++b) out[b] = c->pos_off[b];
    return SCV_OK;
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_sink_update(scv_cache* c, const void* k, const void* v, const int64_t* first_frame, int32_t n_frames,
                           void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if ((s = check_ptr(k, "k", true)) != SCV_OK) return s;
    if ((s = check_ptr(v, "v", true)) != SCV_OK) return s;
    if (c->g.S_f < 1) return fail(SCV_E_SHAPE, "the cache has no sink slots (sink_frames == 0)");
    if (n_frames < 1 || n_frames > c->g.S_f)
      return fail(SCV_E_SHAPE, "n_frames must be in [1, sink_frames = " + std::to_string(c->g.S_f) + "]");
    if ((s = check_times(c, first_frame, n_frames)) != SCV_OK) return s;
    if ((s = check_positions(c, first_frame, n_frames)) != SCV_OK) return s;
    scv::RopeArgs a = base_rope_args(c, first_frame, n_frames);
    set_cache_targets(c, &a);
    a.k_in = k;
    a.v_in = v;
    a.rotate_k = 1;
    a.to_sink = 1;
    return hip_status(scv::launch_rope_append(a, static_cast<hipStream_t>(stream)), "sink_update launch");
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_rope3d_append_sink(scv_cache* c, const void* q, void* q_rot, const void* k, const void* v,
                                  const int64_t* t0, int32_t n_frames, int32_t sink_first, int32_t sink_frames,
                                  void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if ((q == nullptr) != (q_rot == nullptr)) return fail(SCV_E_INVALID, "give both q and q_rot or neither");
    if ((s = check_ptr(q, "q", false)) != SCV_OK) return s;
    if ((s = check_ptr(q_rot, "q_rot", false)) != SCV_OK) return s;
    if ((s = check_ptr(k, "k", true)) != SCV_OK) return s;
    if ((s = check_ptr(v, "v", true)) != SCV_OK) return s;
    if ((s = check_times(c, t0, n_frames < 1 ? 1 : n_frames)) != SCV_OK) return s;
    if ((s = check_append_frames(c, t0, n_frames)) != SCV_OK) return s;
    if ((s = check_positions(c, t0, n_frames)) != SCV_OK) return s;
    if (c->g.S_f < 1) return fail(SCV_E_SHAPE, "the cache has no sink slots (sink_frames == 0)");
    if (sink_frames < 1 || sink_frames > c->g.S_f)
      return fail(SCV_E_SHAPE, "sink_frames must be in [1, " + std::to_string(c->g.S_f) + "]");
    if (sink_first < 0 || int64_t(sink_first) + sink_frames > n_frames)
      return fail(SCV_E_SHAPE, "sink_first + sink_frames must lie inside the call's n_frames frames");
    for (int b = 0; b < c->g.B; ++b)
      if (t0[b] < c->g.S_f)
        return fail(SCV_E_RANGE, "t0[" + std::to_string(b) + "] = " + std::to_string(t0[b]) +
                                     " would append into a sink slot; the fused sink update needs t0 >= sink_frames");
    scv::RopeArgs a = base_rope_args(c, t0, n_frames);
    set_cache_targets(c, &a);
    a.q_in = q;
    a.q_out = q_rot;
    a.k_in = k;
    a.v_in = v;
    a.rotate_k = 1;
    a.sink_first = sink_first;
    a.sink_frames = sink_frames;
    return hip_status(scv::launch_rope_append(a, static_cast<hipStream_t>(stream)), "rope3d_append_sink launch");
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_qkv_rope_append(scv_cache* c, const void* x, int32_t d_model, const void* w_qkv, void* q_rot,
                               const int64_t* t0, int32_t n_frames, void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if (c->g.dtype != SCV_BF16) return fail(SCV_E_DTYPE, "the fused projection needs dtype SCV_BF16");
    if ((s = check_ptr(x, "x", true)) != SCV_OK) return s;
    if ((s = check_ptr(w_qkv, "w_qkv", true)) != SCV_OK) return s;
    if ((s = check_ptr(q_rot, "q_rot", true)) != SCV_OK) return s;
    if (d_model < 32 || d_model % 32 != 0 || d_model > 65536)
      return fail(SCV_E_SHAPE, "d_model must be a multiple of 32 in [32, 65536]");
    if ((s = check_times(c, t0, n_frames < 1 ? 1 : n_frames)) != SCV_OK) return s;
    if ((s = check_append_frames(c, t0, n_frames)) != SCV_OK) return s;
    if ((s = check_positions(c, t0, n_frames)) != SCV_OK) return s;
    if (3 * int64_t(c->g.H) > 65535) return fail(SCV_E_SHAPE, "the fused projection supports at most 21845 heads");
    if (int64_t(n_frames) * c->g.P * d_model * 2 >= (int64_t(1) << 31))
      return fail(SCV_E_SHAPE, "n_frames * P * d_model * 2 bytes must stay below 2^31 per stream");
    if (int64_t(n_frames) * c->g.P >= (int64_t(1) << 24))
      return fail(SCV_E_SHAPE, "n_frames * P must stay below 2^24 tokens per call");
    scv::QkvArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = x;
    a.w = w_qkv;
    a.q_out = q_rot;
    a.cache_k = c->base + c->lay.k_offset;
    a.cache_v = c->base + c->lay.v_offset;
    a.stamps = reinterpret_cast<int64_t*>(c->base + c->lay.stamps_offset);
    a.tab_h = reinterpret_cast<const float2*>(c->base + c->lay.table_h_offset);
    a.tab_w = reinterpret_cast<const float2*>(c->base + c->lay.table_w_offset);
    a.d_model = d_model;
    a.n_frames = n_frames;
    a.g = c->g;
    {
      // token tile: rounds of workgroups over the compute units times the
      // work of one workgroup (proportional to its token count)
      const int64_t ntok = int64_t(n_frames) * c->g.P;
      const int64_t pairs = (3 * int64_t(c->g.H) + 1) / 2 * c->g.B;
      const int cus = device_cu_count();
      auto cost = [&](int64_t tile) { return ((ntok + tile - 1) / tile * pairs + cus - 1) / cus * tile; };
      a.token_tile = cost(384) < cost(256) ? 384 : 256;
      // the epilogue keeps its RoPE tables in LDS; 384-token tiles leave
      // more room for them
      const int D = c->g.D;
      auto fits = [&](int tile) { return scv::qkv_table_bytes(c->g, tile) <= scv::qkv_table_capacity(D, tile / 128); };
      if (!fits(a.token_tile)) a.token_tile = 384;
      if (!fits(a.token_tile))
        return fail(SCV_E_SHAPE, "the fused projection's RoPE tables (frames per tile x dt/2 + grid_h x dh/2 + "
                                 "grid_w x dw/2 pairs) exceed its LDS space");
    }
    for (int b = 0; b < c->g.B; ++b) {
      a.t0[b] = t0[b];
      a.pos_off[b] = c->pos_off[b];
    }
    for (int j = 0; j < c->g.dt / 2; ++j) a.omega_t[j] = c->om.t[j];
    return hip_status(scv::launch_qkv_rope(a, static_cast<hipStream_t>(stream)), "qkv_rope_append launch");
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

int32_t scv_attention_splits(const scv_cache* c, const int64_t* t0, int32_t n_frames, int32_t kv_splits,
                             size_t ws_bytes) {
  try {
    if (!c || n_frames < 1 || kv_splits < -2) return 0;
    if (t0 && check_times(c, t0, n_frames) != SCV_OK) return 0;
    return resolve_splits(c, t0, n_frames, kv_splits, ws_bytes);
  } catch (...) {
    return 0;
  }
}

size_t scv_attention_workspace_bytes(const scv_cache* c, int32_t n_frames, int32_t kv_splits) {
  try {
    if (!c || n_frames < 1 || kv_splits < -2) return 0;
    return workspace_bytes(c, n_frames, resolve_splits(c, nullptr, n_frames, kv_splits, SIZE_MAX));
  } catch (...) {
    return 0;
  }
}

size_t scv_attention_request_workspace_bytes(const scv_cache* c, const int64_t* t0, int32_t n_frames,
                                             int32_t kv_splits) {
  try {
    if (!c || !t0 || n_frames < 1 || kv_splits < -2) return 0;
    if (check_times(c, t0, n_frames) != SCV_OK) return 0;
    const int splits = resolve_splits(c, t0, n_frames, kv_splits, SIZE_MAX);
    if (splits >= 0) return workspace_bytes(c, n_frames, splits);
    return lean_workspace_bytes(c, lean_ctas(c, t0, n_frames, splits == -2));
  } catch (...) {
    return 0;
  }
}

}  // extern "C"

// The library's own workspace for scv_chunk_attention_scratch: device memory
// that exists on every GPU the library runs on from module load to process
// end, so that the call allocates nothing.  Host code never passes this name
// to a kernel (on the host it is only a stand-in for the symbol): it uses the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SCV_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = SCV_SCRATCH_BYTES;

// chunk_attention with the workspace ws of ws_bytes bytes (the caller's, or
// the library's static scratch when from_scratch).
scv_status chunk_attention_impl(const scv_cache* c, const void* q_rot, const int64_t* t0, int32_t n_frames, void* o,
                                float* lse, int32_t kv_splits, void* ws, size_t ws_bytes, void* stream,
                                bool from_scratch) {
  {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if ((s = check_ptr(q_rot, "q_rot", true)) != SCV_OK) return s;
    if ((s = check_ptr(o, "o", true)) != SCV_OK) return s;
    if ((s = check_ptr(lse, "lse", false)) != SCV_OK) return s;
    if (n_frames < 1 || n_frames > c->g.k_max * c->g.C)
      return fail(SCV_E_SHAPE, "n_frames must be in [1, max_query_chunks*chunk_frames]");
    if (kv_splits < -2) return fail(SCV_E_INVALID, "kv_splits must be >= -2");
    if ((s = check_times(c, t0, n_frames)) != SCV_OK) return s;
    // with kv_splits = 0 the choice sees t0 and the workspace given
    const int splits = resolve_splits(c, t0, n_frames, kv_splits, ws ? ws_bytes : 0);
    int16_t lean_units[scv::kMaxBatch * scv::kMaxQueryChunks];
    LeanPlan plan{0, 0};
    if (splits < 0) {
      class_units(c, t0, n_frames, lean_units);
      plan = lean_plan(c, n_frames, lean_units, splits == -2);
    }
    const size_t need = splits < 0 ? lean_workspace_bytes(c, plan.ctas) : workspace_bytes(c, n_frames, splits);
    if (need > 0 && from_scratch && need > ws_bytes)
      return fail(SCV_E_WORKSPACE, "this request's schedule needs " + std::to_string(need) +
                                       " bytes of workspace; the library's static scratch holds " +
                                       std::to_string(ws_bytes) + " (use scv_chunk_attention with a workspace)");
    if (need > 0) {
      if (!ws) return fail(SCV_E_WORKSPACE, "workspace is NULL; need " + std::to_string(need) + " bytes");
      if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(SCV_E_ALIGN, "workspace must be 256-byte aligned");
      if (ws_bytes < need)
        return fail(SCV_E_WORKSPACE, "workspace holds " + std::to_string(ws_bytes) + " bytes; need " +
                                         std::to_string(need));
    }
    scv::AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.g = c->g;
    a.q = q_rot;
    a.o = o;
    a.lse = lse;
    a.cache_k = c->base + c->lay.k_offset;
    a.cache_v = c->base + c->lay.v_offset;
    a.stamps = reinterpret_cast<const int64_t*>(c->base + c->lay.stamps_offset);
    a.n_frames = n_frames;
    a.Nq = n_frames * c->g.P;
    {
      const int rows_wg = scv::attn_rows_per_workgroup(c->g);
      a.rows_per_chunk = c->g.C * c->g.P;
      a.qtiles_per_chunk = (std::min(a.rows_per_chunk, a.Nq) + rows_wg - 1) / rows_wg;
      a.n_qtiles = ((n_frames + c->g.C - 1) / c->g.C) * a.qtiles_per_chunk;
    }
    const bool lean = splits < 0;
    a.splits = lean ? 1 : splits;
    {
      // work classes (chunk, stream), longest first: the keys each chunk can
      // see once its history is in the cache (ties keep their natural order)
      const int nch = (n_frames + c->g.C - 1) / c->g.C;
      const int ncls = nch * c->g.B;
      int64_t len[scv::kMaxBatch * scv::kMaxQueryChunks];
      for (int b = 0; b < c->g.B; ++b)
        for (int ch = 0; ch < nch; ++ch) {
          a.cls_order[ch + nch * b] = int16_t(ch + nch * b);
          len[ch + nch * b] = seen_frames(c, t0[b] + int64_t(ch) * c->g.C);
        }
      std::stable_sort(a.cls_order, a.cls_order + ncls, [&](int16_t x, int16_t y) { return len[x] > len[y]; });
    }
    a.tiles_total = int32_t(c->g.rows_pad / scv::kKeyTile);
    a.tiles_per_split = (a.tiles_total + splits - 1) / splits;
    a.scale_ln = float(1.0 / std::sqrt(double(c->g.D)));
    a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(c->g.D)));
    for (int b = 0; b < c->g.B; ++b) a.t0[b] = t0[b];
    if (splits > 1) {
      const size_t rows = size_t(c->g.B) * c->g.H * size_t(a.Nq);
      a.part_o = static_cast<float*>(ws);
      a.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(size_t(splits) * rows * c->g.D * 4, 256));
    }
    if (lean) {
      std::memcpy(a.cls_units, lean_units, sizeof(lean_units));
      a.lean = 1;
      a.lean_ctas = plan.ctas;
      a.lean_units = plan.units;
      a.lean_v0 = plan.v0;
      a.lean_u0 = plan.u0;
      a.lean_round = plan.round;
      a.part_o = static_cast<float*>(ws);
      a.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                            align_up(size_t(plan.ctas) * 2 * scv::kAttnRowsBf16 * c->g.D * 4, 256));
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = hip_status(scv::launch_chunk_attention(a, st), "chunk_attention launch")) != SCV_OK) return s;
    if (lean) {
      if ((s = hip_status(scv::launch_attn_lean_merge(a, st), "attn_lean_merge launch")) != SCV_OK) return s;
    } else if (splits > 1) {
      scv::MergeArgs m;
      m.part_o = a.part_o;
      m.part_lse = a.part_lse;
      m.o = o;
      m.lse = lse;
      m.splits = splits;
      m.Nq = a.Nq;
      m.g = c->g;
      if ((s = hip_status(scv::launch_attn_merge(m, st), "attn_merge launch")) != SCV_OK) return s;
    }
    return SCV_OK;
  }
}

// Device address of `scratch` on the current device, looked up once per
// device; nullptr (message in g_last_error) when the lookup fails.
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* ptr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    g_last_error = "no current HIP device (or more than 64 devices)";
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_error = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return nullptr;
    }
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace

extern "C" {

scv_status scv_chunk_attention(const scv_cache* c, const void* q_rot, const int64_t* t0, int32_t n_frames, void* o,
                               float* lse, int32_t kv_splits, void* ws, size_t ws_bytes, void* stream) {
  try {
    return chunk_attention_impl(c, q_rot, t0, n_frames, o, lse, kv_splits, ws, ws_bytes, stream, false);
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_chunk_attention_scratch(const scv_cache* c, const void* q_rot, const int64_t* t0, int32_t n_frames,
                                       void* o, float* lse, int32_t kv_splits, void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    void* ws = scratch_on_current_device();
    if (!ws) return SCV_E_HIP;
    return chunk_attention_impl(c, q_rot, t0, n_frames, o, lse, kv_splits, ws, kScratchBytes, stream, true);
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

size_t scv_rope_table_floats(const scv_cache* c, int32_t n_frames) {
  if (!c || n_frames < 1) return 0;
  return 2 * (size_t(c->g.B) * n_frames * (c->g.dt / 2) + size_t(c->g.grid_h) * (c->g.dh / 2) +
              size_t(c->g.grid_w) * (c->g.dw / 2));
}

scv_status scv_rope_tables(const scv_cache* c, const int64_t* t0, int32_t n_frames, float* out, size_t n_floats,
                           void* stream) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if ((s = check_ptr(out, "out", true)) != SCV_OK) return s;
    if (n_frames < 1 || n_frames > 65535) return fail(SCV_E_SHAPE, "n_frames must be in [1, 65535]");
    if ((s = check_times(c, t0, n_frames)) != SCV_OK) return s;
    if ((s = check_positions(c, t0, n_frames)) != SCV_OK) return s;
    const size_t need = scv_rope_table_floats(c, n_frames);
    if (n_floats < need) return fail(SCV_E_SHAPE, "out holds fewer than " + std::to_string(need) + " floats");
    const size_t nt = size_t(c->g.B) * n_frames * (c->g.dt / 2);
    const size_t nh = size_t(c->g.grid_h) * (c->g.dh / 2);
    float2* base = reinterpret_cast<float2*>(out);
    int64_t pos[scv::kMaxBatch];
    for (int b = 0; b < c->g.B; ++b) pos[b] = t0[b] - c->pos_off[b];
    return hip_status(scv::launch_rope_tables(c->g, c->om, pos, n_frames, out, base + nt, base + nt + nh,
                                              static_cast<hipStream_t>(stream)),
                      "rope table launch");
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

scv_status scv_debug_stamps(const scv_cache* c, int64_t* out, size_t n) {
  try {
    scv_status s;
    if ((s = check_cache(c)) != SCV_OK) return s;
    if (!out) return fail(SCV_E_INVALID, "out is NULL");
    const size_t need = size_t(c->g.B) * size_t(c->g.n_slots);
    if (n < need) return fail(SCV_E_SHAPE, "out holds fewer than " + std::to_string(need) + " entries");
    if ((s = hip_status(hipDeviceSynchronize(), "device synchronise")) != SCV_OK) return s;
    return hip_status(hipMemcpy(out, c->base + c->lay.stamps_offset, need * sizeof(int64_t), hipMemcpyDeviceToHost),
                      "stamps copy");
  } catch (...) {
    return fail(SCV_E_INVALID, "internal error");
  }
}

const char* scv_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
