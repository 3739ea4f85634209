// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "scv.h"

namespace scv {

constexpr int kMaxBatch = 64;
constexpr int kMaxSlots = 64;
constexpr int kMaxAxisPairs = 64;  // d_a / 2 <= head_dim / 2 <= 64
constexpr int kMaxQueryChunks = 8;
constexpr int kKeyTile = 64;       // rows per attention key tile
constexpr int64_t kMaxTime = int64_t(1) << 40;
constexpr int kAttnRowsBf16 = 256;  // query rows per attention workgroup (bf16)
constexpr int kAttnRowsF32 = 128;   // query rows per attention workgroup (fp32)

// Everything about a cache that kernels need, resolved once on the host.
struct Geometry {
  int32_t B, H, D, dt, dh, dw;
  int32_t grid_h, grid_w, P;
  int32_t S_f, W, C, k_max, R, n_slots;
  int64_t slot_rows, rows, rows_pad;
  int32_t dtype;     // scv_dtype of q, k, v, o and the cached values
  int32_t qk_dtype;  // scv_dtype of rotated q/k and the cached keys
  int32_t elem_bytes;
  double base;
};

// fp64 frequency ladders omega_{a,j} = base^(-2j/d_a), passed by value.
struct Omegas {
  double t[kMaxAxisPairs];
  double h[kMaxAxisPairs];
  double w[kMaxAxisPairs];
};

// Rotation / append kernel arguments (by value).
struct RopeArgs {
  const void* q_in;
  void* q_out;       // null: no query work
  const void* k_in;
  void* k_out;       // k destination when not appending (in-place rope)
  const void* v_in;  // null: no values
  void* cache_k;     // null: no append
  void* cache_v;
  int64_t* stamps;
  const float2* tab_h;
  const float2* tab_w;
  int32_t n_frames;
  int32_t rotate_k;  // 0: k is already rotated (kv_append_roll)
  int32_t to_sink;   // 1: frame f of the call goes to sink slot f (sink update)
  int32_t sink_first;   // with sink_frames > 0: frames sink_first .. +sink_frames-1 of the
  int32_t sink_frames;  // call also go to sink slots 0 .. sink_frames-1 (append + sink update)
  Geometry g;
  int64_t t0[kMaxBatch];       // global frame of the call's first frame
  int64_t pos_off[kMaxBatch];  // time position = global frame - pos_off
  double omega_t[kMaxAxisPairs];
};

// RoPE refresh arguments (by value): turn the time pairs of every cached
// key of stream b by -delta[b] * omega_t.
struct RefreshArgs {
  void* cache_k;
  Geometry g;
  int64_t delta[kMaxBatch];
  double omega_t[kMaxAxisPairs];
};

// Fused QKV projection + RoPE + append arguments (by value).
struct QkvArgs {
  const void* x;      // [B][Ntok][d_model] layer input (dtype)
  const void* w;      // [3*H*D][d_model] projection weight (dtype)
  void* q_out;        // [B][Ntok][H][D] rotated queries (qk_dtype)
  void* cache_k;
  void* cache_v;
  int64_t* stamps;
  const float2* tab_h;
  const float2* tab_w;
  int32_t d_model;
  int32_t n_frames;
  int32_t token_tile;  // tokens per workgroup: 256 or 384
  Geometry g;
  int64_t t0[kMaxBatch];
  int64_t pos_off[kMaxBatch];
  double omega_t[kMaxAxisPairs];
};

// LDS bytes left to the fused projection's epilogue for its RoPE tables and
// frame row bases: its two K-slice stages (x and weight rows, 64 deep) less
// one 32-token staging block per wave (8 waves); tile = 128 * TB tokens.
constexpr int qkv_table_capacity(int D, int TB) { return 2 * (TB * 128 * 64 * 2 + 2 * D * 64 * 2) - 8 * 32 * D * 2; }

// LDS bytes those tables take for a tile of `tile` tokens: the time pairs of
// every frame the tile can span, the height and width tables, one int32 row
// base per frame.
inline int64_t qkv_table_bytes(const Geometry& g, int tile) {
  const int64_t nf = (tile - 1 + g.P - 1) / g.P + 1;
  return (nf * (g.dt / 2) + int64_t(g.grid_h) * (g.dh / 2) + int64_t(g.grid_w) * (g.dw / 2)) * 8 + nf * 4;
}

// Attention kernel arguments (by value).
struct AttnArgs {
  const void* q;
  void* o;          // final output (splits == 1)
  float* lse;       // nullable final lse (splits == 1)
  float* part_o;    // [splits][B][H][Nq][D] fp32 (splits > 1)
  float* part_lse;  // [splits][B][H][Nq]
  const void* cache_k;
  const void* cache_v;
  const int64_t* stamps;
  int32_t n_frames;
  int32_t Nq;             // n_frames * P query rows per stream
  int32_t n_qtiles;       // n_chunks * qtiles_per_chunk
  int32_t qtiles_per_chunk;  // query tiles never straddle two query chunks
  int32_t rows_per_chunk;    // chunk_frames * P
  int32_t splits;
  int32_t tiles_total;    // rows_pad / kKeyTile
  int32_t tiles_per_split;
  float scale_log2;       // log2(e) / sqrt(D)
  float scale_ln;         // 1 / sqrt(D)
  Geometry g;
  int64_t t0[kMaxBatch];
  // (chunk, stream) work classes, class id = chunk + n_chunks * stream, in
  // the order workgroups should start (longest first)
  int16_t cls_order[kMaxBatch * kMaxQueryChunks];
  // Balanced schedule (lean != 0, bf16 kernel only).  Work units are
  // (query tile, visited key tile) pairs; the items (stream, head, chunk,
  // query tile) are laid end to end, stream-major, then head, chunk and
  // tile, each taking cls_units[chunk + n_chunks * stream] units.  The grid
  // has lean_ctas workgroups; workgroup v (after the XCD renumbering) takes
  // units [v * lean_units / lean_ctas, (v + 1) * lean_units / lean_ctas).
  // An item cut by a range boundary leaves normalised fp32 partials in
  // part_o / part_lse at [v][slot][row] (slot 0: the workgroup's first item,
  // 1: its last) for attn_lean_merge_kernel.
  // With lean_v0 > 0 the first lean_v0 ranges are whole items instead (range
  // v = item v, run in rounds of lean_round workgroups), and only the units
  // [lean_u0, lean_units) of the remaining items are cut into the
  // lean_ctas - lean_v0 equal ranges.
  int32_t lean;
  int32_t lean_ctas;
  int64_t lean_units;
  int32_t lean_v0;
  int32_t lean_round;
  int64_t lean_u0;
  int16_t cls_units[kMaxBatch * kMaxQueryChunks];
};

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  void* o;
  float* lse;
  int32_t splits;
  int32_t Nq;
  Geometry g;
};

inline int attn_rows_per_workgroup(const Geometry& g) {
  return g.dtype == SCV_BF16 ? kAttnRowsBf16 : kAttnRowsF32;
}

// cos/sin of the fp64 angle pos * omega, rounded to fp32 (round to nearest).
__device__ __forceinline__ float2 rope_cos_sin(int64_t pos, double omega) {
  const double th = static_cast<double>(pos) * omega;
  double s, c;
  sincos(th, &s, &c);
  return make_float2(static_cast<float>(c), static_cast<float>(s));
}

// Launchers (return the hipError_t of the launch).
hipError_t launch_rope_append(const RopeArgs& a, hipStream_t s);
hipError_t launch_rope_tables(const Geometry& g, const Omegas& om, const int64_t* t0, int32_t n_frames,
                              float* out_t, float2* out_h, float2* out_w, hipStream_t s);
hipError_t launch_rope_refresh(const RefreshArgs& a, hipStream_t s);
hipError_t launch_qkv_rope(const QkvArgs& a, hipStream_t s);
hipError_t launch_cache_reset(const Geometry& g, void* kv_base, size_t kv_bytes, int64_t* stamps, hipStream_t s);
hipError_t launch_chunk_attention(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_attn_lean_merge(const AttnArgs& a, hipStream_t s);

}  // namespace scv
