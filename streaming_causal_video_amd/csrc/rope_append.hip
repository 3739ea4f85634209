// 3D RoPE at a global time index, fused with the append/roll of keys and
// values into the sink-pinned ring cache (gfx950).
//
// What is computed follows "Accelerating Video Generation Inference with
// Sequential-Parallel 3D Positional Encoding Using a Global Time Index"
// (section 2(b): the block's start frame is the global time index, so each
// token's time position is t0 + frame offset, computed locally; section 2(c):
// cos/sin precomputed into contiguous tables, no host-side work per step) and
// the sink + rolling-window cache of "StreamDiffusionV2: A Streaming System
// for Dynamic and Interactive Video Generation" (paper-review blog, section 2).
//
// These kernels are HBM-bound: per (token, head) row they read q, k, v once
// and write q_rot, k_rot, v once (6 passes of d*elem bytes).  Layout choices:
//  * one workgroup = 64 consecutive tokens of one frame x one head, so the
//    frame (hence the ring slot and the time angle) is uniform per workgroup;
//  * 16-byte vector loads/stores along head_dim, 16 B per lane;
//  * values are stored transposed ([head][d][row]) so the attention kernel
//    can feed V^T straight into the MFMA A operand; the transpose goes
//    through LDS and leaves as 16-byte row-contiguous stores;
//  * the time-axis cos/sin of the workgroup's frame is evaluated in fp64 at
//    workgroup start (one entry per lane), the row/column tables are static
//    per cache and read through L1/L2;
//  * a workgroup's four 16-token passes load their inputs one pass ahead,
//    with no load behind a branch, so two passes of loads are in flight.
#include <type_traits>

#include "scv_internal.h"

namespace scv {
namespace {

struct TableArgs {
  Geometry g;
  Omegas om;
  int64_t t0[kMaxBatch];
  int32_t n_frames;
  float2* out_t;  // [B][n_frames][dt/2] (nullable)
  float2* out_h;  // [grid_h][dh/2]       (nullable)
  float2* out_w;  // [grid_w][dw/2]       (nullable)
};

__global__ __launch_bounds__(256) void rope_tables_kernel(TableArgs a) {
  const Geometry& g = a.g;
  const int pt = g.dt / 2, ph = g.dh / 2, pw = g.dw / 2;
  const int64_t n_t = a.out_t ? int64_t(g.B) * a.n_frames * pt : 0;
  const int64_t n_h = a.out_h ? int64_t(g.grid_h) * ph : 0;
  const int64_t n_w = a.out_w ? int64_t(g.grid_w) * pw : 0;
  const int64_t total = n_t + n_h + n_w;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    if (i < n_t) {
      const int j = int(i % pt);
      const int64_t bf = i / pt;
      const int f = int(bf % a.n_frames);
      const int b = int(bf / a.n_frames);
      a.out_t[i] = rope_cos_sin(a.t0[b] + f, a.om.t[j]);
    } else if (i < n_t + n_h) {
      const int64_t r = i - n_t;
      a.out_h[r] = rope_cos_sin(r / ph, a.om.h[r % ph]);
    } else {
      const int64_t r = i - n_t - n_h;
      a.out_w[r] = rope_cos_sin(r / pw, a.om.w[r % pw]);
    }
  }
}

// Zero the key/value region (16-byte stores) and mark every slot empty.
__global__ __launch_bounds__(256) void cache_reset_kernel(uint4* kv, int64_t n16, int64_t* stamps, int64_t n_stamps) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n16; i += stride) kv[i] = make_uint4(0, 0, 0, 0);
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n_stamps; i += stride) stamps[i] = -1;
}

template <typename T>
struct Vec16 {  // elements of T in 16 bytes
  static constexpr int N = 16 / int(sizeof(T));
};

template <typename T>
__device__ __forceinline__ void unpack16(const uint4 u, float* x) {
  if constexpr (sizeof(T) == 4) {
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z);
    x[3] = __uint_as_float(u.w);
  } else if constexpr (std::is_same<T, _Float16>::value) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(w[i] & 0xffffu)));
      x[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(w[i] >> 16)));
    }
  } else {  // bf16: the upper half of an fp32
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// Two fp32 values rounded (to nearest even, native conversion) into the
// 16-bit type T and packed.  fp16 saturates: a value beyond the largest
// finite fp16 is stored as +-65504 instead of +-inf (rotated keys stay
// finite, so attention over them stays defined).
template <typename T>
__device__ __forceinline__ uint32_t pack_x2(float lo, float hi) {
  if constexpr (std::is_same<T, _Float16>::value) {
    lo = __builtin_amdgcn_fmed3f(lo, -65504.f, 65504.f);
    hi = __builtin_amdgcn_fmed3f(hi, -65504.f, 65504.f);
  }
  const T a = static_cast<T>(lo);
  const T b = static_cast<T>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// fp32 values rounded to T, 16 bytes worth (4 fp32 or 8 16-bit values).
template <typename T>
__device__ __forceinline__ uint4 pack16(const float* x) {
  if constexpr (sizeof(T) == 4) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
  } else {
    return make_uint4(pack_x2<T>(x[0], x[1]), pack_x2<T>(x[2], x[3]), pack_x2<T>(x[4], x[5]),
                      pack_x2<T>(x[6], x[7]));
  }
}

constexpr int kTokTile = 64;

// One workgroup: tokens [p0, p0+64) of frame f of stream b, one head.
// T: type of q, k, v inputs and cached values; QT: type of rotated q/k.
// ALL: the chunk append (q rotated out, k rotated and v into the cache), so
// every input and output exists and no load or store sits behind a branch.
template <typename T, typename QT, int D, bool ALL>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeArgs a) {
  static_assert(sizeof(T) == sizeof(QT), "rotated and input elements share a size");
  constexpr int EPV = Vec16<T>::N;      // elements per 16-byte vector
  constexpr int TPR = D / EPV;          // threads per token row
  constexpr int TPP = 256 / TPR;        // tokens per pass
  constexpr int ROW_U32 = D * int(sizeof(T)) / 4 + 1;  // odd pitch: spreads banks
  const Geometry& g = a.g;
  const int tiles_per_frame = (g.P + kTokTile - 1) / kTokTile;
  const int tile = blockIdx.x % tiles_per_frame;
  const int head = blockIdx.x / tiles_per_frame;
  const int f = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t gframe = a.t0[b] + f;
  const int64_t tpos = gframe - a.pos_off[b];  // time position (after RoPE refreshes)
  const int p0 = tile * kTokTile;
  const int nvalid = min(kTokTile, g.P - p0);
  const int pt = g.dt / 2, pth = (g.dt + g.dh) / 2;
  const bool to_cache = ALL || a.cache_k != nullptr;
  const bool do_q = ALL || a.q_out != nullptr;
  const bool do_k = ALL || a.k_in != nullptr;
  const bool do_v = ALL || a.v_in != nullptr;
  const bool rotate_k = ALL || a.rotate_k;
  const bool need_angles = do_q || (do_k && rotate_k);

  __shared__ float2 tab_t[kMaxAxisPairs];
  __shared__ uint32_t vtile[kTokTile * ROW_U32];

  if (need_angles && int(threadIdx.x) < pt) tab_t[threadIdx.x] = rope_cos_sin(tpos, a.omega_t[threadIdx.x]);

  int64_t slot = 0;
  if (to_cache) slot = a.to_sink ? f : (gframe < g.S_f ? gframe : g.S_f + gframe % g.R);
  // append + sink update in one launch: this frame is also written to sink
  // slot sslot (same rotated k, same v)
  const int sslot = f - a.sink_first;
  const bool also_sink = to_cache && !a.to_sink && sslot >= 0 && sslot < a.sink_frames;

  __syncthreads();

  const int dg = threadIdx.x % TPR;
  const int64_t Ntok = int64_t(a.n_frames) * g.P;
  // A pass covers TPP tokens.  Its inputs (q, k, v and the height and width
  // cos/sin) are loaded one pass ahead: the loads of pass i+1 are issued
  // before the rotations and stores of pass i, so a wave has two passes of
  // loads in flight instead of waiting for q, then k, then v in turn.
  constexpr int kPasses = kTokTile / TPP;
  struct PassIn {
    uint4 q, k, v;
    float2 tv[EPV / 2], gv[EPV / 2];  // time (LDS) and height/width (global) entries
  };
  // Loads take no branch (a branch makes the compiler wait for every load
  // in flight where it joins): tokens past the frame's end load a valid
  // token of the tile instead (their results are dropped, their V rows
  // zeroed), and each pair loads both its time entry (LDS) and its height or
  // width entry (global) and keeps the one it needs.
  auto load_pass = [&](int pass, PassIn& in) __attribute__((always_inline)) {
    const int tt = pass * TPP + int(threadIdx.x) / TPR;
    const bool valid = tt < nvalid;
    const int p = valid ? p0 + tt : p0;
    const int64_t in_off = ((int64_t(b) * Ntok + int64_t(f) * g.P + p) * g.H + head) * D + dg * EPV;
    in.q = in.k = in.v = make_uint4(0, 0, 0, 0);
    if (do_q) in.q = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.q_in) + in_off);
    if (do_k) in.k = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.k_in) + in_off);
    if (do_v) in.v = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.v_in) + in_off);
    if (need_angles) {
      const int yy = p / g.grid_w, xx = p - (p / g.grid_w) * g.grid_w;
#pragma unroll
      for (int i = 0; i < EPV / 2; ++i) {
        const int pj = dg * (EPV / 2) + i;
        in.tv[i] = tab_t[pj < pt ? pj : 0];
        const float2* gp = pj < pth ? a.tab_h + max(yy * (g.dh / 2) + (pj - pt), 0) : a.tab_w + (xx * (g.dw / 2) + (pj - pth));
        in.gv[i] = *gp;
      }
    }
  };
  auto rotate = [&](const uint4 raw, const PassIn& in) __attribute__((always_inline)) {
    float x[EPV], y[EPV];
    unpack16<T>(raw, x);
#pragma unroll
    for (int i = 0; i < EPV / 2; ++i) {
      const float2 cs = dg * (EPV / 2) + i < pt ? in.tv[i] : in.gv[i];
      y[2 * i] = x[2 * i] * cs.x - x[2 * i + 1] * cs.y;
      y[2 * i + 1] = x[2 * i] * cs.y + x[2 * i + 1] * cs.x;
    }
    return pack16<QT>(y);
  };
  // FULL: every token of the tile exists (all but the last tile of a frame
  // whose token count is not a multiple of 64), so nothing in the loop
  // depends on the lane: no branch for the compiler to wait at
  auto passes = [&](auto full_c) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_c)::value;
    PassIn in[2];
    load_pass(0, in[0]);
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const PassIn& cur = in[pass & 1];
      if (pass + 1 < kPasses) load_pass(pass + 1, in[(pass + 1) & 1]);
      const int tt = pass * TPP + int(threadIdx.x) / TPR;
      const int p = p0 + tt;
      const bool valid = FULL || tt < nvalid;
      const int64_t in_off = ((int64_t(b) * Ntok + int64_t(f) * g.P + p) * g.H + head) * D + dg * EPV;
      if (do_q && valid) *reinterpret_cast<uint4*>(static_cast<QT*>(a.q_out) + in_off) = rotate(cur.q, cur);
      if (do_k && valid) {
        const uint4 outv = rotate_k ? rotate(cur.k, cur) : cur.k;
        if (to_cache) {
          const int64_t row = slot * g.slot_rows + p;
          QT* dst = static_cast<QT*>(a.cache_k) + ((int64_t(b) * g.H + head) * g.rows_pad + row) * D + dg * EPV;
          *reinterpret_cast<uint4*>(dst) = outv;
          if (also_sink) *reinterpret_cast<uint4*>(dst + (int64_t(sslot) - slot) * g.slot_rows * D) = outv;
        } else {
          *reinterpret_cast<uint4*>(static_cast<QT*>(a.k_out) + in_off) = outv;
        }
      }
      if (do_v) {
        // rows past the frame's end are zero (they become slot padding)
        uint32_t* r = &vtile[tt * ROW_U32 + dg * 4];
        r[0] = valid ? cur.v.x : 0u;
        r[1] = valid ? cur.v.y : 0u;
        r[2] = valid ? cur.v.z : 0u;
        r[3] = valid ? cur.v.w : 0u;
      }
    }
  };
  if (nvalid == kTokTile)
    passes(std::true_type{});
  else
    passes(std::false_type{});

  if (do_v) {
    __syncthreads();
    // Transposed write: for each d, tokens p0 .. p0+nvalid (rounded up to a
    // whole vector; rows past P up to slot_rows belong to this slot's padding).
    constexpr int CPR = kTokTile / EPV;  // vectors per d-row
    const int nvec = (nvalid + EPV - 1) / EPV;
    T* vbase = static_cast<T*>(a.cache_v) + (int64_t(b) * g.H + head) * D * g.rows_pad + slot * g.slot_rows + p0;
    for (int idx = threadIdx.x; idx < D * CPR; idx += 256) {
      const int d = idx / CPR, c = idx % CPR;
      if (c >= nvec) continue;
      uint4 out;
      if constexpr (sizeof(T) == 4) {
        out.x = vtile[(c * 4 + 0) * ROW_U32 + d];
        out.y = vtile[(c * 4 + 1) * ROW_U32 + d];
        out.z = vtile[(c * 4 + 2) * ROW_U32 + d];
        out.w = vtile[(c * 4 + 3) * ROW_U32 + d];
      } else {
        uint32_t h[8];
        const int sh = (d & 1) * 16;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (vtile[(c * 8 + e) * ROW_U32 + (d >> 1)] >> sh) & 0xffffu;
        out = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      }
      *reinterpret_cast<uint4*>(vbase + int64_t(d) * g.rows_pad + c * EPV) = out;
      if (also_sink) *reinterpret_cast<uint4*>(vbase + int64_t(d) * g.rows_pad + c * EPV + (int64_t(sslot) - slot) * g.slot_rows) = out;
    }
  }

  if (to_cache && tile == 0 && head == 0 && threadIdx.x == 0) {
    a.stamps[int64_t(b) * g.n_slots + slot] = gframe;
    if (also_sink) a.stamps[int64_t(b) * g.n_slots + sslot] = gframe;
  }
}

// RoPE refresh: every cached key row of stream b, head h (all rows_pad rows:
// empty slots and padding rows are zero and stay zero) has its time pairs
// turned by -delta[b] * omega_t, i.e. (x, y) -> (x c + y s, y c - x s) with
// c, s the fp32-rounded cos/sin of the fp64 angle delta[b] * omega_j; the
// rest of the row is untouched.  Only the 16-byte chunks that hold time dims
// are read and written.  One workgroup = kRefreshRows rows of one (b, h).
constexpr int kRefreshRows = 256;

template <typename QT, int D>
__global__ __launch_bounds__(256) void rope_refresh_kernel(RefreshArgs a) {
  constexpr int EPV = Vec16<QT>::N;
  const Geometry& g = a.g;
  const int b = blockIdx.z, head = blockIdx.y;
  const int64_t delta = a.delta[b];
  if (delta == 0) return;  // uniform per workgroup
  const int pt = g.dt / 2;
  const int chunks = (g.dt + EPV - 1) / EPV;  // 16-byte chunks holding time dims
  __shared__ float2 tab[kMaxAxisPairs];
  if (int(threadIdx.x) < pt) tab[threadIdx.x] = rope_cos_sin(delta, a.omega_t[threadIdx.x]);
  __syncthreads();
  const int64_t r0 = int64_t(blockIdx.x) * kRefreshRows;
  const int nrows = int(min<int64_t>(kRefreshRows, g.rows_pad - r0));
  QT* base = static_cast<QT*>(a.cache_k) + ((int64_t(b) * g.H + head) * g.rows_pad + r0) * D;
  // kU chunks per thread at a time: all their loads go out before the first
  // rotation and store (a load cannot pass a store through the same
  // pointer, so chunk by chunk each would wait a full memory latency)
  constexpr int kU = 8;
  const int n = nrows * chunks;
  for (int i0 = threadIdx.x; i0 < n; i0 += kU * 256) {
    uint4 raw[kU];
    uint4* ptr[kU];
    int cc[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(i0 + u * 256, n - 1);  // past the end: load a valid chunk, store nothing
      const int r = i / chunks, c = i - (i / chunks) * chunks;
      cc[u] = c;
      ptr[u] = reinterpret_cast<uint4*>(base + int64_t(r) * D + c * EPV);
      raw[u] = *ptr[u];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (i0 + u * 256 >= n) break;
      float x[EPV];
      unpack16<QT>(raw[u], x);
#pragma unroll
      for (int e = 0; e < EPV / 2; ++e) {
        // pairs past the time dims keep their values (a select, not a
        // branch: lanes of one wave hold different chunks)
        const int j = cc[u] * (EPV / 2) + e;
        const bool on = j < pt;
        const float2 t = tab[on ? j : 0];
        const float uu = x[2 * e], v = x[2 * e + 1];
        x[2 * e] = on ? uu * t.x + v * t.y : uu;
        x[2 * e + 1] = on ? v * t.x - uu * t.y : v;
      }
      *ptr[u] = pack16<QT>(x);
    }
  }
}

template <typename QT, int D>
hipError_t launch_rope_refresh_t(const RefreshArgs& a, hipStream_t s) {
  dim3 grid(unsigned((a.g.rows_pad + kRefreshRows - 1) / kRefreshRows), a.g.H, a.g.B);
  hipLaunchKernelGGL((rope_refresh_kernel<QT, D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename QT>
hipError_t launch_rope_refresh_d(const RefreshArgs& a, hipStream_t s) {
  if (a.g.D == 128) return launch_rope_refresh_t<QT, 128>(a, s);
  return launch_rope_refresh_t<QT, 64>(a, s);
}

template <typename T, typename QT, int D>
hipError_t launch_rope_append_t(const RopeArgs& a, hipStream_t s) {
  const int tiles_per_frame = (a.g.P + kTokTile - 1) / kTokTile;
  dim3 grid(tiles_per_frame * a.g.H, a.n_frames, a.g.B);
  const bool all = a.q_in && a.q_out && a.k_in && a.v_in && a.cache_k && a.rotate_k;
  if (all)
    hipLaunchKernelGGL((rope_append_kernel<T, QT, D, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((rope_append_kernel<T, QT, D, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, typename QT>
hipError_t launch_rope_append_d(const RopeArgs& a, hipStream_t s) {
  if (a.g.D == 128) return launch_rope_append_t<T, QT, 128>(a, s);
  return launch_rope_append_t<T, QT, 64>(a, s);
}

}  // namespace

hipError_t launch_rope_append(const RopeArgs& a, hipStream_t s) {
  if (a.g.dtype == SCV_BF16) {
    if (a.g.qk_dtype == SCV_FP16) return launch_rope_append_d<__bf16, _Float16>(a, s);
    return launch_rope_append_d<__bf16, __bf16>(a, s);
  }
  return launch_rope_append_d<float, float>(a, s);
}

hipError_t launch_rope_refresh(const RefreshArgs& a, hipStream_t s) {
  if (a.g.qk_dtype == SCV_FP16) return launch_rope_refresh_d<_Float16>(a, s);
  if (a.g.qk_dtype == SCV_BF16) return launch_rope_refresh_d<__bf16>(a, s);
  return launch_rope_refresh_d<float>(a, s);
}

hipError_t launch_rope_tables(const Geometry& g, const Omegas& om, const int64_t* t0, int32_t n_frames, float* out_t,
                              float2* out_h, float2* out_w, hipStream_t s) {
  TableArgs a{};
  a.g = g;
  a.om = om;
  a.n_frames = n_frames;
  if (t0)
    for (int b = 0; b < g.B; ++b) a.t0[b] = t0[b];
  a.out_t = reinterpret_cast<float2*>(out_t);
  a.out_h = out_h;
  a.out_w = out_w;
  const int64_t total = (out_t ? int64_t(g.B) * n_frames * (g.dt / 2) : 0) + int64_t(g.grid_h) * (g.dh / 2) +
                        int64_t(g.grid_w) * (g.dw / 2);
  const int blocks = int(std::min<int64_t>((total + 255) / 256, 1024));
  hipLaunchKernelGGL(rope_tables_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cache_reset(const Geometry& g, void* kv_base, size_t kv_bytes, int64_t* stamps, hipStream_t s) {
  const int64_t n16 = int64_t(kv_bytes / 16);
  const int blocks = int(std::min<int64_t>((n16 + 255) / 256, 4096));
  hipLaunchKernelGGL(cache_reset_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, s, static_cast<uint4*>(kv_base),
                     n16, stamps, int64_t(g.B) * g.n_slots);
  return hipGetLastError();
}

}  // namespace scv
