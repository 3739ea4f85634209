// Block-causal chunk attention over a sink-pinned ring KV cache (gfx950).
//
// What is computed: for every query row of the new chunk, softmax attention
// (scale 1/sqrt(d)) over the cached frames it may see -- the pinned sink
// frames, the fixed-size window before its chunk, and its own chunk -- as in
// the sink-token guided rolling KV cache of "StreamDiffusionV2: A Streaming
// System for Dynamic and Interactive Video Generation" (paper-review blog,
// section 2) with causal KV-cached attention at a global time index from
// "Accelerating Video Generation Inference with Sequential-Parallel 3D
// Positional Encoding Using a Global Time Index" (sections 1 and 2).
//
// Kernel design (MI355X / CDNA4, wave64):
//  * Workgroup = 4 waves = 128 query rows of one (stream, head[, key split]);
//    each wave owns 32 query rows for the whole key loop.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
//    wave's Q held in VGPRs).  In the accumulator each lane then holds one
//    query column and 16 of every 32 keys, so the row max / row sum need a
//    single exchange with lane ^ 32, and P^T (rounded to bf16) is directly
//    the B operand of O^T += V^T P^T -- no LDS round trip for P.
//  * V is stored transposed in the cache ([d][row]); staging permutes keys
//    inside each 16-key group as 0-3,8-11 | 4-7,12-15 so that the V^T A
//    operand of each lane is one 16-byte LDS read matching P^T's key order.
//  * K and V^T tiles (64 keys) are double-buffered in LDS with XOR chunk
//    swizzles; global loads for tile i+1 are issued before the MFMAs of tile
//    i and written to LDS after them, one barrier per tile.
//  * Online softmax in fp32 with exp2 (scale * log2 e folded into one FMA).
//  * Frame visibility is evaluated once per workgroup from the slot stamps;
//    tiles no query of the workgroup may see are skipped, fully visible
//    tiles run unmasked, others are masked per key.
//  * Optional key splits write normalised fp32 partials + lse, combined by
//    attn_merge (lse-weighted).
// An fp32 instantiation (v_mfma_f32_32x32x2_f32) follows the same structure.
#include "scv_internal.h"

namespace scv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kBlockM = 32 * kWaves;  // query rows per workgroup
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Frame-slot visibility masks per query chunk, the workgroup's union and
// intersection, and per-key classification.
struct Visibility {
  uint64_t any;  // slots some query of the workgroup may see
  uint64_t all;  // slots every query of the workgroup may see
  uint64_t mine; // slots this lane's query may see
};

__device__ __forceinline__ uint64_t tile_slot_bits(const Geometry& g, int t) {
  const int64_t r0 = int64_t(t) * kKeyTile;
  if (r0 >= g.rows) return 0;
  const int s_lo = int(r0 / g.slot_rows);
  const int s_hi = int(min(r0 + kKeyTile - 1, g.rows - 1) / g.slot_rows);
  const uint64_t hi = s_hi >= 63 ? ~uint64_t(0) : ((uint64_t(1) << (s_hi + 1)) - 1);
  return hi & ~((uint64_t(1) << s_lo) - 1);
}

// Branch-free per-key visibility (rows < 2^31: at most 64 slots of <= 2^20
// rows).  Evaluated with bitwise ands and applied with a select, so no
// per-element divergent branch reaches the accumulator registers.
__device__ __forceinline__ bool key_visible(const Geometry& g, uint64_t mask, int row) {
  const int slot_rows = int(g.slot_rows);
  const int slot = row / slot_rows;
  const int p = row - slot * slot_rows;
  const uint32_t in_rows = row < int(g.rows);
  const uint32_t in_slot = p < g.P;
  const uint32_t seen = uint32_t(mask >> (slot & 63)) & 1u;
  return (in_rows & in_slot & seen) != 0;
}

template <int ROWS_PER_WG>
__device__ __forceinline__ Visibility compute_visibility(const AttnArgs& a, int b, int qtile, int qrow, bool qvalid,
                                                         uint64_t* vis_mask) {
  const Geometry& g = a.g;
  const int n_chunks = (a.n_frames + g.C - 1) / g.C;
  const int64_t t0 = a.t0[b];
  if (int(threadIdx.x) < n_chunks) {
    const int64_t s_c = t0 + int64_t(threadIdx.x) * g.C;
    uint64_t m = 0;
    for (int s = 0; s < g.n_slots; ++s) {
      const int64_t st = a.stamps[int64_t(b) * g.n_slots + s];
      if (st >= 0 && st < s_c + g.C && (st < g.S_f || st >= s_c - g.W)) m |= uint64_t(1) << s;
    }
    vis_mask[threadIdx.x] = m;
  }
  __syncthreads();
  const int rows_per_chunk = g.P * g.C;
  const int row_lo = qtile * ROWS_PER_WG;
  const int row_hi = min(row_lo + ROWS_PER_WG, a.Nq) - 1;
  Visibility v;
  v.any = 0;
  v.all = ~uint64_t(0);
  for (int c = row_lo / rows_per_chunk; c <= row_hi / rows_per_chunk; ++c) {
    v.any |= vis_mask[c];
    v.all &= vis_mask[c];
  }
  v.mine = vis_mask[qvalid ? qrow / rows_per_chunk : row_lo / rows_per_chunk];
  return v;
}

// ---------------------------------------------------------------------------
// bf16 inputs, fp32 accumulation
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void chunk_attn_bf16_kernel(AttnArgs a) {
  constexpr int CH = D / 8;                  // 16-byte chunks per key row
  constexpr int KROW = D * 2;                // bytes per key row
  constexpr int KBYTES = kKeyTile * KROW;
  constexpr int VROW = kKeyTile * 2;         // bytes per V^T row (64 keys)
  constexpr int K_LOADS = kKeyTile * CH / 256;
  constexpr int V_PAIRS = D * 4 / 256;       // (2 x 16 B) per thread per tile
  constexpr int KS = D / 16;                 // k-steps of QK^T
  constexpr int DB = D / 32;                 // 32-row blocks of O^T
  static_assert(K_LOADS >= 1 && V_PAIRS >= 1, "tile sizes");

  __shared__ __attribute__((aligned(16))) char smem[2][KBYTES + D * VROW];
  __shared__ uint64_t vis_mask[kMaxQueryChunks];

  const Geometry& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int qtile = blockIdx.x, head = blockIdx.y;
  const int b = blockIdx.z / a.splits, split = blockIdx.z % a.splits;
  const int qrow = qtile * kBlockM + wave * 32 + l32;
  const bool qvalid = qrow < a.Nq;

  const Visibility vis = compute_visibility<kBlockM>(a, b, qtile, qrow, qvalid, vis_mask);

  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(t_begin + a.tiles_per_split, a.tiles_total);
  auto next_tile = [&](int t) {
    while (t < t_end && (tile_slot_bits(g, t) & vis.any) == 0) ++t;
    return t;
  };

  // Q^T operand: lane (l32, hl) holds q[qrow][16*kk + 8*hl .. +8].
  bf16x8 qf[KS];
  {
    const __bf16* qp =
        static_cast<const __bf16*>(a.q) + ((int64_t(b) * a.Nq + (qvalid ? qrow : 0)) * g.H + head) * D + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 u = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, u);
    }
  }

  floatx16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;

  const char* kbase = static_cast<const char*>(a.cache_k) + (int64_t(b) * g.H + head) * g.rows_pad * KROW;
  const char* vbase = static_cast<const char*>(a.cache_v) + (int64_t(b) * g.H + head) * D * g.rows_pad * 2;
  uint4 kreg[K_LOADS];
  uint4 vreg[V_PAIRS][2];

  auto gload = [&](int t) {
    const int64_t r0 = int64_t(t) * kKeyTile;
#pragma unroll
    for (int j = 0; j < K_LOADS; ++j) {
      const int i = tid + 256 * j, row = i / CH, c = i % CH;
      kreg[j] = *reinterpret_cast<const uint4*>(kbase + (r0 + row) * KROW + c * 16);
    }
#pragma unroll
    for (int j = 0; j < V_PAIRS; ++j) {
      const int i = tid + 256 * j, row = i >> 2, gq = i & 3;
      const char* p = vbase + int64_t(row) * g.rows_pad * 2 + (r0 + 16 * gq) * 2;
      vreg[j][0] = *reinterpret_cast<const uint4*>(p);
      vreg[j][1] = *reinterpret_cast<const uint4*>(p + 16);
    }
  };
  auto lds_store = [&](int stage) {
    char* ks = smem[stage];
    char* vs = smem[stage] + KBYTES;
#pragma unroll
    for (int j = 0; j < K_LOADS; ++j) {
      const int i = tid + 256 * j, row = i / CH, c = i % CH;
      *reinterpret_cast<uint4*>(ks + row * KROW + ((c ^ (row & (CH - 1))) * 16)) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < V_PAIRS; ++j) {
      const int i = tid + 256 * j, row = i >> 2, gq = i & 3, sw = row & 7;
      const uint4 A = vreg[j][0], Bv = vreg[j][1];
      *reinterpret_cast<uint4*>(vs + row * VROW + (((2 * gq) ^ sw) * 16)) = make_uint4(A.x, A.y, Bv.x, Bv.y);
      *reinterpret_cast<uint4*>(vs + row * VROW + (((2 * gq + 1) ^ sw) * 16)) = make_uint4(A.z, A.w, Bv.z, Bv.w);
    }
  };

  auto compute = [&](int stage, int t) {
    const char* ks = smem[stage];
    const char* vs = smem[stage] + KBYTES;
    floatx16 s0 = floatx16{}, s1 = floatx16{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int c = 2 * kk + hl;
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(ks + l32 * KROW + ((c ^ (l32 & (CH - 1))) * 16));
      const bf16x8 k1 =
          *reinterpret_cast<const bf16x8*>(ks + (32 + l32) * KROW + ((c ^ ((32 + l32) & (CH - 1))) * 16));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[kk], s1, 0, 0, 0);
    }
    // accumulator element i of lane (l32, hl) is key 8*(i/4) + 4*hl + i%4 (+32 for s1)
    const int64_t r0 = int64_t(t) * kKeyTile;
    const bool full = ((tile_slot_bits(g, t) & ~vis.all) == 0) && (r0 + kKeyTile <= g.rows) && (g.slot_rows == g.P);
    if (!full) {
      const int r0i = int(r0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i / 4) + 4 * hl + (i & 3);
        s0[i] = key_visible(g, vis.mine, r0i + key) ? s0[i] : -INFINITY;
        s1[i] = key_visible(g, vis.mine, r0i + 32 + key) ? s1[i] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float msc = (m_new == -INFINITY) ? 0.f : m_new * a.scale_log2;
    const float alpha = fast_exp2(m_run * a.scale_log2 - msc);
    float rs = 0.f;
    bf16x8 pk[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = fast_exp2(__builtin_fmaf(s0[i], a.scale_log2, -msc));
      const float p1 = fast_exp2(__builtin_fmaf(s1[i], a.scale_log2, -msc));
      rs += p0 + p1;
      pk[i / 8][i % 8] = static_cast<__bf16>(p0);
      pk[2 + i / 8][i % 8] = static_cast<__bf16>(p1);
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    // O^T += V^T P^T over 4 groups of 16 keys
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = db * 32 + l32;
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vs + row * VROW + ((((2 * g4) + hl) ^ (row & 7)) * 16));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[g4], o[db], 0, 0, 0);
      }
    }
  };

  int t = next_tile(t_begin);
  if (t < t_end) {
    gload(t);
    lds_store(0);
  }
  __syncthreads();
  int stage = 0;
  while (t < t_end) {
    const int tn = next_tile(t + 1);
    if (tn < t_end) gload(tn);
    compute(stage, t);
    if (tn < t_end) lds_store(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    t = tn;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run * a.scale_log2 + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (!qvalid) return;
  if (a.splits == 1) {
    __bf16* op = static_cast<__bf16*>(a.o) + ((int64_t(b) * a.Nq + qrow) * g.H + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * hl;
        const __bf16 v0 = static_cast<__bf16>(o[db][4 * q4 + 0] * inv);
        const __bf16 v1 = static_cast<__bf16>(o[db][4 * q4 + 1] * inv);
        const __bf16 v2 = static_cast<__bf16>(o[db][4 * q4 + 2] * inv);
        const __bf16 v3 = static_cast<__bf16>(o[db][4 * q4 + 3] * inv);
        uint2 w;
        w.x = uint32_t(__builtin_bit_cast(uint16_t, v0)) | (uint32_t(__builtin_bit_cast(uint16_t, v1)) << 16);
        w.y = uint32_t(__builtin_bit_cast(uint16_t, v2)) | (uint32_t(__builtin_bit_cast(uint16_t, v3)) << 16);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    }
    if (a.lse && hl == 0) a.lse[(int64_t(b) * g.H + head) * a.Nq + qrow] = lse_v;
  } else {
    float* pp = a.part_o + (((int64_t(split) * g.B + b) * g.H + head) * a.Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * hl;
        *reinterpret_cast<float4*>(pp + d0) = make_float4(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv,
                                                           o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv);
      }
    }
    if (hl == 0) a.part_lse[((int64_t(split) * g.B + b) * g.H + head) * a.Nq + qrow] = lse_v;
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs (v_mfma_f32_32x32x2_f32)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void chunk_attn_f32_kernel(AttnArgs a) {
  constexpr int CH = D / 4;                  // 16-byte chunks per key row
  constexpr int KROW = D * 4;
  constexpr int KBYTES = kKeyTile * KROW;
  constexpr int VROW = kKeyTile * 4;         // 256 bytes per V^T row
  constexpr int K_LOADS = kKeyTile * CH / 256;
  constexpr int V_LOADS = D * 16 / 256;
  constexpr int DB = D / 32;
  constexpr int M8 = D / 8;                  // groups of 8 head dims
  static_assert(K_LOADS >= 1 && V_LOADS >= 1, "tile sizes");

  __shared__ __attribute__((aligned(16))) char smem[2][KBYTES + D * VROW];
  __shared__ uint64_t vis_mask[kMaxQueryChunks];

  const Geometry& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int qtile = blockIdx.x, head = blockIdx.y;
  const int b = blockIdx.z / a.splits, split = blockIdx.z % a.splits;
  const int qrow = qtile * kBlockM + wave * 32 + l32;
  const bool qvalid = qrow < a.Nq;

  const Visibility vis = compute_visibility<kBlockM>(a, b, qtile, qrow, qvalid, vis_mask);
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(t_begin + a.tiles_per_split, a.tiles_total);
  auto next_tile = [&](int t) {
    while (t < t_end && (tile_slot_bits(g, t) & vis.any) == 0) ++t;
    return t;
  };

  // lane half hl owns head dims 8m + 4hl + e (m < D/8, e < 4) of the contraction
  floatx4 qf[M8];
  {
    const float* qp =
        static_cast<const float*>(a.q) + ((int64_t(b) * a.Nq + (qvalid ? qrow : 0)) * g.H + head) * D + 4 * hl;
#pragma unroll
    for (int m = 0; m < M8; ++m) {
      const float4 u = qvalid ? *reinterpret_cast<const float4*>(qp + 8 * m) : make_float4(0.f, 0.f, 0.f, 0.f);
      qf[m] = floatx4{u.x, u.y, u.z, u.w};
    }
  }
  floatx16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;

  const char* kbase = static_cast<const char*>(a.cache_k) + (int64_t(b) * g.H + head) * g.rows_pad * KROW;
  const char* vbase = static_cast<const char*>(a.cache_v) + (int64_t(b) * g.H + head) * D * g.rows_pad * 4;
  uint4 kreg[K_LOADS], vreg[V_LOADS];
  auto gload = [&](int t) {
    const int64_t r0 = int64_t(t) * kKeyTile;
#pragma unroll
    for (int j = 0; j < K_LOADS; ++j) {
      const int i = tid + 256 * j, row = i / CH, c = i % CH;
      kreg[j] = *reinterpret_cast<const uint4*>(kbase + (r0 + row) * KROW + c * 16);
    }
#pragma unroll
    for (int j = 0; j < V_LOADS; ++j) {
      const int i = tid + 256 * j, row = i >> 4, c = i & 15;
      vreg[j] = *reinterpret_cast<const uint4*>(vbase + int64_t(row) * g.rows_pad * 4 + r0 * 4 + c * 16);
    }
  };
  auto lds_store = [&](int stage) {
    char* ks = smem[stage];
    char* vs = smem[stage] + KBYTES;
#pragma unroll
    for (int j = 0; j < K_LOADS; ++j) {
      const int i = tid + 256 * j, row = i / CH, c = i % CH;
      *reinterpret_cast<uint4*>(ks + row * KROW + ((c ^ (row & (CH - 1))) * 16)) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < V_LOADS; ++j) {
      const int i = tid + 256 * j, row = i >> 4, c = i & 15;
      *reinterpret_cast<uint4*>(vs + row * VROW + ((c ^ (row & 15)) * 16)) = vreg[j];
    }
  };
  auto compute = [&](int stage, int t) {
    const char* ks = smem[stage];
    const char* vs = smem[stage] + KBYTES;
    floatx16 s[2] = {floatx16{}, floatx16{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = kb * 32 + l32;
#pragma unroll
      for (int m = 0; m < M8; ++m) {
        const int c = 2 * m + hl;
        const floatx4 kf = *reinterpret_cast<const floatx4*>(ks + row * KROW + ((c ^ (row & (CH - 1))) * 16));
#pragma unroll
        for (int e = 0; e < 4; ++e) s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[e], qf[m][e], s[kb], 0, 0, 0);
      }
    }
    const int64_t r0 = int64_t(t) * kKeyTile;
    const bool full = ((tile_slot_bits(g, t) & ~vis.all) == 0) && (r0 + kKeyTile <= g.rows) && (g.slot_rows == g.P);
    if (!full) {
      const int r0i = int(r0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kb][i] = key_visible(g, vis.mine, r0i + 32 * kb + 8 * (i / 4) + 4 * hl + (i & 3)) ? s[kb][i] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[0][i], s[1][i]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float msc = (m_new == -INFINITY) ? 0.f : m_new * a.scale_log2;
    const float alpha = fast_exp2(m_run * a.scale_log2 - msc);
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = fast_exp2(__builtin_fmaf(s[kb][i], a.scale_log2, -msc));
        rs += s[kb][i];
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int row = db * 32 + l32;
          const int c = 8 * kb + 2 * i4 + hl;
          const floatx4 vf = *reinterpret_cast<const floatx4*>(vs + row * VROW + ((c ^ (row & 15)) * 16));
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[e], s[kb][4 * i4 + e], o[db], 0, 0, 0);
        }
  };

  int t = next_tile(t_begin);
  if (t < t_end) {
    gload(t);
    lds_store(0);
  }
  __syncthreads();
  int stage = 0;
  while (t < t_end) {
    const int tn = next_tile(t + 1);
    if (tn < t_end) gload(tn);
    compute(stage, t);
    if (tn < t_end) lds_store(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    t = tn;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run * a.scale_log2 + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (!qvalid) return;
  float* dst;
  if (a.splits == 1)
    dst = static_cast<float*>(a.o) + ((int64_t(b) * a.Nq + qrow) * g.H + head) * D;
  else
    dst = a.part_o + (((int64_t(split) * g.B + b) * g.H + head) * a.Nq + qrow) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * hl;
      *reinterpret_cast<float4*>(dst + d0) = make_float4(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv,
                                                          o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv);
    }
  if (hl == 0) {
    if (a.splits == 1) {
      if (a.lse) a.lse[(int64_t(b) * g.H + head) * a.Nq + qrow] = lse_v;
    } else {
      a.part_lse[((int64_t(split) * g.B + b) * g.H + head) * a.Nq + qrow] = lse_v;
    }
  }
}

// ---------------------------------------------------------------------------
// split-KV merge: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  const Geometry& g = a.g;
  const int DG = g.D / 4;
  const int64_t total = int64_t(g.B) * g.H * a.Nq * DG;
  const int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  if (idx >= total) return;
  const int dg = int(idx % DG);
  int64_t rest = idx / DG;
  const int q = int(rest % a.Nq);
  rest /= a.Nq;
  const int h = int(rest % g.H);
  const int b = int(rest / g.H);
  const int64_t plane = int64_t(g.B) * g.H * a.Nq;  // rows per split
  const int64_t row = (int64_t(b) * g.H + h) * a.Nq + q;
  float m = -INFINITY;
  for (int s = 0; s < a.splits; ++s) m = fmaxf(m, a.part_lse[s * plane + row]);
  float lse = -INFINITY;
  if (m != -INFINITY) {
    float sum = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float l = a.part_lse[s * plane + row];
      if (l != -INFINITY) sum += __expf(l - m);
    }
    lse = m + __logf(sum);
  }
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (lse != -INFINITY) {
    for (int s = 0; s < a.splits; ++s) {
      const float l = a.part_lse[s * plane + row];
      if (l == -INFINITY) continue;
      const float w = __expf(l - lse);
      const float4 v = *reinterpret_cast<const float4*>(a.part_o + (s * plane + row) * g.D + 4 * dg);
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
  }
  T* op = static_cast<T*>(a.o) + ((int64_t(b) * a.Nq + q) * g.H + h) * g.D + 4 * dg;
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float4*>(op) = acc;
  } else {
    const __bf16 v0 = static_cast<__bf16>(acc.x), v1 = static_cast<__bf16>(acc.y);
    const __bf16 v2 = static_cast<__bf16>(acc.z), v3 = static_cast<__bf16>(acc.w);
    uint2 w;
    w.x = uint32_t(__builtin_bit_cast(uint16_t, v0)) | (uint32_t(__builtin_bit_cast(uint16_t, v1)) << 16);
    w.y = uint32_t(__builtin_bit_cast(uint16_t, v2)) | (uint32_t(__builtin_bit_cast(uint16_t, v3)) << 16);
    *reinterpret_cast<uint2*>(op) = w;
  }
  if (a.lse && dg == 0) a.lse[row] = lse;
}

}  // namespace

hipError_t launch_chunk_attention(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.n_qtiles, a.g.H, a.g.B * a.splits);
  if (a.g.dtype == SCV_BF16) {
    if (a.g.D == 128)
      hipLaunchKernelGGL(chunk_attn_bf16_kernel<128>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(chunk_attn_bf16_kernel<64>, grid, dim3(256), 0, s, a);
  } else {
    if (a.g.D == 128)
      hipLaunchKernelGGL(chunk_attn_f32_kernel<128>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(chunk_attn_f32_kernel<64>, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_merge(const MergeArgs& a, hipStream_t s) {
  const int64_t total = int64_t(a.g.B) * a.g.H * a.Nq * (a.g.D / 4);
  dim3 grid(unsigned((total + 255) / 256));
  if (a.g.dtype == SCV_BF16)
    hipLaunchKernelGGL(attn_merge_kernel<__bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_merge_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace scv
