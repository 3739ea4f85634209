// QKV projection with the 3D RoPE and the cache append fused into its
// epilogue (gfx950): q, k, v = x W^T for the new frames, q rotated into
// q_rot, k rotated and v written straight into their ring slots.
//
// The fusion of the projection with Causal-RoPE into one kernel follows
// "Accelerating Video Generation Inference with Sequential-Parallel 3D
// Positional Encoding Using a Global Time Index" (section 2(c), operator
// fusion); RoPE and the slot rule are those of rope_append.hip.  Compared
// with a projection followed by rope3d_append, q, k and v never travel
// through HBM between the two.
//
// GEMM: C = x W^T with M = tokens of one stream, N = 3*H*D features, K =
// d_model.  A workgroup computes two feature blocks of D features (two
// heads of q, k or v) for 256 or 384 tokens; 8 waves (two per SIMD) of 64
// or 96 tokens x D features, fp32 accumulators, 32x32x16 bf16 MFMA.  Both
// operands are K-contiguous in memory (x rows, weight rows) and move global
// -> LDS with the 16-byte direct loads of gfx950 into two stages of 64-deep
// K slices (80 KB, or 64 KB, at D = 128): slice kt+1 loads while slice kt is
// computed (its loads spread over the first MFMA groups), one barrier per
// slice; inside a slice each fragment is read one MFMA group ahead of its
// use.  Workgroups are ordered in bands of token tiles so that the ones an
// XCD runs at once share their x and weight slices in its L2.  A slice row
// is 128 bytes, one whole cache line of x or of the weight per load
// (32-deep slices, half lines, measured 3-7% slower); a d_model that is an
// odd multiple of 32 ends with a 32-deep slice.  The 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7),
// which puts any 16 consecutive rows of a fragment read on distinct banks.
// For q and k the MFMA computes C^T (features as rows) so that each lane
// holds the dim pairs (2j, 2j+1) of one token, which RoPE rotates in
// registers; for v it computes C (tokens as rows) so that each lane holds 4
// consecutive tokens of one feature.
// Epilogue: once every wave is done with the ring, it holds the RoPE
// tables (time pairs of the tile's frames computed from fp64 angles, copies
// of the height and width tables), so that every cos/sin comes from LDS, the
// ring row base of each of the tile's frames, and one staging area per wave: a wave rotates and rounds a 32-token block,
// writes it into its area and reads it back as 16-byte pieces of whole rows
// (a token's D features for q and k, 8 consecutive tokens of one feature for
// the transposed value cache), so that the stores leave in contiguous
// 64-byte or longer runs instead of 8-byte pieces scattered over 32 rows.
#include <type_traits>

#include "scv_internal.h"

namespace scv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kQK = 64;        // reduction depth of one LDS slice
constexpr int kQTokGroups = 4; // waves per feature block
constexpr int kBand = 6;       // token tiles per band of the workgroup order
constexpr int kSpread = 8;     // MFMA groups over which a slice's loads are issued

__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(lds_base), "v"(voff), "s"(base) : "m0", "memory");
}
// a pointer every lane holds the same value of, in scalar registers (the
// direct-to-LDS loads take their base address from an SGPR pair)
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// byte offset of 16-byte chunk c of row r in a slice (128-byte rows)
__device__ __forceinline__ int slice_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// fp32 -> T (round to nearest even).  fp16 saturates: a value beyond the
// largest finite fp16 is stored as +-65504 instead of +-inf, so rotated keys
// stay finite and the attention over them stays defined.
template <typename T>
__device__ __forceinline__ uint16_t bits16(float x) {
  if constexpr (std::is_same<T, _Float16>::value) x = __builtin_amdgcn_fmed3f(x, -65504.f, 65504.f);
  return __builtin_bit_cast(uint16_t, static_cast<T>(x));
}

// One workgroup: 128*TB tokens of one stream x two feature blocks of D
// features (two heads of q, k or v; the blocks may belong to different
// ones); 8 waves, two per SIMD, so that one wave's MFMAs cover the other's
// waits; each wave computes 32*TB tokens of one block (the two waves of a
// SIMD: the same block, token groups wq and wq + 2).  TB = 3 (384 tokens,
// 160 KB of LDS) gives fewer, larger workgroups than TB = 2 (256 tokens);
// the host picks the one whose grid fills the chip better.
// (4 waves of 128x128 tiles -- half the LDS bytes per MFMA -- measured 1.5x
// slower: a lone wave per SIMD stalls on its own loads.)
template <typename QT, int D, int TB>
__global__ __launch_bounds__(512, 1) void qkv_rope_kernel(QkvArgs a) {
  constexpr int kQM = 32 * TB * kQTokGroups;   // tokens per workgroup
  constexpr int kQStages = 2;
  constexpr int kTokGroups = kQTokGroups;
  constexpr int kQWaves = 2 * kTokGroups;
  constexpr int kThreads = 64 * kQWaves;
  constexpr int XB = kQM * kQK * 2;            // x slice bytes
  constexpr int WB = 2 * D * kQK * 2;          // weight slice bytes (two blocks)
  constexpr int STAGE = XB + WB;
  constexpr int X_DMA = XB / 1024 / kQWaves;   // 1 KB loads per wave per stage
  constexpr int W_DMA = WB / 1024 / kQWaves;
  constexpr int DMA = X_DMA + W_DMA;
  constexpr int DB = D / 32;
  static_assert(X_DMA >= 1 && W_DMA >= 1, "tile sizes");
  __shared__ __attribute__((aligned(1024))) char smem[kQStages * STAGE];

  const Geometry& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the two waves of a SIMD (w, w + 4) share a feature block and take token
  // groups wq and wq + 2, so that in a workgroup with few tokens (the last
  // token tile) the busy waves spread over the SIMDs
  const int grp = wave % 2, wq = wave / 2;  // feature block, token group
  const int hl = lane >> 5, l32 = lane & 31;
  // Workgroups go to the 8 XCDs round robin; renumber them so that each
  // XCD runs a contiguous range of logical tiles, ordered in bands of
  // kBand token tiles (token tile fastest within a band, then feature pair,
  // then band, then stream): the ~32 workgroups an XCD runs at once cover a
  // compact block of token tiles x feature pairs, whose x and weight slices
  // its L2 serves to all of them.
  int mt, fpair, b;
  {
    const int nx = gridDim.x, ny = gridDim.y, n = nx * ny * gridDim.z;
    const int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const int xcd = id % 8, k = id / 8;
    const int base = n / 8, extra = n % 8;
    const int logical = xcd * base + min(xcd, extra) + k;
    b = logical / (nx * ny);
    const int r = logical - b * (nx * ny);
    const int band = r / (kBand * ny), first = band * kBand;
    const int width = min(kBand, nx - first);  // the last band may be narrower
    const int q = r - band * (kBand * ny);
    mt = first + q % width;
    fpair = q / width;
  }
  const int n_blocks = 3 * g.H;
  const int fb0 = 2 * fpair;
  const int fb = fb0 + grp;                  // this wave's feature block
  const bool fb_valid = fb < n_blocks;
  const int sel = fb / g.H, head = fb - sel * g.H;  // 0: q, 1: k, 2: v
  const int Ntok = a.n_frames * g.P;
  const int m0 = mt * kQM;
  // a wave whose feature block does not exist or whose tokens all lie past
  // the end skips its MFMAs and epilogue, keeping its loads and barriers
  const bool busy = fb_valid && m0 + 32 * TB * wq < Ntok;
  const int Dm = a.d_model;
  const int f_lo = m0 / g.P;
  const int pt = g.dt / 2, pth = (g.dt + g.dh) / 2;

  // ---- global -> LDS slices ----
  // Piece (wave * X_DMA + j) * 64 + lane of a stage's x part is 16-byte
  // chunk c of row r = piece / 8, stored at chunk position
  // (lane % 8) = c ^ ((r / 2) % 8), so c = c0 ^ (4 * (piece / 64 % 2)) with
  // c0 = (lane % 8) ^ (lane / 16); the weight part likewise.  Offsets are
  // recomputed for every slice from two lane values, which keeps ten
  // registers free for the fragment pipeline below.
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  const char* const xs = uniform_ptr(static_cast<const char*>(a.x) + int64_t(b) * Ntok * Dm * 2);
  const char* const ws = uniform_ptr(static_cast<const char*>(a.w) + int64_t(fb0) * D * Dm * 2);
  const int w_rows = min(2, n_blocks - fb0) * D;  // weight rows that exist
  const int n_full = Dm / kQK;              // 64-deep slices
  const bool half_tail = Dm % kQK != 0;     // then one more, 32 deep
  // LDS: the x stages [2][XB], then the weight stages [2][WB], so that every
  // fragment read reaches its stage with an immediate offset below 64 KB
  // load j (0 <= j < DMA) of this wave for slice kt into stage stg: x
  // pieces first, then weight pieces; lrow = lane / 8 and c0 come in
  // through an empty asm per slice
  auto issue_one = [&](int kt, int stg, int j, int lrow, int c0) __attribute__((always_inline)) {
    const int64_t k0 = int64_t(kt) * kQK * 2;
    // the 32-deep slice: second-half chunks (c >= 4) repeat the first half
    const bool tail = kt == n_full;
    if (j < X_DMA) {
      const int blk = wave * X_DMA + j;
      const int c = c0 ^ ((blk & 1) << 2);
      const int tok = min(m0 + blk * 8 + lrow, Ntok - 1);  // rows past the last token repeat it (outputs dropped)
      const uint32_t off = uint32_t(tok) * uint32_t(Dm * 2) + uint32_t(c << 4) - (tail ? uint32_t(c >> 2) << 6 : 0u);
      dma16(xs + k0, off, lds0 + uint32_t(stg * XB + blk * 1024));
    } else {
      const int blk = wave * W_DMA + (j - X_DMA);
      const int c = c0 ^ ((blk & 1) << 2);
      const int rr = min(blk * 8 + lrow, w_rows - 1);  // a missing second block repeats the last row (unused)
      const uint32_t off = uint32_t(rr) * uint32_t(Dm * 2) + uint32_t(c << 4) - (tail ? uint32_t(c >> 2) << 6 : 0u);
      dma16(ws + k0, off, lds0 + uint32_t(2 * XB + stg * WB + blk * 1024));
    }
  };
  auto lane_parts = [&](int& lrow, int& c0) __attribute__((always_inline)) {
    lrow = lane >> 3;
    c0 = (lane & 7) ^ (lane >> 4);
    asm volatile("" : "+v"(lrow));
    asm volatile("" : "+v"(c0));
  };
  auto issue = [&](int kt, int stg) __attribute__((always_inline)) {
    int lrow, c0;
    lane_parts(lrow, c0);
#pragma unroll
    for (int j = 0; j < DMA; ++j) issue_one(kt, stg, j, lrow, c0);
  };

  floatx16_t acc[DB * TB];
#pragma unroll
  for (int i = 0; i < DB * TB; ++i) acc[i] = floatx16_t{};

  // this lane's fragment offsets in stage 0 for step kk = 0 (chunk hl of its
  // row); step kk reads chunk 2*kk + hl, at offset ^ (kk * 32) since the
  // swizzle is an XOR; a 32-row block adds 4096 bytes, a stage XB or WB
  int xoff = slice_off(32 * TB * wq + l32, hl);
  int woff = 2 * XB + slice_off(D * grp + l32, hl);

  // Fragment pipeline: a wave's 16-deep step is DB groups of TB MFMAs, one
  // group per weight fragment.  The read of the next group's weight
  // fragment (and, in the last group, of the next step's x fragments) is
  // issued before the current group's MFMAs, so its LDS latency hides
  // behind them instead of stalling the wave; the SIMD's other wave covers
  // what is left.  Every wave passes the same barriers; the MFMA operand
  // order (C^T for q and k, C for v) is per wave.
  auto gemm = [&](auto trans_tag) {
    constexpr bool kTrans = decltype(trans_tag)::value;  // C^T: features as rows
    auto group = [&](const bf16x8_t (&x)[TB], const bf16x8_t& w, int db) __attribute__((always_inline)) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if constexpr (kTrans)
          acc[db * TB + tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, x[tb], acc[db * TB + tb], 0, 0, 0);
        else
          acc[db * TB + tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[tb], w, acc[db * TB + tb], 0, 0, 0);
      }
    };
    const int n_k = n_full + (half_tail ? 1 : 0);
    // two stages: slice kt+1 loads while slice kt is computed
    issue(0, 0);
    if (n_k > 1) issue(1, 1);
    // slice kt (in stage kt % 2) with NKK 16-deep steps: one instance for
    // the 64-deep slices, one for a 32-deep tail
    auto slice = [&](auto nkk_c, int kt) __attribute__((always_inline)) {
      constexpr int NKK = decltype(nkk_c)::value;
      const int stg = kt & 1;
      // the offsets pass through an empty asm each slice, so that the step
      // offsets are formed anew (one XOR each; stages and blocks are
      // multiples of 1 KB, which the XOR leaves alone) and block offsets
      // become read immediates, instead of all being hoisted out of the
      // loop into registers
      int xo = xoff + stg * XB, wo = woff + stg * WB;
      asm volatile("" : "+v"(xo));
      asm volatile("" : "+v"(wo));
      auto read_x = [&](int kk, bf16x8_t (&x)[TB]) __attribute__((always_inline)) {
        const int o = xo ^ (kk << 5);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) x[tb] = *reinterpret_cast<const bf16x8_t*>(smem + o + tb * 4096);
      };
      auto read_w = [&](int kk, int db) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8_t*>(smem + (wo ^ (kk << 5)) + db * 4096);
      };
      if (kt == 0 && n_k > 1)
        wait_vm<DMA>();
      else
        wait_vm<0>();
      __syncthreads();  // slice kt landed everywhere; slice kt-1 is done everywhere
      // slice kt+1's loads (into the stage slice kt-1 used) are spread over
      // the first kSpread groups, so that a wave never stalls on issuing
      // them all at once behind the other waves' loads
      const bool load_next = kt >= 1 && kt + 1 < n_k;
      if (!busy) {
        if (load_next) issue(kt + 1, stg ^ 1);
        return;
      }
      int lrow = 0, c0 = 0;
      if (load_next) lane_parts(lrow, c0);
      bf16x8_t x[2][TB], w[2];
      read_x(0, x[0]);
      w[0] = read_w(0, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int cur = (kk * DB + db) & 1;
          const int grp_i = kk * DB + db;
          if (NKK == 4 && grp_i < kSpread && load_next) {
#pragma unroll
            for (int j = grp_i * DMA / kSpread; j < (grp_i + 1) * DMA / kSpread; ++j) issue_one(kt + 1, stg ^ 1, j, lrow, c0);
          }
          // the reads first, then the group's MFMAs; the next step's x
          // fragments two groups ahead of their first use
          if (db + 2 == DB && kk + 1 < NKK) {
            read_x(kk + 1, x[(kk + 1) & 1]);
            w[cur ^ 1] = read_w(kk, db + 1);
            __builtin_amdgcn_sched_group_barrier(0x100, TB + 1, 0);
          } else if (db + 1 < DB) {
            w[cur ^ 1] = read_w(kk, db + 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          } else if (kk + 1 < NKK) {
            w[cur ^ 1] = read_w(kk + 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          group(x[kk & 1], w[cur], db);
          __builtin_amdgcn_sched_group_barrier(0x008, TB, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int kt = 0; kt < n_full; ++kt) slice(std::integral_constant<int, 4>{}, kt);
    if (half_tail) slice(std::integral_constant<int, 2>{}, n_full);
  };

  const int64_t t0 = a.t0[b];
  auto slot_of = [&](int f) -> int64_t {
    const int64_t gf = t0 + f;
    return gf < g.S_f ? gf : g.S_f + gf % g.R;
  };

  if (sel < 2)
    gemm(std::true_type{});
  else
    gemm(std::false_type{});

  // ---- after the K loop the ring holds, from its start, the RoPE tables
  // (cos/sin of the time pairs of the frames this tile spans, computed from
  // fp64 angles, then copies of the height and width tables), the ring row
  // base of each of those frames, and, at its end, one staging area per wave
  // through which the outputs leave in whole 16-byte pieces of contiguous
  // rows.  The host checks that the tables fit (qkv_table_bytes). ----
  constexpr int kStageOut = 32 * D * 2;  // one 32-token x D block
  constexpr int kOutBase = qkv_table_capacity(D, TB);
  static_assert(kOutBase + kQWaves * kStageOut == kQStages * STAGE, "epilogue layout");
  float2* tab = reinterpret_cast<float2*>(smem);
  char* outst = smem + kOutBase + wave * kStageOut;  // this wave's staging area
  const int dh2 = g.dh / 2, dw2 = g.dw / 2;
  const int f_hi = (min(m0 + kQM, Ntok) - 1) / g.P;
  const int nf = f_hi - f_lo + 1;  // frames the tile spans
  const int h_base = nf * pt, w_base = h_base + g.grid_h * dh2;
  // ring row of token t of frame f (frame-relative to the call) is
  // row_base[f - f_lo] + t
  int* row_base = reinterpret_cast<int*>(tab + w_base + g.grid_w * dw2);
  __syncthreads();  // every wave is done with the ring
  for (int i = tid; i < nf * pt; i += kThreads) {
    const int fi = i / pt, j = i - fi * pt;
    tab[i] = rope_cos_sin(t0 + f_lo + fi - a.pos_off[b], a.omega_t[j]);
  }
  for (int i = tid; i < g.grid_h * dh2; i += kThreads) tab[h_base + i] = a.tab_h[i];
  for (int i = tid; i < g.grid_w * dw2; i += kThreads) tab[w_base + i] = a.tab_w[i];
  for (int i = tid; i < nf; i += kThreads)
    row_base[i] = int(slot_of(f_lo + i) * g.slot_rows - int64_t(f_lo + i) * g.P);
  __syncthreads();
  if (!busy) return;
  // t / P and p / grid_w through a float reciprocal and one correction step
  // (exact: tokens per call stay below 2^24, so the estimate is off by at
  // most one)
  const float inv_p = 1.0f / float(g.P), inv_w = 1.0f / float(g.grid_w);
  auto div_fix = [](int n, int d, float inv, int& q, int& r) __attribute__((always_inline)) {
    q = int(float(n) * inv);
    r = n - q * d;
    if (r < 0) {
      --q;
      r += d;
    } else if (r >= d) {
      ++q;
      r -= d;
    }
  };

  if (sel < 2) {
    // lane: token 32TB*wq + 32tb + l32 of the tile; dims 32db + 8e + 4hl + 0..3,
    // that is pairs j = 16db + 4e + 2hl + 0..1.  Staging: [32 tokens][D],
    // 16-byte chunk c of row r at c ^ (r % kChunks).
    constexpr int kChunks = D / 8;
    QT* const out_base = sel == 0 ? static_cast<QT*>(a.q_out) + (int64_t(b) * Ntok * g.H + head) * D
                                  : static_cast<QT*>(a.cache_k) + (int64_t(b) * g.H + head) * g.rows_pad * D;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int tile0 = m0 + 32 * TB * wq + 32 * tb;  // first token of this block
      {
        const int t = min(tile0 + l32, Ntok - 1);  // rows past the last token are computed but not stored
        int f, p, yy, xx;
        div_fix(t, g.P, inv_p, f, p);
        div_fix(p, g.grid_w, inv_w, yy, xx);
        // table entry of pair j: j + (time, height or width base)
        const int bt = (f - f_lo) * pt, bh = h_base + yy * dh2 - pt, bw = w_base + xx * dw2 - pth;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[db * TB + tb][4 * e + i];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const int j = 16 * db + 4 * e + 2 * hl + pp;
              const float2 cs = tab[j + (j < pt ? bt : (j < pth ? bh : bw))];
              const float u = v[2 * pp], w = v[2 * pp + 1];
              v[2 * pp] = u * cs.x - w * cs.y;
              v[2 * pp + 1] = u * cs.y + w * cs.x;
            }
            uint2 o;
            o.x = uint32_t(bits16<QT>(v[0])) | (uint32_t(bits16<QT>(v[1])) << 16);
            o.y = uint32_t(bits16<QT>(v[2])) | (uint32_t(bits16<QT>(v[3])) << 16);
            const int c = (4 * db + e) ^ (l32 % kChunks);
            *reinterpret_cast<uint2*>(outst + l32 * (D * 2) + c * 16 + hl * 8) = o;
          }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");  // the block is in LDS (this wave only)
      // read back 16 bytes of one row per lane: rows r = (64 / kChunks) n + lane / kChunks
#pragma unroll
      for (int n = 0; n < 32 * kChunks / 64; ++n) {
        const int r = n * (64 / kChunks) + lane / kChunks, c = lane % kChunks;
        const uint4 val = *reinterpret_cast<const uint4*>(outst + r * (D * 2) + ((c ^ (r % kChunks)) << 4));
        const int t = tile0 + r;
        if (t < Ntok) {
          int64_t row;
          if (sel == 0) {
            row = int64_t(t) * g.H;
          } else {
            int f, p;
            div_fix(t, g.P, inv_p, f, p);
            row = row_base[f - f_lo] + t;
          }
          *reinterpret_cast<uint4*>(out_base + row * D + c * 8) = val;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");  // reads done before the next block overwrites
    }
  } else {
    // lane: feature 32db + l32; tokens 32TB*wq + 32tb + 8e + 4hl + 0..3.
    // Staging: [D features][32 tokens], 64-byte rows, 16-byte chunk c (8
    // tokens) of row r at c ^ ((r / 4) % 4); each row then leaves as 8-token
    // pieces, one 16-byte store where the 8 tokens are 16-byte aligned in one
    // frame, else token by token.
    uint16_t* vt = static_cast<uint16_t*>(a.cache_v) + (int64_t(b) * g.H + head) * D * g.rows_pad;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int tile0 = m0 + 32 * TB * wq + 32 * tb;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const floatx16_t& c = acc[db * TB + tb];
          uint2 o;
          o.x = uint32_t(bits16<__bf16>(c[4 * e])) | (uint32_t(bits16<__bf16>(c[4 * e + 1])) << 16);
          o.y = uint32_t(bits16<__bf16>(c[4 * e + 2])) | (uint32_t(bits16<__bf16>(c[4 * e + 3])) << 16);
          const int r = 32 * db + l32;
          *reinterpret_cast<uint2*>(outst + r * 64 + ((e ^ ((r >> 2) & 3)) << 4) + hl * 8) = o;
        }
      // this lane's 8 tokens (the same in every row it stores)
      const int t = tile0 + 8 * (lane & 3);
      int f, p;
      div_fix(min(t, Ntok - 1), g.P, inv_p, f, p);
      const bool whole = (p & 7) == 0 && p + 7 < g.P && t + 7 < Ntok;
      const int row0 = t < Ntok ? row_base[f - f_lo] + t : 0;
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#pragma unroll
      for (int n = 0; n < D * 4 / 64; ++n) {
        const int r = 16 * n + (lane >> 2), c = lane & 3;
        const uint4 val = *reinterpret_cast<const uint4*>(outst + r * 64 + ((c ^ ((r >> 2) & 3)) << 4));
        if (t >= Ntok) continue;
        uint16_t* vrow = vt + int64_t(r) * g.rows_pad;
        if (whole) {
          *reinterpret_cast<uint4*>(vrow + row0) = val;
        } else {
          const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (t + i < Ntok) {
              int fi, pi;
              div_fix(t + i, g.P, inv_p, fi, pi);
              vrow[row_base[fi - f_lo] + t + i] = uint16_t(w4[i / 2] >> (16 * (i & 1)));
            }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    }
    // stamps: the frames whose first token lies in this tile (one writer:
    // the wave group holding v head 0)
    if (head == 0 && wq == 0 && lane == 0) {
      for (int f = (m0 + g.P - 1) / g.P; f * g.P < min(m0 + kQM, Ntok); ++f)
        a.stamps[int64_t(b) * g.n_slots + slot_of(f)] = t0 + f;
    }
  }
}

template <typename QT, int D, int TB>
hipError_t launch_qkv_t(const QkvArgs& a, hipStream_t s) {
  const int ntok = a.n_frames * a.g.P;
  const int qm = 32 * TB * kQTokGroups;
  dim3 grid(unsigned((ntok + qm - 1) / qm), unsigned((3 * a.g.H + 1) / 2), unsigned(a.g.B));
  hipLaunchKernelGGL((qkv_rope_kernel<QT, D, TB>), grid, dim3(512), 0, s, a);
  return hipGetLastError();
}

template <typename QT, int D>
hipError_t launch_qkv_d(const QkvArgs& a, hipStream_t s) {
  return a.token_tile == 384 ? launch_qkv_t<QT, D, 3>(a, s) : launch_qkv_t<QT, D, 2>(a, s);
}

}  // namespace

hipError_t launch_qkv_rope(const QkvArgs& a, hipStream_t s) {
  const bool f16 = a.g.qk_dtype == SCV_FP16;
  if (a.g.D == 128) return f16 ? launch_qkv_d<_Float16, 128>(a, s) : launch_qkv_d<__bf16, 128>(a, s);
  return f16 ? launch_qkv_d<_Float16, 64>(a, s) : launch_qkv_d<__bf16, 64>(a, s);
}

}  // namespace scv
