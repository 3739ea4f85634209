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
// computed, one barrier per slice.  A slice row is 128 bytes, one whole
// cache line of x or of the weight per load (32-deep slices, half lines,
// measured 3-7% slower); a d_model that is an odd multiple of 32 ends with
// a 32-deep slice.  The 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7),
// which puts any 16 consecutive rows of a fragment read on distinct banks.
// For q and k the MFMA computes C^T (features as rows) so that each lane
// holds the dim pairs (2j, 2j+1) of one token, which RoPE rotates in
// registers; for v it computes C (tokens as rows) so that each lane holds 4
// consecutive tokens of one feature.
// Epilogue: once every wave is done with the ring, it holds the RoPE
// tables (time pairs of the tile's frames computed from fp64 angles, copies
// of the height and width tables), so that every cos/sin comes from LDS, and
// one staging area per wave: a wave rotates and rounds a 32-token block,
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

// byte offset of 16-byte chunk c of row r in a slice (64-byte rows)
__device__ __forceinline__ int slice_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// fp32 -> T (round to nearest even).  fp16 saturates: a value beyond the
// largest finite fp16 is stored as +-65504 instead of +-inf, so rotated keys
// stay finite and the attention over them stays defined.
// cos/sin of a time pair whose frame is not in the LDS table (a tile
// spanning more frames than the table holds); out of line so that the
// compiler never evaluates it speculatively on the common path
__device__ __attribute__((noinline)) float2 rope_cos_sin_slow(int64_t pos, double omega) {
  return rope_cos_sin(pos, omega);
}

template <typename T>
__device__ __forceinline__ uint16_t bits16(float x) {
  if constexpr (std::is_same<T, _Float16>::value) x = __builtin_amdgcn_fmed3f(x, -65504.f, 65504.f);
  return __builtin_bit_cast(uint16_t, static_cast<T>(x));
}

// One workgroup: 128*TB tokens of one stream x two feature blocks of D
// features (two heads of q, k or v; the blocks may belong to different
// ones); 8 waves, two per SIMD, so that one wave's MFMAs cover the other's
// waits; each wave computes 32*TB tokens of one block.  TB = 3 (384 tokens,
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
  const int grp = wave / kTokGroups, wq = wave % kTokGroups;  // feature block, token group
  const int hl = lane >> 5, l32 = lane & 31;
  // Workgroups go to the 8 XCDs round robin; renumber them so that each
  // XCD runs a contiguous range of (token tile fastest, feature pair,
  // stream): its few feature pairs' weights stay in its L2 while the token
  // tiles stream past.
  int mt, fpair, b;
  {
    const int nx = gridDim.x, ny = gridDim.y, n = nx * ny * gridDim.z;
    const int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const int xcd = id % 8, k = id / 8;
    const int base = n / 8, extra = n % 8;
    const int logical = xcd * base + min(xcd, extra) + k;
    mt = logical % nx;
    fpair = (logical / nx) % ny;
    b = logical / (nx * ny);
  }
  const int n_blocks = 3 * g.H;
  const int fb0 = 2 * fpair;
  const int fb = fb0 + grp;                  // this wave's feature block
  const bool fb_valid = fb < n_blocks;
  const int sel = fb / g.H, head = fb - sel * g.H;  // 0: q, 1: k, 2: v
  const int Ntok = a.n_frames * g.P;
  const int m0 = mt * kQM;
  const int Dm = a.d_model;
  const int f_lo = m0 / g.P;
  const int pt = g.dt / 2, pth = (g.dt + g.dh) / 2;

  // ---- global -> LDS slices (source offsets are loop invariant) ----
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  const char* xbase = static_cast<const char*>(a.x) + int64_t(b) * Ntok * Dm * 2;
  const char* wbase = static_cast<const char*>(a.w) + int64_t(fb0) * D * Dm * 2;
  const int w_rows = min(2, n_blocks - fb0) * D;  // weight rows that exist
  // hi: bit j set where load j of this lane fetches a chunk of the second
  // half of the 128-byte row piece (moved back by 64 bytes in a final
  // 32-deep slice, whose second half lies past the end of the row)
  uint32_t xo[X_DMA], wo[W_DMA], hi = 0;
#pragma unroll
  for (int j = 0; j < X_DMA; ++j) {
    const int piece = (wave * X_DMA + j) * 64 + lane, r = piece >> 3, c = (piece & 7) ^ ((r >> 1) & 7);
    const int tok = min(m0 + r, Ntok - 1);  // rows past the last token repeat it (outputs dropped)
    xo[j] = uint32_t(tok) * uint32_t(Dm * 2) + uint32_t(c << 4);
    hi |= uint32_t(c >> 2) << j;
  }
#pragma unroll
  for (int j = 0; j < W_DMA; ++j) {
    const int piece = (wave * W_DMA + j) * 64 + lane, r = piece >> 3, c = (piece & 7) ^ ((r >> 1) & 7);
    const int rr = min(r, w_rows - 1);  // a missing second block repeats the last row (unused)
    wo[j] = uint32_t(rr) * uint32_t(Dm * 2) + uint32_t(c << 4);
    hi |= uint32_t(c >> 2) << (X_DMA + j);
  }
  const int n_full = Dm / kQK;              // 64-deep slices
  const bool half_tail = Dm % kQK != 0;     // then one more, 32 deep
  // LDS: the x stages [2][XB], then the weight stages [2][WB], so that every
  // fragment read reaches its stage with an immediate offset below 64 KB
  auto issue = [&](int kt, int stg) {
    const int64_t k0 = int64_t(kt) * kQK * 2;
    const uint32_t back = kt == n_full ? hi : 0u;  // the 32-deep slice: second-half chunks repeat the first half
#pragma unroll
    for (int j = 0; j < X_DMA; ++j)
      dma16(uniform_ptr(xbase + k0), xo[j] - (((back >> j) & 1u) << 6),
            lds0 + uint32_t(stg * XB + (wave * X_DMA + j) * 1024));
#pragma unroll
    for (int j = 0; j < W_DMA; ++j)
      dma16(uniform_ptr(wbase + k0), wo[j] - (((back >> (X_DMA + j)) & 1u) << 6),
            lds0 + uint32_t(2 * XB + stg * WB + (wave * W_DMA + j) * 1024));
  };

  floatx16_t acc[DB * TB];
#pragma unroll
  for (int i = 0; i < DB * TB; ++i) acc[i] = floatx16_t{};

  // this lane's fragment offsets in stage 0 (chunk 2*kk + hl of the row); a
  // 32-row block adds 4096 bytes, a stage XB or WB
  int xoff[4], woff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    xoff[kk] = slice_off(32 * TB * wq + l32, 2 * kk + hl);
    woff[kk] = 2 * XB + slice_off(D * grp + l32, 2 * kk + hl);
  }

  // Every wave passes the same barriers; the MFMA operand order (C^T for q
  // and k, C for v) is per wave.  A wave reads the fragments of a 16-deep
  // step and then runs its MFMAs; the SIMD's other wave covers the wait.
  struct Frags {
    bf16x8_t x[TB], w[DB];
  };
  auto read = [&](int stg, int kk, Frags& f) __attribute__((always_inline)) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
      f.x[tb] = *reinterpret_cast<const bf16x8_t*>(smem + xoff[kk] + stg * XB + tb * 4096);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      f.w[db] = *reinterpret_cast<const bf16x8_t*>(smem + woff[kk] + stg * WB + db * 4096);
  };
  auto gemm = [&](auto trans_tag) {
    constexpr bool kTrans = decltype(trans_tag)::value;  // C^T: features as rows
    auto mma = [&](const Frags& f) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          if constexpr (kTrans)
            acc[db * TB + tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[db], f.x[tb], acc[db * TB + tb], 0, 0, 0);
          else
            acc[db * TB + tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.x[tb], f.w[db], acc[db * TB + tb], 0, 0, 0);
        }
    };
    const int n_k = n_full + (half_tail ? 1 : 0);
    // two stages: slice kt+1 loads while slice kt is computed
    issue(0, 0);
    if (n_k > 1) issue(1, 1);
    // slice kt in stage kt % 2 (a constant: the loop is unrolled twice)
    auto slice = [&](auto stg_c, int kt) __attribute__((always_inline)) {
      constexpr int stg = decltype(stg_c)::value;
      // the offsets pass through an empty asm each slice, so that offset +
      // stage is formed at the read (as its immediate) instead of being
      // hoisted out of the loop into registers
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        asm volatile("" : "+v"(xoff[kk]));
        asm volatile("" : "+v"(woff[kk]));
      }
      if (kt == 0 && n_k > 1)
        wait_vm<DMA>();
      else
        wait_vm<0>();
      __syncthreads();  // slice kt landed everywhere; slice kt-1 is done everywhere
      if (kt >= 1 && kt + 1 < n_k) issue(kt + 1, stg ^ 1);
      const int n_kk = kt == n_full ? 2 : 4;  // 16-deep steps in this slice
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk >= n_kk) break;
        Frags f;
        read(stg, kk, f);
        mma(f);
      }
    };
    int kt = 0;
    for (; kt + 2 <= n_k; kt += 2) {
      slice(std::integral_constant<int, 0>{}, kt);
      slice(std::integral_constant<int, 1>{}, kt + 1);
    }
    if (kt < n_k) slice(std::integral_constant<int, 0>{}, kt);
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
  // fp64 angles, then copies of the height and width tables) and, at its
  // end, one staging area per wave through which the outputs leave in whole
  // 16-byte pieces of contiguous rows ----
  constexpr int kRing = kQStages * STAGE;
  constexpr int kStageOut = 32 * D * 2;             // one 32-token x D block
  constexpr int kOutBase = kRing - kQWaves * kStageOut;
  static_assert(kOutBase >= 16384, "room for the tables");
  float2* tab = reinterpret_cast<float2*>(smem);
  char* outst = smem + kOutBase + wave * kStageOut;  // this wave's staging area
  const int dh2 = g.dh / 2, dw2 = g.dw / 2;
  const int hw_n = g.grid_h * dh2 + g.grid_w * dw2;
  const int f_hi = (min(m0 + kQM, Ntok) - 1) / g.P;
  constexpr int kTabCap = kOutBase / int(sizeof(float2));
  const bool hw_lds = hw_n <= kTabCap / 2;  // else read from global memory
  const int nf_tab = min(f_hi - f_lo + 1, (kTabCap - (hw_lds ? hw_n : 0)) / max(pt, 1));
  const int h_base = nf_tab * pt, w_base = h_base + g.grid_h * dh2;
  __syncthreads();  // every wave is done with the ring
  for (int i = tid; i < nf_tab * pt; i += kThreads) {
    const int fi = i / pt, j = i - fi * pt;
    tab[i] = rope_cos_sin(t0 + f_lo + fi - a.pos_off[b], a.omega_t[j]);
  }
  if (hw_lds) {
    for (int i = tid; i < g.grid_h * dh2; i += kThreads) tab[h_base + i] = a.tab_h[i];
    for (int i = tid; i < g.grid_w * dw2; i += kThreads) tab[w_base + i] = a.tab_w[i];
  }
  __syncthreads();
  if (!fb_valid) return;
  // frame of token t and its ring row (slot * slot_rows + position)
  auto ring_row = [&](int t) -> int64_t {
    const int f = t / g.P;
    return slot_of(f) * g.slot_rows + (t - f * g.P);
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
        const int f = t / g.P, p = t - f * g.P;
        const int yy = p / g.grid_w, xx = p - yy * g.grid_w;
        const int fi = f - f_lo;
        // entry bases such that pair j's entry is base + j
        const int tbase = fi * pt;
        const int hbase = h_base + yy * dh2 - pt, wbase = w_base + xx * dw2 - pth;
        const bool t_in_tab = fi < nf_tab;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int d0 = 32 * db + 8 * e + 4 * hl;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[db * TB + tb][4 * e + i];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
              const int j = d0 / 2 + pp;
              float2 cs;
              if (j < pt) {
                if (t_in_tab)
                  cs = tab[tbase + j];
                else
                  cs = rope_cos_sin_slow(t0 + f - a.pos_off[b], a.omega_t[j]);
              } else if (hw_lds) {
                cs = tab[j < pth ? hbase + j : wbase + j];
              } else {
                cs = j < pth ? a.tab_h[yy * dh2 + (j - pt)] : a.tab_w[xx * dw2 + (j - pth)];
              }
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
          const int64_t row = sel == 0 ? int64_t(t) * g.H : ring_row(t);
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
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#pragma unroll
      for (int n = 0; n < D * 4 / 64; ++n) {
        const int r = 16 * n + (lane >> 2), c = lane & 3;
        const uint4 val = *reinterpret_cast<const uint4*>(outst + r * 64 + ((c ^ ((r >> 2) & 3)) << 4));
        const int t = tile0 + 8 * c;
        if (t >= Ntok) continue;
        uint16_t* vrow = vt + int64_t(r) * g.rows_pad;
        const int f = t / g.P, p = t - f * g.P;
        if ((p & 7) == 0 && p + 7 < g.P && t + 7 < Ntok) {
          *reinterpret_cast<uint4*>(vrow + slot_of(f) * g.slot_rows + p) = val;
        } else {
          const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (t + i < Ntok) vrow[ring_row(t + i)] = uint16_t(w4[i / 2] >> (16 * (i & 1)));
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
