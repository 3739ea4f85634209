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
// -> LDS with the 16-byte direct loads of gfx950 into a ring of 32-deep K
// slices (4 stages of 32 KB, or 3 of 40 KB, at D = 128), loaded up to three
// slices ahead.  Rows of a slice are 64 bytes; the 16-byte chunk c of row r
// sits at c ^ ((r >> 2) & 3), which puts any 16 consecutive rows of a
// fragment read on distinct banks.
// For q and k the MFMA computes C^T (features as rows) so that each lane
// holds the dim pairs (2j, 2j+1) of one token, which RoPE rotates in
// registers; for v it computes C (tokens as rows) so that each lane holds 4
// consecutive tokens of one feature: one 8-byte store into the transposed
// value cache.
#include <type_traits>

#include "scv_internal.h"

namespace scv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kQK = 32;        // reduction depth of one LDS stage
constexpr int kQTokGroups = 4; // waves per feature block
constexpr int kTabFrames = 8;  // time-axis cos/sin of up to 8 frames in LDS

__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(lds_base), "v"(voff), "s"(base) : "m0", "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// byte offset of 16-byte chunk c of row r in a slice (64-byte rows)
__device__ __forceinline__ int slice_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

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
// waits; each wave computes 32*TB tokens of one block.  TB = 3 (384 tokens,
// a 3-stage ring) gives fewer, larger workgroups than TB = 2 (256 tokens, a
// 4-stage ring); the host picks the one whose grid fills the chip better.
// (4 waves of 128x128 tiles -- half the LDS bytes per MFMA -- measured 1.5x
// slower: a lone wave per SIMD stalls on its own loads.)
template <typename QT, int D, int TB>
__global__ __launch_bounds__(512, 1) void qkv_rope_kernel(QkvArgs a) {
  constexpr int kQM = 32 * TB * kQTokGroups;   // tokens per workgroup
  constexpr int kQStages = TB >= 3 ? 3 : 4;
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
  __shared__ float2 tab_t[kTabFrames * kMaxAxisPairs];

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

  // time-axis cos/sin of the frames this tile starts in (fp64 angles)
  {
    const int nf = min(kTabFrames, a.n_frames - f_lo);
    for (int i = tid; i < nf * pt; i += kThreads) {
      const int fi = i / pt, j = i - fi * pt;
      tab_t[fi * kMaxAxisPairs + j] = rope_cos_sin(a.t0[b] + f_lo + fi - a.pos_off[b], a.omega_t[j]);
    }
  }

  // ---- global -> LDS slices (source offsets are loop invariant) ----
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  const char* xbase = static_cast<const char*>(a.x) + int64_t(b) * Ntok * Dm * 2;
  const char* wbase = static_cast<const char*>(a.w) + int64_t(fb0) * D * Dm * 2;
  const int w_rows = min(2, n_blocks - fb0) * D;  // weight rows that exist
  uint32_t xo[X_DMA], wo[W_DMA];
#pragma unroll
  for (int j = 0; j < X_DMA; ++j) {
    const int piece = (wave * X_DMA + j) * 64 + lane, r = piece >> 2, cs = piece & 3;
    const int tok = min(m0 + r, Ntok - 1);  // rows past the last token repeat it (outputs dropped)
    xo[j] = uint32_t(tok) * uint32_t(Dm * 2) + uint32_t((cs ^ ((r >> 2) & 3)) << 4);
  }
#pragma unroll
  for (int j = 0; j < W_DMA; ++j) {
    const int piece = (wave * W_DMA + j) * 64 + lane, r = piece >> 2, cs = piece & 3;
    const int rr = min(r, w_rows - 1);  // a missing second block repeats the last row (unused)
    wo[j] = uint32_t(rr) * uint32_t(Dm * 2) + uint32_t((cs ^ ((r >> 2) & 3)) << 4);
  }
  auto issue = [&](int kt, int stg) {
    const uint32_t dst = lds0 + uint32_t(stg * STAGE);
    const int64_t k0 = int64_t(kt) * kQK * 2;
#pragma unroll
    for (int j = 0; j < X_DMA; ++j) dma16(xbase + k0, xo[j], dst + uint32_t((wave * X_DMA + j) * 1024));
#pragma unroll
    for (int j = 0; j < W_DMA; ++j) dma16(wbase + k0, wo[j], dst + uint32_t(XB + (wave * W_DMA + j) * 1024));
  };

  floatx16_t acc[DB * TB];
#pragma unroll
  for (int i = 0; i < DB * TB; ++i) acc[i] = floatx16_t{};

  // fragment offsets inside a stage (chunk 2*kk + hl of the row)
  int xoff[2][TB], woff[2][DB];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) xoff[kk][tb] = slice_off(32 * TB * wq + 32 * tb + l32, 2 * kk + hl);
#pragma unroll
    for (int db = 0; db < DB; ++db) woff[kk][db] = XB + slice_off(D * grp + 32 * db + l32, 2 * kk + hl);
  }

  // Every wave passes the same barriers; the MFMA operand order (C^T for q
  // and k, C for v) is per wave.  Fragments of the next 16-deep step are read
  // while the MFMAs of the current one run, also across the barrier that
  // publishes the next slice: a trip reads step 1 of slice kt, runs step 0,
  // waits for slice kt+1, reads its step 0 and runs step 1 of slice kt.
  struct Frags {
    bf16x8_t x[TB], w[DB];
  };
  auto read = [&](const char* st, int kk, Frags& f) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) f.x[tb] = *reinterpret_cast<const bf16x8_t*>(st + xoff[kk][tb]);
#pragma unroll
    for (int db = 0; db < DB; ++db) f.w[db] = *reinterpret_cast<const bf16x8_t*>(st + woff[kk][db]);
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
    const int n_k = Dm / kQK;
    // wait until slice kt has landed (slices after it may still be loading)
    auto wait_slice = [&](int kt) {
      const int ahead = min(n_k - 1 - kt, kQStages - 2);
      if (ahead >= 2)
        wait_vm<2 * DMA>();
      else if (ahead == 1)
        wait_vm<DMA>();
      else
        wait_vm<0>();
    };
#pragma unroll
    for (int i = 0; i < kQStages - 1; ++i)
      if (i < n_k) issue(i, i);
    if constexpr (TB >= 3) {
      // 96-token waves: no registers for a second fragment set; the SIMD's
      // other wave covers the fragment waits
      for (int kt = 0; kt < n_k; ++kt) {
        wait_slice(kt);
        __syncthreads();  // slice kt landed everywhere; slice kt-1 is done everywhere
        if (kt + kQStages - 1 < n_k) issue(kt + kQStages - 1, (kt + kQStages - 1) % kQStages);
        const char* st = smem + (kt % kQStages) * STAGE;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          Frags f;
          read(st, kk, f);
          mma(f);
        }
      }
      return;
    }
    wait_slice(0);
    __syncthreads();
    if (kQStages - 1 < n_k) issue(kQStages - 1, kQStages - 1);
    Frags f0, f1;
    read(smem, 0, f0);
    for (int kt = 0; kt < n_k; ++kt) {
      const char* st = smem + (kt % kQStages) * STAGE;
      read(st, 1, f1);
      mma(f0);
      if (kt + 1 < n_k) {
        wait_slice(kt + 1);
        __syncthreads();  // slice kt+1 landed everywhere; slice kt-1... kt's reads are done everywhere
        if (kt + kQStages < n_k) issue(kt + kQStages, (kt + kQStages) % kQStages);
        read(smem + ((kt + 1) % kQStages) * STAGE, 0, f0);
      }
      mma(f1);
    }
  };

  const int64_t t0 = a.t0[b];
  auto slot_of = [&](int f) -> int64_t {
    const int64_t gf = t0 + f;
    return gf < g.S_f ? gf : g.S_f + gf % g.R;
  };

  if (sel < 2) {
    gemm(std::true_type{});
    if (!fb_valid) return;  // after the last barrier
    // lane: token 32TB*wq + 32tb + l32 of the tile; dims 32db + 8e + 4hl + 0..3
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int t = m0 + 32 * TB * wq + 32 * tb + l32;
      if (t >= Ntok) continue;
      const int f = t / g.P, p = t - f * g.P;
      const int yy = p / g.grid_w, xx = p - yy * g.grid_w;
      const int fi = f - f_lo;
      QT* dst;
      if (sel == 0)
        dst = static_cast<QT*>(a.q_out) + ((int64_t(b) * Ntok + t) * g.H + head) * D;
      else
        dst = static_cast<QT*>(a.cache_k) + ((int64_t(b) * g.H + head) * g.rows_pad + slot_of(f) * g.slot_rows + p) * D;
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
            if (j < pt)
              cs = fi < kTabFrames ? tab_t[fi * kMaxAxisPairs + j] : rope_cos_sin(t0 + f - a.pos_off[b], a.omega_t[j]);
            else if (j < pth)
              cs = a.tab_h[yy * (g.dh / 2) + (j - pt)];
            else
              cs = a.tab_w[xx * (g.dw / 2) + (j - pth)];
            const float u = v[2 * pp], w = v[2 * pp + 1];
            v[2 * pp] = u * cs.x - w * cs.y;
            v[2 * pp + 1] = u * cs.y + w * cs.x;
          }
          uint2 o;
          o.x = uint32_t(bits16<QT>(v[0])) | (uint32_t(bits16<QT>(v[1])) << 16);
          o.y = uint32_t(bits16<QT>(v[2])) | (uint32_t(bits16<QT>(v[3])) << 16);
          *reinterpret_cast<uint2*>(dst + d0) = o;
        }
    }
  } else {
    gemm(std::false_type{});
    if (!fb_valid) return;
    // lane: feature 32db + l32; tokens 32TB*wq + 32tb + 8e + 4hl + 0..3
    uint16_t* vt = static_cast<uint16_t*>(a.cache_v) + (int64_t(b) * g.H + head) * D * g.rows_pad;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint16_t* vrow = vt + int64_t(32 * db + l32) * g.rows_pad;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tk = m0 + 32 * TB * wq + 32 * tb + 8 * e + 4 * hl;
          if (tk >= Ntok) continue;
          const floatx16_t& c = acc[db * TB + tb];
          const int f = tk / g.P, p = tk - f * g.P;
          if ((p & 3) == 0 && p + 3 < g.P && tk + 3 < Ntok) {
            uint2 o;
            o.x = uint32_t(bits16<__bf16>(c[4 * e])) | (uint32_t(bits16<__bf16>(c[4 * e + 1])) << 16);
            o.y = uint32_t(bits16<__bf16>(c[4 * e + 2])) | (uint32_t(bits16<__bf16>(c[4 * e + 3])) << 16);
            *reinterpret_cast<uint2*>(vrow + slot_of(f) * g.slot_rows + p) = o;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ti = tk + i;
              if (ti >= Ntok) break;
              const int fi2 = ti / g.P, pi = ti - fi2 * g.P;
              vrow[slot_of(fi2) * g.slot_rows + pi] = bits16<__bf16>(c[4 * e + i]);
            }
          }
        }
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
