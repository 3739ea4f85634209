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
// d_model.  A workgroup computes one head of q, k or v (D features) for 256
// tokens; 4 waves (one per SIMD) of 64 tokens x D features, fp32
// accumulators in VGPRs, 32x32x16 bf16 MFMA.  Both operands are K-contiguous
// in memory (x rows, weight rows) and move global -> LDS with the 16-byte
// direct loads of gfx950 into a 3-stage ring of 32-deep K slices (24 KB per
// stage at D = 128, so two workgroups share a CU).  Rows of a slice are 64
// bytes; the 16-byte chunk c of row r sits at c ^ ((r >> 2) & 3), which puts
// any 16 consecutive rows of a fragment read on distinct banks.
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

constexpr int kQM = 256;       // tokens per workgroup
constexpr int kQK = 32;        // reduction depth of one LDS stage
constexpr int kQStages = 3;
constexpr int kQWaves = 4;     // 64 tokens per wave
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

template <typename T>
__device__ __forceinline__ uint16_t bits16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<T>(x));
}

template <typename QT, int D>
__global__ __launch_bounds__(256, 2) void qkv_rope_kernel(QkvArgs a) {
  constexpr int XB = kQM * kQK * 2;            // x slice bytes
  constexpr int WB = D * kQK * 2;              // weight slice bytes
  constexpr int STAGE = XB + WB;
  constexpr int X_DMA = XB / 1024 / kQWaves;   // 1 KB loads per wave per stage
  constexpr int W_DMA = WB / 1024 / kQWaves;
  constexpr int DMA = X_DMA + W_DMA;
  constexpr int DB = D / 32, TB = 2;
  static_assert(W_DMA >= 1, "tile sizes");
  __shared__ __attribute__((aligned(1024))) char smem[kQStages * STAGE];
  __shared__ float2 tab_t[kTabFrames * kMaxAxisPairs];

  const Geometry& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, l32 = lane & 31;
  const int mt = blockIdx.x, nb = blockIdx.y, b = blockIdx.z;
  const int sel = nb / g.H, head = nb - sel * g.H;  // 0: q, 1: k, 2: v
  const int Ntok = a.n_frames * g.P;
  const int m0 = mt * kQM;
  const int Dm = a.d_model;
  const int f_lo = m0 / g.P;
  const int pt = g.dt / 2, pth = (g.dt + g.dh) / 2;

  // time-axis cos/sin of the frames this tile starts in (fp64 angles)
  if (sel < 2) {
    const int nf = min(kTabFrames, a.n_frames - f_lo);
    for (int i = tid; i < nf * pt; i += 256) {
      const int fi = i / pt, j = i - fi * pt;
      tab_t[fi * kMaxAxisPairs + j] = rope_cos_sin(a.t0[b] + f_lo + fi - a.pos_off[b], a.omega_t[j]);
    }
  }

  // ---- global -> LDS slices (source offsets are loop invariant) ----
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  const char* xbase = static_cast<const char*>(a.x) + int64_t(b) * Ntok * Dm * 2;
  const char* wbase = static_cast<const char*>(a.w) + int64_t(nb) * D * Dm * 2;
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
    wo[j] = uint32_t(r) * uint32_t(Dm * 2) + uint32_t((cs ^ ((r >> 2) & 3)) << 4);
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
    for (int tb = 0; tb < TB; ++tb) xoff[kk][tb] = slice_off(64 * wave + 32 * tb + l32, 2 * kk + hl);
#pragma unroll
    for (int db = 0; db < DB; ++db) woff[kk][db] = XB + slice_off(32 * db + l32, 2 * kk + hl);
  }

  auto gemm = [&](auto trans_tag) {
    constexpr bool kTrans = decltype(trans_tag)::value;  // C^T: features as rows
    const int n_k = Dm / kQK;
    issue(0, 0);
    if (n_k > 1) issue(1, 1);
    for (int kt = 0; kt < n_k; ++kt) {
      if (kt + 1 < n_k)
        wait_vm<DMA>();
      else
        wait_vm<0>();
      __syncthreads();  // slice kt landed everywhere; slice kt-1 is done everywhere
      if (kt + 2 < n_k) issue(kt + 2, (kt + 2) % kQStages);
      const char* st = smem + (kt % kQStages) * STAGE;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t xf[TB], wf[DB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) xf[tb] = *reinterpret_cast<const bf16x8_t*>(st + xoff[kk][tb]);
#pragma unroll
        for (int db = 0; db < DB; ++db) wf[db] = *reinterpret_cast<const bf16x8_t*>(st + woff[kk][db]);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            if constexpr (kTrans)
              acc[db * TB + tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[db], xf[tb], acc[db * TB + tb], 0, 0, 0);
            else
              acc[db * TB + tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[tb], wf[db], acc[db * TB + tb], 0, 0, 0);
          }
      }
    }
  };

  const int64_t t0 = a.t0[b];
  auto slot_of = [&](int f) -> int64_t {
    const int64_t gf = t0 + f;
    return gf < g.S_f ? gf : g.S_f + gf % g.R;
  };

  if (sel < 2) {
    gemm(std::true_type{});
    // lane: token 64w + 32tb + l32 of the tile; dims 32db + 8e + 4hl + 0..3
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int t = m0 + 64 * wave + 32 * tb + l32;
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
    // lane: feature 32db + l32; tokens 64w + 32tb + 8e + 4hl + 0..3
    uint16_t* vt = static_cast<uint16_t*>(a.cache_v) + (int64_t(b) * g.H + head) * D * g.rows_pad;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      uint16_t* vrow = vt + int64_t(32 * db + l32) * g.rows_pad;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tk = m0 + 64 * wave + 32 * tb + 8 * e + 4 * hl;
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
    // stamps: the frames whose first token lies in this tile
    if (head == 0 && tid == 0) {
      for (int f = (m0 + g.P - 1) / g.P; f * g.P < min(m0 + kQM, Ntok); ++f)
        a.stamps[int64_t(b) * g.n_slots + slot_of(f)] = t0 + f;
    }
  }
}

template <typename QT, int D>
hipError_t launch_qkv_t(const QkvArgs& a, hipStream_t s) {
  const int ntok = a.n_frames * a.g.P;
  dim3 grid(unsigned((ntok + kQM - 1) / kQM), unsigned(3 * a.g.H), unsigned(a.g.B));
  hipLaunchKernelGGL((qkv_rope_kernel<QT, D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_rope(const QkvArgs& a, hipStream_t s) {
  const bool f16 = a.g.qk_dtype == SCV_FP16;
  if (a.g.D == 128) return f16 ? launch_qkv_t<_Float16, 128>(a, s) : launch_qkv_t<__bf16, 128>(a, s);
  return f16 ? launch_qkv_t<_Float16, 64>(a, s) : launch_qkv_t<__bf16, 64>(a, s);
}

}  // namespace scv
