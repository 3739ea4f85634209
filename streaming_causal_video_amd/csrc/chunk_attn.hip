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
// Kernels (MI355X / CDNA4, wave64):
//  * chunk_attn_bf16_kernel (bf16 / fp16 operands, fp32 accumulation):
//    8 waves = 256 query rows of one query chunk of one (stream, head[, key
//    split]), 32 rows per wave, two waves per SIMD; each wave runs its key
//    loop software-pipelined in 32-key units, the softmax of one unit
//    interleaved instruction by instruction with the MFMAs of its
//    neighbours; 64-key tiles move global -> LDS by direct 16-byte loads
//    into 4-stage K and V^T rings.  Details above the kernel.
//  * chunk_attn_f32_kernel (fp32 end to end): 4 waves = 128 query rows,
//    v_mfma_f32_32x32x2_f32, double-buffered LDS tiles staged through VGPRs.
//  * attn_merge_kernel: combines the normalised fp32 partials of key splits
//    (lse-weighted).
//  * Balanced schedule (bf16 kernel): instead of one workgroup per query
//    tile and key split, the launch's work -- query tile x visited key tile
//    units -- is cut into equal ranges, one per workgroup, so that every
//    compute unit runs equally long; attn_lean_merge_kernel combines the
//    partials of query tiles cut by range boundaries.
// Shared by both attention kernels:
//  * S^T = K Q^T on MFMA (A = K rows from LDS, B = the wave's Q in VGPRs),
//    so each lane holds one query column and 16 of every 32 keys: the row
//    max / row sum need one exchange with lane ^ 32, and P^T is directly the
//    B operand of O^T += V^T P^T -- no LDS round trip for P.
//  * V is stored transposed in the cache ([d][row]).
//  * Online softmax in fp32 with exp2 (the fp32 kernel folds scale * log2 e
//    into one FMA; the bf16 kernel folds it into Q and the running
//    reference into the S^T accumulator's start value, so a score costs one
//    exponential and no other arithmetic before it).
//  * Query tiles never straddle query chunks; each workgroup derives the
//    slots its chunk may see from the stamps once, skips invisible tiles and
//    masks the hidden keys of partly visible ones.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "scv_internal.h"

namespace scv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// 8 QK^T operand elements (bf16 or fp16) and the matching 32x32x16 MFMA.
template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  typedef bf16x8 type;
};
template <>
struct Vec8<_Float16> {
  typedef halfx8 type;
};
__device__ __forceinline__ floatx16 mfma_32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma_32x32x16(halfx8 a, halfx8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr int kWaves = 4;
constexpr int kBlockM = 32 * kWaves;  // query rows per workgroup
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Query tiles never straddle two query chunks: tile i of chunk c covers rows
// [c * rows_per_chunk + i * ROWS, ...) up to the end of the chunk.  Every
// query of a workgroup therefore sees the same frame slots.
struct QueryTile {
  int chunk;
  int row_lo;   // first query row
  int row_end;  // one past the last query row (<= row_lo when the tile is empty)
};

template <int ROWS_PER_WG>
__device__ __forceinline__ QueryTile query_tile(const AttnArgs& a, int qtile) {
  QueryTile q;
  q.chunk = qtile / a.qtiles_per_chunk;
  const int i = qtile - q.chunk * a.qtiles_per_chunk;
  q.row_lo = q.chunk * a.rows_per_chunk + i * ROWS_PER_WG;
  q.row_end = min(min(q.row_lo + ROWS_PER_WG, (q.chunk + 1) * a.rows_per_chunk), a.Nq);
  return q;
}

__device__ __forceinline__ uint64_t tile_slot_bits(const Geometry& g, int t) {
  const int64_t r0 = int64_t(t) * kKeyTile;
  if (r0 >= g.rows) return 0;
  const int s_lo = int(r0 / g.slot_rows);
  const int s_hi = int(min(r0 + kKeyTile - 1, g.rows - 1) / g.slot_rows);
  const uint64_t hi = s_hi >= 63 ? ~uint64_t(0) : ((uint64_t(1) << (s_hi + 1)) - 1);
  return hi & ~((uint64_t(1) << s_lo) - 1);
}

// Frame slots the queries of chunk `chunk` of stream b may see: lane s of
// every wave tests slot s (n_slots <= 64) and a ballot gathers the mask, so
// the result is a wave-uniform scalar without a trip through LDS.  A sink
// slot is seen when its frame does not lie after the chunk (block-causal
// only); a ring slot also needs its frame inside the window.
__device__ __forceinline__ uint64_t chunk_slot_mask(const AttnArgs& a, int b, int chunk) {
  const Geometry& g = a.g;
  const int s = threadIdx.x & 63;
  const int64_t s_c = a.t0[b] + int64_t(chunk) * g.C;
  bool seen = false;
  if (s < g.n_slots) {
    const int64_t st = a.stamps[int64_t(b) * g.n_slots + s];
    seen = st >= 0 && st < s_c + g.C && (s < g.S_f || st >= s_c - g.W);
  }
  return __ballot(seen);
}

// Visible keys of tile t as a 64-bit mask (bit r = key row r0 + r): rows of
// visible slots that hold tokens (slot padding and rows past the last slot
// excluded).  Scalar work, done only for tiles that are not fully visible.
__device__ __forceinline__ uint64_t tile_key_mask(const Geometry& g, uint64_t slots, int t) {
  const int r0 = t * kKeyTile;
  const int sr = int(g.slot_rows);
  const int rows = int(g.rows);
  uint64_t m = 0;
  int s = r0 / sr;
  for (int base = s * sr; base < r0 + kKeyTile && base < rows; base += sr, ++s) {
    if ((slots >> s) & 1) {
      const int lo = max(base, r0) - r0;
      const int hi = min(min(base + g.P, r0 + kKeyTile), rows) - r0;
      if (hi > lo) m |= (hi - lo == 64 ? ~uint64_t(0) : ((uint64_t(1) << (hi - lo)) - 1)) << lo;
    }
  }
  return m;
}

// Is every key row of tile t visible under the slot mask?
__device__ __forceinline__ bool tile_full(const Geometry& g, uint64_t slots, int t) {
  return ((tile_slot_bits(g, t) & ~slots) == 0) && (int64_t(t + 1) * kKeyTile <= g.rows) && (g.slot_rows == g.P);
}

// ---------------------------------------------------------------------------
// bf16 inputs, fp32 accumulation; QKT = format of the rotated q/k operands
// (bf16, or fp16 for 3 more mantissa bits at the same MFMA rate).
//
// Workgroup = 8 waves = 256 query rows of one (stream, head[, key split]);
// each wave owns 32 query rows for the whole key loop, so a wave's S^T,
// P^T, Q and O^T all stay in VGPRs; waves w and w + 4 share a SIMD.  Each
// wave walks the keys in 32-key units: step u issues the MFMAs of P V of
// unit u-1 and of S^T of unit u+1, and between every two MFMAs the LDS read
// of a later fragment and the exponential, sum and bf16 conversion of one
// score of unit u -- so the matrix core and the VALU work side by side
// within each wave instead of in alternating phases.
// Tiles of 64 keys move global -> LDS through the 16-byte direct loads of
// gfx950 (no VGPR staging) into K and V^T rings of 4 stages, two tiles
// ahead of use, with one barrier per two tiles.  In LDS, K rows are permuted inside each 16-row
// group (bits 2 and 3 of the row index swapped) so that the S^T accumulator
// of lane half h holds, per 16-key group, exactly keys 8h..8h+7 of that
// group: P^T then pairs with V^T read in natural key order (one 16-byte read
// per lane).  Both tiles carry an XOR swizzle of 16-byte chunks that puts
// any 16 consecutive lanes of a fragment read on distinct banks (64 banks
// of 4 bytes).
// Softmax rescaling is lazy: the reference max moves only when an
// exponential would exceed 2^10, detected from the row sums after the fact.
// ---------------------------------------------------------------------------
// Direct global -> LDS load of 16 bytes per lane: lane l writes LDS byte
// address lds_base + 16*l (lds_base wave-uniform, via M0) from base + voff
// (base wave-uniform in SGPRs, voff the lane's unsigned 32-bit offset, kept
// in a register that is never rewritten, so issuing the next load never
// waits for this one to read its address).  Issued through inline assembly
// so that the compiler does not guard later LDS reads of other buffers with
// waits on these loads; the kernel waits for them itself (vmcnt) before the
// barrier that publishes a tile.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(lds_base), "v"(voff), "s"(base) : "m0", "memory");
}
// wait until at most N vector-memory operations of this wave are in flight
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// max / sum of x over lanes l and l ^ 32 (one v_permlane32_swap)
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(a, b, c) as one v_max3_f32.  Through fmaxf the compiler would first
// quiet the NaNs of each input (one more instruction per element); the
// inputs here are MFMA results and running maxima, never NaN.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Workgroups are handed to the 8 XCDs of the chip round robin by linear
// index, each XCD with its own L2.  The work items -- ((chunk, stream) class
// fastest, then split, then query tile, then head) -- are renumbered so that
// every XCD runs a contiguous range of them: the query tiles of one head
// then share that head's K/V in one L2 instead of each XCD fetching it from
// HBM, and every XCD gets the same mix of classes (chunks and streams differ
// in length near a stream's start).  Inside its range an XCD starts the
// classes in the order the host ranks them (longest first), so the longest
// workgroups start first.
constexpr int kXcds = 8;
struct WorkItem {
  int qtile;  // chunk * qtiles_per_chunk + tile in chunk
  int head;
  int bz;     // stream * splits + split
};
__device__ __forceinline__ WorkItem attn_work_item(const AttnArgs& a) {
  const int nx = gridDim.x, ny = gridDim.y;
  const int n = nx * ny * gridDim.z;
  const int id = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const int xcd = id % kXcds, k = id / kXcds;
  const int base = n / kXcds, extra = n % kXcds;  // XCDs below `extra` run one more
  const int lo = xcd * base + min(xcd, extra);
  const int cnt = base + (xcd < extra ? 1 : 0);
  const int nch = a.n_qtiles / a.qtiles_per_chunk;
  const int ncls = nch * a.g.B;
  // In [lo, lo + cnt) class position cp sits at positions p = (cp - r0) mod
  // ncls + ncls*i; classes whose first position lies below `rem` hold one
  // more item.  items_before(cp) counts the items of the classes before cp.
  const int q = cnt / ncls, rem = cnt - q * ncls, r0 = lo % ncls;
  auto items_before = [&](int cp) {
    const int in_a = max(0, min(cp, min(r0 + rem, ncls)) - r0);  // [r0, r0 + rem) below cp
    const int in_b = max(0, min(cp, r0 + rem - ncls));           // its wrapped part [0, r0 + rem - ncls)
    return cp * q + in_a + in_b;
  };
  // the class of the k-th item: the last class position cp with items_before(cp) <= k
  int c_lo = 0, c_hi = ncls - 1;
  while (c_lo < c_hi) {
    const int mid = (c_lo + c_hi + 1) >> 1;
    if (items_before(mid) <= k)
      c_lo = mid;
    else
      c_hi = mid - 1;
  }
  const int cp = c_lo;
  const int p = (cp - r0 + ncls) % ncls + ncls * (k - items_before(cp));
  const int rest = (lo + p) / ncls;
  const int split = rest % a.splits;
  const int rest2 = rest / a.splits;
  const int cls = a.cls_order[cp];
  const int chunk = cls % nch, b = cls / nch;
  WorkItem w;
  w.qtile = chunk * a.qtiles_per_chunk + rest2 % a.qtiles_per_chunk;
  w.head = rest2 / a.qtiles_per_chunk;
  w.bz = b * a.splits + split;
  return w;
}

// LDS row r of a K tile holds key row kperm(r) of the tile.
__device__ __forceinline__ int kperm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

constexpr int kBf16Waves = 8;                  // waves per workgroup (2 per SIMD)
constexpr int kRowsBf16 = 32 * kBf16Waves;     // 256 query rows per workgroup
static_assert(kRowsBf16 == kAttnRowsBf16, "host and kernel agree on the query tile");
constexpr int kStages = 4;                   // LDS tile ring
constexpr int kDmaWaves = kBf16Waves;          // every wave moves its share of a tile

template <int D>
struct Bf16Tile {
  static constexpr int CH = D / 8;               // 16-byte chunks per K row
  static constexpr int KROW = D * 2;             // bytes per K row
  static constexpr int KBYTES = kKeyTile * KROW;
  static constexpr int VROW = kKeyTile * 2;      // bytes per V^T row (64 keys)
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int K_DMA = KBYTES / 1024 / kDmaWaves;  // 1 KB loads per loading wave
  static constexpr int V_DMA = VBYTES / 1024 / kDmaWaves;
  static constexpr int DMA = K_DMA + V_DMA;      // loads per loading wave per tile
  static constexpr int K_ROWS_PER_DMA = 1024 / KROW;
  static constexpr int KS = D / 16;              // k-steps of QK^T
  static constexpr int DB = D / 32;              // 32-row blocks of O^T
  // chunk swizzle of LDS row r: rows of 256 bytes span all 64 banks, rows of
  // 128 bytes half of them (so row pairs share a swizzle value)
  static __device__ __forceinline__ int kswz(int r) { return KROW == 256 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int vswz(int r) { return (r >> 1) & 7; }
};

// Walk over the key tiles of a split [t_begin, t_end) that hold a key of a
// visible slot, one run of consecutive visible slots at a time: inside a run
// the next tile is t + 1 and whether it is fully visible is a range test, so
// the loop pays a few scalar operations per tile; opening the next run costs
// a couple of bit scans.  Tiles come out in increasing order; a tile shared
// by two runs (a run gap shorter than a tile) is visited once, and its mask
// covers both runs.
struct RunWalk {
  int t, t_end;
  int last;     // last tile of the current run (clipped to the split)
  int ff, fu;   // tiles ff .. fu of the run hold visible keys only
  int s_next;   // first slot after the current run
  bool exact;   // slot_rows == P: no padding rows inside a run
  bool valid;

  // Opens the first run at or after slot from_slot with a tile >= min_t.
  __device__ __forceinline__ bool open(const Geometry& g, uint64_t slots, int from_slot, int min_t) {
    while (from_slot < g.n_slots) {
      const uint64_t m = slots & (~uint64_t(0) << from_slot);
      if (m == 0) return false;
      const int s0 = __builtin_ctzll(m);
      const uint64_t inv = ~slots & (~uint64_t(0) << s0);
      const int s1 = min(inv ? int(__builtin_ctzll(inv)) : 64, g.n_slots);
      const int sr = int(g.slot_rows);
      const int r_lo = s0 * sr, r_hi = (s1 - 1) * sr + g.P;  // rows of the run's tokens
      last = min((r_hi - 1) >> 6, t_end - 1);
      ff = (r_lo + kKeyTile - 1) >> 6;
      fu = (r_hi >> 6) - 1;
      s_next = s1;
      t = max(r_lo >> 6, min_t);
      if (t >= t_end) return false;
      if (t <= last) return true;
      from_slot = s1;
    }
    return false;
  }
  __device__ __forceinline__ void init(const Geometry& g, uint64_t slots, int t_begin, int t_end_) {
    t_end = t_end_;
    exact = g.slot_rows == g.P;
    valid = t_begin < t_end && open(g, slots, int((int64_t(t_begin) * kKeyTile) / g.slot_rows), t_begin);
  }
  // the next tile with a visible key (the first one when `first`); t_end when
  // there is none
  __device__ __forceinline__ int next(const Geometry& g, uint64_t slots, bool first, bool* full) {
    if (first) {
      if (!valid) return t_end;
    } else if (__builtin_expect(t < last, 1)) {  // inside a run: the common case
      ++t;
    } else if (!open(g, slots, s_next, t + 1)) {
      t = t_end;
      return t_end;
    }
    *full = exact ? (t >= ff && t <= fu) : tile_full(g, slots, t);
    return t;
  }
  // Moves n visits ahead (whole runs at a time), so that the current tile
  // is the one next() would return after n more calls; valid turns false
  // when fewer than n visits remain.
  __device__ __forceinline__ void skip(const Geometry& g, uint64_t slots, int n) {
    while (valid && n > 0) {
      const int step = min(n, last - t);
      t += step;
      n -= step;
      if (n == 0) break;
      valid = open(g, slots, s_next, t + 1);  // the next visit opens the next run
      --n;
    }
  }
};

// ---------------------------------------------------------------------------
// Balanced schedule: the work of a launch, counted in units of one query
// tile against one visited key tile, is cut into lean_ctas equal ranges, one
// per workgroup, so that every compute unit runs the same number of tile
// steps whatever the number of query tiles per head (a launch of 228 query
// tiles on 256 compute units otherwise leaves 28 of them idle).  Items are
// laid end to end stream-major, then head, query chunk and query tile.
// ---------------------------------------------------------------------------
struct LeanItem {
  int b, head, chunk, tile;  // tile: query tile inside its chunk
  int64_t start;             // first unit of the item
  int units;
};

template <int ROWS>
__device__ __forceinline__ int chunk_qtiles(const AttnArgs& a, int ch) {
  return (min(a.rows_per_chunk, a.Nq - ch * a.rows_per_chunk) + ROWS - 1) / ROWS;
}

// The item holding unit u (0 <= u < lean_units).
template <int ROWS>
__device__ __forceinline__ LeanItem lean_item_at(const AttnArgs& a, int64_t u) {
  const int nch = a.n_qtiles / a.qtiles_per_chunk;
  LeanItem it{};
  int64_t base = 0;
  for (int b = 0; b < a.g.B; ++b) {
    int64_t per_head = 0;
    for (int ch = 0; ch < nch; ++ch) per_head += int64_t(chunk_qtiles<ROWS>(a, ch)) * a.cls_units[ch + nch * b];
    if (u < base + per_head * a.g.H || b == a.g.B - 1) {
      const int h = int((u - base) / per_head);
      base += int64_t(h) * per_head;
      it.b = b;
      it.head = h;
      for (int ch = 0; ch < nch; ++ch) {
        const int un = a.cls_units[ch + nch * b];
        const int64_t span = int64_t(chunk_qtiles<ROWS>(a, ch)) * un;
        if (u < base + span || ch == nch - 1) {
          it.chunk = ch;
          it.tile = int((u - base) / un);
          it.start = base + int64_t(it.tile) * un;
          it.units = un;
          return it;
        }
        base += span;
      }
    }
    base += per_head * a.g.H;
  }
  return it;
}

// The idx-th item (0 <= idx < B * H * query tiles per head).
template <int ROWS>
__device__ __forceinline__ LeanItem lean_item_by_index(const AttnArgs& a, int idx) {
  const int nch = a.n_qtiles / a.qtiles_per_chunk;
  int per_head_items = 0;
  for (int ch = 0; ch < nch; ++ch) per_head_items += chunk_qtiles<ROWS>(a, ch);
  LeanItem it{};
  it.b = idx / (per_head_items * a.g.H);
  it.head = (idx / per_head_items) % a.g.H;
  int r = idx % per_head_items;
  int64_t base = 0;
  for (int b = 0; b < it.b; ++b) {
    int64_t per_head = 0;
    for (int ch = 0; ch < nch; ++ch) per_head += int64_t(chunk_qtiles<ROWS>(a, ch)) * a.cls_units[ch + nch * b];
    base += per_head * a.g.H;
  }
  int64_t per_head = 0;
  for (int ch = 0; ch < nch; ++ch) per_head += int64_t(chunk_qtiles<ROWS>(a, ch)) * a.cls_units[ch + nch * it.b];
  base += per_head * it.head;
  for (int ch = 0; ch < nch; ++ch) {
    const int n = chunk_qtiles<ROWS>(a, ch);
    const int un = a.cls_units[ch + nch * it.b];
    if (r < n) {
      it.chunk = ch;
      it.tile = r;
      it.start = base + int64_t(r) * un;
      it.units = un;
      return it;
    }
    r -= n;
    base += int64_t(n) * un;
  }
  return it;
}

// Index of the item holding unit u (items numbered as lean_item_by_index).
template <int ROWS>
__device__ __forceinline__ int lean_item_index_at(const AttnArgs& a, int64_t u) {
  const LeanItem it = lean_item_at<ROWS>(a, u);
  const int nch = a.n_qtiles / a.qtiles_per_chunk;
  int per_head_items = 0, before = 0;
  for (int ch = 0; ch < nch; ++ch) {
    const int n = chunk_qtiles<ROWS>(a, ch);
    if (ch < it.chunk) before += n;
    per_head_items += n;
  }
  return (it.b * a.g.H + it.head) * per_head_items + before + it.tile;
}

// First unit of workgroup range v, and the range holding unit u: ranges
// below lean_v0 are whole items, the rest cut the remaining units equally.
__device__ __forceinline__ int64_t lean_range_start(const AttnArgs& a, int v) {
  if (v < a.lean_v0) return lean_item_by_index<kRowsBf16>(a, v).start;
  return a.lean_u0 + int64_t(v - a.lean_v0) * (a.lean_units - a.lean_u0) / (a.lean_ctas - a.lean_v0);
}
__device__ __forceinline__ int lean_range_of(const AttnArgs& a, int64_t u) {
  if (u < a.lean_u0) return lean_item_index_at<kRowsBf16>(a, u);
  const int nt = a.lean_ctas - a.lean_v0;
  return a.lean_v0 + int(((u - a.lean_u0 + 1) * nt - 1) / (a.lean_units - a.lean_u0));
}
// Workgroup blockIdx.x runs range v.  Workgroups go to the 8 XCDs round
// robin; the cut ranges of one XCD are consecutive, so the items of a head
// mostly stay in one L2; whole-item ranges are renumbered the same way
// inside each round of lean_round workgroups, so that an XCD's compute
// units run consecutive query tiles of a head side by side, walking the
// same key tiles at the same time.
__device__ __forceinline__ int lean_range_index(const AttnArgs& a) {
  const int c = blockIdx.x;
  if (c < a.lean_v0) {
    const int R = a.lean_round, r = c / R, k = c - r * R;
    return (R % kXcds == 0) ? r * R + (k % kXcds) * (R / kXcds) + k / kXcds : c;
  }
  const int G = a.lean_ctas - a.lean_v0, t = c - a.lean_v0;
  return a.lean_v0 + ((G % kXcds == 0) ? (t % kXcds) * (G / kXcds) + t / kXcds : t);
}

template <int D, typename QKT>
__global__ __launch_bounds__(512, 1) void chunk_attn_bf16_kernel(AttnArgs a) {
  typedef typename Vec8<QKT>::type qk8;
  typedef Bf16Tile<D> T;
  static_assert(T::K_DMA >= 1 && T::V_DMA >= 1, "tile sizes");
  constexpr int KS = T::KS, DB = T::DB;

  __shared__ __attribute__((aligned(1024))) char smem[kStages * T::STAGE];

  const Geometry& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, l32 = lane & 31;

  // One segment: the visits [vis_lo, vis_hi) of key tiles [t_begin, t_end)
  // of query tile qtile of (stream b, head), written as the output or as
  // normalised fp32 partials (row r of the tile at part row prow + r).
  struct Segment {
    int head, b, qtile, t_begin, t_end;
    int vis_lo, vis_hi;  // vis_hi = INT_MAX: to the end of the range
    bool partial;
    int64_t prow;
  };
  auto run_segment = [&](const Segment& sg) __attribute__((always_inline)) {
  const int head = sg.head, b = sg.b;
  int t_begin = sg.t_begin, t_end = sg.t_end;
  const int vis_lo = sg.vis_lo, vis_hi = sg.vis_hi;
  const bool partial = sg.partial;
  const int64_t prow = sg.prow;
  const QueryTile qt = query_tile<kRowsBf16>(a, sg.qtile);
  if (qt.row_lo >= qt.row_end) return;  // an empty tile of a partial last chunk (grid schedule)
  const int qrow = qt.row_lo + wave * 32 + l32;
  const bool qvalid = qrow < qt.row_end;
  // A wave whose 32 rows all lie past the tile's end (the last tile of a
  // head or chunk) skips its MFMAs and softmax but keeps its share of the
  // tile loads and every barrier; the idle SIMD time leaves power to the
  // others.
  const bool active = qt.row_lo + wave * 32 < qt.row_end;

  // frame slots every query of this workgroup may see (wave-uniform)
  const uint64_t slots = chunk_slot_mask(a, b, qt.chunk);

  // ---- global -> LDS tile copies ----
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)smem));
  const char* kbase = static_cast<const char*>(a.cache_k) + (int64_t(b) * g.H + head) * g.rows_pad * T::KROW;
  const int64_t vpitch = g.rows_pad * 2;  // bytes per V^T row in the cache
  const char* vbase = static_cast<const char*>(a.cache_v) + (int64_t(b) * g.H + head) * D * vpitch;
  // per-lane source offsets inside a tile (loop invariant); LDS is filled
  // linearly and the swizzle is applied on the source side
  const int dw = wave;
  uint32_t kvo[T::K_DMA], vvo[T::V_DMA];
#pragma unroll
  for (int i = 0; i < T::K_DMA; ++i) {
    const int r = (dw * T::K_DMA + i) * T::K_ROWS_PER_DMA + lane / T::CH;  // LDS row
    kvo[i] = uint32_t(kperm(r) * T::KROW + (((lane % T::CH) ^ T::kswz(r)) * 16));
  }
#pragma unroll
  for (int i = 0; i < T::V_DMA; ++i) {
    const int r = (dw * T::V_DMA + i) * 8 + (lane >> 3);  // d row
    vvo[i] = uint32_t((lane >> 3) * vpitch + (((lane & 7) ^ T::vswz(r)) * 16));
  }
  // LDS holds two rings of kStages stages: K tiles at [0, KRING) and V^T
  // tiles at [KRING, 2*KRING).  Visit v's K tile goes to K stage v % 4 and
  // its V^T tile to V stage v % 4.
  constexpr int KRING = kStages * T::KBYTES;
  // load i of this wave's share of the K (V^T) tile t into stage stg
  auto issue_k1 = [&](int t, int stg, int i) __attribute__((always_inline)) {
    const int64_t r0 = int64_t(t) * kKeyTile;
    dma16(kbase + r0 * T::KROW, kvo[i], lds0 + uint32_t(stg * T::KBYTES + (dw * T::K_DMA + i) * 1024));
  };
  auto issue_v1 = [&](int t, int stg, int i) __attribute__((always_inline)) {
    const int64_t r0 = int64_t(t) * kKeyTile;
    const int n = dw * T::V_DMA + i;
    dma16(vbase + int64_t(n * 8) * vpitch + r0 * 2, vvo[i], lds0 + uint32_t(KRING + stg * T::VBYTES + n * 1024));
  };
  auto issue_k = [&](int t, int stg) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::K_DMA; ++i) issue_k1(t, stg, i);
  };
  auto issue_v = [&](int t, int stg) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < T::V_DMA; ++i) issue_v1(t, stg, i);
  };

  // Q^T operand: lane (l32, hl) holds q[qrow][16*kk + 8*hl .. +8], scaled
  // by log2(e)/sqrt(d) and rounded once more to the operand type, so that
  // S^T comes out of the MFMAs in log2 units and the softmax needs no
  // multiply per score.
  qk8 qf[KS];
  {
    const QKT* qp =
        static_cast<const QKT*>(a.q) + ((int64_t(b) * a.Nq + (qvalid ? qrow : 0)) * g.H + head) * D + 8 * hl;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 u = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
      const qk8 x = __builtin_bit_cast(qk8, u);
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[kk][i] = static_cast<QKT>(static_cast<float>(x[i]) * a.scale_log2);
    }
  }
  // Q has landed before any tile load is issued: a wait the compiler sees
  // (s_waitcnt vmcnt(0)), so that it does not place one at the first use of
  // Q inside the tile loop, where it would also wait for the prefetched tiles.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // loop-invariant LDS byte offsets of this lane's K and V^T fragments inside
  // stage 0 of their ring (a stage adds a constant)
  int koff[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) koff[kk] = l32 * T::KROW + (((2 * kk + hl) ^ T::kswz(l32)) * 16);
  int voff[4];
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) voff[g4] = KRING + l32 * T::VROW + (((2 * g4 + hl) ^ T::vswz(l32)) * 16);

  floatx16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = floatx16{};
  // Softmax state in log2 units (scores are q.k * log2(e)/sqrt(d)): m_run
  // is the row's reference (-inf until the row has seen a key), msc_run the
  // reference the scores are taken against (0 while m_run is -inf).  The
  // S^T MFMAs start from sbias = -msc_run, so the accumulator holds
  // score - reference and the exponentials need no subtraction either.
  float m_run = -INFINITY, l_run = 0.f;
  float msc_run = 0.f;
  floatx16 sbias = floatx16{};
  constexpr float kPBound = 1024.f;    // largest exponential kept (2^10)

  // The key loop runs in units of 32 keys (half a tile): unit u = 2v + h is
  // half h of visit v.  Unit u's S^T (its 32 keys in kperm order x this
  // wave's 32 queries) lives in sb[u % 2], its P^T in pb[u % 2] (16-key
  // groups gg).
  floatx16 sb[2];
  bf16x8 pb[2][2];
  constexpr int kPVH = 2 * DB;  // P V MFMAs per unit
  constexpr int kQKH = KS;      // S^T MFMAs per unit
  static_assert(kPVH % 4 == 0 && kQKH % 4 == 0, "fragment ring slots repeat per step");
  // Fragment ring: the LDS operand of MFMA j of a step sits in ring[j % 4],
  // read kLookahead MFMAs ahead; the reads run across step boundaries (the
  // last MFMAs of a step read the first fragments of the next step, whose
  // tiles were published at an earlier barrier), so no step starts with the
  // matrix core waiting a full LDS latency.
  constexpr int kLookahead = 3;
  uint4 ring[4];

  // One operand source of a step: P V of half h of the V^T tile in stage st
  // (fragments n = gg * DB + db), or S^T of half h of the K tile in stage st
  // (fragments kk).
  struct Src {
    bool pv;
    int st, h;
  };
  auto read_frag = [&](const Src& src, int j) __attribute__((always_inline)) {
    if (src.pv) {
      const int db = j % DB, gg = j / DB;
      return *reinterpret_cast<const uint4*>(smem + voff[2 * src.h + gg] + src.st * T::VBYTES + db * 32 * T::VROW);
    }
    return *reinterpret_cast<const uint4*>(smem + koff[j] + src.st * T::KBYTES + src.h * 32 * T::KROW);
  };
  // Masks the keys of half h of tile t that no query here may see.  Element
  // i of a half's S^T in lane half hl is key kperm(8(i/4) + 4hl + i%4) of the
  // half, that is key 16(a>>1) + 8hl + 4(a&1) + i%4 with a = i/4.
  auto mask = [&](floatx16& s, int t, int h) __attribute__((always_inline)) {
    const uint64_t km = tile_key_mask(g, slots, t) >> (32 * h + 8 * hl);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int a4 = i / 4;
      const int bit = 16 * (a4 >> 1) + 4 * (a4 & 1) + (i & 3);
      s[i] = ((km >> bit) & 1) ? s[i] : -INFINITY;
    }
  };
  // Exponentials 2^(s - shift), rounded to bf16 into p, with their fp32 sum
  // over this lane's 16 keys (two chains).
  auto exps = [&](const floatx16& s, float shift, bf16x8 (&p)[2], float& rs) __attribute__((always_inline)) {
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float f0 = fast_exp2(s[i] - shift);
      const float f1 = fast_exp2(s[i + 1] - shift);
      p[i / 8][i % 8] = static_cast<__bf16>(f0);
      p[i / 8][i % 8 + 1] = static_cast<__bf16>(f1);
      acc[0] += f0;
      acc[1] += f1;
    }
    rs = acc[0] + acc[1];
  };
  // The exponentials were taken against the running reference; their row
  // sums show whether an element exceeds 2^10 or no reference exists yet.
  // Only then is the row max computed, the reference raised, O^T and l
  // rescaled and the exponentials redone -- so elements never exceed 2^10
  // and the common path has no max reduction in front of the exponentials.
  // s_next (when NEXT) is S^T of the next unit, computed against the old
  // reference: it moves with it.
  auto finish_softmax = [&](floatx16& s, bf16x8 (&p)[2], float& rs, auto next_c,
                            floatx16& s_next) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_c)::value;
    // (marked unlikely so that the rescale is laid out away from the key
    // loop and the common path runs on without a taken branch)
    if (__builtin_expect(__any((rs > kPBound) || (m_run == -INFINITY)), 0)) {
      // row max with v_max3_f32 issued directly (see vmax3); the fence makes
      // the wait states an MFMA result needs before such reads explicit
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(s));
      const float a0 = vmax3(s[0], s[1], s[2]), a1 = vmax3(s[3], s[4], s[5]);
      const float a2 = vmax3(s[6], s[7], s[8]), a3 = vmax3(s[9], s[10], s[11]);
      const float a4 = vmax3(s[12], s[13], s[14]), a5 = vmax3(s[15], a0, a1);
      // row max of (score - msc_run), in log2 units
      const float d = max_halves(vmax3(a2, a3, vmax3(a4, a5, -INFINITY)));
      const float m_new = fmaxf(m_run, msc_run + d);
      const float msc_new = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      const float shift = msc_new - msc_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m_run = m_new;
      msc_run = msc_new;
#pragma unroll
      for (int i = 0; i < 16; ++i) sbias[i] = -msc_new;
      if constexpr (NEXT) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(s_next));
        s_next -= shift;
      }
      exps(s, shift, p, rs);
    }
    l_run += rs;
  };
  // One step of npv + nqk MFMAs (P V of the previous unit with p_prv from
  // source pv_src, then S^T of the next unit into s_cur from source qk_src)
  // with the softmax of this unit (s_prv -> p_new; sum in rs) spread over
  // them, element by element; the reads of the next step's first fragments
  // (source nx_src, when NX) close it.  Each MFMA, the LDS read kLookahead
  // MFMAs ahead and its share of the softmax form one group that the
  // compiler keeps in this order (sched_barrier), so the SIMD issues MFMA
  // and VALU work side by side instead of in phases.
  // SM: the step carries a softmax; OWN: it reads its own first fragments
  // (the step before did not).
  // extra(j) adds work to MFMA group j (the tile loads after a barrier).
  auto step_ops = [&](auto npv_c, auto nqk_c, auto sm_c, auto own_c, auto nx_c, const Src& pv_src,
                      const Src& qk_src, const Src& nx_src, const bf16x8 (&p_prv)[2], floatx16& s_cur,
                      const floatx16& s_prv, bf16x8 (&p_new)[2], float& rs, auto&& extra) __attribute__((always_inline)) {
    constexpr int NPV = decltype(npv_c)::value, NQK = decltype(nqk_c)::value;
    constexpr bool SM = decltype(sm_c)::value, OWN = decltype(own_c)::value, NX = decltype(nx_c)::value;
    constexpr int N = NPV + NQK;
    static_assert(N > 0 && 16 % N == 0, "16 softmax elements per step");
    constexpr int EPC = SM ? 16 / N : 0;  // softmax elements per MFMA group
    float acc[2] = {0.f, 0.f};
    float fprev = 0.f;
    uint32_t pw[2][4];  // P^T of this unit, two bf16 per word
    if constexpr (NQK > 0) s_cur = sbias;
    // fragment j of this step, or of the next one for j >= N
    auto fetch = [&](int j) __attribute__((always_inline)) {
      if (j < NPV) {
        ring[j % 4] = read_frag(pv_src, j);
      } else if (j < N) {
        ring[j % 4] = read_frag(qk_src, j - NPV);
      } else if constexpr (NX) {
        ring[j % 4] = read_frag(nx_src, j - N);
      }
    };
    if constexpr (OWN) {
#pragma unroll
      for (int j = 0; j < kLookahead; ++j) fetch(j);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (j < NPV) {
        const int gg = j / DB, db = j % DB;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ring[j % 4]), p_prv[gg], o[db], 0,
                                                        0, 0);
      } else {
        s_cur = mfma_32x32x16(__builtin_bit_cast(qk8, ring[j % 4]), qf[j - NPV], s_cur);
      }
      fetch(j + kLookahead);
      extra(j);
#pragma unroll
      for (int e = j * EPC; e < (j + 1) * EPC; ++e) {
        const float f = fast_exp2(s_prv[e]);
        // each chain starts from its first exponential (no add to zero); the
        // empty volatile asm keeps the sum (and below the bf16 pair) in this
        // group instead of letting them sink to the end of the step
        if (e < 2) {
          acc[e & 1] = f;
        } else {
          acc[e & 1] += f;
          asm volatile("" : "+v"(acc[e & 1]));
        }
        if (e & 1) {
          const bf16x2 pr = {static_cast<__bf16>(fprev), static_cast<__bf16>(f)};
          uint32_t w = __builtin_bit_cast(uint32_t, pr);
          asm volatile("" : "+v"(w));
          pw[e / 8][(e % 8) / 2] = w;
        }
        fprev = f;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SM) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg)
        p_new[gg] = __builtin_bit_cast(bf16x8, make_uint4(pw[gg][0], pw[gg][1], pw[gg][2], pw[gg][3]));
    }
    rs = acc[0] + acc[1];
  };

  // The key loop over every tile with a visible key, software-pipelined per
  // wave in 32-key units: step u runs the MFMAs of P V of unit u-1 and of
  // S^T of unit u+1 with the softmax of unit u interleaved between them
  // (the SIMD's two waves run such steps side by side).  Visit v's tiles: K
  // in K stage v % 4, V^T in V stage v % 4.  Before even visits v a barrier
  // B_v (before the steps 2v-1 and 2v, which compute S^T of visit v) waits
  // for the loads started at B_{v-2} -- K of visits v and v+1, V^T of
  // visits v-1 and v -- then starts those of the next two visits' K and V^T
  // (V^T of v+1 and v+2, K of v+2 and v+3) into stages whose tiles every
  // wave finished before B_v; odd visits pass no barrier.  Tiles that are only partly visible
  // (slot padding, window edges, the row tail) have their hidden keys
  // masked before their softmax.
  RunWalk walk;
  walk.init(g, slots, t_begin, t_end);
  // every tile of the split fully visible (the steady state): no walk needed
  bool dense = false;
  if (t_begin < t_end && int64_t(t_end) * kKeyTile <= g.rows && g.slot_rows == g.P) {
    const int s_lo = int((int64_t(t_begin) * kKeyTile) / g.slot_rows);
    const int s_hi = int((int64_t(t_end) * kKeyTile - 1) / g.slot_rows);
    const uint64_t hi = s_hi >= 63 ? ~uint64_t(0) : ((uint64_t(1) << (s_hi + 1)) - 1);
    dense = ((hi & ~((uint64_t(1) << s_lo) - 1)) & ~slots) == 0;
  }
  // A segment of the balanced schedule: narrow [t_begin, t_end) to the
  // tiles of visits vis_lo .. vis_hi - 1.
  if (vis_lo > 0 || vis_hi != INT_MAX) {
    int t_lo, t_hi = t_end;
    if (dense) {
      const int n = t_end - t_begin;
      t_lo = t_begin + min(vis_lo, n);
      if (vis_hi != INT_MAX) t_hi = t_begin + min(vis_hi, n);
    } else {
      RunWalk w2 = walk;
      w2.skip(g, slots, vis_lo);
      t_lo = w2.valid ? w2.t : t_end;
      if (vis_hi != INT_MAX) {
        w2.skip(g, slots, vis_hi - vis_lo);
        if (w2.valid) t_hi = w2.t;
      }
    }
    t_begin = t_lo;
    t_end = max(t_lo, t_hi);
    walk.init(g, slots, t_begin, t_end);
  }
  // One key loop, instantiated twice: without any masking code when every
  // tile of the split is fully visible, and with masks otherwise.
  auto key_loop = [&](auto masked_tag) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    int dense_t = t_begin - 1;
    auto next_tile = [&](bool first, bool* full) __attribute__((always_inline)) {
      if constexpr (!kMasked) {
        dense_t = first ? t_begin : dense_t + 1;
        *full = true;
        return dense_t < t_end ? dense_t : t_end;
      } else {
        return walk.next(g, slots, first, full);
      }
    };
    auto next_or_end = [&](int prev, bool* full) __attribute__((always_inline)) {
      if (prev >= t_end) {
        *full = true;
        return t_end;
      }
      return next_tile(false, full);
    };
    auto mask_if = [&](floatx16& s, int t, bool full, int h) __attribute__((always_inline)) {
      if constexpr (kMasked) {
        // partial tiles are few (run edges): their masking stays off the
        // loop's straight-line path
        if (__builtin_expect(!full, 0)) mask(s, t, h);
      }
    };
    constexpr int KV = T::K_DMA + T::V_DMA;
    // visit queue: tiles of visits v-1 .. v+3 (t_end: no such visit)
    bool fp = true, f0 = true, f1 = true, f2 = true, f3 = true;
    int tp = t_end;
    int tv0 = next_tile(true, &f0);
    if (tv0 >= t_end) return;
    int tv1 = next_or_end(tv0, &f1);
    int tv2 = next_or_end(tv1, &f2);
    int tv3 = t_end;
    // B_v (even visits v only): wait for every load in flight -- K of
    // visits v and v+1, V^T of visits v-1 and v, issued at B_{v-2} --
    // barrier, then the loads of V^T of visits v+1 and v+2 and K of visits
    // v+2 and v+3 into the stages of V^T of v-3 and v-2 and K of v-2 and
    // v-1, which every wave finished before B_v.  st = v % 4.
    // Every barrier issues the same number of loads: a visit that does not
    // exist loads the first tile again into its (free) stage, so the wait
    // counts need no case analysis and the loads need no branch.
    auto real = [&](int t) __attribute__((always_inline)) { return t < t_end ? t : t_begin; };
    auto barrier_v = [&](int st) __attribute__((always_inline)) {
      wait_vm<0>();
      // A bare s_barrier: __syncthreads() would first wait for this wave's
      // LDS reads in flight, the next step's first fragments, which come from
      // V^T of visit v-1; the loads after this barrier do not overwrite that
      // stage, and every read of the stages they do overwrite completed
      // before its MFMA.  The empty asm statements keep the compiler from
      // moving memory accesses across the barrier.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      tv3 = next_or_end(tv2, &f3);
      if (__builtin_expect(!active, 0)) {
        issue_v(real(tv1), (st + 1) % 4);
        issue_v(real(tv2), (st + 2) % 4);
        issue_k(real(tv2), (st + 2) % 4);
        issue_k(real(tv3), (st + 3) % 4);
      }
    };
    // The same loads issued by a wave with steps: one per odd MFMA group of
    // the step after the barrier (after B_0, of the two steps that follow,
    // which hold the S^T MFMAs only), so that their issue overlaps the MFMAs;
    // load number base + j / 2 goes with group j.
    static_assert(2 * (T::K_DMA + T::V_DMA) <= (2 * DB + KS) / 2, "one load per odd MFMA group of a step");
    static_assert(2 * (T::K_DMA + T::V_DMA) <= 2 * (KS / 2), "one load per odd MFMA group of the first two steps");
    auto loads_in_step = [&](int st, int base) __attribute__((always_inline)) {
      const int t1 = real(tv1), t2 = real(tv2), t3 = real(tv3);
      const int s1 = (st + 1) & 3, s2 = (st + 2) & 3, s3 = (st + 3) & 3;
      return [=, &issue_v1, &issue_k1](int j) __attribute__((always_inline)) {
        if (j & 1) {
          const int i = base + (j >> 1);
          if (i < T::V_DMA)
            issue_v1(t1, s1, i);
          else if (i < 2 * T::V_DMA)
            issue_v1(t2, s2, i - T::V_DMA);
          else if (i < 2 * T::V_DMA + T::K_DMA)
            issue_k1(t2, s2, i - 2 * T::V_DMA);
          else if (i < 2 * T::V_DMA + 2 * T::K_DMA)
            issue_k1(t3, s3, i - 2 * T::V_DMA - T::K_DMA);
        }
      };
    };
    auto no_extra = [](int) __attribute__((always_inline)) {};
    auto advance = [&]() __attribute__((always_inline)) {
      tp = tv0; fp = f0;
      tv0 = tv1; f0 = f1;
      tv1 = tv2; f1 = f2;
      tv2 = tv3; f2 = f3;
    };
    using Yes = std::true_type;
    using No = std::false_type;
    using C0 = std::integral_constant<int, 0>;
    using CPV = std::integral_constant<int, kPVH>;
    using CQK = std::integral_constant<int, kQKH>;

    // ---- B_0 and the first step: S^T of units 0 and 1, softmax of unit 0 ----
    issue_k(tv0, 0);
    issue_v(tv0, 0);
    issue_k(real(tv1), 1);
    barrier_v(0);
    if (active) {
      // S^T of unit 0 alone (the fragment ring then holds the first
      // fragments of the next step)
      float rs;
      step_ops(C0{}, CQK{}, No{}, Yes{}, Yes{}, Src{false, 0, 0}, Src{false, 0, 0}, Src{false, 0, 1}, pb[1], sb[0],
               sb[1], pb[1], rs, loads_in_step(0, 0));
      mask_if(sb[0], tv0, f0, 0);
      // S^T of unit 1 with the softmax of unit 0; then the first fragments
      // of P V of unit 0
      step_ops(C0{}, CQK{}, Yes{}, No{}, Yes{}, Src{false, 0, 0}, Src{false, 0, 1}, Src{true, 0, 0}, pb[1], sb[1],
               sb[0], pb[0], rs, loads_in_step(0, KS / 2));
      // the softmax of unit 0 ran against the reference that existed before
      // it (none): finish it now
      finish_softmax(sb[0], pb[0], rs, Yes{}, sb[1]);
    }
    advance();
    // visit v >= 1 (stage st = v % 4, a constant: the loop is unrolled four
    // times so that every fragment read takes its stage as an immediate
    // offset): steps 2v-1 and 2v
    auto visit = [&](auto st_c) __attribute__((always_inline)) {
      constexpr int st = decltype(st_c)::value, sp = (st + 3) & 3;  // sp: stage of visit v-1
      // the fragment offsets pass through an empty asm each visit, so that
      // offset + stage is formed at the read (as its immediate) instead of
      // being hoisted out of the loop into a register per stage
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) asm volatile("" : "+v"(koff[kk]));
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) asm volatile("" : "+v"(voff[g4]));
      constexpr bool kSync = (st & 1) == 0;  // a barrier before even visits only
      if constexpr (kSync)
        barrier_v(st);
      else
        tv3 = next_or_end(tv2, &f3);
      auto first_extra = [&]() __attribute__((always_inline)) {
        if constexpr (kSync)
          return loads_in_step(st, 0);
        else
          return no_extra;
      };
      // No fragment read crosses a barrier: the tiles a step after B_v
      // reads first (V^T of visit v-1) are only known to have landed in
      // every wave's share once B_v has passed.  So the first step of an
      // even visit reads its own first fragments, and the last step of an
      // odd visit (the one before the next barrier) reads none ahead.
      using OwnA = std::integral_constant<bool, kSync>;
      using NxB = std::integral_constant<bool, kSync>;
      if (__builtin_expect(active, 1)) {
        float rs;
        // step 2v-1: P V of unit 2v-2, S^T of unit 2v, softmax of unit 2v-1
        mask_if(sb[1], tp, fp, 1);
        step_ops(CPV{}, CQK{}, Yes{}, OwnA{}, Yes{}, Src{true, sp, 0}, Src{false, st, 0}, Src{true, sp, 1}, pb[0],
                 sb[0], sb[1], pb[1], rs, first_extra());
        finish_softmax(sb[1], pb[1], rs, Yes{}, sb[0]);
        // step 2v: P V of unit 2v-1, S^T of unit 2v+1, softmax of unit 2v
        mask_if(sb[0], tv0, f0, 0);
        step_ops(CPV{}, CQK{}, Yes{}, No{}, NxB{}, Src{true, sp, 1}, Src{false, st, 1}, Src{true, st, 0}, pb[1],
                 sb[1], sb[0], pb[0], rs, no_extra);
        finish_softmax(sb[0], pb[0], rs, Yes{}, sb[1]);
      }
      advance();
    };
    int st = 1;  // stage of the next visit
    while (true) {
      if (tv0 >= t_end) break;
      visit(std::integral_constant<int, 1>{});
      if (tv0 >= t_end) { st = 2; break; }
      visit(std::integral_constant<int, 2>{});
      if (tv0 >= t_end) { st = 3; break; }
      visit(std::integral_constant<int, 3>{});
      if (tv0 >= t_end) { st = 0; break; }
      visit(std::integral_constant<int, 0>{});
    }
    // after the last visit v = n-1 (stage (st + 3) % 4): the softmax of unit
    // 2n-1 with P V of unit 2n-2, then P V of unit 2n-1.  When n-1 is odd,
    // V^T of visit n-1 was loaded at the last barrier, B_{n-2}: wait for it
    // (every wave's share) first; its last step read no fragments ahead, so
    // the first step here reads its own.
    const bool last_odd = (st & 1) == 0;
    if (last_odd) {
      wait_vm<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    if (active) {
      const int sl = (st + 3) & 3;
      float rs;
      mask_if(sb[1], tp, fp, 1);
      if (last_odd)
        step_ops(CPV{}, C0{}, Yes{}, Yes{}, Yes{}, Src{true, sl, 0}, Src{false, 0, 0}, Src{true, sl, 1}, pb[0], sb[0],
                 sb[1], pb[1], rs, no_extra);
      else
        step_ops(CPV{}, C0{}, Yes{}, No{}, Yes{}, Src{true, sl, 0}, Src{false, 0, 0}, Src{true, sl, 1}, pb[0], sb[0],
                 sb[1], pb[1], rs, no_extra);
      finish_softmax(sb[1], pb[1], rs, No{}, sb[0]);
      step_ops(CPV{}, C0{}, No{}, No{}, No{}, Src{true, sl, 1}, Src{false, 0, 0}, Src{false, 0, 0}, pb[1], sb[0],
               sb[1], pb[0], rs, no_extra);
    }
    wait_vm<0>();  // the loads of visits past the end have landed too
  };
  if (dense)
    key_loop(std::false_type{});
  else
    key_loop(std::true_type{});

  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  if (!qvalid) return;
  if (!partial) {
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
    float* pp = a.part_o + (prow + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * hl;
        *reinterpret_cast<float4*>(pp + d0) = make_float4(o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv,
                                                          o[db][4 * q4 + 2] * inv, o[db][4 * q4 + 3] * inv);
      }
    }
    if (hl == 0) a.part_lse[prow + qrow] = lse_v;
  }
  };  // run_segment

  // Grid schedule: one segment per workgroup (a query tile against one key
  // split).  Balanced schedule: the items the workgroup's unit range
  // [lo, hi) touches -- at most two, as the host keeps ranges no longer
  // than the shortest item -- the later one first: its segment starts that
  // item while the earlier one's ends its item, so neighbouring workgroups
  // walk the same key tiles at the same time.  Two straight-line segments
  // rather than a loop: inside a loop nest the compiler gives the key loop
  // too few registers to keep its fragment reads in flight.
  Segment sg;
  const bool lean = a.lean != 0;
  int lean_v = 0;
  int64_t lean_lo = 0, lean_hi = 0, first_start = 0;
  if (!lean) {
    const WorkItem wi = attn_work_item(a);
    const int split = wi.bz % a.splits;
    sg.head = wi.head;
    sg.b = wi.bz / a.splits;
    sg.qtile = wi.qtile;
    sg.t_begin = split * a.tiles_per_split;
    sg.t_end = min(sg.t_begin + a.tiles_per_split, a.tiles_total);
    sg.vis_lo = 0;
    sg.vis_hi = INT_MAX;
    sg.partial = a.splits > 1;
    sg.prow = ((int64_t(split) * g.B + sg.b) * g.H + sg.head) * a.Nq;
  } else {
    lean_v = lean_range_index(a);
    lean_lo = lean_range_start(a, lean_v);
    lean_hi = lean_range_start(a, lean_v + 1);
    if (lean_hi <= lean_lo) return;
  }
  auto lean_segment = [&](int64_t u) {  // the segment of the item holding unit u
    const LeanItem it = lean_item_at<kRowsBf16>(a, u);
    sg.head = it.head;
    sg.b = it.b;
    sg.qtile = it.chunk * a.qtiles_per_chunk + it.tile;
    sg.t_begin = 0;
    sg.t_end = a.tiles_total;
    sg.vis_lo = int(max(it.start, lean_lo) - it.start);
    // the item's last segment takes every remaining visit
    sg.vis_hi = it.start + it.units <= lean_hi ? INT_MAX : int(lean_hi - it.start);
    sg.partial = sg.vis_lo > 0 || sg.vis_hi != INT_MAX;
    const int slot = it.start <= lean_lo ? 0 : 1;
    sg.prow = (int64_t(lean_v) * 2 + slot) * kRowsBf16 - query_tile<kRowsBf16>(a, sg.qtile).row_lo;
    first_start = it.start;
  };
  if (lean) lean_segment(lean_hi - 1);
  run_segment(sg);
  if (lean && first_start > lean_lo) {
    lean_segment(first_start - 1);
    __syncthreads();  // every wave is done with the first segment's LDS tiles
    run_segment(sg);
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

  const Geometry& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int head = blockIdx.y;
  const QueryTile qt = query_tile<kBlockM>(a, a.n_qtiles - 1 - int(blockIdx.x));
  if (qt.row_lo >= qt.row_end) return;  // an empty tile of a partial last chunk
  const int b = blockIdx.z / a.splits, split = blockIdx.z % a.splits;
  const int qrow = qt.row_lo + wave * 32 + l32;
  const bool qvalid = qrow < qt.row_end;

  const uint64_t slots = chunk_slot_mask(a, b, qt.chunk);
  const int t_begin = split * a.tiles_per_split;
  const int t_end = min(t_begin + a.tiles_per_split, a.tiles_total);
  auto next_tile = [&](int t) {
    while (t < t_end && (tile_slot_bits(g, t) & slots) == 0) ++t;
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
    if (!tile_full(g, slots, t)) {
      // element i of s[kb] in lane half hl is key 32kb + 8(i/4) + 4hl + i%4
      const uint64_t km = tile_key_mask(g, slots, t) >> (4 * hl);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[kb][i] = ((km >> (32 * kb + 8 * (i / 4) + (i & 3))) & 1) ? s[kb][i] : -INFINITY;
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

// ---------------------------------------------------------------------------
// Balanced-schedule merge: an item whose units span several workgroup
// ranges left one normalised partial per non-empty range (slot 0 in every
// range but the first, where it is slot 1 unless the item starts the
// range); lse = log sum exp(lse_s), O = sum exp(lse_s - lse) O_s, taken in
// one pass with a running maximum.  Workgroup = 32 query rows of one item
// (blockIdx.y = row block); each thread owns 16 values of one row.  The
// item's partial rows are listed once per workgroup (up to 64 at a time).
// Items done by a single range were written by the attention kernel.
// ---------------------------------------------------------------------------
constexpr int kMergeRows = 32;
template <int D>
__global__ __launch_bounds__(256) void attn_lean_merge_kernel(AttnArgs a) {
  constexpr int TPR = 256 / kMergeRows;  // threads per row
  constexpr int NV = D / 4 / TPR;        // float4 per thread
  const Geometry& g = a.g;
  // items of whole-item ranges were written by the attention kernel: the
  // grid starts at the first item after them
  const LeanItem it = lean_item_by_index<kRowsBf16>(a, a.lean_v0 + int(blockIdx.x));
  const int c_first = lean_range_of(a, it.start);
  const int c_last = lean_range_of(a, it.start + it.units - 1);
  if (c_first == c_last) return;
  const QueryTile qt = query_tile<kRowsBf16>(a, it.chunk * a.qtiles_per_chunk + it.tile);
  const int r = blockIdx.y * kMergeRows + threadIdx.x / TPR;  // row in the tile
  if (blockIdx.y * kMergeRows >= qt.row_end - qt.row_lo) return;
  const bool rvalid = r < qt.row_end - qt.row_lo;
  const int j0 = threadIdx.x % TPR;
  __shared__ int64_t part[64];
  __shared__ int64_t starts[65];
  __shared__ int n_part;
  const int first_slot = it.start == lean_range_start(a, c_first) ? 0 : 1;
  float m = -INFINITY, sum = 0.f;
  float4 acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = c_first; c0 <= c_last; c0 += 64) {
    __syncthreads();
    // the starts of ranges c0 .. c0 + 64, one per thread, then the list
    const int nc = min(c_last, c0 + 63) - c0 + 1;
    if (int(threadIdx.x) <= nc) starts[threadIdx.x] = lean_range_start(a, c0 + int(threadIdx.x));
    __syncthreads();
    if (threadIdx.x == 0) {
      int n = 0;
      for (int i = 0; i < nc; ++i) {
        const int c = c0 + i;
        if (starts[i + 1] > starts[i])  // ranges with no unit wrote nothing
          part[n++] = (int64_t(c) * 2 + (c == c_first ? first_slot : 0)) * kRowsBf16;
      }
      n_part = n;
    }
    __syncthreads();
    if (!rvalid) continue;
    const int n = n_part;
    // partials in batches of kMergeBatch: every load of a batch is issued
    // before any is used (an item cut into many ranges, as the left-over
    // items of whole-item rounds are, would otherwise wait one memory
    // latency per partial); they are combined in the same order as one by one
    constexpr int kMergeBatch = 4;
    for (int k0 = 0; k0 < n; k0 += kMergeBatch) {
      float lb[kMergeBatch];
      float4 xb[kMergeBatch][NV];
#pragma unroll
      for (int kk = 0; kk < kMergeBatch; ++kk) {
        lb[kk] = -INFINITY;
        if (k0 + kk < n) {
          const int64_t pr = part[k0 + kk] + r;
          lb[kk] = a.part_lse[pr];
#pragma unroll
          for (int v = 0; v < NV; ++v)
            xb[kk][v] = *reinterpret_cast<const float4*>(a.part_o + pr * D + 4 * (j0 + TPR * v));
        }
      }
#pragma unroll
      for (int kk = 0; kk < kMergeBatch; ++kk) {
        const float l = lb[kk];
        if (l == -INFINITY) continue;
        const float4* x = xb[kk];
        const float m_new = fmaxf(m, l);
        const float sc = __expf(m - m_new);  // 0 while m is -inf
        const float w = __expf(l - m_new);
        sum = sum * sc + w;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          acc[v].x = acc[v].x * sc + w * x[v].x;
          acc[v].y = acc[v].y * sc + w * x[v].y;
          acc[v].z = acc[v].z * sc + w * x[v].z;
          acc[v].w = acc[v].w * sc + w * x[v].w;
        }
        m = m_new;
      }
    }
  }
  if (!rvalid) return;
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  const int q = qt.row_lo + r;
  __bf16* op = static_cast<__bf16*>(a.o) + ((int64_t(it.b) * a.Nq + q) * g.H + it.head) * D;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const __bf16 v0 = static_cast<__bf16>(acc[v].x * inv), v1 = static_cast<__bf16>(acc[v].y * inv);
    const __bf16 v2 = static_cast<__bf16>(acc[v].z * inv), v3 = static_cast<__bf16>(acc[v].w * inv);
    uint2 w;
    w.x = uint32_t(__builtin_bit_cast(uint16_t, v0)) | (uint32_t(__builtin_bit_cast(uint16_t, v1)) << 16);
    w.y = uint32_t(__builtin_bit_cast(uint16_t, v2)) | (uint32_t(__builtin_bit_cast(uint16_t, v3)) << 16);
    *reinterpret_cast<uint2*>(op + 4 * (j0 + TPR * v)) = w;
  }
  if (a.lse && j0 == 0) a.lse[(int64_t(it.b) * g.H + it.head) * a.Nq + q] = sum > 0.f ? m + __logf(sum) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_lean_merge(const AttnArgs& a, hipStream_t s) {
  const int nch = a.n_qtiles / a.qtiles_per_chunk;
  int per_head = 0;
  for (int ch = 0; ch < nch; ++ch)
    per_head += (std::min(a.rows_per_chunk, a.Nq - ch * a.rows_per_chunk) + kRowsBf16 - 1) / kRowsBf16;
  dim3 grid(unsigned(per_head * a.g.H * a.g.B - a.lean_v0), kRowsBf16 / kMergeRows);
  if (a.g.D == 128)
    hipLaunchKernelGGL(attn_lean_merge_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_lean_merge_kernel<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_chunk_attention(const AttnArgs& a, hipStream_t s) {
  // grid schedule: one workgroup per (query tile, head, stream * splits);
  // balanced schedule: lean_ctas workgroups over the unit ranges
  if (a.lean && (a.g.dtype != SCV_BF16 || a.lean_ctas < 1)) return hipErrorInvalidValue;
  dim3 grid = a.lean ? dim3(unsigned(a.lean_ctas)) : dim3(a.n_qtiles, a.g.H, a.g.B * a.splits);
  if (a.g.dtype == SCV_BF16) {
    const bool f16 = a.g.qk_dtype == SCV_FP16;
    if (a.g.D == 128) {
      if (f16)
        hipLaunchKernelGGL((chunk_attn_bf16_kernel<128, _Float16>), grid, dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((chunk_attn_bf16_kernel<128, __bf16>), grid, dim3(512), 0, s, a);
    } else {
      if (f16)
        hipLaunchKernelGGL((chunk_attn_bf16_kernel<64, _Float16>), grid, dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((chunk_attn_bf16_kernel<64, __bf16>), grid, dim3(512), 0, s, a);
    }
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
