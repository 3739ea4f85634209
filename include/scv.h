/*
 * scv.h -- streaming chunk attention for MI355X (gfx950): 3D RoPE at a
 * global time index, a sink-pinned ring KV cache, and block-causal
 * attention of a new chunk of latent-frame tokens over sink + window +
 * chunk.  Every call enqueues hand-written HIP kernels on the caller's
 * stream; the library never allocates device memory.
 *
 * Sources (cited by page title and section):
 *  - "StreamDiffusionV2: A Streaming System for Dynamic and Interactive
 *    Video Generation" (paper-review blog), section 2 "core idea": the KV of
 *    the initial frame(s) is a pinned global anchor (sink), the rest of the
 *    cache is a fixed-size sliding window, and the RoPE offset is refreshed.
 *  - "Accelerating Video Generation Inference with Sequential-Parallel 3D
 *    Positional Encoding Using a Global Time Index" (gist.science summary),
 *    section 2(b): the start frame of each generated block is the global
 *    time index, so token time positions need no communication; section
 *    2(c): RoPE cos/sin are precomputed into contiguous tables instead of a
 *    host-side cache.
 *
 * Conventions (readings where the pages are silent):
 *  - Token order inside a call is frame-major then row-major:
 *    token n = f*P + y*grid_w + x, P = grid_h*grid_w, with global time
 *    t = t0[b] + f, row y and column x (all 0-based).
 *  - Head dims [0,d_t) rotate with t, [d_t,d_t+d_h) with y, the rest with x;
 *    adjacent pairs (2j, 2j+1) of an axis block of width d_a rotate by
 *    theta = pos * omega_j, omega_j = rope_base^(-2j/d_a): the fp64 product
 *    of the integer position and omega_j (omega_j = libm pow of the fp64
 *    exponent -(2j)/d_a, computed once per cache on the host); cos/sin are
 *    evaluated in fp64 and rounded to fp32; the rotation runs in fp32 and
 *    rounds once to the storage dtype (round to nearest even).
 *  - Frame g < sink_frames lives in sink slot g (pinned); any later frame g
 *    lives in ring slot sink_frames + (g mod R), R = window_frames +
 *    max_query_chunks * chunk_frames.  Each slot is stamped with the global
 *    frame it holds (-1 = empty).
 *  - Query frames of stream b are t0[b] .. t0[b]+n_frames-1, grouped into
 *    chunks of chunk_frames frames from t0[b].  A query of the chunk that
 *    starts at frame s sees the key of a slot stamped with frame g iff
 *    g < s + chunk_frames and (the slot is a sink slot, or
 *    g >= s - window_frames): block-causal at chunk granularity over sink +
 *    window + its own chunk.  Scores are scaled by 1/sqrt(head_dim).  A
 *    query that sees no key gets O = 0, lse = -inf.
 *  - The time position of frame g of stream b is g - offset[b]; offset[b]
 *    starts at 0 (scv_cache_init) and grows by RoPE refreshes
 *    (scv_rope_refresh).  Frames, stamps and slots are always global frame
 *    indices; only the RoPE angles use time positions.
 *
 * Tensor layouts (device memory, caller-owned, 16-byte aligned, dense):
 *  q, k, v, o : [batch][n_frames*P][heads][head_dim] in the cache dtype;
 *               rotated q and k (q_rot, k_rot) in the cache's qk_dtype.
 *  lse        : [batch][heads][n_frames*P] fp32 (natural log).
 *  t0         : HOST array int64[batch], read during the call only and passed
 *               to the kernels by value (no host sync, no device read).
 *  stream     : a hipStream_t (NULL = the default stream).  All work of a call
 *               is enqueued on it in call order; a cache must be used by one
 *               stream at a time.
 *
 * Errors: every entry point validates its arguments first and returns a
 * negative scv_status with nothing enqueued; SCV_E_HIP reports a failed
 * launch (message in scv_last_error()).  Asynchronous device faults surface
 * at the caller's next synchronisation.  No C++ exception crosses the ABI.
 */
#ifndef SCV_H
#define SCV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum scv_status {
  SCV_OK = 0,
  SCV_E_INVALID = -1,   /* null handle/pointer or invalid config value      */
  SCV_E_SHAPE = -2,     /* n_frames or size out of the supported range      */
  SCV_E_DTYPE = -3,     /* dtype / head_dim combination not supported       */
  SCV_E_ALIGN = -4,     /* a device pointer is not 16-byte aligned          */
  SCV_E_RANGE = -5,     /* a time index outside [0, 2^40)                   */
  SCV_E_STATE = -6,     /* cache buffer too small for the config            */
  SCV_E_WORKSPACE = -7, /* workspace missing or smaller than required       */
  SCV_E_HIP = -8        /* a HIP runtime call or kernel launch failed       */
} scv_status;

typedef enum scv_dtype { SCV_FP32 = 0, SCV_BF16 = 1, SCV_FP16 = 2 } scv_dtype;

/* Shape of one streaming cache; every stream of the batch shares it. */
typedef struct scv_config {
  int32_t batch;            /* streams B, 1..64                              */
  int32_t heads;            /* H >= 1                                        */
  int32_t head_dim;         /* d: 64 or 128                                  */
  int32_t rope_split[3];    /* d_t, d_h, d_w: even, >= 2, sum = head_dim     */
  double rope_base;         /* > 1                                           */
  int32_t grid_h, grid_w;   /* latent grid, P = grid_h*grid_w <= 2^20        */
  int32_t sink_frames;      /* S_f >= 0                                      */
  int32_t window_frames;    /* W >= 0                                        */
  int32_t chunk_frames;     /* C >= 1                                        */
  int32_t max_query_chunks; /* k, 1..8; ring R = W + k*C; S_f + R <= 64      */
  int32_t dtype;            /* scv_dtype of q, k, v, o (SCV_FP32, SCV_BF16)  */
  int32_t qk_dtype;         /* format of the ROTATED q and k (q_rot, cached  */
                            /* keys) and of the QK^T MFMA operands:          */
                            /* 0 = same as dtype; SCV_FP16 (dtype SCV_BF16   */
                            /* only) keeps 3 more mantissa bits at the same  */
                            /* MFMA rate for inputs whose rotated values     */
                            /* stay within +-65504; a rotated value beyond   */
                            /* that range is stored saturated to +-65504     */
                            /* (finite: attention stays defined, but such    */
                            /* keys and queries are no longer exact)         */
} scv_config;

/* Byte layout of the caller's cache buffer (offsets from its base). */
typedef struct scv_cache_layout {
  size_t total_bytes;
  size_t stamps_offset;  /* int64 [B][n_slots]: frame held by each slot      */
  size_t table_h_offset; /* fp32 [grid_h][d_h/2][2]: cos, sin of row angles  */
  size_t table_w_offset; /* fp32 [grid_w][d_w/2][2]: cos, sin of col angles  */
  size_t k_offset;       /* qk_dtype [B][H][rows_pad][d]: rotated keys       */
  size_t v_offset;       /* dtype [B][H][d][rows_pad]: values, transposed    */
  int64_t n_slots;       /* S_f + R frame slots                              */
  int64_t ring_frames;   /* R                                                */
  int64_t slot_rows;     /* rows per slot: P rounded up to a multiple of 8   */
  int64_t rows;          /* n_slots * slot_rows; slot s owns rows            */
                         /* [s*slot_rows, s*slot_rows + P)                   */
  int64_t rows_pad;      /* rows rounded up to a multiple of 64              */
  int64_t elem_bytes;    /* 4 (fp32) or 2 (bf16)                             */
} scv_cache_layout;

typedef struct scv_cache scv_cache; /* opaque host-side descriptor */

/* Bytes of device memory a cache with this config needs (0 if the config
 * is invalid; scv_last_error() then says why). */
size_t scv_cache_bytes(const scv_config* cfg);

/* Layout of the cache buffer for this config (host only). */
scv_status scv_cache_layout_of(const scv_config* cfg, scv_cache_layout* out);

/* Create a host descriptor over a caller-owned device buffer of at least
 * scv_cache_bytes(cfg) bytes (256-byte aligned).  No device work; the
 * buffer must outlive the handle.  Per-cache constants are fixed here: the
 * RoPE frequency ladders omega (fp64, libm pow).  Call scv_cache_init
 * before any other call on the handle. */
scv_status scv_cache_create(const scv_config* cfg, void* dev_buf, size_t bytes, scv_cache** out);

/* Free the host descriptor (never the device buffer).  NULL is a no-op. */
scv_status scv_cache_destroy(scv_cache* c);

/* cache_init(sink).  Zeroes the key/value region, marks every slot empty,
 * and computes the static fp32 cos/sin tables of the row and column axes.
 * If sink_k and sink_v are non-NULL they hold the raw (unrotated) k and v
 * of the sink frames 0..S_f-1 ([B][S_f*P][H][d]); they are rotated at global
 * times 0..S_f-1 and written into the pinned sink slots (the initial frames'
 * KV as the global anchor, StreamDiffusionV2 review, section 2). */
scv_status scv_cache_init(scv_cache* c, const void* sink_k, const void* sink_v, void* stream);

/* rope3d_apply(q, k, t0, grid).  Rotates q and/or k in place by split t/h/w
 * RoPE at global time t0[b] + f (Causal-RoPE SP paper, section 2(b)); the
 * spatial grid is the cache's.  The rotated values are written in the
 * cache's qk_dtype (with SCV_FP16 the buffers then hold fp16 values).
 * Either pointer may be NULL (not both).  1 <= n_frames <= 65535 and
 * n_frames*P < 2^31. */
scv_status scv_rope3d_apply(const scv_cache* c, void* q, void* k, const int64_t* t0, int32_t n_frames,
                            void* stream);

/* kv_append_roll(chunk): the rolling KV cache with its sink anchor of the
 * StreamDiffusionV2 review (section 2: the initial frames' KV stay pinned as
 * the global anchor, the rest of the cache is a fixed-size window that rolls
 * forward with the stream).  Writes the already-rotated keys k_rot (qk_dtype)
 * and the values v of frames t0[b] .. t0[b]+n_frames-1 into their slots
 * (sink frames into the pinned sink, later frames into the ring, evicting
 * what the slot held) and stamps the slots.  Among the frames of one call at most R may
 * be ring frames.  Appending the same frames again is idempotent. */
scv_status scv_kv_append_roll(scv_cache* c, const void* k_rot, const void* v, const int64_t* t0, int32_t n_frames,
                              void* stream);

/* Fused rope3d_apply + kv_append_roll in one kernel (the Causal-RoPE SP
 * paper, section 2(c), fuses RoPE with its neighbouring operator to save
 * launches and memory passes; here the neighbour is the cache append, one
 * HBM pass instead of three).  q is rotated into q_rot
 * (qk_dtype; q_rot == q rotates in place), k is rotated and written with v
 * into the cache; k itself is not modified.  q and q_rot may both be NULL
 * (append only). */
scv_status scv_rope3d_append(scv_cache* c, const void* q, void* q_rot, const void* k, const void* v,
                             const int64_t* t0, int32_t n_frames, void* stream);

/* QKV projection fused with 3D RoPE and the append (Causal-RoPE SP paper,
 * section 2(c): the projection and Causal-RoPE run as one kernel).  For the
 * layer input x ([B][n_frames*P][d_model], dtype SCV_BF16 only) of frames
 * t0[b] .. t0[b]+n_frames-1 and the weight w_qkv ([3*H*d][d_model]: rows
 * 0 .. H*d-1 are the q features, feature h*d + i being dim i of head h, then
 * the k features, then the v features), computes q, k, v = x w^T with fp32
 * accumulation (no bias, no normalisation), rotates q into q_rot
 * ([B][n_frames*P][H][d], qk_dtype) and k into the cache, writes v into the
 * cache and stamps the slots -- the same result as scv_rope3d_append on the
 * projected q, k, v, except that q, k and v are rounded once, after RoPE.
 * d_model: a multiple of 32 in [32, 65536], with n_frames*P*d_model*2 < 2^31.
 * Frame rules as for scv_kv_append_roll. */
scv_status scv_qkv_rope_append(scv_cache* c, const void* x, int32_t d_model, const void* w_qkv, void* q_rot,
                               const int64_t* t0, int32_t n_frames, void* stream);

/* RoPE refresh (StreamDiffusionV2 review, section 2, and the gist.science
 * StreamDiffusionV2 summary, section 2.A.2: the position offset is reset
 * periodically so positions stay bounded on long streams).  Moves stream b's
 * time origin forward by delta[b] frames: the time pairs of every cached key
 * of stream b (sink and ring) are turned by -delta[b] * omega_t -- angle the
 * fp64 product delta[b] * omega_j, cos/sin rounded to fp32, rotation in fp32,
 * one rounding to qk_dtype -- and the stream's offset grows by delta[b], so
 * later rotations use time position (frame - offset).  Values, stamps and
 * slots are unchanged; attention outputs change only by rounding.
 * delta: HOST array int64[batch], each >= 0 (0 = leave the stream alone),
 * with the new offset below 2^40.  Later calls must keep every time position
 * they rotate at >= 0 (SCV_E_RANGE otherwise).  Reads and writes the first
 * ceil(d_t * elem / 16) 16-byte chunks of every key row. */
scv_status scv_rope_refresh(scv_cache* c, const int64_t* delta, void* stream);

/* Current time offsets of the streams (host int64[batch], host only). */
scv_status scv_time_offsets(const scv_cache* c, int64_t* out);

/* Sink update (StreamDiffusionV2 review, section 2, and the gist.science
 * summary, section 2.A.2: the sink tokens are refreshed from recent
 * content; which frames to take is the caller's choice).  Sink slot j
 * (j < n_frames, 1 <= n_frames <= sink_frames) of stream b takes frame
 * first_frame[b] + j: k (raw, [B][n_frames*P][H][d] in the dtype) is rotated
 * at that frame's time position and written with v; the slot is stamped
 * with the frame.  Ring slots and the other sink slots are untouched.  A
 * sink slot is seen by every query chunk that does not end before its frame
 * (no window rule).  first_frame: HOST array int64[batch]. */
scv_status scv_sink_update(scv_cache* c, const void* k, const void* v, const int64_t* first_frame, int32_t n_frames,
                           void* stream);

/* scv_rope3d_append and a sink update from the same chunk in one launch (the
 * sink refreshed from recent content, as for scv_sink_update; the fusion of
 * neighbouring operators as in the Causal-RoPE SP paper, section 2(c)).  The
 * result equals scv_rope3d_append(c, q, q_rot, k, v, t0, n_frames) followed
 * by scv_sink_update on frames sink_first .. sink_first+sink_frames-1 of the
 * same k and v (first_frame[b] = t0[b] + sink_first): those frames' rotated
 * keys and values are written a second time, into sink slots 0 ..
 * sink_frames-1, which are stamped with the frames; nothing is read twice.
 * Needs sink_frames in [1, cache sink_frames], sink_first >= 0,
 * sink_first + sink_frames <= n_frames and every t0[b] >= the cache's
 * sink_frames (a chunk whose own frames would land in sink slots is
 * refused with SCV_E_RANGE: its two writes would target the same slot).
 * Other rules and errors as for scv_rope3d_append. */
scv_status scv_rope3d_append_sink(scv_cache* c, const void* q, void* q_rot, const void* k, const void* v,
                                  const int64_t* t0, int32_t n_frames, int32_t sink_first, int32_t sink_frames,
                                  void* stream);

/* Schedule chunk_attention will use for this request: a key split count
 * >= 1 (grid schedule: one workgroup per query tile, head and split), or
 * SCV_SCHEDULE_BALANCED = -1 (bf16 only: the work, counted in query-tile x
 * visited-key-tile units, is cut into equal ranges, a multiple of the
 * compute-unit count of them, each range at most as long as the shortest
 * query tile's key walk; a query tile cut by range boundaries leaves fp32
 * partials that a merge kernel combines -- this keeps every compute unit
 * busy when the query tiles do not fill whole rounds of the chip).
 * SCV_SCHEDULE_ROUNDS = -2 is the balanced schedule with whole-item rounds
 * (bf16 only, all query tiles visiting the same number of key tiles, more
 * of them than compute units): the first rounds run whole query tiles, one
 * per workgroup, with the compute units of an XCD on consecutive query
 * tiles of a head so that they share its keys and values in L2, and only
 * the query tiles left over are cut into equal ranges -- far less HBM
 * traffic (the 720p layer: 3.1x instead of 10.7x the algorithmic bytes) in
 * about the same time; kv_splits = 0 picks it where the model finds it
 * cheaper than the equal cut, and a request for it falls back to -1 where
 * it does not apply.
 * kv_splits > 0 asks for that many splits (capped at 64 and at the number
 * of 64-key tiles); kv_splits = -1 asks for the balanced schedule (the fp32
 * path, and tiles too short for it, fall back to one split).  kv_splits = 0
 * lets a makespan model choose among all of them from the device's compute-unit
 * count: with t0 (HOST int64[batch], nullable) it counts the key tiles each
 * stream's chunks visit; with t0 = NULL it assumes every chunk sees sink +
 * window + chunk (the steady state).  Only schedules whose workspace fits
 * ws_bytes are considered (SIZE_MAX: no limit).  Returns 0 on invalid
 * arguments. */
#define SCV_SCHEDULE_BALANCED (-1)
#define SCV_SCHEDULE_ROUNDS (-2)
int32_t scv_attention_splits(const scv_cache* c, const int64_t* t0, int32_t n_frames, int32_t kv_splits,
                             size_t ws_bytes);

/* Workspace bytes chunk_attention needs for this request with
 * kv_splits > 0, -1 or -2 (steady-state key counts), or the most the
 * steady-state choice of kv_splits = 0 needs (0 when it runs without
 * splits).  With kv_splits = 0, chunk_attention picks among the schedules
 * this workspace (and t0) allows. */
size_t scv_attention_workspace_bytes(const scv_cache* c, int32_t n_frames, int32_t kv_splits);

/* Workspace bytes of the schedule scv_attention_splits(c, t0, n_frames,
 * kv_splits, SIZE_MAX) selects, for these t0 (HOST int64[batch]); 0 on
 * invalid arguments or when the schedule needs none. */
size_t scv_attention_request_workspace_bytes(const scv_cache* c, const int64_t* t0, int32_t n_frames,
                                             int32_t kv_splits);

/* chunk_attention(q, cache) -> o: causal attention of the new chunk over the
 * KV cache (Causal-RoPE SP paper, sections 1 and 2(a): full spatio-temporal
 * attention of a generated block over the cached keys of earlier blocks)
 * restricted to the sink + rolling window of the StreamDiffusionV2 review,
 * section 2.  Block-causal attention of the rotated
 * queries q_rot (qk_dtype) of frames t0[b] .. t0[b]+n_frames-1
 * (1 <= n_frames <= k*C) over the cached frames each query may see; o gets
 * the normalised output in the cache dtype, lse (nullable) the natural-log
 * softmax normaliser.  QK^T and PV run on MFMA with fp32 accumulation
 * (qk_dtype operands for QK^T; dtype operands for PV), softmax in fp32; P is
 * rounded to the dtype before PV.  With more than one split, or the
 * balanced schedule, the pieces of a query tile write normalised fp32
 * partials into ws (256-byte aligned) and a merge kernel combines them
 * (lse-weighted).  kv_splits (-2, -1, 0 or a split count) chooses as
 * scv_attention_splits(c, t0, n_frames, kv_splits, ws ? ws_bytes : 0)
 * does; a forced schedule whose workspace exceeds ws_bytes fails with
 * SCV_E_WORKSPACE. */
scv_status scv_chunk_attention(const scv_cache* c, const void* q_rot, const int64_t* t0, int32_t n_frames, void* o,
                               float* lse, int32_t kv_splits, void* ws, size_t ws_bytes, void* stream);

/* chunk_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and schedule choice as scv_chunk_attention, with the
 * workspace taken from a static device array of SCV_SCRATCH_BYTES bytes that
 * the library holds on every GPU it runs on until the process ends.  The
 * call allocates nothing (no hipMalloc, no allocating library routine).
 * kv_splits = 0 chooses among the schedules whose workspace fits the
 * scratch; a forced schedule (kv_splits > 0, -1 or -2) that needs more fails
 * with SCV_E_WORKSPACE and nothing enqueued.  Every call on a GPU shares
 * that GPU's scratch: calls whose executions overlap on one GPU (several
 * streams, several threads) race and must be serialised by the caller.
 * Nothing in the scratch needs to start at zero: a call writes every part
 * of it that it reads. */
#define SCV_SCRATCH_BYTES ((size_t)128 << 20)
scv_status scv_chunk_attention_scratch(const scv_cache* c, const void* q_rot, const int64_t* t0, int32_t n_frames,
                                       void* o, float* lse, int32_t kv_splits, void* stream);

/* The fp32 cos/sin tables the kernels use for this request, written to the
 * device buffer out (fp32, n_floats >= scv_rope_table_floats(c, n_frames)):
 * [B][n_frames][d_t/2][2] for time, then [grid_h][d_h/2][2] for rows, then
 * [grid_w][d_w/2][2] for columns.  For checking only. */
size_t scv_rope_table_floats(const scv_cache* c, int32_t n_frames);
scv_status scv_rope_tables(const scv_cache* c, const int64_t* t0, int32_t n_frames, float* out, size_t n_floats,
                           void* stream);

/* The slot stamps (int64 [B][S_f + R]: the global frame each slot holds, -1
 * when empty) copied to the host array out (n >= B * (S_f + R) entries).
 * Synchronises the device first (every enqueued append has landed), so it is
 * meant for checking, not for the streaming loop. */
scv_status scv_debug_stamps(const scv_cache* c, int64_t* out, size_t n);

/* Message describing the last non-OK status on this thread. */
const char* scv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SCV_H */
