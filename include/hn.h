/*
 * hn.h - segment-causal, action-aware attention over an INT8 sliding-window
 * KV cache, for one AMD Instinct MI355X (gfx950).
 *
 * The method is the attention of the Hy-Nomas segment-autoregressive MMDiT
 * as described on these pages:
 *   [T] fluxbbs.com, "Hy-Nomas 拆解：8B 世界模型用 20.53 GiB 显存跑 100 秒"
 *       (section "架构" = architecture; "单卡 4090 怎么做到的" = how one 4090
 *       does it; "训练流程" = training)
 *   [H] hyphentech.top, "腾讯 Hy-Nomas 开放权重：一张 RTX 4090 能跑怎样的交互式视频世界？"
 *       (section "标准方案和单卡方案不是同一套成本", its configuration table
 *       and the warning under it)
 *   [G] papers.ananclaw.com, "Hy-Nomas：腾讯混元开源的自由交互世界生成模型 · 干货攻略"
 *       (section "这是什么" = what it is: model-card architecture and method
 *       paragraph; "离线 prompt JSON 格式" = prompt JSON format)
 *
 * Conventions shared by every entry point
 *  - Every function returns hn_status; HN_OK (0) on success.  Nothing prints,
 *    throws or exits.  On failure hn_last_error() holds a message for the
 *    calling thread.
 *  - All argument checks happen on the host before anything is enqueued.  A
 *    call that fails enqueues no GPU work and leaves the cache counters
 *    unchanged.  Kernel launch failures map to HN_ERR_HIP.  Faults inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Device buffers are allocated by the caller, must stay alive until the
 *    enqueued work completes, and are never freed by the library.  The
 *    library allocates no device memory and never synchronises the stream.
 *  - bf16 tensors supplied by the caller are token-major [tokens][H][D],
 *    rows contiguous, D = HN_HEAD_DIM = 128 (the MMDiT uses 16 heads of 128
 *    dims: [G] "这是什么", architecture bullet).  The INT8 cache is the
 *    library's own head-major layout (below).
 *  - Work runs on the given HIP stream (0 = the null stream).
 *  - Outputs are bitwise reproducible from run to run: tile order is fixed
 *    and no reduction uses atomics.
 */
#ifndef HN_H
#define HN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HN_HEAD_DIM 128
#define HN_MAX_ACTIONS 64   /* action tails per segment */
#define HN_TILE 128         /* query/key tile of block-sparse keep lists */

typedef enum {
  HN_OK = 0,
  HN_ERR_NULL = 1,         /* a required pointer is NULL */
  HN_ERR_INVALID = 2,      /* inconsistent sizes or layout */
  HN_ERR_UNSUPPORTED = 3,  /* valid but not supported (e.g. head_dim != 128) */
  HN_ERR_CAPACITY = 4,     /* description-head store or buffer too small */
  HN_ERR_WORKSPACE = 5,    /* workspace / output buffer too small */
  HN_ERR_ORDER = 6,        /* segment order or stale tile plan */
  HN_ERR_HIP = 7           /* a HIP runtime call failed */
} hn_status;

const char* hn_status_string(hn_status s);
/* Message of the last failing call made by this thread ("" if none). */
const char* hn_last_error(void);

/* Token layout of the current segment (host memory, read during the call).
 *
 * A segment carries text then video.  Its text is one description head,
 * visible to every later segment, followed by m action tails; tail j is
 * visible only to this segment's video queries whose latent frame lies in
 * its time window ([T] "架构", action-aware causal attention; [G] prompt
 * JSON: each segment lists contained_actions with start/end times).
 * Text rows are ordered head, tail_0 .. tail_{m-1}; video rows are
 * frame-major, tokens_per_frame tokens per latent frame.
 * Windows are half-open in local latent frames: 0 <= f0 <= f1 <= frames.
 */
typedef struct hn_seg_layout {
  int32_t index;              /* 0-based segment index; must equal cache->segments */
  int32_t frames;             /* F latent frames (>= 1) */
  int32_t tokens_per_frame;   /* P, must equal cache->tokens_per_frame */
  int32_t head_len;           /* h description-head tokens (>= 0) */
  int32_t num_actions;        /* m action tails (0 .. HN_MAX_ACTIONS) */
  int32_t reserved0;
  const int32_t* action_len;  /* [m] tokens per tail (>= 0) */
  const int32_t* action_f0;   /* [m] first latent frame of the window */
  const int32_t* action_f1;   /* [m] one past the last latent frame */
} hn_seg_layout;

/* The INT8 KV cache of earlier segments.
 *
 * Keys and values are stored as INT8 with one fp32 scale per (token, head)
 * and computed in 16-bit floating point ([T] "单卡 4090 怎么做到的", first
 * technique: INT8 storage, BF16 compute; see hn_seg_attn_fwd for the 16-bit
 * type the history takes).  Video of
 * earlier segments lives in a ring of W latent frames, oldest frame evicted
 * first ([T] same section, second technique: 18 history frames; [H]
 * configuration table, history row).  Description heads of every earlier
 * segment live in a separate head store, since heads stay visible across
 * segments ([T] "架构").  Tails are never stored: no later segment sees them.
 *
 * Device buffers (caller-allocated; sizes from hn_kv_cache_sizes):
 *   ring_k, ring_v   int8  [H][W*P][D]   token t of ring slot s at row s*P+t
 *   ring_ks, ring_vs fp32  [H][W*P]
 *   heads_k, heads_v int8  [H][head_cap][D], heads of segments 0,1,.. in order
 *   heads_ks, heads_vs fp32 [H][head_cap]
 * Global latent frame g (frames of all earlier segments + local frame) lives
 * in ring slot g mod W.  The counters are host-side and updated by
 * hn_kv_quant_append; zero them (or call hn_kv_cache_reset) for a new video.
 * The whole struct is plain data: saving it and the buffers saves the cache.
 * With no window, give W >= the total number of latent frames.
 */
typedef struct hn_kv_cache {
  int32_t num_heads;          /* H >= 1 */
  int32_t head_dim;           /* D, must be 128 */
  int32_t tokens_per_frame;   /* P >= 1 */
  int32_t window_frames;      /* W >= 1, ring capacity in latent frames */
  int32_t head_cap_tokens;    /* head-store capacity in tokens (>= 0) */
  int32_t reserved0;
  int8_t* ring_k;
  int8_t* ring_v;
  float* ring_ks;
  float* ring_vs;
  int8_t* heads_k;
  int8_t* heads_v;
  float* heads_ks;
  float* heads_vs;
  int64_t frames_seen;        /* latent frames appended so far */
  int32_t head_tokens;        /* valid tokens in the head store */
  int32_t segments;           /* segments appended so far */
} hn_kv_cache;

/* Bytes of each cache buffer for the given shape (any output may be NULL). */
hn_status hn_kv_cache_sizes(int32_t num_heads, int32_t window_frames, int32_t tokens_per_frame,
                            int32_t head_cap_tokens, size_t* ring_bytes, size_t* ring_scale_bytes,
                            size_t* heads_bytes, size_t* heads_scale_bytes);
/* Zero the counters (frames_seen, head_tokens, segments); buffers untouched. */
hn_status hn_kv_cache_reset(hn_kv_cache* cache);

/* Quantize the current segment's keys/values and append them to the cache.
 *
 * Per (token, head) row x of 128 bf16 values, in IEEE fp32:
 *   amax = max|x_i|;  scale = amax / 127 (correctly rounded);
 *   q_i = round_half_even(x_i / scale) (correctly rounded quotient), clamped
 *   to [-127, 127]; a row with amax == 0 stores scale 0 and q 0.
 * (The pages state INT8 storage with float scales only, [T] first
 * technique; this formula is the library's reading of it.)
 * Written: the head rows [0, h) of k_txt/v_txt into the head store at
 * [head_tokens, head_tokens + h); the last min(F, W) latent frames of
 * k_vid/v_vid into ring slots (frames_seen + f) mod W.  Frames the window
 * drops at once, and the action tails, are not read.
 * Then frames_seen += F, head_tokens += h, segments += 1.
 *
 * k_txt, v_txt : bf16 [h + sum(a)][H][D] (device); may be NULL if h == 0
 * k_vid, v_vid : bf16 [F*P][H][D] (device)
 * Errors: HN_ERR_ORDER if seg->index != cache->segments; HN_ERR_CAPACITY if
 * the head store would overflow; HN_ERR_INVALID on inconsistent shapes.
 * Call it after every hn_seg_attn_fwd of the segment (the cache must not
 * yet hold the segment the queries belong to).
 */
hn_status hn_kv_quant_append(hn_kv_cache* cache, const hn_seg_layout* seg,
                             const void* k_txt, const void* v_txt,
                             const void* k_vid, const void* v_vid,
                             hipStream_t stream);

/* Host archive of history frames that left the GPU window.
 *
 * The single-GPU configuration keeps a window of W history frames on the GPU
 * and archives earlier history to CPU memory ([H] configuration table,
 * history row; [T] "单卡 4090 怎么做到的", second technique).  The archive holds,
 * in global frame order, the INT8 codes and scales of every frame the ring
 * gave up, exactly as the ring held them, so that hn_kv_cache_rewind can put
 * them back.  Frames a single segment longer than W drops at once were never
 * in the ring and are not archived.
 *
 * Buffers are host memory allocated by the caller, pinned (hipHostMalloc) so
 * that the copies run asynchronously on the stream; head-major like the ring:
 *   k, v   int8 [H][cap_frames*P][D]   archived frame i, token t at row i*P+t
 *   ks, vs fp32 [H][cap_frames*P]
 * Archived frame i is global latent frame first_frame + i.  The counters are
 * host-side; zero them for a new video.
 */
typedef struct hn_kv_archive {
  int8_t* k;
  int8_t* v;
  float* ks;
  float* vs;
  int32_t cap_frames;         /* capacity in latent frames */
  int32_t reserved0;
  int64_t first_frame;        /* global frame of archived frame 0 */
  int64_t frames;             /* frames held */
} hn_kv_archive;

/* Enqueue device-to-host copies of the ring frames that
 * hn_kv_quant_append(cache, seg, ...) is about to overwrite: appending F
 * frames after frames_seen = fs with window W evicts global frames
 * [fs - min(fs, W), max(that, min(fs, fs + F - min(fs + F, W)))).  Call it
 * right before that append, on the same stream (or one ordered before it);
 * the copies finish before the append's kernel starts overwriting.  Appends
 * archive->frames; the first eviction into an empty archive sets
 * first_frame.  Errors: HN_ERR_ORDER if seg->index != cache->segments or the
 * frames do not continue the archive; HN_ERR_CAPACITY if they do not fit
 * (nothing enqueued either way).
 */
hn_status hn_kv_archive_evict(const hn_kv_cache* cache, const hn_seg_layout* seg,
                              hn_kv_archive* archive, hipStream_t stream);

/* Rewind the cache to an earlier segment boundary: the state right after
 * `segments` segments were appended, when it had seen `frames_seen` latent
 * frames and held `head_tokens` head tokens (as saved from the counters at
 * that time).  History frames of that window which the ring has since given
 * up are copied back from the archive into their ring slots (host-to-device,
 * on the stream); frames the ring still holds stay; the archive keeps only
 * the frames older than that window; head tokens past head_tokens are
 * dropped.  Later appends continue from the rewound state.  Errors:
 * HN_ERR_INVALID if the target is not earlier than or equal to the current
 * counters; HN_ERR_CAPACITY if the archive lacks a frame the window needs.
 */
hn_status hn_kv_cache_rewind(hn_kv_cache* cache, hn_kv_archive* archive, int64_t frames_seen,
                             int32_t head_tokens, int32_t segments, hipStream_t stream);

/* Optional block-sparse keep list (device memory, caller-owned).
 *
 * After the first two denoising steps only 25% of the candidate video blocks
 * are kept ([T] "单卡 4090 怎么做到的", fourth technique).  Query tiles are
 * HN_TILE rows of the segment's video queries; video key tiles are HN_TILE
 * tokens, numbered first over the history video still in the window (oldest
 * frame first, ragged last tile), then over the segment's own video (ragged
 * last tile).  Row t of the CSR lists the video tiles query tile t keeps, in
 * strictly increasing order; ids out of range, repeated or out of order are
 * skipped.  Text (heads and visible tails) is always kept.
 */
typedef struct hn_block_sparse {
  int32_t tile_q;             /* must be HN_TILE */
  int32_t tile_k;             /* must be HN_TILE */
  int32_t n_qtiles;           /* must be ceil(F*P / HN_TILE) */
  int32_t reserved0;
  const int32_t* row_ptr;     /* [n_qtiles + 1], row_ptr[0] = 0, non-decreasing */
  const int32_t* col;         /* [row_ptr[n_qtiles]] video tile ids */
} hn_block_sparse;

typedef enum { HN_MASK_TILE_PLAN = 0, HN_MASK_DENSE = 1 } hn_mask_mode;

/* Optional choices of a tile plan (host memory, read during the call).  A
 * NULL pointer, or 0 in a field, leaves the choice to the library (below).
 * They exist for tuning and testing; every value gives the same attention up
 * to rounding. */
typedef struct hn_plan_opts {
  int32_t n_splits;           /* key splits per video query tile: 0 = automatic, else 1 .. 16 */
  int32_t n_splits_text;      /* key splits per text query tile: 0 = automatic, else 1 .. 16 */
  int32_t tile_rows;          /* query rows per tile of a plan without keep list: 0 = automatic
                                 (256 or 384, see hn_tile_plan), 128, 256 or 384; plans with a
                                 keep list always use HN_TILE */
  int32_t whole_tiles;        /* with n_splits > 1 forced: leading video query tiles that run
                                 unsplit (the others are split n_splits ways; >= n_qtiles: none
                                 split); 0 = every tile split.  Must be 0 when n_splits < 2 */
} hn_plan_opts;

/* Tile plan for one (cache state, segment, keep list); filled by
 * hn_attn_mask_build in TILE_PLAN mode and consumed by hn_seg_attn_fwd.
 * It may be reused by every attention call of the segment (all blocks and
 * denoising steps with the same keep list).  Tiles 0 .. n_qtiles-1 cover
 * the video queries, tiles n_qtiles .. n_qtiles+n_text_tiles-1 the text
 * queries (head and tails).
 * Split-KV: when (heads x video query tiles) would leave the GPU's block
 * slots (one per compute unit for 256- and 384-row tiles, two for 128-row
 * ones) poorly filled, query tiles' keys are split into n_splits contiguous
 * ranges that run as separate blocks; each writes a partial result into the
 * workspace and a merge kernel combines them (one softmax, exactly as
 * without the split up to rounding).  Either every video tile is split
 * (n_whole = 0), or only the tiles from n_whole on, so that the whole tiles
 * fill full rounds of blocks and the split pieces of the others the last
 * one.  The choice comes from the device's compute-unit count and the
 * layout (opts->n_splits and opts->whole_tiles force one).
 * Text query tiles, which follow all video tiles in a joint launch, get
 * their own count: the one (of 1, 2, 4, 8, 16) with the least estimated
 * makespan when the blocks are dealt to the slots in order, so that they
 * fill what the video blocks leave free; tiles of fewer than 4096 keys stay
 * whole (opts->n_splits_text forces a count).  Dense plans use 256- or
 * 384-row query tiles, whichever gives the smaller estimated makespan (the
 * 384-row block stages each key tile for more rows but leaves more compute
 * units idle on small grids); opts->tile_rows = 128, 256 or 384 forces a
 * height.  With n_splits > 1
 * attention calls that share one plan workspace must not overlap in time
 * (same stream, or ordered), since they write its partial area. */
typedef struct hn_tile_plan {
  const void* dev;            /* = the workspace the plan was written to */
  int32_t tile_q;             /* query rows per plan tile */
  int32_t n_qtiles;           /* video query tiles: ceil(F*P / tile_q) */
  int32_t n_text_tiles;       /* text query tiles: ceil((h + sum a) / tile_q) */
  int32_t max_spans;          /* span slots per query tile */
  int32_t seg_index;          /* cache/segment state the plan was built for */
  int32_t head_tokens;
  int64_t frames_seen;
  int32_t sparse;             /* 1 if a keep list was merged */
  int32_t n_splits;           /* key splits per video query tile (split-KV), 1 .. 16 */
  int64_t visible_pairs;      /* unmasked (video query, key) pairs per head; -1 if sparse */
  int64_t visible_pairs_text; /* unmasked (text query, key) pairs per head */
  int32_t n_splits_text;      /* key splits per text query tile, 1 .. 16 */
  int32_t n_whole;            /* leading video query tiles that run unsplit when n_splits > 1
                                 (0 .. n_qtiles-1); 0 when n_splits = 1 */
} hn_tile_plan;

/* Workspace bytes TILE_PLAN mode needs with the same opts (0 on invalid
 * arguments): the span lists, plus, with split-KV, H x (split tiles x
 * splits, plus the text tiles' pieces) x tile_q x (128 + 1) floats of
 * partial results. */
size_t hn_attn_workspace_size(const hn_kv_cache* cache, const hn_seg_layout* seg,
                              const hn_block_sparse* sparse, const hn_plan_opts* opts);

/* Build the attention mask of the current segment's queries.
 *
 * Visibility of key k for the video query at local frame f
 * ([T] "架构": segment-causal and action-aware attention; [H] warning under
 * the table: the window bounds history only):
 *   earlier segment's head            : always
 *   earlier segment's tails           : never (not in the cache)
 *   earlier video in the ring window  : always (evicted frames: never)
 *   own head                          : always
 *   own tail j                        : iff action_f0[j] <= f < action_f1[j]
 *   own video                         : always (bidirectional in a segment)
 *   later segments                    : never (not in the cache yet)
 *   with a keep list: video keys only in the query tile's kept tiles.
 * Text queries (the segment's own head and tail tokens, which the MMDiT
 * attends jointly with its video) follow the same segment-causal rule; tail
 * windows are stated only for video frames, so the reading taken is: a token
 * of tail j sees tail j and no other tail, a head token sees no tail.  Keep
 * lists concern video query tiles only; text queries attend densely.
 *
 * opts (nullable): split counts and tile height (hn_plan_opts); in DENSE mode
 *   only tile_rows matters (the expansion is the same for every height).
 *   Invalid values give HN_ERR_INVALID.
 * TILE_PLAN: `out` is the workspace (>= hn_attn_workspace_size bytes, device,
 *   16-byte aligned).  For every query tile a kernel writes the list of key
 *   spans to visit, each classified against the tile's rows as full or
 *   partial (a row range then restricts it); empty spans are dropped.  `plan`
 *   is filled.  row0/nrows are ignored.
 * DENSE: `out` is uint8 [nrows][Lk] (device) for query rows
 *   [row0, row0 + nrows) -- rows [0, F*P) are the video queries, rows
 *   [F*P, F*P + h + sum(a)) the text queries -- in the canonical key order
 *   [history heads, oldest segment first | history video in the window,
 *    oldest frame first | own head | own tails | own video],
 *   Lk = head_tokens + kept_frames*P + h + sum(a) + F*P; 1 = visible.  It is
 *   expanded from the same span lists (a debugging and test view).  `plan`
 *   must be NULL.
 */
hn_status hn_attn_mask_build(const hn_kv_cache* cache, const hn_seg_layout* seg,
                             const hn_block_sparse* sparse, const hn_plan_opts* opts, hn_mask_mode mode,
                             int32_t row0, int32_t nrows, void* out, size_t out_bytes,
                             hn_tile_plan* plan, hipStream_t stream);

/* Attention of the current segment's video queries (and, if q_txt is given,
 * its text queries) over the cache and the segment's own text and video,
 * with one softmax over the union of visible keys (the mask of
 * hn_attn_mask_build); one launch covers both query sets:
 *   O[q] = sum_k softmax_k(sm_scale * Q[q].K[k]) V[k]
 * History keys/values are the dequantized INT8 values q*scale; the segment's
 * own keys/values are used as given (quantization is storage-only,
 * [T] "单卡 4090 怎么做到的", first technique).  16-bit MFMA with fp32
 * accumulation and online softmax: the segment's own tiles in BF16 (its
 * inputs' type); the history tiles in FP16 (q times the scale rounded to
 * FP16, the product rounded to FP16: within 2^-10 of q*scale for rows whose
 * largest |value| is at least 0.0078, within 4e-6 absolute below that,
 * against an FP16 copy of Q), which keeps the history nearly as close to
 * q*scale as the segment's own values are to their inputs.  The
 * FP16 path holds history values with |K| <= 65,024 and |V| <= 8.3e6; a tile
 * outside that range sends its query tile through BF16 for every key.
 *
 * plan         : from hn_attn_mask_build(TILE_PLAN) for this exact cache
 *                state and segment, workspace still intact; else HN_ERR_ORDER
 * q_vid        : bf16 [F*P][H][D]
 * q_txt        : bf16 [h + sum(a)][H][D] text queries, or NULL to skip them
 * k_txt, v_txt : bf16 [h + sum(a)][H][D] (may be NULL if h + sum(a) == 0)
 * k_vid, v_vid : bf16 [F*P][H][D]
 * o_vid        : bf16 [F*P][H][D] (output; must not alias the inputs)
 * o_txt        : bf16 [h + sum(a)][H][D] output of the text queries; required
 *                iff q_txt is given and h + sum(a) > 0
 * lse, lse_txt : fp32 [H][F*P] / [H][h + sum(a)] natural-log softmax
 *                normalisers, or NULL
 * sm_scale     : score scale > 0, normally 1/sqrt(128) (else HN_ERR_INVALID)
 */
hn_status hn_seg_attn_fwd(const hn_kv_cache* cache, const hn_seg_layout* seg,
                          const hn_tile_plan* plan, const void* q_vid, const void* q_txt,
                          const void* k_txt, const void* v_txt,
                          const void* k_vid, const void* v_vid,
                          void* o_vid, void* o_txt, float* lse, float* lse_txt,
                          float sm_scale, hipStream_t stream);

/* Bytes of the library's own plan buffer for hn_seg_attn_fwd_noalloc: one
 * per GPU the library runs on, held until the process ends. */
#define HN_NOALLOC_PLAN_BYTES (4u << 20)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the tile
 * plan (hn_attn_mask_build, TILE_PLAN mode) and the attention
 * (hn_seg_attn_fwd) in one call, with the plan written to a device buffer of
 * the library's own (HN_NOALLOC_PLAN_BYTES per GPU, a static array) instead
 * of a caller workspace.  Nothing is allocated: the buffer's address on the
 * current device is looked up once, on the first call on that device.  Its
 * plans never split keys (split-KV partial results would need far more
 * memory), so the outputs equal, bit for bit, those of hn_seg_attn_fwd with a
 * plan built with opts n_splits = n_splits_text = 1.
 * Arguments: as hn_seg_attn_fwd, with `sparse` (nullable) as in
 * hn_attn_mask_build.  Every call on one GPU shares that GPU's buffer and
 * leaves its plan there: calls that overlap in time on one GPU (streams not
 * ordered against each other) race; serialise them.
 * Errors: as hn_seg_attn_fwd and hn_attn_mask_build; HN_ERR_WORKSPACE if the
 * plan needs more than HN_NOALLOC_PLAN_BYTES (keep lists of very long
 * segments); HN_ERR_HIP if the buffer's address cannot be obtained.  All are
 * returned before anything is enqueued.
 */
hn_status hn_seg_attn_fwd_noalloc(const hn_kv_cache* cache, const hn_seg_layout* seg,
                                  const hn_block_sparse* sparse, const void* q_vid, const void* q_txt,
                                  const void* k_txt, const void* v_txt, const void* k_vid,
                                  const void* v_vid, void* o_vid, void* o_txt, float* lse,
                                  float* lse_txt, float sm_scale, hipStream_t stream);

/* Camera cross-attention of the current segment's video tokens.
 *
 * Each latent frame carries one camera token (four consecutive frame poses
 * folded into a 64-dimensional vector, linearly projected with a residual
 * MLP), and in every MMDiT block the video tokens read the time-aligned
 * camera tokens of their own segment by cross-attention; relative poses are
 * computed inside the segment ([T] "架构", camera paragraph; [G] "这是什么",
 * extrinsics cross-attention path).  The projections need trained weights
 * and are outside this library: the camera tokens' keys and values come in.
 * The video token at local latent frame f sees camera tokens f' of the same
 * segment with |f' - f| <= radius:
 *   O[q] = sum_{f'} softmax(sm_scale * Q[q].K_cam[f']) V_cam[f']
 * radius 0 is the stated time alignment (one key, weight exactly 1: O is
 * the frame's camera value); larger radii widen it.
 *
 * q_vid        : bf16 [F*P][H][D] (device)
 * k_cam, v_cam : bf16 [F][H][D] (device), one token per latent frame
 * o_vid        : bf16 [F*P][H][D] (output; must not alias the inputs)
 * lse          : fp32 [H][F*P] natural-log softmax normaliser, or NULL
 * Errors: HN_ERR_NULL, HN_ERR_INVALID (shape, radius < 0, non-finite scale),
 * HN_ERR_UNSUPPORTED (F*P*H of 2^28 (token, head) rows or more).
 */
hn_status hn_camera_attn_fwd(const hn_seg_layout* seg, int32_t num_heads, int32_t radius,
                             const void* q_vid, const void* k_cam, const void* v_cam,
                             void* o_vid, float* lse, float sm_scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HN_H */
