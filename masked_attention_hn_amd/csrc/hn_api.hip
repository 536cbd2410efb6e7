// Host side of the C ABI: argument checks, cache bookkeeping, launches.
//
// Every check runs before anything is enqueued; a failing call leaves the
// cache counters untouched.  Nothing here allocates device memory or
// synchronises a stream.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <mutex>
#include <queue>
#include <vector>

#include "hn_internal.h"

// The plan buffer of hn_seg_attn_fwd_noalloc.  Each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code this name is only a handle for hipGetSymbolAddress: kernels, copies and
// fills take the per-device address that call returns (scratch_address below).
static __device__ __align__(256) unsigned char scratch[HN_NOALLOC_PLAN_BYTES];

namespace {

thread_local char g_err[512] = "";

hn_status fail(hn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

hn_status ok() {
  g_err[0] = '\0';
  return HN_OK;
}

hn_status check_cache(const hn_kv_cache* c) {
  if (!c) return fail(HN_ERR_NULL, "cache is NULL");
  if (c->head_dim != HN_HEAD_DIM)
    return fail(HN_ERR_UNSUPPORTED, "head_dim %d unsupported (only %d)", c->head_dim, HN_HEAD_DIM);
  if (c->num_heads < 1) return fail(HN_ERR_INVALID, "num_heads %d < 1", c->num_heads);
  if (c->tokens_per_frame < 1) return fail(HN_ERR_INVALID, "tokens_per_frame %d < 1", c->tokens_per_frame);
  if (c->window_frames < 1) return fail(HN_ERR_INVALID, "window_frames %d < 1", c->window_frames);
  if (c->head_cap_tokens < 0) return fail(HN_ERR_INVALID, "head_cap_tokens %d < 0", c->head_cap_tokens);
  if ((int64_t)c->window_frames * c->tokens_per_frame > INT_MAX / 2)
    return fail(HN_ERR_UNSUPPORTED, "ring of %d x %d tokens too large", c->window_frames, c->tokens_per_frame);
  if (c->frames_seen < 0 || c->head_tokens < 0 || c->segments < 0 || c->head_tokens > c->head_cap_tokens)
    return fail(HN_ERR_INVALID, "cache counters are inconsistent");
  if (!c->ring_k || !c->ring_v || !c->ring_ks || !c->ring_vs)
    return fail(HN_ERR_NULL, "cache ring buffers are NULL");
  if (c->head_cap_tokens > 0 && (!c->heads_k || !c->heads_v || !c->heads_ks || !c->heads_vs))
    return fail(HN_ERR_NULL, "cache head-store buffers are NULL");
  return HN_OK;
}

hn_status check_seg(const hn_kv_cache* c, const hn_seg_layout* s, int64_t* text_len) {
  if (!s) return fail(HN_ERR_NULL, "segment layout is NULL");
  if (s->frames < 1) return fail(HN_ERR_INVALID, "frames %d < 1", s->frames);
  if (s->tokens_per_frame != c->tokens_per_frame)
    return fail(HN_ERR_INVALID, "segment tokens_per_frame %d != cache %d", s->tokens_per_frame,
                c->tokens_per_frame);
  if ((int64_t)s->frames * s->tokens_per_frame > INT_MAX / 2)
    return fail(HN_ERR_UNSUPPORTED, "segment of %d x %d tokens too large", s->frames, s->tokens_per_frame);
  if (s->head_len < 0) return fail(HN_ERR_INVALID, "head_len %d < 0", s->head_len);
  if (s->num_actions < 0 || s->num_actions > HN_MAX_ACTIONS)
    return fail(HN_ERR_UNSUPPORTED, "num_actions %d outside [0, %d]", s->num_actions, HN_MAX_ACTIONS);
  if (s->num_actions > 0 && (!s->action_len || !s->action_f0 || !s->action_f1))
    return fail(HN_ERR_NULL, "action arrays are NULL");
  int64_t tl = s->head_len;
  for (int j = 0; j < s->num_actions; ++j) {
    if (s->action_len[j] < 0) return fail(HN_ERR_INVALID, "action %d has length %d", j, s->action_len[j]);
    if (s->action_f0[j] < 0 || s->action_f0[j] > s->action_f1[j] || s->action_f1[j] > s->frames)
      return fail(HN_ERR_INVALID, "action %d window [%d, %d) not inside [0, %d]", j, s->action_f0[j],
                  s->action_f1[j], s->frames);
    tl += s->action_len[j];
  }
  if (tl > INT_MAX / 2) return fail(HN_ERR_UNSUPPORTED, "text of %lld tokens too large", (long long)tl);
  *text_len = tl;
  return HN_OK;
}

int kept_frames(const hn_kv_cache* c) {
  return (int)std::min<int64_t>(c->frames_seen, c->window_frames);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (256 on MI355X; also the answer when
// no device is visible, so that sizes computed on a host agree).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

// Per-block cost of the split models below, in key-equivalents on top of a
// block's keys: Q load, first tile, partial write, share of the merge; a
// constant fitted to same-run measurements of text splits.
constexpr double kBlockOverhead = 1600.0;

// Greedy list schedule: blocks dealt in order to the earliest free of the
// slots; deal() adds `count` blocks of cost `cost`.
struct SlotSim {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  explicit SlotSim(int64_t slots) {
    for (int64_t i = 0; i < slots; ++i) free_at.push(0.0);
  }
  void deal(int64_t count, double cost) {
    for (int64_t i = 0; i < count; ++i) {
      const double t = free_at.top();
      free_at.pop();
      free_at.push(t + cost);
    }
  }
  double end() {
    double t_end = 0.0;
    while (!free_at.empty()) {
      t_end = std::max(t_end, free_at.top());
      free_at.pop();
    }
    return t_end;
  }
};

// Key splits of the video query tiles (split-KV): n_whole leading tiles of
// every head run whole, the others are split n_splits ways (n_whole = 0:
// every tile split; n_splits = 1: none).  A split costs fp32 partial
// results, a merge and one more first-tile latency.  With 384-row tiles the
// hybrid below (64 of 69 tiles whole, the last 5 split in 3) against two
// uniform splits, same runs: 1280x704 steady state 9.19 vs 9.62-9.75 ms,
// its 7th segment 41.43-41.44 vs 42.31 ms.  Measured with 256-row tiles and
// uniform splits:
//   1280x704 steady state, 16 heads: 1,664 blocks of 256 rows = 6.5 rounds on
//     256 CUs; 1 / 2 / 3 / 4 splits 10.22 / 9.60 / 10.48 / 9.95 ms per
//     launch, and the 7th segment (158k INT8 history keys) 44.77 / 42.13 /
//     44.28 / 42.80 ms;
//   its 2-head share: 208 blocks, one round; 1 / 2 / 3 / 4 splits
//     1.270 / 1.380 / 1.384 / 1.466 ms;
//   the 480x832 segment: 736 blocks, 2.9 rounds; 1 / 2 splits 1.059 /
//     1.129 ms.
// A grid of at most one block per two CUs is split to about one block per
// CU, with no fewer than 1024 keys per split.  Larger grids take, of
//   unsplit; two uniform splits (each half keeping >= 8192 keys); and the
//   hybrid: the whole tiles fill as many full rounds as they can, and the
//   last T tiles of every head (T x H >= the tasks left over) are split in
//   s = slots / (T x H) pieces (>= 2, >= 1024 keys each), which fill one
//   last round,
// the one with the least makespan when the blocks are dealt in order to the
// earliest free slot (whole tiles first, as the kernel dispatches them),
// each costing its keys plus kBlockOverhead.  blocks_per_cu is how many
// blocks of the plan's tile height share a CU.
struct VideoSplit {
  int n_splits = 1, n_whole = 0;
  double makespan = 0.0;  // key-equivalents per slot
};
VideoSplit choose_video_splits(int H, int n_qtiles, int64_t keys_per_tile, int blocks_per_cu) {
  VideoSplit best;
  const int64_t cus = device_cus();
  const int64_t tasks = (int64_t)H * n_qtiles;
  if (tasks <= 0) return best;
  const double keys = (double)keys_per_tile;
  if (2 * tasks <= cus) {
    int64_t sp = ceil_div(cus, tasks);
    sp = std::min<int64_t>(sp, keys_per_tile / 1024);
    sp = std::min<int64_t>(sp, HN_MAX_SPLITS);
    best.n_splits = (int)std::max<int64_t>(sp, 1);
    best.makespan = keys / best.n_splits + kBlockOverhead;
    return best;
  }
  const int64_t slots = cus * std::max(blocks_per_cu, 1);
  auto uniform = [&](int sp) {
    return (double)ceil_div(tasks * sp, slots) * (keys / sp + kBlockOverhead);
  };
  best.makespan = uniform(1);
  if (keys_per_tile >= 16384 && uniform(2) < best.makespan) {
    best.n_splits = 2;
    best.makespan = uniform(2);
  }
  const int64_t rest = tasks % slots;
  if (rest > 0) {
    const int64_t T = ceil_div(rest, H);  // split tiles per head
    const int64_t pieces = T * H;
    int64_t sp = std::min<int64_t>(slots / pieces, keys_per_tile / 1024);
    sp = std::min<int64_t>(sp, HN_MAX_SPLITS);
    if (T < n_qtiles && sp >= 2) {
      SlotSim sim(slots);
      sim.deal(tasks - pieces, keys + kBlockOverhead);
      sim.deal(pieces * sp, keys / sp + kBlockOverhead);
      const double t = sim.end();
      if (t < best.makespan) {
        best.n_splits = (int)sp;
        best.n_whole = (int)(n_qtiles - T);
        best.makespan = t;
      }
    }
  }
  return best;
}

// Key splits per text query tile.  The text tiles of a joint launch run after
// the video tiles and fill what the video blocks leave of the last round, or
// rounds of their own.  The count taken is the one whose estimated makespan is
// least when the blocks are dealt in order to the earliest free slot (the
// video blocks first, as choose_video_splits laid them out, then the text
// pieces), each block costing its keys plus kBlockOverhead, a constant fitted
// to same-run measurements with 256-row tiles and uniformly split video: 4
// splits on the 480x832 segment, where the video left 32 of 256 slots free
// in its last round, and 8 on the 1280x704 one, where it filled its last
// round (joint launch 2.5% faster than with 4).  With 384-row tiles it takes
// 4 on both (the 1280x704 video now ends in split pieces): same-run joint
// launches within 0.7% of 8 either way (9.83-9.87 vs 9.80 ms; the 7th
// segment 43.59-43.66 vs 43.70 ms).  Ties go to the fewer splits (the
// 2-head share's 10 text tiles run whole beside its 208 video blocks).
// Text tiles with fewer than 4096 keys are not split, and pieces keep at
// least 1,024 keys.
int choose_text_splits(int H, const VideoSplit& v, int n_qtiles, int64_t video_keys_per_tile,
                       int n_text_tiles, int64_t keys_per_tile, int blocks_per_cu) {
  if (n_text_tiles <= 0 || keys_per_tile < 4096) return 1;
  const int64_t slots = std::max<int64_t>(device_cus() * std::max(blocks_per_cu, 1), 1);
  const double kv = (double)video_keys_per_tile;
  int best = 1;
  double best_t = 0.0;
  for (int sp = 1; sp <= HN_MAX_SPLITS; sp *= 2) {
    if (sp > 1 && keys_per_tile / sp < 1024) break;
    SlotSim sim(slots);
    if (v.n_splits == 1) {
      sim.deal((int64_t)H * n_qtiles, kv + kBlockOverhead);
    } else {
      sim.deal((int64_t)H * v.n_whole, kv + kBlockOverhead);
      sim.deal((int64_t)H * (n_qtiles - v.n_whole) * v.n_splits, kv / v.n_splits + kBlockOverhead);
    }
    sim.deal((int64_t)H * n_text_tiles * sp, (double)keys_per_tile / sp + kBlockOverhead);
    const double t_end = sim.end();
    if (sp == 1 || t_end < best_t * (1.0 - 1e-9)) {
      best_t = t_end;
      best = sp;
    }
  }
  return best;
}

// Query rows per tile of a dense plan: 256-row blocks (two waves per SIMD, Q
// in registers) or 384-row ones (three waves per SIMD, Q in LDS), both one
// block per CU.  A 384-row block stages (and dequantizes) each key tile for
// 1.5x the rows, which measured 1% faster per row on the 480x832 segment,
// 5% on the 1280x704 steady state and 7.5% on its 7th segment (INT8 history
// dominant), same runs; but it has two thirds as many blocks to fill the
// CUs with: the 2-head share took 1.613 ms with 138 384-row blocks against
// 1.277 ms with 208 256-row ones.  The height taken is the one with the
// smaller estimated makespan: choose_video_splits' makespan for it x rows,
// a 384-row block's row-keys weighted 0.95.  Blocks of 256 rows beat
// 128-row ones even where they leave CUs idle (the 2-head share:
// 1.215-1.217 ms with 208 256-row blocks against 1.464 ms with 414 128-row
// blocks, and 1.45-1.47 against 1.67-1.68 ms with its text queries), so 128
// rows are taken only for keep lists, or when asked for (opts->tile_rows:
// 128, 256 or 384 forces that height; tuning, tests).
int choose_dense_rows(int H, int lq, int64_t keys_per_tile) {
  int best_rows = 256;
  double best_t = 0.0;
  for (const int rows : {256, 384}) {
    const int nq = (int)ceil_div(lq, rows);
    const double t = choose_video_splits(H, nq, keys_per_tile, 1).makespan * rows * (rows == 384 ? 0.95 : 1.0);
    if (rows == 256 || t < best_t) {
      best_t = t;
      best_rows = rows;
    }
  }
  return best_rows;
}

// A plan's query-tile height is one the attention kernel has an instance for.
bool valid_tile_rows(int rows, bool sparse) {
  return sparse ? rows == HN_TILE : hn::attn_rows_supported(rows);
}

hn_status check_opts(const hn_plan_opts* o, bool sparse) {
  if (!o) return HN_OK;
  if (o->n_splits < 0 || o->n_splits > HN_MAX_SPLITS || o->n_splits_text < 0 ||
      o->n_splits_text > HN_MAX_SPLITS)
    return fail(HN_ERR_INVALID, "split counts %d / %d outside [0, %d]", o->n_splits, o->n_splits_text,
                HN_MAX_SPLITS);
  if (o->tile_rows != 0 && !hn::attn_rows_supported(o->tile_rows))
    return fail(HN_ERR_INVALID, "tile_rows %d is not 0, 128, 256 or 384", o->tile_rows);
  if (sparse && o->tile_rows != 0 && o->tile_rows != HN_TILE)
    return fail(HN_ERR_INVALID, "a keep list fixes %d-row query tiles", HN_TILE);
  if (o->whole_tiles < 0 || (o->whole_tiles != 0 && o->n_splits < 2))
    return fail(HN_ERR_INVALID, "whole_tiles %d needs a forced split count > 1 (n_splits %d)", o->whole_tiles,
                o->n_splits);
  return HN_OK;
}

// Plan parameters for the current state; validates the keep list and opts.
hn_status make_plan_params(const hn_kv_cache* c, const hn_seg_layout* s, const hn_block_sparse* sp,
                           const hn_plan_opts* opts, hn::PlanParams* pp) {
  int64_t tl = 0;
  hn_status st = check_cache(c);
  if (st != HN_OK) return st;
  if ((st = check_seg(c, s, &tl)) != HN_OK) return st;
  if ((st = check_opts(opts, sp != nullptr)) != HN_OK) return st;
  std::memset(pp, 0, sizeof(*pp));
  const int P = c->tokens_per_frame;
  const int lq = s->frames * P;
  const int kf = kept_frames(c);
  if (sp) pp->tile_q = HN_TILE;
  else if (opts && opts->tile_rows != 0) pp->tile_q = opts->tile_rows;
  else pp->tile_q = choose_dense_rows(c->num_heads, lq, (int64_t)c->head_tokens + tl + (int64_t)kf * P + lq);
  pp->n_qtiles = (int)ceil_div(lq, pp->tile_q);
  pp->n_text_tiles = (int)ceil_div(tl, pp->tile_q);
  pp->lq = lq;
  pp->P = P;
  pp->head_tokens = c->head_tokens;
  pp->kept_frames = kf;
  pp->ring_tokens = kf * P;
  pp->ring_rot = (int)(((c->frames_seen - kf) % c->window_frames) * P);
  pp->head_len = s->head_len;
  pp->text_len = (int)tl;
  pp->m = s->num_actions;
  int off = s->head_len;
  for (int j = 0; j < s->num_actions; ++j) {
    pp->tail_off[j] = off;
    pp->tail_len[j] = s->action_len[j];
    pp->tail_f0[j] = s->action_f0[j];
    pp->tail_f1[j] = s->action_f1[j];
    off += s->action_len[j];
  }
  pp->n_hist_tiles = (int)ceil_div(pp->ring_tokens, HN_TILE);
  pp->n_own_tiles = (int)ceil_div(lq, HN_TILE);
  {
    // keys a video query tile visits (a keep list keeps about its share of video)
    int64_t keys = (int64_t)pp->head_tokens + tl;
    int64_t video = (int64_t)pp->ring_tokens + lq;
    if (sp && sp->row_ptr && pp->n_qtiles > 0) video = video / 4;
    // dense 256- and 384-row blocks run one per CU, 128-row blocks two
    const int bpc = pp->tile_q >= 256 ? 1 : 2;
    VideoSplit v;
    if (opts && opts->n_splits > 0) {
      v.n_splits = opts->n_splits;
      v.n_whole = opts->whole_tiles;
    } else {
      v = choose_video_splits(c->num_heads, pp->n_qtiles, keys + video, bpc);
    }
    // canonical form: n_whole = 0 without a split; a split of no tile is none
    if (v.n_splits == 1 || v.n_whole >= pp->n_qtiles) {
      v.n_splits = 1;
      v.n_whole = 0;
    }
    pp->n_splits = v.n_splits;
    pp->n_whole = v.n_whole;
    // text queries see heads, the whole ring and the own video (no keep list)
    pp->n_splits_text = (opts && opts->n_splits_text > 0)
                            ? opts->n_splits_text
                            : choose_text_splits(c->num_heads, v, pp->n_qtiles, keys + video, pp->n_text_tiles,
                                                 keys + (int64_t)pp->ring_tokens + lq, bpc);
  }
  int max_spans = 4 + s->num_actions;
  if (sp) {
    if (sp->tile_q != HN_TILE || sp->tile_k != HN_TILE)
      return fail(HN_ERR_UNSUPPORTED, "block-sparse tiles %dx%d unsupported (only %d)", sp->tile_q,
                  sp->tile_k, HN_TILE);
    if (sp->n_qtiles != pp->n_qtiles)
      return fail(HN_ERR_INVALID, "block-sparse n_qtiles %d != %d", sp->n_qtiles, pp->n_qtiles);
    if (!sp->row_ptr || !sp->col) return fail(HN_ERR_NULL, "block-sparse arrays are NULL");
    pp->sparse = 1;
    pp->row_ptr = sp->row_ptr;
    pp->col = sp->col;
    // every kept tile may become its own span; one history tile may wrap the ring
    max_spans = 4 + s->num_actions + pp->n_hist_tiles + 1 + pp->n_own_tiles;
  }
  pp->max_spans = max_spans;
  return HN_OK;
}

int plan_vt(const hn::PlanParams& pp) {
  return hn::vt_count(pp.n_qtiles, pp.n_text_tiles, pp.n_whole, pp.n_splits, pp.n_splits_text);
}

// Virtual tiles with a partial-result slot: [part_vt0, n_vt) -- from the first
// split video tile on when video tiles are split, the text tiles when only
// they are, none otherwise.
void plan_partials(int n_qtiles, int n_text_tiles, int nw, int ns, int nst, int* part_vt0, int* n_pvt) {
  const int n_vt = hn::vt_count(n_qtiles, n_text_tiles, nw, ns, nst);
  if (ns > 1) {
    *part_vt0 = nw;
    *n_pvt = n_vt - nw;
  } else if (nst > 1 && n_text_tiles > 0) {
    *part_vt0 = n_qtiles;
    *n_pvt = n_vt - n_qtiles;
  } else {
    *part_vt0 = n_vt;
    *n_pvt = 0;
  }
}

size_t plan_ws_bytes(const hn_kv_cache* c, const hn::PlanParams& pp) {
  int v0 = 0, np = 0;
  plan_partials(pp.n_qtiles, pp.n_text_tiles, pp.n_whole, pp.n_splits, pp.n_splits_text, &v0, &np);
  return hn::plan_bytes(c->num_heads, plan_vt(pp), pp.max_spans, pp.tile_q, np);
}

hn_status hip_fail(hipError_t e, const char* what) {
  return fail(HN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Global frames [g0, g1) that leave the W-frame window when F frames are
// appended after fs (see hn_kv_archive_evict in hn.h).
void evicted_range(int64_t fs, int64_t F, int64_t W, int64_t* g0, int64_t* g1) {
  const int64_t kept_before = std::min(fs, W);
  const int64_t kept_after = std::min(fs + F, W);
  *g0 = fs - kept_before;
  *g1 = std::max(*g0, std::min(fs, fs + F - kept_after));
}

hn_status check_archive(const hn_kv_archive* a) {
  if (!a) return fail(HN_ERR_NULL, "archive is NULL");
  if (a->cap_frames < 0 || a->frames < 0 || a->frames > a->cap_frames || a->first_frame < 0)
    return fail(HN_ERR_INVALID, "archive counters are inconsistent");
  if (a->cap_frames > 0 && (!a->k || !a->v || !a->ks || !a->vs))
    return fail(HN_ERR_NULL, "archive buffers are NULL");
  return HN_OK;
}

// Copy global frames [g0, g1) between their ring slots and the archive (both
// head-major), in runs that do not wrap the ring: per tensor one 2-D copy of
// H rows of run*P tokens.
hn_status archive_copy(const hn_kv_cache* c, const hn_kv_archive* a, int64_t g0, int64_t g1, bool to_host,
                       hipStream_t stream) {
  const int64_t W = c->window_frames, P = c->tokens_per_frame, H = c->num_heads;
  const size_t ring_rows = (size_t)(W * P), arch_rows = (size_t)a->cap_frames * P;
  const hipMemcpyKind kind = to_host ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
  for (int64_t g = g0; g < g1;) {
    const int64_t slot = g % W;
    const int64_t n = std::min(g1 - g, W - slot);
    const size_t r_row = (size_t)(slot * P), a_row = (size_t)((g - a->first_frame) * P);
    struct { void* ring; void* arch; size_t elem; } t[4] = {
        {c->ring_k, a->k, HN_HEAD_DIM}, {c->ring_v, a->v, HN_HEAD_DIM},
        {c->ring_ks, a->ks, sizeof(float)}, {c->ring_vs, a->vs, sizeof(float)}};
    for (const auto& x : t) {
      char* ring = static_cast<char*>(x.ring) + r_row * x.elem;
      char* arch = static_cast<char*>(x.arch) + a_row * x.elem;
      const size_t width = (size_t)n * P * x.elem;
      const size_t rp = ring_rows * x.elem, ap = arch_rows * x.elem;
      const hipError_t e = to_host ? hipMemcpy2DAsync(arch, ap, ring, rp, width, (size_t)H, kind, stream)
                                   : hipMemcpy2DAsync(ring, rp, arch, ap, width, (size_t)H, kind, stream);
      if (e != hipSuccess) return hip_fail(e, to_host ? "archive copy to host" : "archive copy to device");
    }
    g += n;
  }
  return HN_OK;
}

// The host description of a plan built from pp into the device buffer dev.
void fill_plan(const hn::PlanParams& pp, const hn_kv_cache* c, const hn_seg_layout* s, void* dev,
               hn_tile_plan* plan) {
  plan->dev = dev;
  plan->tile_q = pp.tile_q;
  plan->n_qtiles = pp.n_qtiles;
  plan->n_text_tiles = pp.n_text_tiles;
  plan->max_spans = pp.max_spans;
  plan->seg_index = s->index;
  plan->head_tokens = c->head_tokens;
  plan->frames_seen = c->frames_seen;
  plan->sparse = pp.sparse;
  plan->n_splits = pp.n_splits;
  plan->n_splits_text = pp.n_splits_text;
  plan->n_whole = pp.n_whole;
  {
    // text queries: every text row sees heads, ring, own head and own
    // video; a tail row also sees its own tail
    const int64_t base = (int64_t)pp.head_tokens + pp.ring_tokens + s->head_len + pp.lq;
    int64_t pairs = (int64_t)pp.text_len * base;
    for (int j = 0; j < s->num_actions; ++j) pairs += (int64_t)s->action_len[j] * s->action_len[j];
    plan->visible_pairs_text = pairs;
  }
  if (pp.sparse) {
    plan->visible_pairs = -1;
  } else {
    int64_t pairs = 0;
    const int64_t base = (int64_t)pp.head_tokens + pp.ring_tokens + s->head_len + pp.lq;
    for (int f = 0; f < s->frames; ++f) {
      int64_t n = base;
      for (int j = 0; j < s->num_actions; ++j)
        if (s->action_f0[j] <= f && f < s->action_f1[j]) n += s->action_len[j];
      pairs += n * pp.P;
    }
    plan->visible_pairs = pairs;
  }
}

// Per-device address of `scratch`, looked up on the first call on each
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

hn_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HN_ERR_UNSUPPORTED, "device %d: the no-allocation path keeps %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the plan buffer");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return HN_OK;
}

// Every check of an attention call and its kernel parameters; enqueues
// nothing.  *partials says whether some launched tile is split (merge needed).
hn_status attn_prepare(const hn_kv_cache* c, const hn_seg_layout* s, const hn_tile_plan* plan,
                       const void* q_vid, const void* q_txt, const void* k_txt, const void* v_txt,
                       const void* k_vid, const void* v_vid, void* o_vid, void* o_txt, float* lse,
                       float* lse_txt, float sm_scale, hn::AttnParams* out, hn::MergeParams* merge,
                       bool* partials_out) {
  hn_status st = check_cache(c);
  if (st != HN_OK) return st;
  int64_t tl = 0;
  if ((st = check_seg(c, s, &tl)) != HN_OK) return st;
  if (!plan || !plan->dev) return fail(HN_ERR_NULL, "plan is NULL");
  if (s->index != c->segments)
    return fail(HN_ERR_ORDER, "segment index %d but the cache holds %d segments", s->index, c->segments);
  const int P = c->tokens_per_frame;
  const int lq = s->frames * P;
  const int tq = plan->tile_q;
  if (plan->seg_index != s->index || plan->frames_seen != c->frames_seen ||
      plan->head_tokens != c->head_tokens || !valid_tile_rows(tq, plan->sparse != 0) ||
      plan->n_qtiles != (int)ceil_div(lq, tq) || plan->n_text_tiles != (int)ceil_div(tl, tq) ||
      plan->n_splits < 1 || plan->n_splits > HN_MAX_SPLITS || plan->n_splits_text < 1 ||
      plan->n_splits_text > HN_MAX_SPLITS || plan->n_whole < 0 ||
      (plan->n_splits == 1 ? plan->n_whole != 0 : plan->n_whole >= plan->n_qtiles))
    return fail(HN_ERR_ORDER, "tile plan was built for another cache state or segment");
  if (!q_vid || !k_vid || !v_vid || !o_vid) return fail(HN_ERR_NULL, "q/k/v/o video pointer is NULL");
  if (tl > 0 && (!k_txt || !v_txt)) return fail(HN_ERR_NULL, "k_txt/v_txt is NULL");
  const bool text_q = q_txt != nullptr && tl > 0;
  if (text_q && !o_txt) return fail(HN_ERR_NULL, "o_txt is NULL while q_txt is given");
  // the kernel takes a tile's max over raw scores, valid for a positive scale
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(HN_ERR_INVALID, "sm_scale %g is not a positive finite number", (double)sm_scale);
  // the kernel addresses every source through 32-bit buffer offsets
  const int64_t tok_bytes = (int64_t)c->num_heads * HN_HEAD_DIM * 2;
  const int64_t lim = INT_MAX;
  if ((int64_t)lq * tok_bytes > lim || tl * tok_bytes > lim ||
      (int64_t)c->head_cap_tokens * HN_HEAD_DIM > lim ||
      (int64_t)c->window_frames * P * HN_HEAD_DIM > lim)
    return fail(HN_ERR_UNSUPPORTED, "a key/value source exceeds 2 GiB");
  hn::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  p.H = c->num_heads;
  p.lq = lq;
  p.lq_txt = (int32_t)tl;
  p.n_qtiles = plan->n_qtiles;
  p.n_splits = plan->n_splits;
  p.n_splits_text = plan->n_splits_text;
  p.n_whole = plan->n_whole;
  p.n_vt = hn::vt_count(plan->n_qtiles, plan->n_text_tiles, p.n_whole, plan->n_splits, plan->n_splits_text);
  p.n_tiles = hn::vt_count(plan->n_qtiles, text_q ? plan->n_text_tiles : 0, p.n_whole, plan->n_splits,
                           plan->n_splits_text);
  // partial results exist iff some launched tile is split
  const bool partials = plan->n_splits > 1 || (text_q && plan->n_splits_text > 1);
  plan_partials(plan->n_qtiles, plan->n_text_tiles, p.n_whole, plan->n_splits, plan->n_splits_text, &p.part_vt0,
                &p.n_pvt);
  p.tile_rows = plan->tile_q;
  p.max_spans = plan->max_spans;
  // whole video tiles first on every XCD, then the rest (see AttnParams)
  p.a_tasks = p.H * p.n_whole;
  p.a_per_xcd = (p.a_tasks + 7) / 8;
  p.b_tasks = p.H * (p.n_tiles - p.n_whole);
  p.b_per_xcd = (p.b_tasks + 7) / 8;
  p.head_cap = c->head_cap_tokens;
  p.ring_cap = c->window_frames * P;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.txt_len = (int32_t)tl;
  p.has_i8 = (c->head_tokens > 0 || kept_frames(c) > 0) ? 1 : 0;
  p.counts = static_cast<const int32_t*>(plan->dev);
  p.spans = reinterpret_cast<const hn::Span*>(static_cast<const char*>(plan->dev) +
                                              hn::plan_counts_bytes(p.n_vt));
  if (p.n_pvt > 0) {
    char* base = const_cast<char*>(static_cast<const char*>(plan->dev)) +
                 hn::align256(hn::plan_spans_bytes(p.n_vt, plan->max_spans));
    p.part_o = reinterpret_cast<float*>(base);
    p.part_lse = reinterpret_cast<float*>(base + hn::plan_partial_o_bytes(p.H, p.n_pvt, plan->tile_q));
  }
  p.q = static_cast<const __bf16*>(q_vid);
  p.q_txt = text_q ? static_cast<const __bf16*>(q_txt) : nullptr;
  p.k_txt = static_cast<const __bf16*>(k_txt);
  p.v_txt = static_cast<const __bf16*>(v_txt);
  p.k_vid = static_cast<const __bf16*>(k_vid);
  p.v_vid = static_cast<const __bf16*>(v_vid);
  p.heads_k = c->heads_k; p.heads_v = c->heads_v; p.heads_ks = c->heads_ks; p.heads_vs = c->heads_vs;
  p.ring_k = c->ring_k; p.ring_v = c->ring_v; p.ring_ks = c->ring_ks; p.ring_vs = c->ring_vs;
  p.o = static_cast<__bf16*>(o_vid);
  p.o_txt = text_q ? static_cast<__bf16*>(o_txt) : nullptr;
  p.lse = lse;
  p.lse_txt = text_q ? lse_txt : nullptr;
  *out = p;
  *partials_out = partials;
  if (partials) {
    hn::MergeParams& m = *merge;
    std::memset(&m, 0, sizeof(m));
    m.H = p.H;
    m.n_splits = p.n_splits;
    m.n_whole = p.n_whole;
    m.n_splits_text = p.n_splits_text;
    m.part_vt0 = p.part_vt0;
    m.n_pvt = p.n_pvt;
    m.tile_rows = plan->tile_q;
    m.n_qtiles = plan->n_qtiles;
    m.n_tiles = plan->n_qtiles + (text_q ? plan->n_text_tiles : 0);
    m.lq = lq;
    m.lq_txt = (int32_t)tl;
    m.part_o = p.part_o;
    m.part_lse = p.part_lse;
    m.o = p.o;
    m.o_txt = p.o_txt;
    m.lse = p.lse;
    m.lse_txt = p.lse_txt;
  }
  return HN_OK;
}

hn_status attn_launch(const hn::AttnParams& p, const hn::MergeParams& m, bool partials, hipStream_t stream) {
  hipError_t e = hn::launch_attn(p, stream);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (partials) {
    e = hn::launch_merge(m, stream);
    if (e != hipSuccess) return hip_fail(e, "split merge launch");
  }
  return ok();
}

}  // namespace

extern "C" {

const char* hn_status_string(hn_status s) {
  switch (s) {
    case HN_OK: return "ok";
    case HN_ERR_NULL: return "null pointer";
    case HN_ERR_INVALID: return "invalid argument";
    case HN_ERR_UNSUPPORTED: return "unsupported";
    case HN_ERR_CAPACITY: return "capacity exceeded";
    case HN_ERR_WORKSPACE: return "workspace too small";
    case HN_ERR_ORDER: return "segment order or stale plan";
    case HN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* hn_last_error(void) { return g_err; }

hn_status hn_kv_cache_sizes(int32_t H, int32_t W, int32_t P, int32_t cap, size_t* ring_bytes,
                            size_t* ring_scale_bytes, size_t* heads_bytes, size_t* heads_scale_bytes) {
  if (H < 1 || W < 1 || P < 1 || cap < 0) return fail(HN_ERR_INVALID, "invalid cache shape");
  const size_t ring = (size_t)H * W * P;
  if (ring_bytes) *ring_bytes = ring * HN_HEAD_DIM;
  if (ring_scale_bytes) *ring_scale_bytes = ring * sizeof(float);
  if (heads_bytes) *heads_bytes = (size_t)H * cap * HN_HEAD_DIM;
  if (heads_scale_bytes) *heads_scale_bytes = (size_t)H * cap * sizeof(float);
  return ok();
}

hn_status hn_kv_cache_reset(hn_kv_cache* c) {
  if (!c) return fail(HN_ERR_NULL, "cache is NULL");
  c->frames_seen = 0;
  c->head_tokens = 0;
  c->segments = 0;
  return ok();
}

hn_status hn_kv_quant_append(hn_kv_cache* c, const hn_seg_layout* s, const void* k_txt,
                             const void* v_txt, const void* k_vid, const void* v_vid,
                             hipStream_t stream) {
  hn_status st = check_cache(c);
  if (st != HN_OK) return st;
  int64_t tl = 0;
  if ((st = check_seg(c, s, &tl)) != HN_OK) return st;
  if (s->index != c->segments)
    return fail(HN_ERR_ORDER, "segment index %d but the cache holds %d segments", s->index, c->segments);
  if (!k_vid || !v_vid) return fail(HN_ERR_NULL, "k_vid/v_vid is NULL");
  if (s->head_len > 0 && (!k_txt || !v_txt)) return fail(HN_ERR_NULL, "k_txt/v_txt is NULL");
  if ((int64_t)c->head_tokens + s->head_len > c->head_cap_tokens)
    return fail(HN_ERR_CAPACITY, "head store holds %d of %d tokens; %d more do not fit", c->head_tokens,
                c->head_cap_tokens, s->head_len);
  const int P = c->tokens_per_frame;
  const int surv = std::min(s->frames, c->window_frames);
  if (((int64_t)s->head_len + (int64_t)surv * P) * c->num_heads >= (int64_t(1) << 31))
    return fail(HN_ERR_UNSUPPORTED, "segment of %d head + %d video tokens x %d heads: 2^31 rows or more",
                s->head_len, surv * P, c->num_heads);
  hn::AppendParams p;
  std::memset(&p, 0, sizeof(p));
  p.H = c->num_heads;
  p.head_len = s->head_len;
  const int frame0 = s->frames - surv;  // first surviving frame of the segment
  p.vid_first = frame0 * P;
  p.n_vid = surv * P;
  p.P = P;
  p.W = c->window_frames;
  p.slot0 = (int32_t)((c->frames_seen + frame0) % c->window_frames);
  p.head_pos = c->head_tokens;
  p.head_cap = c->head_cap_tokens;
  p.ring_cap = c->window_frames * P;
  hn::div_magic((uint32_t)p.H, p.mag_h, p.sh_h);
  hn::div_magic((uint32_t)P, p.mag_p, p.sh_p);
  p.k_txt = static_cast<const __bf16*>(k_txt);
  p.v_txt = static_cast<const __bf16*>(v_txt);
  p.k_vid = static_cast<const __bf16*>(k_vid);
  p.v_vid = static_cast<const __bf16*>(v_vid);
  p.ring_k = c->ring_k; p.ring_v = c->ring_v; p.ring_ks = c->ring_ks; p.ring_vs = c->ring_vs;
  p.heads_k = c->heads_k; p.heads_v = c->heads_v; p.heads_ks = c->heads_ks; p.heads_vs = c->heads_vs;
  hipError_t e = hn::launch_quant_append(p, stream);
  if (e != hipSuccess) return hip_fail(e, "quant_append launch");
  c->frames_seen += s->frames;
  c->head_tokens += s->head_len;
  c->segments += 1;
  return ok();
}

hn_status hn_kv_archive_evict(const hn_kv_cache* c, const hn_seg_layout* s, hn_kv_archive* a,
                              hipStream_t stream) {
  hn_status st = check_cache(c);
  if (st != HN_OK) return st;
  int64_t tl = 0;
  if ((st = check_seg(c, s, &tl)) != HN_OK) return st;
  if ((st = check_archive(a)) != HN_OK) return st;
  if (s->index != c->segments)
    return fail(HN_ERR_ORDER, "segment index %d but the cache holds %d segments", s->index, c->segments);
  int64_t g0 = 0, g1 = 0;
  evicted_range(c->frames_seen, s->frames, c->window_frames, &g0, &g1);
  if (g1 == g0) return ok();
  const int64_t first = a->frames == 0 ? g0 : a->first_frame;
  if (g0 != first + a->frames)
    return fail(HN_ERR_ORDER, "evicted frames [%lld, %lld) do not continue the archive (next %lld)",
                (long long)g0, (long long)g1, (long long)(first + a->frames));
  if (g1 - first > a->cap_frames)
    return fail(HN_ERR_CAPACITY, "archive holds %d frames; %lld needed", a->cap_frames,
                (long long)(g1 - first));
  hn_kv_archive tmp = *a;
  tmp.first_frame = first;
  if ((st = archive_copy(c, &tmp, g0, g1, true, stream)) != HN_OK) return st;
  a->first_frame = first;
  a->frames = g1 - first;
  return ok();
}

hn_status hn_kv_cache_rewind(hn_kv_cache* c, hn_kv_archive* a, int64_t frames_seen, int32_t head_tokens,
                             int32_t segments, hipStream_t stream) {
  hn_status st = check_cache(c);
  if (st != HN_OK) return st;
  if (frames_seen < 0 || frames_seen > c->frames_seen || head_tokens < 0 || head_tokens > c->head_tokens ||
      segments < 0 || segments > c->segments ||
      (segments == c->segments && (frames_seen != c->frames_seen || head_tokens != c->head_tokens)))
    return fail(HN_ERR_INVALID, "rewind target (%lld frames, %d head tokens, %d segments) is not an "
                "earlier state of (%lld, %d, %d)", (long long)frames_seen, head_tokens, segments,
                (long long)c->frames_seen, c->head_tokens, c->segments);
  const int64_t W = c->window_frames;
  const int64_t lo = frames_seen - std::min(frames_seen, W);            // window of the target state
  const int64_t in_ring = c->frames_seen - std::min(c->frames_seen, W);  // oldest frame the ring holds
  const int64_t hi = std::min(frames_seen, in_ring);                     // [lo, hi) must come back
  if (a && (st = check_archive(a)) != HN_OK) return st;
  if (hi > lo) {
    if (!a || a->frames == 0 || lo < a->first_frame || hi > a->first_frame + a->frames)
      return fail(HN_ERR_CAPACITY, "frames [%lld, %lld) are needed but not in the archive",
                  (long long)lo, (long long)hi);
    if ((st = archive_copy(c, a, lo, hi, false, stream)) != HN_OK) return st;
  }
  if (a) a->frames = std::max<int64_t>(0, std::min<int64_t>(a->frames, lo - a->first_frame));
  c->frames_seen = frames_seen;
  c->head_tokens = head_tokens;
  c->segments = segments;
  return ok();
}

size_t hn_attn_workspace_size(const hn_kv_cache* c, const hn_seg_layout* s, const hn_block_sparse* sp,
                              const hn_plan_opts* opts) {
  hn::PlanParams pp;
  if (make_plan_params(c, s, sp, opts, &pp) != HN_OK) return 0;
  return plan_ws_bytes(c, pp);
}

hn_status hn_attn_mask_build(const hn_kv_cache* c, const hn_seg_layout* s, const hn_block_sparse* sp,
                             const hn_plan_opts* opts, hn_mask_mode mode, int32_t row0, int32_t nrows,
                             void* out, size_t out_bytes, hn_tile_plan* plan, hipStream_t stream) {
  hn::PlanParams pp;
  hn_status st = make_plan_params(c, s, sp, opts, &pp);
  if (st != HN_OK) return st;
  if (!out) return fail(HN_ERR_NULL, "output buffer is NULL");
  if (mode == HN_MASK_TILE_PLAN) {
    if (!plan) return fail(HN_ERR_NULL, "plan is NULL");
    if (reinterpret_cast<uintptr_t>(out) % 16 != 0) return fail(HN_ERR_INVALID, "workspace not 16-byte aligned");
    const size_t need = plan_ws_bytes(c, pp);
    if (out_bytes < need)
      return fail(HN_ERR_WORKSPACE, "workspace of %zu bytes; %zu needed", out_bytes, need);
    hipError_t e = hn::launch_plan(pp, out, stream);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    fill_plan(pp, c, s, out, plan);
    return ok();
  }
  if (mode != HN_MASK_DENSE) return fail(HN_ERR_INVALID, "unknown mask mode %d", (int)mode);
  if (plan) return fail(HN_ERR_INVALID, "plan must be NULL in DENSE mode");
  if (row0 < 0 || nrows < 0 || (int64_t)row0 + nrows > (int64_t)pp.lq + pp.text_len)
    return fail(HN_ERR_INVALID, "rows [%d, %d) outside [0, %d)", row0, row0 + nrows, pp.lq + pp.text_len);
  if ((size_t)pp.max_spans * sizeof(hn::Span) > 64 * 1024)
    return fail(HN_ERR_UNSUPPORTED, "%d spans per tile exceed the dense expander's LDS", pp.max_spans);
  hn::DenseParams d;
  std::memset(&d, 0, sizeof(d));
  d.plan = pp;
  d.row0 = row0;
  d.nrows = nrows;
  d.lk = (int64_t)pp.head_tokens + pp.ring_tokens + pp.text_len + pp.lq;
  d.W = c->window_frames;
  d.frames_seen = c->frames_seen;
  d.out = static_cast<uint8_t*>(out);
  if (out_bytes < (size_t)nrows * (size_t)d.lk)
    return fail(HN_ERR_WORKSPACE, "dense mask needs %zu bytes; %zu given", (size_t)nrows * (size_t)d.lk,
                out_bytes);
  hipError_t e = hn::launch_dense(d, stream);
  if (e != hipSuccess) return hip_fail(e, "dense mask launch");
  return ok();
}

hn_status hn_seg_attn_fwd(const hn_kv_cache* c, const hn_seg_layout* s, const hn_tile_plan* plan,
                          const void* q_vid, const void* q_txt, const void* k_txt, const void* v_txt,
                          const void* k_vid, const void* v_vid, void* o_vid, void* o_txt, float* lse,
                          float* lse_txt, float sm_scale, hipStream_t stream) {
  hn::AttnParams p;
  hn::MergeParams m;
  bool partials = false;
  const hn_status st = attn_prepare(c, s, plan, q_vid, q_txt, k_txt, v_txt, k_vid, v_vid, o_vid, o_txt, lse,
                                    lse_txt, sm_scale, &p, &m, &partials);
  if (st != HN_OK) return st;
  return attn_launch(p, m, partials, stream);
}

hn_status hn_seg_attn_fwd_noalloc(const hn_kv_cache* c, const hn_seg_layout* s, const hn_block_sparse* sp,
                                  const void* q_vid, const void* q_txt, const void* k_txt, const void* v_txt,
                                  const void* k_vid, const void* v_vid, void* o_vid, void* o_txt, float* lse,
                                  float* lse_txt, float sm_scale, hipStream_t stream) {
  // no key splits: the plan is counts and spans only (no partial results)
  const hn_plan_opts unsplit = {1, 1, 0, 0};
  hn::PlanParams pp;
  hn_status st = make_plan_params(c, s, sp, &unsplit, &pp);
  if (st != HN_OK) return st;
  const size_t need = plan_ws_bytes(c, pp);
  if (need > (size_t)HN_NOALLOC_PLAN_BYTES)
    return fail(HN_ERR_WORKSPACE, "plan of %zu bytes exceeds the %zu-byte buffer of the no-allocation path", need,
                (size_t)HN_NOALLOC_PLAN_BYTES);
  // every argument check first (the plan's device address does not take part
  // in them), then the buffer's address, then the same parameters with it
  hn_tile_plan plan;
  std::memset(&plan, 0, sizeof(plan));
  fill_plan(pp, c, s, reinterpret_cast<void*>(alignof(hn::Span)), &plan);
  hn::AttnParams p;
  hn::MergeParams m;
  bool partials = false;
  st = attn_prepare(c, s, &plan, q_vid, q_txt, k_txt, v_txt, k_vid, v_vid, o_vid, o_txt, lse, lse_txt, sm_scale,
                    &p, &m, &partials);
  if (st != HN_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != HN_OK) return st;
  plan.dev = ws;
  st = attn_prepare(c, s, &plan, q_vid, q_txt, k_txt, v_txt, k_vid, v_vid, o_vid, o_txt, lse, lse_txt, sm_scale,
                    &p, &m, &partials);
  if (st != HN_OK) return st;
  const hipError_t e = hn::launch_plan(pp, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "plan launch");
  return attn_launch(p, m, partials, stream);
}

hn_status hn_camera_attn_fwd(const hn_seg_layout* s, int32_t num_heads, int32_t radius, const void* q_vid,
                             const void* k_cam, const void* v_cam, void* o_vid, float* lse, float sm_scale,
                             hipStream_t stream) {
  if (!s) return fail(HN_ERR_NULL, "segment layout is NULL");
  if (s->frames < 1 || s->tokens_per_frame < 1)
    return fail(HN_ERR_INVALID, "segment of %d frames x %d tokens", s->frames, s->tokens_per_frame);
  if (num_heads < 1) return fail(HN_ERR_INVALID, "num_heads %d < 1", num_heads);
  if (radius < 0) return fail(HN_ERR_INVALID, "radius %d < 0", radius);
  if (!q_vid || !k_cam || !v_cam || !o_vid) return fail(HN_ERR_NULL, "q/k/v/o pointer is NULL");
  if (!std::isfinite(sm_scale)) return fail(HN_ERR_INVALID, "sm_scale is not finite");
  const int64_t rows = (int64_t)s->frames * s->tokens_per_frame;
  // (token, head) row numbers stay below 2^28, and with 16 rows per
  // 256-thread block the launch's thread count below 2^32
  if (rows * num_heads >= ((int64_t)1 << 28) || (rows + 15) / 16 * num_heads >= ((int64_t)1 << 24))
    return fail(HN_ERR_UNSUPPORTED, "segment of %lld tokens x %d heads: 2^28 rows or more", (long long)rows,
                num_heads);
  hn::CameraParams p;
  std::memset(&p, 0, sizeof(p));
  p.H = num_heads;
  p.P = s->tokens_per_frame;
  p.F = s->frames;
  p.radius = std::min(radius, s->frames);
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.rows = rows;
  hn::div_magic((uint32_t)p.H, p.mag_h, p.sh_h);
  hn::div_magic((uint32_t)p.P, p.mag_p, p.sh_p);
  p.q = static_cast<const __bf16*>(q_vid);
  p.k = static_cast<const __bf16*>(k_cam);
  p.v = static_cast<const __bf16*>(v_cam);
  p.o = static_cast<__bf16*>(o_vid);
  p.lse = lse;
  hipError_t e = hn::launch_camera_attn(p, stream);
  if (e != hipSuccess) return hip_fail(e, "camera attention launch");
  return ok();
}

}  // extern "C"
