// Tile plan (per query tile: the key spans to visit) and its dense expansion.
//
// Visibility rules ("Hy-Nomas 拆解" teardown, section "架构"): inside a segment
// attention is bidirectional; a segment sees itself and earlier segments only;
// each segment's text is a description head, visible across segments, and
// action tails visible only inside their own segment and time window.  The
// history window bounds earlier video only, never the current segment
// (hyphentech explainer, warning under the configuration table).  With a keep
// list, video keys outside the query tile's kept 128-token tiles are dropped
// (teardown, "单卡 4090 怎么做到的", fourth technique).
//
// The spans of one query tile, in visiting order:
//   earlier description heads | history video in the window (ring slot order,
//   or the kept tiles, oldest first, when sparse) | own head | own tails |
//   own video (or its kept tiles).
// Each span is classified against the query tile's rows: tails whose window
// covers every row are full, tails covering none are dropped, the rest are
// partial and carry their row range [f0*P, f1*P).  Adjacent spans of the same
// source that are both full (or share a row range) are merged, so a dense plan
// has at most 4 + m spans per tile.
//
// Text-query tiles (the segment's head and tail tokens as queries) follow the
// video tiles.  Same segment-causal rule; their rows are text rows, tail j is
// visible only to its own rows [off_j, off_j + a_j) and never to head rows,
// and they attend densely (keep lists concern video query tiles): at most
// 4 + m spans as well.
//
// Split-KV: with n_splits > 1 every video query tile from n_whole on (the
// first n_whole run whole; n_splits_text > 1: every text query tile) becomes
// that many virtual tiles (split fastest), each the same span list clipped
// to one contiguous range
// of its keys in visiting order, with range boundaries on multiples of 64
// keys; the attention kernel writes partial results for each and a merge
// kernel combines them.
#include <climits>

#include "hn_internal.h"

namespace hn {
namespace {

// Emits one query tile's spans in visiting order.  The last span is held in
// registers until the next one cannot extend it, so nothing written is read
// back (a store followed by a load of the same address costs a memory round
// trip per span).  With a clip window [lo, hi) (split-KV) each span is cut to
// the part of the window it covers, counting keys in visiting order; the
// writer also counts the keys of all spans (out may be null to count only).
struct SpanWriter {
  Span* out;
  int n;
  int cap;
  int R0, R1;              // rows of the query tile
  int64_t lo, hi;          // clip window in keys of the visiting order
  int64_t total;           // keys of the spans flushed so far
  bool has;
  Span cur;

  __device__ void init(Span* o, int c, int r0, int r1, int64_t l, int64_t h) {
    out = o; n = 0; cap = c; R0 = r0; R1 = r1; lo = l; hi = h; total = 0; has = false;
  }
  __device__ void flush() {
    if (!has) return;
    has = false;
    const int64_t len = cur.k1 - cur.k0;
    const int64_t a = lo > total ? lo : total;
    const int64_t b = hi < total + len ? hi : total + len;
    if (out && a < b && n < cap) {
      Span s = cur;
      s.k0 = cur.k0 + (int)(a - total);
      s.k1 = s.k0 + (int)(b - a);
      out[n++] = s;
    }
    total += len;
  }
  __device__ void emit(int src, int k0, int k1, int r0, int r1) {
    if (k1 <= k0) return;
    const int a = max(r0, R0), b = min(r1, R1);
    if (a >= b) return;  // no row of this tile sees it
    const int full = (r0 <= R0 && R1 <= r1) ? 1 : 0;
    if (full) { r0 = 0; r1 = INT_MAX; }
    if (has && cur.src == src && cur.k1 == k0 && cur.r0 == r0 && cur.r1 == r1) {
      cur.k1 = k1;
      return;
    }
    flush();
    cur.src = src; cur.k0 = k0; cur.k1 = k1; cur.r0 = r0; cur.r1 = r1; cur.full = full;
    cur.pad0 = 0; cur.pad1 = 0;
    has = true;
  }
  __device__ int finish() {
    flush();
    return n;
  }
};

// History-video tile c (canonical, oldest frame first) -> ring slot space.
__device__ void emit_ring_tile(SpanWriter& w, const PlanParams& p, int c) {
  const int a = c * TILE;
  const int b = min(a + TILE, p.ring_tokens);
  if (b <= a) return;
  const int len = b - a;
  const int s0 = (a + p.ring_rot) % p.ring_tokens;
  if (s0 + len <= p.ring_tokens) {
    w.emit(SRC_RING, s0, s0 + len, 0, INT_MAX);
  } else {
    w.emit(SRC_RING, s0, p.ring_tokens, 0, INT_MAX);
    w.emit(SRC_RING, 0, s0 + len - p.ring_tokens, 0, INT_MAX);
  }
}

// Spans of text-query tile tt (text rows [tt*tile_q, ...)).
__device__ void emit_text_spans(const PlanParams& p, SpanWriter& w) {
  w.emit(SRC_HEADS, 0, p.head_tokens, 0, INT_MAX);
  w.emit(SRC_RING, 0, p.ring_tokens, 0, INT_MAX);
  w.emit(SRC_TXT, 0, p.head_len, 0, INT_MAX);
  for (int j = 0; j < p.m; ++j) {
    const int off = p.tail_off[j];
    w.emit(SRC_TXT, off, off + p.tail_len[j], off, off + p.tail_len[j]);
  }
  w.emit(SRC_VID, 0, p.lq, 0, INT_MAX);
}

// Spans of video query tile qt.
__device__ void emit_video_spans(const PlanParams& p, int qt, SpanWriter& w) {
  int c_begin = 0, c_end = 0;
  if (p.sparse) {
    c_begin = p.row_ptr[qt];
    c_end = p.row_ptr[qt + 1];
  }
  const int n_video_tiles = p.n_hist_tiles + p.n_own_tiles;

  // earlier segments' description heads: always visible
  w.emit(SRC_HEADS, 0, p.head_tokens, 0, INT_MAX);
  // history video still in the window
  if (!p.sparse) {
    w.emit(SRC_RING, 0, p.ring_tokens, 0, INT_MAX);
  } else {
    int last = -1;
    for (int i = c_begin; i < c_end; ++i) {
      const int c = p.col[i];
      if (c <= last || c >= n_video_tiles) continue;
      last = c;
      if (c < p.n_hist_tiles) emit_ring_tile(w, p, c);
    }
  }
  // own description head: always visible
  w.emit(SRC_TXT, 0, p.head_len, 0, INT_MAX);
  // own action tails: rows whose latent frame is inside [f0, f1)
  for (int j = 0; j < p.m; ++j) {
    const int off = p.tail_off[j];
    w.emit(SRC_TXT, off, off + p.tail_len[j], p.tail_f0[j] * p.P, p.tail_f1[j] * p.P);
  }
  // own video: bidirectional inside the segment
  if (!p.sparse) {
    w.emit(SRC_VID, 0, p.lq, 0, INT_MAX);
  } else {
    int last = -1;
    for (int i = c_begin; i < c_end; ++i) {
      const int c = p.col[i];
      if (c <= last || c >= n_video_tiles) continue;
      last = c;
      if (c >= p.n_hist_tiles) {
        const int a = (c - p.n_hist_tiles) * TILE;
        w.emit(SRC_VID, a, min(a + TILE, p.lq), 0, INT_MAX);
      }
    }
  }
}

// Spans of query tile qt (video tiles, then text tiles), clipped to the keys
// [lo, hi) of its visiting order; returns the number written.  total_out, if
// given, receives the tile's key count.
__device__ int build_tile_spans(const PlanParams& p, int qt, Span* out, int64_t lo = 0,
                                int64_t hi = INT64_MAX, int64_t* total_out = nullptr) {
  SpanWriter w;
  if (qt >= p.n_qtiles) {
    const int r0 = (qt - p.n_qtiles) * p.tile_q;
    w.init(out, p.max_spans, r0, min(r0 + p.tile_q, p.text_len), lo, hi);
    emit_text_spans(p, w);
  } else {
    const int r0 = qt * p.tile_q;
    w.init(out, p.max_spans, r0, min(r0 + p.tile_q, p.lq), lo, hi);
    emit_video_spans(p, qt, w);
  }
  const int n = w.finish();
  if (total_out) *total_out = w.total;
  return n;
}

// Key position where split i of n begins (multiples of 64 keys).
__device__ int64_t split_bound(int64_t total, int i, int n) {
  if (i >= n) return total;
  return (total * i / n) & ~(int64_t)63;
}

// Span list of virtual tile vt = (query tile, key split): a counting pass for
// the tile's keys, then the spans clipped to this split's range.
__device__ int build_spans(const PlanParams& p, int vt, Span* out) {
  int qt, split, n_split;
  vt_decode(vt, p.n_qtiles, p.n_whole, p.n_splits, p.n_splits_text, qt, split, n_split);
  if (n_split == 1) return build_tile_spans(p, qt, out);
  int64_t total = 0;
  build_tile_spans(p, qt, nullptr, 0, INT64_MAX, &total);
  return build_tile_spans(p, qt, out, split_bound(total, split, n_split),
                          split_bound(total, split + 1, n_split));
}

// One thread per virtual tile.  Text tiles start at a fresh wave, so that no
// wave walks both the video and the text span builder one after the other.
__global__ __launch_bounds__(64) void plan_kernel(PlanParams p, int32_t* counts, Span* spans) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int n_vid = vt_video(p.n_qtiles, p.n_whole, p.n_splits);
  const int pad = (n_vid + 63) & ~63;
  int vt;
  if (i < n_vid) vt = i;
  else if (i < pad) return;
  else vt = n_vid + (i - pad);
  if (vt >= vt_count(p.n_qtiles, p.n_text_tiles, p.n_whole, p.n_splits, p.n_splits_text)) return;
  counts[vt] = build_spans(p, vt, spans + (int64_t)vt * p.max_spans);
}

// Canonical column of key k of a source (see hn.h, DENSE mode).
__device__ int64_t canon_col(const DenseParams& d, int src, int k) {
  const PlanParams& p = d.plan;
  switch (src) {
    case SRC_HEADS:
      return k;
    case SRC_RING: {
      const int slot = k / p.P;
      const int pp = k - slot * p.P;
      const int oldest = p.ring_rot / p.P;
      const int i = (slot - oldest + d.W) % d.W;
      return (int64_t)p.head_tokens + (int64_t)i * p.P + pp;
    }
    case SRC_TXT:
      return (int64_t)p.head_tokens + p.ring_tokens + k;
    default:
      return (int64_t)p.head_tokens + p.ring_tokens + p.text_len + k;
  }
}

__global__ __launch_bounds__(256) void dense_kernel(DenseParams d) {
  extern __shared__ Span sh_spans[];
  __shared__ int sh_n;
  // rows [0, lq) are video queries, rows [lq, lq + text_len) text queries;
  // spans carry row ranges in the local rows of their query set
  const int qrow = d.row0 + blockIdx.x;
  const bool text = qrow >= d.plan.lq;
  const int row = text ? qrow - d.plan.lq : qrow;
  const int tile = text ? d.plan.n_qtiles + row / d.plan.tile_q : row / d.plan.tile_q;
  uint8_t* out = d.out + (int64_t)blockIdx.x * d.lk;
  for (int64_t c = threadIdx.x; c < d.lk; c += blockDim.x) out[c] = 0;
  if (threadIdx.x == 0) sh_n = build_tile_spans(d.plan, tile, sh_spans);
  __syncthreads();
  const int n = sh_n;
  for (int e = 0; e < n; ++e) {
    const Span s = sh_spans[e];
    if (row < s.r0 || row >= s.r1) continue;
    for (int k = s.k0 + threadIdx.x; k < s.k1; k += blockDim.x) out[canon_col(d, s.src, k)] = 1;
  }
}

}  // namespace

hipError_t launch_plan(const PlanParams& p, void* workspace, hipStream_t s) {
  int32_t* counts = reinterpret_cast<int32_t*>(workspace);
  const int n_vt = vt_count(p.n_qtiles, p.n_text_tiles, p.n_whole, p.n_splits, p.n_splits_text);
  Span* spans = reinterpret_cast<Span*>(reinterpret_cast<char*>(workspace) + plan_counts_bytes(n_vt));
  const int n_vid = vt_video(p.n_qtiles, p.n_whole, p.n_splits);
  const int threads = ((n_vid + 63) & ~63) + (n_vt - n_vid);
  const int blocks = (threads + 63) / 64;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(blocks), dim3(64), 0, s, p, counts, spans);
  return hipGetLastError();
}

hipError_t launch_dense(const DenseParams& d, hipStream_t s) {
  if (d.nrows == 0) return hipSuccess;
  const size_t shmem = (size_t)d.plan.max_spans * sizeof(Span);
  hipLaunchKernelGGL(dense_kernel, dim3(d.nrows), dim3(256), shmem, s, d);
  return hipGetLastError();
}

}  // namespace hn
