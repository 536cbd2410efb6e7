// Internal types shared by the host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hn.h"

namespace hn {

constexpr int D = HN_HEAD_DIM;
constexpr int TILE = HN_TILE;
#define HN_MAX_SPLITS 16  // key splits per query tile (split-KV)

// Key sources an attention span can come from.
enum Src : int32_t {
  SRC_HEADS = 0,  // INT8 head store (description heads of earlier segments)
  SRC_RING = 1,   // INT8 video ring (history frames still in the window), slot order
  SRC_TXT = 2,    // bf16 text rows of the current segment (head, tails)
  SRC_VID = 3,    // bf16 video rows of the current segment
};

// One contiguous run of keys of one source, visited by one query tile.
// Query rows outside [r0, r1) must not see it (action-tail window).
struct __attribute__((aligned(16))) Span {
  int32_t src;
  int32_t k0, k1;   // key range inside the source
  int32_t r0, r1;   // visible query rows [r0, r1) (segment-local video rows)
  int32_t full;     // 1 if every row of the query tile is inside [r0, r1)
  int32_t pad0, pad1;
};
static_assert(sizeof(Span) == 32, "Span layout");

// Everything the span builder needs; passed by value to kernels.
struct PlanParams {
  int32_t n_qtiles;      // video query tiles
  int32_t n_text_tiles;  // text query tiles, after the video tiles
  int32_t n_splits;      // key-range splits per split video query tile (split-KV); 1 = none
  int32_t n_whole;       // leading video query tiles that run unsplit (0 if n_splits == 1)
  int32_t n_splits_text; // key-range splits per text query tile
  int32_t tile_q;
  int32_t lq;            // F*P video queries
  int32_t P;
  int32_t max_spans;
  int32_t head_tokens;   // history heads in the head store
  int32_t kept_frames;   // history frames in the ring window
  int32_t ring_rot;      // slot-space offset (tokens) of the oldest kept frame
  int32_t ring_tokens;   // kept_frames * P
  int32_t head_len;      // own head h
  int32_t text_len;      // h + sum(a)
  int32_t m;             // tails
  int32_t tail_off[HN_MAX_ACTIONS];
  int32_t tail_len[HN_MAX_ACTIONS];
  int32_t tail_f0[HN_MAX_ACTIONS];
  int32_t tail_f1[HN_MAX_ACTIONS];
  // block sparsity
  int32_t sparse;
  int32_t n_hist_tiles;
  int32_t n_own_tiles;
  const int32_t* row_ptr;
  const int32_t* col;
};

// Workspace layout of a tile plan over n_vt virtual tiles (query tile x key
// split, split fastest): int32 count[n_vt] padded to 256 bytes, then
// Span spans[n_vt][max_spans]; with splits, then (256-byte aligned) the
// partial results float o[H][n_pvt][rows][D] and float lse[H][n_pvt][rows]
// of the n_pvt virtual tiles from part_vt0 on (from the first split video
// tile on when video tiles are split, else only the text tiles).
inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
inline size_t plan_counts_bytes(int n_vt) { return align256((size_t)n_vt * sizeof(int32_t)); }
inline size_t plan_spans_bytes(int n_vt, int max_spans) {
  return plan_counts_bytes(n_vt) + (size_t)n_vt * max_spans * sizeof(Span);
}
inline size_t plan_partial_o_bytes(int H, int n_vt, int rows) {
  return align256((size_t)H * n_vt * rows * D * sizeof(float));
}
inline size_t plan_partial_lse_bytes(int H, int n_vt, int rows) {
  return align256((size_t)H * n_vt * rows * sizeof(float));
}
inline size_t plan_bytes(int H, int n_vt, int max_spans, int rows, int n_pvt) {
  size_t b = align256(plan_spans_bytes(n_vt, max_spans));
  if (n_pvt > 0) b += plan_partial_o_bytes(H, n_pvt, rows) + plan_partial_lse_bytes(H, n_pvt, rows);
  return b;
}

// Virtual tiles: the first nw video query tiles whole, the other video query
// tiles split ns ways, then every text query tile split nst ways, split
// index fastest.  (nw = 0: every video tile split ns ways.)
__host__ __device__ inline int vt_video(int n_qtiles, int nw, int ns) { return nw + (n_qtiles - nw) * ns; }
__host__ __device__ inline int vt_count(int n_qtiles, int n_text_tiles, int nw, int ns, int nst) {
  return vt_video(n_qtiles, nw, ns) + n_text_tiles * nst;
}
__host__ __device__ inline int vt_first(int tile, int n_qtiles, int nw, int ns, int nst) {
  if (tile < nw) return tile;
  if (tile < n_qtiles) return nw + (tile - nw) * ns;
  return vt_video(n_qtiles, nw, ns) + (tile - n_qtiles) * nst;
}
__host__ __device__ inline void vt_decode(int vt, int n_qtiles, int nw, int ns, int nst, int& tile, int& split,
                                          int& n_split) {
  const int nv = vt_video(n_qtiles, nw, ns);
  if (vt < nw) {
    tile = vt;
    split = 0;
    n_split = 1;
  } else if (vt < nv) {
    const int r = vt - nw;
    tile = nw + r / ns;
    split = r - (r / ns) * ns;
    n_split = ns;
  } else {
    const int r = vt - nv;
    tile = n_qtiles + r / nst;
    split = r - (r / nst) * nst;
    n_split = nst;
  }
}

struct AttnParams {
  int32_t H;
  int32_t lq;            // video query rows
  int32_t n_qtiles;      // video query tiles
  int32_t n_tiles;       // virtual tiles per head this launch covers (video, then text if any)
  int32_t n_splits;      // key splits per split video query tile; > 1: write partials, merge after
  int32_t n_whole;       // leading video query tiles that run unsplit
  int32_t n_splits_text; // key splits per text query tile
  int32_t n_vt;          // virtual tiles per head in the plan
  int32_t part_vt0;      // first virtual tile with a partial-result slot
  int32_t n_pvt;         // partial-result slots per head
  int32_t lq_txt;        // text query rows
  int32_t tile_rows;     // query rows per plan tile (selects the kernel instance)
  int32_t max_spans;
  // Blocks come in two classes, each spread evenly over the 8 XCDs and the
  // first dispatched first on every XCD: the whole video tiles (virtual
  // tiles [0, n_whole) of every head), then the rest ([n_whole, n_tiles):
  // split video tiles, text tiles), so that the split pieces fill the last
  // round.  With n_whole = 0 there is only the second class.
  int32_t a_tasks, a_per_xcd;
  int32_t b_tasks, b_per_xcd;
  int32_t head_cap;      // head-store stride (tokens) per head
  int32_t ring_cap;      // ring stride (tokens) per head = W*P
  float scale_log2;      // sm_scale * log2(e)
  int32_t txt_len;       // h + sum(a) text rows of the current segment
  int32_t has_i8;        // the plan may visit INT8 sources (history heads or ring frames)
  const int32_t* counts;
  const Span* spans;
  const __bf16* q;
  const __bf16* q_txt;
  const __bf16* k_txt;
  const __bf16* v_txt;
  const __bf16* k_vid;
  const __bf16* v_vid;
  const int8_t* heads_k;
  const int8_t* heads_v;
  const float* heads_ks;
  const float* heads_vs;
  const int8_t* ring_k;
  const int8_t* ring_v;
  const float* ring_ks;
  const float* ring_vs;
  __bf16* o;
  __bf16* o_txt;
  float* lse;
  float* lse_txt;
  float* part_o;         // [H][n_vt][tile_rows][D] when any tile is split
  float* part_lse;       // [H][n_vt][tile_rows]
};

// Merge of split-KV partials into the final O (bf16) and lse.
struct MergeParams {
  int32_t H;
  int32_t n_splits;
  int32_t n_whole;
  int32_t n_splits_text;
  int32_t part_vt0;      // first virtual tile with a partial-result slot
  int32_t n_pvt;         // partial-result slots per head
  int32_t tile_rows;
  int32_t n_qtiles;      // video query tiles
  int32_t n_tiles;       // query tiles merged (video, then text if any)
  int32_t lq, lq_txt;
  const float* part_o;
  const float* part_lse;
  __bf16* o;
  __bf16* o_txt;
  float* lse;
  float* lse_txt;
};

// Multiplier m and shift k for unsigned division by d >= 1 of numerators
// below 2^31: with l = ceil(log2 d), k = 31 + l and m = ceil(2^k / d) (at
// most 2^32 - 1), n / d == (n * m) >> k for every n < 2^31, because
// 0 <= m d - 2^k < d <= 2^l = 2^(k - 31) (Granlund and Montgomery, "Division
// by invariant integers using multiplication", PLDI 1994, section 4).
inline void div_magic(uint32_t d, uint32_t& m, int32_t& k) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  k = 31 + l;
  m = (uint32_t)(((1ull << k) + d - 1) / d);
}

struct AppendParams {
  int32_t H;
  int32_t head_len;       // head rows to store
  int32_t vid_first;      // first video row read (first surviving frame * P)
  int32_t n_vid;          // surviving video rows
  int32_t P;
  int32_t W;
  int32_t slot0;          // ring slot of the first surviving frame
  int32_t head_pos;       // head-store row of the first new head token
  int32_t head_cap;
  int32_t ring_cap;       // W*P
  uint32_t mag_h, mag_p;  // division by H and by P: n / H == (n * mag_h) >> sh_h
  int32_t sh_h, sh_p;     //   for n < 2^31 (div_magic)
  const __bf16* k_txt;
  const __bf16* v_txt;
  const __bf16* k_vid;
  const __bf16* v_vid;
  int8_t* ring_k;
  int8_t* ring_v;
  float* ring_ks;
  float* ring_vs;
  int8_t* heads_k;
  int8_t* heads_v;
  float* heads_ks;
  float* heads_vs;
};

struct DenseParams {
  PlanParams plan;
  int32_t row0, nrows;
  int64_t lk;             // columns
  int32_t W;
  int32_t pad0;
  int64_t frames_seen;
  uint8_t* out;
};

// Camera cross-attention of the video tokens of one segment.
struct CameraParams {
  int32_t H;
  int32_t P;             // tokens per latent frame
  int32_t F;             // latent frames (= camera tokens)
  int32_t radius;        // visible camera tokens: |f' - f| <= radius
  float scale_log2;      // sm_scale * log2(e)
  int32_t sh_h, sh_p;    // division by H and by P (div_magic): n / H == (n * mag_h) >> sh_h
  uint32_t mag_h, mag_p;
  int64_t rows;          // F * P video tokens (< 2^28 / H, so every index below 2^31)
  const __bf16* q;       // [rows][H][D]
  const __bf16* k;       // [F][H][D]
  const __bf16* v;       // [F][H][D]
  __bf16* o;             // [rows][H][D]
  float* lse;            // [H][rows] or null
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Query rows per tile of a dense (keep-list free) plan; keep-list plans use HN_TILE.
// query-tile heights the attention kernel has an instance for
bool attn_rows_supported(int rows);

// Launchers (defined next to their kernels); return the HIP error of the launch.
hipError_t launch_quant_append(const AppendParams& p, hipStream_t s);
hipError_t launch_plan(const PlanParams& p, void* workspace, hipStream_t s);
hipError_t launch_dense(const DenseParams& p, hipStream_t s);
hipError_t launch_attn(const AttnParams& p, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_camera_attn(const CameraParams& p, hipStream_t s);

}  // namespace hn
