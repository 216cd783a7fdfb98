// Internal interfaces between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// Work-groups of a grid-stride launch over `items` work-items: enough to fill
// the chip many times over, bounded so the grid never exceeds what one launch
// dimension takes.
inline unsigned grid_blocks(int64_t items, int threads) {
  const int64_t b = (items + threads - 1) / threads;
  return (unsigned)(b < (1 << 18) ? (b > 0 ? b : 1) : (1 << 18));
}

// ---------------------------------------------------------------- indexer
enum ScoreMode { kScoreBlockMax = 0, kScoreFlat = 1, kScorePool = 2 };

struct ScoreArgs {
  const uint8_t *ik_codes;    // [n_seq][cap][64]
  const uint8_t *ik_scales;   // [n_seq][cap][4]
  int64_t cap;
  int32_t n_seq;
  const uint16_t *q_idx;      // bf16 [R][8][128]
  const float *w;             // [R][8]
  const int32_t *row_seq;     // [R]
  const int32_t *row_nvis;    // [R]
  int32_t max_nvis;
  const int32_t *pool_blocks; // [R][k_blocks]  (pool mode)
  const int32_t *n_pool;      // [R]            (pool mode)
  int32_t k_blocks;
  uint32_t *keys_out;         // [R][out_stride] order-preserving score keys
  int64_t out_stride;
  // block-max scan that first appends each row's newest entry (entry
  // n_vis - 1 of its sequence) to both planes (null: no append)
  const float *app_lat;       // [R][512]
  const float *app_ik;        // [R][128]
  uint8_t *kv_codes_w, *kv_scales_w, *ik_codes_w, *ik_scales_w;
};

// Entries per work-group of the scoring kernel (scan / flat, and pool mode).
constexpr int kScoreChunk = 512;
constexpr int kScorePoolChunk = 256;

hipError_t launch_score(ScoreMode mode, const ScoreArgs &a, int32_t n_rows, int64_t slots,
                        hipStream_t stream);

enum CountKind { kCountFixed = 0, kCountNvis = 1, kCountNvisBlocks = 2 };
enum MapKind { kMapId = 0, kMapPool = 1 };

struct SelectArgs {
  const uint32_t *keys_in;    // [R][in_stride]
  const int32_t *ids_in;      // [R][in_stride] or null (id = position)
  int64_t in_stride;
  int32_t count_kind;
  int32_t count_fixed;
  const int32_t *row_seq;
  const int32_t *row_nvis;
  int32_t n_seq;
  int32_t max_nvis;
  int32_t k;
  // intermediate level outputs: [R][n_chunks * k], zero-keyed holes
  uint32_t *keys_out;
  int32_t *ids_out;
  int64_t out_stride;
  // final level outputs
  int32_t *out;               // [R][k], ascending, -1 padded
  int32_t *n_out;             // [R]
  int32_t map_kind;
  const int32_t *pool_blocks; // [R][k_blocks] (map_kind == kMapPool)
  const int32_t *n_pool;
  int32_t k_blocks;
};

// Keys held by one selection work-group (32 per thread), and the largest pool
// (in blocks) a selection maps through.
constexpr int kSelectChunk = 16384;
// Rows of up to this many keys (and no carried ids) are selected in one level
// by a work-group holding 32 keys per thread.
constexpr int kSelectChunkWide = 32768;
constexpr int kMaxPoolBlocks = 4096;

hipError_t launch_select(const SelectArgs &a, int32_t n_rows, int32_t n_chunks, bool final_level,
                         bool wide, hipStream_t stream);
// Two levels of one launch: a1 the first level over n_chunks chunks per row
// (its outputs in a1.keys_out / ids_out), a2 the final level over them; the
// last chunk of each row to finish runs a2.  counters: [n_rows], zero between
// calls.  Requires n_chunks * a1.k <= kSelectChunk.
hipError_t launch_select_levels(const SelectArgs &a1, const SelectArgs &a2, uint32_t *counters,
                                int32_t n_rows, int32_t n_chunks, hipStream_t stream);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const uint8_t *kv_codes;    // [n_seq][cap][256]
  const uint8_t *kv_scales;   // [n_seq][cap][32]
  int64_t cap;
  int32_t n_seq;
  const uint16_t *q;          // bf16 [R][H][512]
  const int32_t *row_seq;
  const int32_t *topk;        // [R][k_pos] or null (no global keys)
  const int32_t *n_topk;
  int32_t k_pos;
  const uint8_t *swa_kv;      // [n_seq][swa_len][512] E4M3 or null
  int64_t swa_len;
  const int32_t *swa_end;
  int32_t swa_window;
  float scale_log2;           // softmax scale * log2(e)
  float *o;                   // [R][H][512]
  float *lse;                 // [R][H]
  int32_t merge_in;           // 1: start from (o, lse) as an earlier result
  // split of a row's keys over several work-groups (n_split > 1), and for
  // very few rows of 16 or 32 heads of its output channels (quarters):
  // unnormalised partial results, merged by a second kernel or (quarters) by
  // the last work-group to finish
  int32_t n_split;
  int32_t tiles_per_split;    // key tiles per work-group
  int32_t quarters;           // 1: the quarter kernel (a workspace is attached)
  float *part_o;              // [R][n_split][H][512]
  float *part_ml;             // [R][n_split][4][H][2] (quarters: one copy per channel
                              // quarter) or [R][n_split][H][2]: running max in log2
                              // units, sum
  uint32_t *counters;         // quarters: [R][n_heads / 16][kAttnRowCounters] arrival
                              // counters, zero between calls
  // set by launch_attention: all heads, head groups per row (a work-group
  // takes one group of 16 or 32 heads), rows
  int32_t n_heads;
  int32_t n_hgroups;
  int32_t n_rows;
};

// Key tiles per attention work-group step.
constexpr int kAttnTileKeys = 64;

// The attention workspace starts with kAttnCounterBytes of arrival counters
// (kAttnRowCounters per row and group of 16 heads: one per channel quarter,
// one for the quarters' merges), then the partial results.
constexpr int kAttnRowCounters = 8;
constexpr size_t kAttnCounterBytes = 16384;

// Work-group split of the attention rows: n_split partial results per row,
// with quarters also four channel quarters (bytes = 0: no split, no
// workspace).
struct AttnPlan {
  int32_t n_split;
  int32_t tiles_per_split;
  size_t bytes;
  int32_t quarters;
};
AttnPlan plan_attention(int32_t n_rows, int32_t n_heads, int32_t k_pos, int32_t window);

hipError_t launch_attention(const AttnArgs &a, int32_t n_heads, int32_t n_rows, hipStream_t stream);
// The 64-head kernel alone (one work-group per row or split of a row; the
// caller sets n_heads = 64, n_hgroups = 1 and n_rows).  Built in its own
// translation unit: its O accumulators stay in the matrix-core registers.
hipError_t launch_attention_h64(const AttnArgs &a, int64_t blocks, hipStream_t stream);

// ---------------------------------------------------------------- quantise
hipError_t launch_quantize(const float *x, int64_t n, int dim, int group, const int64_t *dst_rows,
                           uint8_t *codes, uint8_t *scales, int64_t plane_rows, hipStream_t stream);
hipError_t launch_append(const float *lat, const float *ik, int64_t n, const int64_t *dst_rows,
                         uint8_t *kv_codes, uint8_t *kv_scales, uint8_t *ik_codes, uint8_t *ik_scales,
                         int64_t plane_rows, hipStream_t stream);

// ---------------------------------------------------------- cache records
// Entry records of 356 bytes (the four planes' bytes of one entry, in plane
// order) for entries [first, first + count) of one sequence; `plane_row0` is
// the plane row of the first entry.  export: planes -> records; import:
// records -> planes.
hipError_t launch_records(bool to_records, uint8_t *kv_codes, uint8_t *kv_scales, uint8_t *ik_codes,
                          uint8_t *ik_scales, int64_t plane_row0, int64_t count, uint8_t *records,
                          hipStream_t stream);

}  // namespace csa2
