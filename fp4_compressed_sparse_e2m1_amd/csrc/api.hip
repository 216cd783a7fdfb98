// C ABI of libcsa2: argument validation, workspace planning and launches.
// The operations and their sources are documented in include/csa2.h.
#include <math.h>

#include <mutex>

#include "../../include/csa2.h"
#include "internal.h"

using namespace csa2;

namespace {

constexpr int kMaxBlocks = 4096;
constexpr int kMaxPos = 4096;
constexpr int kMaxAttnPos = 65536;
constexpr int kMaxGridY = 65535;
constexpr size_t kAlign = 256;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Levels of the chunked Top-k selection for rows of up to n_max keys.
int plan_levels(int64_t n_max, int k, int64_t *chunks) {
  int levels = 0;
  int64_t n = n_max;
  if (n <= kSelectChunkWide) {     // one level (the wide selection above kSelectChunk keys)
    chunks[0] = 1;
    return 1;
  }
  while (n > kSelectChunk && levels < 7) {
    const int64_t ch = (n + kSelectChunk - 1) / kSelectChunk;
    chunks[levels++] = ch;
    n = ch * k;
  }
  chunks[levels++] = 1;
  return levels;
}

// Bytes of one ping-pong buffer (keys + ids) of a selection.
size_t select_scratch(int32_t rows, int64_t n_max, int k) {
  int64_t chunks[8];
  const int levels = plan_levels(n_max, k, chunks);
  if (levels == 1) return 0;
  return (size_t)rows * (size_t)chunks[0] * (size_t)k * 8;
}

// Flat mode (every visible entry a candidate) scores and selects its rows in
// passes of at most this many bytes of entry keys and selection scratch, so
// its workspace is bounded by this size (or one row's need) however many
// rows a call has.
constexpr size_t kFlatPassBytes = (size_t)256 << 20;

// Rows per flat-mode pass: as many as fit kFlatPassBytes (whole groups of 8,
// the many-row scoring kernel's group), at least one.
int32_t flat_pass_rows(int32_t n_rows, int32_t max_nvis, int32_t k_pos) {
  const size_t per_row = round_up((size_t)(max_nvis > 0 ? max_nvis : 1) * 4) + 2 * select_scratch(1, max_nvis, k_pos);
  int64_t rb = (int64_t)(kFlatPassBytes / per_row);
  if (rb >= 8) rb -= rb % 8;
  rb = rb < 1 ? 1 : rb;
  return (int32_t)(rb < n_rows ? rb : n_rows);
}

struct Layout {
  size_t counters = 0;  // arrival counters of the fused block selection (zero between calls)
  size_t keys_a = 0;    // block keys or flat entry keys
  size_t keys_b = 0;    // pool candidate keys
  size_t ping = 0, pong = 0;
  size_t half = 0;      // bytes of one ping-pong buffer
  size_t total = 0;
};

// Workspace layout of an indexer call.
Layout plan_workspace(int32_t op, int32_t rows, int32_t max_nvis, int32_t k_blocks, int32_t k_pos) {
  Layout L;
  size_t off = 0;
  size_t half = 0;
  if (k_blocks > 0) {
    if (op == CSA2_OP_INDEX_FULL || op == CSA2_OP_INDEX_POOL) {
      L.counters = off;
      off += round_up((size_t)rows * 4);
      const int64_t nb = ((int64_t)max_nvis + 7) / 8;
      if (op == CSA2_OP_INDEX_FULL) {
        L.keys_a = off;
        off += round_up((size_t)rows * (size_t)(nb > 0 ? nb : 1) * 4);
      }
      half = select_scratch(rows, nb, k_blocks);
    }
    L.keys_b = off;
    off += round_up((size_t)rows * (size_t)k_blocks * 8 * 4);
    const size_t h2 = select_scratch(rows, (int64_t)k_blocks * 8, k_pos);
    half = half > h2 ? half : h2;
  } else {
    const int32_t rb = flat_pass_rows(rows, max_nvis, k_pos);
    L.keys_a = off;
    off += round_up((size_t)rb * (size_t)(max_nvis > 0 ? max_nvis : 1) * 4);
    half = select_scratch(rb, max_nvis, k_pos);
  }
  half = round_up(half);
  L.half = half;
  L.ping = off;
  off += half;
  L.pong = off;
  off += half;
  L.total = off;
  return L;
}

struct SelectOut {
  int32_t *out;
  int32_t *n_out;
  int32_t map_kind;
  const int32_t *pool_blocks;
  const int32_t *n_pool;
  int32_t k_blocks;
};

// counters (optional, [rows], zero between calls): two levels whose second
// is one chunk then run as one launch.
hipError_t run_select(const uint32_t *keys, int64_t stride, int count_kind, int count_fixed,
                      int64_t n_max, int k, const int32_t *row_seq, const int32_t *row_nvis,
                      int32_t n_seq, int32_t max_nvis, const SelectOut &fin, uint8_t *ping,
                      uint8_t *pong, size_t half, int32_t rows, hipStream_t stream,
                      uint32_t *counters = nullptr) {
  int64_t chunks[8];
  const int levels = plan_levels(n_max, k, chunks);
  const bool fused = counters && levels == 2 && chunks[0] * k <= kSelectChunk;
  SelectArgs first = {};
  const uint32_t *kin = keys;
  const int32_t *iin = nullptr;
  int64_t in_stride = stride;
  int ckind = count_kind;
  int cfixed = count_fixed;
  for (int l = 0; l < levels; ++l) {
    SelectArgs a = {};
    a.keys_in = kin;
    a.ids_in = iin;
    a.in_stride = in_stride;
    a.count_kind = ckind;
    a.count_fixed = cfixed;
    a.row_seq = row_seq;
    a.row_nvis = row_nvis;
    a.n_seq = n_seq;
    a.max_nvis = max_nvis;
    a.k = k;
    const bool final_level = (l == levels - 1);
    if (!final_level) {
      uint8_t *buf = (l % 2 == 0) ? ping : pong;
      const int64_t out_stride = chunks[l] * k;
      a.keys_out = reinterpret_cast<uint32_t *>(buf);
      a.ids_out = reinterpret_cast<int32_t *>(buf + half / 2);
      a.out_stride = out_stride;
      if (fused) {
        first = a;        // launched with the final level below
      } else {
        hipError_t e = launch_select(a, rows, (int32_t)chunks[l], false, false, stream);
        if (e != hipSuccess) return e;
      }
      kin = a.keys_out;
      iin = a.ids_out;
      in_stride = out_stride;
      ckind = kCountFixed;
      cfixed = (int)out_stride;
    } else {
      a.out = fin.out;
      a.n_out = fin.n_out;
      a.map_kind = fin.map_kind;
      a.pool_blocks = fin.pool_blocks;
      a.n_pool = fin.n_pool;
      a.k_blocks = fin.k_blocks;
      if (fused) {
        hipError_t e = launch_select_levels(first, a, counters, rows, (int32_t)chunks[0], stream);
        if (e != hipSuccess) return e;
        continue;
      }
      // a single level over more keys than one chunk: the wide selection
      const bool wide = levels == 1 && n_max > kSelectChunk;
      hipError_t e = launch_select(a, rows, 1, true, wide, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

bool cache_ok(const csa2_cache *c, bool need_kv, bool need_ik) {
  if (!c || c->cap < 1 || c->n_seq < 1) return false;
  if (need_kv && (!c->kv_codes || !c->kv_scales || !aligned(c->kv_codes, 16) ||
                  !aligned(c->kv_scales, 2)))
    return false;
  if (need_ik && (!c->ik_codes || !c->ik_scales || !aligned(c->ik_codes, 16))) return false;
  return true;
}

// Shared body of index_full / index_reindex.
// Host checks shared by every indexer entry point.
csa2_status check_index_args(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                             const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                             int32_t max_nvis) {
  if (!cache_ok(cache, false, true)) return CSA2_E_INVALID_ARG;
  if (!q_idx || !w || !row_seq || !row_nvis) return CSA2_E_INVALID_ARG;
  if (n_rows < 1 || max_nvis < 0 || (int64_t)max_nvis > cache->cap) return CSA2_E_INVALID_ARG;
  if (!aligned(q_idx, 16) || !aligned(w, 4)) return CSA2_E_INVALID_ARG;
  if (n_rows > kMaxGridY || max_nvis > 0x7FFFFFF0) return CSA2_E_UNSUPPORTED;
  return CSA2_OK;
}

ScoreArgs score_args(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                     const int32_t *row_seq, const int32_t *row_nvis, int32_t max_nvis) {
  ScoreArgs sa = {};
  sa.ik_codes = cache->ik_codes;
  sa.ik_scales = cache->ik_scales;
  sa.cap = cache->cap;
  sa.n_seq = cache->n_seq;
  sa.q_idx = q_idx;
  sa.w = w;
  sa.row_seq = row_seq;
  sa.row_nvis = row_nvis;
  sa.max_nvis = max_nvis;
  return sa;
}

// Every argument check of an indexer call except the workspace's.
csa2_status check_indexer(int32_t op, const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                          const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                          int32_t max_nvis, const uint32_t *ext_block_keys, const int32_t *pool_in,
                          const int32_t *n_pool_in, int32_t k_blocks, int32_t k_pos,
                          const int32_t *pool_out, const int32_t *n_pool_out, const int32_t *topk,
                          const int32_t *n_topk) {
  const csa2_status cs = check_index_args(cache, q_idx, w, row_seq, row_nvis, n_rows, max_nvis);
  if (cs != CSA2_OK) return cs;
  if (!topk || !n_topk || k_pos < 1 || k_blocks < 0) return CSA2_E_INVALID_ARG;
  if (k_pos > kMaxPos || k_blocks > kMaxBlocks) return CSA2_E_UNSUPPORTED;
  const bool pool_mode = k_blocks > 0;
  if ((op == CSA2_OP_INDEX_FULL || op == CSA2_OP_INDEX_POOL) && pool_mode &&
      (!pool_out || !n_pool_out))
    return CSA2_E_INVALID_ARG;
  if (op == CSA2_OP_INDEX_POOL && (!pool_mode || !ext_block_keys || !aligned(ext_block_keys, 4)))
    return CSA2_E_INVALID_ARG;
  if (op == CSA2_OP_INDEX_REINDEX && pool_mode && (!pool_in || !n_pool_in)) return CSA2_E_INVALID_ARG;
  return CSA2_OK;
}

csa2_status run_indexer(int32_t op, const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                        const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                        int32_t max_nvis, const uint32_t *ext_block_keys, const int32_t *pool_in,
                        const int32_t *n_pool_in, int32_t k_blocks, int32_t k_pos,
                        int32_t *pool_out, int32_t *n_pool_out, int32_t *topk, int32_t *n_topk,
                        void *workspace, size_t workspace_bytes, void *stream_ptr) {
  const csa2_status cs = check_indexer(op, cache, q_idx, w, row_seq, row_nvis, n_rows, max_nvis,
                                       ext_block_keys, pool_in, n_pool_in, k_blocks, k_pos, pool_out,
                                       n_pool_out, topk, n_topk);
  if (cs != CSA2_OK) return cs;
  const bool pool_mode = k_blocks > 0;
  const Layout L = plan_workspace(op, n_rows, max_nvis, k_blocks, k_pos);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, kAlign)) return CSA2_E_WORKSPACE;

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  ScoreArgs sa = score_args(cache, q_idx, w, row_seq, row_nvis, max_nvis);
  hipError_t e = hipSuccess;

  if (!pool_mode) {
    // flat: every visible entry is a candidate; the rows go in passes that
    // fit the bounded workspace (one pass unless the rows are many)
    const int32_t rb = flat_pass_rows(n_rows, max_nvis, k_pos);
    sa.keys_out = reinterpret_cast<uint32_t *>(ws + L.keys_a);
    sa.out_stride = max_nvis > 0 ? max_nvis : 1;
    for (int32_t r0 = 0; r0 < n_rows; r0 += rb) {
      const int32_t nr = n_rows - r0 < rb ? n_rows - r0 : rb;
      ScoreArgs sp = sa;
      sp.q_idx = q_idx + (int64_t)r0 * 8 * 128;
      sp.w = w + (int64_t)r0 * 8;
      sp.row_seq = row_seq + r0;
      sp.row_nvis = row_nvis + r0;
      e = launch_score(kScoreFlat, sp, nr, max_nvis, stream);
      if (e != hipSuccess) return CSA2_E_HIP;
      SelectOut fin = {topk + (int64_t)r0 * k_pos, n_topk + r0, kMapId, nullptr, nullptr, 0};
      e = run_select(sp.keys_out, sp.out_stride, kCountNvis, 0, max_nvis, k_pos, row_seq + r0,
                     row_nvis + r0, cache->n_seq, max_nvis, fin, ws + L.ping, ws + L.pong, L.half, nr,
                     stream);
      if (e != hipSuccess) return CSA2_E_HIP;
    }
    return CSA2_OK;
  }

  const int32_t *pool = pool_in;
  const int32_t *npool = n_pool_in;
  if (op == CSA2_OP_INDEX_FULL || op == CSA2_OP_INDEX_POOL) {
    // scan: block max of every visible entry's score, then the block Top-k
    const int64_t nb = ((int64_t)max_nvis + 7) / 8;
    const int64_t nb_stride = nb > 0 ? nb : 1;
    const uint32_t *bkeys = ext_block_keys;
    if (op == CSA2_OP_INDEX_FULL) {
      sa.keys_out = reinterpret_cast<uint32_t *>(ws + L.keys_a);
      sa.out_stride = nb_stride;
      e = launch_score(kScoreBlockMax, sa, n_rows, max_nvis, stream);
      if (e != hipSuccess) return CSA2_E_HIP;
      bkeys = sa.keys_out;
    }
    SelectOut fin = {pool_out, n_pool_out, kMapId, nullptr, nullptr, 0};
    e = run_select(bkeys, nb_stride, kCountNvisBlocks, 0, nb, k_blocks, row_seq, row_nvis,
                   cache->n_seq, max_nvis, fin, ws + L.ping, ws + L.pong, L.half, n_rows, stream,
                   reinterpret_cast<uint32_t *>(ws + L.counters));
    if (e != hipSuccess) return CSA2_E_HIP;
    pool = pool_out;
    npool = n_pool_out;
  }
  // re-score the pool's entries and keep the best k_pos positions
  sa.pool_blocks = pool;
  sa.n_pool = npool;
  sa.k_blocks = k_blocks;
  sa.keys_out = reinterpret_cast<uint32_t *>(ws + L.keys_b);
  sa.out_stride = (int64_t)k_blocks * 8;
  e = launch_score(kScorePool, sa, n_rows, (int64_t)k_blocks * 8, stream);
  if (e != hipSuccess) return CSA2_E_HIP;
  SelectOut fin = {topk, n_topk, kMapPool, pool, npool, k_blocks};
  e = run_select(sa.keys_out, sa.out_stride, kCountFixed, k_blocks * 8, (int64_t)k_blocks * 8, k_pos,
                 row_seq, row_nvis, cache->n_seq, max_nvis, fin, ws + L.ping, ws + L.pong, L.half,
                 n_rows, stream);
  return e == hipSuccess ? CSA2_OK : CSA2_E_HIP;
}

bool swa_ok(const csa2_swa *s) {
  return s && s->kv && s->row_end && s->len >= 0 && s->window >= 0 && s->window <= 1024 &&
         aligned(s->kv, 16);
}

// Fills the split fields of `a`; CSA2_E_WORKSPACE if a workspace is given but
// smaller than the plan needs.
csa2_status attach_workspace(AttnArgs &a, int32_t n_rows, int32_t n_heads, int32_t k_pos,
                             int32_t window, void *workspace, size_t workspace_bytes) {
  const AttnPlan p = plan_attention(n_rows, n_heads, k_pos, window);
  a.n_split = 1;
  a.tiles_per_split = p.tiles_per_split;
  a.quarters = 0;
  a.counters = nullptr;
  if (!workspace || p.bytes == 0) return CSA2_OK;
  if (workspace_bytes < p.bytes || !aligned(workspace, kAlign)) return CSA2_E_WORKSPACE;
  a.n_split = p.n_split;
  a.quarters = p.quarters;
  a.counters = static_cast<uint32_t *>(workspace);
  a.part_o = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + kAttnCounterBytes);
  a.part_ml = a.part_o + (size_t)n_rows * p.n_split * n_heads * 512;
  return CSA2_OK;
}

// Shared checks and launch of csa2_cache_export / csa2_cache_import.
csa2_status run_records(bool to_records, const csa2_cache *cache, int32_t seq, int64_t first,
                        int64_t count, const uint8_t *records, void *stream) {
  if (!cache_ok(cache, true, true)) return CSA2_E_INVALID_ARG;
  if (!aligned(cache->kv_scales, 4) || !aligned(cache->ik_scales, 4)) return CSA2_E_INVALID_ARG;
  if (seq < 0 || seq >= cache->n_seq || first < 0 || count < 0 || first > cache->cap ||
      count > cache->cap - first)
    return CSA2_E_INVALID_ARG;
  if (count == 0) return CSA2_OK;
  if (!records || !aligned(records, 4)) return CSA2_E_INVALID_ARG;
  if (count > ((int64_t)1 << 32)) return CSA2_E_UNSUPPORTED;
  hipError_t e = launch_records(to_records, cache->kv_codes, cache->kv_scales, cache->ik_codes,
                                cache->ik_scales, (int64_t)seq * cache->cap + first, count,
                                const_cast<uint8_t *>(records), reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : CSA2_E_HIP;
}

// Scratch of csa2_index_full_noalloc: one array per device, in the library's
// code object, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: kernels and copies only ever
// receive the device address that hipGetSymbolAddress returns for the
// current device (scratch_address below).
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];

// Device address of the current device's scratch array, looked up once per
// device (with that device current) on its first use.
hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_status[dev] = (r == hipSuccess && p == nullptr) ? hipErrorInvalidSymbol : r;
    g_scratch_ptr[dev] = g_scratch_status[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_status[dev];
}

}  // namespace

extern "C" {

csa2_status csa2_index_full_noalloc(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                                    const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                                    int32_t max_nvis, int32_t k_blocks, int32_t k_pos,
                                    int32_t *pool_blocks, int32_t *n_pool, int32_t *topk,
                                    int32_t *n_topk, void *stream) {
  const csa2_status cs = check_indexer(CSA2_OP_INDEX_FULL, cache, q_idx, w, row_seq, row_nvis, n_rows,
                                       max_nvis, nullptr, nullptr, nullptr, k_blocks, k_pos, pool_blocks,
                                       n_pool, topk, n_topk);
  if (cs != CSA2_OK) return cs;
  const size_t need = plan_workspace(CSA2_OP_INDEX_FULL, n_rows, max_nvis, k_blocks, k_pos).total;
  if (need > (size_t)CSA2_NOALLOC_SCRATCH_BYTES) return CSA2_E_UNSUPPORTED;
  void *ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return CSA2_E_HIP;
  return run_indexer(CSA2_OP_INDEX_FULL, cache, q_idx, w, row_seq, row_nvis, n_rows, max_nvis,
                     nullptr, nullptr, nullptr, k_blocks, k_pos, pool_blocks, n_pool, topk, n_topk,
                     ws, (size_t)CSA2_NOALLOC_SCRATCH_BYTES, stream);
}

csa2_status csa2_quantize_fp4(const float *x, int64_t n, int32_t dim, int32_t group,
                              const int64_t *dst_rows, uint8_t *codes, uint8_t *scales,
                              int64_t plane_rows, void *stream) {
  if (n < 0 || plane_rows < 0 || (!dst_rows && plane_rows < n)) return CSA2_E_INVALID_ARG;
  if (group != 16 && group != 32) return CSA2_E_UNSUPPORTED;
  if (dim < 32 || dim > 4096 || dim % group != 0) return CSA2_E_UNSUPPORTED;
  if (n == 0) return CSA2_OK;
  if (!x || !codes || !scales) return CSA2_E_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, group == 16 ? 8 : 16)) return CSA2_E_INVALID_ARG;
  if (n > ((int64_t)1 << 40) / dim) return CSA2_E_UNSUPPORTED;
  hipError_t e = launch_quantize(x, n, dim, group, dst_rows, codes, scales, plane_rows,
                                 reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : CSA2_E_HIP;
}

csa2_status csa2_cache_append(const csa2_cache *cache, const float *latent, const float *ikey,
                              int64_t n, const int64_t *dst_rows, void *stream) {
  if (n < 0) return CSA2_E_INVALID_ARG;
  if (!cache_ok(cache, true, true)) return CSA2_E_INVALID_ARG;
  if (n == 0) return CSA2_OK;
  if (!latent || !ikey || !dst_rows) return CSA2_E_INVALID_ARG;
  if (!aligned(latent, 16) || !aligned(ikey, 16) || !aligned(dst_rows, 8)) return CSA2_E_INVALID_ARG;
  if (n > ((int64_t)1 << 40) / 512) return CSA2_E_UNSUPPORTED;
  const int64_t plane_rows = (int64_t)cache->n_seq * cache->cap;
  hipError_t e = launch_append(latent, ikey, n, dst_rows, cache->kv_codes, cache->kv_scales,
                               cache->ik_codes, cache->ik_scales, plane_rows,
                               reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : CSA2_E_HIP;
}

csa2_status csa2_cache_export(const csa2_cache *cache, int32_t seq, int64_t first, int64_t count,
                              uint8_t *records, void *stream) {
  return run_records(true, cache, seq, first, count, records, stream);
}

csa2_status csa2_cache_import(const csa2_cache *cache, int32_t seq, int64_t first, int64_t count,
                              const uint8_t *records, void *stream) {
  return run_records(false, cache, seq, first, count, records, stream);
}

size_t csa2_workspace_size(int32_t op, int32_t n_rows, int32_t max_nvis, int32_t k_blocks,
                           int32_t k_pos) {
  if ((op != CSA2_OP_INDEX_FULL && op != CSA2_OP_INDEX_REINDEX && op != CSA2_OP_INDEX_POOL) ||
      n_rows < 1 || max_nvis < 0 || k_blocks < 0 || k_blocks > kMaxBlocks || k_pos < 1 ||
      k_pos > kMaxPos || (op == CSA2_OP_INDEX_POOL && k_blocks < 1))
    return 0;
  return plan_workspace(op, n_rows, max_nvis, k_blocks, k_pos).total;
}

csa2_status csa2_index_full(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                            const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                            int32_t max_nvis, int32_t k_blocks, int32_t k_pos,
                            int32_t *pool_blocks, int32_t *n_pool, int32_t *topk,
                            int32_t *n_topk, void *workspace, size_t workspace_bytes,
                            void *stream) {
  return run_indexer(CSA2_OP_INDEX_FULL, cache, q_idx, w, row_seq, row_nvis, n_rows, max_nvis,
                     nullptr, nullptr, nullptr, k_blocks, k_pos, pool_blocks, n_pool, topk, n_topk,
                     workspace, workspace_bytes, stream);
}

csa2_status csa2_index_scan(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                            const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                            int32_t max_nvis, uint32_t *block_keys, void *stream) {
  const csa2_status cs = check_index_args(cache, q_idx, w, row_seq, row_nvis, n_rows, max_nvis);
  if (cs != CSA2_OK) return cs;
  if (!block_keys || !aligned(block_keys, 4)) return CSA2_E_INVALID_ARG;
  ScoreArgs sa = score_args(cache, q_idx, w, row_seq, row_nvis, max_nvis);
  const int64_t nb = ((int64_t)max_nvis + 7) / 8;
  sa.keys_out = block_keys;
  sa.out_stride = nb > 0 ? nb : 1;
  hipError_t e = launch_score(kScoreBlockMax, sa, n_rows, max_nvis, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : CSA2_E_HIP;
}

csa2_status csa2_index_scan_append(const csa2_cache *cache, const float *latent, const float *ikey,
                                   const uint16_t *q_idx, const float *w, const int32_t *row_seq,
                                   const int32_t *row_nvis, int32_t n_rows, int32_t max_nvis,
                                   uint32_t *block_keys, void *stream) {
  if (!cache_ok(cache, true, true)) return CSA2_E_INVALID_ARG;
  const csa2_status cs = check_index_args(cache, q_idx, w, row_seq, row_nvis, n_rows, max_nvis);
  if (cs != CSA2_OK) return cs;
  if (!block_keys || !aligned(block_keys, 4)) return CSA2_E_INVALID_ARG;
  if (!latent || !ikey || !aligned(latent, 16) || !aligned(ikey, 16)) return CSA2_E_INVALID_ARG;
  if (n_rows > cache->n_seq) return CSA2_E_INVALID_ARG;   // rows name distinct sequences
  ScoreArgs sa = score_args(cache, q_idx, w, row_seq, row_nvis, max_nvis);
  const int64_t nb = ((int64_t)max_nvis + 7) / 8;
  sa.keys_out = block_keys;
  sa.out_stride = nb > 0 ? nb : 1;
  sa.app_lat = latent;
  sa.app_ik = ikey;
  sa.kv_codes_w = cache->kv_codes;
  sa.kv_scales_w = cache->kv_scales;
  sa.ik_codes_w = cache->ik_codes;
  sa.ik_scales_w = cache->ik_scales;
  hipError_t e = launch_score(kScoreBlockMax, sa, n_rows, max_nvis, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : CSA2_E_HIP;
}

csa2_status csa2_index_pool(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                            const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                            int32_t max_nvis, const uint32_t *block_keys, int32_t k_blocks,
                            int32_t k_pos, int32_t *pool_blocks, int32_t *n_pool, int32_t *topk,
                            int32_t *n_topk, void *workspace, size_t workspace_bytes,
                            void *stream) {
  if (k_blocks < 1) return CSA2_E_INVALID_ARG;
  return run_indexer(CSA2_OP_INDEX_POOL, cache, q_idx, w, row_seq, row_nvis, n_rows, max_nvis,
                     block_keys, nullptr, nullptr, k_blocks, k_pos, pool_blocks, n_pool, topk,
                     n_topk, workspace, workspace_bytes, stream);
}

csa2_status csa2_index_reindex(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                               const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                               int32_t max_nvis, const int32_t *pool_blocks,
                               const int32_t *n_pool, int32_t k_blocks, int32_t k_pos,
                               int32_t *topk, int32_t *n_topk, void *workspace,
                               size_t workspace_bytes, void *stream) {
  const int32_t kb = pool_blocks ? k_blocks : 0;
  if (pool_blocks && k_blocks < 1) return CSA2_E_INVALID_ARG;
  return run_indexer(CSA2_OP_INDEX_REINDEX, cache, q_idx, w, row_seq, row_nvis, n_rows, max_nvis,
                     nullptr, pool_blocks, n_pool, kb, k_pos, nullptr, nullptr, topk, n_topk,
                     workspace, workspace_bytes, stream);
}

csa2_status csa2_sparse_attn(const csa2_cache *cache, const uint16_t *q, int32_t n_heads,
                             const int32_t *row_seq, int32_t n_rows, const int32_t *topk,
                             const int32_t *n_topk, int32_t k_pos, float scale,
                             const csa2_swa *swa, float *o, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream) {
  if (!cache_ok(cache, true, false)) return CSA2_E_INVALID_ARG;
  if (!q || !row_seq || !topk || !n_topk || !o || !lse) return CSA2_E_INVALID_ARG;
  if (n_rows < 0 || k_pos < 1 || !isfinite(scale)) return CSA2_E_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4)) return CSA2_E_INVALID_ARG;
  if (n_heads != 16 && n_heads != 32 && n_heads != 64) return CSA2_E_UNSUPPORTED;
  if (k_pos > kMaxAttnPos) return CSA2_E_UNSUPPORTED;
  if (swa && !swa_ok(swa)) return CSA2_E_INVALID_ARG;
  if (n_rows == 0) return CSA2_OK;
  AttnArgs a = {};
  a.kv_codes = cache->kv_codes;
  a.kv_scales = cache->kv_scales;
  a.cap = cache->cap;
  a.n_seq = cache->n_seq;
  a.q = q;
  a.row_seq = row_seq;
  a.topk = topk;
  a.n_topk = n_topk;
  a.k_pos = k_pos;
  if (swa) {
    a.swa_kv = swa->kv;
    a.swa_len = swa->len;
    a.swa_end = swa->row_end;
    a.swa_window = swa->window;
  }
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o = o;
  a.lse = lse;
  a.merge_in = 0;
  const csa2_status ws = attach_workspace(a, n_rows, n_heads, k_pos, swa ? swa->window : 0,
                                          workspace, workspace_bytes);
  if (ws != CSA2_OK) return ws;
  hipError_t e = launch_attention(a, n_heads, n_rows, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : CSA2_E_HIP;
}

csa2_status csa2_swa_merge(const uint16_t *q, int32_t n_heads, const int32_t *row_seq,
                           int32_t n_rows, const csa2_swa *swa, int32_t n_seq, float scale,
                           float *o, float *lse, void *workspace, size_t workspace_bytes,
                           void *stream) {
  if (!q || !row_seq || !o || !lse || !swa_ok(swa)) return CSA2_E_INVALID_ARG;
  if (n_rows < 0 || n_seq < 1 || !isfinite(scale)) return CSA2_E_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(lse, 4)) return CSA2_E_INVALID_ARG;
  if (n_heads != 16 && n_heads != 32 && n_heads != 64) return CSA2_E_UNSUPPORTED;
  if (n_rows == 0) return CSA2_OK;
  AttnArgs a = {};
  a.cap = 1;
  a.n_seq = n_seq;
  a.q = q;
  a.row_seq = row_seq;
  a.swa_kv = swa->kv;
  a.swa_len = swa->len;
  a.swa_end = swa->row_end;
  a.swa_window = swa->window;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o = o;
  a.lse = lse;
  a.merge_in = 1;
  const csa2_status ws = attach_workspace(a, n_rows, n_heads, 0, swa->window, workspace,
                                          workspace_bytes);
  if (ws != CSA2_OK) return ws;
  hipError_t e = launch_attention(a, n_heads, n_rows, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? CSA2_OK : CSA2_E_HIP;
}

size_t csa2_attn_workspace_size(int32_t n_rows, int32_t n_heads, int32_t k_pos,
                                int32_t swa_window) {
  if (n_rows < 0 || (n_heads != 16 && n_heads != 32 && n_heads != 64) || k_pos < 0 ||
      k_pos > kMaxAttnPos || swa_window < 0 || swa_window > 1024)
    return 0;
  // the most any call of 1 .. n_rows rows needs (the split, and so the
  // bytes, are not monotonic in the row count; rows past 191 never split)
  size_t most = 0;
  const int32_t n = n_rows < 191 ? n_rows : 191;
  for (int32_t r = 1; r <= n; ++r) {
    const size_t b = plan_attention(r, n_heads, k_pos, swa_window).bytes;
    most = b > most ? b : most;
  }
  return most;
}

const char *csa2_status_string(csa2_status status) {
  switch (status) {
    case CSA2_OK: return "CSA2_OK";
    case CSA2_E_INVALID_ARG: return "CSA2_E_INVALID_ARG: invalid argument";
    case CSA2_E_UNSUPPORTED: return "CSA2_E_UNSUPPORTED: shape or size not supported";
    case CSA2_E_WORKSPACE: return "CSA2_E_WORKSPACE: workspace missing, misaligned or too small";
    case CSA2_E_HIP: return "CSA2_E_HIP: HIP runtime error";
  }
  return "CSA2: unknown status";
}

const char *csa2_version(void) { return "csa2 0.1.0 gfx950"; }

}  // extern "C"
