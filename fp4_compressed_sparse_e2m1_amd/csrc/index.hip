// S2-S4: indexer scoring.
//
// Scoring [P1 "무엇과 다른가": the indexer Q scores the indexer keys, which
// are stored next to the main KV; the first decoder Full layer scans the whole
// visible range, later layers only the pool of 2,048 blocks x 8 positions
// (P3 "레이어 40개 가운데 4개만 전역 캐시를 만듭니다")].  The score of entry j
// for a query row is  sum_h w_h * max(0, q_h . k_hat_j)  over 8 heads of 128
// dims, k_hat = E2M1 code x E4M3 scale (one scale per 32 channels).
//
// One wave scores 16 entries per step with four 16x16x32 f16 MFMAs:
//   rows (M) = 16 query heads (8 real, 8 zero), columns (N) = 16 entries,
//   contraction (K) = 128 key channels in 4 steps of 32.
// (Rows that share a sequence are scored in pairs instead -- MFMA rows = two
// queries' 8 heads -- by score_rows_kernel below.)
// Lane (G = lane/16, c = lane%16) loads 16 contiguous bytes of entry c's code
// row -- channels [32G, 32G+32), exactly one scale group -- so the wave reads
// a 1 KiB contiguous tile with one 16-byte load per lane.  MFMA step t uses
// channels 32G + 8t .. +7 from lane group G (the contraction order is
// permuted consistently in the query operand, which does not change the sum).
// Each lane converts its 32 codes with the hardware E2M1 -> f16 conversion
// (unit scale, exact) and multiplies by its group's E4M3 scale in f16
// (exact: the product has at most 6 significant bits).  The bf16 query is
// converted to f16 once per work-group.  Products are exact in the MFMA and
// accumulate in fp32.
//
// The Top-K selection over the scores is in select.hip.

#include "device.h"
#include "encode.h"
#include "internal.h"

#include <type_traits>

namespace csa2 {
namespace {

constexpr int kScoreThreads = 256;
// Scoring of at least this many rows, at least two per sequence on average,
// shares each key tile among 8 rows.
constexpr int kScoreRowsMin = 8;
// Entries per work-group of the many-row scoring (32 tiles per wave).
constexpr int kScoreRowsChunk = 2048;

// Entries per work-group: long contiguous runs for the scan, short ones for the
// pool gather (its pool-id -> key loads form a dependent chain).
template <int MODE>
constexpr int score_chunk() { return MODE == kScorePool ? kScorePoolChunk : kScoreChunk; }

template <int MODE, int U = 4, int CHUNK = score_chunk<MODE>(),
          bool ILV = false, bool ROWFAST = false>
__global__ void __launch_bounds__(kScoreThreads)
score_kernel(ScoreArgs a) {
  constexpr int kChunk = CHUNK;
  constexpr int kTilesPerWave = kChunk / (4 * 16);
  int r = ROWFAST ? blockIdx.x : blockIdx.y;
  int chunk_id = ROWFAST ? blockIdx.y : blockIdx.x;
  if (MODE == kScoreBlockMax && !ROWFAST && a.app_ik) {
    // A scan with an append takes each row's chunks from the last (where a
    // decode row's newest entry sits, encoded by that work-group before its
    // scan), and the first work-groups dispatched, (x, 0) for x < n_rows,
    // trade places with the rows' first ones, (0, x): every row's appending
    // work-group starts at once and its longer run hides under the rest of
    // the grid.  (Rows stay the slow index otherwise: interleaving the rows'
    // chunks measured slower.)
    const int x = blockIdx.x, y = blockIdx.y;
    const int n_sw = (int)(gridDim.x < gridDim.y ? gridDim.x : gridDim.y);
    if (y == 0 && x < n_sw) {
      r = x;
      chunk_id = (int)gridDim.x - 1;
    } else if (x == 0 && y < n_sw) {
      r = 0;
      chunk_id = (int)gridDim.x - 1 - y;
    } else {
      r = y;
      chunk_id = (int)gridDim.x - 1 - x;
    }
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = lane >> 4;
  const int c = lane & 15;

  int seq = a.row_seq[r];
  int n_vis = a.row_nvis[r];
  n_vis = n_vis < 0 ? 0 : (n_vis > a.max_nvis ? a.max_nvis : n_vis);
  if (seq < 0 || seq >= a.n_seq) {
    seq = 0;
    n_vis = 0;
  }
  int np = 0;
  if (MODE == kScorePool) {
    np = a.n_pool[r];
    np = np < 0 ? 0 : (np > a.k_blocks ? a.k_blocks : np);
  }
  // slots of this row: entries (scan / flat) or candidate slots (pool)
  const int64_t n_slots = (MODE == kScorePool) ? (int64_t)8 * a.k_blocks : (int64_t)n_vis;
  const int64_t chunk0 = (int64_t)chunk_id * kChunk;
  if (chunk0 >= n_slots) return;

  // A scan with an append: the work-group whose chunk holds the row's newest
  // entry (n_vis - 1) first encodes it into both planes, as the append kernel
  // would; the work-group barrier orders those stores before its own loads of
  // the chunk (no other work-group reads the entry: one row per sequence).
  if constexpr (MODE == kScoreBlockMax) {
    const int64_t p = (int64_t)n_vis - 1;
    if (a.app_ik && p >= chunk0 && p < chunk0 + kChunk) {
      const int tid = threadIdx.x;
      const int64_t prow = (int64_t)seq * a.cap + p;   // the entry's plane row
      if (tid < 32)
        encode_group<16>(a.app_lat + (int64_t)r * 512 + 16 * tid, a.kv_codes_w + prow * 256 + 8 * tid,
                         a.kv_scales_w + prow * 32 + tid);
      else if (tid < 36)
        encode_group<32>(a.app_ik + (int64_t)r * 128 + 32 * (tid - 32), a.ik_codes_w + prow * 64 + 16 * (tid - 32),
                         a.ik_scales_w + prow * 4 + (tid - 32));
      __syncthreads();
    }
  }

  // Query operand: lane (G, c) holds head c's channels 32G + 8t .. +7, t = 0..3,
  // times the head's power of two 2^k (from its largest |q| over the four
  // lanes that hold it); relu commutes with the positive factor, so each
  // head's weight takes 2^-k instead.
  uint4 qr[4] = {};
  if (c < 8) {
    const uint4 *qp = reinterpret_cast<const uint4 *>(a.q_idx + ((int64_t)r * 8 + c) * 128 + 32 * G);
#pragma unroll
    for (int t = 0; t < 4; ++t) qr[t] = qp[t];
  }
  u16x2 m2 = {0, 0};
#pragma unroll
  for (int t = 0; t < 4; ++t) m2 = bf16x8_absmax(qr[t], m2);
  const int kq = q_prescale_exp(umax_rows(absmax_bits(m2)));
  f16x8 qa[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) qa[t] = bf16x8_to_f16_scaled(qr[t], exp2i(kq));
  float wh[4] = {0.f, 0.f, 0.f, 0.f};
  if (G < 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wh[i] = a.w[(int64_t)r * 8 + 4 * G + i];
  }
  // the weight of head 4G + i takes the exponent held by lane 4G + i
#pragma unroll
  for (int i = 0; i < 4; ++i) wh[i] *= exp2i(-__builtin_amdgcn_ds_bpermute(4 * (4 * G + i), kq));

  const uint8_t *codes_base = a.ik_codes + (int64_t)seq * a.cap * 64;
  const uint8_t *scales_base = a.ik_scales + (int64_t)seq * a.cap * 4;
  uint32_t *out_row = a.keys_out + (int64_t)r * a.out_stride;

  // tile t of this wave: contiguous per wave, or interleaved across the 4 waves
  auto tile_slot0 = [&](int t) -> int64_t {
    return ILV ? chunk0 + ((int64_t)t * 4 + wave) * 16 : chunk0 + ((int64_t)wave * kTilesPerWave + t) * 16;
  };
  // FULL: every slot of the chunk is a visible entry (all chunks of a scan
  // but a row's last), so loads need no masking and the tiles' addresses are
  // constant offsets from one base.
  const bool block_writer = lane < 16 && (c & 7) == 0;
  auto run = [&](auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    // FULL: this lane's code / scale addresses of tile 0; tile t adds a
    // constant (the tiles of a chunk are at fixed distances)
    const int64_t slot00 = tile_slot0(0) + c;
    const uint8_t *cbase = codes_base + slot00 * 64 + 16 * G;
    const uint8_t *sbase = scales_base + slot00 * 4 + G;
    for (int tb = 0; tb < kTilesPerWave; tb += U) {
      if (!FULL && tile_slot0(tb) >= n_slots) break;
      uint4 craw[U];
      uint32_t sraw[U];
      int64_t slot[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        slot[u] = tile_slot0(tb + u) + c;
        if (FULL) {
          const int64_t d = ILV ? ((int64_t)(tb + u) * 4) * 16 : (int64_t)(tb + u) * 16;
          valid[u] = true;
          if (MODE == kScoreBlockMax) {
            // The scan reads every key once: non-temporal loads keep its
            // stream from evicting what the later layers reuse from L2 and the
            // Infinity Cache (pool keys, gathered latents, SWA rows).
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(cbase + d * 64));
            craw[u] = uint4{v[0], v[1], v[2], v[3]};
            sraw[u] = __builtin_nontemporal_load(sbase + d * 4);
          } else {
            craw[u] = *reinterpret_cast<const uint4 *>(cbase + d * 64);
            sraw[u] = sbase[d * 4];
          }
          continue;
        }
        int64_t entry;
        if (MODE == kScorePool) {
          // the pool id is read whether or not p < n_pool, so the read need
          // not wait for the count; p is clamped into the row (the tiles
          // after the first of a group can start past the row's 8 k_blocks
          // slots, and such slots are masked: p >= k_blocks >= n_pool)
          const int64_t p = slot[u] >> 3;
          const int64_t pc = p < a.k_blocks ? p : (int64_t)a.k_blocks - 1;
          const int b = a.pool_blocks[(int64_t)r * a.k_blocks + pc];
          entry = (int64_t)b * 8 + (slot[u] & 7);
          valid[u] = (p < np) && b >= 0 && entry < n_vis;
        } else {
          entry = slot[u];
          valid[u] = entry < n_vis;
        }
        const int64_t e_ld = valid[u] ? entry : 0;
        craw[u] = *reinterpret_cast<const uint4 *>(codes_base + e_ld * 64 + 16 * G);
        sraw[u] = scales_base[e_ld * 4 + G];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const _Float16 s = e4m3_to_f16(sraw[u]);
        const f16x8 sv = f16x8{s, s, s, s, s, s, s, s};
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma16x16x32(qa[0], e2m1x8_to_f16(craw[u].x) * sv, acc);
        acc = mfma16x16x32(qa[1], e2m1x8_to_f16(craw[u].y) * sv, acc);
        acc = mfma16x16x32(qa[2], e2m1x8_to_f16(craw[u].z) * sv, acc);
        acc = mfma16x16x32(qa[3], e2m1x8_to_f16(craw[u].w) * sv, acc);
        // lane (G, c): d[head 4G + i][entry c]; heads 8..15 are zero padding
        float part = wh[0] * relu(acc[0]) + wh[1] * relu(acc[1]);
        part += wh[2] * relu(acc[2]) + wh[3] * relu(acc[3]);
        const float score = part + swap_rows16(part);   // heads 0..3 + heads 4..7
        if (MODE == kScoreBlockMax) {
          uint32_t key = score_key(score);
          if (!FULL) key = valid[u] ? key : 0u;
          key = umax8(key);
          const int64_t blk = slot[u] >> 3;
          if (block_writer && (FULL || blk * 8 < n_slots)) out_row[blk] = key;
        } else if (MODE == kScoreFlat) {
          if (lane < 16 && valid[u]) out_row[slot[u]] = score_key(score);
        } else {
          if (lane < 16 && slot[u] < n_slots) out_row[slot[u]] = valid[u] ? score_key(score) : 0u;
        }
      }
    }
  };
  if (MODE != kScorePool && chunk0 + kChunk <= n_slots)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// Scoring of many query rows that share sequences: prefill (consecutive query
// tokens of one sequence, flat mode) and multi-query decode (several queries of
// one sequence, e.g. draft tokens checked together, block-max mode).  A
// work-group takes kRows = 2 * RP consecutive rows and one chunk of entries.
// Each 16-entry tile is loaded and dequantised once and multiplied against
// every pair of rows: MFMA rows 0..7 are the first row's 8 heads and rows
// 8..15 the second row's, so no matrix row is padding and the key reads and
// conversions are shared by the work-group's rows of one sequence.  Rows of
// one work-group that belong to different sequences are scored one sequence
// at a time (each pass covers the rows of one sequence).  MODE: kScoreFlat
// writes every visible entry's key, kScoreBlockMax the maximum key of each
// block of 8 entries (over the row's visible entries).
template <int RP, int MODE>
__global__ void __launch_bounds__(kScoreThreads)
score_rows_kernel(ScoreArgs a, int32_t n_rows) {
  static_assert(MODE == kScoreFlat || MODE == kScoreBlockMax, "flat or block-max scoring");
  static_assert(RP % 2 == 0, "row pairs are combined two at a time");
  constexpr int kRows = 2 * RP;
  constexpr int kTilesPerWave = kScoreRowsChunk / (4 * 16);
  constexpr int U = 4;
  const int r0 = blockIdx.y * kRows;
  const int64_t chunk0 = (int64_t)blockIdx.x * kScoreRowsChunk;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = lane >> 4;
  const int c = lane & 15;

  int seq[kRows], nv[kRows];
  uint32_t pending = 0;
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int r = r0 + i;
    seq[i] = -1;
    nv[i] = 0;
    if (r < n_rows) {
      const int s = a.row_seq[r];
      int n = a.row_nvis[r];
      n = n < 0 ? 0 : (n > a.max_nvis ? a.max_nvis : n);
      if (s < 0 || s >= a.n_seq) n = 0;
      seq[i] = s;
      nv[i] = n;
      if (n > chunk0) pending |= 1u << i;
    }
  }
  if (!pending) return;

  // Query operand of pair p: lane (G, c) holds MFMA row c = head (c & 7) of
  // row 2p + (c >> 3), channels 32G + 8t .. +7 for step t.
  f16x8 qa[RP][4];
  // Output side: lane (G, c) ends with MFMA rows 4G .. 4G+3 = heads
  // 4(G & 1) .. +3 of row 2p + (G >> 1), entry c.
  float wh[RP][4];
#pragma unroll
  // Each (row, head) enters with its power of two 2^k (from its largest |q|
  // over the four lanes that hold it) and its weight takes 2^-k: the weight
  // of lane (G, c)'s output head 4 (G & 1) + i of row 2p + (G >> 1) takes the
  // exponent of lane 4G + i, which holds that head.
  for (int p = 0; p < RP; ++p) {
    const int rq = r0 + 2 * p + (c >> 3);
    uint4 qr[4] = {};
    if (rq < n_rows) {
      const uint4 *qp = reinterpret_cast<const uint4 *>(a.q_idx + ((int64_t)rq * 8 + (c & 7)) * 128 + 32 * G);
#pragma unroll
      for (int t = 0; t < 4; ++t) qr[t] = qp[t];
    }
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) m2 = bf16x8_absmax(qr[t], m2);
    const int kq = q_prescale_exp(umax_rows(absmax_bits(m2)));
#pragma unroll
    for (int t = 0; t < 4; ++t) qa[p][t] = bf16x8_to_f16_scaled(qr[t], exp2i(kq));
    const int rw = r0 + 2 * p + (G >> 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float wv = rw < n_rows ? a.w[(int64_t)rw * 8 + 4 * (G & 1) + i] : 0.f;
      wh[p][i] = wv * exp2i(-__builtin_amdgcn_ds_bpermute(4 * (4 * G + i), kq));
    }
  }

  while (pending) {
    const int lead = __builtin_ctz(pending);
    int s = 0;
#pragma unroll
    for (int i = 0; i < kRows; ++i)
      if (i == lead) s = seq[i];
    uint32_t act = 0;
    int nmax = 0, nmin = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      if (((pending >> i) & 1u) && seq[i] == s) {
        act |= 1u << i;
        nmax = nv[i] > nmax ? nv[i] : nmax;
        nmin = nv[i] < nmin ? nv[i] : nmin;
      }
    }
    pending &= ~act;
    // Two row pairs share one epilogue: lane (G, c) ends with the score of
    // row 2p + 2(G & 1) + (G >> 1) (p even), entry c, and writes it when that
    // row is in this pass and the entry is below its n_vis.
    int wr_nv[RP / 2];
    uint32_t *out[RP / 2];
#pragma unroll
    for (int p2 = 0; p2 < RP / 2; ++p2) {
      const int i = 4 * p2 + 2 * (G & 1) + (G >> 1);
      int n = 0;
#pragma unroll
      for (int j = 0; j < kRows; ++j)
        if (j == i) n = nv[j];
      wr_nv[p2] = ((act >> i) & 1u) ? n : 0;
      out[p2] = a.keys_out + (int64_t)(r0 + i) * a.out_stride;
    }
    const int slot00 = (int)chunk0 + wave * kTilesPerWave * 16 + c;
    const uint8_t *codes_base = a.ik_codes + (int64_t)s * a.cap * 64;
    const uint8_t *scales_base = a.ik_scales + (int64_t)s * a.cap * 4;
    auto run = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      // batch of U tiles starting at tile tb: raw code and scale loads
      auto load = [&](int tb, uint4 *craw, uint32_t *sraw) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = slot00 + (tb + u) * 16;
          const int e_ld = (FULL || e < nmax) ? e : 0;
          craw[u] = *reinterpret_cast<const uint4 *>(codes_base + (int64_t)e_ld * 64 + 16 * G);
          sraw[u] = scales_base[(int64_t)e_ld * 4 + G];
        }
      };
      auto compute = [&](int tb, const uint4 *craw, const uint32_t *sraw) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int e = slot00 + (tb + u) * 16;
          const _Float16 sc = e4m3_to_f16(sraw[u]);
          const f16x8 sv = f16x8{sc, sc, sc, sc, sc, sc, sc, sc};
          const f16x8 k0 = e2m1x8_to_f16(craw[u].x) * sv;
          const f16x8 k1 = e2m1x8_to_f16(craw[u].y) * sv;
          const f16x8 k2 = e2m1x8_to_f16(craw[u].z) * sv;
          const f16x8 k3 = e2m1x8_to_f16(craw[u].w) * sv;
          f32x4 acc[RP];
#pragma unroll
          for (int p = 0; p < RP; ++p) {
            acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[p] = mfma16x16x32(qa[p][0], k0, acc[p]);
            acc[p] = mfma16x16x32(qa[p][1], k1, acc[p]);
            acc[p] = mfma16x16x32(qa[p][2], k2, acc[p]);
            acc[p] = mfma16x16x32(qa[p][3], k3, acc[p]);
          }
#pragma unroll
          for (int p2 = 0; p2 < RP / 2; ++p2) {
            float pa = wh[2 * p2][0] * relu(acc[2 * p2][0]) + wh[2 * p2][1] * relu(acc[2 * p2][1]);
            pa += wh[2 * p2][2] * relu(acc[2 * p2][2]) + wh[2 * p2][3] * relu(acc[2 * p2][3]);
            float pb = wh[2 * p2 + 1][0] * relu(acc[2 * p2 + 1][0]) + wh[2 * p2 + 1][1] * relu(acc[2 * p2 + 1][1]);
            pb += wh[2 * p2 + 1][2] * relu(acc[2 * p2 + 1][2]) + wh[2 * p2 + 1][3] * relu(acc[2 * p2 + 1][3]);
            // heads 0..3 + heads 4..7 of one row per lane: even G keeps its
            // own pair, odd G the next
            const bool odd = (G & 1) != 0;
            const float x = odd ? pb : pa;
            const float y = odd ? pa : pb;
            const float score = x + swap_rows16(y);
            if (MODE == kScoreFlat) {
              // every score is written once and read once by the selection:
              // non-temporal, like the selection's loads of them
              if (e < wr_nv[p2]) __builtin_nontemporal_store(score_key(score), &out[p2][e]);
            } else {
              // maximum over the visible entries of each block of 8 (lanes
              // c .. c + 7 of a 16-lane row hold one block of one row)
              const uint32_t key = umax8(e < wr_nv[p2] ? score_key(score) : 0u);
              if ((c & 7) == 0 && e < wr_nv[p2]) out[p2][e >> 3] = key;
            }
          }
        }
      };
      // tiles of this wave that hold entries below nmax
      int n_tiles = kTilesPerWave;
      if (!FULL) {
        const int left = nmax - (slot00 - c);
        n_tiles = left <= 0 ? 0 : (left >= kTilesPerWave * 16 ? kTilesPerWave : (left + 15) / 16);
      }
      if (n_tiles == 0) return;
      // two batches in flight: the next batch's loads are issued before the
      // current batch is converted and multiplied
      uint4 ca[U], cb[U];
      uint32_t sa_[U], sb[U];
      load(0, ca, sa_);
      if constexpr (FULL) {
        // a whole chunk: every pass issues the same loads (the last one
        // re-reads its own second batch), so no load is conditional and each
        // wait names exactly the batch it needs
        static_assert(kTilesPerWave % (2 * U) == 0, "whole passes per chunk");
#pragma unroll 1
        for (int tb = 0; tb < kTilesPerWave; tb += 2 * U) {
          load(tb + U, cb, sb);
          compute(tb, ca, sa_);
          load(tb + 2 * U < kTilesPerWave ? tb + 2 * U : tb + U, ca, sa_);
          compute(tb + U, cb, sb);
        }
      } else {
        for (int tb = 0; tb < n_tiles; tb += 2 * U) {
          if (tb + U < n_tiles) load(tb + U, cb, sb);
          compute(tb, ca, sa_);
          if (tb + U >= n_tiles) break;
          if (tb + 2 * U < n_tiles) load(tb + 2 * U, ca, sa_);
          compute(tb + U, cb, sb);
        }
      }
    };
    if (chunk0 + kScoreRowsChunk <= nmin)
      run(std::true_type{});
    else
      run(std::false_type{});
  }
}

}  // namespace

hipError_t launch_score(ScoreMode mode, const ScoreArgs &a, int32_t n_rows, int64_t slots,
                        hipStream_t stream) {
  const int chunk = mode == kScorePool ? kScorePoolChunk : kScoreChunk;
  const int64_t chunks = (slots + chunk - 1) / chunk;
  if (chunks == 0 || n_rows == 0) return hipSuccess;
  // Rows that share sequences (at least two rows per sequence on average)
  // share each key tile: the many-row kernel.  Rows of distinct sequences run
  // one per work-group.
  // (A scan with an append keeps one row per work-group: its rows name
  // distinct sequences.)
  if (mode != kScorePool && !a.app_ik && n_rows >= kScoreRowsMin && n_rows >= 2 * (int64_t)a.n_seq &&
      slots <= ((int64_t)1 << 30)) {
    // 8 rows per work-group; 4 when the sequences have at most 4 rows each on
    // average (a few queries per sequence), so a work-group's rows are mostly
    // one sequence's and no pass multiplies against rows it does not score
    const int rp = n_rows <= 4 * (int64_t)a.n_seq ? 2 : 4;
    dim3 grid((unsigned)((slots + kScoreRowsChunk - 1) / kScoreRowsChunk),
              (unsigned)((n_rows + 2 * rp - 1) / (2 * rp)));
    if (mode == kScoreFlat) {
      if (rp == 2)
        score_rows_kernel<2, kScoreFlat><<<grid, kScoreThreads, 0, stream>>>(a, n_rows);
      else
        score_rows_kernel<4, kScoreFlat><<<grid, kScoreThreads, 0, stream>>>(a, n_rows);
    } else {
      if (rp == 2)
        score_rows_kernel<2, kScoreBlockMax><<<grid, kScoreThreads, 0, stream>>>(a, n_rows);
      else
        score_rows_kernel<4, kScoreBlockMax><<<grid, kScoreThreads, 0, stream>>>(a, n_rows);
    }
    return hipGetLastError();
  }
  dim3 grid((unsigned)chunks, (unsigned)n_rows);
  switch (mode) {
    case kScoreBlockMax: score_kernel<kScoreBlockMax><<<grid, kScoreThreads, 0, stream>>>(a); break;
    case kScoreFlat: score_kernel<kScoreFlat><<<grid, kScoreThreads, 0, stream>>>(a); break;
    default: score_kernel<kScorePool><<<grid, kScoreThreads, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace csa2
