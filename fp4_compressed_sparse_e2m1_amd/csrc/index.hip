// S2-S4: indexer scoring and Top-K selection.
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
// Selection: scores are mapped to order-preserving uint32 keys (0 = no
// candidate).  A 1,024-thread work-group holds up to 16,384 keys of one row in
// registers (16 per thread; 32 per thread for rows of up to 32,768 keys that
// are selected in one level).  One LDS histogram of up to 4,096 bins over the
// first digit -- a window ending at the largest key, or the plain digit below
// the highest bit in which the keys differ -- names the bin holding the k-th
// key; the keys at or above that bin are gathered, in position order with
// their ids, into an LDS list; the remaining bits are resolved from the list
// and the output is compacted from it, ties at the threshold going to the
// lowest positions.  A generic radix path (12-bit digits, then one wave on the
// keys still in play, then a ballot-ordered compaction from registers) covers
// the cases the list cannot hold.  Rows with more keys are cut into chunks
// whose Top-k survivors feed a further level, which keeps the result exact
// because a global Top-k element is in its chunk's Top-k.

#include "device.h"
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
  const int r = ROWFAST ? blockIdx.x : blockIdx.y;
  const int chunk_id = ROWFAST ? blockIdx.y : blockIdx.x;
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

// ------------------------------------------------------------- selection
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
// Keys per thread: a work-group holds one chunk of up to kSelectChunk keys in
// registers.  Thread (wave w, lane l) holds positions w * kSelSpan + 64 j + l,
// j < kKeysPerThread, so every wave owns a contiguous range and every load is
// lane-contiguous.
constexpr int kKeysPerThread = kSelectChunk / kSelThreads;
constexpr int kSelSpan = 64 * kKeysPerThread;
// Radix digits: up to 12 bits while the whole work-group counts, 10 bits once
// one wave finishes alone on at most kCandCap keys gathered in LDS.
constexpr int kSelBits = 12;
constexpr int kSelBins = 1 << kSelBits;
constexpr int kWaveBits = 10;
constexpr int kCandCap = 2048;
// First digit of the common case: a window of kSelBins bins of 2^kWinShift
// key units ending at the largest key (for scores >= 0: the top four octaves
// at 1/1024-octave resolution).  It is used when the keys span more than the
// plain 12-bit first digit would resolve that finely.
constexpr int kWinShift = 13;
// (key, id) pairs at or above the threshold's window bin, kept in LDS in
// position order.
constexpr int kListCap = 4096;

// Reductions over the 64 lanes of a wave (DPP inside 16-lane rows, then the
// row swaps); every lane receives the result.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, int lane, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppXor1, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppXor2, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppHalfMirror, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppRowRor8, 0xF, 0xF, false));
  const auto s16 = __builtin_amdgcn_permlane16_swap((int)x, (int)x, false, false);
  x = op(x, (uint32_t)(((lane >> 4) & 1) ? s16[0] : s16[1]));
  const auto s32 = __builtin_amdgcn_permlane32_swap((int)x, (int)x, false, false);
  return op(x, (uint32_t)(lane < 32 ? s32[1] : s32[0]));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each row
// of 16 lanes (DPP, zero fill), then the totals of the lower rows added from
// lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(x, 15);
  const int t1 = __builtin_amdgcn_readlane(x, 31);
  const int t2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row == 0 ? 0 : (row == 1 ? t0 : (row == 2 ? t0 + t1 : t0 + t1 + t2)));
}

// Orders the LDS accesses of one wave before and after it (no work-group
// barrier: the other waves are not involved).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct Digit {
  int digit;   // bin holding the k_rem-th largest key
  int above;   // keys in higher bins
  int count;   // keys in that bin
  int total;   // keys in the whole histogram
};

// One wave finds, in a histogram of nb bins (a power of two, 2 .. 4096), the
// bin that holds the k_rem-th largest key, counting from the top bin down.
// Lane l first sums the l-th group of nb/64 bins from the top; a prefix sum
// over the lanes names the group, and a second one over that group's bins
// (one per lane) names the bin.
__device__ __forceinline__ Digit find_digit(const uint32_t *hist, int nb, int k_rem, int lane) {
  const int per = nb >= 64 ? nb / 64 : 1;
  const int top = nb - lane * per;        // this lane's group: bins [top - per, top)
  int local = 0;
  if (top > 0) {
    if (per >= 4) {
      for (int i = 0; i < per; i += 4) {
        const uint4 v = *reinterpret_cast<const uint4 *>(&hist[top - per + i]);
        local += (int)(v.x + v.y + v.z + v.w);
      }
    } else {
      for (int i = 0; i < per; ++i) local += (int)hist[top - per + i];
    }
  }
  const int incl = wave_incl_scan(local, lane);
  const unsigned long long hit = __ballot(incl >= k_rem);
  const int o = hit ? __ffsll((long long)hit) - 1 : 0;      // the group holding the bin
  const int excl_o = __builtin_amdgcn_readlane(incl - local, o);
  const int gtop = nb - o * per;
  const int c = lane < per ? (int)hist[gtop - 1 - lane] : 0;
  const int cum = excl_o + wave_incl_scan(c, lane);
  const unsigned long long hit2 = __ballot(lane < per && cum >= k_rem);
  const int l2 = hit2 ? __ffsll((long long)hit2) - 1 : 0;
  Digit d;
  d.total = __builtin_amdgcn_readlane(incl, 63);
  d.digit = gtop - 1 - l2;
  d.count = __builtin_amdgcn_readlane(c, l2);
  d.above = __builtin_amdgcn_readlane(cum, l2) - d.count;
  return d;
}

// KPT keys per thread: a work-group holds up to kSelThreads * KPT keys of a
// row (16: the chunk of the multi-level selection; 32: a whole row of up to
// 32,768 keys in one level).
template <bool FINAL, bool IDS, int KPT = kKeysPerThread>
__global__ void __launch_bounds__(kSelThreads)
select_kernel(SelectArgs a) {
  constexpr int kKeys = KPT;
  constexpr int kSpan = 64 * KPT;
  constexpr int kChunkKeys = kSelThreads * KPT;
  __shared__ __attribute__((aligned(16))) uint32_t hist[kSelBins];
  __shared__ uint32_t s_lkey[kListCap];   // the list's keys; the candidates of the generic path
  __shared__ int32_t s_lid[kListCap];
  __shared__ int32_t s_pool[FINAL ? kMaxPoolBlocks : 1];
  __shared__ int s_red[kSelWaves * 2];
  __shared__ uint32_t s_min[kSelWaves], s_max[kSelWaves];
  __shared__ int s_digit, s_above, s_ncand, s_flag;
  __shared__ uint32_t s_thr;
  __shared__ int s_keq;

  const int r = blockIdx.y;
  const int chunk = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int n_row;
  if (a.count_kind == kCountFixed) {
    n_row = a.count_fixed;
  } else {
    int seq = a.row_seq[r];
    int nv = a.row_nvis[r];
    nv = nv < 0 ? 0 : (nv > a.max_nvis ? a.max_nvis : nv);
    if (seq < 0 || seq >= a.n_seq) nv = 0;
    n_row = (a.count_kind == kCountNvis) ? nv : (nv + 7) / 8;
  }
  const int64_t start = (int64_t)chunk * kChunkKeys;
  int n = (int)((int64_t)n_row - start);
  n = n < 0 ? 0 : (n > kChunkKeys ? kChunkKeys : n);

  // keys (and carried ids) into registers.  The loads are bounded by the
  // row's stride, which the host knows, not by the row's count n, so they do
  // not wait for the count; positions at or past n are cleared afterwards.
  const uint32_t *kin = a.keys_in + (int64_t)r * a.in_stride + start;
  const int64_t in_left = a.in_stride - start;
  const int n_ld = in_left < kChunkKeys ? (int)in_left : kChunkKeys;
  const int base = wave * kSpan + lane;
  uint32_t key[kKeys];
#pragma unroll
  for (int j = 0; j < kKeys; ++j) {
    const int i = base + 64 * j;
    key[j] = i < n_ld ? __builtin_nontemporal_load(&kin[i]) : 0u;   // read once
  }
  int32_t ids[IDS ? kKeys : 1];
  if (IDS) {
    const int32_t *idin = a.ids_in + (int64_t)r * a.in_stride + start;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const int i = base + 64 * j;
      ids[j] = i < n_ld ? idin[i] : -1;
    }
  }
  // the pool row, for mapping candidate slots to entries (read in full;
  // slots past n_pool are masked when mapped)
  int np = 0;
  if (FINAL && a.map_kind == kMapPool) {
    for (int i = tid; i < a.k_blocks; i += kSelThreads) s_pool[i] = a.pool_blocks[(int64_t)r * a.k_blocks + i];
    np = a.n_pool[r];
    np = np < 0 ? 0 : (np > a.k_blocks ? a.k_blocks : np);
  }
#pragma unroll
  for (int j = 0; j < kKeys; ++j) {
    if (base + 64 * j >= n) {
      key[j] = 0u;
      if (IDS) ids[j] = -1;
    }
  }
  // count, min and max of the valid (non-zero) keys
  uint32_t nvalid = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < kKeys; ++j) {
    nvalid += key[j] != 0u;
    if (key[j] != 0u) kmin = kmin < key[j] ? kmin : key[j];
    kmax = kmax > key[j] ? kmax : key[j];
  }
  nvalid = wave_reduce(nvalid, lane, [](uint32_t x, uint32_t y) { return x + y; });
  kmin = wave_reduce(kmin, lane, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
  kmax = wave_reduce(kmax, lane, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
  if (lane == 0) {
    s_red[wave] = (int)nvalid;
    s_min[wave] = kmin;
    s_max[wave] = kmax;
  }
#pragma unroll
  for (int i = 0; i < kSelBins / kSelThreads; ++i) hist[tid + kSelThreads * i] = 0;
  __syncthreads();
  int nv_all = 0;
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int v = 0; v < kSelWaves; ++v) {
    nv_all += s_red[v];
    kmin = kmin < s_min[v] ? kmin : s_min[v];
    kmax = kmax > s_max[v] ? kmax : s_max[v];
  }
  const int k_eff = nv_all < a.k ? nv_all : a.k;

  int32_t *out = FINAL ? a.out + (int64_t)r * a.k : nullptr;
  uint32_t *kout = FINAL ? nullptr : a.keys_out + (int64_t)r * a.out_stride + (int64_t)chunk * a.k;
  int32_t *iout = FINAL ? nullptr : a.ids_out + (int64_t)r * a.out_stride + (int64_t)chunk * a.k;
  // writes kept key k (carried id or chunk position `id`) to output slot pos
  auto emit = [&](int pos, uint32_t k, int id) {
    if (FINAL) {
      if (a.map_kind == kMapPool) {
        const int p = id >> 3;
        const int b = (p < np) ? s_pool[p] : -1;
        id = b * 8 + (id & 7);
      }
      out[pos] = id;
    } else {
      kout[pos] = k;
      iout[pos] = id;
    }
  };

  // Common case: one first digit, then a list.  The first digit is either a
  // window of kSelBins bins of 2^kWinShift key units ending at the largest
  // key (when the keys spread beyond what a plain 12-bit digit resolves that
  // finely), or the plain digit of up to 12 bits below the highest bit in
  // which the keys differ.  Its histogram names the bin that holds the
  // k_eff-th largest key; every key at or above that bin goes, in position
  // order, into an LDS list (about k_eff keys plus one bin); the remaining
  // (at most 13) bits are resolved block-wide from the list, and the output
  // is compacted from the list.  Falls back to the generic path when the
  // k_eff-th key lies below the window or the list would overflow.
  bool listed = false;
  if (k_eff < nv_all && kmin != kmax) {
    const int hb = 31 - __clz(kmin ^ kmax);
    const bool win = hb > kWinShift + kSelBits - 1;
    const int shift0 = win ? kWinShift : (hb + 1 > kSelBits ? hb + 1 - kSelBits : 0);
    const int width0 = win ? kSelBits : hb + 1 - shift0;
    // first-digit bin of a key: (key >> shift0) - base_bin, in [0, 2^width0)
    // for every valid key at or above the window (all valid keys share the
    // bits above hb in the plain case)
    const uint32_t top_bin = kmax >> shift0;
    const uint32_t base_bin =
        win ? (top_bin >= (uint32_t)(kSelBins - 1) ? top_bin - (kSelBins - 1) : 0u) : (top_bin >> width0) << width0;
#pragma unroll
    for (int j = 0; j < kKeys; ++j)
      if (key[j] != 0u && (key[j] >> shift0) >= base_bin) atomicAdd(&hist[(key[j] >> shift0) - base_bin], 1u);
    __syncthreads();
    if (wave == 0) {
      const Digit d = find_digit(hist, 1 << width0, k_eff, lane);
      if (lane == 0) {
        s_digit = d.digit;
        s_above = d.above;
        s_ncand = d.count;
        s_flag = d.total >= k_eff && d.above + d.count <= kListCap;
      }
    }
    __syncthreads();
    listed = s_flag != 0;
    if (listed) {
      // bins 0 .. 191 serve the two refining passes below
      if (tid < 192) hist[tid] = 0;
      const uint32_t lo_key = (base_bin + (uint32_t)s_digit) << shift0;
      const int n_list = s_above + s_ncand;
      const unsigned long long lt = (1ull << lane) - 1ull;
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) cnt += __popcll(__ballot(key[j] != 0u && key[j] >= lo_key));
      if (lane == 0) s_red[wave] = cnt;
      __syncthreads();
      int off = 0;
      for (int v = 0; v < wave; ++v) off += s_red[v];
#pragma unroll
      for (int j = 0; j < kKeys; ++j) {
        const bool m = key[j] != 0u && key[j] >= lo_key;
        const unsigned long long bm = __ballot(m);
        if (m) {
          const int e = off + __popcll(bm & lt);
          s_lkey[e] = key[j];
          s_lid[e] = IDS ? ids[j] : (int)(start + base + 64 * j);
        }
        off += __popcll(bm);
      }
      __syncthreads();
      // The remaining shift0 (<= 13) bits, from the list held in registers
      // (thread t: entries 4t .. 4t+3): up to 7 bits counted in bins 0..127,
      // then the rest (<= 6) in bins 128..191.
      uint32_t lk[4];
      int32_t li[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        lk[q] = e < n_list ? s_lkey[e] : 0u;
        li[q] = e < n_list ? s_lid[e] : -1;
      }
      const int wA = shift0 < 7 ? shift0 : 7;
      const int sA = shift0 - wA;
      uint32_t prefix = lo_key;
      int k_rem = k_eff - s_above;
      if (wA > 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (lk[q] != 0u && (lk[q] >> shift0) == (prefix >> shift0))
            atomicAdd(&hist[(lk[q] >> sA) & ((1u << wA) - 1u)], 1u);
        __syncthreads();
        if (wave == 0) {
          const Digit d = find_digit(hist, 1 << wA, k_rem, lane);
          if (lane == 0) {
            s_digit = d.digit;
            s_above = d.above;
          }
        }
        __syncthreads();
        prefix |= (uint32_t)s_digit << sA;
        k_rem -= s_above;
      }
      if (sA > 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (lk[q] != 0u && (lk[q] >> sA) == (prefix >> sA)) atomicAdd(&hist[128 + (lk[q] & ((1u << sA) - 1u))], 1u);
        __syncthreads();
        if (wave == 0) {
          const Digit d = find_digit(hist + 128, 1 << sA, k_rem, lane);
          if (lane == 0) {
            s_digit = d.digit;
            s_above = d.above;
          }
        }
        __syncthreads();
        prefix |= (uint32_t)s_digit;
        k_rem -= s_above;
      }
      // every thread has followed the same digits
      const uint32_t thr = prefix;
      const int k_eq = k_rem;
      // ordered compaction of the list; above-threshold and tie counts
      // travel packed in one prefix sum
      int packed = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) packed += (int)(lk[q] > thr) + ((int)(lk[q] == thr) << 16);
      const int incl = wave_incl_scan(packed, lane);
      if (lane == 63) s_red[wave] = incl;
      __syncthreads();
      int run = incl - packed;
      for (int v = 0; v < wave; ++v) run += s_red[v];
      int run_gt = run & 0xFFFF, run_eq = run >> 16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool gt = lk[q] > thr;
        const bool eq = lk[q] == thr;
        if (gt || (eq && run_eq < k_eq)) emit(run_gt + (run_eq < k_eq ? run_eq : k_eq), lk[q], li[q]);
        run_gt += gt;
        run_eq += eq;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kSelBins / kSelThreads; ++i) hist[tid + kSelThreads * i] = 0;
      __syncthreads();
    }
  }

  // Generic path.  Radix select of the k_eff-th largest key.  Bits above the highest bit in
  // which the smallest and largest valid keys differ are common to all valid
  // keys, so the digits start there: 12-bit digits counted by the whole
  // work-group from registers, until the keys still in play fit in LDS; one
  // wave then gathers nothing more and finishes them with 10-bit digits.
  if (!listed) {
    uint32_t thr = 0u;
    int k_eq = 0;
    if (k_eff < nv_all) {
      const uint32_t diff = kmin ^ kmax;
      if (diff == 0u) {
        thr = kmin;
        k_eq = k_eff;
      } else {
        const int hb = 31 - __clz(diff);
        uint32_t mask = hb >= 31 ? 0u : ~((2u << hb) - 1u);
        uint32_t prefix = kmin & mask;
        int k_rem = k_eff;
        int top = hb;
        bool gathered = false;
        while (top >= 0) {
          const int width = top + 1 < kSelBits ? top + 1 : kSelBits;
          const int shift = top + 1 - width;
          const uint32_t dmask = (1u << width) - 1u;
  #pragma unroll
          for (int j = 0; j < kKeys; ++j)
            if (key[j] != 0u && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
          __syncthreads();
          if (wave == 0) {
            const Digit d = find_digit(hist, 1 << width, k_rem, lane);
            if (lane == 0) {
              s_digit = d.digit;
              s_above = d.above;
              s_ncand = d.count;
            }
          }
          __syncthreads();
          prefix |= (uint32_t)s_digit << shift;
          mask |= dmask << shift;
          k_rem -= s_above;
          const int ncand = s_ncand;
          top = shift - 1;
  #pragma unroll
          for (int i = 0; i < kSelBins / kSelThreads; ++i) hist[tid + kSelThreads * i] = 0;
          if (top >= 0 && ncand <= kCandCap) {
            // gather the keys still in play, wave by wave (per-wave counts,
            // then each wave's offset)
            const unsigned long long lt = (1ull << lane) - 1ull;
            int cnt = 0;
  #pragma unroll
            for (int j = 0; j < kKeys; ++j)
              cnt += __popcll(__ballot(key[j] != 0u && (key[j] & mask) == prefix));
            if (lane == 0) s_red[wave] = cnt;
            __syncthreads();
            int off = 0;
            for (int v = 0; v < wave; ++v) off += s_red[v];
  #pragma unroll
            for (int j = 0; j < kKeys; ++j) {
              const bool m = key[j] != 0u && (key[j] & mask) == prefix;
              const unsigned long long bm = __ballot(m);
              if (m) s_lkey[off + __popcll(bm & lt)] = key[j];
              off += __popcll(bm);
            }
            gathered = true;
          }
          __syncthreads();
          if (gathered) break;
        }
        if (gathered) {
          if (wave == 0) {
            const int ncand = s_ncand;
            while (top >= 0) {
              const int width = top + 1 < kWaveBits ? top + 1 : kWaveBits;
              const int shift = top + 1 - width;
              const uint32_t dmask = (1u << width) - 1u;
              for (int i = lane; i < ncand; i += 64) {
                const uint32_t k = s_lkey[i];
                if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
              }
              wave_sync();
              const Digit d = find_digit(hist, 1 << width, k_rem, lane);
              prefix |= (uint32_t)d.digit << shift;
              mask |= dmask << shift;
              k_rem -= d.above;
              wave_sync();
              for (int i = lane; i < (1 << width); i += 64) hist[i] = 0;
              wave_sync();
              top = shift - 1;
            }
            if (lane == 0) {
              s_thr = prefix;
              s_keq = k_rem;
            }
          }
          __syncthreads();
          thr = s_thr;
          k_eq = s_keq;
        } else {
          thr = prefix;
          k_eq = k_rem;
        }
      }
    }

    // Ordered compaction from registers: a key's output position is (#keys
    // above the threshold before it) + min(#threshold ties before it, k_eq),
    // counted with ballots; ties are taken lowest position first.
    uint32_t cgt = 0, ceq = 0;
  #pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      cgt += key[j] > thr;
      ceq += (key[j] == thr) && (base + 64 * j < n);
    }
    cgt = wave_reduce(cgt, lane, [](uint32_t x, uint32_t y) { return x + y; });
    ceq = wave_reduce(ceq, lane, [](uint32_t x, uint32_t y) { return x + y; });
    if (lane == 0) {
      s_red[wave] = (int)cgt;
      s_red[kSelWaves + wave] = (int)ceq;
    }
    __syncthreads();
    int run_gt = 0, run_eq = 0;
    for (int v = 0; v < wave; ++v) {
      run_gt += s_red[v];
      run_eq += s_red[kSelWaves + v];
    }
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
  #pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const int i = base + 64 * j;
      const uint32_t k = key[j];
      const bool gt = k > thr;
      const bool eq = (k == thr) && i < n;
      const unsigned long long bgt = __ballot(gt), beq = __ballot(eq);
      const int my_gt = run_gt + __popcll(bgt & lt_mask);
      const int my_eq = run_eq + __popcll(beq & lt_mask);
      run_gt += __popcll(bgt);
      run_eq += __popcll(beq);
      if (gt || (eq && my_eq < k_eq))
        emit(my_gt + (my_eq < k_eq ? my_eq : k_eq), k, IDS ? ids[j] : (int)(start + i));
    }
  }  // generic path
  if (FINAL) {
    for (int i = k_eff + tid; i < a.k; i += kSelThreads) out[i] = -1;
    if (tid == 0) a.n_out[r] = k_eff;
  } else {
    for (int i = k_eff + tid; i < a.k; i += kSelThreads) {
      kout[i] = 0u;
      iout[i] = -1;
    }
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
  if (mode != kScorePool && n_rows >= kScoreRowsMin && n_rows >= 2 * (int64_t)a.n_seq &&
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


hipError_t launch_select(const SelectArgs &a, int32_t n_rows, int32_t n_chunks, bool final_level,
                         bool wide, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  dim3 grid((unsigned)n_chunks, (unsigned)n_rows);
  const bool ids = a.ids_in != nullptr;
  if (wide) {
    // one level over up to kSelectChunkWide keys per row (no carried ids)
    if (!final_level || ids || n_chunks != 1) return hipErrorInvalidValue;
    select_kernel<true, false, kSelectChunkWide / kSelThreads><<<grid, kSelThreads, 0, stream>>>(a);
    return hipGetLastError();
  }
  if (final_level) {
    if (ids)
      select_kernel<true, true><<<grid, kSelThreads, 0, stream>>>(a);
    else
      select_kernel<true, false><<<grid, kSelThreads, 0, stream>>>(a);
  } else {
    if (ids)
      select_kernel<false, true><<<grid, kSelThreads, 0, stream>>>(a);
    else
      select_kernel<false, false><<<grid, kSelThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace csa2
