// S5 + S6: sparse attention over the selected FP4 latents, with the SWA branch
// folded into the same softmax or merged onto an earlier result.
//
// [P1 "무엇과 다른가": every CSA2 mode attends with its own global Q over the
// Top-K of the main KV; P3 "레이어 40개 가운데 4개만 전역 캐시를 만듭니다": the
// main KV is a 512-channel latent; P3 "전역 어텐션과 지역 어텐션": a 128-token
// sliding-window branch; P3 "4비트로 적어도 되는 이유": the SWA cache is FP8.]
// The latent is shared by all heads and is both key and value (one latent per
// entry, no separate V in the 356-B entry).
//
// This file holds the 16- and 32-head kernel (keys split between the waves of
// a work-group, described below), the merge kernel of split rows and the
// launch plan; 64-head layers run the kernel in attention64.hip.  Both use the
// online (running max) softmax in base 2; the running max is only raised
// when a tile's maximum exceeds it by more than 2^8, so most tiles skip the
// rescale of O.  Probabilities enter the P.V product in f16 and the
// normaliser sums the same rounded values, so the weights stay normalised.
#include "device.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kMergeSplitLimit = 64;     // splits a merge accepts
// work-groups a split spreads the rows over (the GPU has 256 CUs)
constexpr int kSplitWorkGroups = 256;
// rows x head groups up to which a split also divides the output channels
// (the quarter kernel); more rows are split by key ranges only
constexpr int kQuarterRows = 16;
constexpr float kLazyRescale = 8.0f;   // log2 units

// Raw share of one key for lane (G, c) of wave w: the key at tile slot
// 16w + c, channels [128G, 128G + 128) -- 64 bytes of E2M1 codes and the 8
// scale bytes of those channels, or 128 E4M3 bytes of an SWA row.
struct KeyFp4 {
  uint4 a[4];
  uint2 sc;
  bool valid;
};
struct KeySwa {
  uint4 a[8];
  bool valid;
};

// Sparse attention, one work-group (4 waves) per (query row, range of its key
// tiles, group of 16 heads) -- or, for very few rows (QUARTERS, below), per
// (row, range, head group, quarter of the 512 output channels).  Keys arrive
// in tiles of 64; wave w owns the tile's keys 16w .. 16w + 15 with all 512
// channels.
//   * Lane (G, c) gathers channels [128G, 128G + 128) of key 16w + c and
//     dequantises them to f16 (exact).
//   * Logits: S^T = K Q^T by 16x16x32 MFMAs over the 512 channels (four
//     independent chains of four); lane (G, c) ends with the logits of keys
//     4G .. 4G + 3 for head c, so a head's maximum over the wave's keys takes
//     three in-lane steps and two lane swaps.  Only the per-head maxima of the
//     four waves cross between waves.
//   * Online softmax in base 2, the running max raised only when a tile
//     exceeds it by more than 2^8 (the O rescale is skipped, by wave ballot,
//     otherwise).  Probabilities enter P.V in f16 and the normaliser sums the
//     same rounded values.
//   * P.V: the waves' P rows and dequantised keys go to LDS; wave w then
//     accumulates channels 128w .. 128w + 127 of O over all 64 keys of the
//     tile, the V operand read back with the hardware transposed LDS read, as
//     O^T = V^T P^T (each lane ends with four consecutive channels of one
//     head, stored with 16-B writes).
// Two work-group barriers per 64 keys.  A 32- or 64-head layer runs 2 or 4
// head groups per row, given block ids that put them on one XCD, so the keys
// they all gather come from its L2.  When a row is split over n_split ranges
// of its tiles, each work-group leaves its unnormalised O, running maxima and
// sums in the workspace for attn_merge_kernel.
//
// QUARTERS (rows x head groups <= kQuarterRows) spreads each row over about
// 256 work-groups: n_split ranges of its key tiles x head groups x four
// channel quarters Q, and merges without a second kernel.
//   * Every wave runs its own online softmax over its 16 keys of each tile
//     (the logits are computed as above), so a tile takes no work-group
//     barrier.  For P.V the 16 lanes that hold channels [128Q, 128Q + 128)
//     stage them in the wave's own LDS rows, and O^T (16 channels x 16 heads
//     per block, eight blocks) += V^T P^T by 16x16x16 MFMAs: V^T through the
//     transposed LDS read, P^T straight from the logit lanes.
//   * At the end the four waves' running maxima, sums and O are merged
//     through LDS into one partial result per work-group (unnormalised O of
//     16 heads x 128 channels, maximum and sum per head).
//   * The work-groups of one (row, head group, quarter) count their arrivals
//     in a counter of the workspace; the last to arrive merges the n_split
//     partials by their log-sum-exp weights, in split order (and the earlier
//     result when merging into (o, lse)), and sets the counter back to zero.
//     The quarters of one (row, split) gather the same keys and all the
//     work-groups of a row get block ids equal modulo 8, so they run on one
//     XCD and share its L2.
constexpr int kKsHeads = 16;
constexpr int kKsVStride = 512 + 8;    // halves per LDS key row (16-B writes of 16 rows on distinct banks)
constexpr int kKsPStride = 64 + 8;     // halves per LDS P row
constexpr int kVqStride = 128 + 8;     // halves per LDS row of one key's channel quarter
constexpr int kOqStride = 128 + 4;     // floats per LDS row of one head's partial O (quarters)
// Raw buffer accesses: the descriptor word of gfx9 raw (untyped) buffers, and
// the cache-policy bit SC1 (device scope) of a buffer load or store.
constexpr int kRawBufferFlags = 0x00020000;
constexpr int kDeviceScope = 16;

// The end of a quarter work-group: the four waves' running maxima, sums and O
// become one partial result; its arrival is counted; and the last of the
// n_split work-groups of its (row, head group, quarter) merges all of them
// into o and lse (with the earlier result when merge_in is set).
__device__ __forceinline__ void quarter_epilogue(const AttnArgs &a, const f32x4 (&acc)[8], float m_run,
                                               float l_wave, int r, int sp, int hg, int Q) {
  constexpr int H = kKsHeads;
  __shared__ __attribute__((aligned(16))) float s_oq[4 * H][kOqStride];   // the waves' O
  __shared__ float s_wm[4][H], s_wl[4][H];                                // the waves' maxima, sums
  __shared__ float s_M[H], s_L[H];                                        // the work-group's
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int G = lane >> 4;
  const int c = lane & 15;
  const int HT = a.n_heads;
  const int h0 = hg * H;
  // the work-group's maximum and sum of head c, and this wave's share of O
  // rescaled to that maximum
  if (G == 0) {
    s_wm[w][c] = m_run;
    s_wl[w][c] = l_wave;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) M = fmaxf(M, s_wm[v][c]);
  float L = 0.f;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float mv = s_wm[v][c];
    L += mv == -INFINITY ? 0.f : s_wl[v][c] * exp2f(mv - M);
  }
  const float f = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
  if (tid < H) {   // wave 0, lane c = tid: head tid
    s_M[tid] = M;
    s_L[tid] = L;
  }
  float *so = s_oq[w * H + c];
#pragma unroll
  for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4 *>(so + 16 * db + 4 * G) = acc[db] * f;
  __syncthreads();
  // thread (hh, j): head h0 + hh, channels 128Q + 8j .. +7, the waves summed
  // in order
  const int hh = tid >> 4;
  const int j = tid & 15;
  f32x4 o0 = f32x4{0.f, 0.f, 0.f, 0.f}, o1 = o0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    o0 += *reinterpret_cast<const f32x4 *>(&s_oq[v * H + hh][8 * j]);
    o1 += *reinterpret_cast<const f32x4 *>(&s_oq[v * H + hh][8 * j + 4]);
  }
  float *orow = a.o + ((int64_t)r * HT + h0 + hh) * 512 + 128 * Q + 8 * j;
  if (a.n_split == 1 && !a.merge_in) {
    // the row is not split (only its channel quarters are): normalise and store
    const float Lh = s_L[hh];
    const float inv = Lh > 0.f ? 1.f / Lh : 0.f;
    *reinterpret_cast<f32x4 *>(orow) = o0 * inv;
    *reinterpret_cast<f32x4 *>(orow + 4) = o1 * inv;
    if (Q == 0 && j == 0)
      a.lse[(int64_t)r * HT + h0 + hh] = Lh > 0.f ? (s_M[hh] + log2f(Lh)) * 0.6931471805599453f : -INFINITY;
    return;
  }
  // The partial goes out with device-scope stores (SC1: written through to
  // the level all XCDs see), every one of them complete before the
  // work-group barrier, so before its arrival is counted; the last arrival
  // sets the counter back to zero and reads the partials with device-scope
  // loads.  (A release / acquire fence pair would write back / invalidate
  // the whole L2 instead, which costs more than the partials.)
  const int ns = a.n_split;
  const __amdgpu_buffer_rsrc_t rs_o =
      __builtin_amdgcn_make_buffer_rsrc(a.part_o, 0, (int)((size_t)a.n_rows * ns * HT * 512 * 4), kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t rs_ml =
      __builtin_amdgcn_make_buffer_rsrc(a.part_ml, 0, (int)((size_t)a.n_rows * ns * 4 * HT * 2 * 4), kRawBufferFlags);
  const int64_t part = (int64_t)r * ns + sp;
  const int off_o = (int)(((part * HT + h0 + hh) * 512 + 128 * Q + 8 * j) * 4);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o0), rs_o, off_o, 0, kDeviceScope);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o1), rs_o, off_o + 16, 0, kDeviceScope);
  if (tid < H) {   // wave 0, lane c = tid: head tid's maximum and sum
    const int off_ml = (int)(((part * 4 + Q) * HT + h0 + tid) * 2 * 4);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, make_float2(M, L)), rs_ml, off_ml, 0, kDeviceScope);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t *cnt = a.counters + ((int64_t)r * a.n_hgroups + hg) * kAttnRowCounters;
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(cnt + Q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == (uint32_t)(a.n_split - 1);
    if (last) __hip_atomic_store(cnt + Q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;

  // Merge: the earlier result (merge_in) enters first with weight 1 at its
  // own maximum, then the splits in ascending order, each folded in by its
  // log-sum-exp weight (online: the running sum is rescaled when the maximum
  // rises).
  const int h = h0 + hh;
  const int ml_base = (int)((((int64_t)r * ns * 4 + Q) * HT + h) * 2 * 4);
  const int ml_step = 4 * HT * 2 * 4;
  const int o_base = (int)((((int64_t)r * ns * HT + h) * 512 + 128 * Q + 8 * j) * 4);
  const int o_step = HT * 512 * 4;
  float Mr = -INFINITY, Lr = 0.f;
  f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
  if (a.merge_in) {
    const float lin = a.lse[(int64_t)r * HT + h];
    if (lin != -INFINITY) {
      Mr = lin * 1.4426950408889634f;
      Lr = 1.f;
      a0 = *reinterpret_cast<const f32x4 *>(orow);
      a1 = *reinterpret_cast<const f32x4 *>(orow + 4);
    }
  }
  // the partials of up to kBatch splits are requested together (indices
  // past the last split re-read it and are not folded in)
  constexpr int kBatch = 8;
  for (int s0 = 0; s0 < ns; s0 += kBatch) {
    float2 ml[kBatch];
    f32x4 v0[kBatch], v1[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = s0 + u < ns ? s0 + u : ns - 1;
      ml[u] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rs_ml, ml_base + s * ml_step, 0, kDeviceScope));
      v0[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_o, o_base + s * o_step, 0, kDeviceScope));
      v1[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs_o, o_base + s * o_step + 16, 0, kDeviceScope));
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u < ns && ml[u].y > 0.f) {
        const float Mn = fmaxf(Mr, ml[u].x);
        const float sc = Mr == -INFINITY ? 0.f : exp2f(Mr - Mn);
        const float ws = exp2f(ml[u].x - Mn);
        Lr = Lr * sc + ws * ml[u].y;
        a0 = a0 * sc + v0[u] * ws;
        a1 = a1 * sc + v1[u] * ws;
        Mr = Mn;
      }
    }
  }
  const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
  *reinterpret_cast<f32x4 *>(orow) = a0 * inv;
  *reinterpret_cast<f32x4 *>(orow + 4) = a1 * inv;
  const float lse = Lr > 0.f ? (Mr + log2f(Lr)) * 0.6931471805599453f : -INFINITY;
  if (!a.merge_in) {
    if (Q == 0 && j == 0) a.lse[(int64_t)r * HT + h] = lse;
    return;
  }
  // Every quarter's merge reads the earlier lse above: the last of the four
  // to finish writes the new one (all four compute the same value).
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(cnt + 4, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == 3u;
    if (last) __hip_atomic_store(cnt + 4, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (s_last && j == 0) a.lse[(int64_t)r * HT + h] = lse;
}

// Modes of attn_kernel: whole rows; rows split over ranges of their key
// tiles (accumulating O with four heads of one channel per lane, which
// measured faster for the partials); ranges and channel quarters.
constexpr int kModeRows = 0;
constexpr int kModeRanges = 1;
constexpr int kModeQuarters = 2;

template <int MODE>
__global__ void __launch_bounds__(kAttnThreads)
attn_kernel(AttnArgs a) {
  constexpr bool QUARTERS = MODE == kModeQuarters;
  constexpr bool OT = MODE == kModeRows;   // O^T accumulators (else O; quarters: their own)
  constexpr int H = kKsHeads;
  // the tile's keys and P rows, shared by the four waves
  __shared__ __attribute__((aligned(16))) _Float16 s_v[QUARTERS ? 1 : kAttnTileKeys * kKsVStride];
  __shared__ __attribute__((aligned(16))) _Float16 s_p[QUARTERS ? 1 : H * kKsPStride];
  __shared__ __attribute__((aligned(16))) float s_wmax[H][4];
  __shared__ __attribute__((aligned(16))) float s_alpha[H];
  __shared__ float s_wl[4][H];
  __shared__ float s_m[H], s_l[H];
  // quarters: each wave's V rows of the quarter
  __shared__ __attribute__((aligned(16))) _Float16 s_vq[QUARTERS ? 4 : 1][QUARTERS ? 16 * kVqStride : 1];

  // Work-group -> (row, split, head group), or (row, split, head group,
  // quarter): work-groups go to the 8 XCDs in turn, and the head groups of a
  // (row, split) -- all the work-groups of a row, with quarters -- get block
  // ids equal modulo 8, so they run on one XCD; the grid is padded to whole
  // sets of 8.
  const int HT = a.n_heads;
  int r, hg = 0, sp = 0, Q = 0;
  if constexpr (QUARTERS) {
    const int units = a.n_split * a.n_hgroups * 4;
    const int i = blockIdx.x >> 3;
    const int m = i / units;
    const int u = i - m * units;
    r = 8 * m + (blockIdx.x & 7);
    Q = u & 3;
    hg = (u >> 2) % a.n_hgroups;
    sp = (u >> 2) / a.n_hgroups;
  } else {
    int rs = blockIdx.x;   // (row, split)
    if (a.n_hgroups > 1) {
      const int per = 8 * a.n_hgroups;
      const int blk = blockIdx.x / per;
      const int rem = blockIdx.x - blk * per;
      hg = rem >> 3;
      rs = blk * 8 + (rem & 7);
    }
    r = rs / a.n_split;
    sp = rs - r * a.n_split;
  }
  if (r >= a.n_rows) return;
  const int h0 = hg * H;
  // split rows fold (o, lse) in at the merge
  constexpr bool ranges = MODE != kModeRows;
  const bool merge_in = !ranges && a.merge_in;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int G = lane >> 4;
  const int c = lane & 15;

  constexpr int TK = kAttnTileKeys;
  // this work-group's first tile
  const int t_begin = ranges ? sp * a.tiles_per_split : 0;
  const int32_t *topk = a.topk ? a.topk + (int64_t)r * a.k_pos : nullptr;
  // The entry id of this lane's key in tile T, read ahead of need and without
  // waiting for n_topk (every slot below k_pos is inside the row).
  auto load_id = [&](int T) -> int32_t {
    const int slot = T * TK + 16 * w + c;
    return (topk && slot < a.k_pos) ? topk[slot] : -1;
  };
  // The ids of the first three tiles and Q go out before the per-row scalars:
  // scalar loads return out of order, so a use of any of them waits for all,
  // and these loads need none of them.
  int32_t id0 = load_id(t_begin), id1 = load_id(t_begin + 1), id2 = load_id(t_begin + 2);
  uint4 q_raw[16];
  {
    const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + ((int64_t)r * HT + h0 + c) * 512 + 128 * G);
#pragma unroll
    for (int t = 0; t < 16; ++t) q_raw[t] = qp[t];
  }
  __builtin_amdgcn_sched_barrier(0);

  // the per-row scalars are read together and unconditionally (an absent
  // array is stood in for by row_seq); the empty asm takes all three at this
  // point, so one wait covers them and no load is moved into a branch that
  // depends on another
  const int32_t *ntp = a.topk ? a.n_topk : a.row_seq;
  const int32_t *sep = a.swa_kv ? a.swa_end : a.row_seq;
  int seq = a.row_seq[r];
  int n_g = ntp[r];
  int end32 = sep[r];
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::"s"(seq), "s"(n_g), "s"(end32));
  n_g = a.topk ? n_g : 0;
  int64_t end = a.swa_kv ? end32 : 0;
  const bool seq_ok = seq >= 0 && seq < a.n_seq;
  if (!seq_ok) seq = 0;
  n_g = (!seq_ok || n_g < 0) ? 0 : (n_g > a.k_pos ? a.k_pos : n_g);
  int64_t s0 = 0;
  int n_s = 0;
  if (a.swa_kv && seq_ok) {
    end = end < 0 ? 0 : (end > a.swa_len ? a.swa_len : end);
    s0 = end - a.swa_window;
    s0 = s0 < 0 ? 0 : s0;
    n_s = (int)(end - s0);
  }
  const int n_gt = (n_g + TK - 1) / TK;
  const int n_all = n_gt + (n_s + TK - 1) / TK;
  // this work-group's tiles: [t_begin, t_end)
  int t_end = ranges ? t_begin + a.tiles_per_split : n_all;
  t_end = t_end < n_all ? t_end : n_all;

  // Q operand: qa[t] = 2^k q[r][h0 + c][128G + 8t .. +7] in f16, t < 16 (the
  // contraction over the 512 channels runs in this lane-consistent order),
  // with the power of two 2^k of head h0 + c (its largest |q| over the four
  // lanes that hold it); sl = scale * log2(e) * 2^-k scales its logits back
  f16x8 qa[16];
  float sl;
  {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int t = 0; t < 16; ++t) m2 = bf16x8_absmax(q_raw[t], m2);
    const int k = q_prescale_exp(umax_rows(absmax_bits(m2)));
    const float up = exp2i(k);
    sl = a.scale_log2 * exp2i(-k);
#pragma unroll
    for (int t = 0; t < 16; ++t) qa[t] = bf16x8_to_f16_scaled(q_raw[t], up);
  }

  // Accumulators, lane (G, c), block db: whole rows: O[head h0 + c][channels
  // 128w + 16db + 4G .. +3] (four consecutive channels of one head, stored
  // with one 16-B access); ranges: element i is O[head h0 + 4G + i][channel
  // 128w + 16db + c]; quarters: O[head h0 + c][channels 128Q + 16db + 4G ..
  // +3], over this wave's keys only
  f32x4 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (merge_in) {
    const int64_t hrow = (int64_t)r * HT + h0 + c;
    if (a.lse[hrow] != -INFINITY) {
#pragma unroll
      for (int db = 0; db < 8; ++db)
        acc[db] = *reinterpret_cast<const f32x4 *>(a.o + hrow * 512 + 128 * w + 16 * db + 4 * G);
    }
  }
  // softmax state of head c, in every lane (G, c) of every wave: the running
  // max (log2 units), and the normaliser as per-lane partial sums reduced at
  // the end (split: of this wave's keys)
  float m_run = -INFINITY, l_thr = 0.f;
  if (merge_in) {
    const float lin = a.lse[(int64_t)r * HT + h0 + c];
    if (lin != -INFINITY) {
      m_run = lin * 1.4426950408889634f;
      l_thr = (w == 0 && G == 0) ? 1.f : 0.f;
    }
  }

  const uint8_t *kv_codes = a.kv_codes + (int64_t)seq * a.cap * 256;
  const uint8_t *kv_scales = a.kv_scales + (int64_t)seq * a.cap * 32;
  const uint8_t *swa = a.swa_kv ? a.swa_kv + ((int64_t)seq * a.swa_len) * 512 : nullptr;

  auto load_fp4 = [&](int T, int32_t id) {
    KeyFp4 k;
    const int slot = T * TK + 16 * w + c;
    const int64_t e = slot < n_g ? id : -1;
    k.valid = e >= 0 && e < a.cap;
    const int64_t el = k.valid ? e : 0;
    const uint4 *cp = reinterpret_cast<const uint4 *>(kv_codes + el * 256 + 64 * G);
#pragma unroll
    for (int j = 0; j < 4; ++j) k.a[j] = cp[j];
    k.sc = *reinterpret_cast<const uint2 *>(kv_scales + el * 32 + 8 * G);
    return k;
  };
  auto load_swa = [&](int Ts) {       // tile index within the SWA rows
    KeySwa k;
    const int slot = Ts * TK + 16 * w + c;
    k.valid = slot < n_s;
    const int64_t row = k.valid ? s0 + slot : 0;
    const uint4 *p = reinterpret_cast<const uint4 *>(swa + row * 512 + 128 * G);
#pragma unroll
    for (int j = 0; j < 8; ++j) k.a[j] = p[j];
    return k;
  };
  // dequantise to kf[t] = channels 128G + 8t .. +7 (skipped keys load entry 0
  // and are zeroed, so no stale byte pattern can reach the P.V product)
  f16x8 kf[16];
  auto dequant_fp4 = [&](const KeyFp4 &k) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t sw = (t < 8 ? k.sc.x : k.sc.y) >> (8 * ((t >> 1) & 3));
      const _Float16 sc = e4m3_to_f16(sw & 0xFFu);
      const uint32_t dw = t % 4 == 0 ? k.a[t / 4].x : t % 4 == 1 ? k.a[t / 4].y : t % 4 == 2 ? k.a[t / 4].z : k.a[t / 4].w;
      kf[t] = e2m1x8_to_f16(dw) * f16x8{sc, sc, sc, sc, sc, sc, sc, sc};
      if (!k.valid) kf[t] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  };
  auto dequant_swa = [&](const KeySwa &k) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint4 v = k.a[t / 2];
      kf[t] = (t % 2 == 0) ? e4m3x8_to_f16(v.x, v.y) : e4m3x8_to_f16(v.z, v.w);
      if (!k.valid) kf[t] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  };

  // One tile (the dequantised keys in kf): logits, online softmax, P.V.
  auto compute = [&](bool valid) {
    // the wave's valid keys (lanes 0..15 hold keys 0..15)
    const uint32_t vmask = (uint32_t)__builtin_amdgcn_ballot_w64(valid) & 0xFFFFu;
    f32x4 q0 = {0.f, 0.f, 0.f, 0.f}, q1 = q0, q2 = q0, q3 = q0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      q0 = mfma16x16x32(kf[t], qa[t], q0);
      q1 = mfma16x16x32(kf[4 + t], qa[4 + t], q1);
      q2 = mfma16x16x32(kf[8 + t], qa[8 + t], q2);
      q3 = mfma16x16x32(kf[12 + t], qa[12 + t], q3);
    }
    // lane (G, c): logits of keys 4G + i for head c
    float sv[4];
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = (q0[i] + q1[i]) + (q2[i] + q3[i]);
      sv[i] = ((vmask >> (4 * G + i)) & 1u) ? x * sl : -INFINITY;
      lmax = fmaxf(lmax, sv[i]);
    }
    lmax = fmaxf(lmax, swap_rows16(lmax));                       // lanes c, c + 16
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(lmax), __float_as_int(lmax), false, false);
      lmax = fmaxf(lmax, __int_as_float(lane < 32 ? sw[1] : sw[0]));   // and c + 32, c + 48
    }
    // the tile's maximum of head c (split: over this wave's keys of the tile)
    float tmax = lmax;
    if constexpr (!QUARTERS) {
      if (G == 0) s_wmax[c][w] = lmax;
      __syncthreads();
      const float4 wm = *reinterpret_cast<const float4 *>(&s_wmax[c][0]);
      tmax = fmaxf(fmaxf(wm.x, wm.y), fmaxf(wm.z, wm.w));
    }
    float m_new = m_run;
    if (m_run == -INFINITY || tmax > m_run + kLazyRescale) m_new = fmaxf(tmax, m_run);
    // the hardware exp2 (no denormal-range fix-up): arguments are <= 2^8, and
    // results below 2^-126 are negligible weights (f16 drops them too)
    const float alpha = (m_run == -INFINITY || m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    _Float16 ph[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = (m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_new);
      ph[i] = (_Float16)p;
      psum += (float)ph[i];
    }
    l_thr = l_thr * alpha + psum;
    m_run = m_new;
    if constexpr (QUARTERS) {
      // channels [128Q, 128Q + 128) of the wave's 16 keys to its own LDS rows
      if (G == Q) {
#pragma unroll
        for (int t = 0; t < 16; ++t) *reinterpret_cast<f16x8 *>(&s_vq[w][c * kVqStride + 8 * t]) = kf[t];
      }
      wave_sync();
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[db] *= alpha;
      }
      // O^T += V^T P^T over the wave's 16 keys: V[keys 4G .. 4G + 3][channel
      // 128Q + 16db + c] (rows 4G + c/4, read transposed), P[head c][keys
      // 4G .. 4G + 3] as the logit lanes hold it
      const f16x4 pb = f16x4{ph[0], ph[1], ph[2], ph[3]};
      const _Float16 *vr = &s_vq[w][(4 * G + (c >> 2)) * kVqStride + 4 * (c & 3)];
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db] = mfma16x16x16(lds_read_tr16(vr + 16 * db), pb, acc[db]);
      wave_sync();   // these reads end before the next tile's writes
    } else {
      if (w == 0 && G == 0) s_alpha[c] = alpha;
      // this wave's keys (all channels) and P values to LDS
#pragma unroll
      for (int t = 0; t < 16; ++t)
        *reinterpret_cast<f16x8 *>(&s_v[(16 * w + c) * kKsVStride + 128 * G + 8 * t]) = kf[t];
      *reinterpret_cast<f16x4 *>(&s_p[c * kKsPStride + 16 * w + 4 * G]) = f16x4{ph[0], ph[1], ph[2], ph[3]};
      __syncthreads();
      // O^T[quarter w, :] = alpha * O^T + V^T P^T over the tile's 64 keys (the
      // rescale is skipped while the running maxima of these heads stand still)
      if constexpr (OT) {
        const float al = s_alpha[c];
        if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
          for (int db = 0; db < 8; ++db) acc[db] *= al;
        }
      } else {
        const float4 al = *reinterpret_cast<const float4 *>(&s_alpha[4 * G]);
        if (__builtin_amdgcn_ballot_w64(al.x != 1.f || al.y != 1.f || al.z != 1.f || al.w != 1.f)) {
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            acc[db][0] *= al.x;
            acc[db][1] *= al.y;
            acc[db][2] *= al.z;
            acc[db][3] *= al.w;
          }
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // P[head c][keys 32kk + 8G .. +7] and V[keys 32kk + 8G .. +7][channel
        // 128w + 16db + c] (rows 32kk + 8G + 4h + c/4, h = 0, 1, read
        // transposed): O^T += V^T P^T, or O += P V
        const f16x8 pa = *reinterpret_cast<const f16x8 *>(&s_p[c * kKsPStride + 32 * kk + 8 * G]);
        const _Float16 *r0 = &s_v[(32 * kk + 8 * G + (c >> 2)) * kKsVStride + 128 * w + 4 * (c & 3)];
        const _Float16 *r1 = r0 + 4 * kKsVStride;
#pragma unroll
        for (int db = 0; db < 8; db += 2) {
          f16x8 vb[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const f16x4 lo = lds_read_tr16(r0 + 16 * (db + u));
            const f16x4 hi = lds_read_tr16(r1 + 16 * (db + u));
            vb[u] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
#pragma unroll
          for (int u = 0; u < 2; ++u)
            acc[db + u] = OT ? mfma16x16x32(vb[u], pa, acc[db + u]) : mfma16x16x32(pa, vb[u], acc[db + u]);
        }
      }
      // (the next tile writes LDS only after its first barrier, which every
      // wave reaches after finishing these reads)
    }
  };

  // Top-K tiles: while a tile is computed the next two are in flight (the
  // gathers are random HBM reads); the tile registers rotate by copy.
  const int g_end = t_end < n_gt ? t_end : n_gt;
  {
    KeyFp4 ka, kb;
    if (t_begin < g_end) ka = load_fp4(t_begin, id0);
    if (t_begin + 1 < g_end) kb = load_fp4(t_begin + 1, id1);
    for (int T = t_begin; T < g_end; ++T) {
      dequant_fp4(ka);
      const bool v = ka.valid;
      ka = kb;
      if (T + 2 < g_end) kb = load_fp4(T + 2, id2);
      id2 = load_id(T + 3);
      compute(v);
    }
  }
  // SWA tiles (consecutive rows), the next one in flight
  {
    const int sw_begin = (t_begin > n_gt ? t_begin : n_gt) - n_gt;
    const int sw_end = t_end - n_gt;
    KeySwa ks;
    if (sw_begin < sw_end) ks = load_swa(sw_begin);
    for (int Ts = sw_begin; Ts < sw_end; ++Ts) {
      dequant_swa(ks);
      const bool v = ks.valid;
      if (Ts + 1 < sw_end) ks = load_swa(Ts + 1);
      compute(v);
    }
  }

  // normaliser of head c: the lanes of head c, then the waves
  float l_wave;
  {
    float l = l_thr + swap_rows16(l_thr);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(l), __float_as_int(l), false, false);
    l += __int_as_float(lane < 32 ? sw[1] : sw[0]);
    l_wave = l;
  }
  if constexpr (QUARTERS) {
    quarter_epilogue(a, acc, m_run, l_wave, r, sp, hg, Q);
  } else {
    if (G == 0) s_wl[w][c] = l_wave;
    __syncthreads();
    if (tid < H) {
      s_m[tid] = m_run;                   // lane tid holds head tid's state
      s_l[tid] = (s_wl[0][tid] + s_wl[1][tid]) + (s_wl[2][tid] + s_wl[3][tid]);
    }
    __syncthreads();
    if constexpr (MODE == kModeRanges) {
      // unnormalised partial: O, running max (log2 units) and sum per head,
      // merged by attn_merge_kernel
      const int64_t part = (int64_t)r * a.n_split + sp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float *prow = a.part_o + (part * HT + h0 + 4 * G + i) * 512 + 128 * w + c;
#pragma unroll
        for (int db = 0; db < 8; ++db) prow[16 * db] = acc[db][i];
      }
      if (tid < H) {
        a.part_ml[(part * HT + h0 + tid) * 2] = s_m[tid];
        a.part_ml[(part * HT + h0 + tid) * 2 + 1] = s_l[tid];
      }
      return;
    }
    // normalise and store
    const float l = s_l[c];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *orow = a.o + ((int64_t)r * HT + h0 + c) * 512 + 128 * w + 4 * G;
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4 *>(orow + 16 * db) = acc[db] * inv;
    if (tid < H) {
      const float lt = s_l[tid];
      a.lse[(int64_t)r * HT + h0 + tid] = lt > 0.f ? (s_m[tid] + log2f(lt)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

// Merge of the split partials of a row: the softmax over the union of the
// splits' key sets (and of the earlier result in (o, lse) when merge_in is
// set), by their log-sum-exp.  A block handles 2 heads x 512 channels of one
// row (4 outputs per thread); the per-split maxima and sums are staged in LDS.
constexpr int kMergeMaxSplit = kMergeSplitLimit;

__global__ void __launch_bounds__(256)
attn_merge_kernel(AttnArgs a, int H) {
  __shared__ float s_w[2][kMergeMaxSplit + 1];   // weight of each split (+ the earlier result)
  __shared__ float s_L[2], s_M[2];
  const int per_row = H / 2;
  const int r = blockIdx.x / per_row;
  const int h0 = 2 * (blockIdx.x - r * per_row);
  const int tid = threadIdx.x;
  const int ns = a.n_split;
  const int hh = tid >> 7;                 // which of the two heads
  const int d = (tid & 127) * 4;           // four channels
  const int h = h0 + hh;
  const float *po = a.part_o + (((int64_t)r * ns) * H + h) * 512 + d;
  // The first (up to) kMergeBatch splits' partials are requested before the
  // weights are known, so their loads overlap the weight computation; further
  // splits are read in batches of the same size.
  constexpr int kMergeBatch = 32;
  float4 v[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u)
    if (u < ns) v[u] = *reinterpret_cast<const float4 *>(po + (int64_t)u * H * 512);
  // wave 0 weighs the splits of head h0, wave 1 those of head h0 + 1; lane s
  // holds split s
  const int lane = tid & 63;
  const int wv = tid >> 6;
  if (wv < 2) {
    const int hw = h0 + wv;
    float m_in = -INFINITY;
    if (a.merge_in) {
      const float lin = a.lse[(int64_t)r * H + hw];
      if (lin != -INFINITY) m_in = lin * 1.4426950408889634f;
    }
    float m = -INFINITY, l = 0.f;
    if (lane < ns) {
      const float *ml = a.part_ml + (((int64_t)r * ns + lane) * H + hw) * 2;
      m = ml[0];
      l = ml[1];
    }
    float M = (l > 0.f) ? m : -INFINITY;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    M = fmaxf(M, m_in);
    const float wgt = (l > 0.f && M != -INFINITY) ? exp2f(m - M) : 0.f;
    float L = wgt * l;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
    const float win = (m_in != -INFINITY) ? exp2f(m_in - M) : 0.f;
    L += win;
    if (lane < ns) s_w[wv][lane] = wgt;
    if (lane == 0) {
      s_w[wv][ns] = win;
      s_L[wv] = L;
      s_M[wv] = M;
    }
  }
  __syncthreads();
  const float L = s_L[hh];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // splits in ascending order (a fixed summation order)
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) {
    if (u < ns) {
      const float wgt = s_w[hh][u];
      acc.x += wgt * v[u].x;
      acc.y += wgt * v[u].y;
      acc.z += wgt * v[u].z;
      acc.w += wgt * v[u].w;
    }
  }
  for (int s0 = kMergeBatch; s0 < ns; s0 += kMergeBatch) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
      if (s0 + u < ns) v[u] = *reinterpret_cast<const float4 *>(po + (int64_t)(s0 + u) * H * 512);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (s0 + u < ns) {
        const float wgt = s_w[hh][s0 + u];
        acc.x += wgt * v[u].x;
        acc.y += wgt * v[u].y;
        acc.z += wgt * v[u].z;
        acc.w += wgt * v[u].w;
      }
    }
  }
  float4 *orow = reinterpret_cast<float4 *>(a.o + ((int64_t)r * H + h) * 512 + d);
  const float win = s_w[hh][ns];
  if (win > 0.f) {
    const float4 oi = *orow;
    acc.x += win * oi.x;
    acc.y += win * oi.y;
    acc.z += win * oi.z;
    acc.w += win * oi.w;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *orow = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if ((tid & 127) == 0)
    a.lse[(int64_t)r * H + h] = L > 0.f ? (s_M[hh] + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

}  // namespace


AttnPlan plan_attention(int32_t n_rows, int32_t n_heads, int32_t k_pos, int32_t window) {
  // keys per tile of the kernel that serves this head count
  const int tk = n_heads == 64 ? 32 : kAttnTileKeys;
  const int max_tiles = (k_pos + tk - 1) / tk + (window + tk - 1) / tk;
  AttnPlan p = {1, max_tiles > 0 ? max_tiles : 1, 0, 0};
  // Few rows leave most of the 256 CUs idle: spread each row over several
  // work-groups, about kSplitWorkGroups in all -- ranges of its key tiles
  // (one tile each when that many fit), and for very few rows of 16 or 32
  // heads also the head groups and the four channel quarters.  Many rows
  // fill the GPU already, and splitting them would only add partial-result
  // traffic.
  if (n_rows >= 192) return p;
  const int hg = n_heads == 64 ? 1 : n_heads / kKsHeads;
  const bool quarters = n_heads != 64 && n_rows * hg <= kQuarterRows;
  const int per_split = quarters ? 4 * hg : 1;   // work-groups per (row, range)
  int split = (kSplitWorkGroups + n_rows * per_split - 1) / (n_rows * per_split);
  const int tiles = p.tiles_per_split;
  split = split < tiles ? split : tiles;
  int tps = (tiles + split - 1) / split;
  split = (tiles + tps - 1) / tps;
  split = split < kMergeSplitLimit ? split : kMergeSplitLimit;
  tps = (tiles + split - 1) / split;
  if (split <= 1 && !quarters) return p;
  p.n_split = split;
  p.tiles_per_split = tps;
  p.quarters = quarters ? 1 : 0;
  // counters, partial O, and the partial maxima and sums (one copy per
  // channel quarter)
  p.bytes = kAttnCounterBytes + (size_t)n_rows * split * n_heads * 512 * sizeof(float) +
            (size_t)n_rows * split * (quarters ? 4 : 1) * n_heads * 2 * sizeof(float);
  return p;
}

hipError_t launch_attention(const AttnArgs &args, int32_t n_heads, int32_t n_rows, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  // 16- and 32-head layers: attn_kernel, 16 heads per work-group; 64-head
  // layers: the 64-head kernel, one work-group per row (or range).  Rows
  // split by key ranges are merged by attn_merge_kernel, quarter splits by
  // their own work-groups.
  AttnArgs a = args;
  a.n_heads = n_heads;
  a.n_hgroups = n_heads == 64 ? 1 : n_heads / kKsHeads;
  a.n_rows = n_rows;
  const int64_t row_sets = (n_rows + 7) / 8;
  hipError_t e;
  if (n_heads == 64) {
    e = launch_attention_h64(a, (int64_t)n_rows * a.n_split, stream);
  } else if (a.quarters) {
    const int64_t blocks = row_sets * 8 * a.n_split * a.n_hgroups * 4;
    attn_kernel<kModeQuarters><<<dim3((unsigned)blocks), kAttnThreads, 0, stream>>>(a);
    return hipGetLastError();
  } else {
    const int64_t rs = (int64_t)n_rows * a.n_split;
    const int64_t blocks = a.n_hgroups == 1 ? rs : ((rs + 7) / 8) * 8 * a.n_hgroups;
    if (a.n_split > 1)
      attn_kernel<kModeRanges><<<dim3((unsigned)blocks), kAttnThreads, 0, stream>>>(a);
    else
      attn_kernel<kModeRows><<<dim3((unsigned)blocks), kAttnThreads, 0, stream>>>(a);
    e = hipGetLastError();
  }
  if (e != hipSuccess || a.n_split <= 1) return e;
  attn_merge_kernel<<<dim3((unsigned)(n_rows * n_heads / 2)), 256, 0, stream>>>(a, n_heads);
  return hipGetLastError();
}

}  // namespace csa2
