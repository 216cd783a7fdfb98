// S5 + S6 for 64-head layers: sparse attention over the selected FP4
// latents with the SWA branch folded into the same softmax (or merged onto an
// earlier result), one work-group per query row for all 64 heads.
//
// [P1 "무엇과 다른가": every CSA2 mode attends with its own global Q over the
// Top-K of the main KV; P3 "레이어 40개 가운데 4개만 전역 캐시를 만듭니다": the
// main KV is a 512-channel latent shared by all heads, both key and value;
// P3 "전역 어텐션과 지역 어텐션": a 128-token sliding-window branch; P3 "4비트로
// 적어도 되는 이유": the SWA cache is FP8.]
//
// One work-group of 8 waves (two per SIMD, so each hides the other's LDS and
// matrix-core latencies) handles a row, or a split of its keys, for all 64
// heads, so each selected key is gathered and dequantised exactly once.  Keys
// come in tiles of 32 (two blocks of 16).  Wave w = 4 h2 + q:
//   A(t): gathers and dequantises (exact, f16) the channel quarter
//         [128q, 128q + 128) of key block h2 of tile t, stores it in LDS
//         (natural [key][channel] layout) and computes the partial logits
//         S^T = K Q^T over that quarter for all 64 heads (16x16x32 MFMAs, Q
//         held in registers, pre-scaled by a power of two per head and
//         quarter that brings it into f16 range exactly); the partials, scaled
//         back and times the softmax scale, go to LDS ([quarter][head][key]).
//   B(t): online softmax (base 2) of heads 8w .. 8w + 7: lane l sums the four
//         quarter partials of head 8w + l % 8 for keys 4 (l / 8) .. + 3 and
//         writes the probabilities (f16) and the head's rescale factor.  The
//         running max is raised only when a tile exceeds it by more than 2^8,
//         so most tiles leave O alone; P enters P.V in f16 and the normaliser
//         sums the same rounded values.
//   C(t): O^T[channels 64w .. 64w + 63][all heads] = alpha * O^T + V^T P^T
//         over the tile's 32 keys, the V operand read back from LDS with the
//         hardware transposed read (each eighth of the channels read once).
// The stages are software-pipelined, two work-group barriers per tile:
//     [C(t-1) + B(t)]  barrier  [A(t+1)]  barrier
// and each wave's raw gathers are issued three tiles ahead of their use.
#include "device.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 512;
constexpr float kLazyRescale = 8.0f;   // log2 units: the running max moves only past 2^8
constexpr int kKeys = 32;              // keys per tile
constexpr int kSPS = 32 + 4;           // floats per partial-logit row (one head, 32 keys + pad)
constexpr int kVS = 128 + 8;           // halves per LDS key row (a quarter's 128 channels + pad)
constexpr int kPS = 32 + 8;            // halves per P row
// scheduling-fence mask: ALU, transcendental and LDS instructions may be
// moved across the fence, global-memory instructions may not
constexpr int kAllButVmem = 0x0001 | 0x0080 | 0x0400;

// A lane's raw share of one key block (key c of block h2, the lane's 32
// channels of quarter q): the E2M1 codes in a and the key's two scale bytes
// for those channels in sc, or bytes 0..15 of the lane's 32 E4M3 bytes of an
// SWA row in a (bytes 16..31 are read one step before use).  ok (the same in
// every lane): bit s says slot s of the tile holds a key (both blocks).
// Nothing is computed from the loaded values until they are used (a use
// waits for the load).
struct RawBlock {
  uint4 a;
  uint32_t sc;
  uint32_t ok;
};

__global__ void __launch_bounds__(kThreads)
attn_h64_kernel(AttnArgs a) {
  constexpr int H = 64;
  __shared__ __attribute__((aligned(16))) float s_part[4][H][kSPS];
  __shared__ __attribute__((aligned(16))) _Float16 s_vn[2][4][kKeys * kVS];
  __shared__ __attribute__((aligned(16))) _Float16 s_p[2][H * kPS];
  __shared__ __attribute__((aligned(16))) float s_alpha[2][H];
  __shared__ float s_m[H], s_l[H];

  const int rs = blockIdx.x;
  if (rs >= a.n_rows * a.n_split) return;
  const int r = rs / a.n_split;
  const int sp = rs - r * a.n_split;
  const bool split = a.n_split > 1;
  const bool merge_in = a.merge_in && !split;   // with a split the merge kernel folds (o, lse) in
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int q = w & 3;           // channel quarter (A)
  const int h2 = w >> 2;         // key block (A)
  const int G = lane >> 4;
  const int c = lane & 15;
  const int hs = 8 * w + (lane & 7);    // softmax head (B)
  const int ks = 4 * (lane >> 3);      // its first key in the tile (B)

  constexpr int TK = kKeys;
  const int t_begin = split ? sp * a.tiles_per_split : 0;
  const int32_t *topk = a.topk ? a.topk + (int64_t)r * a.k_pos : nullptr;
  // Every step of the pipeline issues the same loads in the same order, none
  // of them conditional, so the compiler's count of loads in flight is exact
  // and each wait waits only for the load it needs (the load counter is in
  // order).  Loads for tiles outside [t_begin, t_end) read row 0 of the
  // sequence's cache (or of its SWA rows when it has no Top-K keys): never
  // used, and readable whenever the work-group has a tile at all (no gather
  // of any kind is issued otherwise).
  const int32_t *id_src = topk ? topk : a.row_seq;
  const int id_lim = topk ? a.k_pos : 1;
  // entry ids of tile T's keys c and 16 + c (the slot clamped into the row;
  // slots past n_topk are masked when the codes are gathered)
  auto load_ids = [&](int T, int32_t (&e)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int slot = T * TK + 16 * kb + c;
      e[kb] = id_src[slot < id_lim ? slot : id_lim - 1];
    }
  };
  // the ids of the first six tiles go out first: they need nothing else
  int32_t e0[2], e1[2], e2[2], n0[2], n1[2], n2[2];
  load_ids(t_begin, e0);
  load_ids(t_begin + 1, e1);
  load_ids(t_begin + 2, e2);
  load_ids(t_begin + 3, n0);
  load_ids(t_begin + 4, n1);
  load_ids(t_begin + 5, n2);
  // then Q (bf16, converted once the first gathers are out: the load counter
  // is in order, so waiting for Q does not wait for them)
  uint4 q_raw[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const uint4 *qp = reinterpret_cast<const uint4 *>(a.q + ((int64_t)r * H + 16 * hb + c) * 512 + 128 * q + 32 * G);
#pragma unroll
    for (int t = 0; t < 4; ++t) q_raw[hb][t] = qp[t];
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
  int t_end = split ? t_begin + a.tiles_per_split : n_all;
  t_end = t_end < n_all ? t_end : n_all;

  const uint8_t *kv_codes = a.kv_codes + (int64_t)seq * a.cap * 256;
  const uint8_t *kv_scales = a.kv_scales + (int64_t)seq * a.cap * 32;
  const uint8_t *swa = a.swa_kv ? a.swa_kv + ((int64_t)seq * a.swa_len) * 512 : nullptr;
  const uint8_t *dummy = n_gt > 0 ? kv_codes : swa;

  auto tile_mask = [&](bool ok0, bool ok1) {
    return ((uint32_t)__builtin_amdgcn_ballot_w64(ok0) & 0xFFFFu) |
           (((uint32_t)__builtin_amdgcn_ballot_w64(ok1) & 0xFFFFu) << 16);
  };
  // key block h2 of tile T: Top-K (T < n_gt), SWA rows (n_gt <= T < n_all)
  // or outside the work-group's range (T >= t_end: dummy loads)
  auto load_raw = [&](int T, const int32_t (&e)[2]) {
    RawBlock t;
    const bool is_g = T < n_gt && T < t_end;
    const bool is_s = T >= n_gt && T < t_end;
    bool ok[2];
    int64_t el = 0, row = 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int slot_g = T * TK + 16 * kb + c;
      const int slot_s = (T - n_gt) * TK + 16 * kb + c;
      const int64_t id = slot_g < n_g ? e[kb] : -1;
      const bool ok_g = is_g && id >= 0 && id < a.cap;
      const bool ok_s = is_s && slot_s < n_s;
      ok[kb] = ok_g || ok_s;
      if (kb == h2) {
        el = ok_g ? id : 0;
        row = s0 + (ok_s ? slot_s : 0);
      }
    }
    const uint8_t *pa = is_g ? kv_codes + el * 256 + 64 * q + 16 * G
                             : is_s ? swa + row * 512 + 128 * q + 32 * G : dummy + 64 * q + 16 * G;
    const uint8_t *ps = is_g ? kv_scales + el * 32 + 8 * q + 2 * G : pa;
    t.a = *reinterpret_cast<const uint4 *>(pa);
    t.sc = *reinterpret_cast<const uint16_t *>(ps);
    t.ok = tile_mask(ok[0], ok[1]);
    return t;
  };
  // bytes 16..31 of the lane's share of an SWA block (a dummy load for any
  // other tile)
  auto load_hi = [&](int T) {
    const bool is_s = T >= n_gt && T < t_end;
    const int slot_s = (T - n_gt) * TK + 16 * h2 + c;
    const int64_t row = s0 + ((is_s && slot_s < n_s) ? slot_s : 0);
    const uint8_t *p = is_s ? swa + row * 512 + 128 * q + 32 * G + 16 : dummy + 64 * q + 16 * G;
    return *reinterpret_cast<const uint4 *>(p);
  };

  struct Slot {
    RawBlock t;
    int32_t nid[2];
  };
  Slot sl0, sl1, sl2;
  uint4 bh;
  const bool has_tiles = t_begin < t_end;
  if (has_tiles) {
    // (the scheduling fences keep the loads in the order of need)
    __builtin_amdgcn_sched_barrier(0);
    sl0.t = load_raw(t_begin, e0);
    sl1.t = load_raw(t_begin + 1, e1);
    bh = load_hi(t_begin);
    sl2.t = load_raw(t_begin + 2, e2);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    sl0.nid[kb] = n0[kb];
    sl1.nid[kb] = n1[kb];
    sl2.nid[kb] = n2[kb];
  }

  // Q operand of the logits: qa[hb][t] = 2^k q[r][16hb + c][128q + 32G + 8t
  // .. +7] in f16 (the contraction runs over the quarter in this
  // lane-consistent order), with a power of two 2^k per head and quarter (from
  // the largest |q| of head 16hb + c in quarter q, over the four lanes that
  // hold it).  The partial logits are scaled back on the way out, together
  // with the softmax scale: sl[hb] = scale * log2(e) * 2^-k.
  f16x8 qa[4][4];
  float sl[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    u16x2 m2 = {0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) m2 = bf16x8_absmax(q_raw[hb][t], m2);
    const int k = q_prescale_exp(umax_rows(absmax_bits(m2)));
#pragma unroll
    for (int t = 0; t < 4; ++t) qa[hb][t] = bf16x8_to_f16_scaled(q_raw[hb][t], exp2i(k));
    sl[hb] = a.scale_log2 * exp2i(-k);
  }

  // O^T accumulators: acc[hb][db] lane (G, c) holds
  // O[16hb + c][64w + 16db + 4G + i]
  f32x4 acc[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (merge_in) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int64_t h = (int64_t)r * H + 16 * hb + c;
      if (a.lse[h] != -INFINITY) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[hb][db] = *reinterpret_cast<const f32x4 *>(a.o + h * 512 + 64 * w + 16 * db + 4 * G);
      }
    }
  }
  // softmax state of head hs in its eight lanes: the running max (log2
  // units) and the normaliser as per-lane partial sums, reduced at the end
  float m_run = -INFINITY, l_thr = 0.f;
  if (merge_in) {
    const float lin = a.lse[(int64_t)r * H + hs];
    if (lin != -INFINITY) {
      m_run = lin * 1.4426950408889634f;
      l_thr = lane < 8 ? 1.f : 0.f;
    }
    // Wait for the earlier result here: otherwise the first use of the
    // accumulators inside the loop would carry a wait for every load in flight
    // (the count cannot tell these loads apart from the gathers), on every pass.
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
  }

  uint32_t mask = 0;        // present keys of the tile whose logits are in s_part

  // ---- A(T): dequantise key block h2 and quarter q of tile T, store it,
  // partial logits.  An absent Top-K key gets scale 0 (every E2M1 code is
  // finite, so its values become 0); an absent SWA row is zeroed before
  // decoding (E4M3 has NaN codes): no stale byte pattern reaches P.V.
  auto stage_a = [&](int T, const RawBlock &t, const uint4 &hi_raw) {
    f16x8 kf[4];
    const bool ok = (t.ok >> (16 * h2 + c)) & 1u;
    if (T < n_gt || T >= t_end) {      // (a tile past t_end is all absent: zeros)
      const _Float16 sa = ok ? e4m3_to_f16(t.sc & 0xFFu) : (_Float16)0.f;
      const _Float16 sb = ok ? e4m3_to_f16((t.sc >> 8) & 0xFFu) : (_Float16)0.f;
      const f16x8 va = f16x8{sa, sa, sa, sa, sa, sa, sa, sa};
      const f16x8 vb = f16x8{sb, sb, sb, sb, sb, sb, sb, sb};
      kf[0] = e2m1x8_to_f16(t.a.x) * va;
      kf[1] = e2m1x8_to_f16(t.a.y) * va;
      kf[2] = e2m1x8_to_f16(t.a.z) * vb;
      kf[3] = e2m1x8_to_f16(t.a.w) * vb;
    } else {
      const uint4 lo = ok ? t.a : uint4{0u, 0u, 0u, 0u};
      const uint4 hi = ok ? hi_raw : uint4{0u, 0u, 0u, 0u};
      kf[0] = e4m3x8_to_f16(lo.x, lo.y);
      kf[1] = e4m3x8_to_f16(lo.z, lo.w);
      kf[2] = e4m3x8_to_f16(hi.x, hi.y);
      kf[3] = e4m3x8_to_f16(hi.z, hi.w);
    }
    mask = t.ok;
    _Float16 *vn = &s_vn[T & 1][q][(16 * h2 + c) * kVS + 32 * G];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f16x8 *>(vn + 8 * i) = kf[i];
    // lane (G, c): S^T[key 16h2 + 4G + i][head 16hb + c] over quarter q
    f32x4 sacc[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) sacc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) sacc[hb] = mfma16x16x32(kf[i], qa[hb][i], sacc[hb]);
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
      *reinterpret_cast<f32x4 *>(&s_part[q][16 * hb + c][16 * h2 + 4 * G]) = sacc[hb] * sl[hb];
  };

  // ---- B(T): online softmax of head hs over keys ks .. ks + 3 of tile T
  auto stage_b = [&](int T) {
    const f32x4 x = (*reinterpret_cast<const f32x4 *>(&s_part[0][hs][ks]) +
                     *reinterpret_cast<const f32x4 *>(&s_part[1][hs][ks])) +
                    (*reinterpret_cast<const f32x4 *>(&s_part[2][hs][ks]) +
                     *reinterpret_cast<const f32x4 *>(&s_part[3][hs][ks]));
    float sv[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = ((mask >> (ks + j)) & 1u) ? x[j] : -INFINITY;
      tmax = fmaxf(tmax, sv[j]);
    }
    // the eight lanes of head hs: l ^ 8, l ^ 16, l ^ 32
    tmax = fmaxf(tmax, dpp<kDppRowRor8>(tmax));
    tmax = fmaxf(tmax, swap_rows16(tmax));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(tmax), __float_as_int(tmax), false, false);
      tmax = fmaxf(tmax, __int_as_float(lane < 32 ? sw[1] : sw[0]));
    }
    const float m_new = (m_run == -INFINITY || tmax > m_run + kLazyRescale) ? fmaxf(tmax, m_run) : m_run;
    // the hardware exp2 (no denormal-range fix-up): arguments are <= 2^8, and
    // results below 2^-126 are negligible weights (f16 drops them too)
    const float alpha = (m_run == -INFINITY || m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;     // an all-absent tile: sv = -inf gives 0
    f16x4 ph;
#pragma unroll
    for (int j = 0; j < 4; ++j) ph[j] = (_Float16)__builtin_amdgcn_exp2f(sv[j] - m_sub);
    float psum = __builtin_amdgcn_fdot2(f16x2{ph[0], ph[1]}, f16x2{1, 1}, 0.f, false);
    psum = __builtin_amdgcn_fdot2(f16x2{ph[2], ph[3]}, f16x2{1, 1}, psum, false);
    l_thr = l_thr * alpha + psum;
    m_run = m_new;
    *reinterpret_cast<f16x4 *>(&s_p[T & 1][hs * kPS + ks]) = ph;
    s_alpha[T & 1][hs] = alpha;          // the eight lanes of the head write the same value
  };

  // ---- C(T): O^T[channels 64w .. 64w + 63][all heads] = alpha * O^T + V^T P^T
  // over the tile's 32 keys.  The rescale (rare) comes first, on its own.
  auto rescale = [&](int T) {
    float al[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) al[hb] = s_alpha[T & 1][16 * hb + c];
    if (__builtin_amdgcn_ballot_w64(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f)) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[hb][db] *= al[hb];
    }
  };
  auto stage_c = [&](int T) {
    // B operand: P^T[keys 8G .. 8G + 7][head 16hb + c]
    f16x8 pb[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) pb[hb] = *reinterpret_cast<const f16x8 *>(&s_p[T & 1][(16 * hb + c) * kPS + 8 * G]);
    // A operand of channel block db: V^T[channel 64w + 16db + c][keys 8G .. 8G + 7],
    // read transposed from rows 8G + 4h + c/4 (h = 0, 1) of quarter w / 2,
    // channels 64 (w % 2) + 16db + 4 (c % 4)
    const _Float16 *r0 = &s_vn[T & 1][w >> 1][(8 * G + (c >> 2)) * kVS + 64 * (w & 1) + 4 * (c & 3)];
    const _Float16 *r1 = r0 + 4 * kVS;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const f16x4 lo = lds_read_tr16(r0 + 16 * db);
      const f16x4 hi = lds_read_tr16(r1 + 16 * db);
      const f16x8 va = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) acc[hb][db] = mfma16x16x32(va, pb[hb], acc[hb][db]);
    }
  };

  // Pipeline.  Raw blocks live in three register slots, tile t_begin + j in
  // slot j mod 3, each with the entry ids of the tile three later.  A(T)
  // empties the slot of tile T, which then receives tile T + 3 and the ids of
  // tile T + 6, so every gather is issued three steps before its use (the
  // upper halves of an SWA block's rows one step before, and ahead of that
  // step's gathers).
  //   A(t0) barrier B(t0) barrier A(t0 + 1) barrier
  //   then per tile T > t0:  [C(T - 1) + B(T)] barrier [A(T + 1)] barrier
  //   and C of the last tile.
  // The last step's A works on a tile past t_end (all absent, into buffers no
  // later stage reads), which keeps every step alike.  The loop is unrolled
  // by three so every slot is a fixed set of registers.
  if (has_tiles) {
    // A(T + 1) from slot nxt, then the loads that refill it
    // (the fences let arithmetic and LDS work move across them, not loads)
    auto advance = [&](int T, Slot &nxt) {
      stage_a(T + 1, nxt.t, bh);
      __builtin_amdgcn_sched_barrier(kAllButVmem);
      bh = load_hi(T + 2);
      __builtin_amdgcn_sched_barrier(kAllButVmem);
      nxt.t = load_raw(T + 4, nxt.nid);
      __builtin_amdgcn_sched_barrier(kAllButVmem);
      load_ids(T + 7, nxt.nid);
      __builtin_amdgcn_sched_barrier(kAllButVmem);
    };
    advance(t_begin - 1, sl0);
    __syncthreads();
    stage_b(t_begin);
    __syncthreads();
    advance(t_begin, sl1);
    __syncthreads();
    auto step = [&](int T, Slot &nxt) {
      rescale(T - 1);
      stage_c(T - 1);
      stage_b(T);
      __syncthreads();
      advance(T, nxt);
      __syncthreads();
    };
    for (int T = t_begin + 1; T < t_end; T += 3) {
      step(T, sl2);
      if (T + 1 >= t_end) break;
      step(T + 1, sl0);
      if (T + 2 >= t_end) break;
      step(T + 2, sl1);
    }
    rescale(t_end - 1);
    stage_c(t_end - 1);
  }

  // normaliser of head hs: its eight lanes
  {
    float l = l_thr + dpp<kDppRowRor8>(l_thr);
    l += swap_rows16(l);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(l), __float_as_int(l), false, false);
    l += __int_as_float(lane < 32 ? sw[1] : sw[0]);
    if (lane < 8) {
      s_m[hs] = m_run;
      s_l[hs] = l;
    }
  }
  __syncthreads();
  if (split) {
    // unnormalised partial: O, running max (log2 units) and sum per head
    const int64_t part = (int64_t)r * a.n_split + sp;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      float *prow = a.part_o + (part * H + 16 * hb + c) * 512 + 64 * w + 4 * G;
#pragma unroll
      for (int db = 0; db < 4; ++db) *reinterpret_cast<f32x4 *>(prow + 16 * db) = acc[hb][db];
    }
    if (tid < H) {
      a.part_ml[(part * H + tid) * 2] = s_m[tid];
      a.part_ml[(part * H + tid) * 2 + 1] = s_l[tid];
    }
    return;
  }
  // normalise and store
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int h = 16 * hb + c;
    const float l = s_l[h];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *orow = a.o + ((int64_t)r * H + h) * 512 + 64 * w + 4 * G;
#pragma unroll
    for (int db = 0; db < 4; ++db) *reinterpret_cast<f32x4 *>(orow + 16 * db) = acc[hb][db] * inv;
  }
  if (tid < H) {
    const float l = s_l[tid];
    a.lse[(int64_t)r * H + tid] = l > 0.f ? (s_m[tid] + log2f(l)) * 0.6931471805599453f : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attention_h64(const AttnArgs &a, int64_t blocks, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  attn_h64_kernel<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace csa2
