// S3-S4: Top-K selection over order-preserving score keys.
//
// Selection: scores are mapped to order-preserving uint32 keys (0 = no
// candidate).  A 1,024-thread work-group holds up to 16,384 keys of one row in
// registers (16 per thread; 32 per thread for rows of up to 32,768 keys that
// are selected in one level).  One LDS histogram of up to 4,096 bins over the
// first digit -- a window ending at the largest key, or the plain digit below
// the highest bit in which the keys differ -- names the bin holding the k-th
// key; the keys at or above that bin are gathered, in position order with
// their ids, into an LDS list; the threshold inside that bin is found by
// ranking the bin's keys directly when it holds at most 64, else by resolving
// the remaining bits from the list with two more digits, and the output is
// compacted from the list, ties at the threshold going to the lowest
// positions.  A generic radix path (12-bit digits, then one wave on the
// keys still in play, then a ballot-ordered compaction from registers) covers
// the cases the list cannot hold.  Rows with more keys are cut into chunks
// whose Top-k survivors feed a further level, which keeps the result exact
// because a global Top-k element is in its chunk's Top-k.

#include "device.h"
#include "internal.h"

namespace csa2 {
namespace {

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

struct Digit {
  int digit;   // bin holding the k_rem-th largest key
  int above;   // keys in higher bins
  int count;   // keys in that bin
  int total;   // keys in the whole histogram
};

// Sum of s[v] over the waves v below `wave` (lane v reads s[v]).
__device__ __forceinline__ int sum_below(const int *s, int wave, int lane) {
  const int x = lane < wave ? s[lane] : 0;
  return (int)wave_reduce((uint32_t)x, lane, [](uint32_t p, uint32_t q) { return p + q; });
}

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
    if (per == 64) {
      // 4,096 bins: sixteen 16-B reads per lane, eight in flight at once; lane l
      // starts its group at read l mod 16, so that the lanes' reads (256 B
      // apart) fall on different banks
#pragma unroll
      for (int h = 0; h < 16; h += 8) {
        uint4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[i] = *reinterpret_cast<const uint4 *>(&hist[top - 64 + 4 * ((h + i + lane) & 15)]);
#pragma unroll
        for (int i = 0; i < 8; ++i) local += (int)(v[i].x + v[i].y + v[i].z + v[i].w);
      }
    } else if (per >= 4) {
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
// One selection work-group: row r, chunk `chunk` of its keys.  COH_IN reads
// the keys and ids with device-scope loads and COH_OUT writes the level's
// outputs with device-scope stores (both written through to / read from the
// level every XCD sees): the two levels of select_levels_kernel hand their
// data over inside one launch.
template <bool FINAL, bool IDS, int KPT, bool COH_IN, bool COH_OUT>
__device__ __forceinline__ void select_run(const SelectArgs &a, int r, int chunk) {
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
  __shared__ uint32_t s_bin[64];   // the boundary bin's keys, when it holds at most 64
  __shared__ int s_nbin;

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
    if constexpr (COH_IN)
      key[j] = i < n_ld ? __hip_atomic_load(&kin[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    else
      key[j] = i < n_ld ? __builtin_nontemporal_load(&kin[i]) : 0u;   // read once
  }
  int32_t ids[IDS ? kKeys : 1];
  if (IDS) {
    const int32_t *idin = a.ids_in + (int64_t)r * a.in_stride + start;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const int i = base + 64 * j;
      if constexpr (COH_IN)
        ids[j] = i < n_ld ? __hip_atomic_load(&idin[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -1;
      else
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
  // a store of this level's intermediate output
  auto put = [](auto *p, auto v) {
    if constexpr (COH_OUT)
      __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *p = v;
  };
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
      put(kout + pos, k);
      put(iout + pos, id);
    }
  };

  // Common case: one first digit, then a list.  The first digit is either a
  // window of kSelBins bins of 2^kWinShift key units ending at the largest
  // key (when the keys spread beyond what a plain 12-bit digit resolves that
  // finely), or the plain digit of up to 12 bits below the highest bit in
  // which the keys differ.  Its histogram names the bin that holds the
  // k_eff-th largest key; every key at or above that bin goes, in position
  // order, into an LDS list (about k_eff keys plus one bin); the threshold
  // inside the bin comes from ranking its keys (at most 64 of them) or from
  // the remaining (at most 13) bits resolved block-wide from the list, and the output
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
      if (tid == 0) s_nbin = 0;
      const uint32_t lo_key = (base_bin + (uint32_t)s_digit) << shift0;
      const int n_list = s_above + s_ncand;
      const unsigned long long lt = (1ull << lane) - 1ull;
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < kKeys; ++j) cnt += __popcll(__ballot(key[j] != 0u && key[j] >= lo_key));
      if (lane == 0) s_red[wave] = cnt;
      __syncthreads();
      int off = sum_below(s_red, wave, lane);
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
      uint32_t thr;
      int k_eq;
      const int n_bin = s_ncand;   // the boundary bin's keys, all in the list
      if (n_bin >= 1 && n_bin <= 64) {
        // Few keys share the boundary bin: rank them directly.  Every thread
        // adds its list entries of that bin to s_bin (in any order: only their
        // values matter), and wave 0 takes the (k_eff - s_above)-th largest of
        // them by counting, for each, the bin's keys above it and at least it.
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (lk[q] != 0u && (lk[q] >> shift0) == (lo_key >> shift0)) s_bin[atomicAdd(&s_nbin, 1)] = lk[q];
        __syncthreads();
        if (wave == 0) {
          const int k_rem = k_eff - s_above;
          const uint32_t v = lane < n_bin ? s_bin[lane] : 0u;
          int gt = 0, ge = 0;
          for (int i = 0; i < n_bin; ++i) {
            const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)v, i);
            gt += o > v;
            ge += o >= v;
          }
          const unsigned long long hit = __ballot(lane < n_bin && gt < k_rem && ge >= k_rem);
          const int l = hit ? __ffsll((long long)hit) - 1 : 0;
          const uint32_t tv = (uint32_t)__builtin_amdgcn_readlane((int)v, l);
          const int tg = __builtin_amdgcn_readlane(gt, l);
          if (lane == 0) {
            s_thr = tv;
            s_keq = k_rem - tg;
          }
        }
        __syncthreads();
        thr = s_thr;
        k_eq = s_keq;
      } else {
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
        thr = prefix;
        k_eq = k_rem;
      }
      // ordered compaction of the list; above-threshold and tie counts
      // travel packed in one prefix sum
      int packed = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) packed += (int)(lk[q] > thr) + ((int)(lk[q] == thr) << 16);
      const int incl = wave_incl_scan(packed, lane);
      if (lane == 63) s_red[wave] = incl;
      __syncthreads();
      int run = incl - packed + sum_below(s_red, wave, lane);
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
            int off = sum_below(s_red, wave, lane);
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
    int run_gt = sum_below(s_red, wave, lane);
    int run_eq = sum_below(s_red + kSelWaves, wave, lane);
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
      put(kout + i, 0u);
      put(iout + i, -1);
    }
  }
}

template <bool FINAL, bool IDS, int KPT = kKeysPerThread>
__global__ void __launch_bounds__(kSelThreads)
select_kernel(SelectArgs a) {
  select_run<FINAL, IDS, KPT, false, false>(a, blockIdx.y, blockIdx.x);
}

// Two levels in one launch: every work-group selects the Top-k of its chunk
// (level 1, keys and ids written with device-scope stores) and counts its
// arrival in counters[r]; the last of the row's chunks to arrive sets the
// counter back to zero and runs the final level over the row's survivors
// (device-scope loads).
__global__ void __launch_bounds__(kSelThreads)
select_levels_kernel(SelectArgs a1, SelectArgs a2, uint32_t *counters) {
  __shared__ int s_last;
  const int r = blockIdx.y;
  select_run<false, false, kKeysPerThread, false, true>(a1, r, blockIdx.x);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counters + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == gridDim.x - 1;
    if (last) __hip_atomic_store(counters + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  select_run<true, true, kKeysPerThread, true, false>(a2, r, 0);
}

}  // namespace

hipError_t launch_select_levels(const SelectArgs &a1, const SelectArgs &a2, uint32_t *counters,
                                int32_t n_rows, int32_t n_chunks, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  if (n_chunks < 1 || (int64_t)n_chunks * a1.k > kSelectChunk) return hipErrorInvalidValue;
  select_levels_kernel<<<dim3((unsigned)n_chunks, (unsigned)n_rows), kSelThreads, 0, stream>>>(a1, a2, counters);
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
