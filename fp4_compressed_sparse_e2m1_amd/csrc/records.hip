// Cache records: an entry's 356 stored bytes (the 288-B latent -- 256 B of
// E2M1 codes and 32 B of E4M3 scales -- then the 68-B indexer key -- 64 B of
// codes and 4 B of scales) as one contiguous record [P3 "레이어 40개 가운데
// 4개만 전역 캐시를 만듭니다": 356 B per entry, 890 B per token], so a range
// of a sequence's entries can leave the GPU and come back byte for byte.
//
// One thread per 4-byte word: a record is 89 words (64 + 8 + 16 + 1), every
// plane row is a whole number of words, and consecutive threads write (or
// read) consecutive record words; the grid is bounded and strides over
// longer ranges.
#include "device.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kRecordWords = 89;
constexpr int kRecordThreads = 256;

template <bool TO_RECORDS>
__global__ void __launch_bounds__(kRecordThreads)
records_kernel(uint32_t *kv_codes, uint32_t *kv_scales, uint32_t *ik_codes, uint32_t *ik_scales,
               int64_t plane_row0, int64_t count, uint32_t *records) {
  for (int64_t t = (int64_t)blockIdx.x * kRecordThreads + threadIdx.x; t < count * kRecordWords;
       t += (int64_t)gridDim.x * kRecordThreads) {
    const int64_t e = t / kRecordWords;
    const int w = (int)(t - e * kRecordWords);
    const int64_t row = plane_row0 + e;
    uint32_t *p;
    if (w < 64)
      p = kv_codes + row * 64 + w;
    else if (w < 72)
      p = kv_scales + row * 8 + (w - 64);
    else if (w < 88)
      p = ik_codes + row * 16 + (w - 72);
    else
      p = ik_scales + row;
    if (TO_RECORDS)
      records[t] = *p;
    else
      *p = records[t];
  }
}

}  // namespace

hipError_t launch_records(bool to_records, uint8_t *kv_codes, uint8_t *kv_scales, uint8_t *ik_codes,
                          uint8_t *ik_scales, int64_t plane_row0, int64_t count, uint8_t *records,
                          hipStream_t stream) {
  if (count == 0) return hipSuccess;
  const dim3 grid(grid_blocks(count * kRecordWords, kRecordThreads));
  auto w32 = [](uint8_t *x) { return reinterpret_cast<uint32_t *>(x); };
  if (to_records)
    records_kernel<true><<<grid, kRecordThreads, 0, stream>>>(w32(kv_codes), w32(kv_scales), w32(ik_codes),
                                                              w32(ik_scales), plane_row0, count, w32(records));
  else
    records_kernel<false><<<grid, kRecordThreads, 0, stream>>>(w32(kv_codes), w32(kv_scales), w32(ik_codes),
                                                               w32(ik_scales), plane_row0, count, w32(records));
  return hipGetLastError();
}

}  // namespace csa2
