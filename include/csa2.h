/*
 * libcsa2 -- CSA2 (Compressed Sparse Attention 2) hot path for AMD MI355X
 * (gfx950), C ABI.
 *
 * The library implements the global-attention path of a CSA2 layer as the
 * pages describe it:
 *   - P1: onedev.kr digest "KV 캐시를 토큰당 890바이트로 압축한 552B 멀티모달
 *     MoE, DeepSeek-V4.1-Flash", section "무엇과 다른가" (how it differs):
 *     the Full / Reindex / Reuse layer modes, the FP4 global KV cache and the
 *     hierarchical sparse indexer;
 *   - P3: genexis.ai explainer "100만 토큰을 0.9GB에, 딥시크 V4.1 논문이 KV
 *     캐시를 줄인 방법", sections "레이어 40개 가운데 4개만 전역 캐시를
 *     만듭니다" (entry layout, 2,048 blocks of 8, Top-512), "4비트로 적어도
 *     되는 이유" (FP4 with one 8-bit scale per 16 values, FP8 SWA cache) and
 *     "전역 어텐션과 지역 어텐션" (the 128-token SWA branch).
 *
 * A layer in each mode is a sequence of calls:
 *   Full    = csa2_cache_append (its new entries, both planes; or
 *             csa2_quantize_fp4 per plane)
 *             + csa2_index_full + csa2_sparse_attn [+ csa2_swa_merge];
 *             or, one new entry per sequence, csa2_index_scan_append +
 *             csa2_index_pool + csa2_sparse_attn [+ csa2_swa_merge]
 *   Reindex = csa2_index_reindex (on the Full layer's cache and pool)
 *             + csa2_sparse_attn [+ csa2_swa_merge]
 *   Reuse   = csa2_sparse_attn [+ csa2_swa_merge] on the inherited Top-K.
 * csa2_sparse_attn can fold the SWA branch into the same softmax (pass a
 * csa2_swa); csa2_swa_merge adds it to an earlier global-only result.
 *
 * Conventions for every call:
 *   - Every array argument is a DEVICE pointer owned by the caller (for
 *     example a torch tensor's storage); struct arguments are host pointers
 *     to structs that hold device pointers.  The library allocates no memory
 *     and keeps no pointer after it returns; scratch memory is the caller's
 *     `workspace`, sized by csa2_workspace_size().  The one exception is
 *     csa2_index_full_noalloc, whose scratch is a static per-device array
 *     (its only global state is that array's address per device).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued on it; CSA2_OK means "validated and enqueued".  Device faults
 *     show up at the caller's next synchronisation.
 *   - Arguments are validated on the host before anything is launched; on a
 *     validation status (CSA2_E_INVALID_ARG, CSA2_E_UNSUPPORTED,
 *     CSA2_E_WORKSPACE) nothing has been written or launched.  CSA2_E_HIP
 *     reports a failed launch; a call that enqueues several kernels may have
 *     enqueued the ones before the failing one.
 *   - Device-side counts (row_nvis, n_pool, n_topk, SWA ends) are clamped to
 *     the host-side maxima; out-of-range sequence ids make a row empty;
 *     entry ids outside [0, cap) are skipped.  These guards keep every access
 *     in bounds; such inputs are still outside the contract.
 *   - Results are deterministic: fixed reduction orders, Top-K lists sorted
 *     ascending.
 *   - NaN or infinite inputs are outside the contract.
 *   - Q and q_idx may hold any finite bf16 values.  Each head enters the f16
 *     contractions times a power of two 2^k that puts its largest |q| in
 *     [2^15, 2^16), and the f32 results are scaled back by 2^-k, so every
 *     value at least 2^-29 times the head's largest converts exactly (smaller
 *     ones round on the f16 subnormal grid; k is capped at 100, so a head
 *     whose largest |q| is below 2^-85 keeps a smaller factor).  The scaled
 *     logits (scale * q.k) and the index scores must be finite in fp32.
 *
 * Data layout in HBM (one plane per field, struct-of-arrays):
 *   kv_codes  [n_seq][cap][256] uint8   main latent, 512 E2M1 codes
 *   kv_scales [n_seq][cap][32]  uint8   main latent, one E4M3FN scale per 16 ch
 *   ik_codes  [n_seq][cap][64]  uint8   indexer key, 128 E2M1 codes
 *   ik_scales [n_seq][cap][4]   uint8   indexer key, one E4M3FN scale per 32 ch
 * 256 + 32 + 64 + 4 = 356 bytes per entry (P3, "레이어 40개 가운데 4개만...").
 * E2M1 codes: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa (OCP
 * MX); channel 2k is the low nibble of byte k, channel 2k+1 the high nibble.
 * Scales: OCP E4M3FN (bias 7, max 448), always >= 0.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSA2_OK = 0,
    CSA2_E_INVALID_ARG = 1,  /* null pointer, negative or inconsistent size */
    CSA2_E_UNSUPPORTED = 2,  /* valid but outside what the kernels implement */
    CSA2_E_WORKSPACE = 3,    /* workspace missing or smaller than required */
    CSA2_E_HIP = 4           /* a HIP runtime call or launch failed */
} csa2_status;

/* Operation ids for csa2_workspace_size(). */
enum { CSA2_OP_INDEX_FULL = 1, CSA2_OP_INDEX_REINDEX = 2, CSA2_OP_INDEX_POOL = 3 };

/* Global (compressed) KV cache of one Full layer: four device planes, laid
 * out as in the header comment.  Entry j of sequence s lives at row
 * s * cap + j of every plane. */
typedef struct {
    uint8_t *kv_codes;
    uint8_t *kv_scales;
    uint8_t *ik_codes;
    uint8_t *ik_scales;
    int64_t cap;    /* entries per sequence (>= 1) */
    int32_t n_seq;  /* sequences (>= 1) */
} csa2_cache;

/* Sliding-window (SWA) branch of one layer [P3 "전역 어텐션과 지역 어텐션":
 * the local branch sees the last 128 tokens; "4비트로 적어도 되는 이유":
 * the SWA cache stays 8-bit].
 *   kv      : device, OCP E4M3FN bytes [n_seq][len][512], unit scale; each row
 *             is one token's 512-d SWA key, which is also its value.
 *   len     : rows per sequence (>= 0).
 *   row_end : device int32 [n_rows]: for query row r the window is rows
 *             [max(0, end - window), end) of sequence row_seq[r], with end
 *             clamped to [0, len].
 *   window  : window length in rows, 0..1024 (128 in the pages' model). */
typedef struct {
    const uint8_t *kv;
    int64_t len;
    const int32_t *row_end;
    int32_t window;
} csa2_swa;

/* S1 -- FP4 quantise / append [P3 "4비트로 적어도 되는 이유": NVFP4 without
 * the second-level global scale, one 8-bit scale per 16 channels; P3
 * "레이어 40개 가운데 4개만..." for the 512-ch latent (288 B) and the 128-d
 * indexer key (68 B)].
 * For each row r < n of x (fp32 [n][dim]) and each group of `group`
 * channels: amax = max |x|; scale = E4M3FN round-to-nearest-even of amax/6
 * (saturating at 448); each value's code = E2M1 round-to-nearest-even of
 * |x|/scale (saturating at 6; 0 if the scale is 0), sign bit = (x < 0).
 * Row r is written to plane row dst_rows[r] (device int64 [n]) or to row r
 * when dst_rows is NULL:
 *   codes  + dst * (dim/2)       (dim/2 bytes)
 *   scales + dst * (dim/group)   (dim/group bytes).
 * The planes hold plane_rows rows; rows whose dst lies outside
 * [0, plane_rows) are skipped.
 * To append entry j of sequence s to a csa2_cache, use dst = s * cap + j with
 * (dim, group) = (512, 16) on kv_* and (128, 32) on ik_* and
 * plane_rows = n_seq * cap.
 * Requires n >= 0, group in {16, 32}, dim % group == 0, 32 <= dim <= 4096,
 * plane_rows >= 0 (and plane_rows >= n when dst_rows is NULL). */
csa2_status csa2_quantize_fp4(const float *x, int64_t n, int32_t dim, int32_t group,
                              const int64_t *dst_rows, uint8_t *codes, uint8_t *scales,
                              int64_t plane_rows, void *stream);

/* S1 -- append new entries to a cache, both planes in one launch [the same
 * encoding as csa2_quantize_fp4, P3 "4비트로 적어도 되는 이유"; the entry is the
 * 288-B latent plus the 68-B indexer key, P3 "레이어 40개 가운데 4개만..."].
 * For each i < n: latent row i (fp32 [n][512]) is encoded with group 16 into
 * kv_codes / kv_scales row dst_rows[i], and indexer-key row i (fp32
 * [n][128]) with group 32 into ik_codes / ik_scales row dst_rows[i]; the
 * bytes written equal those of csa2_quantize_fp4 on each plane.  dst_rows is
 * a device int64 [n] of plane rows (seq * cap + position); rows outside
 * [0, n_seq * cap) are skipped.  latent and ikey must be 16-B aligned.
 * Requires n >= 0 and a cache with all four planes. */
csa2_status csa2_cache_append(const csa2_cache *cache, const float *latent, const float *ikey,
                              int64_t n, const int64_t *dst_rows, void *stream);

/* Cache records -- export and import of stored entries, byte for byte
 * [P3 "레이어 40개 가운데 4개만 전역 캐시를 만듭니다": a stored entry is
 * 356 B (the 288-B latent and the 68-B indexer key), 890 B per token at 2.5
 * entries; the pages keep such caches beyond the GPU for later reuse].
 * A record is one entry's 356 bytes in the order of the planes:
 *   [0, 256)   kv_codes   [256, 288) kv_scales
 *   [288, 352) ik_codes   [352, 356) ik_scales
 * and entries first .. first + count - 1 of sequence seq form count
 * consecutive records (count * 356 bytes) in `records`, a DEVICE buffer
 * owned by the caller (copy it to or from host memory with the caller's own
 * stream).  csa2_cache_export writes the records from the cache's planes;
 * csa2_cache_import writes the planes from the records (the entries' previous
 * bytes are replaced).  Both are plain byte copies: an exported and
 * re-imported range is bit-identical.
 * Requires a cache with all four planes (each 4-B aligned), 0 <= seq < n_seq,
 * first >= 0, count >= 0, first + count <= cap, and a 4-B aligned `records`
 * (may be NULL when count = 0). */
#define CSA2_RECORD_BYTES 356
csa2_status csa2_cache_export(const csa2_cache *cache, int32_t seq, int64_t first, int64_t count,
                              uint8_t *records, void *stream);
csa2_status csa2_cache_import(const csa2_cache *cache, int32_t seq, int64_t first, int64_t count,
                              const uint8_t *records, void *stream);

/* Scratch bytes that csa2_index_full (op CSA2_OP_INDEX_FULL),
 * csa2_index_reindex (op CSA2_OP_INDEX_REINDEX) or csa2_index_pool (op
 * CSA2_OP_INDEX_POOL) needs for these sizes; k_blocks = 0 selects flat mode
 * (not valid for CSA2_OP_INDEX_POOL).  Flat mode scores and selects its rows
 * in passes of at most 256 MiB of scratch, so its size stays below that
 * bound (or one row's own need, 4 B per visible entry plus selection
 * scratch) however many rows a call has.  In block mode the workspace of
 * csa2_index_full and csa2_index_pool begins with arrival counters (4 B per
 * row) for a block selection that runs its two levels in one launch: zero-fill
 * the workspace before its first use; every call that completes leaves the
 * counters at zero again, so one workspace serves any number of calls (calls
 * that share it must not overlap in time).  Returns 0 for invalid arguments. */
size_t csa2_workspace_size(int32_t op, int32_t n_rows, int32_t max_nvis, int32_t k_blocks,
                           int32_t k_pos);

/* S2-S4 -- Full-mode indexer [P1 "무엇과 다른가": a Full layer computes its
 * own indexer Q and selects Top-K afresh; the first decoder Full layer scans
 * the whole causally visible range and keeps up to 2,048 blocks of 8
 * positions as the candidate pool; P3 "레이어 40개 가운데 4개만..."].
 * For each query row r (n_rows rows):
 *   seq = row_seq[r], n_vis = min(row_nvis[r], max_nvis) visible entries
 *   0..n_vis-1 of that sequence;
 *   score(j) = sum_h w[r][h] * max(0, sum_c q_idx[r][h][c] * k_hat_j[c]),
 *   h < 8, c < 128, k_hat = decoded indexer key (fp32 accumulation);
 *   block mode (k_blocks > 0): block b = entries [8b, 8b+8) ∩ visible,
 *   block score = max of its entry scores; the best min(k_blocks, #blocks)
 *   blocks (score descending, ties to the lower block id) form the pool,
 *   written ascending to pool_blocks[r][0..k_blocks) (-1 padded) with the
 *   count in n_pool[r]; the pool's entries are re-scored with the same
 *   query and the best min(k_pos, |pool entries|) positions are kept;
 *   flat mode (k_blocks == 0, used for encoder prefill): the best k_pos of
 *   all visible entries are kept, pool outputs are not written (may be NULL);
 *   topk[r][0..k_pos) receives the kept entry ids ascending, -1 padded;
 *   n_topk[r] the count.
 * Types: q_idx bf16 bits [n_rows][8][128]; w fp32 [n_rows][8]; row_seq,
 * row_nvis int32 [n_rows]; outputs int32.
 * Several rows may name the same sequence (prefill query tokens, or several
 * decode queries of one sequence checked together); when the rows are at
 * least twice the cache's sequences, the scoring reads each indexer key once
 * for up to 8 consecutive rows of one sequence, so such rows are best laid
 * out sequence by sequence.  Results do not depend on the layout.
 * Requires 1 <= n_rows, 0 <= max_nvis <= cap, max_nvis < 2^31 - 8,
 * 0 <= k_blocks <= 4096, 1 <= k_pos <= 4096, and workspace_bytes >=
 * csa2_workspace_size(CSA2_OP_INDEX_FULL, n_rows, max_nvis, k_blocks, k_pos). */
csa2_status csa2_index_full(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                            const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                            int32_t max_nvis, int32_t k_blocks, int32_t k_pos,
                            int32_t *pool_blocks, int32_t *n_pool, int32_t *topk,
                            int32_t *n_topk, void *workspace, size_t workspace_bytes,
                            void *stream);

/* csa2_index_full without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments (minus the workspace),
 * results and rules as csa2_index_full.  The scratch memory is a static
 * array of CSA2_NOALLOC_SCRATCH_BYTES inside the library, one per device,
 * held until the process ends; the current device's array is used (the
 * stream must belong to the current device), and its address is looked up
 * once per device on the first call there.  The call allocates nothing.
 * The array starts zeroed and keeps the last call's contents; a call relies
 * only on the block selection's arrival counters being zero, which every
 * completed call leaves them (see csa2_workspace_size).  Calls that overlap
 * on one device (on different streams, or from different
 * threads before the earlier one's kernels finished) share the array and
 * race: order them on one stream.
 * Returns CSA2_E_UNSUPPORTED when these sizes need more scratch than the
 * array holds, i.e. csa2_workspace_size(CSA2_OP_INDEX_FULL, n_rows,
 * max_nvis, k_blocks, k_pos) > CSA2_NOALLOC_SCRATCH_BYTES (16 MiB: enough
 * for, e.g., 16 decode rows at 2^20 visible entries with 2,048 blocks and
 * Top-512; flat mode needs 4 B per row and visible entry). */
#define CSA2_NOALLOC_SCRATCH_BYTES (16u << 20)
csa2_status csa2_index_full_noalloc(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                                    const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                                    int32_t max_nvis, int32_t k_blocks, int32_t k_pos,
                                    int32_t *pool_blocks, int32_t *n_pool, int32_t *topk,
                                    int32_t *n_topk, void *stream);

/* S2 alone -- the scan stage of csa2_index_full in block mode, for callers
 * that schedule or time the context-proportional scan separately.  For each
 * row, writes the score of every visible block (as csa2_index_full defines
 * it) to block_keys[r][b], b < ceil(n_vis / 8), as an order-preserving
 * uint32 image of the fp32 score: key = bits ^ 0x80000000 for scores >= +0,
 * key = ~bits for negative scores (a larger key means a larger score).
 * block_keys: device uint32 [n_rows][ceil(max_nvis / 8)] (row stride
 * ceil(max_nvis / 8), at least 1); slots past a row's block count are left
 * untouched.  Same argument rules as csa2_index_full. */
csa2_status csa2_index_scan(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                            const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                            int32_t max_nvis, uint32_t *block_keys, void *stream);

/* S1 + S2 in one launch -- a decode step's append of each row's new entry
 * followed by the block-mode scan of csa2_index_scan [P3 "레이어 40개 가운데
 * 4개만...": each Full layer stores the step's new entry in both planes and
 * then scores every visible entry, the new one included].  For each row r
 * with 0 <= row_seq[r] < n_seq and n = min(row_nvis[r], max_nvis) >= 1,
 * latent row r (fp32 [n_rows][512]) and indexer-key row r (fp32
 * [n_rows][128]) are encoded into plane row row_seq[r] * cap + n - 1 with the
 * bytes csa2_cache_append writes there; then block_keys is written exactly as
 * csa2_index_scan writes it on the updated cache.  Other rows append nothing.
 * Precondition: the rows name distinct sequences (one new entry per
 * sequence, as in a decode step); rows sharing a sequence give unspecified
 * plane bytes and keys for it (every access stays inside the planes).  A
 * launch reads no entry another row writes, so no ordering beyond the stream
 * is needed.  latent and ikey must be 16-B aligned; the cache needs all four
 * planes; n_rows > n_seq is rejected (CSA2_E_INVALID_ARG), other rules as
 * csa2_index_scan. */
csa2_status csa2_index_scan_append(const csa2_cache *cache, const float *latent, const float *ikey,
                                   const uint16_t *q_idx, const float *w, const int32_t *row_seq,
                                   const int32_t *row_nvis, int32_t n_rows, int32_t max_nvis,
                                   uint32_t *block_keys, void *stream);

/* S3 + S4 on a finished scan -- the remaining stages of csa2_index_full in
 * block mode: block Top-k_blocks from block_keys (as written by
 * csa2_index_scan for the same rows), the pool, its re-scoring with the same
 * q_idx and w, and the Top-k_pos positions.  Outputs and limits as
 * csa2_index_full with k_blocks >= 1; workspace sized with
 * CSA2_OP_INDEX_POOL.  csa2_index_scan followed by csa2_index_pool gives the
 * same results as csa2_index_full. */
csa2_status csa2_index_pool(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                            const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                            int32_t max_nvis, const uint32_t *block_keys, int32_t k_blocks,
                            int32_t k_pos, int32_t *pool_blocks, int32_t *n_pool, int32_t *topk,
                            int32_t *n_topk, void *workspace, size_t workspace_bytes,
                            void *stream);

/* S4 -- Reindex-mode indexer [P1 "무엇과 다른가": a Reindex layer reuses
 * the earlier layer's main KV and indexer K and re-scores with its own
 * indexer Q; P3 "레이어 40개 가운데 4개만...": it picks 512 positions inside
 * the candidate pool, so a query never scores more than 16,384 positions].
 * Scores, per row, the entries of the given pool (pool_blocks[r][0..n_pool[r])
 * ascending, as csa2_index_full writes them; entries at or beyond n_vis are
 * skipped) with this layer's q_idx and w, and keeps the best
 * min(k_pos, #candidates) as in csa2_index_full.  pool_blocks == NULL selects
 * flat mode (all visible entries are candidates; n_pool and k_blocks unused).
 * Same types and limits as csa2_index_full. */
csa2_status csa2_index_reindex(const csa2_cache *cache, const uint16_t *q_idx, const float *w,
                               const int32_t *row_seq, const int32_t *row_nvis, int32_t n_rows,
                               int32_t max_nvis, const int32_t *pool_blocks,
                               const int32_t *n_pool, int32_t k_blocks, int32_t k_pos,
                               int32_t *topk, int32_t *n_topk, void *workspace,
                               size_t workspace_bytes, void *stream);

/* S5 (+S6) -- sparse attention over the selected FP4 latents [P1
 * "무엇과 다른가": all three modes attend with their own global Q over the
 * (possibly inherited) Top-K of the main KV; P3 "전역 어텐션과 지역 어텐션"].
 * For each row r and head h < n_heads: the keys are the decoded 512-d main
 * latents c_hat_j of j = topk[r][i], i < min(n_topk[r], k_pos), j >= 0 (the
 * latent is both key and value, shared by all heads);
 * logits = scale * (q[r][h] . c_hat_j); o[r][h] = softmax-weighted sum of
 * the c_hat_j; lse[r][h] = natural-log log-sum-exp of the logits.
 * With swa != NULL the window rows of the SWA branch join the same softmax
 * (the result equals csa2_sparse_attn without swa followed by
 * csa2_swa_merge).  With no keys at all, o = 0 and lse = -inf.
 * Types: q bf16 bits [n_rows][n_heads][512]; topk int32 [n_rows][k_pos];
 * n_topk int32 [n_rows]; o fp32 [n_rows][n_heads][512]; lse fp32
 * [n_rows][n_heads]; q and o 16-B aligned.  Requires n_heads in {16, 32, 64}, n_rows >= 0,
 * 1 <= k_pos <= 65536, scale finite.
 * workspace (optional, 256-B aligned, csa2_attn_workspace_size bytes): with
 * it, a small batch spreads each row's keys over several work-groups and
 * merges their partial results; with workspace == NULL every row runs in one
 * work-group (same results up to fp32 rounding order, slower for few rows).
 * The workspace must be zero-filled before it is first passed to this
 * function or to csa2_swa_merge: its first 16 KiB hold arrival counters,
 * which every call that completes leaves at zero again (the rest is scratch),
 * so one zero-filled workspace serves any number of calls.  Calls that share
 * a workspace must not overlap in time (they would share the counters). */
csa2_status csa2_sparse_attn(const csa2_cache *cache, const uint16_t *q, int32_t n_heads,
                             const int32_t *row_seq, int32_t n_rows, const int32_t *topk,
                             const int32_t *n_topk, int32_t k_pos, float scale,
                             const csa2_swa *swa, float *o, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream);

/* S6 -- SWA branch and log-sum-exp merge [P3 "전역 어텐션과 지역 어텐션";
 * the merge is the softmax over the union of the two key sets].
 * On entry (o, lse) hold a result over some key set G (for example
 * csa2_sparse_attn without swa; lse = -inf means G is empty).  Computes the
 * attention of the same q over the SWA window rows S and leaves in (o, lse)
 * the result over G ∪ S:
 *   m = max(lse_G, lse_S); o = (e^(lse_G-m) o_G + e^(lse_S-m) o_S) /
 *   (e^(lse_G-m) + e^(lse_S-m)); lse = m + log(e^(lse_G-m) + e^(lse_S-m)).
 * Same types, limits and workspace rule as csa2_sparse_attn; swa must not be
 * NULL. */
csa2_status csa2_swa_merge(const uint16_t *q, int32_t n_heads, const int32_t *row_seq,
                           int32_t n_rows, const csa2_swa *swa, int32_t n_seq, float scale,
                           float *o, float *lse, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Scratch bytes that lets csa2_sparse_attn (k_pos, swa_window = the SWA
 * window or 0 without SWA) or csa2_swa_merge (k_pos = 0) split the rows of
 * any call with 1 .. n_rows rows over several work-groups (the most any of
 * those row counts needs); 0 when none of them splits (a NULL workspace is
 * then fine).  Zero-fill it before its first use (see csa2_sparse_attn).
 * Returns 0 for invalid arguments. */
size_t csa2_attn_workspace_size(int32_t n_rows, int32_t n_heads, int32_t k_pos,
                                int32_t swa_window);

/* Human-readable name of a status code (static string). */
const char *csa2_status_string(csa2_status status);

/* Library version, for example "csa2 0.1.0 gfx950". */
const char *csa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
