/*
 * CSA2 reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, CPU implementation of what the CSA2 hot path computes, in
 * fp64.  Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library; the product path (libcsa2) never links,
 * calls or includes anything from this directory, and this file shares no code
 * with it.
 *
 * Sources (pages cited by title and section):
 *  [P1] onedev.kr digest "KV 캐시를 토큰당 890바이트로 압축한 552B 멀티모달 MoE,
 *       DeepSeek-V4.1-Flash", section "무엇과 다른가" (how it differs): the three
 *       CSA2 modes, FP4 global KV, the hierarchical sparse indexer.
 *  [P3] genexis.ai explainer "100만 토큰을 0.9GB에, 딥시크 V4.1 논문이 KV 캐시를
 *       줄인 방법", sections "레이어 40개 가운데 4개만 전역 캐시를 만듭니다"
 *       (356-B entry, 2,048 blocks of 8, Top-512) and "4비트로 적어도 되는 이유"
 *       (NVFP4 without the second-level scale, one 8-bit scale per 16 values,
 *       448 x 6 range), "전역 어텐션과 지역 어텐션" (SWA window of 128).
 *  Format definitions: OCP Microscaling (MX) v1.0 for E2M1, OCP 8-bit floating
 *  point (OFP8) for E4M3FN.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *  - scale = round-to-nearest-even of amax/6 into E4M3FN (saturating at 448);
 *  - value = round-to-nearest-even of |x|/scale into E2M1 (saturating at 6);
 *    a group whose scale rounds to zero stores magnitude 0;
 *  - sign bit = (x < 0); channel 2k in the low nibble of byte k;
 *  - indexer key: 128 channels, one E4M3 scale per 32 channels (64 + 4 = 68 B);
 *  - index score = sum_h w_h * max(0, q_h . k) over 8 heads of 128 dims;
 *  - block score = max over the visible entries of an aligned block of 8;
 *  - ranking: score descending, then lower index first; output ascending.
 *
 * Parity pins (what each function is checked against) are listed in the test
 * files; no function here is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* E2M1 (OCP MX): 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf/NaN.
 * e == 0 is subnormal: m * 2^-1; otherwise (1 + m/2) * 2^(e-1). */
double oracle_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E4M3FN (OFP8): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no inf;
 * S.1111.111 is NaN; e == 0 is subnormal: (m/8) * 2^-6. */
double oracle_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Values of the 127 finite non-negative E4M3FN codes and of the 8 E2M1
 * magnitudes, filled once when the library is loaded (the same numbers
 * oracle_e4m3_value and oracle_e2m1_value return). */
static double g_e4m3_pos[0x7F];
static double g_e2m1_pos[8];
__attribute__((constructor)) static void fill_tables(void)
{
    for (int b = 0; b <= 0x7E; ++b) g_e4m3_pos[b] = oracle_e4m3_value(b);
    for (int c = 0; c < 8; ++c) g_e2m1_pos[c] = oracle_e2m1_value(c);
}

/* Nearest non-negative E4M3FN value to v >= 0, ties to the even code
 * (mantissa LSB 0).  Exhaustive search over the 127 finite non-negative codes;
 * values above 448 therefore land on 448 (saturation). */
static int encode_e4m3_nonneg(double v)
{
    int best = 0;
    double best_d = fabs(v - g_e4m3_pos[0]);
    for (int b = 1; b <= 0x7E; ++b) {
        double d = fabs(v - g_e4m3_pos[b]);
        if (d < best_d || (d == best_d && (b & 1) == 0 && (best & 1) == 1)) {
            best = b;
            best_d = d;
        }
    }
    return best;
}

/* Nearest E2M1 magnitude code (0..7) to y >= 0, ties to the even code. */
static int encode_e2m1_mag(double y)
{
    int best = 0;
    double best_d = fabs(y - g_e2m1_pos[0]);
    for (int c = 1; c <= 7; ++c) {
        double d = fabs(y - g_e2m1_pos[c]);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* --------------------------------------------------------- FP4 encoding */

/* Quantise n rows of `dim` fp32 values into E2M1 codes with one E4M3 scale
 * per `group` channels [P3 "4비트로 적어도 되는 이유"; P3 "레이어 40개 가운데
 * 4개만..." for the 512-ch / 128-d entry].
 * codes: [n][dim/2] bytes, channel 2k low nibble, 2k+1 high nibble.
 * scales: [n][dim/group] E4M3FN bytes. */
void oracle_quantize(const float *x, int64_t n, int dim, int group,
                     uint8_t *codes, uint8_t *scales)
{
    int ngroups = dim / group;
    for (int64_t r = 0; r < n; ++r) {
        const float *row = x + r * dim;
        uint8_t *crow = codes + r * (dim / 2);
        memset(crow, 0, (size_t)(dim / 2));
        for (int g = 0; g < ngroups; ++g) {
            double amax = 0.0;
            for (int i = 0; i < group; ++i) {
                double a = fabs((double)row[g * group + i]);
                if (a > amax) amax = a;
            }
            int sbyte = encode_e4m3_nonneg(amax / 6.0);
            double s = oracle_e4m3_value(sbyte);
            scales[r * ngroups + g] = (uint8_t)sbyte;
            for (int i = 0; i < group; ++i) {
                int ch = g * group + i;
                double xv = (double)row[ch];
                int mag = (s == 0.0) ? 0 : encode_e2m1_mag(fabs(xv) / s);
                int code = (xv < 0.0 ? 8 : 0) | mag;
                crow[ch / 2] |= (uint8_t)((ch & 1) ? (code << 4) : code);
            }
        }
    }
}

/* Exact decode: x_hat = E2M1(code) * E4M3(scale). out: [n][dim] fp64. */
void oracle_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t n,
                       int dim, int group, double *out)
{
    int ngroups = dim / group;
    for (int64_t r = 0; r < n; ++r) {
        for (int ch = 0; ch < dim; ++ch) {
            uint8_t byte = codes[r * (dim / 2) + ch / 2];
            int code = (ch & 1) ? (byte >> 4) : (byte & 15);
            double s = oracle_e4m3_value(scales[r * ngroups + ch / group]);
            out[r * dim + ch] = oracle_e2m1_value(code) * s;
        }
    }
}

/* bf16 bit pattern -> exact fp64. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------ indexer */

/* Index score of candidate entries for one query row [P1 "무엇과 다른가":
 * the indexer Q scores entries against the indexer key projected from main
 * KV; the combination over 8 heads with ReLU and per-head weights is the
 * reading taken where the pages give no formula].
 * q_idx: bf16 [8][128]; w: [8]; ik_codes/ik_scales: the sequence's indexer
 * planes ([n][64], [n][4]); entries: candidate entry ids; scores: [n_cand]. */
void oracle_index_scores(const uint16_t *q_idx, const float *w,
                         const uint8_t *ik_codes, const uint8_t *ik_scales,
                         const int64_t *entries, int64_t n_cand, double *scores)
{
    double q[8][128];
    for (int h = 0; h < 8; ++h)
        for (int c = 0; c < 128; ++c) q[h][c] = bf16_to_double(q_idx[h * 128 + c]);
    double k[128];
    for (int64_t i = 0; i < n_cand; ++i) {
        int64_t j = entries[i];
        oracle_dequantize(ik_codes + j * 64, ik_scales + j * 4, 1, 128, 32, k);
        double score = 0.0;
        for (int h = 0; h < 8; ++h) {
            double d = 0.0;
            for (int c = 0; c < 128; ++c) d += q[h][c] * k[c];
            if (d > 0.0) score += (double)w[h] * d;
        }
        scores[i] = score;
    }
}

/* Ranking helper: indices ordered by value descending, ties by lower index.
 * The comparator reads the values through a thread-local pointer so that
 * rows may be processed from several threads. */
static __thread const double *g_rank_vals;
static int cmp_rank(const void *a, const void *b)
{
    int64_t i = *(const int64_t *)a, j = *(const int64_t *)b;
    double vi = g_rank_vals[i], vj = g_rank_vals[j];
    if (vi > vj) return -1;
    if (vi < vj) return 1;
    return (i < j) ? -1 : (i > j);
}
static int cmp_i64(const void *a, const void *b)
{
    int64_t i = *(const int64_t *)a, j = *(const int64_t *)b;
    return (i < j) ? -1 : (i > j);
}

/* Keep the k best of vals[0..n) (descending value, ties to lower index) and
 * write their positions in ascending order to out[0..min(k,n)); returns the
 * count. */
static int64_t rank_select(const double *vals, int64_t n, int64_t k, int64_t *out)
{
    int64_t *order = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) order[i] = i;
    g_rank_vals = vals;
    qsort(order, (size_t)n, sizeof(int64_t), cmp_rank);
    int64_t m = n < k ? n : k;
    memcpy(out, order, (size_t)m * sizeof(int64_t));
    qsort(out, (size_t)m, sizeof(int64_t), cmp_i64);
    free(order);
    return m;
}

/* Hierarchical pool, first stage [P3 "레이어 40개 가운데 4개만...": the first
 * decoder Full layer picks up to 2,048 high-scoring blocks of 8 positions;
 * P1 "무엇과 다른가" for the block-of-8 example].
 * entry_scores: scores of entries 0..n_vis-1.  Block b covers entries
 * [8b, 8b+8) ∩ [0, n_vis); its score is the max over those entries.
 * Writes the kept block ids ascending to pool_blocks and their block scores to
 * block_scores (optional, [ceil(n_vis/8)]); returns the pool size. */
int64_t oracle_block_pool(const double *entry_scores, int64_t n_vis, int64_t k_blk,
                          int32_t *pool_blocks, double *block_scores)
{
    int64_t nb = (n_vis + 7) / 8;
    double *bs = (double *)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(double));
    for (int64_t b = 0; b < nb; ++b) {
        double m = -INFINITY;
        for (int64_t j = 8 * b; j < 8 * b + 8 && j < n_vis; ++j)
            if (entry_scores[j] > m) m = entry_scores[j];
        bs[b] = m;
        if (block_scores) block_scores[b] = m;
    }
    int64_t *kept = (int64_t *)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(int64_t));
    int64_t m = rank_select(bs, nb, k_blk, kept);
    for (int64_t i = 0; i < m; ++i) pool_blocks[i] = (int32_t)kept[i];
    free(kept);
    free(bs);
    return m;
}

/* Candidate entries of a pool: the visible entries of the kept blocks, in
 * ascending order.  Returns the count (<= 8 * n_pool). */
int64_t oracle_pool_entries(const int32_t *pool_blocks, int64_t n_pool, int64_t n_vis,
                            int64_t *entries)
{
    int64_t c = 0;
    for (int64_t p = 0; p < n_pool; ++p)
        for (int64_t e = 0; e < 8; ++e) {
            int64_t j = 8 * (int64_t)pool_blocks[p] + e;
            if (j < n_vis) entries[c++] = j;
        }
    return c;
}

/* Top-K positions [P3 "레이어 40개 가운데 4개만...": the Reindex layers pick
 * 512 positions inside the candidate pool].  scores[i] belongs to entry
 * cand[i]; keeps min(k, n_cand) best, writes their entry ids ascending into
 * topk[0..k) and pads with -1; returns the count. */
int64_t oracle_topk(const double *scores, const int64_t *cand, int64_t n_cand, int64_t k,
                    int32_t *topk)
{
    int64_t *kept = (int64_t *)malloc((size_t)(n_cand > 0 ? n_cand : 1) * sizeof(int64_t));
    int64_t m = rank_select(scores, n_cand, k, kept);
    for (int64_t i = 0; i < k; ++i) topk[i] = (i < m) ? (int32_t)cand[kept[i]] : -1;
    free(kept);
    return m;
}

/* ---------------------------------------------------------- attention */

/* Softmax attention of H query heads over n_keys keys of 512 dims with the
 * value equal to the key (the main-KV latent is shared by all heads and
 * serves as both K and V) [P1 "무엇과 다른가": every mode attends with its own
 * global Q over the main KV; P3 "전역 어텐션과 지역 어텐션" for the SWA branch].
 * q: bf16 [H][512]; keys: fp64 [n_keys][512]; logits = scale * q_h . key.
 * o: [H][512], lse: [H] (natural log of the softmax normaliser).  With no
 * keys, o = 0 and lse = -inf. */
void oracle_attention(const uint16_t *q, int H, const double *keys, int64_t n_keys,
                      double scale, double *o, double *lse)
{
    double *logit = (double *)malloc((size_t)(n_keys > 0 ? n_keys : 1) * sizeof(double));
    for (int h = 0; h < H; ++h) {
        double qh[512];
        for (int c = 0; c < 512; ++c) qh[c] = bf16_to_double(q[h * 512 + c]);
        double mx = -INFINITY;
        for (int64_t j = 0; j < n_keys; ++j) {
            double d = 0.0;
            for (int c = 0; c < 512; ++c) d += qh[c] * keys[j * 512 + c];
            logit[j] = scale * d;
            if (logit[j] > mx) mx = logit[j];
        }
        for (int c = 0; c < 512; ++c) o[h * 512 + c] = 0.0;
        if (n_keys == 0) {
            lse[h] = -INFINITY;
            continue;
        }
        double denom = 0.0;
        for (int64_t j = 0; j < n_keys; ++j) denom += exp(logit[j] - mx);
        for (int64_t j = 0; j < n_keys; ++j) {
            double p = exp(logit[j] - mx) / denom;
            for (int c = 0; c < 512; ++c) o[h * 512 + c] += p * keys[j * 512 + c];
        }
        lse[h] = mx + log(denom);
    }
    free(logit);
}

/* Merge of two attention results over disjoint key sets by their
 * log-sum-exp: the result is the softmax over the union.  An empty branch has
 * lse = -inf and contributes nothing. */
void oracle_lse_merge(const double *o_a, const double *lse_a, const double *o_b,
                      const double *lse_b, int H, int dim, double *o, double *lse)
{
    for (int h = 0; h < H; ++h) {
        double la = lse_a[h], lb = lse_b[h];
        if (la == -INFINITY && lb == -INFINITY) {
            for (int c = 0; c < dim; ++c) o[h * dim + c] = 0.0;
            lse[h] = -INFINITY;
            continue;
        }
        double m = la > lb ? la : lb;
        double wa = exp(la - m), wb = exp(lb - m);
        for (int c = 0; c < dim; ++c)
            o[h * dim + c] = (wa * o_a[h * dim + c] + wb * o_b[h * dim + c]) / (wa + wb);
        lse[h] = m + log(wa + wb);
    }
}

/* E4M3FN SWA rows -> fp64 (unit scale). */
void oracle_decode_e4m3_rows(const uint8_t *rows, int64_t n, int dim, double *out)
{
    for (int64_t i = 0; i < n * dim; ++i) out[i] = oracle_e4m3_value(rows[i]);
}
