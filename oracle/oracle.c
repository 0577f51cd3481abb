/*
 * CPU oracle for sparse NVFP4-MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the HIP path is
 * checked against.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py may load it; the library under sparse_mla_decode_amd/ never
 * links, includes or calls anything here, and nothing here is shared with it
 * (no headers, no tables, no constants).
 *
 * It is deliberately plain and slow: scalar loops, every floating-point step
 * in IEEE fp64, no blocking, no fusion, no reordering beyond what the
 * definitions state.  Sources:
 *
 *  [P1] "Prime Inference: serving GLM-5.3 to agents is a KV-cache problem"
 *       (ai.thesatyajit.com), section "Four bits per latent value: where 352
 *       comes from" (the FP8-vs-NVFP4 byte table) and section "A kernel that
 *       reads four bits directly" (-1 entries, on-chip unpack, split merge).
 *  [P3] Prime Intellect's "Prime Inference" launch post (aioga.com copy,
 *       English text), the paragraphs on compressing the MLA latent with NVFP4
 *       and on the native sparse-MLA kernel.
 *  [P5] "GLM-5.3 PCP/DCP long-context on H200" (asivanadi0.github.io),
 *       section 1 (every selected KV row serves all heads) and section 6
 *       (sparse_mla_force_mqa keeps every head on the MQA form).
 *
 * Where the pages are silent, the readings taken are:
 *   - the 64 rope values are plain OCP FP8 E4M3 bytes with no scale; only the
 *     512 latent values are NVFP4 (this is the only split that gives 352 B);
 *   - FP8 means OCP E4M3FN (bias 7, max 448, no infinities, S.1111.111 = NaN);
 *   - a block's scale is the E4M3 value nearest amax/6 (ties to even), with
 *     no second-level scale;
 *   - each latent value becomes the e2m1 value nearest x/S (ties to the even
 *     code), saturating at 6; a zero scale gives magnitude 0;
 *   - the sign bit of the input is copied into the nibble / rope byte;
 *   - element 2i is the low nibble of byte i, element 2i+1 the high nibble;
 *   - row bytes: [0,256) nibbles, [256,288) scales in block order,
 *     [288,352) rope; a page is 64 consecutive rows;
 *   - K is all 576 decoded values, V is the first 512 (the latent);
 *   - lse is the natural log of the sum of exp(scale * q.k), scale included;
 *     an empty selection gives out = 0 and lse = -inf;
 *   - an index t is used iff 0 <= t < L_b, t/64 < max_pages and its physical
 *     page lies in [0, num_pages); anything else (-1 padding included) is
 *     skipped; a repeated index counts once per occurrence;
 *   - the lean FP8 row the byte table of [P1] compares against is the 576
 *     values as OCP E4M3 bytes in dim order (latent then rope), no scale,
 *     each the E4M3 value nearest the input (ties to even, saturating at
 *     448, sign copied) -- the same rule as the NVFP4 row's rope bytes;
 *   - the staged path's temporary FP8 copy is that lean FP8 row, made from
 *     the decoded NVFP4 values by the same nearest-E4M3 rule.
 *
 * Inputs must be finite; behaviour on NaN/Inf inputs is not defined here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define LATENT 512
#define ROPE 64
#define DIM (LATENT + ROPE)
#define BLOCK 16
#define NBLOCKS (LATENT / BLOCK)
#define NIB_BYTES (LATENT / 2)
#define SCALE_OFF NIB_BYTES
#define ROPE_OFF (SCALE_OFF + NBLOCKS)
#define ROW_BYTES (ROPE_OFF + ROPE)
#define FP8_ROW_BYTES DIM
#define PAGE_ROWS 64

/* ---------------------------------------------------------------------- */
/* OCP FP8 E4M3FN                                                           */
/* ---------------------------------------------------------------------- */

/* Exact value of an E4M3FN code: exponent field e, mantissa field m.
 * e == 0: m/8 * 2^-6 (subnormal); otherwise (1 + m/8) * 2^(e-7);
 * S.1111.111 is NaN. */
double oracle_e4m3_value(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = (m / 8.0) * pow(2.0, -6);
    else
        mag = (1.0 + m / 8.0) * pow(2.0, e - 7);
    return s ? -mag : mag;
}

/* Code of the E4M3 value nearest |num| / den (den > 0), ties to the code with
 * an even mantissa, the sign bit of num copied.  The finite non-negative
 * codes 0x00..0x7E form an increasing grid; |num|/den is compared against
 * den * (midpoint of two neighbours), which is exact in fp64 for den = 1 and
 * den = 6 (a midpoint has at most 5 significant bits).  Past the last
 * midpoint the largest finite value (448) is nearest, so saturation needs no
 * special case. */
uint8_t oracle_e4m3_nearest(double num, double den)
{
    double a = fabs(num);
    uint8_t sign = signbit(num) ? 0x80 : 0x00;
    for (int c = 0; c < 0x7E; ++c) {
        double lo = oracle_e4m3_value((uint8_t)c);
        double hi = oracle_e4m3_value((uint8_t)(c + 1));
        double mid = den * ((lo + hi) / 2.0);
        if (a < mid)
            return sign | (uint8_t)c;
        if (a == mid)
            return sign | (uint8_t)((c % 2 == 0) ? c : c + 1);
    }
    return sign | 0x7E;
}

/* ---------------------------------------------------------------------- */
/* e2m1 (FP4) nibbles                                                       */
/* ---------------------------------------------------------------------- */

/* Magnitudes of the eight e2m1 codes: 1 exponent-bias, 2 exponent bits, 1
 * mantissa bit; code 1 is the only subnormal. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(uint8_t nib)
{
    double v = E2M1_MAG[nib & 7];
    return (nib & 8) ? -v : v;
}

/* Nibble whose value times S is nearest x: magnitude code by midpoint
 * comparison (S * midpoint is exact in fp64), ties to the even code,
 * saturating at 6; S == 0 gives magnitude 0; sign bit of x copied. */
uint8_t oracle_e2m1_nearest(double x, double S)
{
    double a = fabs(x);
    uint8_t sign = signbit(x) ? 0x8 : 0x0;
    if (S == 0.0)
        return sign;
    for (int c = 0; c < 7; ++c) {
        double mid = S * ((E2M1_MAG[c] + E2M1_MAG[c + 1]) / 2.0);
        if (a < mid)
            return sign | (uint8_t)c;
        if (a == mid)
            return sign | (uint8_t)((c % 2 == 0) ? c : c + 1);
    }
    return sign | 7;
}

/* Array forms of the three scalar functions above (for exhaustive tests). */
void oracle_e4m3_value_many(const uint8_t *codes, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_value(codes[i]);
}

void oracle_e4m3_nearest_many(const double *num, int64_t n, double den, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = oracle_e4m3_nearest(num[i], den);
}

void oracle_e2m1_nearest_many(const double *x, const double *S, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = oracle_e2m1_nearest(x[i], S[i]);
}

/* ---------------------------------------------------------------------- */
/* Rows                                                                     */
/* ---------------------------------------------------------------------- */

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One 576-value BF16 row -> one 352-byte NVFP4 row [P1 byte table; P3]. */
void oracle_quant_row(const uint16_t *x, uint8_t *row)
{
    uint8_t nib[LATENT];
    memset(row, 0, ROW_BYTES);
    for (int b = 0; b < NBLOCKS; ++b) {
        double amax = 0.0;
        for (int j = 0; j < BLOCK; ++j) {
            double a = fabs(bf16_value(x[b * BLOCK + j]));
            if (a > amax)
                amax = a;
        }
        uint8_t s = oracle_e4m3_nearest(amax, 6.0);
        double S = oracle_e4m3_value(s);
        row[SCALE_OFF + b] = s;
        for (int j = 0; j < BLOCK; ++j)
            nib[b * BLOCK + j] = oracle_e2m1_nearest(bf16_value(x[b * BLOCK + j]), S);
    }
    for (int i = 0; i < NIB_BYTES; ++i)
        row[i] = (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));
    for (int j = 0; j < ROPE; ++j)
        row[ROPE_OFF + j] = oracle_e4m3_nearest(bf16_value(x[LATENT + j]), 1.0);
}

/* Timing infrastructure, no arithmetic: the thread count of the OpenMP
 * loops that take none as an argument (the row quantisers) for later calls
 * from the calling thread; nthreads <= 0 keeps the current one.  Returns the
 * count those loops will use (1 without OpenMP). */
int oracle_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* One 352-byte row -> its 576 exact values: latent d is
 * e2m1(nibble d) * E4M3(scale of block d/16), rope j is E4M3(byte j). */
void oracle_dequant_row(const uint8_t *row, double *k)
{
    for (int d = 0; d < LATENT; ++d) {
        uint8_t byte = row[d / 2];
        uint8_t nib = (d % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        k[d] = oracle_e2m1_value(nib) * oracle_e4m3_value(row[SCALE_OFF + d / BLOCK]);
    }
    for (int j = 0; j < ROPE; ++j)
        k[LATENT + j] = oracle_e4m3_value(row[ROPE_OFF + j]);
}

void oracle_quant_rows(const uint16_t *x, int64_t n, uint8_t *rows)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        oracle_quant_row(x + i * DIM, rows + i * ROW_BYTES);
}

void oracle_dequant_rows(const uint8_t *rows, int64_t n, double *k)
{
    for (int64_t i = 0; i < n; ++i)
        oracle_dequant_row(rows + i * ROW_BYTES, k + i * DIM);
}

/* Paged append: row i goes to slot s = slot_mapping[i], i.e. page s / 64,
 * row s % 64 of that page.  Negative slots and slots past the cache are
 * skipped.  Returns the number of rows written. */
int64_t oracle_kv_quant_append(const uint16_t *x, int64_t n, const int32_t *slot_mapping,
                               uint8_t *cache, int64_t num_pages)
{
    int64_t written = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t s = slot_mapping[i];
        if (s < 0 || s >= num_pages * PAGE_ROWS)
            continue;
        oracle_quant_row(x + i * DIM, cache + s * ROW_BYTES);
        ++written;
    }
    return written;
}

/* ---------------------------------------------------------------------- */
/* Lean FP8 rows [P1 byte table: 576 B per row in FP8]                       */
/* ---------------------------------------------------------------------- */

/* One 576-value BF16 row -> 576 E4M3 bytes, dim order, no scale. */
void oracle_quant_row_fp8(const uint16_t *x, uint8_t *row)
{
    for (int d = 0; d < DIM; ++d)
        row[d] = oracle_e4m3_nearest(bf16_value(x[d]), 1.0);
}

/* One 576-byte FP8 row -> its 576 exact values. */
void oracle_dequant_row_fp8(const uint8_t *row, double *k)
{
    for (int d = 0; d < DIM; ++d)
        k[d] = oracle_e4m3_value(row[d]);
}

void oracle_quant_rows_fp8(const uint16_t *x, int64_t n, uint8_t *rows)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        oracle_quant_row_fp8(x + i * DIM, rows + i * FP8_ROW_BYTES);
}

void oracle_dequant_rows_fp8(const uint8_t *rows, int64_t n, double *k)
{
    for (int64_t i = 0; i < n; ++i)
        oracle_dequant_row_fp8(rows + i * FP8_ROW_BYTES, k + i * DIM);
}

/* Paged append of FP8 rows: the slot rules of oracle_kv_quant_append. */
int64_t oracle_kv_quant_append_fp8(const uint16_t *x, int64_t n, const int32_t *slot_mapping,
                                   uint8_t *cache, int64_t num_pages)
{
    int64_t written = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t s = slot_mapping[i];
        if (s < 0 || s >= num_pages * PAGE_ROWS)
            continue;
        oracle_quant_row_fp8(x + i * DIM, cache + s * FP8_ROW_BYTES);
        ++written;
    }
    return written;
}

/* ---------------------------------------------------------------------- */
/* Sparse MLA decode                                                         */
/* ---------------------------------------------------------------------- */

/* For each sequence b and head h, with the selected rows k_t (t over the
 * usable entries of topk[b], in list order):
 *     s_t = softmax_scale * sum_d q[b,h,d] * k_t[d]          (d < 576)
 *     out[b,h,:] = sum_t exp(s_t) * k_t[0:512] / sum_t exp(s_t)
 *     lse[b,h]   = ln sum_t exp(s_t)
 * evaluated with the usual max shift m = max_t s_t.  This is softmax
 * attention of the absorbed query over the selected latent rows, all heads
 * reading the same rows [P5 sections 1 and 6; P3 native kernel paragraph].
 * Usable entries: 0 <= t < seq_lens[b], t/64 < max_pages and
 * 0 <= page_table[b][t/64] < num_pages [P1, the -1 entries of short
 * contexts].  out is [B,H,512], lse is [B,H], both fp64. */
typedef void (*dequant_fn)(const uint8_t *row, double *k);

static void decode_rows(const uint16_t *q, const uint8_t *cache, int row_bytes, dequant_fn dequant,
                        int64_t num_pages, const int32_t *page_table, int32_t max_pages,
                        const int32_t *seq_lens, const int32_t *topk, int32_t batch, int32_t heads,
                        int32_t topk_len, double softmax_scale, double *out, double *lse,
                        int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    double *k = (double *)malloc(sizeof(double) * (size_t)(topk_len > 0 ? topk_len : 1) * DIM);
    for (int32_t b = 0; b < batch; ++b) {
        int64_t L = seq_lens[b];
        int64_t n = 0;
        for (int32_t i = 0; i < topk_len; ++i) {
            int64_t t = topk[(int64_t)b * topk_len + i];
            if (t < 0 || t >= L || (t / PAGE_ROWS) >= max_pages)
                continue;
            int64_t page = page_table[(int64_t)b * max_pages + t / PAGE_ROWS];
            if (page < 0 || page >= num_pages)
                continue;
            const uint8_t *row = cache + (page * PAGE_ROWS + t % PAGE_ROWS) * row_bytes;
            dequant(row, k + n * DIM);
            ++n;
        }
        int32_t h;
#pragma omp parallel for schedule(dynamic)
        for (h = 0; h < heads; ++h) {
            const uint16_t *qh = q + ((int64_t)b * heads + h) * DIM;
            double *o = out + ((int64_t)b * heads + h) * LATENT;
            double qd[DIM];
            for (int d = 0; d < DIM; ++d)
                qd[d] = bf16_value(qh[d]);
            if (n == 0) {
                for (int d = 0; d < LATENT; ++d)
                    o[d] = 0.0;
                lse[(int64_t)b * heads + h] = -INFINITY;
                continue;
            }
            double *s = (double *)malloc(sizeof(double) * (size_t)n);
            double m = -INFINITY;
            for (int64_t i = 0; i < n; ++i) {
                double acc = 0.0;
                for (int d = 0; d < DIM; ++d)
                    acc += qd[d] * k[i * DIM + d];
                s[i] = softmax_scale * acc;
                if (s[i] > m)
                    m = s[i];
            }
            double l = 0.0;
            for (int d = 0; d < LATENT; ++d)
                o[d] = 0.0;
            for (int64_t i = 0; i < n; ++i) {
                double w = exp(s[i] - m);
                l += w;
                for (int d = 0; d < LATENT; ++d)
                    o[d] += w * k[i * DIM + d];
            }
            for (int d = 0; d < LATENT; ++d)
                o[d] /= l;
            lse[(int64_t)b * heads + h] = m + log(l);
            free(s);
        }
    }
    free(k);
}

/* Decode over the NVFP4 cache [num_pages][64][352]. */
void oracle_sparse_mla_decode(const uint16_t *q, const uint8_t *cache, int64_t num_pages,
                              const int32_t *page_table, int32_t max_pages,
                              const int32_t *seq_lens, const int32_t *topk, int32_t batch,
                              int32_t heads, int32_t topk_len, double softmax_scale,
                              double *out, double *lse, int nthreads)
{
    decode_rows(q, cache, ROW_BYTES, oracle_dequant_row, num_pages, page_table, max_pages,
                seq_lens, topk, batch, heads, topk_len, softmax_scale, out, lse, nthreads);
}

/* The same decode over the lean FP8 cache [num_pages][64][576]. */
void oracle_sparse_mla_decode_fp8(const uint16_t *q, const uint8_t *cache, int64_t num_pages,
                                  const int32_t *page_table, int32_t max_pages,
                                  const int32_t *seq_lens, const int32_t *topk, int32_t batch,
                                  int32_t heads, int32_t topk_len, double softmax_scale,
                                  double *out, double *lse, int nthreads)
{
    decode_rows(q, cache, FP8_ROW_BYTES, oracle_dequant_row_fp8, num_pages, page_table,
                max_pages, seq_lens, topk, batch, heads, topk_len, softmax_scale, out, lse,
                nthreads);
}

/* ---------------------------------------------------------------------- */
/* Staged path [P1 staged-vs-native figure and the paragraph before it; P3   */
/* first implementation]                                                    */
/* ---------------------------------------------------------------------- */

/* The staged path's gather-unpack: every usable entry e of topk[b] (the
 * rule of decode_rows) has its NVFP4 row decoded and each of the 576 values
 * re-encoded as the E4M3 value nearest it (ties to even, saturating at 448):
 * a lean FP8 row, written to row b * kpad + e of `staged` (kpad = topk_len
 * rounded up to 64), and staged_topk[b][e] = e.  An unusable entry gets
 * staged_topk[b][e] = -1 and its staged row is left as it was.  Attention
 * over the copy is then the FP8 decode with page table [b][p] = b * kpad/64
 * + p and seq_lens = kpad. */
void oracle_stage_rows_fp8(const uint8_t *cache, int64_t num_pages, const int32_t *page_table,
                           int32_t max_pages, const int32_t *seq_lens, const int32_t *topk,
                           int32_t batch, int32_t topk_len, uint8_t *staged, int32_t *staged_topk)
{
    int64_t kpad = ((int64_t)topk_len + PAGE_ROWS - 1) / PAGE_ROWS * PAGE_ROWS;
    double k[DIM];
    for (int32_t b = 0; b < batch; ++b) {
        int64_t L = seq_lens[b];
        for (int32_t e = 0; e < topk_len; ++e) {
            int64_t t = topk[(int64_t)b * topk_len + e];
            int32_t *st = staged_topk + (int64_t)b * topk_len + e;
            *st = -1;
            if (t < 0 || t >= L || (t / PAGE_ROWS) >= max_pages)
                continue;
            int64_t page = page_table[(int64_t)b * max_pages + t / PAGE_ROWS];
            if (page < 0 || page >= num_pages)
                continue;
            oracle_dequant_row(cache + (page * PAGE_ROWS + t % PAGE_ROWS) * ROW_BYTES, k);
            uint8_t *dst = staged + ((int64_t)b * kpad + e) * FP8_ROW_BYTES;
            for (int d = 0; d < DIM; ++d)
                dst[d] = oracle_e4m3_nearest(k[d], 1.0);
            *st = e;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Top-k select of the indexer's scores [P1 section "Decode: TP4, and the    */
/* copies it keeps": an indexer picks the top cached positions, at most      */
/* 2,048 per query; the prefill-timing figure's "DSA indexer (logits,       */
/* top-k)"]                                                                  */
/* ---------------------------------------------------------------------- */

typedef struct {
    float score;
    int32_t index;
} scored_t;

/* higher score first; equal scores by lower index */
static int by_score_desc(const void *pa, const void *pb)
{
    const scored_t *a = (const scored_t *)pa, *b = (const scored_t *)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->index > b->index) - (a->index < b->index);
}

/* For each query b: the positions of the min(topk, L_b) largest of
 * scores[b][0 .. L_b), best first (equal scores by lower position), then -1
 * up to topk.  L_b = seq_lens[b] clamped to [0, ld].  Scores must be finite. */
void oracle_topk_select(const float *scores, int64_t ld, const int32_t *seq_lens, int32_t batch,
                        int32_t topk, int32_t *out)
{
    for (int32_t b = 0; b < batch; ++b) {
        int64_t L = seq_lens[b];
        if (L < 0)
            L = 0;
        if (L > ld)
            L = ld;
        scored_t *v = (scored_t *)malloc(sizeof(scored_t) * (size_t)(L > 0 ? L : 1));
        for (int64_t i = 0; i < L; ++i) {
            v[i].score = scores[(int64_t)b * ld + i];
            v[i].index = (int32_t)i;
        }
        qsort(v, (size_t)L, sizeof(scored_t), by_score_desc);
        for (int32_t e = 0; e < topk; ++e)
            out[(int64_t)b * topk + e] = e < L ? v[e].index : -1;
        free(v);
    }
}

int oracle_row_bytes(void) { return ROW_BYTES; }
int oracle_fp8_row_bytes(void) { return FP8_ROW_BYTES; }
int oracle_page_rows(void) { return PAGE_ROWS; }
