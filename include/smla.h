/*
 * smla.h -- C ABI of the MI355X (gfx950) sparse NVFP4-MLA decode library.
 *
 * Two operations make up the decode-side hot path of sparse multi-head latent
 * attention over a paged, NVFP4-compressed latent KV cache:
 *
 *   smla_kv_quant_append   BF16 KV rows -> 352-byte NVFP4 rows in the paged cache
 *   smla_sparse_mla_decode q, cache, page table, top-k indices -> out, lse
 *
 * and the same pair over the lean FP8 row that the pages compare NVFP4 with
 * (smla_kv_quant_append_fp8, smla_sparse_mla_decode_fp8; see the end).
 *
 * Sources (page titles; no other document is needed to read this header):
 *   [P1] "Prime Inference: serving GLM-5.3 to agents is a KV-cache problem",
 *        section "Four bits per latent value: where 352 comes from" (row bytes:
 *        512 latent values at 4 bits = 256 B, one FP8 scale per 16 values =
 *        32 B, 64 rope values in FP8 = 64 B) and section "A kernel that reads
 *        four bits directly" (selected rows are unpacked on chip; -1 entries of
 *        short contexts carry no data).
 *   [P3] Prime Intellect's "Prime Inference" launch post, the paragraphs on the
 *        NVFP4 latent and on the native sparse-MLA kernel (FP16 operands,
 *        FP32 accumulation, no intermediate buffer in GPU memory).
 *   [P5] "GLM-5.3 PCP/DCP long-context on H200", section 1 (every selected KV
 *        row serves all heads of the absorbed query).
 *
 * Row format (one token, 352 bytes; readings where the pages are silent):
 *   bytes [0,256)   latent values 0..511 as e2m1 nibbles, value 2i in the low
 *                   nibble of byte i, value 2i+1 in the high nibble;
 *   bytes [256,288) one OCP FP8 E4M3 (E4M3FN) scale per block of 16 latent
 *                   values, in block order; scale = E4M3 value nearest
 *                   amax(|block|)/6 (ties to even); nibble = e2m1 value
 *                   nearest x/scale (ties to the even code, saturating at 6,
 *                   0 when the scale is 0); the input's sign bit is copied;
 *   bytes [288,352) the 64 rope values as OCP FP8 E4M3 (nearest, ties to
 *                   even, saturating at +-448), no scale.
 * A page holds 64 consecutive rows (22,528 bytes); the cache is
 * [num_pages][64][352] bytes.  Token t of sequence b lives in physical page
 * page_table[b][t / 64], row t % 64.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers on the current HIP device, except that
 *     `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - The caller owns every buffer.  The library allocates nothing, frees
 *     nothing and keeps no pointer after a call returns.
 *   - Work is enqueued asynchronously on `stream`; nothing is synchronised.
 *   - Arguments are validated on the host before anything is launched.  On
 *     any error the call returns a negative SMLA_ERR_* code and no buffer is
 *     touched.  smla_strerror() names the code.
 *   - Device-resident data (indices, slots, page ids, sequence lengths) is
 *     never trusted: an entry outside its valid range is skipped, never
 *     dereferenced.
 *   - Inputs (rows, q) must be finite.  q must also lie inside the FP16 range
 *     (|q| < 65504), because the score contraction runs on FP16 operands.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_LATENT 512
#define SMLA_ROPE 64
#define SMLA_DIM 576
#define SMLA_ROW_BYTES 352
#define SMLA_PAGE_ROWS 64
#define SMLA_PAGE_BYTES (SMLA_PAGE_ROWS * SMLA_ROW_BYTES)
#define SMLA_FP8_ROW_BYTES 576
#define SMLA_MAX_TOPK 2048

enum {
    SMLA_OK = 0,
    SMLA_ERR_NULL = -1,        /* a required pointer is NULL                  */
    SMLA_ERR_SHAPE = -2,       /* a size is out of range                       */
    SMLA_ERR_UNSUPPORTED = -3, /* a supported-but-not-built configuration      */
    SMLA_ERR_ALIGN = -4,       /* a pointer is not aligned as documented       */
    SMLA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required   */
    SMLA_ERR_LAUNCH = -6,      /* the HIP runtime rejected a kernel launch     */
    SMLA_ERR_DEVICE = -7,      /* no usable gfx950 device is current           */
    SMLA_ERR_SCRATCH = -8      /* the shape needs more than the static scratch */
};

/* Human-readable name of a status code (static storage, never NULL). */
const char *smla_strerror(int code);

/* Library ABI version (major * 100 + minor). */
int smla_version(void);

/*
 * Quantise n BF16 rows into the paged NVFP4 cache [P1 row-bytes table; P3].
 *
 *   rows_bf16     [n][576] BF16 (latent 0..511, then rope 0..63), 16-byte aligned
 *   n             number of rows, 0 <= n <= 2^31-1 (n == 0 enqueues nothing)
 *   slot_mapping  [n] int32; row i is written to slot s = slot_mapping[i],
 *                 i.e. cache page s / 64, row s % 64.  A slot < 0 (e.g. -1)
 *                 or >= num_pages*64 is skipped.  Two rows naming the same
 *                 slot in one call: which one lands is unspecified.
 *   cache         [num_pages][64][352] uint8, 256-byte aligned
 *   num_pages     1 <= num_pages <= 2^25
 *
 * The packed bytes equal, bit for bit, the format rules stated at the top.
 */
int smla_kv_quant_append(const void *rows_bf16, int64_t n, const int32_t *slot_mapping,
                         uint8_t *cache, int64_t num_pages, void *stream);

/*
 * Bytes of device workspace smla_sparse_mla_decode needs for this shape
 * (0 means none).  The workspace holds per-split partial results between
 * the two kernels a call may enqueue; its contents on entry do not matter.
 * Calls that overlap in time must not share a workspace.
 */
size_t smla_decode_workspace_bytes(int32_t batch, int32_t heads, int32_t topk);

/*
 * Sparse MLA decode over the NVFP4 cache [P1 kernel section; P3 native
 * kernel paragraph; P5 section 1].  For each sequence b and head h, over the
 * usable entries t of topk_indices[b] (list order, repeats counted):
 *
 *     k_t      = the 576 values of row t decoded exactly from the cache
 *     s_t      = softmax_scale * sum_{d<576} q[b,h,d] * k_t[d]
 *     out[b,h] = sum_t exp(s_t) k_t[0:512] / sum_t exp(s_t)
 *     lse[b,h] = ln sum_t exp(s_t)            (natural log, scale included)
 *
 * An entry t is usable iff 0 <= t < seq_lens[b], t/64 < max_pages and
 * 0 <= page_table[b][t/64] < num_pages; all others (the -1 padding of short
 * contexts among them) are skipped and cost no cache read.  With no usable
 * entry, out[b,h,:] = 0 and lse[b,h] = -inf.
 *
 *   q_bf16        [batch][heads][576] BF16, 16-byte aligned
 *   cache         [num_pages][64][352] uint8, 256-byte aligned, 1 <= num_pages <= 2^25
 *   page_table    [batch][max_pages] int32, max_pages >= 1
 *   seq_lens      [batch] int32
 *   topk_indices  [batch][topk] int32
 *   batch         1 <= batch <= 65535
 *   heads         16 or 64
 *   topk          1 <= topk <= 2048
 *   out           [batch][heads][512] fp32, 16-byte aligned (written)
 *   lse           [batch][heads] fp32 (written)
 *   workspace     >= smla_decode_workspace_bytes(batch, heads, topk) bytes,
 *                 256-byte aligned, any contents (may be NULL when that size
 *                 is 0)
 *
 * Scores use FP16 operands (q and the decoded values; the decoded values are
 * exact in FP16) with FP32 accumulation; softmax weights are rounded to FP16
 * for the value contraction; the sums run in FP32.
 */
int smla_sparse_mla_decode(const void *q_bf16, const uint8_t *cache, int64_t num_pages,
                           const int32_t *page_table, int32_t max_pages,
                           const int32_t *seq_lens, const int32_t *topk_indices,
                           int32_t batch, int32_t heads, int32_t topk, float softmax_scale,
                           float *out, float *lse, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * ---- Lean FP8 rows [P1 row-bytes table: FP8 row = 512 + 64 bytes] ----
 *
 * Row format (one token, 576 bytes): the 576 values (latent 0..511, then
 * rope 0..63) as OCP FP8 E4M3 bytes in dim order, no scale, each the E4M3
 * value nearest the input (ties to even, saturating at +-448, sign copied):
 * the rule of the NVFP4 row's rope bytes.  A page is 64 rows (36,864 bytes);
 * the cache is [num_pages][64][576] bytes.  K is the 576 decoded values, V
 * the first 512.
 *
 * The three calls below take the same arguments, with the same meaning,
 * conventions and errors, as their NVFP4 counterparts above; only the row
 * format of `cache` differs.  smla_decode_workspace_bytes_fp8 may differ from
 * the NVFP4 figure for the same shape (an FP8 split scans at most 1024
 * entries).
 */
int smla_kv_quant_append_fp8(const void *rows_bf16, int64_t n, const int32_t *slot_mapping,
                             uint8_t *cache, int64_t num_pages, void *stream);

size_t smla_decode_workspace_bytes_fp8(int32_t batch, int32_t heads, int32_t topk);

int smla_sparse_mla_decode_fp8(const void *q_bf16, const uint8_t *cache, int64_t num_pages,
                               const int32_t *page_table, int32_t max_pages,
                               const int32_t *seq_lens, const int32_t *topk_indices,
                               int32_t batch, int32_t heads, int32_t topk, float softmax_scale,
                               float *out, float *lse, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * ---- Staged path (ablation of the fused decode) [P1 section "A kernel
 * that reads four bits directly", the staged-vs-native figure and the
 * paragraph before it; P3, the first implementation] ----
 *
 * smla_stage_rows_fp8 is the staged path's gather-unpack: it reads the
 * selected NVFP4 rows and writes a lean FP8 copy of each to HBM, where
 * smla_sparse_mla_decode_fp8 then reads it.  The two calls together move
 * 352 + 576 + 576 bytes per selected row, against 352 for the fused
 * smla_sparse_mla_decode; they exist to measure that difference.
 *
 *   cache .. topk       as for smla_sparse_mla_decode (an NVFP4 cache);
 *                       entry usability follows the same rule
 *   staged              [batch * kpad / 64][64][576] uint8, device, 256-B
 *                       aligned, kpad = topk rounded up to a multiple of 64.
 *                       Usable entry e of sequence b is written to row
 *                       b * kpad + e: each of its 576 decoded values as the
 *                       E4M3 byte nearest it (ties to even, saturating at
 *                       +-448; the rope bytes are copied).  Rows of unusable
 *                       entries are not written.
 *   staged_topk         [batch][topk] int32, device: e for a usable entry,
 *                       -1 otherwise
 *
 * Attention over the copy is smla_sparse_mla_decode_fp8 with cache =
 * staged (num_pages = batch * kpad / 64), page_table [batch][kpad / 64]
 * holding b * kpad / 64 + p, seq_lens all kpad, and topk_indices =
 * staged_topk.  Errors: SMLA_ERR_SHAPE (batch not in [1, 65535], topk not in
 * [1, 2048], max_pages < 1, num_pages not in [1, 2^25]), SMLA_ERR_NULL,
 * SMLA_ERR_ALIGN (cache or staged not 256-B aligned, an int32 array not 4-B
 * aligned), SMLA_ERR_DEVICE, SMLA_ERR_LAUNCH.  Asynchronous on `stream`;
 * nothing is allocated.
 */
int smla_stage_rows_fp8(const uint8_t *cache, int64_t num_pages, const int32_t *page_table,
                        int32_t max_pages, const int32_t *seq_lens, const int32_t *topk_indices,
                        int32_t batch, int32_t topk, uint8_t *staged, int32_t *staged_topk,
                        void *stream);

/*
 * ---- Multi-token decode [P5 section 4, "The deployment, spelled out": MTP
 * speculative decoding with three draft tokens; P1 section "A kernel that
 * reads four bits directly": several query tokens per launch] ----
 *
 * `tokens` query tokens per sequence (the accepted token and its drafts),
 * each with its own top-k list, over the same NVFP4 cache and page table.
 * Token j (0-based) of sequence b sits at position seq_lens[b] - tokens + j
 * and sees positions [0, seq_lens[b] - (tokens - 1 - j)): an entry at or past
 * that is skipped like any out-of-range entry.  With tokens = 1 this is
 * smla_sparse_mla_decode.  All tokens of a sequence run on one XCD, so rows
 * that several of its tokens select are read from that XCD's L2.
 *
 *   q             [batch][tokens][heads][576] bf16
 *   page_table    [batch][max_pages], seq_lens [batch]: per sequence, as above
 *   topk_indices  [batch][tokens][topk] int32
 *   out, lse      [batch][tokens][heads][512] fp32, [batch][tokens][heads] fp32
 *   workspace     smla_decode_workspace_bytes_mtp(batch, tokens, heads, topk)
 *
 * Errors as smla_sparse_mla_decode; SMLA_ERR_SHAPE also for tokens not in
 * [1, 16] or batch * tokens > 65535.
 */
size_t smla_decode_workspace_bytes_mtp(int32_t batch, int32_t tokens, int32_t heads,
                                       int32_t topk);

int smla_sparse_mla_decode_mtp(const void *q_bf16, const uint8_t *cache, int64_t num_pages,
                               const int32_t *page_table, int32_t max_pages,
                               const int32_t *seq_lens, const int32_t *topk_indices,
                               int32_t batch, int32_t tokens, int32_t heads, int32_t topk,
                               float softmax_scale, float *out, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * ---- Top-k select [P1 section "Decode: TP4, and the copies it keeps": an
 * indexer picks the top cached positions, at most 2,048 per query; the
 * prefill-timing figure lists the indexer's logits and top-k as separate
 * steps] ----
 *
 * The step upstream of the decode: for each query b, the positions of the
 * min(topk, L_b) largest of scores[b][0 .. L_b), then -1 up to topk, as the
 * decode's topk_indices.  L_b = seq_lens[b] clamped to [0, ld].  The order of
 * the list, and which of several equal scores at the threshold are taken,
 * are unspecified (the set of scores taken is always the top min(topk, L_b)).
 * Scores must be finite; -0 counts as just below +0.
 *
 *   scores        [batch][ld] fp32, device, 16-B aligned, ld a multiple of 4
 *   seq_lens      [batch] int32, device
 *   topk_indices  [batch][topk] int32, device (output)
 *   workspace     smla_topk_workspace_bytes(batch, ld) bytes, 256-B aligned.
 *                 It must be zero-filled before its first use; every call
 *                 leaves it all zero again, ready for a call of any shape.
 *                 Calls that share a workspace must not overlap.
 *
 * Errors: SMLA_ERR_SHAPE (batch not in [1, 65535], topk not in [1, 2048], ld
 * not a multiple of 4 in [4, 2^30]), SMLA_ERR_NULL, SMLA_ERR_ALIGN,
 * SMLA_ERR_WORKSPACE (missing or short), SMLA_ERR_DEVICE, SMLA_ERR_LAUNCH.
 * Asynchronous on `stream`; three kernel launches; nothing is allocated.
 */
size_t smla_topk_workspace_bytes(int32_t batch, int64_t ld);

int smla_topk_select(const float *scores, int64_t ld, const int32_t *seq_lens, int32_t batch,
                     int32_t topk, int32_t *topk_indices, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * ---- Append and decode in one launch [P1 section "A kernel that reads four
 * bits directly" (the decode); section "Four bits per latent value: where
 * 352 comes from" (the row the append writes)] ----
 *
 * One decode step of sequences that each gained one token: the result, in
 * the cache and in out/lse, is exactly that of
 *   smla_kv_quant_append(new_rows_bf16, batch, new_slots, cache, num_pages),
 * then smla_sparse_mla_decode(q_bf16, cache, ..., softmax_scale, out, lse),
 * in one kernel launch (plus the split merge): every decode workgroup of
 * sequence b quantises new row b itself and reads it from LDS wherever its
 * list translates to slot new_slots[b]; one workgroup per sequence writes
 * the row to the cache.
 *
 *   new_rows_bf16  [batch][576] BF16, device, 16-B aligned: row b is
 *                  sequence b's newest token (latent 512 + rope 64)
 *   new_slots      [batch] int32, device: page * 64 + row of the cache slot
 *                  it goes to; a slot outside [0, num_pages * 64) skips the
 *                  row (as the append does)
 *   the rest       as for smla_sparse_mla_decode (seq_lens already count
 *                  the new token); workspace as sized by
 *                  smla_decode_workspace_bytes(batch, heads, topk)
 *
 * The slots of the new rows must be distinct, and slot new_slots[b] must be
 * read, through the page table, by no list but sequence b's (the page that
 * receives a sequence's newest token belongs to that sequence alone).
 * Errors: those of the two calls it stands for.  Asynchronous on `stream`.
 */
int smla_append_decode(const void *new_rows_bf16, const int32_t *new_slots, const void *q_bf16,
                       uint8_t *cache, int64_t num_pages, const int32_t *page_table,
                       int32_t max_pages, const int32_t *seq_lens, const int32_t *topk_indices,
                       int32_t batch, int32_t heads, int32_t topk, float softmax_scale, float *out,
                       float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * ---- Decode that allocates nothing, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc) ----
 *
 * smla_sparse_mla_decode with the same arguments, meaning, conventions and
 * errors, minus the workspace: the split partials go to a scratch array the
 * library holds in device memory (a static device array of
 * SMLA_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, kept until the
 * process ends).  The call performs no allocation of any kind.  A shape
 * whose split partials need more than SMLA_NOALLOC_SCRATCH_BYTES (that is,
 * smla_decode_workspace_bytes(batch, heads, topk) > SMLA_NOALLOC_SCRATCH_BYTES)
 * is refused with SMLA_ERR_SCRATCH before anything is launched; every other
 * shape smla_sparse_mla_decode takes is accepted, with bit-identical results.
 *
 * All calls on one GPU share that GPU's scratch array: two calls that
 * overlap in time on the same GPU (different streams, or different host
 * threads without ordering) race on it and give undefined results.  Calls
 * ordered on one stream are safe.  The first call on a device looks up the
 * array's device address (once per device, cached); that lookup can return
 * SMLA_ERR_DEVICE.
 */
#define SMLA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

int smla_sparse_mla_decode_noalloc(const void *q_bf16, const uint8_t *cache, int64_t num_pages,
                                   const int32_t *page_table, int32_t max_pages,
                                   const int32_t *seq_lens, const int32_t *topk_indices,
                                   int32_t batch, int32_t heads, int32_t topk,
                                   float softmax_scale, float *out, float *lse, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SMLA_H */
