// sparse_mla_decode for queries of 64 heads: one workgroup serves all 64 heads
// of a (query, split), so each selected row is unpacked once for the scores
// and once for the values, whatever the head count.
//
// What it computes is the decode of sparse_mla_decode.hip: "Prime Inference:
// serving GLM-5.3 to agents is a KV-cache problem", section "A kernel that
// reads four bits directly" (load the selected 352-byte rows, unpack on chip,
// score, softmax and blend; -1 entries carry no data) and Prime Intellect's
// launch post, native-kernel paragraph (FP16 operands, FP32 accumulation;
// the blocks sharing a query merge their partial results).  Every selected
// row serves all heads of the query ("GLM-5.3 PCP/DCP long-context on
// H200", section 1): at 64 heads a row carries 64 x 2,176 FLOPs against its
// 352 bytes, which puts the kernel on the FP16 matrix-core roof of gfx950.
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, 64-wide waves, 160 KB LDS):
//   * one 512-thread workgroup per (query, split) and CU; a split is a slice
//     of at most 1024 list entries.  Waves 0-3 score, waves 4-7 contract
//     values, one of each kind per SIMD;
//   * the query of 64 heads x 576 values does not fit one wave's registers
//     (288 of them), so score wave w = dh + 2 rh holds the 64 heads over
//     half of the dims (dh: latent 256 dh .. +256 and rope 32 dh .. +32, 144
//     registers) and scores rows 32 rh .. 32 rh + 31 of every 64-row tile
//     over those dims: MFMA 32x32x16 f16 with the unpacked rows as the A
//     operand and the query as B, so a lane's accumulators hold 16 rows of
//     one head.  Each row is unpacked exactly once.  The two waves sharing
//     rh then swap the halves of the partial scores they do not finalise
//     through LDS (16 KB per tile), and wave (dh, rh) finalises the scores,
//     softmax weights and running max of heads 32 dh .. 32 dh + 31;
//   * a step has two phases, split by a barrier M(s): in phase 1 the score
//     waves unpack and score tile s while the value waves contract the first
//     32 rows of tile s - 1; in phase 2 the score waves add the partner
//     halves (written before M(s)) and finish the softmax of tile s while the
//     value waves contract the other 32 rows -- so the matrix pipe of a SIMD
//     has the value wave's work while its score wave is in the softmax;
//   * value wave v owns output columns 128 v .. 128 v + 127 of all 64 heads
//     (128 accumulator registers): the transposing 4-bit LDS read hands a
//     lane 16 rows of one column still packed, unpacked and scaled once for
//     both 32-head halves of MFMA 32x32x16 f16;
//   * rows travel HBM -> LDS still packed by direct-to-LDS loads issued by
//     the value waves, three tiles ahead, in a ring of five 22.5 KB slots;
//   * online softmax as in the 16/32-head kernel: the first tile sets the
//     running max, later tiles move it only when a score passes it by more
//     than kSlack (log2 units), and then the tile is re-weighted from its kept
//     scores one step later; the weight sums are kept by the score waves;
//   * the splits of a query write normalised f16 partials with (max, sum),
//     which the merge kernel of sparse_mla_decode.hip combines.
#include "smla_internal.h"
#include "decode_device.h"

namespace smla {
namespace {

using namespace dev;

constexpr int kThreads = 512;
constexpr int kTile = 64;
constexpr int kHeads = 64;
constexpr int kKSteps = kDim / 32;             // 18 score k-steps of 16 dims per lane half
constexpr float kSlack = 8.0f;                 // log2 headroom before the running max moves
constexpr int kNBuf = 5;                       // ring slots
constexpr int kAhead = 3;                      // tile s + 3 is loaded in step s
constexpr int kTileBytes = kTile * kRowBytes;  // 22,528
constexpr int kDmaPerTile = kTileBytes / 1024; // 22 wave-wide 16-byte loads per tile
constexpr int kMaxDma = (kDmaPerTile + 3) / 4; // 6 per value wave
constexpr int kPStride = kTile + 8;            // f16 per weight row (one head)
constexpr int kSStride = kTile + 8;            // f16 per scale-table row (one block)
constexpr int kMaxPerSplit = 1024;             // list entries one workgroup scans

// LDS layout (bytes).  The query is staged at the start through ring slots
// 3-4, the exchange area and the weight tiles, which hold nothing before the
// first step.
constexpr int kRingOff = 0;
constexpr int kXOff = kRingOff + kNBuf * kTileBytes;            // 112,640
constexpr int kXBytes = 4 * 4096;                               // (rh, hb) x 64 lanes x 16 floats
constexpr int kPOff = kXOff + kXBytes;                          // 129,024
constexpr int kPBytes = 2 * kHeads * kPStride * 2;              // 18,432 (two tiles)
constexpr int kStOff = kPOff + kPBytes;                         // 147,456
constexpr int kStBytes = 2 * 32 * kSStride * 2;                 // 9,216
constexpr int kRowIdOff = kStOff + kStBytes;                    // 156,672
constexpr int kSmallOff = kRowIdOff + kMaxPerSplit * 4;         // 160,768
constexpr int kQOff = 3 * kTileBytes;                           // 67,584
constexpr int kQBytes = kHeads * kDim * 2;                      // 73,728
static_assert(kQOff + kQBytes <= kRowIdOff, "the query staging must end before the row ids");
static_assert(kXOff % 1024 == 0 && kPOff % 16 == 0 && kStOff % 16 == 0, "alignment");

// the small area
struct Small {
    uint32_t flags[4];        // per score wave: a score of the last tile passed max + slack
    float red[4][32];         // per score wave: the last tile's max per head
    float first[2][kHeads];   // first tile: per row half, max per head
    float alpha[kHeads];      // rescale factors when the running max moved
    float sum[2][kHeads];     // per row half, weight sums per head
    float m[kHeads];          // final running max per head (log2 units)
    int32_t scan[4];          // prologue: usable entries per value wave
};
static_assert(kSmallOff + (int)sizeof(Small) <= 160 * 1024, "LDS budget");
static_assert(kQOff + kQBytes <= kStOff, "the query staging must end before the scale tables");

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_h64_kernel(const uint16_t *__restrict__ q, const uint8_t *__restrict__ cache,
                       int64_t num_pages, const int32_t *__restrict__ page_table,
                       int32_t max_pages, const int32_t *__restrict__ seq_lens,
                       const int32_t *__restrict__ topk_idx, int32_t topk, float scale_log2,
                       float *__restrict__ out, float *__restrict__ lse,
                       _Float16 *__restrict__ part_o, float *__restrict__ part_ml, int32_t batch,
                       int32_t tokens, int32_t splits, int32_t per_split) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmallOff + sizeof(Small)];
    uint8_t *const ring = smem + kRingOff;
    Small &sm = *reinterpret_cast<Small *>(smem + kSmallOff);
    uint32_t *const rowid_lds = reinterpret_cast<uint32_t *>(smem + kRowIdOff);
    const uint32_t smem_addr = (uint32_t)(size_t)(lds_void_t *)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31;
    const int g = lane >> 5;

    // ---- (query, split): consecutive workgroups go to consecutive XCDs, so
    // every split and query token of sequence sq runs on XCD sq % 8.  Query
    // b is token j of sequence sq = b / tokens and sees positions
    // [0, seq_lens[sq] - (tokens - 1 - j)) ----
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int rest = id >> 3;
    const int split = rest % splits;
    const int r_seq = rest / splits;
    const int sq = (r_seq / tokens) * 8 + xcd;
    if (sq >= batch) return;
    const int b = sq * tokens + r_seq % tokens;
    const int e_begin = split * per_split;
    const int e_end = min(topk, e_begin + per_split);

    auto count_valid = [&]() {
        return __builtin_amdgcn_readfirstlane(sm.scan[0] + sm.scan[1] + sm.scan[2] + sm.scan[3]);
    };
    auto slot_addr = [&](int T) { return (uint32_t)((T % kNBuf) * kTileBytes); };
    uint8_t *const xch = smem + kXOff;
    _Float16 *const p_lds = reinterpret_cast<_Float16 *>(smem + kPOff);
    _Float16 *const st_lds = reinterpret_cast<_Float16 *>(smem + kStOff);

    if (wave < 4) {
        // =========================== score waves ===========================
        const int dh = wave & 1;          // dims half
        const int rh = wave >> 1;         // row half of each tile
        const int G = 2 * dh + g;         // this lane's 128 latent + 16 rope dims
        const int head = 32 * dh + n32;   // the head whose softmax this lane finalises
        // The query of 64 heads goes HBM -> LDS once: load i = (2 dh' + hb) * 18 + j
        // puts, for lane l, the B operand of score k-step j of head
        // 32 hb + l % 32 over the dims of group 2 dh' + l / 32 into 1 KB.
        {
            const uint32_t q_lds = smem_addr + kQOff;
            for (int i = wave; i < 4 * kKSteps; i += 4) {
                const int dq = i / (2 * kKSteps), hb = (i / kKSteps) & 1, j = i % kKSteps;
                const int Gq = 2 * dq + g;
                const int d0 = (j < 16) ? (128 * Gq + 8 * j) : (512 + 16 * Gq + 8 * (j - 16));
                dma16(q + ((int64_t)b * kHeads + 32 * hb + n32) * kDim + d0, q_lds + (uint32_t)i * 1024u);
            }
        }
        __syncthreads();                                             // P1: counts published
        const int n_valid = count_valid();
        const int n_tiles = (n_valid + kTile - 1) / kTile;
        __syncthreads();                                             // P2: row ids in LDS
        wait_vmcnt_n<0>();
        __syncthreads();                                             // Q: query and tile 0 landed
        half8_t qb[2][kKSteps];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int j = 0; j < kKSteps; ++j) {
                const uint4 v = *reinterpret_cast<const uint4 *>(
                    smem + kQOff + ((2 * dh + hb) * kKSteps + j) * 1024 + 16 * lane);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                half2_t h[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) h[k] = bf16x2_to_f16x2(w4[k]);
                qb[hb][j] = join(h[0], h[1], h[2], h[3]);
            }

        // this lane's packed bytes of a tile: row 32 rh + n32, nibbles of dims
        // 128 G .. +128, their 8 block scales, rope dims 16 G .. +16 (the
        // 16-byte pieces of row r sit swapped by nv_swz(r))
        const int row = 32 * rh + n32;
        int nib_off[4];
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) nib_off[jp] = row * kRowBytes + 16 * ((4 * G + jp) ^ nv_swz(row));
        const int sc_off = row * kRowBytes + 16 * ((kScaleOff / 16 + (G >> 1)) ^ nv_swz(row)) + 8 * (G & 1);
        const int rope_off = row * kRowBytes + 16 * ((kRopeOff / 16 + G) ^ nv_swz(row));
        struct Packed {
            uint4 nib[4];
            uint2 sc;
            uint4 rope;
        };
        // the {S, S} f16 pairs of the lane's 8 block scales (E4M3 -> f16, exact)
        auto scale_pairs = [&](const uint2 &sc, half2_t (&sp)[8]) {
            const uint32_t d0 = __builtin_amdgcn_perm(0u, sc.x, 0x01010000u);
            const uint32_t d1 = __builtin_amdgcn_perm(0u, sc.x, 0x03030202u);
            const uint32_t d2 = __builtin_amdgcn_perm(0u, sc.y, 0x01010000u);
            const uint32_t d3 = __builtin_amdgcn_perm(0u, sc.y, 0x03030202u);
            sp[0] = fp8x2<false>(d0); sp[1] = fp8x2<true>(d0);
            sp[2] = fp8x2<false>(d1); sp[3] = fp8x2<true>(d1);
            sp[4] = fp8x2<false>(d2); sp[5] = fp8x2<true>(d2);
            sp[6] = fp8x2<false>(d3); sp[7] = fp8x2<true>(d3);
        };
        auto load_packed = [&](int T, Packed &pk) {
            const uint8_t *tb = ring + slot_addr(T);
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) pk.nib[jp] = *reinterpret_cast<const uint4 *>(tb + nib_off[jp]);
            pk.sc = *reinterpret_cast<const uint2 *>(tb + sc_off);
            pk.rope = *reinterpret_cast<const uint4 *>(tb + rope_off);
        };

        // running max of `head` (log2 units; set by the first tile), the
        // weight sum of this lane's rows (tiles before the last weighted),
        // the weight sum and d = score - max of the tile last weighted (kept
        // for a re-weight in the next step)
        float m_run = 0.0f, lsum = 0.0f, ls_prev = 0.0f;
        float dk[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) dk[i] = 0.0f;

        // f16 weights 2^dk of this lane's rows 4 r4 .. 4 r4 + 3 into the
        // weight tile [head][row] of tile T (rows 32 rh + 8 r4 + 4 g + 0..3)
        auto weights4 = [&](int T, int r4, float &sum) {
            _Float16 *prow = p_lds + ((T & 1) * kHeads + head) * kPStride + 32 * rh + 4 * g + 8 * r4;
            float e[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                e[k] = __builtin_amdgcn_exp2f(dk[4 * r4 + k]);
                sum += e[k];
            }
            *reinterpret_cast<half4_t *>(prow) =
                half4_t{(_Float16)e[0], (_Float16)e[1], (_Float16)e[2], (_Float16)e[3]};
        };
        auto tile_max = [&]() {
            float mx = fmaxf(fmaxf(fmaxf(dk[0], dk[1]), fmaxf(dk[2], dk[3])),
                             fmaxf(fmaxf(dk[4], dk[5]), fmaxf(dk[6], dk[7])));
            return fmaxf(mx, fmaxf(fmaxf(fmaxf(dk[8], dk[9]), fmaxf(dk[10], dk[11])),
                                   fmaxf(fmaxf(dk[12], dk[13]), fmaxf(dk[14], dk[15]))));
        };
        // maximum over the two lane halves (which hold the other 16 rows of
        // the same head)
        auto halves_max = [&](float mx) { return fmaxf(mx, __shfl_xor(mx, 32, 64)); };

        // the packed bytes of tile s are read in phase 2 of step s - 1 (tile
        // s is complete from M(s - 1) on), so that the read's latency falls
        // under the softmax instead of at the head of step s
        Packed pk;
        if (n_tiles > 0) load_packed(0, pk);
        for (int s = 0; s <= n_tiles; ++s) {
            __syncthreads();                                                 // B(s)
            // ---- phase 1 ----
            const uint4 fl = *reinterpret_cast<const uint4 *>(&sm.flags[0]);
            // (a) tile s - 1 moved the running max (rare): new max from the
            // flagged waves' maxima (an unflagged wave's scores lie within
            // kSlack of the old max), re-weight that tile from its kept d,
            // publish the rescale factors; the value waves rescale O after S(s)
            if (s >= 1 && __builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w) != 0) {
                const uint32_t f0 = dh == 0 ? fl.x : fl.y, f1 = dh == 0 ? fl.z : fl.w;
                const float mt = fmaxf(m_run, fmaxf(f0 ? sm.red[dh][n32] : -INFINITY,
                                                    f1 ? sm.red[dh + 2][n32] : -INFINITY));
                const float shift = m_run - mt;  // <= 0
                const float alpha = __builtin_amdgcn_exp2f(shift);
                if (rh == 0 && g == 0) sm.alpha[head] = alpha;
                m_run = mt;
                lsum *= alpha;
#pragma unroll
                for (int i = 0; i < 16; ++i) dk[i] += shift;
                ls_prev = 0.0f;
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) weights4(s - 1, r4, ls_prev);
                __syncthreads();                                             // S(s)
            }
            if (s >= 1) lsum += ls_prev;
            float16_t keep;
            if (s < n_tiles) {
                // (b) tile s: block scales, unpack, score over this wave's dims
                half2_t sp[8];
                scale_pairs(pk.sc, sp);
                float16_t acc[2];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[hb][i] = 0.0f;
                // k-step j's B operand is unpacked during step j - 1's two
                // MFMAs (half after each), so the unpack runs under the
                // matrix pipe instead of between its instructions
                auto unpack2 = [&](int j, int h) {   // dims 8 j + 4 h .. + 4 of the lane's group
                    if (j < 16) {
                        const uint32_t w = pk.nib[j >> 2][j & 3];
                        const half2_t sv = sp[j >> 1];
                        return h == 0 ? join2(fp4x2<0>(w) * sv, fp4x2<1>(w) * sv)
                                      : join2(fp4x2<2>(w) * sv, fp4x2<3>(w) * sv);
                    }
                    const uint32_t r = pk.rope[2 * (j - 16) + h];
                    return join2(fp8x2<false>(r), fp8x2<true>(r));
                };
                half4_t kl = unpack2(0, 0), kh = unpack2(0, 1);
#pragma unroll
                for (int j = 0; j < kKSteps; ++j) {
                    const half8_t kb = join4(kl, kh);
                    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb, qb[0][j], acc[0], 0, 0, 0);
                    if (j + 1 < kKSteps) kl = unpack2(j + 1, 0);
                    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb, qb[1][j], acc[1], 0, 0, 0);
                    if (j + 1 < kKSteps) kh = unpack2(j + 1, 1);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // 4 VALU
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // 4 VALU
                }
                // the partner's head block to the exchange area; this block kept
                float4_t *xw = reinterpret_cast<float4_t *>(xch + ((rh * 2 + (1 - dh)) * 4096) + 16 * lane);
                const float16_t &send = dh == 0 ? acc[1] : acc[0];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    xw[64 * r4] = float4_t{send[4 * r4], send[4 * r4 + 1], send[4 * r4 + 2], send[4 * r4 + 3]};
                keep = dh == 0 ? acc[0] : acc[1];
            }
            __syncthreads();                                                 // M(s)
            // ---- phase 2: softmax of tile s from both dims halves ----
            if (s >= n_tiles) continue;
            // tile s's block scales, transposed [block][row] for the value
            // waves (they read them in step s + 1); zero for the last tile's
            // padding rows (row 0 of page 0), so that their bytes cannot
            // reach the output
            {
                half2_t sp[8];
                scale_pairs(pk.sc, sp);
                const bool real = (s + 1) * kTile <= n_valid || s * kTile + row < n_valid;
                _Float16 *sc = st_lds + (s & 1) * 32 * kSStride + row;
#pragma unroll
                for (int k = 0; k < 8; ++k) sc[(8 * G + k) * kSStride] = real ? sp[k][0] : (_Float16)0.0f;
            }
            if (s + 1 < n_tiles) load_packed(s + 1, pk);
            {
                const float4_t *xr = reinterpret_cast<const float4_t *>(xch + ((rh * 2 + dh) * 4096) + 16 * lane);
                float4_t x[4];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) x[r4] = xr[64 * r4];
                const float mr = s == 0 ? 0.0f : m_run;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = 32 * rh + 8 * (i >> 2) + 4 * g + (i & 3);
                    const float v = fmaf(keep[i] + x[i >> 2][i & 3], scale_log2, -mr);
                    dk[i] = s * kTile + r < n_valid ? v : -INFINITY;
                }
            }
            float mx = tile_max();
            if (s == 0) {
                // the first tile sets the running max: both row halves'
                // maxima through LDS and one extra barrier F
                mx = halves_max(mx);
                if (g == 0) sm.first[rh][head] = mx;
                __syncthreads();                                             // F
                m_run = fmaxf(sm.first[0][head], sm.first[1][head]);
#pragma unroll
                for (int i = 0; i < 16; ++i) dk[i] -= m_run;
            } else {
                // a flag per wave (a score passed the running max by more
                // than kSlack); only a flagged wave (rare) publishes its tile
                // maxima per head
                const bool flagged = __ballot(mx > kSlack) != 0;
                if (lane == 0) sm.flags[wave] = flagged;
                if (flagged) {
                    mx = halves_max(mx);
                    if (g == 0) sm.red[wave][n32] = mx + m_run;
                }
            }
            ls_prev = 0.0f;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) weights4(s, r4, ls_prev);
        }
        // weight sums of this wave's 32 rows per head, and the running max
        lsum += __shfl_xor(lsum, 32, 64);
        if (g == 0) {
            sm.sum[rh][head] = lsum;
            if (rh == 0) sm.m[head] = m_run;
        }
        __syncthreads();                                                     // E
        return;
    }

    // ---- prologue (value waves): validate, translate and compact the
    // split's entries into LDS (list order kept).  All index loads are issued
    // before any is used; an entry outside its range reads a harmless
    // in-range word instead.  Thread v = tid - 256 takes entries
    // [v per_thread, (v + 1) per_thread) ----
    const int per_thread = (per_split + 255) / 256;  // <= 4
    uint32_t rid[4];
    int cnt_valid = 0, incl = 0;
    {
        const int vt = tid - 256;
        const int64_t L = (int64_t)seq_lens[sq] - (tokens - 1 - (b - sq * tokens));
        int32_t tv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = e_begin + vt * per_thread + i;
            tv[i] = (i < per_thread) ? topk_idx[(int64_t)b * topk + min(e, topk - 1)] : -1;
        }
        bool ok[4];
        int32_t pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = e_begin + vt * per_thread + i;
            const int64_t t = tv[i];
            ok[i] = i < per_thread && e < e_end && t >= 0 && t < L && (t >> 6) < max_pages;
            pv[i] = page_table[(int64_t)sq * max_pages + (ok[i] ? (t >> 6) : 0)];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t page = pv[i];
            rid[i] = (ok[i] && page >= 0 && page < num_pages) ? (uint32_t)(page * kPageRows + (tv[i] & 63))
                                                              : 0xFFFFFFFFu;
            cnt_valid += rid[i] != 0xFFFFFFFFu;
        }
        incl = cnt_valid;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d, 64);
            if (lane >= d) incl += v;
        }
        if (lane == 63) sm.scan[wave - 4] = incl;
        // no tile has flagged a running-max move yet (tile 0 never writes
        // its flags: it sets the max)
        if (vt < 4) sm.flags[vt] = 0u;
    }
    __syncthreads();                                                         // P1
    const int n_valid = count_valid();
    const int n_tiles = (n_valid + kTile - 1) / kTile;
    const int n_pad = n_tiles * kTile;
    {
        int pos = incl - cnt_valid;
#pragma unroll
        for (int w = 0; w < 3; ++w) pos += (w < wave - 4) ? sm.scan[w] : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (rid[i] != 0xFFFFFFFFu) rowid_lds[pos++] = rid[i];
        // the last tile is padded with row 0 of page 0 (always in the cache);
        // the padding rows get zero weight and zero block scales
        if (tid - 256 < n_pad - n_valid) rowid_lds[n_valid + tid - 256] = 0u;
    }
    __syncthreads();                                                         // P2

    // =========================== value waves ===========================
    const int v = wave - 4;
    // tile loads: wave v issues the wave-wide loads i = v, v + 4, ...: load i
    // fills LDS bytes [1024 i, 1024 i + 1024) of the tile slot, lane l the
    // 16-byte piece (64 i + l) % 22 of row (64 i + l) / 22, taken from piece
    // ((64 i + l) % 22) ^ nv_swz(row) of the cache row
    const int n_dma = (kDmaPerTile - v + 3) / 4;   // 6 or 5
    int dma_ro[kMaxDma];   // row in the tile << 16 | byte offset in the cache row
#pragma unroll
    for (int k = 0; k < kMaxDma; ++k) {
        const int sl = 64 * (v + 4 * k) + lane;
        const int r = min(sl / 22, kTile - 1);
        dma_ro[k] = (r << 16) | (16 * ((sl % 22) ^ nv_swz(r)));
    }
    auto tile_rows = [&](int T, uint32_t (&rk)[kMaxDma]) {
        const uint32_t *rows = rowid_lds + T * kTile;
#pragma unroll
        for (int k = 0; k < kMaxDma; ++k) rk[k] = rows[dma_ro[k] >> 16];
    };
    auto tile_dma_part = [&](int T, const uint32_t (&rk)[kMaxDma], int k0, int k1) {
        const uint32_t dst = smem_addr + slot_addr(T) + (uint32_t)(v * 1024);
#pragma unroll
        for (int k = 0; k < kMaxDma; ++k)
            if (k >= k0 && k < k1 && k < n_dma)
                dma16(cache + (size_t)rk[k] * kRowBytes + (dma_ro[k] & 0xFFFF), dst + (uint32_t)(k * 4 * 1024));
    };
    // tile t is in LDS once at most the loads of the tiles issued after it
    // are outstanding (`after` of them, 0..2)
    auto wait_tile = [&](int after) {
        if (after <= 0) wait_vmcnt_n<0>();
        else if (after == 1) { if (n_dma == 6) wait_vmcnt_n<6>(); else wait_vmcnt_n<5>(); }
        else { if (n_dma == 6) wait_vmcnt_n<12>(); else wait_vmcnt_n<10>(); }
    };

    // tiles 0 and 1 now; tile 0 complete before Q (the score waves read it
    // right after B(0))
    {
        uint32_t rk[kMaxDma];
        for (int T = 0; T <= 1 && T < n_tiles; ++T) {
            tile_rows(T, rk);
            tile_dma_part(T, rk, 0, kMaxDma);
        }
        if (n_tiles > 0) wait_tile(n_tiles > 1 ? 1 : 0);
    }
    __syncthreads();                                                         // Q

    // O[hb][cb] (MFMA 32x32x16 C layout): head 32 hb + 8 (i/4) + 4 g + i%4,
    // column 128 v + 32 cb + n32.  A tile's rows enter MFMA (rb, t) as
    // k = rows 32 rb + 16 g + 8 t + i.
    float16_t o[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[hb][cb][i] = 0.0f;
    // packed values of the tile awaiting contraction: lanes 16 G'..16 G'+15
    // read 8 bytes = 16 columns of rows 32 rb + 16 (G'/2) + 0..15; lane j of
    // the group receives column j of those rows (ds_read_b64_tr_b4)
    int2_t vv[4][2];
    const uint32_t v_lane = (uint32_t)((16 * g + (lane & 15)) * kRowBytes + 64 * v + 8 * ((lane >> 4) & 1));
    auto read_values = [&](int T, int rb) {
        // piece 4 v + cb of row r sits at 4 v + (cb ^ nv_swz(r)); rows
        // 16 g + lane % 16 and those 32 further have the same nv_swz
        const uint8_t *tb = ring + slot_addr(T);
        const uint8_t *vb0 = tb + v_lane + 16 * nv_swz(lane & 15);
        const uint8_t *vb1 = tb + v_lane + 16 * (1 - nv_swz(lane & 15));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            vv[cb][rb] = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_int2_t *)(
                (__attribute__((address_space(3))) const uint8_t *)((cb & 1 ? vb1 : vb0) + 32 * rb * kRowBytes +
                                                                     32 * (cb >> 1))));
    };
    // lane parts of the weight and scale-table addresses
    const int p_lane = n32 * kPStride + 16 * g;                    // f16 index
    const int s_lane = (8 * v + (n32 >> 4)) * kSStride + 16 * g;   // f16 index (block 8 v + 2 cb + n32/16)

    // MFMAs of row groups rt0 .. rt1 - 1 (rows 32 rb + 16 g + 8 t ..) of the
    // tile whose packed values are in registers; each group's weights and
    // block scales are read one group ahead: pa_n and sv_n hold group rt0's
    // on entry and group rt1's (from weights pw, scales sw_next) on exit
    half8_t pa_n[2], sv_n[4];
    auto read_pa = [&](const _Float16 *pw, int rt, half8_t (&pa)[2]) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
            pa[hb] = *reinterpret_cast<const half8_t *>(pw + hb * 32 * kPStride + 32 * (rt >> 1) + 8 * (rt & 1));
    };
    auto read_sv = [&](const _Float16 *sw, int rt, half8_t (&sv)[4]) {
        const int off = 32 * (rt >> 1) + 8 * (rt & 1);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            sv[cb] = *reinterpret_cast<const half8_t *>(sw + 2 * cb * kSStride + off);
    };
    // half (h = 0: rows 0..3, h = 1: rows 4..7 of the group) of the B
    // operand of row group rt and column block cb: 4-bit values to f16,
    // times each row's block scale
    auto unpack_v = [&](int rt, int cb, const half8_t &ss, int h) {
        const uint32_t w = (uint32_t)vv[cb][rt >> 1][rt & 1];
        const half2_t sa = {ss[4 * h], ss[4 * h + 1]}, sb = {ss[4 * h + 2], ss[4 * h + 3]};
        return h == 0 ? join2(fp4x2<0>(w) * sa, fp4x2<1>(w) * sb) : join2(fp4x2<2>(w) * sa, fp4x2<3>(w) * sb);
    };
    auto contract = [&](const _Float16 *pw, const _Float16 *sw, int rt0, int rt1, const _Float16 *pw_next,
                        const _Float16 *sw_next, bool next) {
        half8_t sv[4], pa[2];
        half4_t vl = unpack_v(rt0, 0, sv_n[0], 0), vh = unpack_v(rt0, 0, sv_n[0], 1);
#pragma unroll
        for (int i = 4 * rt0; i < 4 * rt1; ++i) {
            const int rt = i >> 2, cb = i & 3;
            if (cb == 0) {
                // this row group's operands, the next group's on their way
#pragma unroll
                for (int k = 0; k < 4; ++k) sv[k] = sv_n[k];
#pragma unroll
                for (int k = 0; k < 2; ++k) pa[k] = pa_n[k];
                if (rt + 1 < rt1) {
                    read_sv(sw, rt + 1, sv_n);
                    read_pa(pw, rt + 1, pa_n);
                } else if (next) {
                    read_sv(sw_next, rt1 & 3, sv_n);
                    read_pa(pw_next, rt1 & 3, pa_n);
                }
            }
            // the B operand of column block cb is in (vl, vh); the next
            // block's is unpacked under this block's two MFMAs
            const half8_t vb = join4(vl, vh);
            const bool more = i + 1 < 4 * rt1;
            const int rn = (i + 1) >> 2, cn = (i + 1) & 3;
            const half8_t &sn = cn == 0 ? sv_n[0] : sv[cn];
            o[0][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[0], vb, o[0][cb], 0, 0, 0);
            if (more) vl = unpack_v(rn, cn, sn, 0);
            o[1][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[1], vb, o[1][cb], 0, 0, 0);
            if (more) vh = unpack_v(rn, cn, sn, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // 4 VALU
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // 4 VALU
        }
    };

    uint32_t rk[kMaxDma];   // row ids of the next tile to load
    for (int s = 0; s <= n_tiles; ++s) {
        __syncthreads();                                                     // B(s)
        // ---- phase 1 ----
        const uint4 fl = *reinterpret_cast<const uint4 *>(&sm.flags[0]);
        const bool prev = s >= 1;   // tile s - 1 to contract in this step
        if (prev && __builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w) != 0) {
            // tile s - 1 moved the running max: the score waves re-weight it
            // before S(s); O (tiles up to s - 2) is rescaled
            __syncthreads();                                                 // S(s)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float a = sm.alpha[32 * hb + 8 * (i >> 2) + 4 * g + (i & 3)];
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) o[hb][cb][i] *= a;
                }
        }
        const _Float16 *sw = st_lds + ((s - 1) & 1) * 32 * kSStride + s_lane;
        const _Float16 *pw = p_lds + ((s - 1) & 1) * kHeads * kPStride + p_lane;
        if (prev) {
            // operands of tile s - 1 (weights and block scales written in
            // phase 2 of step s - 1, packed values complete since M(s - 2)):
            // the first row group's weights and scales, both row blocks'
            // packed values
            read_pa(pw, 0, pa_n);
            read_sv(sw, 0, sv_n);
            read_values(s - 1, 0);
            read_values(s - 1, 1);
        }
        // the loads of tile s + 3 (s = 0: tiles 2 and 3) into the slot of
        // tile s - 2, issued while the operands are on their way
        for (int T = s == 0 ? 2 : s + kAhead; T <= s + kAhead && T < n_tiles; ++T) {
            tile_rows(T, rk);
            tile_dma_part(T, rk, 0, kMaxDma);
        }
        // tile s + 1 complete before M(s) (the score waves read it in phase
        // 2): tiles s + 2 and s + 3 may stay in flight
        if (s + 1 < n_tiles) wait_tile(min(2, n_tiles - 2 - s));
        __syncthreads();                                                     // M(s)
        // ---- phase 2: contract tile s - 1 while the score waves finish the
        // softmax of tile s ----
        if (s == 0 && n_tiles > 0) __syncthreads();                          // F
        if (prev) contract(pw, sw, 0, 4, pw, sw, false);
    }
    __syncthreads();                                                         // E

    // ---- epilogue: normalise and store (or publish the split's partial) ----
    const float ln2 = 0.69314718055994530942f;
    const int vt = tid - 256;
    if (splits == 1) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int h = 32 * hb + 8 * (i >> 2) + 4 * g + (i & 3);
                const float l_tot = sm.sum[0][h] + sm.sum[1][h];
                const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
                float *orow = out + ((int64_t)b * kHeads + h) * kLatent + 128 * v + n32;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) orow[32 * cb] = o[hb][cb][i] * inv;
            }
        if (vt < kHeads) {
            const float l_tot = sm.sum[0][vt] + sm.sum[1][vt];
            lse[(int64_t)b * kHeads + vt] = l_tot > 0.f ? (sm.m[vt] + log2f(l_tot)) * ln2 : -INFINITY;
        }
        return;
    }
    // split partial: part_o [query][split][64][4 v][32 n32][4 cb] f16 (a
    // head's 512 values in the value waves' register order, one 8-byte store
    // per head and lane), part_ml [query][split][64][2] = (max, sum).  The
    // partials bypass the L2 (non-temporal), which holds rows other
    // workgroups of this XCD may still read.
    const size_t pidx = (size_t)b * splits + split;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = 32 * hb + 8 * (i >> 2) + 4 * g + (i & 3);
            const float l_tot = sm.sum[0][h] + sm.sum[1][h];
            const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
            const half4_t x4 = {(_Float16)(o[hb][0][i] * inv), (_Float16)(o[hb][1][i] * inv),
                                (_Float16)(o[hb][2][i] * inv), (_Float16)(o[hb][3][i] * inv)};
            uint64_t *dst = reinterpret_cast<uint64_t *>(part_o) + (pidx * kHeads + h) * 128 + v * 32 + n32;
            __builtin_nontemporal_store(__builtin_bit_cast(uint64_t, x4), dst);
        }
    if (vt < kHeads) {
        part_ml[(pidx * kHeads + vt) * 2] = sm.m[vt];
        part_ml[(pidx * kHeads + vt) * 2 + 1] = sm.sum[0][vt] + sm.sum[1][vt];
    }
}

}  // namespace

int h64_max_per_split() { return kMaxPerSplit; }

hipError_t launch_decode_h64(const uint16_t *q, const uint8_t *cache, int64_t num_pages,
                             const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                             const int32_t *topk_idx, int32_t batch, int32_t tokens, int32_t topk,
                             float scale_log2, float *out, float *lse, _Float16 *part_o,
                             float *part_ml, int32_t splits, int32_t per_split, hipStream_t stream) {
    const int blocks = ((batch + 7) / 8) * 8 * tokens * splits;
    hipLaunchKernelGGL(decode_h64_kernel, dim3(blocks), dim3(kThreads), 0, stream, q, cache, num_pages,
                       page_table, max_pages, seq_lens, topk_idx, topk, scale_log2, out, lse, part_o,
                       part_ml, batch, tokens, splits, per_split);
    return hipGetLastError();
}

}  // namespace smla
