// sparse_mla_decode, NVFP4 rows, 32-head groups: one wave per SIMD, each an
// online-softmax decode of its own rows.
//
// What it computes: "Prime Inference: serving GLM-5.3 to agents is a
// KV-cache problem", section "A kernel that reads four bits directly" (load
// the selected 352-byte rows, unpack on chip, score, softmax and blend; -1
// entries carry no data) and Prime Intellect's launch post, native-kernel
// paragraph (FP16 operands, FP32 accumulation; the blocks sharing a query
// merge their partial results).  Every selected row serves all heads of the
// group: "GLM-5.3 PCP/DCP long-context on H200", section 1.
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, 64-wide waves, 160 KB LDS):
//   * one 256-thread workgroup per (query, 32-head group, split) and CU; the
//     split's list entries are dealt to its four waves in chunks of 32
//     (chunk c to wave c % 4), so -1 padding spreads evenly;
//   * each wave validates, translates and compacts its own entries (ballot
//     prefix counts, list order kept), loads its rows HBM -> LDS still packed
//     with direct-to-LDS 16-byte loads, two tiles ahead in a ring of three,
//     and runs the whole decode on them with no barrier and no exchange with
//     the other waves until the end.  A 32-row tile is stored piece-major
//     (16-byte piece p of tile row r at 512 p + 16 r): each of its 11
//     wave-wide loads takes two adjacent pieces (32 contiguous bytes) of all
//     32 rows, so a lane needs one row id and one address per tile;
//   * scores: MFMA 32x32x16 f16 with the tile's rows as A (a lane unpacks 8
//     values of one row per step: e2m1 -> f16 by the hardware converter,
//     times the block scale) and the query of the 32 heads, held in
//     registers, as B;
//   * the score accumulator's layout (lane = head, 16 rows) is the A operand
//     of the value MFMA as it stands: the softmax weights never leave the
//     registers.  Rows enter the value MFMA in the order that layout gives;
//     the values come in the same order from the transposing 4-bit LDS read
//     (ds_read_b64_tr_b4: 16 rows of one column per lane), scaled by the
//     rows' block scales from a small per-wave f16 table the score step
//     writes;
//   * online softmax: the first tile sets the running max; after that it
//     moves only when a score passes it by more than kSlack (log2 units), and
//     then O and the sum are rescaled (wave-local);
//   * the output (32 heads x 512 columns, fp32) stays in the accumulation
//     registers; at the end the four waves' states are combined through LDS
//     into the split's normalised partial (or the output when the list has
//     one split), which the merge kernel combines across splits.
#include "smla_internal.h"
#include "decode_device.h"

#include <type_traits>

namespace smla {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kWThreads = 64 * kWaves;
constexpr int kRows = 32;                      // rows per wave tile
constexpr int kTileB = kRows * kRowBytes;      // 11,264 bytes
constexpr int kLoads = kTileB / 1024;          // wave-wide 16-byte loads per tile (11)
constexpr int kSlots = 3;                      // ring slots per wave: tiles t .. t+2
constexpr int kMaxPerWave = kMaxTopk / kWaves; // list entries a wave can hold (512)
constexpr int kKSteps = kDim / 16;             // 36 score steps of 16 dims
constexpr float kSlack = 15.0f;           // f16 weights up to 2^15
static_assert(kTileB % 1024 == 0, "a tile must be whole wave-wide loads");
static_assert(kSlots * kTileB >= 8 * 4 * 64 * 16, "the combine stages 32 KB per wave in its ring");
static_assert(kKSteps % kWaves == 0 && (kKSteps / kWaves) * 1024 <= kTileB, "a wave stages its query quarter in one slot");

// The tile row that feeds row m of the score MFMA (bit 4 of m into bit 2).
// With the piece-major tile, the score step's 16-byte reads (16 rows, one
// piece) and the value step's transposing reads (the 16 rows of one
// accumulator class, two 8-byte halves) then touch every LDS bank once.
__device__ __forceinline__ int wv_row(int m) { return m ^ (((m >> 4) & 1) << 2); }

__global__ __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_wave_kernel(const uint16_t *__restrict__ q, const uint8_t *__restrict__ cache,
                        int64_t num_pages, const int32_t *__restrict__ page_table,
                        int32_t max_pages, const int32_t *__restrict__ seq_lens,
                        const int32_t *__restrict__ topk_idx, int32_t heads, int32_t topk,
                        float scale_log2, float *__restrict__ out, float *__restrict__ lse,
                        _Float16 *__restrict__ part_o, float *__restrict__ part_ml,
                        int32_t batch, int32_t tokens, int32_t groups, int32_t splits,
                        int32_t per_split) {
    constexpr int HG = 32;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kWaves][kSlots * kTileB];
    // per wave: the tile's block scales as f16, [block][row position], row
    // position 16 c + 8 a + 4 u + v for tile row 16 a + 8 u + 4 c + v
    __shared__ __attribute__((aligned(16))) _Float16 st_lds[kWaves][32][32];
    __shared__ uint32_t rows_lds[kWaves][kMaxPerWave];
    // the query's rope steps (32 .. 35) as B operands, read back every tile
    // (kept out of the registers, which the rest of the query fills)
    __shared__ __attribute__((aligned(16))) half8_t qrope_lds[4][64];
    __shared__ float ml_lds[kWaves][HG][2];
    __shared__ __attribute__((aligned(16))) float fac_lds[kWaves][HG];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31;  // score: row of the tile (A) / head (B, D)
    const int g2 = lane >> 5;   // 8-element k group

    // ---- (query, head group, split): consecutive workgroups go to
    // consecutive XCDs, so every head group, split and query token of
    // sequence sq shares XCD sq % 8 and its L2 ----
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int rest = id >> 3;
    const int split = rest % splits;
    const int hg = (rest / splits) % groups;
    const int r_seq = rest / splits / groups;
    const int sq = (r_seq / tokens) * 8 + xcd;
    if (sq >= batch) return;
    const int b = sq * tokens + r_seq % tokens;
    const int unit = b * groups + hg;
    const int e_begin = split * per_split;
    const int e_end = min(topk, e_begin + per_split);

    // ---- this wave's entries: chunk i of 32 = entries e_begin + 32 (4 i + w)
    // + 0..31; lane l takes chunk 2 k + l / 32, entry l % 32, for k < 8.  The
    // index loads go out first, then this wave's quarter of the query, then
    // (once the indices are in) the page-table loads ----
    const int64_t L = (int64_t)seq_lens[sq] - (tokens - 1 - (b - sq * tokens));
    int32_t tv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int e = e_begin + 32 * (4 * (2 * k + g2) + w) + n32;
        tv[k] = e < e_end ? topk_idx[(int64_t)b * topk + e] : -1;
    }
    // The query as B operands: step j < 32 takes dims 32 (2 (j/4) + g2) +
    // 8 (j%4) + 0..7, step 32 + u takes rope dims 512 + 32 g2 + 8 u + 0..7,
    // of head 32 hg + n32 -- the dims the row unpack below gives lane group
    // g2 at that step.  Wave w loads and converts steps 9 w .. 9 w + 8 into
    // its ring slot 2 (1 KB per step, lane l's 16 bytes at 16 l), which its
    // first tile loads leave free; every wave then reads all 36 steps.  Its
    // loads go out after the page-table loads, so that the index -> page
    // table -> first tile chain does not queue behind them.
    constexpr int kQPer = kKSteps / kWaves;  // 9
    uint32_t rid[8];
    uint4 qraw[kQPer];
    {
        int32_t pv[8];
        bool ok[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t t = tv[k];
            ok[k] = t >= 0 && t < L && (t >> 6) < max_pages;
            pv[k] = page_table[(int64_t)sq * max_pages + (ok[k] ? (t >> 6) : 0)];
        }
        const uint16_t *qh = q + ((int64_t)b * heads + hg * HG + n32) * kDim;
#pragma unroll
        for (int jj = 0; jj < kQPer; ++jj) {
            const int j = kQPer * w + jj;
            const int d0 = j < 32 ? 32 * (2 * (j >> 2) + g2) + 8 * (j & 3) : 512 + 32 * g2 + 8 * (j - 32);
            qraw[jj] = *reinterpret_cast<const uint4 *>(qh + d0);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t page = pv[k];
            rid[k] = (ok[k] && page >= 0 && page < num_pages)
                         ? (uint32_t)(page * kPageRows + (tv[k] & 63)) : 0xFFFFFFFFu;
        }
    }
    // compaction in list order: ballot prefix counts
    int n_w = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const bool v = rid[k] != 0xFFFFFFFFu;
        const uint64_t m = __ballot(v);
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (v) rows_lds[w][n_w + below] = rid[k];
        n_w += __builtin_popcountll(m);
    }
    const int n_tiles = (n_w + kRows - 1) / kRows;
    // the last tile is padded with row 0 of page 0 (always in the cache);
    // padding rows get weight 0 and zero block scales
    if (lane < n_tiles * kRows - n_w) rows_lds[w][n_w + lane] = 0u;

    // ---- the tile ring: load i of tile T fills LDS bytes [1024 i, 1024 i +
    // 1024) of its slot: lane l takes piece 2 i + l / 32 of tile row l % 32,
    // that is bytes 32 i + 16 (l / 32) .. of the row.  The row ids of tile
    // t + 2 are read one step early ----
    const uint32_t ring_w = (uint32_t)(size_t)(lds_void_t *)ring[w];
    auto tile_dma = [&](int T, uint32_t rk) {
        const uint32_t dst = ring_w + (uint32_t)((T % kSlots) * kTileB);
        const uint8_t *src = cache + (size_t)rk * kRowBytes + 16 * g2;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) dma16(src + 32 * i, dst + 1024u * i);
    };
    for (int T = 0; T < 2 && T < n_tiles; ++T) tile_dma(T, rows_lds[w][T * kRows + n32]);
    uint32_t rk_next = 2 < n_tiles ? rows_lds[w][2 * kRows + n32] : 0u;

    // this wave's query quarter, converted, into its slot 2; the whole query
    // from the four slots; then no wave loads a tile into its slot 2 before
    // every wave has read it
#pragma unroll
    for (int jj = 0; jj < kQPer; ++jj) {
        const uint32_t w4[4] = {qraw[jj].x, qraw[jj].y, qraw[jj].z, qraw[jj].w};
        const half8_t h = join(bf16x2_to_f16x2(w4[0]), bf16x2_to_f16x2(w4[1]), bf16x2_to_f16x2(w4[2]),
                               bf16x2_to_f16x2(w4[3]));
        const int j = kQPer * w + jj;
        if (j < 32)
            *reinterpret_cast<half8_t *>(ring[w] + 2 * kTileB + jj * 1024 + 16 * lane) = h;
        else
            qrope_lds[j - 32][lane] = h;
    }
    __syncthreads();
    half8_t qb[32];
#pragma unroll
    for (int j = 0; j < 32; ++j)
        qb[j] = *reinterpret_cast<const half8_t *>(ring[j / kQPer] + 2 * kTileB + (j % kQPer) * 1024 + 16 * lane);
    __syncthreads();

    // ---- per-lane LDS offsets within a tile slot ----
    // score step: tile row wv_row(n32); nibble piece 2 m + g2 at 1024 m
    // further, the scale pieces 16, 17 and the rope pieces 18 + 2 g2, 19 + 2 g2
    const uint32_t s_row = 16u * (uint32_t)wv_row(n32);
    const uint32_t s_nib = s_row + 512u * g2;
    const uint32_t s_sc0 = s_row + 512u * 16 + 2 * g2, s_sc1 = s_row + 512u * 17 + 2 * g2;
    const uint32_t s_rope0 = s_row + 512u * (18 + 2 * g2), s_rope1 = s_rope0 + 512u;
    // value step: lane l of group G = l / 16 (class c = G / 2, column half
    // h = G % 2) reads the 8 bytes of column window 32 cb + 16 h (nibble
    // piece cb, half h) of accumulator row R = 16 (k/8) + 8 ((k%8)/4) + 4 c +
    // k%4, k = l % 16, and receives column 32 cb + 16 h + k of the group's 16
    // rows, in the order of the score accumulator (row position 16 c + k)
    const int vk = lane & 15, vG = lane >> 4, vc = vG >> 1, vh = vG & 1;
    const int vR = 16 * (vk >> 3) + 8 * ((vk & 7) >> 2) + 4 * vc + (vk & 3);
    const uint32_t v_off = 16u * (uint32_t)wv_row(vR) + 8u * vh;  // + 512 cb
    // block scales for the value step: block 2 cb + h, positions 16 c .. 16 c + 15
    const uint8_t *st_w = reinterpret_cast<const uint8_t *>(st_lds[w]);
    const int v_st = (32 * vh + 16 * vc) * 2;
    // scale-table writes of the score step: position of accumulator row n32
    const int my_pos = 16 * ((n32 >> 2) & 1) + 8 * (n32 >> 4) + 4 * ((n32 >> 3) & 1) + (n32 & 3);

    float16_t o[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] = 0.0f;
    // The softmax reference of head n32 (log2 units) is fixed for a pass: the
    // first tile's max.  A weight 2^(s - m_ref) stays exact in f16 while
    // s - m_ref <= kSlack (15); O is then never rescaled, so only matrix
    // instructions touch it.  If a later score passes the reference by more
    // than kSlack, the pass is finished (its O is discarded; it gives the
    // exact max of the wave's rows) and a second pass redoes the rows with
    // that max as the reference, where every weight is at most 1.
    float m_run = 0.0f;
    float m_top = -INFINITY;  // max of this lane's d over the pass (relative to m_run)
    float l_run = 0.0f;       // sum of this lane's weights of head n32
    bool over = false;        // a score passed m_run + kSlack in this pass
    const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};

    auto pass = [&](auto second_c) {
        constexpr bool kSecond = decltype(second_c)::value;
        for (int t = 0; t < n_tiles; ++t) {
            // tile t + 2 into the slot of tile t - 1 (finished in step t - 1),
            // all its loads at once (a direct-to-LDS load can wait at issue,
            // and here that wait blocks nothing but the wait below); then wait
            // for tile t: the loads of t + 1 and t + 2 may be in flight
            if (t + 2 < n_tiles) {
                tile_dma(t + 2, rk_next);
                wait_vmcnt_n<2 * kLoads>();
            } else if (t + 1 < n_tiles) {
                wait_vmcnt_n<kLoads>();
            } else {
                wait_vmcnt_n<0>();
            }
            if (t + 3 < n_tiles) rk_next = rows_lds[w][(t + 3) * kRows + n32];
            const uint8_t *tb = ring[w] + (t % kSlots) * kTileB;

            // ---- scores of the tile's 32 rows for the 32 heads ----
            // the two block scales of step m: bytes 4 m + 2 g2, + 1 of the row's
            // 32 scale bytes (pieces 16, 17)
            auto read_sc = [&](int m) {
                return (uint32_t) * reinterpret_cast<const uint16_t *>(tb + (m < 4 ? s_sc0 : s_sc1) + 4 * (m & 3));
            };
            float16_t acc;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
            const bool real = t * kRows + wv_row(n32) < n_w;  // this lane's row is a selected row
            // nibble pieces two steps ahead of their use; the scheduling
            // barriers keep the compiler from hoisting more reads (their
            // registers) than that
            uint4 nbq[2];
            uint32_t scq[2];
            nbq[0] = *reinterpret_cast<const uint4 *>(tb + s_nib);
            nbq[1] = *reinterpret_cast<const uint4 *>(tb + s_nib + 1024);
            scq[0] = read_sc(0);
            scq[1] = read_sc(1);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint4 nb = nbq[m & 1];
                const uint32_t scm = scq[m & 1];
                if (m < 6) {
                    nbq[m & 1] = *reinterpret_cast<const uint4 *>(tb + s_nib + 1024 * (m + 2));
                    scq[m & 1] = read_sc(m + 2);
                }
                // blocks 4 m + 2 g2 and 4 m + 2 g2 + 1 of the row: {S, S} pairs
                const uint32_t dup = __builtin_amdgcn_perm(0u, scm, 0x01010000u);
                const half2_t sa = fp8x2<false>(dup), sbb = fp8x2<true>(dup);
                // this row's block scales for the value step (zero for padding rows)
                {
                    _Float16 *stp = st_lds[w][4 * m + 2 * g2] + my_pos;
                    stp[0] = real ? sa[0] : (_Float16)0.0f;
                    stp[32] = real ? sbb[0] : (_Float16)0.0f;
                }
                const uint32_t nw[4] = {nb.x, nb.y, nb.z, nb.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const half2_t sv = u < 2 ? sa : sbb;
                    const half8_t kb = join(fp4x2<0>(nw[u]) * sv, fp4x2<1>(nw[u]) * sv,
                                            fp4x2<2>(nw[u]) * sv, fp4x2<3>(nw[u]) * sv);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb, qb[4 * m + u], acc, 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            {
                const uint4 r0 = *reinterpret_cast<const uint4 *>(tb + s_rope0);
                const uint4 r1 = *reinterpret_cast<const uint4 *>(tb + s_rope1);
                const uint32_t rw[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const half8_t kb = join(fp8x2<false>(rw[2 * u]), fp8x2<true>(rw[2 * u]),
                                            fp8x2<false>(rw[2 * u + 1]), fp8x2<true>(rw[2 * u + 1]));
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kb, qrope_lds[u][lane], acc, 0, 0, 0);
                }
            }

            // ---- softmax weights: acc[4 i + j] is accumulator row 8 i + 4 g2 + j
            // (tile row wv_row of it), head n32 ----
            float d[16];
            const int rem = n_w - t * kRows;  // real rows of this tile (1 .. 32 or more)
            if (rem >= kRows) {
#pragma unroll
                for (int k = 0; k < 16; ++k) d[k] = fmaf(acc[k], scale_log2, -m_run);
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int r = wv_row(8 * (k >> 2) + 4 * g2 + (k & 3));
                    d[k] = r < rem ? fmaf(acc[k], scale_log2, -m_run) : -INFINITY;
                }
            }
            if constexpr (!kSecond) {
                float tm = d[0];
#pragma unroll
                for (int k = 1; k < 16; ++k) tm = fmaxf(tm, d[k]);
                if (t == 0) {
                    // the first tile sets the reference
                    tm = fmaxf(tm, __shfl_xor(tm, 32));
                    m_run = tm;
#pragma unroll
                    for (int k = 0; k < 16; ++k) d[k] -= tm;
                    tm = 0.0f;
                }
                m_top = fmaxf(m_top, tm);
                // (once over, the rest of the pass still runs in full -- its O is
                // discarded -- so that O is updated on every path through the
                // loop, which keeps it in the accumulation registers)
                over = over || __ballot(tm > kSlack) != 0;
            }
            half8_t pa[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                half2_t p2[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float2_t f = {__builtin_amdgcn_exp2f(d[8 * a + 2 * k]),
                                        __builtin_amdgcn_exp2f(d[8 * a + 2 * k + 1])};
                    p2[k] = __builtin_convertvector(f, half2_t);
                    l_run = __builtin_amdgcn_fdot2(p2[k], one2, l_run, false);
                }
                pa[a] = join(p2[0], p2[1], p2[2], p2[3]);
            }

            // ---- values: O[head][32 cb + col] += sum over rows P * V ----
            auto read_v = [&](int cb, int2_t &vv, half8_t &s0, half8_t &s1) {
                vv = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                    (lds_int2_t *)((__attribute__((address_space(3))) const uint8_t *)(tb + v_off + 512 * cb)));
                const half8_t *sp = reinterpret_cast<const half8_t *>(st_w + v_st + 128 * cb);
                s0 = sp[0];
                s1 = sp[1];
            };
            int2_t vvq[2];
            half8_t s0q[2], s1q[2];
            read_v(0, vvq[0], s0q[0], s1q[0]);
            read_v(1, vvq[1], s0q[1], s1q[1]);
#pragma unroll
            for (int cb = 0; cb < 16; ++cb) {
                const int2_t vv = vvq[cb & 1];
                const half8_t s0 = s0q[cb & 1], s1 = s1q[cb & 1];
                if (cb < 14) read_v(cb + 2, vvq[cb & 1], s0q[cb & 1], s1q[cb & 1]);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const uint32_t wv = (uint32_t)vv[a];
                    const half8_t ss = a == 0 ? s0 : s1;
                    const half2_t q01 = {ss[0], ss[1]}, q23 = {ss[2], ss[3]}, q45 = {ss[4], ss[5]},
                                  q67 = {ss[6], ss[7]};
                    const half8_t vb = join(fp4x2<0>(wv) * q01, fp4x2<1>(wv) * q23, fp4x2<2>(wv) * q45,
                                            fp4x2<3>(wv) * q67);
                    o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[a], vb, o[cb], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    pass(std::false_type{});
    if (over) {
        // second pass: the exact max of the wave's rows as the reference
        m_top = fmaxf(m_top, __shfl_xor(m_top, 32));
        m_run += m_top;
        l_run = 0.0f;
#pragma unroll
        for (int cb = 0; cb < 16; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[cb][i] = 0.0f;
        for (int T = 0; T < 2 && T < n_tiles; ++T) tile_dma(T, rows_lds[w][T * kRows + n32]);
        rk_next = 2 < n_tiles ? rows_lds[w][2 * kRows + n32] : 0u;
        pass(std::true_type{});
    }

    // ---- combine the four waves: M = max m_w, f_w = 2^(m_w - M) / L with
    // L = sum_w 2^(m_w - M) l_w (waves with no rows have l_w = 0) ----
    l_run += __shfl_xor(l_run, 32);
    if (lane < 32) {
        ml_lds[w][lane][0] = n_tiles > 0 ? m_run : -INFINITY;
        ml_lds[w][lane][1] = l_run;
    }
    __syncthreads();
    float Mh = -INFINITY, Lh = 0.0f;
    if (w == 0 && lane < 32) {
        float mw[kWaves], lw[kWaves];
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            mw[v] = ml_lds[v][lane][0];
            lw[v] = ml_lds[v][lane][1];
            if (lw[v] > 0.f) Mh = fmaxf(Mh, mw[v]);
        }
        const float Ms = Mh == -INFINITY ? 0.f : Mh;
        float fw[kWaves];
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            fw[v] = lw[v] > 0.f ? __builtin_amdgcn_exp2f(mw[v] - Ms) : 0.f;
            Lh += fw[v] * lw[v];
        }
        const float inv = Lh > 0.f ? 1.0f / Lh : 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) fac_lds[v][lane] = fw[v] * inv;
    }
    // each wave stages its O (fp32) in its own ring in two rounds of 256
    // columns: float4 (cb - 8 r, i / 4) of lane l at ((cbl 4 + i4) 64 + l) 16
    // bytes.  Wave v then sums, for 4 column blocks (cbl 4 (v % 2) ..) and two
    // head quads (i4 = 2 (v / 2) ..), the four waves' values times their
    // factors.
    const int r_cb0 = 4 * (w & 1), r_i40 = 2 * (w >> 1);
    const size_t pidx = (size_t)unit * splits + split;
    const float ln2 = 0.69314718055994530942f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (r == 1) __syncthreads();  // round 0's reads are done
        float4_t *stage = reinterpret_cast<float4_t *>(ring[w]);
#pragma unroll
        for (int cbl = 0; cbl < 8; ++cbl)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                stage[(cbl * 4 + i4) * 64 + lane] =
                    float4_t{o[8 * r + cbl][4 * i4], o[8 * r + cbl][4 * i4 + 1],
                             o[8 * r + cbl][4 * i4 + 2], o[8 * r + cbl][4 * i4 + 3]};
        __syncthreads();
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i4 = r_i40 + ii;
            float4_t f[kWaves];
#pragma unroll
            for (int v = 0; v < kWaves; ++v)
                f[v] = *reinterpret_cast<const float4_t *>(&fac_lds[v][8 * i4 + 4 * g2]);
            float4_t sum[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                sum[c] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int v = 0; v < kWaves; ++v) {
                    const float4_t x = reinterpret_cast<const float4_t *>(ring[v])[((r_cb0 + c) * 4 + i4) * 64 + lane];
                    sum[c] += x * f[v];
                }
            }
            // heads 8 i4 + 4 g2 + j; columns 32 cb' + n32, cb' = 8 r + r_cb0 + c
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int h = 8 * i4 + 4 * g2 + j;
                if (splits == 1) {
                    float *orow = out + ((int64_t)b * heads + hg * HG + h) * kLatent + n32;
#pragma unroll
                    for (int c = 0; c < 4; ++c) orow[32 * (8 * r + r_cb0 + c)] = sum[c][j];
                } else {
                    // part_o [pidx][h][4 sw][32 n32][4 cb]: column 128 sw + 32 cb + n32
                    const half4_t x4 = {(_Float16)sum[0][j], (_Float16)sum[1][j], (_Float16)sum[2][j],
                                        (_Float16)sum[3][j]};
                    const int sw = 2 * r + (w & 1);
                    uint64_t *dst = reinterpret_cast<uint64_t *>(part_o) + (pidx * HG + h) * 128 + sw * 32 + n32;
                    if (groups == 1 && tokens == 1)
                        *dst = __builtin_bit_cast(uint64_t, x4);
                    else
                        __builtin_nontemporal_store(__builtin_bit_cast(uint64_t, x4), dst);
                }
            }
        }
    }
    if (w == 0 && lane < 32) {
        const int h = lane;
        if (splits == 1) {
            lse[(int64_t)b * heads + hg * HG + h] = Lh > 0.f ? (Mh + log2f(Lh)) * ln2 : -INFINITY;
        } else {
            part_ml[(pidx * HG + h) * 2] = Mh;
            part_ml[(pidx * HG + h) * 2 + 1] = Lh;
        }
    }
}

}  // namespace

hipError_t launch_decode_wave(const uint16_t *q, const uint8_t *cache, int64_t num_pages,
                              const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                              const int32_t *topk_idx, int32_t batch, int32_t tokens, int32_t heads,
                              int32_t topk, float scale_log2, float *out, float *lse,
                              _Float16 *part_o, float *part_ml, const DecodePlan &plan,
                              hipStream_t stream) {
    const int blocks = ((batch + 7) / 8) * 8 * tokens * plan.groups * plan.splits;
    hipLaunchKernelGGL(decode_wave_kernel, dim3(blocks), dim3(kWThreads), 0, stream, q, cache,
                       num_pages, page_table, max_pages, seq_lens, topk_idx, heads, topk, scale_log2,
                       out, lse, part_o, part_ml, batch, tokens, plan.groups, plan.splits,
                       plan.per_split);
    return hipGetLastError();
}

}  // namespace smla
