// sparse_mla_decode: absorbed-query MLA attention over the top-k selected
// rows of a paged NVFP4 cache, dequantised on chip.
//
// What it computes: "Prime Inference: serving GLM-5.3 to agents is a
// KV-cache problem", section "A kernel that reads four bits directly" (load
// the selected 352-byte rows, unpack on chip, score, softmax and blend; -1
// entries carry no data) and Prime Intellect's launch post, native-kernel
// paragraph (FP16 operands, FP32 accumulation, partial results of the blocks
// sharing a query merged after the split).  Every selected row serves all
// heads of the query: "GLM-5.3 PCP/DCP long-context on H200", section 1.
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, 64-wide waves, 160 KB LDS):
//   * one 256-thread workgroup (4 waves) per (sequence, 16-head group,
//     split); a split is a slice of the top-k list.  A workgroup needs
//     under 80 KB of LDS and at most 256 registers per lane, so two run on
//     every CU and each SIMD interleaves two independent waves;
//   * prologue: the split's entries are validated, translated through the
//     page table and compacted into LDS, so -1 padding and out-of-range
//     entries cost neither a load nor a matrix instruction;
//   * per tile of 64 selected rows, each wave takes 16 rows: its lanes load
//     the 352-byte rows straight into registers in the B-operand layout of
//     v_mfma_f32_16x16x32_f16 (a lane holds a quarter of one row; the next
//     tile is in flight meanwhile), unpack them (e2m1 -> f16 by the hardware
//     converter, times the block scale with a packed f16 multiply; both
//     exact), score them against the query held in registers, and store the
//     unpacked latent part once into an XOR-swizzled LDS tile;
//   * softmax: a per-head running max that moves only when a score passes
//     it by more than kSlack, so after the first tiles the max reductions
//     and the accumulator rescale are skipped; the decision is shared by the
//     waves through LDS;
//   * value contraction: each wave accumulates its 128 of the 512 output
//     columns over all 64 rows, weights and values from LDS (values through
//     the transposing ds_read_b64_tr_b16);
//   * all workgroups of one sequence run on the same XCD (consecutive
//     workgroup ids go to consecutive XCDs), so the head groups re-read each
//     selected row from that XCD's L2;
//   * a split writes its partial (m, l, O) to the workspace and a second,
//     small kernel merges them (a merge inside the first launch would need
//     an agent-scope release per workgroup, an L2 writeback, which costs
//     more than the launch).
#include "smla_internal.h"

namespace smla {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4_t;
typedef __attribute__((address_space(3))) fp16x4_t lds_fp16x4;

constexpr int kThreads = 256;
constexpr int kHeads = 16;                    // heads per workgroup (one MFMA row block)
constexpr int kTile = 64;                     // selected rows per tile (16 per wave)
constexpr int kPStride = kTile + 8;           // f16 elements per LDS weight row (144 B)
constexpr int kKSteps = kDim / 32;            // 18 contraction steps of 32 for the scores
constexpr float kSlack = 8.0f;                // log2 headroom before the running max moves
constexpr int kMaxSplits = 16;

__device__ __forceinline__ half8_t join(half2_t a, half2_t b, half2_t c, half2_t d) {
    half8_t r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// Reductions over the 16 lanes of a row with DPP lane moves (quad swaps,
// half-row mirror, row mirror); every lane ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));  // row_mirror
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return x;
}

__device__ __forceinline__ _Float16 bf16_to_f16(uint32_t h) {
    return (_Float16)__uint_as_float(h << 16);
}

// The part of one row a lane holds: lane group g of a wave owns latent
// bytes [64g, 64g+64) (dims 128g..128g+127), scale bytes [256+8g, +8) and
// rope bytes [288+16g, +16) (rope dims 16g..16g+15).
struct RowPart {
    uint4 nib[4];
    uint2 sc;
    uint4 rope;
};

__device__ __forceinline__ void load_part(RowPart &p, const uint8_t *__restrict__ cache,
                                          uint32_t rid, bool valid, int g) {
    if (valid) {
        const uint8_t *base = cache + (size_t)rid * kRowBytes;
#pragma unroll
        for (int k = 0; k < 4; ++k) p.nib[k] = *reinterpret_cast<const uint4 *>(base + 64 * g + 16 * k);
        p.sc = *reinterpret_cast<const uint2 *>(base + kScaleOff + 8 * g);
        p.rope = *reinterpret_cast<const uint4 *>(base + kRopeOff + 16 * g);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) p.nib[k] = make_uint4(0u, 0u, 0u, 0u);
        p.sc = make_uint2(0u, 0u);
        p.rope = make_uint4(0u, 0u, 0u, 0u);
    }
}

// LDS value tile: [64 rows][512 columns] f16, 16-byte chunks of a row stored
// at chunk ^ (row % 16) so that both the unpacking stores (16 rows, same
// chunk) and the transposing reads (4 rows x 4 chunks) spread over banks.
__device__ __forceinline__ int v_index(int row, int col) {
    return row * kLatent + ((((col >> 3) ^ (row & 15)) << 3) | (col & 7));
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_mla_decode_kernel(const uint16_t *__restrict__ q, const uint8_t *__restrict__ cache,
                              int64_t num_pages, const int32_t *__restrict__ page_table,
                              int32_t max_pages, const int32_t *__restrict__ seq_lens,
                              const int32_t *__restrict__ topk_idx, int32_t heads, int32_t topk,
                              float scale_log2, float *__restrict__ out, float *__restrict__ lse,
                              float *__restrict__ ws_partials, int32_t batch, int32_t groups,
                              int32_t splits, int32_t per_split) {
    __shared__ __attribute__((aligned(16))) _Float16 v_lds[kTile * kLatent];
    __shared__ __attribute__((aligned(16))) _Float16 p_lds[kHeads * kPStride];
    __shared__ uint32_t rowid_lds[kMaxTopk];
    __shared__ float wmax_lds[4][kHeads];
    __shared__ float lsum_lds[4][kHeads];
    __shared__ int32_t scan_lds[4];
    __shared__ uint32_t flag_lds[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 15;   // row (scores) / column (values) within a 16-block
    const int g = lane >> 4;   // 8-element k group

    // ---- which (sequence, head group, split): consecutive workgroups go to
    // consecutive XCDs, so all workgroups of sequence b share XCD b % 8 ----
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int rest = id >> 3;
    const int split = rest % splits;
    const int hg = (rest / splits) % groups;
    const int b = (rest / splits / groups) * 8 + xcd;
    if (b >= batch) return;
    const int unit = b * groups + hg;
    const int e_begin = split * per_split;
    const int e_end = min(topk, e_begin + per_split);

    // ---- prologue: validate, translate, compact the split's entries ----
    const int64_t L = seq_lens[b];
    const int per_thread = (per_split + kThreads - 1) / kThreads;
    uint32_t rid[8];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        rid[i] = 0xFFFFFFFFu;
        const int e = e_begin + tid * per_thread + i;
        if (i < per_thread && e < e_end) {
            const int64_t t = topk_idx[(int64_t)b * topk + e];
            if (t >= 0 && t < L && (t >> 6) < max_pages) {
                const int64_t page = page_table[(int64_t)b * max_pages + (t >> 6)];
                if (page >= 0 && page < num_pages) rid[i] = (uint32_t)(page * kPageRows + (t & 63));
            }
        }
        cnt += rid[i] != 0xFFFFFFFFu;
    }
    // exclusive scan of cnt over the workgroup (list order preserved)
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    if (lane == 63) scan_lds[wave] = incl;
    __syncthreads();
    int before = 0, n_valid = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int s = scan_lds[w];
        before += (w < wave) ? s : 0;
        n_valid += s;
    }
    int pos = before + incl - cnt;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (rid[i] != 0xFFFFFFFFu) rowid_lds[pos++] = rid[i];

    // ---- query for this head group, resident in registers as f16 A operands ----
    // A[m = head][k = 8g + i] at score step j holds dim 128g + 8j + i (latent,
    // j < 16) or 512 + 16g + 8(j-16) + i (rope): the same permutation of the
    // 576 dims that the unpacked rows use below.
    half8_t qa[kKSteps];
    {
        const int head = hg * kHeads + n;
        const uint16_t *qrow = q + ((int64_t)b * heads + head) * kDim;
#pragma unroll
        for (int j = 0; j < kKSteps; ++j) {
            const int d0 = (j < 16) ? (128 * g + 8 * j) : (512 + 16 * g + 8 * (j - 16));
            const uint4 v = *reinterpret_cast<const uint4 *>(qrow + d0);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qa[j][2 * i] = bf16_to_f16(w4[i] & 0xFFFFu);
                qa[j][2 * i + 1] = bf16_to_f16(w4[i] >> 16);
            }
        }
    }
    __syncthreads();  // rowid_lds complete

    const int n_tiles = (n_valid + kTile - 1) / kTile;
    const int row = wave * 16 + n;  // this lane's row within a tile

    float4_t o[8];
    float m_run[4], l_run[4];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) o[nb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) { m_run[r] = -INFINITY; l_run[r] = 0.f; }

    RowPart cur, nxt;
    if (n_tiles > 0) load_part(cur, cache, rowid_lds[min(row, n_valid - 1)], row < n_valid, g);

    for (int tile = 0; tile < n_tiles; ++tile) {
        // (1) next tile's rows in flight while this one is processed
        const int nrow = (tile + 1) * kTile + row;
        if (tile + 1 < n_tiles)
            load_part(nxt, cache, rowid_lds[min(nrow, n_valid - 1)], nrow < n_valid, g);
        // every wave has finished reading the previous tile's values
        if (tile > 0) __syncthreads();

        // (2) unpack this wave's 16 rows, score them, store the latent part
        half2_t s2[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t byte = ((k < 4 ? cur.sc.x : cur.sc.y) >> (8 * (k & 3))) & 0xFFu;
            s2[k] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(byte * 0x0101u, 1.0f, false);
        }
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint4 nq = cur.nib[j >> 2];
            const uint32_t d = (j & 3) == 0 ? nq.x : (j & 3) == 1 ? nq.y : (j & 3) == 2 ? nq.z : nq.w;
            const half2_t sv = s2[j >> 1];
            const half2_t e0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * sv;
            const half2_t e1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * sv;
            const half2_t e2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * sv;
            const half2_t e3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * sv;
            const half8_t kb = join(e0, e1, e2, e3);
            *reinterpret_cast<half8_t *>(v_lds + v_index(row, 128 * g + 8 * j)) = kb;
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[j], kb, acc, 0, 0, 0);
        }
#pragma unroll
        for (int j = 16; j < 18; ++j) {
            const uint32_t d0 = (j == 16) ? cur.rope.x : cur.rope.z;
            const uint32_t d1 = (j == 16) ? cur.rope.y : cur.rope.w;
            const half8_t kb = join(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false),
                                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true),
                                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false),
                                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[j], kb, acc, 0, 0, 0);
        }

        // (3) scores in log2 units; does any head's running max move?  It
        // moves only when a score passes it by more than kSlack (weights stay
        // <= 2^kSlack, fine in f16), so after the first tiles the max, the
        // rescale and their cross-lane reductions are skipped.  The decision
        // is shared by all waves.
        const bool valid = tile * kTile + row < n_valid;
        float x[4];
        bool over = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            x[r] = valid ? acc[r] * scale_log2 : -INFINITY;
            over |= x[r] > m_run[r] + kSlack;
        }
        const uint64_t ballot = __ballot(over);
        if (lane == 0) flag_lds[wave] = ballot != 0;
        __syncthreads();
        if ((flag_lds[0] | flag_lds[1] | flag_lds[2] | flag_lds[3]) != 0) {
            // exact tile maxima per head, exchanged through LDS
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float mx = row16_max(x[r]);
                if (n == 0) wmax_lds[wave][4 * g + r] = mx;
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * g + r;
                const float mt = fmaxf(fmaxf(wmax_lds[0][h], wmax_lds[1][h]),
                                       fmaxf(wmax_lds[2][h], wmax_lds[3][h]));
                const float m_new = fmaxf(m_run[r], mt);
                // m_new = -inf only while nothing valid was seen: keep zeros
                const float alpha =
                    (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run[r] - m_new);
                m_run[r] = m_new;
                l_run[r] *= alpha;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) o[nb][r] *= alpha;
            }
        }

        // (4) f16 weights to LDS; each lane keeps its own share of the sum
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p =
                (m_run[r] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[r] - m_run[r]);
            const _Float16 ph = (_Float16)p;
            p_lds[(4 * g + r) * kPStride + row] = ph;
            l_run[r] += (float)ph;  // the normaliser sums the weights actually used
        }
        __syncthreads();

        // (5) value contraction: this wave's 128 output columns, all 64 rows
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const half8_t pa = *reinterpret_cast<const half8_t *>(p_lds + n * kPStride + 32 * ks + 8 * g);
            const int vr = 32 * ks + 8 * g + (n >> 2);
            fp16x4_t vlo[8], vhi[8];
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int col = 128 * wave + 16 * nb + 4 * (n & 3);
                vlo[nb] = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(
                    (__attribute__((address_space(3))) _Float16 *)(v_lds + v_index(vr, col))));
                vhi[nb] = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(
                    (__attribute__((address_space(3))) _Float16 *)(v_lds + v_index(vr + 4, col))));
            }
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                half8_t vb;
#pragma unroll
                for (int i = 0; i < 4; ++i) { vb[i] = (_Float16)vlo[nb][i]; vb[4 + i] = (_Float16)vhi[nb][i]; }
                o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, vb, o[nb], 0, 0, 0);
            }
        }
        cur = nxt;
    }

    // ---- epilogue: combine the lanes' and the waves' shares of the sums ----
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float ls = row16_sum(l_run[r]);
        if (n == 0) lsum_lds[wave][4 * g + r] = ls;
    }
    __syncthreads();
    float l_tot[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * g + r;
        l_tot[r] = lsum_lds[0][h] + lsum_lds[1][h] + lsum_lds[2][h] + lsum_lds[3][h];
    }

    if (splits == 1) {
        const float ln2 = 0.69314718055994530942f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int head = hg * kHeads + 4 * g + r;
            const float inv = l_tot[r] > 0.f ? 1.0f / l_tot[r] : 0.f;
            float *orow = out + ((int64_t)b * heads + head) * kLatent + 128 * wave + n;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) orow[16 * nb] = o[nb][r] * inv;
            if (wave == 0 && n == 0)
                lse[(int64_t)b * heads + head] =
                    l_tot[r] > 0.f ? (m_run[r] + log2f(l_tot[r])) * ln2 : -INFINITY;
        }
        return;
    }

    // ---- split: publish the partial; the merge kernel combines them ----
    // Partial layout per (unit, split): O[16][512] unnormalised, then m[16]
    // (running max, log2 units) and l[16] (sum of weights).
    const size_t pfl = (size_t)kHeads * kLatent + 2 * kHeads;
    float *part = ws_partials + ((size_t)unit * splits + split) * pfl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int h = 4 * g + r;
        float *prow = part + (size_t)h * kLatent + 128 * wave + n;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) prow[16 * nb] = o[nb][r];
        if (wave == 0 && n == 0) {
            part[(size_t)kHeads * kLatent + h] = m_run[r];
            part[(size_t)kHeads * kLatent + kHeads + h] = l_tot[r];
        }
    }
}

// Merge of the splits' partials: one thread per (unit, head, 4 columns); all
// splits' loads are issued up front, then combined in split order (fixed,
// hence deterministic):
//   M = max_s m_s,  L = sum_s 2^(m_s - M) l_s,  O = sum_s 2^(m_s - M) O_s / L.
__global__ __launch_bounds__(256) void merge_splits_kernel(
    const float *__restrict__ ws_partials, float *__restrict__ out, float *__restrict__ lse,
    int32_t heads, int32_t groups, int32_t splits, int32_t units) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)units * kHeads * (kLatent / 4);
    if (idx >= total) return;
    const int c4 = (int)(idx % (kLatent / 4));
    const int h = (int)((idx / (kLatent / 4)) % kHeads);
    const int unit = (int)(idx / ((int64_t)(kLatent / 4) * kHeads));
    const size_t pfl = (size_t)kHeads * kLatent + 2 * kHeads;
    const float *base = ws_partials + (size_t)unit * splits * pfl;
    float ms[kMaxSplits], ls[kMaxSplits];
    float4_t os[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        if (s < splits) {
            const float *ps = base + s * pfl;
            ms[s] = ps[(size_t)kHeads * kLatent + h];
            ls[s] = ps[(size_t)kHeads * kLatent + kHeads + h];
            os[s] = *reinterpret_cast<const float4_t *>(ps + (size_t)h * kLatent + 4 * c4);
        } else {
            ms[s] = -INFINITY;
            ls[s] = 0.f;
            os[s] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) M = fmaxf(M, ms[s]);
    float L = 0.f;
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s) {
            const float w = __builtin_amdgcn_exp2f(ms[s] - M);
            L += w * ls[s];
            acc += w * os[s];
        }
    }
    const int b = unit / groups;
    const int head = (unit % groups) * kHeads + h;
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    *reinterpret_cast<float4_t *>(out + ((int64_t)b * heads + head) * kLatent + 4 * c4) = acc * inv;
    if (c4 == 0)
        lse[(int64_t)b * heads + head] =
            L > 0.f ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

DecodePlan plan_decode(int batch, int heads, int topk) {
    DecodePlan p;
    p.heads_per_group = kHeads;
    p.groups = heads / kHeads;
    const int units = batch * p.groups;
    const int target = 512;  // two workgroups per CU
    int s = (target + units - 1) / units;
    const int max_s = (topk + kTile - 1) / kTile;
    s = s < 1 ? 1 : s;
    s = s > max_s ? max_s : s;
    s = s > kMaxSplits ? kMaxSplits : s;
    p.splits = s;
    p.per_split = (topk + s - 1) / s;
    p.partial_floats = (size_t)kHeads * kLatent + 2 * kHeads;
    if (s == 1) {
        p.workspace_bytes = 0;
    } else {
        const size_t part = (size_t)units * s * p.partial_floats * sizeof(float);
        p.workspace_bytes = (part + 255) & ~(size_t)255;
    }
    return p;
}

hipError_t launch_sparse_mla_decode(const uint16_t *q, const uint8_t *cache, int64_t num_pages,
                                    const int32_t *page_table, int32_t max_pages,
                                    const int32_t *seq_lens, const int32_t *topk_idx,
                                    int32_t batch, int32_t heads, int32_t topk, float scale,
                                    float *out, float *lse, void *workspace,
                                    const DecodePlan &plan, hipStream_t stream) {
    const int blocks = ((batch + 7) / 8) * 8 * plan.groups * plan.splits;
    float *partials = plan.splits > 1 ? static_cast<float *>(workspace) : nullptr;
    const float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    hipLaunchKernelGGL(sparse_mla_decode_kernel, dim3(blocks), dim3(kThreads), 0, stream, q, cache,
                       num_pages, page_table, max_pages, seq_lens, topk_idx, heads, topk,
                       scale_log2, out, lse, partials, batch, plan.groups, plan.splits,
                       plan.per_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const int units = batch * plan.groups;
    const int64_t threads = (int64_t)units * kHeads * (kLatent / 4);
    hipLaunchKernelGGL(merge_splits_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, partials, out, lse, heads, plan.groups, plan.splits, units);
    return hipGetLastError();
}

}  // namespace smla
