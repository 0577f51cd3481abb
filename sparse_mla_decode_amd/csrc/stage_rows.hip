// stage_rows_fp8: the staged path's gather-unpack, kept as the ablation of the
// fused decode.
//
// "Prime Inference: serving GLM-5.3 to agents is a KV-cache problem", section
// "A kernel that reads four bits directly" (the staged-vs-native figure) and
// the launch post's account of its first implementation: a gather kernel
// reads the selected 352-byte NVFP4 rows, writes a 576-byte FP8 copy of each
// back to HBM, and an FP8 attention kernel reads the copy -- 352 + 576 + 576
// bytes per selected row against 352 for the fused kernel.
//
// The copy is the lean FP8 row: each decoded value e2m1 x S (exact in fp32)
// re-encoded as the E4M3 value nearest it (ties to even, saturating at 448);
// the rope bytes are E4M3 already and are copied.  Entry e of sequence b goes
// to row b * kpad + e of the staged buffer (kpad = topk rounded up to 64), so
// the FP8 decode reads it through the page table [b][p] = b * kpad / 64 + p
// with its list staged_topk[b][e] = e (usable entries) or -1.
//
// Mapping: a 256-thread workgroup stages 64 consecutive entries of one
// sequence.  The first 64 threads validate and translate the entries (one
// index load, one page-table load each) into LDS; then every thread takes 8
// of the 64 x 32 latent blocks (8 nibble bytes and one scale each, one
// 16-byte piece of the copy) and one of the 64 x 4 rope pieces, with all its
// row loads in flight at once.  The decoded
// values (e2m1 x S, exact in fp32) are clamped to [-448, 448] and converted
// by the hardware's round-to-nearest-even FP8 conversion, which is then the
// nearest-E4M3 rule with saturation.
#include "e4m3.h"
#include "smla_internal.h"

namespace smla {
namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));


// e2m1 pair (byte SEL of w, low nibble first) -> two floats, exact
template <int SEL>
__device__ __forceinline__ float2_t fp4x2_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

__global__ __launch_bounds__(256) void stage_rows_fp8_kernel(
    const uint8_t *__restrict__ cache, int64_t num_pages, const int32_t *__restrict__ page_table,
    int32_t max_pages, const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ topk_idx,
    int32_t batch, int32_t topk, int64_t kpad, uint8_t *__restrict__ staged,
    int32_t *__restrict__ staged_topk) {
    __shared__ int64_t row_lds[64];  // cache row of each entry, -1 if unusable
    const int chunks = (int)(kpad / 64);
    const int64_t b = blockIdx.x / chunks;
    const int e0 = (int)(blockIdx.x % chunks) * 64;
    const int tid = threadIdx.x;
    if (tid < 64) {
        const int e = e0 + tid;
        int64_t r = -1;
        if (e < topk) {
            const int64_t t = topk_idx[b * topk + e];
            const int64_t L = seq_lens[b];
            if (t >= 0 && t < L && (t >> 6) < max_pages) {
                const int64_t page = page_table[b * max_pages + (t >> 6)];
                if (page >= 0 && page < num_pages) r = page * kPageRows + (t & 63);
            }
            staged_topk[b * topk + e] = r >= 0 ? e : -1;
        }
        row_lds[tid] = r;
    }
    __syncthreads();
    uint8_t *out_base = staged + (b * kpad + e0) * kFp8RowBytes;
    // Loads first, all of them unconditional (an unusable entry reads row 0
    // of page 0, which every cache has, and is skipped below), so that none
    // waits for another: the 8 latent pieces of this thread (piece p = tid +
    // 256 k is block p % 32 of row p / 32: 8 nibble bytes and a scale byte)
    // and its one rope piece (the 16 bytes 16 (tid % 4) .. of row tid / 4).
    uint2 nib[8];
    uint32_t sc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int p = tid + 256 * k;
        const int64_t r = max(row_lds[p >> 5], (int64_t)0);
        const uint8_t *row = cache + r * kRowBytes;
        nib[k] = *reinterpret_cast<const uint2 *>(row + 8 * (p & 31));
        sc[k] = row[kScaleOff + (p & 31)];
    }
    const int64_t rr = row_lds[tid >> 2];
    const uint4 rope = *reinterpret_cast<const uint4 *>(cache + max(rr, (int64_t)0) * kRowBytes + kRopeOff +
                                                        16 * (tid & 3));
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int p = tid + 256 * k;
        const int rl = p >> 5, j = p & 31;
        if (row_lds[rl] < 0) continue;
        uint4 *dst = reinterpret_cast<uint4 *>(out_base + (int64_t)rl * kFp8RowBytes) + j;
        const float S = (sc[k] & 0x80u) ? -e4m3_mag(sc[k]) : e4m3_mag(sc[k]);
        const uint32_t w[2] = {nib[k].x, nib[k].y};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // byte q of the piece's 8 holds elements 2q (low nibble), 2q + 1
            const uint32_t wq = w[q >> 1];
            const float2_t lo = (q & 1) ? fp4x2_f32<2>(wq) : fp4x2_f32<0>(wq);
            const float2_t hi = (q & 1) ? fp4x2_f32<3>(wq) : fp4x2_f32<1>(wq);
            const float v0 = __builtin_amdgcn_fmed3f(lo[0] * S, -448.0f, 448.0f);
            const float v1 = __builtin_amdgcn_fmed3f(lo[1] * S, -448.0f, 448.0f);
            const float v2 = __builtin_amdgcn_fmed3f(hi[0] * S, -448.0f, 448.0f);
            const float v3 = __builtin_amdgcn_fmed3f(hi[1] * S, -448.0f, 448.0f);
            int r = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
            r = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, r, true);
            o[q] = (uint32_t)r;
        }
        *dst = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (rr >= 0)
        *(reinterpret_cast<uint4 *>(out_base + (int64_t)(tid >> 2) * kFp8RowBytes + kLatent) + (tid & 3)) = rope;
}

}  // namespace

hipError_t launch_stage_rows_fp8(const uint8_t *cache, int64_t num_pages,
                                 const int32_t *page_table, int32_t max_pages,
                                 const int32_t *seq_lens, const int32_t *topk_idx, int32_t batch,
                                 int32_t topk, uint8_t *staged, int32_t *staged_topk,
                                 hipStream_t stream) {
    const int64_t kpad = ((int64_t)topk + kPageRows - 1) / kPageRows * kPageRows;
    hipLaunchKernelGGL(stage_rows_fp8_kernel, dim3((unsigned)(batch * (kpad / 64))), dim3(256), 0,
                       stream, cache, num_pages, page_table, max_pages, seq_lens, topk_idx, batch,
                       topk, kpad, staged, staged_topk);
    return hipGetLastError();
}

}  // namespace smla
