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
// index load, one page-table load each) into LDS; then the 64 x 36 16-byte
// pieces of the copy (pieces 0..31 of a row are its latent blocks -- 8 nibble
// bytes and one scale each -- and 32..35 its rope bytes) are dealt to the
// threads in order, 9 each, so the copy is written as one contiguous stream
// and every thread has all its row loads in flight at once.  The decoded
// values (e2m1 x S, exact in fp32) are clamped to [-448, 448] and converted
// by the hardware's round-to-nearest-even FP8 conversion, which is then the
// nearest-E4M3 rule with saturation.
#include "e4m3.h"
#include "smla_internal.h"

namespace smla {
namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kPieces = kFp8RowBytes / 16;  // 36

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
    uint2 nib[9];
    uint4 rope[9];
    uint32_t sc[9];
    bool use[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int p = tid + 256 * k;  // piece of the 64-row block
        const int rl = p / kPieces, j = p - rl * kPieces;
        const int64_t r = row_lds[rl];
        use[k] = r >= 0;
        const uint8_t *row = cache + (use[k] ? r : 0) * kRowBytes;
        if (j < 32) {
            nib[k] = use[k] ? *reinterpret_cast<const uint2 *>(row + 8 * j) : make_uint2(0u, 0u);
            sc[k] = use[k] ? row[kScaleOff + j] : 0u;
        } else {
            rope[k] = use[k] ? *reinterpret_cast<const uint4 *>(row + kRopeOff + 16 * (j - 32))
                             : make_uint4(0u, 0u, 0u, 0u);
        }
    }
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const int p = tid + 256 * k;
        const int rl = p / kPieces, j = p - rl * kPieces;
        if (!use[k]) continue;
        uint4 *dst = reinterpret_cast<uint4 *>(out_base + (int64_t)rl * kFp8RowBytes) + j;
        if (j >= 32) {
            *dst = rope[k];
            continue;
        }
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
