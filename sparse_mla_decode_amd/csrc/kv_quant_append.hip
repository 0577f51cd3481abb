// kv_quant_append: BF16 KV rows -> 352-byte NVFP4 rows in the paged cache.
//
// Format: "Prime Inference: serving GLM-5.3 to agents is a KV-cache problem",
// section "Four bits per latent value: where 352 comes from" -- the 512 latent
// values as e2m1 nibbles with one FP8 E4M3 scale per 16, the 64 rope values
// as FP8.  The rounding rules (scale = E4M3 nearest amax/6, nibble = e2m1
// nearest x/scale, ties to even, sign copied) are the readings stated in
// include/smla.h; every decision below is taken with exact fp32 operations so
// the bytes are reproducible bit for bit.
//
// Mapping: 32 lanes per row, lane j owns latent block j (16 values) and rope
// values 2j, 2j+1.  A 256-thread workgroup quantises 8 rows.  The kernel is
// HBM-bound (1152 B read and 352 B written per row); loads of a row are one
// contiguous 1 KiB sweep across its 32 lanes.
//
// kv_quant_append_fp8 writes the lean FP8 row of the same section's byte
// table instead: the 576 values as E4M3 bytes in dim order, no scale, each
// the E4M3 value nearest the input (the rope rule).  36 lanes per row, lane j
// owns values 16j .. 16j+15; a 288-thread workgroup quantises 8 rows.
#include "e4m3.h"
#include "smla_internal.h"

namespace smla {
namespace {

// Scale code: E4M3 value nearest amax / 6, ties to even.  The fp32 quotient
// gives a first guess; exact comparisons of amax with 6 * midpoint (a
// midpoint has at most 5 significant bits, so 3 * (lo + hi) is exact) settle
// it, including exact ties.
__device__ __forceinline__ uint32_t scale_code(float amax) {
    uint32_t s = e4m3_nearest(amax * (1.0f / 6.0f)) & 0x7Fu;
    for (int it = 0; it < 3; ++it) {
        if (s < 0x7Eu) {
            float mid6 = 3.0f * (e4m3_mag(s) + e4m3_mag(s + 1));
            if (amax > mid6 || (amax == mid6 && ((s + 1) & 1u) == 0)) { ++s; continue; }
        }
        if (s > 0u) {
            float mid6 = 3.0f * (e4m3_mag(s - 1) + e4m3_mag(s));
            if (amax < mid6 || (amax == mid6 && ((s - 1) & 1u) == 0)) { --s; continue; }
        }
        break;
    }
    return s;
}

// e2m1 magnitude code of a / S: count of midpoints passed.  The midpoints
// 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 (times S, exact) alternate between
// ties-down (even code below) and ties-up (even code above).
__device__ __forceinline__ uint32_t e2m1_code(float a, const float t[7]) {
    uint32_t c = 0;
    c += a > t[0];
    c += a >= t[1];
    c += a > t[2];
    c += a >= t[3];
    c += a > t[4];
    c += a >= t[5];
    c += a > t[6];
    return c;
}

__device__ __forceinline__ float bf16_abs(uint32_t h) { return __uint_as_float((h & 0x7FFFu) << 16); }

__global__ __launch_bounds__(256) void kv_quant_append_kernel(const uint16_t *__restrict__ rows,
                                                              int64_t n,
                                                              const int32_t *__restrict__ slots,
                                                              uint8_t *__restrict__ cache,
                                                              int64_t num_slots) {
    const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    const int j = threadIdx.x & 31;
    if (row >= n) return;
    // the row's loads and the slot's in flight together; the slot decides
    // only the store
    const uint16_t *x = rows + row * kDim;
    const uint4 lo = *reinterpret_cast<const uint4 *>(x + j * kBlock);
    const uint4 hi = *reinterpret_cast<const uint4 *>(x + j * kBlock + 8);
    const uint32_t r = *reinterpret_cast<const uint32_t *>(x + kLatent + 2 * j);
    const int64_t slot = slots[row];
    // (no early return on the slot: the loads would then wait for it)
    const bool ok = slot >= 0 && slot < num_slots;
    uint8_t *dst = cache + (ok ? slot : 0) * kRowBytes;

    // ---- latent block j ----
    uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t amax_bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        amax_bits = max(amax_bits, w[i] & 0x7FFFu);
        amax_bits = max(amax_bits, (w[i] >> 16) & 0x7FFFu);
    }
    const float amax = __uint_as_float(amax_bits << 16);
    const uint32_t s = scale_code(amax);
    const float S = e4m3_mag(s);
    const float t[7] = {0.25f * S, 0.75f * S, 1.25f * S, 1.75f * S, 2.5f * S, 3.5f * S, 5.0f * S};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t h = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        const uint32_t mag = (S == 0.0f) ? 0u : e2m1_code(bf16_abs(h), t);
        const uint32_t nib = mag | ((h >> 12) & 8u);
        packed[i >> 3] |= nib << ((i & 7) * 4);
    }
    if (!ok) return;
    *reinterpret_cast<uint2 *>(dst + j * 8) = make_uint2(packed[0], packed[1]);
    dst[kScaleOff + j] = (uint8_t)s;

    // ---- rope values 2j, 2j+1 ----
    const uint32_t c0 = e4m3_nearest(__uint_as_float((r & 0xFFFFu) << 16));
    const uint32_t c1 = e4m3_nearest(__uint_as_float(r & 0xFFFF0000u));
    *reinterpret_cast<uint16_t *>(dst + kRopeOff + 2 * j) = (uint16_t)(c0 | (c1 << 8));
}

__global__ __launch_bounds__(288) void kv_quant_append_fp8_kernel(const uint16_t *__restrict__ rows,
                                                                   int64_t n,
                                                                   const int32_t *__restrict__ slots,
                                                                   uint8_t *__restrict__ cache,
                                                                   int64_t num_slots) {
    const int64_t row = (int64_t)blockIdx.x * 8 + threadIdx.x / 36;
    const int j = threadIdx.x % 36;
    if (row >= n) return;
    const uint4 lo = *reinterpret_cast<const uint4 *>(rows + row * kDim + 16 * j);
    const uint4 hi = *reinterpret_cast<const uint4 *>(rows + row * kDim + 16 * j + 8);
    const int64_t slot = slots[row];
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t b[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t c0 = e4m3_nearest(__uint_as_float(w[i] << 16));
        const uint32_t c1 = e4m3_nearest(__uint_as_float(w[i] & 0xFFFF0000u));
        b[i >> 1] |= (c0 | (c1 << 8)) << (16 * (i & 1));
    }
    if (slot < 0 || slot >= num_slots) return;
    *reinterpret_cast<uint4 *>(cache + slot * kFp8RowBytes + 16 * j) = make_uint4(b[0], b[1], b[2], b[3]);
}

}  // namespace

hipError_t launch_kv_quant_append_fp8(const uint16_t *rows, int64_t n, const int32_t *slots,
                                      uint8_t *cache, int64_t num_pages, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 7) / 8;
    hipLaunchKernelGGL(kv_quant_append_fp8_kernel, dim3((unsigned)blocks), dim3(288), 0, stream,
                       rows, n, slots, cache, num_pages * kPageRows);
    return hipGetLastError();
}

hipError_t launch_kv_quant_append(const uint16_t *rows, int64_t n, const int32_t *slots,
                                  uint8_t *cache, int64_t num_pages, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 7) / 8;
    hipLaunchKernelGGL(kv_quant_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, rows,
                       n, slots, cache, num_pages * kPageRows);
    return hipGetLastError();
}

}  // namespace smla
