// kv_quant_append: BF16 KV rows -> 352-byte NVFP4 rows in the paged cache.
//
// Format: "Prime Inference: serving GLM-5.3 to agents is a KV-cache problem",
// section "Four bits per latent value: where 352 comes from" -- the 512 latent
// values as e2m1 nibbles with one FP8 E4M3 scale per 16, the 64 rope values
// as FP8.  The rounding rules (scale = E4M3 nearest amax/6, nibble = e2m1
// nearest x/scale, ties to even, sign copied) are the readings stated in
// include/smla.h; every decision below is taken with exact fp32 operations so
// the bytes are reproducible bit for bit (nvfp4_quant.h).
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
#include "nvfp4_quant.h"
#include "smla_internal.h"

namespace smla {
namespace {

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

    const Nvfp4Lane v = nvfp4_quant_lane(lo, hi, r);
    if (!ok) return;
    *reinterpret_cast<uint2 *>(dst + j * 8) = make_uint2(v.nib[0], v.nib[1]);
    dst[kScaleOff + j] = (uint8_t)v.scale;
    *reinterpret_cast<uint16_t *>(dst + kRopeOff + 2 * j) = (uint16_t)v.rope;
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
