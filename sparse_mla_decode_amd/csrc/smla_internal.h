// Internal declarations shared by the library's translation units.
// Format constants follow the row layout of "Prime Inference: serving GLM-5.3
// to agents is a KV-cache problem", section "Four bits per latent value: where
// 352 comes from": 256 B of e2m1 nibbles, 32 E4M3 block scales, 64 E4M3 rope
// bytes per 576-value row (and the 576-byte FP8 row it is compared with).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace smla {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDim = kLatent + kRope;
constexpr int kBlock = 16;                   // latent values per scale
constexpr int kScaleOff = kLatent / 2;       // 256
constexpr int kRopeOff = kScaleOff + kLatent / kBlock;  // 288
constexpr int kRowBytes = kRopeOff + kRope;  // 352
// The lean FP8 row of the same section's byte table: 576 E4M3 bytes, dim order.
constexpr int kFp8RowBytes = kDim;           // 576
constexpr int kPageRows = 64;
constexpr int kMaxTopk = 2048;
constexpr int kMaxBatch = 65535;

// Decode launch plan shared by the host entry points and the kernel.
struct DecodePlan {
    int heads_per_group;  // 16, 32 or 64: heads one workgroup serves from each row
    int groups;           // heads / heads_per_group
    int splits;           // workgroups sharing one (sequence, head group)
    int per_split;        // top-k entries each split scans
    size_t partial_bytes; // bytes of one split's partial result
    size_t workspace_bytes;
};

// Row formats of the decode: the NVFP4 row, or the lean FP8 row.
enum RowFormat { kFmtNvfp4 = 0, kFmtFp8 = 1 };

// batch sequences of `tokens` query tokens each (1 for plain decode)
DecodePlan plan_decode(int batch, int tokens, int heads, int topk, RowFormat fmt);

hipError_t launch_kv_quant_append(const uint16_t *rows, int64_t n, const int32_t *slots,
                                  uint8_t *cache, int64_t num_pages, hipStream_t stream);
hipError_t launch_kv_quant_append_fp8(const uint16_t *rows, int64_t n, const int32_t *slots,
                                      uint8_t *cache, int64_t num_pages, hipStream_t stream);

hipError_t launch_stage_rows_fp8(const uint8_t *cache, int64_t num_pages,
                                 const int32_t *page_table, int32_t max_pages,
                                 const int32_t *seq_lens, const int32_t *topk_idx, int32_t batch,
                                 int32_t topk, uint8_t *staged, int32_t *staged_topk,
                                 hipStream_t stream);

// top-k select: uint32 words of workspace per query, and the launches
int64_t topk_workspace_stride(int64_t ld);
hipError_t launch_topk_select(const float *scores, int64_t ld, const int32_t *seq_lens,
                              int32_t batch, int32_t topk, int32_t *out, uint32_t *ws,
                              hipStream_t stream);

hipError_t launch_sparse_mla_decode(const uint16_t *q, const uint8_t *cache, int64_t num_pages,
                                    const int32_t *page_table, int32_t max_pages,
                                    const int32_t *seq_lens, const int32_t *topk_idx,
                                    int32_t batch, int32_t tokens, int32_t heads, int32_t topk,
                                    float scale, float *out, float *lse, void *workspace,
                                    const DecodePlan &plan, RowFormat fmt, hipStream_t stream,
                                    const uint16_t *new_rows = nullptr,
                                    const int32_t *new_slots = nullptr);

}  // namespace smla
