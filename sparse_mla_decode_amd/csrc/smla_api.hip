// Host side of the C ABI declared in include/smla.h: argument validation
// (everything is checked before anything is launched) and dispatch.
#include "smla.h"
#include "smla_internal.h"

#include <mutex>
#include <string.h>

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SMLA_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SMLA_ERR_DEVICE;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return SMLA_ERR_DEVICE;
    return SMLA_OK;
}

// Cached per process: the library only runs on gfx950 and the answer cannot change.
int device_ok() {
    static int cached = 1;  // 1 = not yet asked
    if (cached == 1) cached = check_device();
    return cached;
}

}  // namespace

extern "C" {

const char *smla_strerror(int code) {
    switch (code) {
        case SMLA_OK: return "ok";
        case SMLA_ERR_NULL: return "a required pointer is NULL";
        case SMLA_ERR_SHAPE: return "a size argument is out of range";
        case SMLA_ERR_UNSUPPORTED: return "unsupported configuration (heads must be 16 or 64)";
        case SMLA_ERR_ALIGN: return "a pointer is not aligned as required";
        case SMLA_ERR_WORKSPACE: return "workspace missing or too small";
        case SMLA_ERR_LAUNCH: return "kernel launch failed";
        case SMLA_ERR_DEVICE: return "no gfx950 device is current";
        case SMLA_ERR_SCRATCH:
            return "the shape needs more split-partial scratch than the static no-allocation "
                   "buffer holds (SMLA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status code";
    }
}

int smla_version(void) { return 101; }

}  // extern "C"

namespace {

int append_rows(const void *rows_bf16, int64_t n, const int32_t *slot_mapping, uint8_t *cache,
                int64_t num_pages, void *stream, smla::RowFormat fmt) {
    if (n < 0 || n > INT32_MAX) return SMLA_ERR_SHAPE;
    if (num_pages < 1 || num_pages > ((int64_t)1 << 25)) return SMLA_ERR_SHAPE;
    if (n == 0) return SMLA_OK;
    if (!rows_bf16 || !slot_mapping || !cache) return SMLA_ERR_NULL;
    if (!aligned(rows_bf16, 16) || !aligned(cache, 256) || !aligned(slot_mapping, 4))
        return SMLA_ERR_ALIGN;
    const int dev = device_ok();
    if (dev != SMLA_OK) return dev;
    const uint16_t *rows = static_cast<const uint16_t *>(rows_bf16);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e =
        fmt == smla::kFmtFp8 ? smla::launch_kv_quant_append_fp8(rows, n, slot_mapping, cache, num_pages, st)
                             : smla::launch_kv_quant_append(rows, n, slot_mapping, cache, num_pages, st);
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

constexpr int32_t kMaxTokens = 16;

bool batch_ok(int32_t batch, int32_t tokens) {
    return batch >= 1 && tokens >= 1 && tokens <= kMaxTokens && (int64_t)batch * tokens <= 65535;
}

size_t workspace_bytes(int32_t batch, int32_t tokens, int32_t heads, int32_t topk,
                       smla::RowFormat fmt) {
    if (!batch_ok(batch, tokens) || (heads != 16 && heads != 64) || topk < 1 ||
        topk > SMLA_MAX_TOPK)
        return 0;
    return smla::plan_decode(batch, tokens, heads, topk, fmt).workspace_bytes;
}

// The checks of every decode argument except the workspace (host only).
int check_decode_args(const void *q_bf16, const uint8_t *cache, int64_t num_pages,
                      const int32_t *page_table, int32_t max_pages, const int32_t *seq_lens,
                      const int32_t *topk_indices, int32_t batch, int32_t tokens, int32_t heads,
                      int32_t topk, const float *out, const float *lse) {
    if (heads != 16 && heads != 64) return SMLA_ERR_UNSUPPORTED;
    if (!batch_ok(batch, tokens) || topk < 1 || topk > SMLA_MAX_TOPK || max_pages < 1 ||
        num_pages < 1 || num_pages > ((int64_t)1 << 25))
        return SMLA_ERR_SHAPE;
    if (!q_bf16 || !cache || !page_table || !seq_lens || !topk_indices || !out || !lse)
        return SMLA_ERR_NULL;
    if (!aligned(q_bf16, 16) || !aligned(out, 16) || !aligned(cache, 256) || !aligned(lse, 4) ||
        !aligned(page_table, 4) || !aligned(seq_lens, 4) || !aligned(topk_indices, 4))
        return SMLA_ERR_ALIGN;
    return SMLA_OK;
}

int decode(const void *q_bf16, const uint8_t *cache, int64_t num_pages, const int32_t *page_table,
           int32_t max_pages, const int32_t *seq_lens, const int32_t *topk_indices, int32_t batch,
           int32_t tokens, int32_t heads, int32_t topk, float softmax_scale, float *out,
           float *lse, void *workspace, size_t workspace_bytes, void *stream,
           smla::RowFormat fmt, const void *new_rows_bf16 = nullptr,
           const int32_t *new_slots = nullptr) {
    const int bad = check_decode_args(q_bf16, cache, num_pages, page_table, max_pages, seq_lens,
                                      topk_indices, batch, tokens, heads, topk, out, lse);
    if (bad != SMLA_OK) return bad;
    const smla::DecodePlan plan = smla::plan_decode(batch, tokens, heads, topk, fmt);
    if (plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan.workspace_bytes) return SMLA_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return SMLA_ERR_ALIGN;
    }
    const int dev = device_ok();
    if (dev != SMLA_OK) return dev;
    const hipError_t e = smla::launch_sparse_mla_decode(
        static_cast<const uint16_t *>(q_bf16), cache, num_pages, page_table, max_pages, seq_lens,
        topk_indices, batch, tokens, heads, topk, softmax_scale, out, lse, workspace, plan, fmt,
        static_cast<hipStream_t>(stream), static_cast<const uint16_t *>(new_rows_bf16), new_slots);
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int smla_kv_quant_append(const void *rows_bf16, int64_t n, const int32_t *slot_mapping,
                         uint8_t *cache, int64_t num_pages, void *stream) {
    return append_rows(rows_bf16, n, slot_mapping, cache, num_pages, stream, smla::kFmtNvfp4);
}

size_t smla_decode_workspace_bytes(int32_t batch, int32_t heads, int32_t topk) {
    return workspace_bytes(batch, 1, heads, topk, smla::kFmtNvfp4);
}

int smla_sparse_mla_decode(const void *q_bf16, const uint8_t *cache, int64_t num_pages,
                           const int32_t *page_table, int32_t max_pages,
                           const int32_t *seq_lens, const int32_t *topk_indices,
                           int32_t batch, int32_t heads, int32_t topk, float softmax_scale,
                           float *out, float *lse, void *workspace, size_t workspace_bytes,
                           void *stream) {
    return decode(q_bf16, cache, num_pages, page_table, max_pages, seq_lens, topk_indices, batch,
                  1, heads, topk, softmax_scale, out, lse, workspace, workspace_bytes, stream,
                  smla::kFmtNvfp4);
}

int smla_append_decode(const void *new_rows_bf16, const int32_t *new_slots, const void *q_bf16,
                       uint8_t *cache, int64_t num_pages, const int32_t *page_table,
                       int32_t max_pages, const int32_t *seq_lens, const int32_t *topk_indices,
                       int32_t batch, int32_t heads, int32_t topk, float softmax_scale, float *out,
                       float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    if (!new_rows_bf16 || !new_slots) return SMLA_ERR_NULL;
    if (!aligned(new_rows_bf16, 16) || !aligned(new_slots, 4)) return SMLA_ERR_ALIGN;
    return decode(q_bf16, cache, num_pages, page_table, max_pages, seq_lens, topk_indices, batch,
                  1, heads, topk, softmax_scale, out, lse, workspace, workspace_bytes, stream,
                  smla::kFmtNvfp4, new_rows_bf16, new_slots);
}

int smla_kv_quant_append_fp8(const void *rows_bf16, int64_t n, const int32_t *slot_mapping,
                             uint8_t *cache, int64_t num_pages, void *stream) {
    return append_rows(rows_bf16, n, slot_mapping, cache, num_pages, stream, smla::kFmtFp8);
}

size_t smla_decode_workspace_bytes_fp8(int32_t batch, int32_t heads, int32_t topk) {
    return workspace_bytes(batch, 1, heads, topk, smla::kFmtFp8);
}

int smla_sparse_mla_decode_fp8(const void *q_bf16, const uint8_t *cache, int64_t num_pages,
                               const int32_t *page_table, int32_t max_pages,
                               const int32_t *seq_lens, const int32_t *topk_indices,
                               int32_t batch, int32_t heads, int32_t topk, float softmax_scale,
                               float *out, float *lse, void *workspace, size_t workspace_bytes,
                               void *stream) {
    return decode(q_bf16, cache, num_pages, page_table, max_pages, seq_lens, topk_indices, batch,
                  1, heads, topk, softmax_scale, out, lse, workspace, workspace_bytes, stream,
                  smla::kFmtFp8);
}

int smla_stage_rows_fp8(const uint8_t *cache, int64_t num_pages, const int32_t *page_table,
                        int32_t max_pages, const int32_t *seq_lens, const int32_t *topk_indices,
                        int32_t batch, int32_t topk, uint8_t *staged, int32_t *staged_topk,
                        void *stream) {
    if (batch < 1 || batch > 65535 || topk < 1 || topk > SMLA_MAX_TOPK || max_pages < 1 ||
        num_pages < 1 || num_pages > ((int64_t)1 << 25))
        return SMLA_ERR_SHAPE;
    if (!cache || !page_table || !seq_lens || !topk_indices || !staged || !staged_topk)
        return SMLA_ERR_NULL;
    if (!aligned(cache, 256) || !aligned(staged, 256) || !aligned(page_table, 4) ||
        !aligned(seq_lens, 4) || !aligned(topk_indices, 4) || !aligned(staged_topk, 4))
        return SMLA_ERR_ALIGN;
    const int dev = device_ok();
    if (dev != SMLA_OK) return dev;
    const hipError_t e = smla::launch_stage_rows_fp8(cache, num_pages, page_table, max_pages,
                                                     seq_lens, topk_indices, batch, topk, staged,
                                                     staged_topk, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

size_t smla_topk_workspace_bytes(int32_t batch, int64_t ld) {
    if (batch < 1 || batch > 65535 || ld < 1 || ld > ((int64_t)1 << 30)) return 0;
    return (size_t)batch * (size_t)smla::topk_workspace_stride(ld) * sizeof(uint32_t);
}

int smla_topk_select(const float *scores, int64_t ld, const int32_t *seq_lens, int32_t batch,
                     int32_t topk, int32_t *topk_indices, void *workspace, size_t workspace_bytes,
                     void *stream) {
    if (batch < 1 || batch > 65535 || topk < 1 || topk > SMLA_MAX_TOPK || ld < 1 ||
        ld > ((int64_t)1 << 30) || (ld & 3) != 0)
        return SMLA_ERR_SHAPE;
    if (!scores || !seq_lens || !topk_indices) return SMLA_ERR_NULL;
    if (!aligned(scores, 16) || !aligned(seq_lens, 4) || !aligned(topk_indices, 4))
        return SMLA_ERR_ALIGN;
    if (!workspace || workspace_bytes < smla_topk_workspace_bytes(batch, ld))
        return SMLA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SMLA_ERR_ALIGN;
    if ((int64_t)batch * ((ld + 4095) / 4096) > INT32_MAX) return SMLA_ERR_SHAPE;
    const int dev = device_ok();
    if (dev != SMLA_OK) return dev;
    const hipError_t e = smla::launch_topk_select(scores, ld, seq_lens, batch, topk, topk_indices,
                                                  static_cast<uint32_t *>(workspace),
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

size_t smla_decode_workspace_bytes_mtp(int32_t batch, int32_t tokens, int32_t heads,
                                       int32_t topk) {
    return workspace_bytes(batch, tokens, heads, topk, smla::kFmtNvfp4);
}

int smla_sparse_mla_decode_mtp(const void *q_bf16, const uint8_t *cache, int64_t num_pages,
                               const int32_t *page_table, int32_t max_pages,
                               const int32_t *seq_lens, const int32_t *topk_indices,
                               int32_t batch, int32_t tokens, int32_t heads, int32_t topk,
                               float softmax_scale, float *out, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream) {
    return decode(q_bf16, cache, num_pages, page_table, max_pages, seq_lens, topk_indices, batch,
                  tokens, heads, topk, softmax_scale, out, lse, workspace, workspace_bytes,
                  stream, smla::kFmtNvfp4);
}

}  // extern "C"

// ---- the decode that allocates nothing ----
// The split partials of smla_sparse_mla_decode_noalloc live in this static
// device array (one copy per GPU, each at its own address).  In host code
// the name `scratch` is only a host-side stand-in: its device address comes
// from hipGetSymbolAddress, taken once per device with that device current,
// and only that address is ever handed to a kernel.
namespace {

__device__ __attribute__((aligned(256))) uint8_t scratch[SMLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices] = {};

// device address of the current device's scratch array (SMLA_OK), looked up
// on the first call on each device and cached
int scratch_address(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SMLA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return SMLA_ERR_DEVICE;
        scratch_ptr[dev] = p;
    }
    *ptr = scratch_ptr[dev];
    return SMLA_OK;
}

}  // namespace

extern "C" int smla_sparse_mla_decode_noalloc(const void *q_bf16, const uint8_t *cache,
                                              int64_t num_pages, const int32_t *page_table,
                                              int32_t max_pages, const int32_t *seq_lens,
                                              const int32_t *topk_indices, int32_t batch,
                                              int32_t heads, int32_t topk, float softmax_scale,
                                              float *out, float *lse, void *stream) {
    const int bad = check_decode_args(q_bf16, cache, num_pages, page_table, max_pages, seq_lens,
                                      topk_indices, batch, 1, heads, topk, out, lse);
    if (bad != SMLA_OK) return bad;
    const size_t need = workspace_bytes(batch, 1, heads, topk, smla::kFmtNvfp4);
    if (need > SMLA_NOALLOC_SCRATCH_BYTES) return SMLA_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        const int dev = device_ok();
        if (dev != SMLA_OK) return dev;
        const int e = scratch_address(&ws);
        if (e != SMLA_OK) return e;
    }
    return decode(q_bf16, cache, num_pages, page_table, max_pages, seq_lens, topk_indices, batch, 1,
                  heads, topk, softmax_scale, out, lse, ws, SMLA_NOALLOC_SCRATCH_BYTES, stream,
                  smla::kFmtNvfp4);
}
