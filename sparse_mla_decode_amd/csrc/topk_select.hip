// topk_select: the positions of the K largest indexer scores of each query,
// the list the decode takes.
//
// "Prime Inference: serving GLM-5.3 to agents is a KV-cache problem", section
// "Decode: TP4, and the copies it keeps": an indexer picks the top cached
// positions, at most 2,048 per query (and the prefill-timing figure lists the
// indexer's logits and top-k as separate steps).  The logits need the model's
// weights; this is the select over given scores.
//
// Radix select over an order-preserving 32-bit key of each fp32 score, in
// three digits (bits 31..21, 20..10, 9..0), then one gather pass:
//   pass 0: histogram of digit 0 over the query's L scores;
//   pass 1: every workgroup finds the bin b0 holding the K-th largest key
//           from that histogram (and how many keys lie above it), then
//           histograms digit 1 of the keys in bin b0;
//   pass 2: likewise b1, then digit 2 of the keys with digits (b0, b1);
//   gather: with the threshold key T = (b0, b1, b2) and n_gt keys above it,
//           every key > T is written, and the first K - n_gt keys equal to T
//           that claim a place.
// Each pass is one launch over (query, 4096-score chunk) workgroups; a
// workgroup histograms its chunk in LDS and adds its non-empty bins to the
// query's histogram with global atomics; the gather reserves output places
// with one atomic per workgroup.  Which of several equal scores at the
// threshold are taken, and the order of the list, are unspecified.
//
// Workspace, per query: hist0[2048], hist1[2048], hist2[1024], state[4]
// (b0, above0, b1, above1), count[2], all uint32.  It must be zero before its
// first use; each call leaves hist0 and hist1 zero again (pass 2 clears
// hist0, the gather clears hist1) and pass 0 clears hist2 and count, so any
// later call may reuse it.
#include "smla_internal.h"

namespace smla {
namespace {

constexpr int kChunk = 4096;          // scores per workgroup
constexpr int kThreads = 256;
constexpr int kPer = kChunk / (4 * kThreads);  // float4 loads per thread (4)
constexpr int kBins0 = 2048, kBins1 = 2048, kBins2 = 1024;
constexpr int kHist0 = 0, kHist1 = kBins0, kHist2 = kBins0 + kBins1;
constexpr int kState = kHist2 + kBins2;
constexpr int kCount = kState + 4;

// Larger key <=> larger score (finite scores; -0 sorts just below +0).
__device__ __forceinline__ uint32_t score_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The bin of hist[0..NB) (global) holding the k-th largest key (k >= 1), and
// the number of keys in the bins above it.  Thread t owns bins
// [NB - (t+1) NB/256, NB - t NB/256), so thread 0 holds the top ones.
template <int NB>
__device__ void find_bin(const uint32_t *hist, uint32_t k, uint32_t *scan_lds, uint32_t *res_lds,
                         uint32_t &bin, uint32_t &above) {
    constexpr int per = NB / kThreads;
    const int tid = threadIdx.x;
    const int top = NB - tid * per;  // one past this thread's highest bin
    uint32_t h[per];
    uint32_t sum = 0;
    if (tid == 0) {  // what a histogram with fewer than k keys would give
        res_lds[0] = 0u;
        res_lds[1] = 0u;
    }
#pragma unroll
    for (int i = 0; i < per; ++i) {
        h[i] = hist[top - 1 - i];
        sum += h[i];
    }
    scan_lds[tid] = sum;
    __syncthreads();
    // exclusive prefix over threads 0..tid-1 (Hillis-Steele on a copy)
    for (int d = 1; d < kThreads; d <<= 1) {
        const uint32_t v = tid >= d ? scan_lds[tid - d] : 0u;
        __syncthreads();
        scan_lds[tid] += v;
        __syncthreads();
    }
    const uint32_t before = scan_lds[tid] - sum;
    if (before < k && k <= before + sum) {
        uint32_t cum = before;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            if (cum + h[i] >= k) {
                res_lds[0] = (uint32_t)(top - 1 - i);
                res_lds[1] = cum;
                break;
            }
            cum += h[i];
        }
    }
    __syncthreads();
    bin = res_lds[0];
    above = res_lds[1];
    __syncthreads();
}

template <int LV>
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ seq_lens,
    int32_t topk, int32_t chunks, uint32_t *__restrict__ ws, int64_t ws_stride) {
    constexpr int NB = LV == 2 ? kBins2 : kBins0;
    __shared__ uint32_t h[NB];
    __shared__ uint32_t scan_lds[kThreads];
    __shared__ uint32_t res_lds[2];
    const int64_t b = blockIdx.x / chunks;
    const int c = (int)(blockIdx.x % chunks);
    const int tid = threadIdx.x;
    const int64_t L = min((int64_t)max(seq_lens[b], 0), ld);
    if (L <= topk) return;  // every position is selected: the gather alone
    const int64_t begin = (int64_t)c * kChunk;
    if (begin >= L) return;  // chunk 0 always passes
    uint32_t *q = ws + b * ws_stride;
    uint32_t prefix = 0;
    if (LV == 0) {
        if (c == 0) {
            for (int i = tid; i < kBins2; i += kThreads) q[kHist2 + i] = 0u;
            if (tid < 2) q[kCount + tid] = 0u;
        }
    } else if (LV == 1) {
        uint32_t b0, a0;
        find_bin<kBins0>(q + kHist0, (uint32_t)topk, scan_lds, res_lds, b0, a0);
        if (c == 0 && tid == 0) {
            q[kState + 0] = b0;
            q[kState + 1] = a0;
        }
        prefix = b0;
    } else {
        const uint32_t b0 = q[kState + 0], a0 = q[kState + 1];
        uint32_t b1, a1;
        find_bin<kBins1>(q + kHist1, (uint32_t)topk - a0, scan_lds, res_lds, b1, a1);
        if (c == 0) {
            if (tid == 0) {
                q[kState + 2] = b1;
                q[kState + 3] = a1;
            }
            for (int i = tid; i < kBins0; i += kThreads) q[kHist0 + i] = 0u;
        }
        prefix = (b0 << 11) | b1;
    }
    for (int i = tid; i < NB; i += kThreads) h[i] = 0u;
    __syncthreads();
    const float *row = scores + b * ld;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i0 = begin + 4 * (int64_t)(tid + kThreads * k);
        if (i0 >= L) break;
        const float4 v = *reinterpret_cast<const float4 *>(row + i0);
        const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (i0 + j >= L) break;
            const uint32_t key = score_key(x[j]);
            if (LV == 0) {
                atomicAdd(&h[key >> 21], 1u);
            } else if (LV == 1) {
                if ((key >> 21) == prefix) atomicAdd(&h[(key >> 10) & 2047u], 1u);
            } else {
                if ((key >> 10) == prefix) atomicAdd(&h[key & 1023u], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t *gh = q + (LV == 0 ? kHist0 : LV == 1 ? kHist1 : kHist2);
    for (int i = tid; i < NB; i += kThreads)
        if (h[i]) atomicAdd(&gh[i], h[i]);
}

__global__ __launch_bounds__(kThreads) void topk_gather_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ seq_lens,
    int32_t topk, int32_t chunks, uint32_t *__restrict__ ws, int64_t ws_stride,
    int32_t *__restrict__ out) {
    __shared__ uint32_t scan_lds[kThreads];
    __shared__ uint32_t res_lds[2];
    __shared__ uint32_t base_lds[2];
    const int64_t b = blockIdx.x / chunks;
    const int c = (int)(blockIdx.x % chunks);
    const int tid = threadIdx.x;
    const int64_t L = min((int64_t)max(seq_lens[b], 0), ld);
    int32_t *o = out + b * topk;
    if (L <= topk) {  // all positions, then -1
        if (c == 0)
            for (int e = tid; e < topk; e += kThreads) o[e] = e < L ? e : -1;
        return;
    }
    const int64_t begin = (int64_t)c * kChunk;
    if (begin >= L) return;
    uint32_t *q = ws + b * ws_stride;
    const uint32_t b0 = q[kState + 0], a0 = q[kState + 1];
    const uint32_t b1 = q[kState + 2], a1 = q[kState + 3];
    uint32_t b2, a2;
    find_bin<kBins2>(q + kHist2, (uint32_t)topk - a0 - a1, scan_lds, res_lds, b2, a2);
    const uint32_t T = (b0 << 21) | (b1 << 10) | b2;
    // keys above T (fewer than topk for a consistent workspace; clamped so
    // that no store can leave the query's list whatever the workspace holds)
    const uint32_t n_gt = min(a0 + a1 + a2, (uint32_t)topk);
    const uint32_t need_eq = (uint32_t)topk - n_gt;
    if (c == 0)
        for (int i = tid; i < kBins1; i += kThreads) q[kHist1 + i] = 0u;
    // this thread's keys above / at the threshold
    const float *row = scores + b * ld;
    uint32_t gt_mask = 0, eq_mask = 0;  // bit 4k + j: score i0(k) + j
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i0 = begin + 4 * (int64_t)(tid + kThreads * k);
        if (i0 >= L) break;
        const float4 v = *reinterpret_cast<const float4 *>(row + i0);
        const float x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (i0 + j >= L) break;
            const uint32_t key = score_key(x[j]);
            gt_mask |= (uint32_t)(key > T) << (4 * k + j);
            eq_mask |= (uint32_t)(key == T) << (4 * k + j);
        }
    }
    const uint32_t n_gt_t = __popc(gt_mask), n_eq_t = __popc(eq_mask);
    // workgroup prefix of both counts (low 16 bits: above, high 16: equal)
    const uint32_t mine = n_gt_t | (n_eq_t << 16);
    scan_lds[tid] = mine;
    __syncthreads();
    for (int d = 1; d < kThreads; d <<= 1) {
        const uint32_t v = tid >= d ? scan_lds[tid - d] : 0u;
        __syncthreads();
        scan_lds[tid] += v;
        __syncthreads();
    }
    const uint32_t incl = scan_lds[tid];
    if (tid == kThreads - 1) {
        base_lds[0] = (incl & 0xFFFFu) ? atomicAdd(&q[kCount + 0], incl & 0xFFFFu) : 0u;
        base_lds[1] = (incl >> 16) ? atomicAdd(&q[kCount + 1], incl >> 16) : 0u;
    }
    __syncthreads();
    uint32_t pg = base_lds[0] + (incl & 0xFFFFu) - n_gt_t;  // places of this thread's keys
    uint32_t pe = base_lds[1] + (incl >> 16) - n_eq_t;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int bit = 4 * k + j;
            const int32_t pos = (int32_t)(begin + 4 * (int64_t)(tid + kThreads * k) + j);
            if ((gt_mask >> bit) & 1u) {
                if (pg < n_gt) o[pg] = pos;  // always true for a consistent workspace
                ++pg;
            } else if ((eq_mask >> bit) & 1u) {
                if (pe < need_eq) o[n_gt + pe] = pos;  // n_gt + pe < topk
                ++pe;
            }
        }
    }
}

}  // namespace

int64_t topk_workspace_stride() { return kCount + 4; }

hipError_t launch_topk_select(const float *scores, int64_t ld, const int32_t *seq_lens,
                              int32_t batch, int32_t topk, int32_t *out, uint32_t *ws,
                              hipStream_t stream) {
    const int32_t chunks = (int32_t)((ld + kChunk - 1) / kChunk);
    const dim3 grid((unsigned)((int64_t)batch * chunks)), block(kThreads);
    const int64_t stride = topk_workspace_stride();
    hipLaunchKernelGGL(topk_hist_kernel<0>, grid, block, 0, stream, scores, ld, seq_lens, topk,
                       chunks, ws, stride);
    hipLaunchKernelGGL(topk_hist_kernel<1>, grid, block, 0, stream, scores, ld, seq_lens, topk,
                       chunks, ws, stride);
    hipLaunchKernelGGL(topk_hist_kernel<2>, grid, block, 0, stream, scores, ld, seq_lens, topk,
                       chunks, ws, stride);
    hipLaunchKernelGGL(topk_gather_kernel, grid, block, 0, stream, scores, ld, seq_lens, topk,
                       chunks, ws, stride, out);
    return hipGetLastError();
}

}  // namespace smla
