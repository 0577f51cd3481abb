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
// three digits (bits 31..21, 20..10, 9..0).  Two passes read every score:
//   pass 0: histogram of digit 0 over the query's L scores (workgroups of
//           2048 to 16384 scores by row length, all of query b on XCD
//           b % 8, where pass 1 finds them in L2: LDS histogram, then the
//           non-empty bins added to the query's histogram with global
//           atomics);
//   pass 1: every workgroup finds, from that histogram, the bin b0 holding
//           the K-th largest key and the count a0 of keys above it; keys
//           above b0 go straight to the list (one atomic per workgroup
//           reserves their places and the candidates' slots), keys in b0
//           are appended to the query's candidate buffer;
//   finish: one workgroup per query loads the candidates into registers
//           and selects the remaining K - a0 keys among them (digit 1, then
//           digit 2 -- by one wave when few keys share the first two
//           digits -- then the keys above the threshold key T and the
//           first of those equal to it).
// When bin b0 holds more keys than the candidate buffer, the finish reads
// them from the scores instead (correct, slower; only for heavily tied data).
// Which of several equal scores at the threshold are taken, and the order of
// the list, are unspecified.
//
// Workspace, per query: hist0[2048], state[4] (b0, a0), count[4] (places
// taken in the list, candidates), then the candidate buffer (cap pairs of key
// and position).  It must be zero before its first use; the finish clears
// every word of its query that the call wrote, so each call leaves the
// workspace all zero, ready for a call of any shape.
#include "decode_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

// Scores per workgroup of the two full passes (threads x loads per thread x
// 4): rows under 64K scores take 2048 (256 threads, 2 float4 each), so that
// short rows still spread over many workgroups; rows under 256K take 4096
// (256 x 4); longer rows take 16384 (512 x 8), so that fewer workgroups add
// into each query's histogram.  Every thread has all its loads in flight
// before it uses any.
constexpr int64_t kMidRow = 65536;
constexpr int64_t kBigRow = 262144;
constexpr int kFinThreads = 1024;
constexpr int kBins0 = 2048, kBins1 = 2048, kBins2 = 1024;
constexpr int kHist0 = 0;
constexpr int kState = kHist0 + kBins0;
constexpr int kCount = kState + 4;    // 8-byte aligned: one 64-bit counter pair
constexpr int kCand = kCount + 4;     // candidate pairs start here (8-byte aligned)
constexpr int64_t kMaxCand = 16384;   // candidates the finish holds (16 per thread, in registers)

// Larger key <=> larger score (finite scores; -0 sorts just below +0).
__device__ __forceinline__ uint32_t score_key(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix over the threads of a workgroup (NT threads): within each
// wave in registers, then the wave totals through LDS.  REUSE: a second
// barrier lets the caller write scan_lds again afterwards (without it, each
// scan needs an array of its own).
template <int NT, bool REUSE = true>
__device__ uint32_t block_scan(uint32_t v, uint32_t *scan_lds) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    v = dev::wave_scan_dpp(v);
    if (lane == 63) scan_lds[wave] = v;
    __syncthreads();
    uint32_t off = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) off += w < wave ? scan_lds[w] : 0u;
    if constexpr (REUSE) __syncthreads();
    return v + off;
}

// Thread t of NT owns bins [NB - (t+1) NB/NT, NB - t NB/NT) of a histogram,
// so thread 0 holds the top ones.  Its bins, highest first (loaded apart
// from find_bin_of so that a caller can issue these loads before others it
// does not wait for yet):
template <int NB, int NT>
__device__ __forceinline__ void load_bins(const uint32_t *hist, uint32_t (&h)[NB / NT]) {
    constexpr int per = NB / NT;
    const int top = NB - (int)threadIdx.x * per;  // one past this thread's highest bin
#pragma unroll
    for (int i = 0; i < per; ++i) h[i] = hist[top - 1 - i];
}

// The bin of hist[0..NB) holding the k-th largest key (k >= 1), and the
// number of keys in the bins above it, from every thread's bins.  With fewer
// than k keys in the histogram the answer is (0, 0).  REUSE: scan_lds and
// res_lds may be written again afterwards (two more barriers).
template <int NB, int NT, bool REUSE = true>
__device__ void find_bin_of(const uint32_t (&h)[NB / NT], uint32_t k, uint32_t *scan_lds,
                            uint32_t *res_lds, uint32_t &bin, uint32_t &above) {
    constexpr int per = NB / NT;
    const int tid = threadIdx.x;
    const int top = NB - tid * per;  // one past this thread's highest bin
    uint32_t sum = 0;
    if (tid == 0) {
        res_lds[0] = 0u;
        res_lds[1] = 0u;
    }
#pragma unroll
    for (int i = 0; i < per; ++i) sum += h[i];
    const uint32_t before = block_scan<NT, REUSE>(sum, scan_lds) - sum;
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
    if constexpr (REUSE) __syncthreads();
}

template <int NB, int NT>
__device__ void find_bin(const uint32_t *hist, uint32_t k, uint32_t *scan_lds, uint32_t *res_lds,
                         uint32_t &bin, uint32_t &above) {
    uint32_t h[NB / NT];
    load_bins<NB, NT>(hist, h);
    find_bin_of<NB, NT>(h, k, scan_lds, res_lds, bin, above);
}

// Pass 0: histogram of digit 0.
template <int kThreads, int kPer>
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ seq_lens,
    int32_t topk, int32_t chunks, uint32_t *__restrict__ ws, int64_t ws_stride, int32_t batch) {
    __shared__ uint32_t h[kBins0];
    // workgroup i runs on XCD i % 8: query b's chunks all go to XCD b % 8
    const int64_t b = (int64_t)((blockIdx.x >> 3) / chunks) * 8 + (blockIdx.x & 7);
    const int c = (int)((blockIdx.x >> 3) % chunks);
    if (b >= batch) return;
    const int tid = threadIdx.x;
    const int64_t L = min((int64_t)max(seq_lens[b], 0), ld);
    if (L <= topk) return;  // every position is selected: the finish alone
    const int64_t begin = (int64_t)c * (4 * kPer * kThreads);
    if (begin >= L) return;  // chunk 0 always passes
    uint32_t *q = ws + b * ws_stride;
    for (int i = tid; i < kBins0; i += kThreads) h[i] = 0u;
    __syncthreads();
    const float *row = scores + b * ld;
    // every load in flight before any is used
    float4 v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i0 = begin + 4 * (int64_t)(tid + kThreads * k);
        v[k] = *reinterpret_cast<const float4 *>(row + min(i0, ld - 4));  // in the row; masked below
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i0 = begin + 4 * (int64_t)(tid + kThreads * k);
        const float x[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i0 + j < L) atomicAdd(&h[score_key(x[j]) >> 21], 1u);
    }
    __syncthreads();
    uint32_t hv[kBins0 / kThreads];
#pragma unroll
    for (int k = 0; k < kBins0 / kThreads; ++k) hv[k] = h[tid + kThreads * k];
#pragma unroll
    for (int k = 0; k < kBins0 / kThreads; ++k)
        if (hv[k]) atomicAdd(&q[kHist0 + tid + kThreads * k], hv[k]);
}

// Pass 1: keys above bin b0 to the list, keys in b0 to the candidates.
template <int kThreads, int kPer>
__global__ __launch_bounds__(kThreads) void topk_split_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ seq_lens,
    int32_t topk, int32_t chunks, uint32_t *__restrict__ ws, int64_t ws_stride, int64_t cap,
    int32_t *__restrict__ out, int32_t batch) {
    __shared__ uint32_t scan_a[kThreads / 64], scan_b[kThreads / 64];  // a wave total each
    __shared__ uint32_t res_lds[2];
    __shared__ uint32_t base_lds[2];
    // workgroup i runs on XCD i % 8: query b's chunks all go to XCD b % 8
    const int64_t b = (int64_t)((blockIdx.x >> 3) / chunks) * 8 + (blockIdx.x & 7);
    const int c = (int)((blockIdx.x >> 3) % chunks);
    if (b >= batch) return;
    const int tid = threadIdx.x;
    const int64_t L = min((int64_t)max(seq_lens[b], 0), ld);
    if (L <= topk) return;
    const int64_t begin = (int64_t)c * (4 * kPer * kThreads);
    if (begin >= L) return;
    uint32_t *q = ws + b * ws_stride;
    const float *row = scores + b * ld;
    // the thread's histogram bins first, then the chunk's scores: loads
    // complete in order, so the scores stay in flight while the threshold
    // bin is found
    uint32_t hb[kBins0 / kThreads];
    load_bins<kBins0, kThreads>(q + kHist0, hb);
    float4 v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i0 = begin + 4 * (int64_t)(tid + kThreads * k);
        v[k] = *reinterpret_cast<const float4 *>(row + min(i0, ld - 4));  // in the row; masked below
    }
    uint32_t b0, a0;
    find_bin_of<kBins0, kThreads, false>(hb, (uint32_t)topk, scan_a, res_lds, b0, a0);
    if (c == 0 && tid == 0) {
        q[kState + 0] = b0;
        q[kState + 1] = a0;
    }
    a0 = min(a0, (uint32_t)topk - 1);  // keeps every store inside the list
    uint32_t gt_mask = 0, in_mask = 0;  // bit 4k + j: score i0(k) + j
    uint32_t keys[4 * kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int64_t i0 = begin + 4 * (int64_t)(tid + kThreads * k);
        const float x[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t key = score_key(x[j]);
            keys[4 * k + j] = key;
            const bool ok = i0 + j < L;
            gt_mask |= (uint32_t)(ok && (key >> 21) > b0) << (4 * k + j);
            in_mask |= (uint32_t)(ok && (key >> 21) == b0) << (4 * k + j);
        }
    }
    const uint32_t n_gt_t = __popc(gt_mask), n_in_t = __popc(in_mask);
    const uint32_t incl = block_scan<kThreads, false>(n_gt_t | (n_in_t << 16), scan_b);
    if (tid == kThreads - 1 && incl != 0u) {
        // both counts in one 64-bit atomic (list places in the low word,
        // candidates in the high one): one request on the query's counters
        // per workgroup
        const unsigned long long add =
            (unsigned long long)(incl & 0xFFFFu) | ((unsigned long long)(incl >> 16) << 32);
        const unsigned long long old =
            atomicAdd(reinterpret_cast<unsigned long long *>(&q[kCount]), add);
        base_lds[0] = (uint32_t)old;
        base_lds[1] = (uint32_t)(old >> 32);
    }
    __syncthreads();
    uint32_t pg = base_lds[0] + (incl & 0xFFFFu) - n_gt_t;
    uint32_t pc = base_lds[1] + (incl >> 16) - n_in_t;
    int32_t *o = out + b * topk;
    uint2 *cand = reinterpret_cast<uint2 *>(q + kCand);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int bit = 4 * k + j;
            const int32_t pos = (int32_t)(begin + 4 * (int64_t)(tid + kThreads * k) + j);
            if ((gt_mask >> bit) & 1u) {
                if (pg < a0) o[pg] = pos;  // always true for a consistent workspace
                ++pg;
            } else if ((in_mask >> bit) & 1u) {
                if (pc < cap) cand[pc] = make_uint2(keys[bit], (uint32_t)pos);
                ++pc;
            }
        }
    }
}

// Finish: one workgroup per query selects the last K - a0 keys among the
// candidates (all in bin b0): digit 1, then digit 2 (one wave ranks the
// keys sharing the first two digits when they are few), then the keys above
// the threshold key and the first equal ones.
__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(
    const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ seq_lens,
    int32_t topk, uint32_t *__restrict__ ws, int64_t ws_stride, int64_t cap,
    int32_t *__restrict__ out) {
    __shared__ uint32_t h[kBins1];
    __shared__ uint32_t scan_lds[kFinThreads / 64];  // a wave total each
    __shared__ uint32_t res_lds[2];
    __shared__ uint32_t place_lds[2];
    __shared__ uint32_t sel_lds[64];
    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t L = min((int64_t)max(seq_lens[b], 0), ld);
    int32_t *o = out + b * topk;
    if (L <= topk) {  // all positions, then -1
        for (int e = tid; e < topk; e += kFinThreads) o[e] = e < L ? e : -1;
        return;
    }
    uint32_t *q = ws + b * ws_stride;
    const uint32_t b0 = q[kState + 0];
    const uint32_t a0 = min(q[kState + 1], (uint32_t)topk - 1);
    const uint32_t n_c = q[kCount + 1];
    const bool in_buf = n_c <= cap;
    const int64_t n_src = in_buf ? (int64_t)n_c : L;
    const uint2 *cand = reinterpret_cast<const uint2 *>(q + kCand);
    const float *row = scores + b * ld;
    const int lane = tid & 63;
    // This thread's candidates, i = tid + kFinThreads k: held in registers
    // for all three passes when the buffer holds them all (every load in
    // flight at once), else read from the scores in each pass.
    constexpr int kLoads = kMaxCand / kFinThreads;  // 16
    uint2 v[kLoads];
    if (in_buf) {
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const int64_t i = tid + (int64_t)kFinThreads * k;
            if (i < n_src) v[k] = cand[i];
        }
    }
    // fn(key, pos) for each of this thread's candidates (from the scores, a
    // key outside bin b0 is no candidate)
    auto each = [&](auto fn) {
        if (in_buf) {
#pragma unroll
            for (int k = 0; k < kLoads; ++k) {
                if ((int64_t)kFinThreads * k >= n_src) break;
                if (tid + (int64_t)kFinThreads * k < n_src) fn(v[k].x, v[k].y);
            }
        } else {
            for (int64_t i = tid; i < n_src; i += kFinThreads) {
                const uint32_t key = score_key(row[i]);
                if ((key >> 21) == b0) fn(key, (uint32_t)i);
            }
        }
    };
    const uint32_t need = (uint32_t)topk - a0;
    // digit 1
    for (int i = tid; i < kBins1; i += kFinThreads) h[i] = 0u;
    __syncthreads();
    each([&](uint32_t key, uint32_t) { atomicAdd(&h[(key >> 10) & 2047u], 1u); });
    __syncthreads();
    uint32_t b1, a1;
    find_bin<kBins1, kFinThreads>(h, need, scan_lds, res_lds, b1, a1);
    // digit 2 among the keys with digits (b0, b1): the threshold key T is
    // the need2-th largest of them, a2 the number above it.  Usually they are
    // a handful, which one wave ranks directly; more (heavily tied data)
    // take a histogram of digit 2.
    const uint32_t p01 = (b0 << 11) | b1;
    const uint32_t need2 = need - min(a1, need - 1);
    const uint32_t n1 = h[b1];  // their number, from the digit-1 histogram
    uint32_t T, a2;
    if (n1 <= 64) {
        if (tid == 0) place_lds[0] = 0u;
        __syncthreads();
        each([&](uint32_t key, uint32_t) {
            if ((key >> 10) == p01) {
                const uint32_t e = atomicAdd(&place_lds[0], 1u);
                if (e < 64) sel_lds[e] = key;
            }
        });
        __syncthreads();
        if (tid < 64) {
            const uint32_t n = min(place_lds[0], 64u);  // n1 for a consistent workspace
            const uint32_t mine = (uint32_t)tid < n ? sel_lds[tid] : 0u;
            uint32_t gt = 0, ge = 0;  // keys above this lane's, and at or above it
            for (uint32_t j = 0; j < n; ++j) {
                const uint32_t kj = __builtin_amdgcn_readlane(mine, j);
                gt += kj > mine;
                ge += kj >= mine;
            }
            const uint64_t hit = __ballot((uint32_t)tid < n && gt < need2 && need2 <= ge);
            if (hit != 0 && tid == (int)__builtin_ctzll(hit)) {
                res_lds[0] = mine;
                res_lds[1] = gt;
            } else if (hit == 0 && tid == 0) {  // an inconsistent workspace only
                res_lds[0] = p01 << 10;
                res_lds[1] = 0u;
            }
        }
        __syncthreads();
        T = res_lds[0];
        a2 = res_lds[1];
        __syncthreads();  // before place_lds and res_lds are used again
    } else {
        __syncthreads();  // every thread has read n1 from h
        for (int i = tid; i < kBins2; i += kFinThreads) h[i] = 0u;
        __syncthreads();
        each([&](uint32_t key, uint32_t) {
            if ((key >> 10) == p01) atomicAdd(&h[key & 1023u], 1u);
        });
        __syncthreads();
        uint32_t b2;
        find_bin<kBins2, kFinThreads>(h, need2, scan_lds, res_lds, b2, a2);
        T = (p01 << 10) | b2;
    }
    const uint32_t n_gt = min(a0 + a1 + a2, (uint32_t)topk - 1);  // keys above T
    const uint32_t need_eq = (uint32_t)topk - n_gt;
    if (tid < 2) place_lds[tid] = 0u;
    __syncthreads();
    // the keys above T after the a0 written by the split pass, then the first
    // need_eq keys equal to T: one LDS atomic per wave and kind reserves the
    // places of all its lanes (in lane order); called by every lane of a wave
    const uint64_t below = (1ull << lane) - 1ull;  // the lanes under this one
    auto place = [&](bool gt, bool eq, uint32_t pos) {
        const uint64_t mg = __ballot(gt), me = __ballot(eq);
        if ((mg | me) == 0) return;
        uint32_t bg = 0, be = 0;
        if (lane == 0) {
            if (mg) bg = atomicAdd(&place_lds[0], (uint32_t)__popcll(mg));
            if (me) be = atomicAdd(&place_lds[1], (uint32_t)__popcll(me));
        }
        bg = __builtin_amdgcn_readfirstlane(bg);  // lane 0's reservations (every lane is active)
        be = __builtin_amdgcn_readfirstlane(be);
        if (gt) {
            const uint32_t pl = a0 + bg + (uint32_t)__popcll(mg & below);
            if (pl < n_gt) o[pl] = (int32_t)pos;
        } else if (eq) {
            const uint32_t e = be + (uint32_t)__popcll(me & below);
            if (e < need_eq) o[n_gt + e] = (int32_t)pos;
        }
    };
    if (in_buf) {
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            if ((int64_t)kFinThreads * k >= n_src) break;
            const bool ok = tid + (int64_t)kFinThreads * k < n_src;
            place(ok && v[k].x > T, ok && v[k].x == T, v[k].y);
        }
    } else {
        for (int64_t i0 = 0; i0 < n_src; i0 += kFinThreads) {  // the same trip count in every lane
            const int64_t i = i0 + tid;
            uint32_t key = 0u;
            bool ok = false;
            if (i < n_src) {
                key = score_key(row[i]);
                ok = (key >> 21) == b0;
            }
            place(ok && key > T, ok && key == T, (uint32_t)i);
        }
    }
    // leave the query's workspace all zero: hist0, state, counts and the
    // candidates written (read by no one after this point)
    __syncthreads();
    for (int i = tid; i < kCand; i += kFinThreads) q[i] = 0u;
    const int64_t used = 2 * min((int64_t)n_c, cap);
    for (int64_t i = tid; i < used; i += kFinThreads) q[kCand + i] = 0u;
}

}  // namespace

int64_t topk_candidate_cap(int64_t ld) { return ld < kMaxCand ? ld : kMaxCand; }

int64_t topk_workspace_stride(int64_t ld) {
    // in uint32 words, a multiple of 64 (256 bytes) per query
    const int64_t words = kCand + 2 * topk_candidate_cap(ld);
    return (words + 63) / 64 * 64;
}

hipError_t launch_topk_select(const float *scores, int64_t ld, const int32_t *seq_lens,
                              int32_t batch, int32_t topk, int32_t *out, uint32_t *ws,
                              hipStream_t stream) {
    const int64_t stride = topk_workspace_stride(ld);
    const int64_t cap = topk_candidate_cap(ld);
#define SMLA_PASSES(NT, PER)                                                                   \
    do {                                                                                       \
        const int64_t ch = 4 * (PER) * (NT);                                                   \
        const int32_t chunks = (int32_t)((ld + ch - 1) / ch);                                  \
        const dim3 grid((unsigned)((int64_t)(batch + 7) / 8 * 8 * chunks)), block(NT);         \
        hipLaunchKernelGGL((topk_hist_kernel<NT, PER>), grid, block, 0, stream, scores, ld,    \
                           seq_lens, topk, chunks, ws, stride, batch);                         \
        hipLaunchKernelGGL((topk_split_kernel<NT, PER>), grid, block, 0, stream, scores, ld,   \
                           seq_lens, topk, chunks, ws, stride, cap, out, batch);               \
    } while (0)
    if (ld >= kBigRow) SMLA_PASSES(512, 8);
    else if (ld >= kMidRow) SMLA_PASSES(256, 4);
    else SMLA_PASSES(256, 2);
#undef SMLA_PASSES
    hipLaunchKernelGGL(topk_finish_kernel, dim3((unsigned)batch), dim3(kFinThreads), 0, stream,
                       scores, ld, seq_lens, topk, ws, stride, cap, out);
    return hipGetLastError();
}

}  // namespace smla
