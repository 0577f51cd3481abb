// sparse_mla_decode: absorbed-query MLA attention over the top-k selected
// rows of a paged NVFP4 cache, dequantised on chip.
//
// What it computes: "Prime Inference: serving GLM-5.3 to agents is a
// KV-cache problem", section "A kernel that reads four bits directly" (load
// the selected 352-byte rows, unpack on chip, score, softmax and blend; -1
// entries carry no data) and Prime Intellect's launch post, native-kernel
// paragraph (FP16 operands, FP32 accumulation; the blocks sharing a query
// merge their partial results).  Every selected row serves all heads of the
// query: "GLM-5.3 PCP/DCP long-context on H200", section 1.
//
// Work decomposition (gfx950: 256 CUs in 8 XCDs, 64-wide waves, 160 KB LDS):
//   * one 512-thread workgroup per (sequence, head group, split) and CU; a
//     head group is 32 heads (16 when a query has only 16), a split a slice
//     of the top-k list.  Waves 0-3 score, waves 4-7 contract values: one
//     wave of each kind per SIMD, so the unpack work of one kind fills the
//     VALU slots left by the other's matrix instructions;
//   * prologue (value waves): the split's entries are validated, translated
//     through the page table and compacted into LDS, so -1 padding and
//     out-of-range entries cost neither a load nor a matrix instruction; the
//     score waves load their query meanwhile;
//   * the selected rows travel HBM -> LDS still packed (352 bytes each) by
//     direct-to-LDS 16-byte loads issued by the value waves: 64 rows = 22
//     wave-wide loads of consecutive bytes; the three tiles after the one
//     being scored are loaded or in flight, in a ring of five, so the
//     gathers are coalesced and deep;
//   * scores: each score wave takes 16 rows of the tile; a lane reads the
//     packed bytes of one row, unpacks them in registers (e2m1 -> f16 by the
//     hardware converter, times the block scale with a packed f16 multiply,
//     rope bytes E4M3 -> f16; all exact) and feeds MFMA 16x16x32 f16 against
//     the query held in registers: one unpack serves every head of the group;
//   * online softmax: the first tile sets the running max; after that it
//     moves only when a score passes it by more than kSlack (log2 units), so
//     normally no max reduction, rescale or extra barrier is needed; when it
//     moves, the tile is re-weighted from its kept scores one step later;
//   * values: each value wave owns 128 of the 512 output columns; the
//     transposing 4-bit LDS read (ds_read_b64_tr_b4) hands a lane 16 rows of
//     one column still packed, which are unpacked and scaled (scales from a
//     per-tile transposed f16 table written by the score waves) and fed to
//     MFMA 32x32x16 f16; the weight sums come from one more MFMA against ones;
//   * all workgroups of one sequence run on the same XCD (consecutive
//     workgroup ids go to consecutive XCDs), so head groups re-read shared
//     rows from that XCD's L2;
//   * a split writes its normalised partial output (f16) with its running
//     max and sum to the workspace, and a second small kernel merges them (a
//     merge inside the first launch would need an agent-scope release per
//     workgroup, an L2 writeback, which costs more than the launch).
#include "smla_internal.h"
#include "decode_device.h"
#include "nvfp4_quant.h"

#include <type_traits>

namespace smla {
namespace {

using namespace dev;

constexpr int kThreads = 512;                   // 4 score waves + 4 value waves, two per SIMD
constexpr int kTile = 64;                       // selected rows per tile (16 per wave)
constexpr int kPStride = kTile + 8;             // f16 per softmax-weight row (144 B)
constexpr int kSStride = kTile + 8;             // f16 per scale-table row (144 B)
constexpr int kKSteps = kDim / 32;              // 18 score steps of 32
constexpr float kSlack = 8.0f;                  // log2 headroom before the running max moves
constexpr int kMaxSplits = 16;
constexpr int kCusPerXcd = 32;                   // 8 XCDs x 32 CUs

// The tile ring for each row format: row bytes, where the rope bytes start,
// ring slots, and how far ahead the loads run (tile s + kAhead is loaded in
// step s, into the slot of tile s - 2).  An FP8 tile is 36 KB, so its ring
// has four slots (one step of slack for the loads instead of two) and a
// split scans at most 1024 entries (4 KB of row ids).
template <int FMT> struct Ring;
template <> struct Ring<kFmtNvfp4> {
    static constexpr int kRow = kRowBytes;      // 352
    static constexpr int kRopeAt = kRopeOff;    // 288
    static constexpr int kNBuf = 5;
    static constexpr int kAhead = 3;
    static constexpr int kMaxPerSplit = kMaxTopk;
};
template <> struct Ring<kFmtFp8> {
    static constexpr int kRow = kFp8RowBytes;   // 576
    static constexpr int kRopeAt = kLatent;     // 512
    static constexpr int kNBuf = 4;
    static constexpr int kAhead = 2;
    static constexpr int kMaxPerSplit = 1024;
};

// FP8 tiles are stored with the latent 16-byte pieces of row r permuted by
// XOR with swz(r) (the rope pieces stay in place): the value waves' 8-byte
// transposing reads of 8 rows x 4 column windows then spread over all LDS
// banks instead of the two that a 576-byte row stride leaves them.
__device__ __forceinline__ int fp8_swz(int r) { return ((r >> 1) & 3) << 1; }

// FUSED (NVFP4 rows, one query token): the call appends each sequence's
// newest BF16 row first (new_rows [batch][576], new_slots [batch]), with the
// result of kv_quant_append followed by the decode.  Every workgroup of
// sequence sq quantises that row itself into LDS (the append's own code) and
// puts those bytes into its tiles wherever a list entry translates to slot
// new_slots[sq] (the bytes its loads fetched from the cache there may
// predate the append); the workgroup of split 0 and head group 0 writes the
// row to the cache.  The slot must be read by no other sequence's list in
// the same call.
template <int MB, int FMT, bool FUSED = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void sparse_mla_decode_kernel(const uint16_t *__restrict__ q, uint8_t *__restrict__ cache,
                              int64_t num_pages, const int32_t *__restrict__ page_table,
                              int32_t max_pages, const int32_t *__restrict__ seq_lens,
                              const int32_t *__restrict__ topk_idx, int32_t heads, int32_t topk,
                              float scale_log2, float *__restrict__ out, float *__restrict__ lse,
                              _Float16 *__restrict__ part_o, float *__restrict__ part_ml,
                              int32_t batch, int32_t tokens, int32_t groups, int32_t splits,
                              int32_t per_split, const uint16_t *__restrict__ new_rows,
                              const int32_t *__restrict__ new_slots) {
    static_assert(!FUSED || FMT == kFmtNvfp4, "the fused append writes NVFP4 rows");
    constexpr int HG = 16 * MB;  // heads of this workgroup
    using R = Ring<FMT>;
    constexpr bool kFp8 = FMT == kFmtFp8;
    constexpr int kNBuf = R::kNBuf;
    constexpr int kAhead = R::kAhead;
    constexpr int kRowB = R::kRow;
    constexpr int kTileBytes = kTile * kRowB;       // 22,528 or 36,864
    constexpr int kChunks = kRowB / 16;             // 16-byte pieces per row (22 or 36)
    constexpr int kDmaPerTile = kTileBytes / 1024;  // wave-wide 16-byte loads per tile (22 or 36)
    constexpr int kMaxDma = (kDmaPerTile + 3) / 4;  // per value wave (6 or 9)
    static_assert(kTileBytes % 1024 == 0, "a tile must be whole wave-wide loads");
    static_assert((kNBuf - 3) * kTileBytes >= 2 * kKSteps * 1024,
                  "the query of 32 heads is staged from ring slot 3 on");
    static_assert(kNBuf - kAhead == 2, "tile s + kAhead goes into the slot of tile s - 2");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kNBuf * kTileBytes];
    __shared__ __attribute__((aligned(16))) _Float16 p_lds[2][32 * kPStride];
    __shared__ __attribute__((aligned(16))) _Float16 st_lds[kFp8 ? 1 : 2][kFp8 ? 8 : 32 * kSStride];
    __shared__ uint32_t rowid_lds[R::kMaxPerSplit];
    __shared__ __attribute__((aligned(16))) float red_lds[2][4][32];  // per-wave tile maxima
    __shared__ float alpha_lds[2][32];    // rescale factors when the running max moved
    __shared__ float sum_lds[4][32];
    __shared__ float m_lds[32];
    __shared__ int32_t scan_lds[8];
    __shared__ __attribute__((aligned(16))) uint32_t flag_lds[2][4];
    // FUSED: the new row's 352 bytes, and which compacted list entries of
    // the split read its slot (bit p of word p / 32)
    __shared__ __attribute__((aligned(16))) uint8_t fresh_lds[FUSED ? kRowBytes : 16];
    // FUSED: the new BF16 row as the score waves load it (score wave w: 1 KB
    // holding latent values 128 w .. 128 w + 127, then rope values 16 w ..
    // 16 w + 15, then repeats of the last 16 bytes)
    __shared__ __attribute__((aligned(16))) uint8_t fresh_raw[FUSED ? 4 * 1024 : 16];
    __shared__ __attribute__((aligned(8))) uint32_t fresh_mask[FUSED ? R::kMaxPerSplit / 32 : 2];
    // FUSED: bit T of fresh_tiles[w] is set when rows 16 w .. 16 w + 15 of
    // tile T hold a marked entry (a split has at most 32 tiles)
    __shared__ uint32_t fresh_tiles[4];
    static_assert(!FUSED || R::kMaxPerSplit <= 32 * kTile, "one bit per tile");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sw = wave & 3;    // score wave: rows 16 sw ..; value wave: columns 128 sw ..
    const int n = lane & 15;    // score MFMA: row within the wave's 16 / head within 16
    const int g = lane >> 4;    // score MFMA: 8-element k group
    const int n32 = lane & 31;  // value MFMA: column within a 32-column block / head
    const int g2 = lane >> 5;   // value MFMA: 8-element k group

    // ---- which (query, head group, split): consecutive workgroups go to
    // consecutive XCDs, so all workgroups of sequence sq -- every head group,
    // split and query token of it -- share XCD sq % 8 (and rows that several
    // of its query tokens select are read from that XCD's L2).  Query b is
    // token j of sequence sq = b / tokens; it sees positions
    // [0, seq_lens[sq] - (tokens - 1 - j)) ----
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

    // number of usable entries of the split, once the value waves have
    // published their counts
    auto count_valid = [&]() {
        return __builtin_amdgcn_readfirstlane(scan_lds[0] + scan_lds[1] + scan_lds[2] + scan_lds[3]);
    };
    // ---- tile ring, loaded by the value waves: value wave v = w - 4 issues
    // the wave-wide loads i = v, v+4, ... of a tile; load i fills LDS bytes
    // [1024 i, 1024 i + 1024) of the tile, lane l the 16-byte piece
    // (64 i + l) % kChunks of row (64 i + l) / kChunks (for FP8 the latent
    // pieces of row r come from piece c ^ fp8_swz(r) of the cache row).
    // Slot (tile % kNBuf); the value waves read tile t in step t + 1, so at
    // step s the loads of tile s + kAhead go into the slot of tile s - 2 ----
    const int n_dma = (kDmaPerTile - sw + 3) / 4;
    int dma_row[kMaxDma], dma_off[kMaxDma];
#pragma unroll
    for (int k = 0; k < kMaxDma; ++k) {
        const int slot = 64 * (sw + 4 * k) + lane;
        const int r = min(slot / kChunks, kTile - 1);
        const int c = slot % kChunks;
        dma_row[k] = r;
        dma_off[k] = 16 * (kFp8 ? (c < kLatent / 16 ? (c ^ fp8_swz(r)) : c) : (c ^ nv_swz(r)));
    }
    const uint32_t ring_addr = (uint32_t)(size_t)(lds_void_t *)ring;
    // the row ids of this wave's loads of tile T, then the loads themselves
    // (split so that the id reads can be issued early)
    auto tile_rows = [&](int T, uint32_t (&rk)[kMaxDma]) {
        const uint32_t *rows = rowid_lds + T * kTile;
#pragma unroll
        for (int k = 0; k < kMaxDma; ++k) rk[k] = rows[dma_row[k]];
    };
    auto tile_dma = [&](int T, const uint32_t (&rk)[kMaxDma]) {
        const uint32_t dst = ring_addr + (uint32_t)((T % kNBuf) * kTileBytes + sw * 1024);
#pragma unroll
        for (int k = 0; k < kMaxDma; ++k)
            if (k < n_dma)
                dma16(cache + (size_t)rk[k] * kRowB + dma_off[k], dst + (uint32_t)(k * 4 * 1024));
    };
    // loads k0 .. k1 - 1 of this wave's share of tile T
    auto tile_dma_part = [&](int T, const uint32_t (&rk)[kMaxDma], int k0, int k1) {
        const uint32_t dst = ring_addr + (uint32_t)((T % kNBuf) * kTileBytes + sw * 1024);
#pragma unroll
        for (int k = 0; k < kMaxDma; ++k)
            if (k >= k0 && k < k1 && k < n_dma)
                dma16(cache + (size_t)rk[k] * kRowB + dma_off[k], dst + (uint32_t)(k * 4 * 1024));
    };
    auto issue = [&](int T) {
        uint32_t rk[kMaxDma];
        tile_rows(T, rk);
        tile_dma(T, rk);
    };
    // flags of the score waves for tile parity pb, as one 16-byte read
    auto read_flags = [&](int pb) {
        const uint4 f = *reinterpret_cast<const uint4 *>(&flag_lds[pb][0]);
        return f;
    };
    // tile t is in LDS once at most the loads of the tiles issued after it
    // are outstanding: `after` of them (value waves only)
    auto wait_tile = [&](int after) {
        if (after <= 0) {
            wait_vmcnt_n<0>();
        } else if (after == 1 && !kFp8) {
            if (n_dma == 6) wait_vmcnt_n<6>();
            else wait_vmcnt_n<5>();
        } else {
            wait_vmcnt(after * n_dma);
        }
    };
    // FUSED: the new row's slot (none: all ones); the score waves quantise
    // the row (below); the value waves clear the entry mask and the tile
    // summary
    uint32_t fresh_slot = 0xFFFFFFFFu;
    if constexpr (FUSED) {
        const int64_t ns = new_slots[sq];
        if (ns >= 0 && ns < num_pages * kPageRows) fresh_slot = (uint32_t)ns;
        if (tid >= 256 && tid - 256 < R::kMaxPerSplit / 32) fresh_mask[tid - 256] = 0u;
        if (tid >= 256 + R::kMaxPerSplit / 32 && tid - 256 - R::kMaxPerSplit / 32 < 4)
            fresh_tiles[tid - 256 - R::kMaxPerSplit / 32] = 0u;
    }
    if (wave < 4) {
        // =========================== score waves ===========================
        if (MB == 1) {  // rows 16..31 of both weight tiles stay zero: MFMA 32x32 over 16 heads
            for (int i = tid; i < 16 * kPStride; i += 256) {
                p_lds[0][16 * kPStride + i] = (_Float16)0.0f;
                p_lds[1][16 * kPStride + i] = (_Float16)0.0f;
            }
        }
        // The query goes HBM -> LDS once per workgroup, by direct-to-LDS
        // loads issued right away (score wave w issues the loads i = w, w+4,
        // ...): load i = 18 mb + j puts, for every lane, that lane's A
        // operand of score step j (heads 16 mb ..) into 1 KB of LDS, so each
        // score wave reads its operands back with one linear 16-byte read per
        // step.  The staging area starts at ring slot 3, whose first tile is
        // loaded only after the initial barrier.
        const uint32_t q_lds = ring_addr + 3u * kTileBytes;
        // FUSED: this wave's quarter of the new row, HBM -> LDS ahead of its
        // query loads (lane l < 16: latent piece l, lanes 16, 17: rope pieces;
        // the other lanes repeat piece 17 into the rest of the 1 KB)
        if constexpr (FUSED) {
            const int pc = lane < 18 ? lane : 17;
            const uint16_t *x = new_rows + (int64_t)sq * kDim;
            dma16(pc < 16 ? x + 128 * sw + 8 * pc : x + kLatent + 16 * sw + 8 * (pc - 16),
                  (uint32_t)(size_t)(lds_void_t *)fresh_raw + (uint32_t)sw * 1024u);
        }
        for (int i = sw; i < MB * kKSteps; i += 4) {
            const int mb = i / kKSteps, j = i % kKSteps;
            const int d0 = (j < 16) ? (128 * g + 8 * j) : (512 + 16 * g + 8 * (j - 16));
            dma16(q + ((int64_t)b * heads + hg * HG + mb * 16 + n) * kDim + d0,
                  q_lds + (uint32_t)i * 1024u);
        }
        // FUSED: once the row's loads have landed (the query loads issued
        // after them may still be in flight), its quarter is quantised with
        // the append's code into fresh_lds and, in the workgroup of split 0
        // and head group 0, written to the cache: lane l gives the nibble
        // byte of latent values 128 sw + 2 l, + 1; lane 8 k also the scale of
        // block 8 sw + k; lanes l < 8 the rope bytes 16 sw + 2 l, + 1
        if constexpr (FUSED) {
            wait_vmcnt((MB * kKSteps - sw + 3) / 4);
            const uint32_t *raw = reinterpret_cast<const uint32_t *>(fresh_raw + sw * 1024);
            uint32_t sc;
            const uint32_t nb = nvfp4_quant_pair(raw[lane], &sc);
            const uint32_t rp = lane < 8 ? nvfp4_rope_pair(raw[64 + lane]) : 0u;
            const int blk = 8 * sw + (lane >> 3);
            fresh_lds[64 * sw + lane] = (uint8_t)nb;
            if ((lane & 7) == 0) fresh_lds[kScaleOff + blk] = (uint8_t)sc;
            if (lane < 8)
                *reinterpret_cast<uint16_t *>(fresh_lds + kRopeOff + 16 * sw + 2 * lane) = (uint16_t)rp;
            if (split == 0 && hg == 0 && fresh_slot != 0xFFFFFFFFu) {
                uint8_t *dst = cache + (size_t)fresh_slot * kRowBytes;
                dst[64 * sw + lane] = (uint8_t)nb;
                if ((lane & 7) == 0) dst[kScaleOff + blk] = (uint8_t)sc;
                if (lane < 8) *reinterpret_cast<uint16_t *>(dst + kRopeOff + 16 * sw + 2 * lane) = (uint16_t)rp;
            }
        }
        // the two barriers of the value waves' prologue; the query is in LDS
        // after the second
        __syncthreads();
        const int n_valid = count_valid();
        const int n_tiles = (n_valid + kTile - 1) / kTile;
        wait_vmcnt_n<0>();
        __syncthreads();
        // FUSED: the tiles in which this wave's rows take the new row
        // (complete after the second barrier)
        uint32_t my_tiles = 0u;
        if constexpr (FUSED) my_tiles = __builtin_amdgcn_readfirstlane(fresh_tiles[sw]);
        // The query in registers as f16 A operands: A[m = head][k = 8g+i] at
        // score step j holds dim 128g + 8j + i (latent, j < 16) or
        // 512 + 16g + 8(j-16) + i (rope), the dims the row unpack produces.
        half8_t qa[MB][kKSteps];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < kKSteps; ++j) {
                const uint4 v = *reinterpret_cast<const uint4 *>(
                    ring + 3 * kTileBytes + (mb * kKSteps + j) * 1024 + 16 * lane);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                half2_t h[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) h[i] = bf16x2_to_f16x2(w4[i]);
                qa[mb][j] = join(h[0], h[1], h[2], h[3]);
            }
        // the value waves load the first tiles and wait until tile 0 is in LDS
        __syncthreads();
        const int row = sw * 16 + n;  // this lane's row within a tile
        // running max per head (log2 units), set by the first tile (0 while
        // that tile is scored, so that its d are the scores themselves)
        float m_run[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) m_run[mb][r] = 0.0f;

        // this wave's packed bytes of one tile, dims 128g .. 128g+127 and rope
        // 16g .. 16g+15: NVFP4 -- 4 x 16 B of nibbles, the 8 block scales, 16
        // rope bytes; FP8 -- 8 x 16 B of latent bytes, 16 rope bytes
        struct PackedNvfp4 {
            uint4 nib[4];
            uint2 sc;
            uint4 rope;
        };
        struct PackedFp8 {
            uint4 lat[8];
            uint4 rope;
        };
        using Packed = typename std::conditional<kFp8, PackedFp8, PackedNvfp4>::type;
        // FP8: the byte offsets of this lane's 8 latent pieces within its row
        // (pieces permuted by fp8_swz(row))
        int lat_off[8];
#pragma unroll
        for (int jp = 0; jp < 8; ++jp) lat_off[jp] = 16 * (8 * g + (jp ^ fp8_swz(row)));
        // NVFP4: the byte offsets of this lane's nibble pieces, scales and
        // rope bytes within its row (pieces swapped by nv_swz(row))
        int nib_off[4];
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) nib_off[jp] = 16 * ((4 * g + jp) ^ nv_swz(row));
        const int sc_off = 16 * ((kScaleOff / 16 + (g >> 1)) ^ nv_swz(row)) + 8 * (g & 1);
        const int rope_off = 16 * ((kRopeOff / 16 + g) ^ nv_swz(row));
        auto load_packed = [&](int T, Packed &pk) {
            const uint8_t *rp = ring + (T % kNBuf) * kTileBytes + row * kRowB;
            if constexpr (kFp8) {
#pragma unroll
                for (int jp = 0; jp < 8; ++jp) pk.lat[jp] = *reinterpret_cast<const uint4 *>(rp + lat_off[jp]);
            } else {
#pragma unroll
                for (int jp = 0; jp < 4; ++jp) pk.nib[jp] = *reinterpret_cast<const uint4 *>(rp + nib_off[jp]);
                pk.sc = *reinterpret_cast<const uint2 *>(rp + sc_off);
            }
            pk.rope = *reinterpret_cast<const uint4 *>(rp + (kFp8 ? R::kRopeAt + 16 * g : rope_off));
        };
        // unpack and score: d = scale_log2 * q.k - m_run of this wave's 16
        // rows (-inf for rows past the end of the list); sp = the {S,S}
        // block-scale pairs
        auto score = [&](int T, const Packed &pk, float (&d)[MB][4], half2_t (&sp)[8]) {
            float4_t acc[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = float4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (kFp8) {
                // E4M3 latent bytes -> f16, exact; dims 128g + 8j .. are bytes 8j ..
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t w0 = pk.lat[j >> 1][2 * (j & 1)], w1 = pk.lat[j >> 1][2 * (j & 1) + 1];
                    const half8_t kb = join(fp8x2<false>(w0), fp8x2<true>(w0), fp8x2<false>(w1),
                                            fp8x2<true>(w1));
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[mb][j], kb, acc[mb], 0, 0, 0);
                }
            } else {
                {
                    const uint32_t d0 = __builtin_amdgcn_perm(0u, pk.sc.x, 0x01010000u);
                    const uint32_t d1 = __builtin_amdgcn_perm(0u, pk.sc.x, 0x03030202u);
                    const uint32_t d2 = __builtin_amdgcn_perm(0u, pk.sc.y, 0x01010000u);
                    const uint32_t d3 = __builtin_amdgcn_perm(0u, pk.sc.y, 0x03030202u);
                    sp[0] = fp8x2<false>(d0); sp[1] = fp8x2<true>(d0);
                    sp[2] = fp8x2<false>(d1); sp[3] = fp8x2<true>(d1);
                    sp[4] = fp8x2<false>(d2); sp[5] = fp8x2<true>(d2);
                    sp[6] = fp8x2<false>(d3); sp[7] = fp8x2<true>(d3);
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t w = pk.nib[j >> 2][j & 3];
                    const half2_t sv = sp[2 * (j >> 2) + ((j & 3) >> 1)];
                    const half8_t kb = join(fp4x2<0>(w) * sv, fp4x2<1>(w) * sv, fp4x2<2>(w) * sv,
                                            fp4x2<3>(w) * sv);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[mb][j], kb, acc[mb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const half8_t kb = join(fp8x2<false>(pk.rope[2 * t]), fp8x2<true>(pk.rope[2 * t]),
                                        fp8x2<false>(pk.rope[2 * t + 1]), fp8x2<true>(pk.rope[2 * t + 1]));
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[mb][16 + t], kb, acc[mb], 0, 0, 0);
            }
            if ((T + 1) * kTile <= n_valid) {  // uniform: every tile but the last is full
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) d[mb][r] = fmaf(acc[mb][r], scale_log2, -m_run[mb][r]);
            } else {
                const bool valid = T * kTile + row < n_valid;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        d[mb][r] = valid ? fmaf(acc[mb][r], scale_log2, -m_run[mb][r]) : -INFINITY;
            }
        };
        // f16 softmax weights 2^d of a tile (d relative to the running max), to LDS
        auto write_weights = [&](int pb, const float (&d)[MB][4]) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p_lds[pb][(mb * 16 + 4 * g + r) * kPStride + row] =
                        (_Float16)__builtin_amdgcn_exp2f(d[mb][r]);
        };

        // FUSED: the rows of this wave (16 sw ..) in tile T that read the new
        // slot get the new row's bytes in LDS before the wave reads them
        // (the tile's loads have landed: it is complete one barrier before);
        // the value waves read them two barriers later
        auto patch_rows = [&](int T) {
            if constexpr (FUSED) {
                if (!((my_tiles >> T) & 1u)) return;
                const uint32_t m16 = (__builtin_amdgcn_readfirstlane(fresh_mask[2 * T + (sw >> 1)]) >>
                                      (16 * (sw & 1))) & 0xFFFFu;
                if (m16 == 0) return;
                for (int i = 0; i < 16; ++i) {
                    if (!((m16 >> i) & 1u)) continue;
                    const int r = 16 * sw + i;
                    if (lane < kRowBytes / 16)
                        *reinterpret_cast<uint4 *>(ring + (T % kNBuf) * kTileBytes + r * kRowB +
                                                   16 * (lane ^ nv_swz(r))) =
                            *reinterpret_cast<const uint4 *>(fresh_lds + 16 * lane);
                }
            }
        };
        Packed pk;
        if (n_tiles > 0) {
            patch_rows(0);
            load_packed(0, pk);
        }
        float dp[MB][4];  // d of the previous tile, for a re-weight

        for (int s = 0; s <= n_tiles + 1; ++s) {
            __syncthreads();                                            // B(s)
            // the flags of tile s - 1 (written in step s - 1), read in every
            // step (they mean something only when tile s - 1 exists) and used
            // only after the scoring, so that the read completes under it
            uint4 fl = read_flags((s + 1) & 1);
            // (a) scores of tile s from the bytes read during step s - 1,
            // relative to the running max
            float d[MB][4];
            half2_t sp[8];
            if (s < n_tiles) score(s, pk, d, sp);
            if (s == 0) {
                // the first tile sets the running max: each wave's tile
                // maxima through LDS (the parity-1 slots, which step 0 does
                // not otherwise touch), one extra barrier F0 (the value
                // waves are idle in step 0)
                if (n_tiles > 0) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float mx = row16_max(d[mb][r]);
                            if (n == 0) red_lds[1][sw][mb * 16 + 4 * g + r] = mx;
                        }
                }
                __syncthreads();                                        // F0
                if (n_tiles > 0) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int h = mb * 16 + 4 * g + r;
                            m_run[mb][r] = fmaxf(fmaxf(red_lds[1][0][h], red_lds[1][1][h]),
                                                 fmaxf(red_lds[1][2][h], red_lds[1][3][h]));
                            d[mb][r] -= m_run[mb][r];
                        }
                }
            }
            // (b) did tile s - 1 move the running max?  Then: new max from
            // the flagged waves' tile maxima (an unflagged wave's scores lie
            // within kSlack of the old max); tile s - 1 is
            // re-weighted from its kept d before S(s), and the d of tile s
            // are moved to the new max; the value waves rescale O and the
            // sum after S(s).  (The scheduling barrier and the empty asm keep
            // the flags' first use, and so the wait for them, after the
            // scoring.)
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" : "+v"(fl.x), "+v"(fl.y), "+v"(fl.z), "+v"(fl.w));
            if (s >= 1 && s - 1 < n_tiles && __builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w) != 0) {
                const int pb = (s - 1) & 1;
                float shift[MB][4];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int h = mb * 16 + 4 * g + r;
                        const float mt = fmaxf(fmaxf(m_run[mb][r], fmaxf(fl.x ? red_lds[pb][0][h] : -INFINITY,
                                                                         fl.y ? red_lds[pb][1][h] : -INFINITY)),
                                               fmaxf(fl.z ? red_lds[pb][2][h] : -INFINITY,
                                                     fl.w ? red_lds[pb][3][h] : -INFINITY));
                        shift[mb][r] = m_run[mb][r] - mt;  // <= 0
                        if (sw == 0 && n == 0) alpha_lds[pb][h] = __builtin_amdgcn_exp2f(shift[mb][r]);
                        m_run[mb][r] = mt;
                        dp[mb][r] += shift[mb][r];
                        d[mb][r] += shift[mb][r];
                    }
                write_weights(pb, dp);
                __syncthreads();                                        // S(s)
            }
            if (s >= n_tiles) continue;
            // (c) this wave's packed bytes of tile s + 1 (complete since
            // B(s)), issued first so that the reads complete under (d)
            if (s + 1 < n_tiles) {
                patch_rows(s + 1);
                load_packed(s + 1, pk);
            }
            // (d) weights of tile s, the tile's transposed block scales for
            // the value waves, and the flag (any score past max + kSlack)
            const int pb = s & 1;
            write_weights(pb, d);
            if constexpr (!kFp8) {
                // zero scales for the last tile's padding rows (see the value
                // waves); every other tile is full (a uniform branch)
                if ((s + 1) * kTile <= n_valid) {
#pragma unroll
                    for (int k = 0; k < 8; ++k) st_lds[pb][(8 * g + k) * kSStride + row] = sp[k][0];
                } else {
                    const bool real = s * kTile + row < n_valid;
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        st_lds[pb][(8 * g + k) * kSStride + row] = real ? sp[k][0] : (_Float16)0.0f;
                }
            }
            bool over = false;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) over |= d[mb][r] > kSlack;
            const bool flagged = __ballot(over) != 0;
            if (lane == 0) flag_lds[pb][sw] = flagged;
            // this wave's tile maxima per head, published only when it flagged
            // (the re-weight takes the maxima of the flagged waves only)
            if (flagged) {
                float mx[MB][4];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx[mb][r] = row16_max(d[mb][r]) + m_run[mb][r];
                if (n == 0) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        *reinterpret_cast<float4_t *>(&red_lds[pb][sw][mb * 16 + 4 * g]) =
                            float4_t{mx[mb][0], mx[mb][1], mx[mb][2], mx[mb][3]};
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) dp[mb][r] = d[mb][r];
        }
        // the final running max, for the value waves
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (sw == 0 && n == 0) m_lds[mb * 16 + 4 * g + r] = m_run[mb][r];
        __syncthreads();                                                // E
        return;
    }

    // ---- prologue (value waves): validate, translate and compact the
    // split's entries.  All index loads are issued before any is used (two
    // round trips); an entry outside its range reads a harmless in-range word
    // instead.  Thread v = tid - 256 takes entries [v per_thread, (v+1) per_thread) ----
    const int per_thread = (per_split + 255) / 256;  // <= 8
    uint32_t rid[8];
    int cnt_valid = 0, incl = 0;
    {
        const int vt = tid - 256;
        const int64_t L = (int64_t)seq_lens[sq] - (tokens - 1 - (b - sq * tokens));
        int32_t tv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = e_begin + vt * per_thread + i;
            tv[i] = (i < per_thread) ? topk_idx[(int64_t)b * topk + min(e, topk - 1)] : -1;
        }
        bool ok[8];
        int32_t pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = e_begin + vt * per_thread + i;
            const int64_t t = tv[i];
            ok[i] = i < per_thread && e < e_end && t >= 0 && t < L && (t >> 6) < max_pages;
            pv[i] = page_table[(int64_t)sq * max_pages + (ok[i] ? (t >> 6) : 0)];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t page = pv[i];
            rid[i] = (ok[i] && page >= 0 && page < num_pages)
                         ? (uint32_t)(page * kPageRows + (tv[i] & 63))
                         : 0xFFFFFFFFu;
            cnt_valid += rid[i] != 0xFFFFFFFFu;
        }
        // inclusive scan of the counts within the wave (list order preserved)
        incl = (int)wave_scan_dpp((uint32_t)cnt_valid);
        if (lane == 63) scan_lds[wave - 4] = incl;
        // Tile 0 as the compaction will write it if every one of the split's
        // first 64 entries is usable (entries a shorter split does not have
        // are padding rows, id 0).  Written now, its loads can go out right
        // after this barrier, before the compaction; scan_lds[4] says whether
        // it holds.  Those entries all lie in the first value wave.
        const int n_entries = e_end - e_begin;
        bool bad = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int p = vt * per_thread + i;
            if (i < per_thread && p < kTile) {
                const bool absent = p >= n_entries;
                bad |= !absent && rid[i] == 0xFFFFFFFFu;
                rowid_lds[p] = (absent || rid[i] == 0xFFFFFFFFu) ? 0u : rid[i];
            }
        }
        if (wave == 4) {
            const bool any_bad = __ballot(bad) != 0;
            if (lane == 0) scan_lds[4] = any_bad ? 0 : 1;
        }
    }
    __syncthreads();
    const int n_valid = count_valid();
    const int n_tiles = (n_valid + kTile - 1) / kTile;
    // tile 0 is already in rowid_lds as the compaction writes it again: its
    // loads go out now (the compaction's stores of the same ids meanwhile
    // change nothing those loads read)
    const bool early0 = n_tiles > 0 && __builtin_amdgcn_readfirstlane(scan_lds[4]) != 0;
    if (early0) issue(0);
    // the last tile is padded with row 0 of page 0 (always in the cache): the
    // loads then need no per-row guard, and the padding rows get zero weight
    const int n_pad = n_tiles * kTile;
    {
        int pos = incl - cnt_valid;
#pragma unroll
        for (int w = 0; w < 3; ++w) pos += (w < wave - 4) ? scan_lds[w] : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (rid[i] != 0xFFFFFFFFu) {
                if (FUSED && rid[i] == fresh_slot) {
                    atomicOr(&fresh_mask[pos >> 5], 1u << (pos & 31));
                    atomicOr(&fresh_tiles[(pos >> 4) & 3], 1u << (pos >> 6));
                }
                rowid_lds[pos++] = rid[i];
            }
        if (tid - 256 < n_pad - n_valid) rowid_lds[n_valid + tid - 256] = 0u;
    }
    __syncthreads();

    // =========================== value waves ===========================
    // o[cb] (MFMA 32x32x16 C layout): head 8(i/4) + 4 g2 + i%4, column
    // 128 sw + 32 cb + n32; a tile's rows enter at MFMA (rb, t) as
    // k = rows 32 rb + 16 g2 + 8 t + i
    float16_t o[4], lacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) o[cb][i] = 0.0f;
        lacc[i] = 0.0f;
    }
    half8_t ones;
#pragma unroll
    for (int i = 0; i < 8; ++i) ones[i] = (_Float16)1.0f;
    // operands of the tile awaiting contraction, held across one barrier:
    // step s contracts tile s - 2 from registers (while the score waves
    // score tile s), then reads the operands of tile s - 1
    half8_t pa[4];
    int2_t vv[4][2];       // NVFP4: packed values per (cb, rb)
    half8_t sv[4][2][2];   // NVFP4: their block scales per (cb, rb, t)
    int2_t vv8[4][4];      // FP8: E4M3 values per (cb, rt)

    // operands of tile s - 1 (read during step s, see below): the packed
    // values through the transposing 4-bit read (lanes 16G..16G+15 read 8
    // bytes = 16 columns of rows 32 rb + 16 (G/2) + 0..15; lane j of the
    // group receives column j of those rows) and the rows' block scales.
    // Reading a slot that holds no tile (before the first and after the
    // last) is harmless: those operands are never used.
    // lane parts of the LDS addresses (bytes): packed values (row
    // 16 g2 + lane % 16 of the 32-row half, columns 128 sw + 16 (lane / 16 % 2)
    // ..), block scales (block 8 sw + n32 / 16, rows 16 g2 ..), weights
    // (head n32, rows 16 g2 ..); the rest of each address is a constant
    const uint32_t v_lane = (uint32_t)((16 * g2 + (lane & 15)) * kRowB + 64 * sw + 8 * ((lane >> 4) & 1));
    const uint32_t s_lane = (uint32_t)(((8 * sw + (n32 >> 4)) * kSStride + 16 * g2) * 2);
    const uint32_t p_lane = (uint32_t)((n32 * kPStride + 16 * g2) * 2);
    // FP8: the transposing 8-bit read gives lane 8h + p of a 16-lane group
    // byte p of the 8-byte words of lanes h, h+2, .., h+14 of the group
    // (probed on the device).  So for MFMA (rb, t) lane l supplies row
    // 32 rb + 8 t + 16 (l/32) + (l%16)/2, column window 128 sw + 32 cb +
    // 16 ((l/16)%2) + 8 (l%2), and receives column 128 sw + 32 cb + n32 of
    // rows 32 rb + 16 g2 + 8 t .. + 7: its B operand, in the row order of
    // the weights.  The window's piece is permuted by fp8_swz of the row,
    // which does not depend on (rb, t), so one lane offset per cb serves all
    // four.
    uint32_t v8_lane[4];
    {
        const int r = 16 * g2 + ((lane & 15) >> 1);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
            v8_lane[cb] = (uint32_t)(r * kRowB + 16 * ((8 * sw + 2 * cb + ((lane >> 4) & 1)) ^ fp8_swz(r)) +
                                     8 * (lane & 1));
    }
    auto read_values = [&](int s, int rb) {
        const int pb = (s + 1) & 1;  // parity of tile s - 1
        const uint8_t *tb = ring + ((s + kNBuf - 1) % kNBuf) * kTileBytes;
        if constexpr (kFp8) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const uint8_t *vb = tb + v8_lane[cb];
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    vv8[cb][2 * rb + t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_int2_t *)(
                        (__attribute__((address_space(3))) const uint8_t *)(vb + (32 * rb + 8 * t) * kRowB)));
            }
        } else {
            // piece 4 sw + cb of the lane's row sits at 4 sw + (cb ^ nv_swz(row))
            const uint8_t *vb0 = tb + v_lane + 16 * nv_swz(lane & 15);
            const uint8_t *vb1 = tb + v_lane + 16 * (1 - nv_swz(lane & 15));
            const uint8_t *sb = reinterpret_cast<const uint8_t *>(st_lds[pb]) + s_lane;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                // columns 128 sw + 32 cb + n32: packed bytes 16 cb further, block 2 cb further
                vv[cb][rb] = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_int2_t *)(
                    (__attribute__((address_space(3))) const uint8_t *)((cb & 1 ? vb1 : vb0) + 32 * rb * kRowB + 32 * (cb >> 1))));
                const half8_t *sp8 = reinterpret_cast<const half8_t *>(sb + (2 * cb * kSStride + 32 * rb) * 2);
                sv[cb][rb][0] = sp8[0];
                sv[cb][rb][1] = sp8[1];
            }
        }
    };

    // The last tile's padding rows (row 0 of page 0) carry zero weight, but a
    // zero weight times a NaN value is NaN, so their value operands are made
    // zero and bytes of rows nobody selected cannot reach the output: NVFP4 --
    // the score waves write zero block scales for them; FP8 -- the bytes are
    // cleared here once read.  rem = real rows of the tile (1..63); operand
    // byte i of (cb, rt) is row 32 (rt / 2) + 16 g2 + 8 (rt % 2) + i.
    auto mask_padding = [&](int rem) {
        if constexpr (kFp8) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int k = min(max(rem - (32 * (rt >> 1) + 16 * g2 + 8 * (rt & 1)), 0), 8);
                const uint32_t m0 = k >= 4 ? 0xFFFFFFFFu : (1u << (8 * k)) - 1u;
                const uint32_t m1 = k >= 8 ? 0xFFFFFFFFu : (k <= 4 ? 0u : (1u << (8 * (k - 4))) - 1u);
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    vv8[cb][rt][0] &= (int)m0;
                    vv8[cb][rt][1] &= (int)m1;
                }
            }
        }
    };

    // tiles 0 and 1 first, then wait until tile 0 is in LDS; tile 2 follows
    // in step 0, after B(0).  A wave's direct-to-LDS load waits at issue
    // while too many of the CU's are outstanding: issued here, tile 2's
    // loads would hold the value waves (and through B(0) the score waves)
    // until tile 1's had drained; after B(0) that wait overlaps the scoring
    // of tile 0.
    // Tile t + 1 is complete one barrier before the score waves read it at
    // the end of step t: before F0 for t = 0, before B(t) after that
    for (int T = early0 ? 1 : 0; T <= 1 && T < n_tiles; ++T) issue(T);
    if (n_tiles > 0) wait_tile(min(1, n_tiles - 1));
    __syncthreads();
    uint32_t rk[kMaxDma];  // row ids of the next tile to load
    if (kAhead < n_tiles) tile_rows(kAhead, rk);

    for (int s = 0; s <= n_tiles + 1; ++s) {
        // tile s + 1 complete before B(s): at most the tiles issued after it
        // (s + 2 .. min(s + kAhead - 1, n_tiles - 1)) may be outstanding
        if (s >= 1 && s + 1 < n_tiles) wait_tile(min(kAhead - 2, n_tiles - 2 - s));
        __syncthreads();                                                // B(s)
        asm volatile("" : "+v"(ones));  // kept in registers, not rebuilt per use
        // step s contracts tile s - 2 (operands in registers) and reads the
        // operands of tile s - 1; the flags of tile s - 1 say whether the
        // score waves re-weight it before S(s) (read in every step, used
        // at its end)
        const bool cur = s >= 1 && s - 1 < n_tiles;
        const uint4 fl = read_flags((s + 1) & 1);
        if (s == 0) {
            for (int T = 2; T < kAhead && T < n_tiles; ++T) issue(T);
            // tile 1 (read by the score waves after F0) is complete before F0
            if (1 < n_tiles) wait_tile(min(kAhead - 2, n_tiles - 2));
            __syncthreads();                                            // F0
        }
        // tile s + kAhead into the slot of tile s - 2 (read for the last time
        // in step s - 1); its row ids were read in step s - 1.  From step 2
        // on the loads are spread over the contraction, a quarter after each
        // row group, so that their waits at issue (see above) fall under the
        // matrix instructions
        const bool dma_now = s + kAhead < n_tiles;
        if (dma_now && s < 2) tile_dma(s + kAhead, rk);
        // the weights of tile s - 1 (A operands); read again after S(s)
        // when the score waves re-weight that tile
        const int pb = (s - 1) & 1;
        const uint8_t *wb = reinterpret_cast<const uint8_t *>(p_lds[pb]) + p_lane;
        auto read_weights = [&](int rt) {
            pa[rt] = *reinterpret_cast<const half8_t *>(wb + (32 * (rt >> 1) + 8 * (rt & 1)) * 2);
        };
        if (s >= 2) {
            // MFMA (rb, t) for every column block cb, so that four
            // independent accumulator chains alternate; one more MFMA
            // against ones sums this wave's quarter (rt = sw) of the weights.
            // The operands of tile s - 1 replace those of tile s - 2 as soon
            // as these are used up.
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int rb = rt >> 1, t = rt & 1;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    half8_t vb;
                    if constexpr (kFp8) {
                        const uint32_t w0 = (uint32_t)vv8[cb][rt][0], w1 = (uint32_t)vv8[cb][rt][1];
                        vb = join(fp8x2<false>(w0), fp8x2<true>(w0), fp8x2<false>(w1), fp8x2<true>(w1));
                    } else {
                        const uint32_t w = (uint32_t)vv[cb][rb][t];
                        const half8_t ss = sv[cb][rb][t];
                        const half2_t s01 = {ss[0], ss[1]}, s23 = {ss[2], ss[3]}, s45 = {ss[4], ss[5]},
                                      s67 = {ss[6], ss[7]};
                        vb = join(fp4x2<0>(w) * s01, fp4x2<1>(w) * s23, fp4x2<2>(w) * s45, fp4x2<3>(w) * s67);
                    }
                    o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[rt], vb, o[cb], 0, 0, 0);
                }
                if (rt == sw) lacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[rt], ones, lacc, 0, 0, 0);
                read_weights(rt);
                if (t == 1) read_values(s, rb);
                if (dma_now) {
                    constexpr int kPer = (kMaxDma + 3) / 4;  // loads per row group (2 or 3)
                    tile_dma_part(s + kAhead, rk, kPer * rt, kPer * rt + kPer);
                }
            }
        } else {
            read_values(s, 0);
            read_values(s, 1);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) read_weights(rt);
        }
        if (kFp8 && s == n_tiles && (n_valid & (kTile - 1)) != 0) mask_padding(n_valid & (kTile - 1));
        if (s + kAhead + 1 < n_tiles) tile_rows(s + kAhead + 1, rk);
        if (cur && __builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w) != 0) {
            // tile s - 1 moved the running max: the score waves re-weight
            // it before S(s); O and the sum (tiles up to s - 2) are rescaled
            __syncthreads();                                            // S(s)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int h = 8 * (i >> 2) + 4 * g2 + (i & 3);
                if (h < HG) {
                    const float a = alpha_lds[pb][h];
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) o[cb][i] *= a;
                    lacc[i] *= a;
                }
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) read_weights(rt);
        }
    }
    // this wave's quarter of the weight sums (all 32 columns of lacc are
    // equal; lanes 0 and 32 hold the heads of g2 = 0 and 1)
    if (n32 == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = 8 * (i >> 2) + 4 * g2 + (i & 3);
            if (h < HG) sum_lds[sw][h] = lacc[i];
        }
    }
    __syncthreads();                                                    // E

    // ---- epilogue: normalise and store (or publish the split's partial) ----
    const float ln2 = 0.69314718055994530942f;
    const int vt = tid - 256;  // 0..255 over the value waves
    if (splits == 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = 8 * (i >> 2) + 4 * g2 + (i & 3);
            if (h >= HG) continue;
            const float l_tot = sum_lds[0][h] + sum_lds[1][h] + sum_lds[2][h] + sum_lds[3][h];
            const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
            float *orow = out + ((int64_t)b * heads + hg * HG + h) * kLatent + 128 * sw + n32;
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) orow[32 * cb] = o[cb][i] * inv;
        }
        if (vt < HG) {
            const float l_tot = sum_lds[0][vt] + sum_lds[1][vt] + sum_lds[2][vt] + sum_lds[3][vt];
            lse[(int64_t)b * heads + hg * HG + vt] =
                l_tot > 0.f ? (m_lds[vt] + log2f(l_tot)) * ln2 : -INFINITY;
        }
        return;
    }
    // split: the normalised partial (f16) and its (m, l) for the merge
    // kernel.  Layout: part_o [unit][split][HG][4 sw][32 n32][4 cb] -- a
    // head's 512 values in the order the value waves hold them, so that a
    // lane writes its four column blocks as one 8-byte store (column
    // 128 sw + 32 cb + n32) -- and part_ml [unit][split][HG][2] = (running
    // max in log2 units, sum).  Where other workgroups on this XCD read the
    // same rows again (two head groups, or several query tokens) the partials
    // are streamed past the L2 (non-temporal stores), which leaves the L2 to
    // those rows.  Otherwise (one head group, one token) no row is read
    // twice, and ordinary stores leave the partials in the L2 for the merge,
    // which runs on the same XCD.
    const size_t pidx = (size_t)unit * splits + split;
    const bool keep_in_l2 = groups == 1 && tokens == 1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int h = 8 * (i >> 2) + 4 * g2 + (i & 3);
        if (h >= HG) continue;
        const float l_tot = sum_lds[0][h] + sum_lds[1][h] + sum_lds[2][h] + sum_lds[3][h];
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        const half4_t x4 = {(_Float16)(o[0][i] * inv), (_Float16)(o[1][i] * inv), (_Float16)(o[2][i] * inv),
                            (_Float16)(o[3][i] * inv)};
        uint64_t *dst = reinterpret_cast<uint64_t *>(part_o) + (pidx * HG + h) * 128 + sw * 32 + n32;
        if (keep_in_l2)
            *dst = __builtin_bit_cast(uint64_t, x4);
        else
            __builtin_nontemporal_store(__builtin_bit_cast(uint64_t, x4), dst);
    }
    if (vt < HG) {
        const float l_tot = sum_lds[0][vt] + sum_lds[1][vt] + sum_lds[2][vt] + sum_lds[3][vt];
        part_ml[(pidx * HG + vt) * 2] = m_lds[vt];
        part_ml[(pidx * HG + vt) * 2 + 1] = l_tot;
    }
}

// Merge of the splits' partials: one single-wave workgroup per (unit, head)
// (four-wave workgroups were slower by 0.1-0.3 us per call), a lane per 16
// contiguous bytes of a head's partial (8 columns, two n32 positions times
// the four column blocks of the layout above); the wave of a head of
// sequence sq runs on XCD sq % 8, where the decode workgroups of sq wrote
// the partials (so they are read from that L2).
// kS is the split count rounded up to 2, 4, 8 or 16.  Every load is issued
// before any is used (one round trip): each split's 16 bytes of the lane's
// columns, and, in lane s, the (m, l) of split s, which every lane then
// takes by readlane.  Splits past the count re-read the last one and get
// weight 0.  They are combined in split order (fixed, hence deterministic):
//   M = max_s m_s,  w_s = 2^(m_s - M) l_s,  out = sum_s w_s O_s / sum_s w_s,
//   lse = ln 2 * (M + log2 sum_s w_s).
template <int kS>
__global__ __launch_bounds__(64) void merge_splits_kernel(
    const _Float16 *__restrict__ part_o, const float *__restrict__ part_ml,
    float *__restrict__ out, float *__restrict__ lse, int32_t heads, int32_t hg_size,
    int32_t groups, int32_t splits, int32_t batch, int32_t tokens) {
    const int xcd = blockIdx.x & 7;
    const int p = __builtin_amdgcn_readfirstlane((int)(blockIdx.x >> 3));
    const int per_seq = groups * hg_size;
    const int r_seq = p / per_seq;
    const int sq = (r_seq / tokens) * 8 + xcd;
    if (sq >= batch) return;
    const int b = sq * tokens + r_seq % tokens;  // query
    const int lane = threadIdx.x & 63;
    const int h = p % hg_size;
    const int unit = b * groups + (p % per_seq) / hg_size;
    half8_t os[kS];
#pragma unroll
    for (int s = 0; s < kS; ++s) {
        const size_t pidx = ((size_t)unit * splits + min(s, splits - 1)) * hg_size + h;
        os[s] = *reinterpret_cast<const half8_t *>(part_o + pidx * kLatent + 8 * lane);
    }
    const float *mlp = part_ml + (((size_t)unit * splits + min(lane, splits - 1)) * hg_size + h) * 2;
    const int mv = __builtin_bit_cast(int, mlp[0]), lv = __builtin_bit_cast(int, mlp[1]);
    float2_t ml[kS];
#pragma unroll
    for (int s = 0; s < kS; ++s)
        ml[s] = float2_t{__builtin_bit_cast(float, __builtin_amdgcn_readlane(mv, s)),
                         __builtin_bit_cast(float, __builtin_amdgcn_readlane(lv, s))};
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kS; ++s) M = fmaxf(M, (s < splits && ml[s][1] > 0.f) ? ml[s][0] : -INFINITY);
    const float Ms = M == -INFINITY ? 0.f : M;  // no usable split: every weight is 0
    float L = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kS; ++s) {
        const float w = (s < splits && ml[s][1] > 0.f) ? __builtin_amdgcn_exp2f(ml[s][0] - Ms) * ml[s][1] : 0.f;
        L += w;
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += w * (float)os[s][k];
    }
    const int head = (unit % groups) * hg_size + h;
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    // acc[4 j + cb]: column 128 (lane / 16) + 32 cb + 2 (lane % 16) + j
    float *orow = out + ((int64_t)b * heads + head) * kLatent + 128 * (lane >> 4) + 2 * (lane & 15);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
        *reinterpret_cast<float2_t *>(orow + 32 * cb) = float2_t{acc[cb] * inv, acc[4 + cb] * inv};
    if (lane == 0)
        lse[(int64_t)b * heads + head] =
            L > 0.f ? (M + log2f(L)) * 0.69314718055994530942f : -INFINITY;
}

}  // namespace

namespace {

// Splits per unit for head groups of `hg` heads.  A workgroup holds a CU,
// and the workgroups of sequence sq all run on XCD sq % 8 (32 CUs): the
// launch stays within one wave of workgroups when the busiest XCD's share
// of them fits its CUs.  At most one split per 64-row tile, at most
// kMaxSplits, and at least as many as the row-id table of a split needs.
int plan_splits(int batch, int tokens, int heads, int hg, int topk, RowFormat fmt) {
    const int seqs_per_xcd = (batch + 7) / 8;
    const int wg_per_split = seqs_per_xcd * tokens * (heads / hg);
    int s = kCusPerXcd / wg_per_split;
    const int max_s = (topk + kTile - 1) / kTile;
    s = s < 1 ? 1 : s;
    s = s > max_s ? max_s : s;
    s = s > kMaxSplits ? kMaxSplits : s;
    const int max_per = fmt == kFmtFp8 ? Ring<kFmtFp8>::kMaxPerSplit : Ring<kFmtNvfp4>::kMaxPerSplit;
    const int min_s = (topk + max_per - 1) / max_per;
    return s < min_s ? min_s : s;
}

int tiles_per_split(int topk, int splits) {
    const int per = (topk + splits - 1) / splits;
    return (per + kTile - 1) / kTile;
}

}  // namespace

DecodePlan plan_decode(int batch, int tokens, int heads, int topk, RowFormat fmt) {
    DecodePlan p;
    p.heads_per_group = heads >= 32 ? 32 : 16;
    int s = plan_splits(batch, tokens, heads, p.heads_per_group, topk, fmt);
    if (heads == 64) {
        // 16-head groups unpack every row twice as often as 32-head ones;
        // they pay when 32-head groups leave splits of at most two tiles
        // (the per-workgroup start dominates) and 16-head groups give as
        // many workgroups, each with more tiles (fewer splits to merge)
        const int s16 = plan_splits(batch, tokens, heads, 16, topk, fmt);
        const int t32 = tiles_per_split(topk, s), t16 = tiles_per_split(topk, s16);
        if (t32 <= 2 && t16 > t32 && 4 * s16 >= 2 * s) {
            p.heads_per_group = 16;
            s = s16;
        }
    }
    p.groups = heads / p.heads_per_group;
    const int units = batch * tokens * p.groups;
    p.splits = s;
    p.per_split = (topk + s - 1) / s;
    p.partial_bytes = (size_t)p.heads_per_group * kLatent * sizeof(_Float16) +
                      (size_t)p.heads_per_group * 2 * sizeof(float);
    if (s == 1) {
        p.workspace_bytes = 0;
    } else {
        const size_t o_bytes = (size_t)units * s * p.heads_per_group * kLatent * sizeof(_Float16);
        const size_t ml_bytes = (size_t)units * s * p.heads_per_group * 2 * sizeof(float);
        p.workspace_bytes = ((o_bytes + 255) & ~(size_t)255) + ((ml_bytes + 255) & ~(size_t)255);
    }
    return p;
}

namespace {

// one single-wave workgroup per (unit, head); the blocks of XCD x take the
// sequences sq = x mod 8
hipError_t launch_merge(const _Float16 *part_o, const float *part_ml, float *out, float *lse,
                        int heads, const DecodePlan &plan, int batch, int tokens,
                        hipStream_t stream) {
    const int64_t per_xcd =
        (int64_t)((batch + 7) / 8) * tokens * plan.groups * plan.heads_per_group;
    const dim3 mg((unsigned)(8 * per_xcd));
#define SMLA_MERGE(S) hipLaunchKernelGGL((merge_splits_kernel<S>), mg, dim3(64), 0, stream, part_o, part_ml, \
                                         out, lse, heads, plan.heads_per_group, plan.groups, plan.splits, \
                                         batch, tokens)
    if (plan.splits <= 2) SMLA_MERGE(2);
    else if (plan.splits <= 4) SMLA_MERGE(4);
    else if (plan.splits <= 8) SMLA_MERGE(8);
    else SMLA_MERGE(16);
#undef SMLA_MERGE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_mla_decode(const uint16_t *q, const uint8_t *cache, int64_t num_pages,
                                    const int32_t *page_table, int32_t max_pages,
                                    const int32_t *seq_lens, const int32_t *topk_idx,
                                    int32_t batch, int32_t tokens, int32_t heads, int32_t topk,
                                    float scale, float *out, float *lse, void *workspace,
                                    const DecodePlan &plan, RowFormat fmt, hipStream_t stream,
                                    const uint16_t *new_rows, const int32_t *new_slots) {
    const int blocks = ((batch + 7) / 8) * 8 * tokens * plan.groups * plan.splits;
    const bool fused = new_rows != nullptr;
    if (fused && (fmt != kFmtNvfp4 || tokens != 1)) return hipErrorInvalidValue;
    const int units = batch * tokens * plan.groups;
    _Float16 *part_o = nullptr;
    float *part_ml = nullptr;
    if (plan.splits > 1) {
        const size_t o_bytes =
            (size_t)units * plan.splits * plan.heads_per_group * kLatent * sizeof(_Float16);
        part_o = static_cast<_Float16 *>(workspace);
        part_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                            ((o_bytes + 255) & ~(size_t)255));
    }
    const float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    // the kernel writes the cache only when it appends (FUSED)
    uint8_t *cache_rw = const_cast<uint8_t *>(cache);
#define SMLA_LAUNCH(MB, FMT, FU)                                                               \
    hipLaunchKernelGGL((sparse_mla_decode_kernel<MB, FMT, FU>), dim3(blocks), dim3(kThreads), 0, \
                       stream, q, cache_rw, num_pages, page_table, max_pages, seq_lens, topk_idx,    \
                       heads, topk, scale_log2, out, lse, part_o, part_ml, batch, tokens,            \
                       plan.groups, plan.splits, plan.per_split, new_rows, new_slots)
    if (fmt == kFmtFp8) {
        if (plan.heads_per_group == 32) SMLA_LAUNCH(2, kFmtFp8, false);
        else SMLA_LAUNCH(1, kFmtFp8, false);
    } else if (fused) {
        if (plan.heads_per_group == 32) SMLA_LAUNCH(2, kFmtNvfp4, true);
        else SMLA_LAUNCH(1, kFmtNvfp4, true);
    } else {
        if (plan.heads_per_group == 32) SMLA_LAUNCH(2, kFmtNvfp4, false);
        else SMLA_LAUNCH(1, kFmtNvfp4, false);
    }
#undef SMLA_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    return launch_merge(part_o, part_ml, out, lse, heads, plan, batch, tokens, stream);
}

}  // namespace smla
