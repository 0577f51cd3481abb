// Quantisation of one BF16 KV row into the 352-byte NVFP4 row, by 32 lanes
// (lane j takes latent block j, values 16j .. 16j+15, and rope values 2j,
// 2j+1) or by four waves of 64 lanes (two latent values per lane).
// Format: "Prime Inference: serving GLM-5.3 to agents is a KV-cache
// problem", section "Four bits per latent value: where 352 comes from" (512
// e2m1 values with one E4M3 scale per 16, the 64 rope values as E4M3).  The
// rounding rules (scale = E4M3 nearest amax/6, nibble = e2m1 nearest x/scale,
// ties to even, sign copied) are the readings stated in include/smla.h;
// every decision is an exact fp32 operation, so the bytes are reproducible
// bit for bit.  Shared by the append kernel and the decode that appends the
// newest row itself.
#pragma once

#include "e4m3.h"

namespace smla {

// Scale code: E4M3 value nearest amax / 6, ties to even.  The fp32 quotient
// gives a first guess; exact comparisons of amax with 6 * midpoint (a
// midpoint has at most 5 significant bits, so 3 * (lo + hi) is exact) settle
// it, including exact ties.
__device__ __forceinline__ uint32_t nvfp4_scale_code(float amax) {
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
__device__ __forceinline__ uint32_t nvfp4_e2m1_code(float a, const float t[7]) {
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

// E4M3 codes of a BF16 pair (low half first) as two bytes, the rope rule.
__device__ __forceinline__ uint32_t nvfp4_rope_pair(uint32_t r) {
    return e4m3_nearest(__uint_as_float((r & 0xFFFFu) << 16)) |
           (e4m3_nearest(__uint_as_float(r & 0xFFFF0000u)) << 8);
}

// One lane's share of the row: its block's 16 nibbles (value 16j + i in
// bits 4 (i % 8) of word i / 8), its block scale, its two rope bytes.
struct Nvfp4Lane {
    uint32_t nib[2];
    uint32_t scale;
    uint32_t rope;  // bytes 0, 1
};

// lo, hi: the block's BF16 values 0-7 and 8-15; r: rope values 2j, 2j+1
__device__ __forceinline__ Nvfp4Lane nvfp4_quant_lane(uint4 lo, uint4 hi, uint32_t r) {
    Nvfp4Lane o;
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t amax_bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        amax_bits = max(amax_bits, w[i] & 0x7FFFu);
        amax_bits = max(amax_bits, (w[i] >> 16) & 0x7FFFu);
    }
    const float amax = __uint_as_float(amax_bits << 16);
    const uint32_t s = nvfp4_scale_code(amax);
    const float S = e4m3_mag(s);
    const float t[7] = {0.25f * S, 0.75f * S, 1.25f * S, 1.75f * S, 2.5f * S, 3.5f * S, 5.0f * S};
    o.nib[0] = 0u;
    o.nib[1] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t h = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        const uint32_t mag = (S == 0.0f) ? 0u : nvfp4_e2m1_code(__uint_as_float((h & 0x7FFFu) << 16), t);
        const uint32_t nib = mag | ((h >> 12) & 8u);
        o.nib[i >> 3] |= nib << ((i & 7) * 4);
    }
    o.scale = s;
    o.rope = nvfp4_rope_pair(r);
    return o;
}

// The same encoding with 64 lanes per 128 latent values: lane l takes
// values 2 (l % 8) and 2 (l % 8) + 1 of block l / 8 (w: that BF16 pair, low
// half first).  The block's amax is the largest magnitude over its 8 lanes
// (DPP quad swaps, then the half-row mirror; integer maxima of the BF16
// magnitude bits, as above), so every decision is the one nvfp4_quant_lane
// takes.  Returns the byte of the two nibbles (value 2 (l % 8) low); *scale
// receives the block's scale code.
__device__ __forceinline__ uint32_t nvfp4_quant_pair(uint32_t w, uint32_t *scale) {
    uint32_t a = max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x141, 0xF, 0xF, true));  // row_half_mirror
    const float amax = __uint_as_float(a << 16);
    const uint32_t s = nvfp4_scale_code(amax);
    const float S = e4m3_mag(s);
    const float t[7] = {0.25f * S, 0.75f * S, 1.25f * S, 1.75f * S, 2.5f * S, 3.5f * S, 5.0f * S};
    uint32_t byte = 0u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t h = i ? (w >> 16) : (w & 0xFFFFu);
        const uint32_t mag = (S == 0.0f) ? 0u : nvfp4_e2m1_code(__uint_as_float((h & 0x7FFFu) << 16), t);
        byte |= (mag | ((h >> 12) & 8u)) << (4 * i);
    }
    *scale = s;
    return byte;
}

}  // namespace smla
