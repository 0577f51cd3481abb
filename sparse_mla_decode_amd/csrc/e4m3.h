// E4M3 (OCP E4M3FN: bias 7, max 448, no infinities) value and nearest-code
// rules shared by the append kernels and the staged path's gather-unpack.
// Every step is an exact fp32 operation, so the codes are reproducible bit
// for bit: nearest value, ties to the even code, saturating at 448, sign of
// the input copied (-0 gives 0x80).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

// Magnitude of an E4M3 code's low 7 bits: (1 + m/8) 2^(e-7), or m 2^-9 when e = 0.
__device__ __forceinline__ float e4m3_mag(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mant = e ? (float)(8u + m) : (float)(2u * m);  // e==0: m/8 * 2^-6 = 2m * 2^-10
    int ex = e ? (int)e - 10 : -10;
    return ldexpf(mant, ex);
}

// E4M3 code (sign copied) of the value nearest v, ties to even, saturating.
__device__ __forceinline__ uint32_t e4m3_nearest(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    float a = __uint_as_float(u & 0x7FFFFFFFu);
    uint32_t code;
    if (a > 448.0f) {
        code = 0x7E;                          // past 448 only 448 is finite
    } else if (a <= 0x1p-10f) {
        code = 0;                             // half the smallest subnormal: ties to 0
    } else if (a < 0x1p-6f) {
        code = (uint32_t)rintf(a * 512.0f);   // subnormal grid m 2^-9; 8 -> 0x08 = 2^-6
    } else {
        int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // a is a normal fp32
        uint32_t m = (uint32_t)rintf(ldexpf(a, 3 - E));           // in [8, 16]
        if (m == 16u) { E += 1; m = 8u; }
        code = ((uint32_t)(E + 7) << 3) | (m - 8u);
    }
    return sign | code;
}

}  // namespace smla
