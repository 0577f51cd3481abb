// Device helpers shared by the kernels: vector types, the NVFP4 tile
// swizzle, exact format converters (e2m1 / E4M3 -> f16 through the gfx950
// scaled converters, BF16 -> f16), DPP row reductions and wave prefix sums,
// and the direct-to-LDS row load with its explicit wait.  Row format: "Prime Inference: serving
// GLM-5.3 to agents is a KV-cache problem", section "Four bits per latent
// value: where 352 comes from".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {
namespace dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) int2_t lds_int2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// NVFP4 tiles are stored with the 16-byte pieces of row r swapped in pairs
// when bit 3 of r is set (piece p at p ^ nv_swz(r)): 16 consecutive rows then
// start in 16 different 16-byte bank groups (a 352-byte row stride alone
// repeats them every 8 rows), for the score waves' 16-byte row reads and
// the value waves' transposing reads alike.
__device__ __forceinline__ int nv_swz(int r) { return (r >> 3) & 1; }

__device__ __forceinline__ half8_t join(half2_t a, half2_t b, half2_t c, half2_t d) {
    half8_t r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

__device__ __forceinline__ half4_t join2(half2_t a, half2_t b) {
    half4_t r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    return r;
}

__device__ __forceinline__ half8_t join4(half4_t a, half4_t b) {
    half8_t r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

// v plus the value of the lane the DPP control names (0 where it names none);
// ROWS masks the 16-lane rows that take the sum (the others keep v)
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t add_dpp(uint32_t v) {
    return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix over the 64 lanes of a wave, in registers: row shifts by
// 1, 2, 4 and 8 give each 16-lane row its own prefix; then rows 1 and 3 add
// lane 15 of the row before, and rows 2 and 3 add lane 31 (the row
// broadcasts of this chip's DPP).  Lane shuffles would make each of the six
// steps an LDS permute round trip.
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v) {
    v = add_dpp<0x111, 0xF>(v);  // row_shr:1
    v = add_dpp<0x112, 0xF>(v);  // row_shr:2
    v = add_dpp<0x114, 0xF>(v);  // row_shr:4
    v = add_dpp<0x118, 0xF>(v);  // row_shr:8
    v = add_dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = add_dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Reductions over the 16 lanes of a row with DPP lane moves (quad swaps,
// half-row mirror, row mirror); every lane ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));  // row_mirror
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return x;
}

// two BF16 values (low half first) -> two f16, rounded to nearest even
__device__ __forceinline__ half2_t bf16x2_to_f16x2(uint32_t w) {
    const float2_t f = {__uint_as_float(w << 16), __uint_as_float(w & 0xFFFF0000u)};
    return __builtin_convertvector(f, half2_t);
}

// e2m1 pair (byte SEL of w) -> f16 pair, exact
template <int SEL>
__device__ __forceinline__ half2_t fp4x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
// E4M3 pair (bytes 0,1 if HI is false, else 2,3 of w) -> f16 pair, exact
template <bool HI>
__device__ __forceinline__ half2_t fp8x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// One wave-wide direct-to-LDS load: lane l's 16 bytes at gptr go to LDS
// byte lds_addr + 16 l.  Written as inline assembly so that the compiler does
// not insert its own (full) waits for it before later LDS reads; the tile
// ring waits for these loads explicitly with wait_vmcnt.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(lds_addr)
                 : "memory", "m0");
}

// Wait until at most N of this wave's memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt_n() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most n of this wave's memory loads are outstanding (n is
// wave-uniform and one of the counts the tile ring produces).
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
#define SMLA_WAIT(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
        SMLA_WAIT(0) SMLA_WAIT(1) SMLA_WAIT(2) SMLA_WAIT(3) SMLA_WAIT(4) SMLA_WAIT(5)
        SMLA_WAIT(6) SMLA_WAIT(7) SMLA_WAIT(8) SMLA_WAIT(9) SMLA_WAIT(10) SMLA_WAIT(11)
        SMLA_WAIT(12) SMLA_WAIT(13) SMLA_WAIT(14) SMLA_WAIT(15) SMLA_WAIT(16) SMLA_WAIT(17)
        SMLA_WAIT(18) SMLA_WAIT(19) SMLA_WAIT(20) SMLA_WAIT(21) SMLA_WAIT(22) SMLA_WAIT(23)
        SMLA_WAIT(24)
#undef SMLA_WAIT
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

}  // namespace dev
}  // namespace smla
