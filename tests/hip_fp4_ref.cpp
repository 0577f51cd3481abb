// Host-side reference for float -> e2m1 (OCP FP4): the software conversion in
// ROCm's HIP headers (the host branch of __hip_cvt_float_to_fp4: round to
// nearest even, saturating), for the oracle's CPU tests only.  The test that
// uses it builds this file with hipcc, host code only, into a temporary
// directory; no GPU code is involved.
#include <hip/hip_fp4.h>
#include <stdint.h>

extern "C" void hip_host_e2m1(const float *x, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)(__hip_cvt_float_to_fp4(x[i], __HIP_E2M1, hipRoundNearest) & 0xF);
}
