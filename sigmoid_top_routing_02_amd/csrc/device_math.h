// Device-side scalar arithmetic shared by the kernels of this library:
// bf16 widening, the fixed binary32 sigmoid used for routing, the E4M3
// encoder and the 1x128 / 128x128 scale rule.  Everything here is exact IEEE
// binary32 arithmetic with explicit FMAs (the library is built with
// -ffp-contract=off), so results are reproducible bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Sigmoid used for the router affinity ("DeepSeek-V3 Technical Report" notes,
// MoE-routing paragraph: sigmoid affinity to each expert's centroid).  The
// pages give no arithmetic; this library fixes one:
//   exp(y): y < -87 -> 0, y > 88.72 -> +inf, else n = rint(y * log2e),
//           r = y - n*ln2 in two FMA steps (Cody-Waite: 16-bit head of ln2,
//           then its tail), p = degree-7 Taylor polynomial of e^r by Horner
//           with coefficients rounded 1/k!, result p * 2^n (exact ldexp).
//   sigmoid(x) = 1 / (1 + exp(-x))  with IEEE add and divide.
__device__ __forceinline__ float exp_fixed(float y) {
    if (y < -87.0f) return 0.0f;
    if (y > 88.72f) return __builtin_inff();
    const float n = __builtin_rintf(y * 0x1.715476p+0f);
    float r = __builtin_fmaf(-n, 0x1.62e400p-1f, y);
    r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
    float p = 0x1.a01a02p-13f;              // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f); // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);  // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);  // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);  // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);            // 1/2!
    p = __builtin_fmaf(p, r, 1.0f);            // 1/1!
    p = __builtin_fmaf(p, r, 1.0f);            // 1/0!
    return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float sigmoid_fixed(float x) {
    const float den = 1.0f + exp_fixed(-x);
    return 1.0f / den;   // correctly rounded binary32 division (HIP default)
}

// Total order on binary32 keys as unsigned integers (larger key -> larger
// integer), after mapping -0 to +0 and NaN to -inf.
__device__ __forceinline__ uint32_t orderable_key(float v) {
    if (v != v) v = -__builtin_inff();
    if (v == 0.0f) v = 0.0f;
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// OCP E4M3 encoding of four binary32 values into one word (a in the low
// byte): round to nearest, ties to even, |v| >= 448 (incl. inf) saturates to
// +-448, NaN -> 0x7F with its sign.  The gfx950 conversion instruction rounds
// the same way; it would turn |v| > 464 and inf into NaN, so larger
// magnitudes are clamped to 448 first (a comparison with NaN is false, so NaN
// passes), and it returns 0xFF for every NaN, so a NaN gets its sign back
// afterwards.  Checked on the GPU, through the 1x128 quantiser, against the
// CPU reference encoder on every binary32 input with |v| <= 448 and every NaN
// of either sign (above 448 the quantiser only passes tile maxima times their
// rounded inverse, checked separately).
__device__ __forceinline__ float e4m3_clamp(float v) {
    return __builtin_fabsf(v) > 448.0f ? __builtin_copysignf(448.0f, v) : v;
}
__device__ __forceinline__ uint32_t e4m3_nan_fix(uint32_t w, float v, int byte) {
    if (v != v) {
        const uint32_t code = ((__float_as_uint(v) >> 24) & 0x80u) | 0x7Fu;
        w = (w & ~(0xFFu << (8 * byte))) | (code << (8 * byte));
    }
    return w;
}
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), (int)w, true);
    w = e4m3_nan_fix(w, a, 0);
    w = e4m3_nan_fix(w, b, 1);
    w = e4m3_nan_fix(w, c, 2);
    return e4m3_nan_fix(w, d, 3);
}

// 1x128 / 128x128 scale rule: inv multiplies the data, scale dequantises.
__device__ __forceinline__ void tile_scale(float amax, float& inv, float& scale) {
    const float iv = 448.0f / amax;
    if (amax == 0.0f || !(__builtin_fabsf(iv) <= 3.4028234663852886e38f)) {
        inv = 1.0f;
        scale = 1.0f;
    } else {
        inv = iv;
        scale = amax / 448.0f;
    }
}

}  // namespace moe
