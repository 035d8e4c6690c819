// Combine and bias update.
//
// Combine -- nlp-lineage summary, "The notation" (the layer's output
// equation), written for GEMM rows:
//     h'[t] = u[t] + y[shared_row0 + t] + sum_k g[t,k] * y[slot_row[t,k]]
// evaluated per element in FP32 in that order (one FMA per routed term);
// bandwidth bound.
//
// Bias update -- "DeepSeek-V3 Technical Report" notes, bias paragraph (the
// sign rule of the auxiliary-loss-free balancing):
//     count * E > T*K:  b -= gamma;   count * E < T*K:  b += gamma;
//     count * E == T*K: b unchanged.
#include "device_math.h"
#include "kernels.h"

namespace moe {
namespace {

typedef uint32_t comb_v4u __attribute__((ext_vector_type(4)));
typedef float comb_v4f __attribute__((ext_vector_type(4)));

// Each block covers COLS_PER_BLOCK columns of one token row (grid.x: column
// blocks, grid.y: tokens, strided); each thread owns one chunk of VEC columns
// (4 for FP32 Y, 8 for bf16 Y: every Y load is 16 bytes).  All K + 2 row loads
// of a chunk are issued before the first arithmetic; the arithmetic then runs
// in the fixed order above.  Y is read once and h' written once, so both go
// through non-temporal loads and stores (they would otherwise evict lines that
// are still useful and, measured on gfx950, run about 17% slower); u keeps
// ordinary loads, which measured faster.
constexpr int COMBINE_COLS_PER_BLOCK = 512;

template <bool Y_F32, int KMAX>
__global__ __launch_bounds__(128) void combine_kernel(const uint16_t* __restrict__ u,
                                                     const void* __restrict__ y,
                                                     int64_t shared_row0,
                                                     const float* __restrict__ gate,
                                                     const int32_t* __restrict__ slot_row,
                                                     int64_t T, int K, int d,
                                                     float* __restrict__ out) {
    constexpr int VEC = Y_F32 ? 4 : 8;          // columns per chunk
    constexpr int UW = VEC / 4;                 // uint2 words of u per chunk
    const int dv = d / VEC;
    const comb_v4u* yv = static_cast<const comb_v4u*>(y);
    const int64_t yrow = (int64_t)d / VEC;      // 16-byte words per Y row
    const int cv = blockIdx.x * blockDim.x + threadIdx.x;
    if (cv >= dv) return;
    for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
        float g[KMAX];
        int64_t r[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            g[k] = k < K ? gate[t * K + k] : 0.0f;
            r[k] = k < K ? slot_row[t * K + k] : 0;
        }
        uint2 uw[UW];
        comb_v4u sh = {0u, 0u, 0u, 0u}, yk[KMAX];
#pragma unroll
        for (int w = 0; w < UW; ++w) uw[w] = reinterpret_cast<const uint2*>(u + t * d)[cv * UW + w];
        if (shared_row0 >= 0) sh = __builtin_nontemporal_load(yv + (shared_row0 + t) * yrow + cv);
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < K) yk[k] = __builtin_nontemporal_load(yv + r[k] * yrow + cv);
        float a[VEC];
#pragma unroll
        for (int w = 0; w < UW; ++w) {
            a[4 * w + 0] = bf16_lo(uw[w].x);
            a[4 * w + 1] = bf16_hi(uw[w].x);
            a[4 * w + 2] = bf16_lo(uw[w].y);
            a[4 * w + 3] = bf16_hi(uw[w].y);
        }
        // the four 32-bit words of a 16-byte Y load, as VEC floats
        auto expand = [&](const comb_v4u& v, float (&f)[VEC]) {
            if constexpr (Y_F32) {
#pragma unroll
                for (int q = 0; q < 4; ++q) f[q] = __uint_as_float(v[q]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f[2 * q] = bf16_lo(v[q]);
                    f[2 * q + 1] = bf16_hi(v[q]);
                }
            }
        };
        if (shared_row0 >= 0) {
            float f[VEC];
            expand(sh, f);
#pragma unroll
            for (int q = 0; q < VEC; ++q) a[q] = a[q] + f[q];
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            float f[VEC];
            expand(yk[k], f);
#pragma unroll
            for (int q = 0; q < VEC; ++q) a[q] = __builtin_fmaf(g[k], f[q], a[q]);
        }
        comb_v4f* o = reinterpret_cast<comb_v4f*>(out + t * d) + cv * (VEC / 4);
#pragma unroll
        for (int w = 0; w < VEC / 4; ++w) {
            const comb_v4f v = {a[4 * w], a[4 * w + 1], a[4 * w + 2], a[4 * w + 3]};
            __builtin_nontemporal_store(v, o + w);
        }
    }
}

__global__ void bias_update_kernel(float* __restrict__ bias, const int32_t* __restrict__ count,
                                   int E, int64_t total, float gamma) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= E) return;
    const int64_t lhs = (int64_t)count[e] * E;
    if (lhs > total) bias[e] = bias[e] - gamma;
    else if (lhs < total) bias[e] = bias[e] + gamma;
}

}  // namespace

hipError_t launch_combine(const uint16_t* u, const void* y, int y_is_f32, int64_t shared_row0,
                          const float* gate, const int32_t* slot_row, int64_t T, int K, int d,
                          float* out, hipStream_t st) {
    const int vec = y_is_f32 ? 4 : 8;
    const int nthr = COMBINE_COLS_PER_BLOCK / vec;                 // 128 or 64
    const int dv = d / vec;
    const dim3 grid((unsigned)((dv + nthr - 1) / nthr), (unsigned)(T < 65535 ? T : 65535));
#define MOE_COMBINE(F, KM) hipLaunchKernelGGL((combine_kernel<F, KM>), dim3(grid), dim3(nthr), 0, st, u, y, \
                                              shared_row0, gate, slot_row, T, K, d, out)
    if (y_is_f32) {
        if (K <= 4) MOE_COMBINE(true, 4);
        else if (K <= 8) MOE_COMBINE(true, 8);
        else MOE_COMBINE(true, 16);
    } else {
        if (K <= 4) MOE_COMBINE(false, 4);
        else if (K <= 8) MOE_COMBINE(false, 8);
        else MOE_COMBINE(false, 16);
    }
#undef MOE_COMBINE
    return hipGetLastError();
}

hipError_t launch_bias_update(float* bias, const int32_t* count, int E, int64_t total,
                              float gamma, hipStream_t st) {
    hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, st, bias, count, E,
                       total, gamma);
    return hipGetLastError();
}

}  // namespace moe
