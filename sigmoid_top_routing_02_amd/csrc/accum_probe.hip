// FP8 MFMA accumulation probe (a measurement, not a step of the layer).
//
// "DeepSeek-V3 Technical Report" notes (learn.ifs.name), FP8-accumulation
// paragraph: on the pages' GPU the matrix-unit accumulator of FP8 products
// has limited precision (the pages put the resulting error near 2% for an
// inner dimension of 4096), which the pages fix by moving each 128-element
// partial sum into FP32 registers.
// This kernel measures the same effect for gfx950's FP8 MFMA with unit scales:
//     chained:  acc = MFMA(a_j, b_j, acc) over all slices j  (the matrix core
//               carries the accumulator from slice to slice)
//     promoted: acc = acc + MFMA(a_j, b_j, 0)                (one MFMA per
//               slice into a fresh accumulator, then an FP32 add: the layer's
//               GEMM path with every scale equal to 1)
// One wave per 16 x 16 output tile, operands loaded straight from global
// memory: this runs on a few hundred rows, so speed does not matter.
#include "kernels.h"

namespace moe {
namespace {

typedef int probe_v8i __attribute__((ext_vector_type(8)));
typedef float probe_v4f __attribute__((ext_vector_type(4)));

// 32 bytes of one MFMA operand: row `row` of a [*, K] E4M3 matrix, the lane's
// 32-byte part `kb` of slice `j`.
__device__ __forceinline__ probe_v8i probe_frag(const uint8_t* m, int64_t row, int K, int j, int kb) {
    const uint4* p = reinterpret_cast<const uint4*>(m + row * K + (int64_t)j * 128 + kb * 32);
    const uint4 x = p[0], y = p[1];
    probe_v8i f;
    f[0] = (int)x.x; f[1] = (int)x.y; f[2] = (int)x.z; f[3] = (int)x.w;
    f[4] = (int)y.x; f[5] = (int)y.y; f[6] = (int)y.z; f[7] = (int)y.w;
    return f;
}

__global__ __launch_bounds__(64) void accum_probe_kernel(const uint8_t* __restrict__ a,
                                                         const uint8_t* __restrict__ b, int N,
                                                         int K, int chained,
                                                         float* __restrict__ out) {
    const int lane = threadIdx.x;
    const int lr = lane & 15, kb = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int n0 = blockIdx.x * 16;
    probe_v4f acc = {0.f, 0.f, 0.f, 0.f};
    const int ns = K / 128;
    for (int j = 0; j < ns; ++j) {
        const probe_v8i fa = probe_frag(a, m0 + lr, K, j, kb);
        const probe_v8i fb = probe_frag(b, n0 + lr, K, j, kb);
        if (chained) {
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa, fb, acc, 0, 0, 0, 0, 0, 0);
        } else {
            const probe_v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                fa, fb, probe_v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = acc[q] + p[q];
        }
    }
    // lane holds rows 4*kb + q of column lr of the tile
#pragma unroll
    for (int q = 0; q < 4; ++q) out[(m0 + 4 * kb + q) * N + n0 + lr] = acc[q];
}

}  // namespace

hipError_t launch_accum_probe(const uint8_t* a_q, const uint8_t* b_q, int M, int N, int K,
                              int chained, float* out, hipStream_t st) {
    hipLaunchKernelGGL(accum_probe_kernel, dim3((unsigned)(N / 16), (unsigned)(M / 16)), dim3(64), 0,
                       st, a_q, b_q, N, K, chained, out);
    return hipGetLastError();
}

}  // namespace moe
