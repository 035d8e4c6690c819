// Combine and bias update.
//
// Combine -- nlp-lineage summary, "The notation": the layer output is the
// input plus the shared experts plus the chosen routed experts weighted by
// their gates,
//     h'[t] = u[t] + y[shared_row0 + t] + sum_k g[t,k] * y[slot_row[t,k]]
// evaluated per element in FP32 in that order (one FMA per routed term);
// bandwidth bound.
//
// Bias update -- "DeepSeek-V3 Technical Report" notes, bias paragraph: after
// each step an overloaded expert's bias is lowered by gamma and an
// underloaded one's raised.  Overloaded: count * E > T*K (above the batch
// mean); an expert exactly at the mean is left alone.
#include "device_math.h"
#include "kernels.h"

namespace moe {
namespace {

template <bool Y_F32>
__device__ __forceinline__ float4 load_y4(const void* y, int64_t row, int d, int c4) {
    if constexpr (Y_F32) {
        return reinterpret_cast<const float4*>(static_cast<const float*>(y) + row * d)[c4];
    } else {
        const uint2 w = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(y) + row * d)[c4];
        return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    }
}

// One block per token row (grid-strided); each thread owns one or two 4-column
// chunks.  All K + 2 row loads of a chunk are issued before the first
// arithmetic, so a wave keeps up to 2 * (K + 2) loads in flight instead of waiting
// for them one by one; the arithmetic then runs in the fixed order above.
template <bool Y_F32, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ u,
                                                      const void* __restrict__ y,
                                                      int64_t shared_row0,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ slot_row,
                                                      int64_t T, int K, int d,
                                                      float* __restrict__ out) {
    constexpr int CH = KMAX > 8 ? 1 : 2;        // 4-column chunks per thread per pass
    const int d4 = d / 4;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        float g[KMAX];
        int64_t r[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            g[k] = k < K ? gate[t * K + k] : 0.0f;
            r[k] = k < K ? slot_row[t * K + k] : 0;
        }
        for (int base = threadIdx.x; base < d4; base += 256 * CH) {
            float4 v[CH], sh[CH], yk[CH][KMAX];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int c4 = base + c * 256;
                if (c4 >= d4) continue;
                const uint2 uw = reinterpret_cast<const uint2*>(u + t * d)[c4];
                v[c] = make_float4(bf16_lo(uw.x), bf16_hi(uw.x), bf16_lo(uw.y), bf16_hi(uw.y));
                if (shared_row0 >= 0) sh[c] = load_y4<Y_F32>(y, shared_row0 + t, d, c4);
#pragma unroll
                for (int k = 0; k < KMAX; ++k)
                    if (k < K) yk[c][k] = load_y4<Y_F32>(y, r[k], d, c4);
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int c4 = base + c * 256;
                if (c4 >= d4) continue;
                float4 a = v[c];
                if (shared_row0 >= 0) {
                    a.x = a.x + sh[c].x; a.y = a.y + sh[c].y; a.z = a.z + sh[c].z; a.w = a.w + sh[c].w;
                }
#pragma unroll
                for (int k = 0; k < KMAX; ++k) {
                    if (k >= K) break;
                    a.x = __builtin_fmaf(g[k], yk[c][k].x, a.x);
                    a.y = __builtin_fmaf(g[k], yk[c][k].y, a.y);
                    a.z = __builtin_fmaf(g[k], yk[c][k].z, a.z);
                    a.w = __builtin_fmaf(g[k], yk[c][k].w, a.w);
                }
                reinterpret_cast<float4*>(out + t * d)[c4] = a;
            }
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
    const unsigned grid = (unsigned)(T < 65536 ? T : 65536);
#define MOE_COMBINE(F, KM) hipLaunchKernelGGL((combine_kernel<F, KM>), dim3(grid), dim3(256), 0, st, u, y, \
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
