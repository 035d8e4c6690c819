// Combine and bias update.
//
// Combine -- nlp-lineage summary, "The notation": the layer output is the
// input plus the shared experts plus the chosen routed experts weighted by
// their gates,
//     h'[t] = u[t] + y[shared_row0 + t] + sum_k g[t,k] * y[slot_row[t,k]]
// evaluated per element in FP32 in that order (one FMA per routed term).  One
// block per token row; 16-byte loads of the K+1 expert rows and of u, 16-byte
// FP32 stores; bandwidth bound.
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

template <bool Y_F32>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ u,
                                                      const void* __restrict__ y,
                                                      int64_t shared_row0,
                                                      const float* __restrict__ gate,
                                                      const int32_t* __restrict__ slot_row,
                                                      int64_t T, int K, int d,
                                                      float* __restrict__ out) {
    const int d4 = d / 4;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        float g[16];
        int64_t r[16];
        for (int k = 0; k < K; ++k) {
            g[k] = gate[t * K + k];
            r[k] = slot_row[t * K + k];
        }
        for (int c4 = threadIdx.x; c4 < d4; c4 += 256) {
            const uint2 uw = reinterpret_cast<const uint2*>(u + t * d)[c4];
            float4 v = make_float4(bf16_lo(uw.x), bf16_hi(uw.x), bf16_lo(uw.y), bf16_hi(uw.y));
            if (shared_row0 >= 0) {
                const float4 s = load_y4<Y_F32>(y, shared_row0 + t, d, c4);
                v.x = v.x + s.x; v.y = v.y + s.y; v.z = v.z + s.z; v.w = v.w + s.w;
            }
            for (int k = 0; k < K; ++k) {
                const float4 yk = load_y4<Y_F32>(y, r[k], d, c4);
                v.x = __builtin_fmaf(g[k], yk.x, v.x);
                v.y = __builtin_fmaf(g[k], yk.y, v.y);
                v.z = __builtin_fmaf(g[k], yk.z, v.z);
                v.w = __builtin_fmaf(g[k], yk.w, v.w);
            }
            reinterpret_cast<float4*>(out + t * d)[c4] = v;
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
    if (y_is_f32)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(256), 0, st, u, y, shared_row0,
                           gate, slot_row, T, K, d, out);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(256), 0, st, u, y, shared_row0,
                           gate, slot_row, T, K, d, out);
    return hipGetLastError();
}

hipError_t launch_bias_update(float* bias, const int32_t* count, int E, int64_t total,
                              float gamma, hipStream_t st) {
    hipLaunchKernelGGL(bias_update_kernel, dim3((E + 255) / 256), dim3(256), 0, st, bias, count, E,
                       total, gamma);
    return hipGetLastError();
}

}  // namespace moe
