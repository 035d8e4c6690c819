// FP8 (OCP E4M3) block quantisers.  "DeepSeek-V3 Technical Report" notes
// (learn.ifs.name), FP8-tiling paragraph: activations are scaled per 1x128
// tile (one token, 128 channels) and weights per 128x128 block so that an
// outlier only affects its own group.  Scale rule (this library's reading):
// amax over the tile, inv = 448/amax, scale = amax/448 (both 1 when amax is 0
// or 448/amax overflows), q = E4M3(x * inv) with round-to-nearest-even and
// saturation.
//
// 1x128: 16 lanes own one tile (8 contiguous values each); the tile maximum
// is a 4-step xor-shuffle inside the 16-lane group.  Streams HBM with 16-byte
// loads and 8-byte stores.
// 128x128: one 256-thread block per block; each thread keeps its 64 values in
// registers between the max reduction and the encode.
#include "device_math.h"
#include "kernels.h"

namespace moe {
namespace {

// Each 16-lane group quantises one 1x128 tile (a lane takes 8 values); every
// thread handles QU tiles at a stride of the whole grid, with all QU loads
// issued before any arithmetic so that QU loads per lane are in flight.
constexpr int QU = 4;

// IDX32: the tile count fits 31 bits, so a tile's row and column block come
// from a 32-bit division (a 64-bit one is a long instruction sequence per tile)
template <bool IN_F32, bool IDX32>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const void* __restrict__ x,
                                                          int64_t rows, int cols,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ scale) {
    const int ntile = cols / 128;
    const int64_t total = rows * (int64_t)ntile * 16;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t g0 = (int64_t)blockIdx.x * 256 + threadIdx.x; g0 - threadIdx.x < total; g0 += stride * QU) {
        float v[QU][8];
        int64_t off[QU], sidx[QU];
        bool live[QU];
        float4 rf[QU][2];     // the raw 16-byte pieces, loaded for every u before any is used
        uint4 rb[QU];
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            // every lane of a 16-lane group has the same `live` (total % 16 == 0)
            const int64_t g = g0 + u * stride;
            live[u] = g < total;
            const int64_t tile = live[u] ? g >> 4 : 0;
            const int part = (int)(g & 15);
            int64_t row;
            int tc;
            if constexpr (IDX32) {
                const uint32_t t32 = (uint32_t)tile, r32 = t32 / (uint32_t)ntile;
                row = r32;
                tc = (int)(t32 - r32 * (uint32_t)ntile);
            } else {
                row = tile / ntile;
                tc = (int)(tile % ntile);
            }
            off[u] = row * cols + (int64_t)tc * 128 + part * 8;
            sidx[u] = part == 0 ? row * ntile + tc : -1;
            // unconditional (a dead u reads tile 0, a valid address), so the
            // QU loads are all in flight before the first value is used
            if constexpr (IN_F32) {
                const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off[u]);
                rf[u][0] = p[0];
                rf[u][1] = p[1];
            } else {
                rb[u] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            if (live[u]) {
                if constexpr (IN_F32) {
                    const float4 a = rf[u][0], b = rf[u][1];
                    v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
                    v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
                } else {
                    const uint4 a = rb[u];
                    v[u][0] = bf16_lo(a.x); v[u][1] = bf16_hi(a.x); v[u][2] = bf16_lo(a.y); v[u][3] = bf16_hi(a.y);
                    v[u][4] = bf16_lo(a.z); v[u][5] = bf16_hi(a.z); v[u][6] = bf16_lo(a.w); v[u][7] = bf16_hi(a.w);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[u][i] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < QU; ++u) {
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float a = __builtin_fabsf(v[u][i]);
                amax = a > amax ? a : amax;
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const float other = __shfl_xor(amax, o, 64);
                amax = other > amax ? other : amax;
            }
            float inv, sc;
            tile_scale(amax, inv, sc);
            if (live[u]) {
                const uint32_t lo = e4m3_encode4(v[u][0] * inv, v[u][1] * inv, v[u][2] * inv, v[u][3] * inv);
                const uint32_t hi = e4m3_encode4(v[u][4] * inv, v[u][5] * inv, v[u][6] * inv, v[u][7] * inv);
                *reinterpret_cast<uint2*>(q + off[u]) = make_uint2(lo, hi);
                if (sidx[u] >= 0) scale[sidx[u]] = sc;
            }
        }
    }
}

__global__ __launch_bounds__(256) void quant_128x128_kernel(const float* __restrict__ w,
                                                            int64_t rows, int cols,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ scale,
                                                            int row_mul, int row_add) {
    __shared__ float wmax[4];
    const int bc = blockIdx.x;
    const int64_t br = blockIdx.y;
    const int tid = threadIdx.x;
    const int cpart = tid & 15;           // 8 columns
    const int rbase = tid >> 4;           // rows rbase + 16*i
    float v[8][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = br * 128 + rbase + 16 * i;
        const float4* p = reinterpret_cast<const float4*>(w + r * cols + (int64_t)bc * 128 + cpart * 8);
        const float4 a = p[0], b = p[1];
        v[i][0] = a.x; v[i][1] = a.y; v[i][2] = a.z; v[i][3] = a.w;
        v[i][4] = b.x; v[i][5] = b.y; v[i][6] = b.z; v[i][7] = b.w;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float m = __builtin_fabsf(v[i][j]);
            amax = m > amax ? m : amax;
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float other = __shfl_xor(amax, o, 64);
        amax = other > amax ? other : amax;
    }
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) amax = wmax[i] > amax ? wmax[i] : amax;
    float inv, sc;
    tile_scale(amax, inv, sc);
    const int64_t dbr = br * row_mul + row_add;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = dbr * 128 + rbase + 16 * i;
        const uint32_t lo = e4m3_encode4(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv);
        const uint32_t hi = e4m3_encode4(v[i][4] * inv, v[i][5] * inv, v[i][6] * inv, v[i][7] * inv);
        *reinterpret_cast<uint2*>(q + r * cols + (int64_t)bc * 128 + cpart * 8) = make_uint2(lo, hi);
    }
    if (tid == 0) scale[dbr * (cols / 128) + bc] = sc;
}

}  // namespace

hipError_t launch_quant_1x128(const void* x, int in_is_f32, int64_t rows, int cols, uint8_t* q,
                              float* scale, hipStream_t st) {
    const int64_t threads = rows * (int64_t)(cols / 128) * 16;
    int64_t blocks = (threads + 256 * QU - 1) / (256 * QU);
    if (blocks > 65536) blocks = 65536;
    const bool idx32 = rows * (int64_t)(cols / 128) < ((int64_t)1 << 31);
    if (in_is_f32) {
        if (idx32)
            hipLaunchKernelGGL((quant_1x128_kernel<true, true>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                               rows, cols, q, scale);
        else
            hipLaunchKernelGGL((quant_1x128_kernel<true, false>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                               rows, cols, q, scale);
    } else {
        if (idx32)
            hipLaunchKernelGGL((quant_1x128_kernel<false, true>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                               rows, cols, q, scale);
        else
            hipLaunchKernelGGL((quant_1x128_kernel<false, false>), dim3((unsigned)blocks), dim3(256), 0, st, x,
                               rows, cols, q, scale);
    }
    return hipGetLastError();
}

hipError_t launch_quant_128x128(const float* w, int64_t rows, int cols, uint8_t* q, float* scale,
                                int row_mul, int row_add, hipStream_t st) {
    dim3 grid((unsigned)(cols / 128), (unsigned)(rows / 128));
    hipLaunchKernelGGL(quant_128x128_kernel, grid, dim3(256), 0, st, w, rows, cols, q, scale,
                       row_mul, row_add);
    return hipGetLastError();
}

}  // namespace moe
