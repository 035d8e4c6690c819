// Input-gradient (dgrad) backward of the layer.
//
// nlp-lineage summary, "The notation": h'_t = u_t + FFN_shared(u_t) +
// sum_k g_k FFN_(i_k)(u_t), with g_k = s_k / D, D = sum of the chosen s, and
// s = sigmoid(u . e) ("DeepSeek-V3 Technical Report" notes, MoE-routing
// paragraph; the bias only selects, so it carries no gradient).  For an
// upstream gradient dh = dL/dh' the chain rule gives, per token t and slot k:
//     a_k = <dh, Y_k>,  dL/ds_k = (a_k - sum_j g_j a_j) / D,
//     dlogit_k = dL/ds_k * s_k (1 - s_k),  dY_k = g_k dh,  dY_shared = dh;
// per expert row (z_g, z_u the GEMM1 outputs): dh_row = W2^T dY, then
//     dz_u = dh_row * SiLU(z_g),  dz_g = dh_row * z_u * sigma(z_g) (1 + z_g (1 - sigma(z_g))),
//     dx = W1^T dz_g + W3^T dz_u;
// and du_t = dh_t + sum of dx over the token's rows + sum_k dlogit_k e_(i_k),
// de_i = sum over the (t,k) that chose i of dlogit_k u_t.
//
// The two expert GEMMs run on the forward's grouped block-scaled FP8 GEMM with
// the packed weights transposed (an exact byte transposition of each 128 x 128
// block and its scale), so their operands are quantised like the forward's:
// dY and dz per 1 x 128 tile along the contraction, fused into the kernels
// that produce them.  The kernels here are bandwidth kernels.
#include "device_math.h"
#include "kernels.h"

namespace moe {
namespace {

// Quantise the 8 values a lane holds of one 1x128 tile whose 16 lanes are
// consecutive in the wave; writes 8 codes at q and, from lane 0 of the group,
// the scale at *sp.
__device__ __forceinline__ void quant_tile8(const float (&v)[8], int part, uint8_t* q, float* sp) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = __builtin_fabsf(v[i]);
        amax = a > amax ? a : amax;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const float other = __shfl_xor(amax, o, 64);
        amax = other > amax ? other : amax;
    }
    float inv, sc;
    tile_scale(amax, inv, sc);
    const uint32_t lo = e4m3_encode4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t hi = e4m3_encode4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    *reinterpret_cast<uint2*>(q) = make_uint2(lo, hi);
    if (part == 0) *sp = sc;
}

typedef float bwd_v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
// the same for data read once: non-temporal loads keep it from evicting lines
// that are still useful
__device__ __forceinline__ void load8_nt(const float* p, float (&v)[8]) {
    const bwd_v4f a = __builtin_nontemporal_load(reinterpret_cast<const bwd_v4f*>(p));
    const bwd_v4f b = __builtin_nontemporal_load(reinterpret_cast<const bwd_v4f*>(p) + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One block of 16 groups of 16 lanes per token (grid-strided); group gr takes
// the 1x128 tiles gr, gr+16, ... of the row.  Per tile a lane holds 8 columns
// of dh; it writes the quantised dY of the shared row and of every slot, and
// adds dh . Y_k into its partial a_k.  The a_k are reduced in a fixed order
// (wave butterflies, then the four waves in LDS); thread 0 finishes the gate
// chain.
template <int KMAX>
__global__ __launch_bounds__(256) void gate_backward_kernel(
    const float* __restrict__ dh, const float* __restrict__ y, int64_t shared_row0,
    const float* __restrict__ gate, const int32_t* __restrict__ slot_row, const float* __restrict__ s,
    const int32_t* __restrict__ idx, int64_t T, int K, int d, int E, uint8_t* __restrict__ dy_q,
    float* __restrict__ dy_s, float* __restrict__ dlogit, float* __restrict__ row_dlogit) {
    __shared__ float red[4][KMAX];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = tid >> 4, part = tid & 15;
    const int ntile = d / 128;
    for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
        float g[KMAX];
        int64_t r[KMAX];
        float acc[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            g[k] = k < K ? gate[t * K + k] : 0.0f;
            r[k] = k < K ? slot_row[t * K + k] : 0;
            acc[k] = 0.0f;
        }
        for (int tile = grp; tile < ntile; tile += 16) {
            const int col = tile * 128 + part * 8;
            float x[8];
            load8(dh + t * d + col, x);
            if (shared_row0 >= 0)
                quant_tile8(x, part, dy_q + (shared_row0 + t) * d + col, dy_s + (shared_row0 + t) * ntile + tile);
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (k >= K) break;
                float yv[8], v[8];
                load8_nt(y + r[k] * d + col, yv);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    acc[k] = __builtin_fmaf(x[i], yv[i], acc[k]);
                    v[i] = g[k] * x[i];
                }
                quant_tile8(v, part, dy_q + r[k] * d + col, dy_s + r[k] * ntile + tile);
            }
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            float a = acc[k];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) a = a + __shfl_xor(a, o, 64);
            if (lane == 0) red[wave][k] = a;
        }
        __syncthreads();
        if (tid == 0) {
            float a[KMAX], sk[KMAX];
            float D = 0.0f, ga = 0.0f;
            for (int k = 0; k < K; ++k) {
                a[k] = ((red[0][k] + red[1][k]) + red[2][k]) + red[3][k];
                sk[k] = s[t * E + idx[t * K + k]];
                D = D + sk[k];
                ga = __builtin_fmaf(g[k], a[k], ga);
            }
            for (int k = 0; k < K; ++k) {
                const float ds = (D == 0.0f) ? 0.0f : (a[k] - ga) / D;
                const float dl = ds * sk[k] * (1.0f - sk[k]);
                dlogit[t * K + k] = dl;
                row_dlogit[r[k]] = dl;
            }
        }
        __syncthreads();
    }
}

// SwiGLU backward on the GEMM1 output z [R, 2I] (gate and up columns
// interleaved per 256-column block: 128 gate, then the 128 up columns of the
// same h columns) and dh_row [R, I]; writes dz in z's layout, quantised per
// 1x128 tile (codes [R, 2I], scales [R, 2I/128]).  One 16-lane group per
// (row, h block); the sigmoid uses the hardware exp and reciprocal (within
// tolerance, not bit-exact).
__global__ __launch_bounds__(256) void swiglu_backward_kernel(const float* __restrict__ z,
                                                              const float* __restrict__ dh_row,
                                                              int64_t R, int I, uint8_t* __restrict__ dz_q,
                                                              float* __restrict__ dz_s) {
    const int nb = I / 128;
    const int64_t total = R * nb * 16;
    for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi - threadIdx.x < total;
         gi += (int64_t)gridDim.x * 256) {
        if (gi >= total) continue;          // whole 16-lane groups (total % 16 == 0)
        const int64_t tile = gi >> 4;
        const int part = (int)(gi & 15);
        const int64_t row = tile / nb;
        const int j = (int)(tile % nb);
        const int c0 = part * 8;
        const float* zr = z + row * 2 * I + (int64_t)j * 256;
        float zg[8], zu[8], dh[8], dzg[8], dzu[8];
        load8_nt(zr + c0, zg);
        load8_nt(zr + 128 + c0, zu);
        load8_nt(dh_row + row * I + (int64_t)j * 128 + c0, dh);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-zg[i]));
            dzu[i] = dh[i] * (zg[i] * sg);
            dzg[i] = dh[i] * zu[i] * sg * (1.0f + zg[i] * (1.0f - sg));
        }
        uint8_t* qr = dz_q + row * 2 * I + (int64_t)j * 256;
        float* sr = dz_s + row * (2 * I / 128) + 2 * j;
        quant_tile8(dzg, part, qr + c0, sr);
        quant_tile8(dzu, part, qr + 128 + c0, sr + 1);
    }
}

// du_t = dh_t + dx[shared_row0 + t] + sum_k dx[slot_row[t,k]] + sum_k dlogit_k e[idx[t,k]],
// in that order, FP32; blocks of 128 threads x 4 columns of one token.
template <int KMAX>
__global__ __launch_bounds__(128) void du_kernel(const float* __restrict__ dh, const float* __restrict__ dx,
                                                 int64_t shared_row0, const int32_t* __restrict__ slot_row,
                                                 const float* __restrict__ dlogit,
                                                 const int32_t* __restrict__ idx,
                                                 const uint16_t* __restrict__ e, int64_t T, int K, int d,
                                                 float* __restrict__ du) {
    const int cv = blockIdx.x * blockDim.x + threadIdx.x;       // float4 column index
    if (cv >= d / 4) return;
    for (int64_t t = blockIdx.y; t < T; t += gridDim.y) {
        float4 a = reinterpret_cast<const float4*>(dh + t * d)[cv];
        if (shared_row0 >= 0) {
            const bwd_v4f v = __builtin_nontemporal_load(reinterpret_cast<const bwd_v4f*>(dx + (shared_row0 + t) * d) + cv);
            a.x = a.x + v.x; a.y = a.y + v.y; a.z = a.z + v.z; a.w = a.w + v.w;
        }
        bwd_v4f xk[KMAX];
        uint2 ek[KMAX];
        float dl[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            xk[k] = __builtin_nontemporal_load(reinterpret_cast<const bwd_v4f*>(dx + (int64_t)slot_row[t * K + k] * d) + cv);
            ek[k] = reinterpret_cast<const uint2*>(e + (int64_t)idx[t * K + k] * d)[cv];
            dl[k] = dlogit[t * K + k];
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            a.x = a.x + xk[k].x; a.y = a.y + xk[k].y; a.z = a.z + xk[k].z; a.w = a.w + xk[k].w;
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k >= K) break;
            a.x = __builtin_fmaf(dl[k], bf16_lo(ek[k].x), a.x);
            a.y = __builtin_fmaf(dl[k], bf16_hi(ek[k].x), a.y);
            a.z = __builtin_fmaf(dl[k], bf16_lo(ek[k].y), a.z);
            a.w = __builtin_fmaf(dl[k], bf16_hi(ek[k].y), a.w);
        }
        const bwd_v4f o = {a.x, a.y, a.z, a.w};
        __builtin_nontemporal_store(o, reinterpret_cast<bwd_v4f*>(du + t * d) + cv);
    }
}

// de_i = sum over the routed rows r of expert i of row_dlogit[r] *
// u[row_token[r]]; one block per (expert, 512 columns): 128 column threads
// (4 columns each) x DE_PHASES row phases, phase p summing rows r0+p,
// r0+p+DE_PHASES, ... (four rows' loads in flight), then the phases added in
// order through LDS, so the result does not depend on timing.
constexpr int DE_PHASES = 8;

__global__ __launch_bounds__(128 * DE_PHASES) void de_kernel(const float* __restrict__ row_dlogit,
                                                             const int32_t* __restrict__ row_token,
                                                             const int32_t* __restrict__ group_offset,
                                                             const uint16_t* __restrict__ u, int d,
                                                             float* __restrict__ de) {
    __shared__ float4 part[DE_PHASES][128];
    const int i = blockIdx.y;
    const int col = threadIdx.x & 127, ph = threadIdx.x >> 7;
    const int cv = blockIdx.x * 128 + col;                       // 4-column index
    const bool live = cv < d / 4;
    const int r0 = group_offset[i], r1 = group_offset[i + 1];
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (live) {
        int r = r0 + ph;
        for (; r + 3 * DE_PHASES < r1; r += 4 * DE_PHASES) {
            uint2 uv[4];
            float w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                w[q] = row_dlogit[r + q * DE_PHASES];
                uv[q] = reinterpret_cast<const uint2*>(u + (int64_t)row_token[r + q * DE_PHASES] * d)[cv];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a.x = __builtin_fmaf(w[q], bf16_lo(uv[q].x), a.x);
                a.y = __builtin_fmaf(w[q], bf16_hi(uv[q].x), a.y);
                a.z = __builtin_fmaf(w[q], bf16_lo(uv[q].y), a.z);
                a.w = __builtin_fmaf(w[q], bf16_hi(uv[q].y), a.w);
            }
        }
        for (; r < r1; r += DE_PHASES) {
            const float w = row_dlogit[r];
            const uint2 uv = reinterpret_cast<const uint2*>(u + (int64_t)row_token[r] * d)[cv];
            a.x = __builtin_fmaf(w, bf16_lo(uv.x), a.x);
            a.y = __builtin_fmaf(w, bf16_hi(uv.x), a.y);
            a.z = __builtin_fmaf(w, bf16_lo(uv.y), a.z);
            a.w = __builtin_fmaf(w, bf16_hi(uv.y), a.w);
        }
    }
    part[ph][col] = a;
    __syncthreads();
    if (ph == 0 && live) {
        float4 t = part[0][col];
#pragma unroll
        for (int p = 1; p < DE_PHASES; ++p) {
            const float4 v = part[p][col];
            t.x = t.x + v.x; t.y = t.y + v.y; t.z = t.z + v.z; t.w = t.w + v.w;
        }
        reinterpret_cast<float4*>(de + (int64_t)i * d)[cv] = t;
    }
}

// out[g][c][r] = in[g][r][c] for bytes, one 128 x 128 block per workgroup
// through LDS, and the block's scale moved to its transposed place.
__global__ __launch_bounds__(256) void transpose_blocks_kernel(const uint8_t* __restrict__ in,
                                                               const float* __restrict__ in_s, int rows,
                                                               int cols, uint8_t* __restrict__ out,
                                                               float* __restrict__ out_s) {
    __shared__ uint8_t tile[128][132];
    const int cb = blockIdx.x, rb = blockIdx.y, g = blockIdx.z;
    const int tid = threadIdx.x;
    const uint8_t* src = in + (int64_t)g * rows * cols + (int64_t)rb * 128 * cols + (int64_t)cb * 128;
    {   // thread: row tid / 2, 64 bytes at (tid & 1) * 64
        const int r = tid >> 1, c0 = (tid & 1) * 64;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)r * cols + c0 + q * 16);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int b = 0; b < 16; ++b) tile[r][c0 + q * 16 + b] = (uint8_t)(w[b >> 2] >> ((b & 3) * 8));
        }
    }
    __syncthreads();
    uint8_t* dst = out + (int64_t)g * rows * cols + (int64_t)cb * 128 * rows + (int64_t)rb * 128;
    {   // thread: output row c = tid / 2 (input column), 64 input rows at (tid & 1) * 64
        const int c = tid >> 1, r0 = (tid & 1) * 64;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int b = 0; b < 16; ++b) w[b >> 2] |= (uint32_t)tile[r0 + q * 16 + b][c] << ((b & 3) * 8);
            *reinterpret_cast<uint4*>(dst + (int64_t)c * rows + r0 + q * 16) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    if (tid == 0) {
        const int nrb = rows / 128, ncb = cols / 128;
        out_s[(int64_t)g * nrb * ncb + (int64_t)cb * nrb + rb] = in_s[(int64_t)g * nrb * ncb + (int64_t)rb * ncb + cb];
    }
}

}  // namespace

hipError_t launch_gate_backward(const float* dh, const float* y, int64_t shared_row0, const float* gate,
                                const int32_t* slot_row, const float* s, const int32_t* idx, int64_t T,
                                int K, int d, int E, uint8_t* dy_q, float* dy_s, float* dlogit,
                                float* row_dlogit, hipStream_t st) {
    const unsigned grid = (unsigned)(T < 65536 ? T : 65536);
#define MOE_GATE_BWD(KM) hipLaunchKernelGGL((gate_backward_kernel<KM>), dim3(grid), dim3(256), 0, st, dh, y, \
                                            shared_row0, gate, slot_row, s, idx, T, K, d, E, dy_q, dy_s, dlogit, row_dlogit)
    if (K <= 4) MOE_GATE_BWD(4);
    else if (K <= 8) MOE_GATE_BWD(8);
    else MOE_GATE_BWD(16);
#undef MOE_GATE_BWD
    return hipGetLastError();
}

hipError_t launch_swiglu_backward(const float* z, const float* dh_row, int64_t R, int I, uint8_t* dz_q,
                                  float* dz_s, hipStream_t st) {
    const int64_t threads = R * (I / 128) * 16;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(swiglu_backward_kernel, dim3((unsigned)blocks), dim3(256), 0, st, z, dh_row, R, I,
                       dz_q, dz_s);
    return hipGetLastError();
}

hipError_t launch_du(const float* dh, const float* dx, int64_t shared_row0, const int32_t* slot_row,
                     const float* dlogit, const int32_t* idx, const uint16_t* e, int64_t T, int K, int d,
                     float* du, hipStream_t st) {
    const dim3 grid((unsigned)((d / 4 + 127) / 128), (unsigned)(T < 65535 ? T : 65535));
#define MOE_DU(KM) hipLaunchKernelGGL((du_kernel<KM>), grid, dim3(128), 0, st, dh, dx, shared_row0, slot_row, \
                                      dlogit, idx, e, T, K, d, du)
    if (K <= 4) MOE_DU(4);
    else if (K <= 8) MOE_DU(8);
    else MOE_DU(16);
#undef MOE_DU
    return hipGetLastError();
}

hipError_t launch_de(const float* row_dlogit, const int32_t* row_token, const int32_t* group_offset,
                     const uint16_t* u, int d, int E, float* de, hipStream_t st) {
    const dim3 grid((unsigned)((d / 4 + 127) / 128), (unsigned)E);
    hipLaunchKernelGGL(de_kernel, grid, dim3(128 * DE_PHASES), 0, st, row_dlogit, row_token, group_offset, u, d, de);
    return hipGetLastError();
}

hipError_t launch_transpose_blocks(const uint8_t* in, const float* in_s, int G, int rows, int cols,
                                   uint8_t* out, float* out_s, hipStream_t st) {
    hipLaunchKernelGGL(transpose_blocks_kernel, dim3((unsigned)(cols / 128), (unsigned)(rows / 128), (unsigned)G),
                       dim3(256), 0, st, in, in_s, rows, cols, out, out_s);
    return hipGetLastError();
}

}  // namespace moe
