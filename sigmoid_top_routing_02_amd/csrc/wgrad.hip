// Operands of the expert weight gradients.
//
// Per expert g, over its GEMM rows r (the forward's dispatch order):
//     dW2_g = sum_r dY_r^T h_r        ([d, I]),    h = SiLU(z_gate) * z_up
//     dW13_g = sum_r dz_r^T x_r       ([2I, d], W13's interleaved row order),
// with dY_r = w_r dh_(token r) (w_r the slot's gate, 1 on the shared rows),
// dz the SwiGLU backward of dh_row, and x_r = u_(token r).  These contract
// over the rows, so each runs on the grouped block-scaled GEMM as one group
// with M = d (or 2I), N = I (or d) and K = the expert's rows padded to a
// multiple of 128, on transposed operands built here: dY^T and dz^T quantised
// per 1 x 128 tile along the rows (the contraction), h^T and x^T per 128 x 128
// block (this library's reading; the pages give no backward tiling).  The
// padding rows are zero.
//
// Layout of each operand, group after group (kb_start[g] = the 128-row blocks
// before group g, nkb_g = blocks of group g, Kp_g = 128 nkb_g):
//     codes  [C, Kp_g] at C * 128 * kb_start[g]
//     1x128 scales  [C, nkb_g] at C * kb_start[g];  128x128 scales
//     [C/128, nkb_g] at CS * kb_start[g], CS = C/128 rounded up to a multiple
//     of 4 (every group's scales start 16-byte aligned).
// One workgroup per (128 columns, 128-row block): each row's token and dY
// weight are found once, the block's values are computed four columns per
// lane into LDS, then quantised along the other axis and written 64 bytes
// per lane.
#include "device_math.h"
#include "kernels.h"

namespace moe {
namespace {

enum { SRC_DY = 0, SRC_H = 1, SRC_DZ = 2, SRC_X = 3 };

struct WgradSrc {
    const float* dh;          // [T, d]
    const float* gate;        // [T, K]
    const int32_t* slot_row;  // [T, K]
    const int32_t* row_token; // [R]
    const float* z;           // [R, 2I]
    const float* dh_row;      // [R, I]
    const uint16_t* u;        // [T, d] bf16
    int64_t shared_row0;
    int K, d, I;
};

__device__ __forceinline__ float sigm(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// the weight of row r's dY: its slot's gate (routed rows), 1 (shared rows).
// The token's K slot rows (K <= 16) are loaded together, then the gate of the
// first slot that holds r.
__device__ __forceinline__ float row_weight(const WgradSrc& s, int64_t r, int64_t t) {
    if (s.shared_row0 >= 0 && r >= s.shared_row0) return 1.0f;
    int32_t sr[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) sr[k] = k < s.K ? s.slot_row[t * s.K + k] : -1;
    int hit = -1;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (hit < 0 && sr[k] == r) hit = k;
    return hit >= 0 ? s.gate[t * s.K + hit] : 0.0f;
}

template <int SRC, bool BLOCK_SCALE>
__global__ __launch_bounds__(256) void wgrad_operand_kernel(WgradSrc s, const int32_t* __restrict__ go,
                                                            const int32_t* __restrict__ kb_start, int G, int C,
                                                            uint8_t* __restrict__ out_q, float* __restrict__ out_s) {
    __shared__ float tile[128][129];
    __shared__ float wmax[4];
    const int tid = threadIdx.x;
    // Sources gathered by token (dY from dh, u^T from u) read each token's row
    // once per GEMM row of the token (K + 1 times): their grids run the row
    // blocks fastest, so those reads of one 128-column block fall close
    // together in time and hit in cache (the other order takes them from HBM).
    constexpr bool GATHER = (SRC == SRC_DY || SRC == SRC_X);
    const int c0 = (GATHER ? blockIdx.y : blockIdx.x) * 128;
    const int kbi = GATHER ? blockIdx.x : blockIdx.y;
    // the grid covers an upper bound of the row blocks (the host does not read
    // the group sizes back); blocks past the last one have nothing to do
    if (kbi >= kb_start[G]) return;
    int lo = 0, hi = G - 1;                                    // the group of this row block
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (kb_start[mid] <= kbi) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int kb0 = kb_start[g], nkb = kb_start[g + 1] - kb0, kbl = kbi - kb0;
    const int64_t rb = (int64_t)go[g] + (int64_t)kbl * 128, rend = go[g + 1];
    // per row of the block: its token and (for dY) its weight, once
    __shared__ int64_t s_tok[128];
    __shared__ float s_w[128];
    if (tid < 128) {
        const int64_t r = rb + tid;
        int64_t t = 0;
        float w = 0.0f;
        if (r < rend) {
            if constexpr (SRC == SRC_DY || SRC == SRC_X) t = s.row_token[r];
            if constexpr (SRC == SRC_DY) w = row_weight(s, r, t);
        }
        s_tok[tid] = t;
        s_w[tid] = w;
    }
    __syncthreads();
    {   // values: thread = 4 columns c0 + 4 (tid & 31), rows (tid >> 5) + 8 j.  The
        // loads of NB rows go out before any of them is used, so NB loads per
        // lane are in flight instead of one (the rows' arithmetic is unchanged)
        const int cq = (tid & 31) * 4, c = c0 + cq;
        const int i0 = tid >> 5;
        // (every load reads a valid row -- rows past the group read the token
        // of s_tok = 0, or the group's last row -- and such rows' values are
        // zeroed below, so no load needs a condition)
        constexpr int NB = (SRC == SRC_DY || SRC == SRC_X) ? 16 : 8;
#pragma unroll
        for (int b = 0; b < 16; b += NB) {
            float4 la[NB], lb[NB], lc[NB];
            uint2 lx[NB];
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) {
                const int i = i0 + 8 * (b + jj);
                const int64_t rl = min(rb + i, rend - 1);
                if constexpr (SRC == SRC_DY) {
                    la[jj] = *reinterpret_cast<const float4*>(s.dh + s_tok[i] * s.d + c);
                } else if constexpr (SRC == SRC_X) {
                    lx[jj] = *reinterpret_cast<const uint2*>(s.u + s_tok[i] * s.d + c);
                } else if constexpr (SRC == SRC_H) {
                    const float* zr = s.z + rl * 2 * s.I + (c >> 7) * 256 + (c & 127);
                    la[jj] = *reinterpret_cast<const float4*>(zr);
                    lb[jj] = *reinterpret_cast<const float4*>(zr + 128);
                } else {
                    const int j = c >> 8, w = c & 255, ic = j * 128 + (w & 127);
                    const float* zr = s.z + rl * 2 * s.I + j * 256 + (w & 127);
                    la[jj] = *reinterpret_cast<const float4*>(zr);
                    lb[jj] = *reinterpret_cast<const float4*>(zr + 128);
                    lc[jj] = *reinterpret_cast<const float4*>(s.dh_row + rl * s.I + ic);
                }
            }
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) {
                const int i = i0 + 8 * (b + jj);
                const int64_t r = rb + i;
                float v[4] = {0.f, 0.f, 0.f, 0.f};
                if (r < rend) {
                    if constexpr (SRC == SRC_DY) {
                        const float4 x = la[jj];
                        const float w = s_w[i];
                        v[0] = w * x.x; v[1] = w * x.y; v[2] = w * x.z; v[3] = w * x.w;
                    } else if constexpr (SRC == SRC_X) {
                        const uint2 x = lx[jj];
                        v[0] = bf16_lo(x.x); v[1] = bf16_hi(x.x); v[2] = bf16_lo(x.y); v[3] = bf16_hi(x.y);
                    } else if constexpr (SRC == SRC_H) {
                        const float4 zg = la[jj], zu = lb[jj];
                        const float g4[4] = {zg.x, zg.y, zg.z, zg.w}, u4[4] = {zu.x, zu.y, zu.z, zu.w};
#pragma unroll
                        for (int q = 0; q < 4; ++q) v[q] = g4[q] * sigm(g4[q]) * u4[q];
                    } else {
                        const int w = c & 255;
                        const float4 zg = la[jj], zu = lb[jj], dh = lc[jj];
                        const float g4[4] = {zg.x, zg.y, zg.z, zg.w}, u4[4] = {zu.x, zu.y, zu.z, zu.w};
                        const float d4[4] = {dh.x, dh.y, dh.z, dh.w};
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float sg = sigm(g4[q]);
                            v[q] = (w < 128) ? d4[q] * u4[q] * sg * (1.0f + g4[q] * (1.0f - sg)) : d4[q] * (g4[q] * sg);
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) tile[i][cq + q] = v[q];
            }
        }
    }
    __syncthreads();
    // output row c0 + (tid >> 1), 64 consecutive k at (tid & 1) * 64
    const int oc = tid >> 1, half = tid & 1;
    float amax = 0.0f;
    for (int q = 0; q < 64; ++q) {
        const float a = __builtin_fabsf(tile[half * 64 + q][oc]);
        amax = a > amax ? a : amax;
    }
    if constexpr (BLOCK_SCALE) {
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float other = __shfl_xor(amax, o, 64);
            amax = other > amax ? other : amax;
        }
        if ((tid & 63) == 0) wmax[tid >> 6] = amax;
        __syncthreads();
        amax = wmax[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) amax = wmax[w] > amax ? wmax[w] : amax;
    } else {
        const float other = __shfl_xor(amax, 1, 64);
        amax = other > amax ? other : amax;
    }
    float inv, sc;
    tile_scale(amax, inv, sc);
    const int64_t Kp = (int64_t)nkb * 128;
    uint8_t* dst = out_q + (int64_t)C * 128 * kb0 + (int64_t)(c0 + oc) * Kp + (int64_t)kbl * 128 + half * 64;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t w4[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int k = half * 64 + q * 16 + p * 4;
            w4[p] = e4m3_encode4(tile[k][oc] * inv, tile[k + 1][oc] * inv, tile[k + 2][oc] * inv,
                                 tile[k + 3][oc] * inv);
        }
        *reinterpret_cast<uint4*>(dst + q * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    if constexpr (BLOCK_SCALE) {
        const int cs = ((C / 128) + 3) & ~3;
        if (tid == 0) out_s[(int64_t)cs * kb0 + (int64_t)(c0 / 128) * nkb + kbl] = sc;
    } else {
        if (half == 0) out_s[(int64_t)C * kb0 + (int64_t)(c0 + oc) * nkb + kbl] = sc;
    }
}

// kb_start[g] = sum_{g' < g} ceil(rows_g' / 128) for g = 0..G, one block:
// per chunk of 256 groups a Hillis-Steele scan in LDS plus the running carry.
__global__ __launch_bounds__(256) void wgrad_block_starts_kernel(const int32_t* __restrict__ go, int G,
                                                                 int32_t* __restrict__ kb_start) {
    __shared__ int32_t buf[256];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < G; base += 256) {
        const int g = base + threadIdx.x;
        const int32_t v = (g < G) ? (go[g + 1] - go[g] + 127) / 128 : 0;
        buf[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int32_t x = (threadIdx.x >= (unsigned)off) ? buf[threadIdx.x - off] : 0;
            __syncthreads();
            buf[threadIdx.x] += x;
            __syncthreads();
        }
        if (g < G) kb_start[g] = carry + buf[threadIdx.x] - v;
        __syncthreads();
        if (threadIdx.x == 255) carry += buf[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) kb_start[G] = carry;
}

}  // namespace

hipError_t launch_wgrad_block_starts(const int32_t* go, int G, int32_t* kb_start, hipStream_t st) {
    hipLaunchKernelGGL(wgrad_block_starts_kernel, dim3(1), dim3(256), 0, st, go, G, kb_start);
    return hipGetLastError();
}

size_t wgrad_ws_bytes(int G, int d, int I) {
    const size_t a = gemm_kgrouped_ws_bytes(G, d, I), b = gemm_kgrouped_ws_bytes(G, 2 * I, d);
    return a > b ? a : b;
}

// dW2 = GEMM(dY^T, h^T) and dW13 = GEMM(dz^T, u^T), each one K-grouped launch
// over all groups (group g's inner dimension is its padded row count); the two
// run one after the other on st and share the workspace.
hipError_t launch_wgrad_gemms(const int32_t* kb_start, int G, int d, int I, const uint8_t* dyT_q,
                              const float* dyT_s, const uint8_t* hT_q, const float* hT_s, const uint8_t* dzT_q,
                              const float* dzT_s, const uint8_t* xT_q, const float* xT_s, float* dw13, float* dw2,
                              void* ws, hipStream_t st) {
    const int cs_h = ((I / 128) + 3) & ~3, cs_x = ((d / 128) + 3) & ~3;
    hipError_t e = launch_grouped_gemm_kgrouped(dyT_q, dyT_s, kb_start, G, d, hT_q, hT_s, cs_h, I, dw2, ws, st);
    if (e != hipSuccess) return e;
    return launch_grouped_gemm_kgrouped(dzT_q, dzT_s, kb_start, G, 2 * I, xT_q, xT_s, cs_x, d, dw13, ws, st);
}

hipError_t launch_wgrad_operands(const float* dh, const float* gate, const int32_t* slot_row,
                                 const int32_t* row_token, const float* z, const float* dh_row,
                                 const uint16_t* u, int64_t shared_row0, int K, int d, int I,
                                 const int32_t* go, const int32_t* kb_start, int G, int n_kb,
                                 uint8_t* dyT_q, float* dyT_s, uint8_t* hT_q, float* hT_s, uint8_t* dzT_q,
                                 float* dzT_s, uint8_t* xT_q, float* xT_s, hipStream_t st) {
    WgradSrc s{dh, gate, slot_row, row_token, z, dh_row, u, shared_row0, K, d, I};
    hipLaunchKernelGGL((wgrad_operand_kernel<SRC_DY, false>), dim3((unsigned)n_kb, (unsigned)(d / 128)), dim3(256),
                       0, st, s, go, kb_start, G, d, dyT_q, dyT_s);
    hipLaunchKernelGGL((wgrad_operand_kernel<SRC_H, true>), dim3((unsigned)(I / 128), (unsigned)n_kb), dim3(256),
                       0, st, s, go, kb_start, G, I, hT_q, hT_s);
    hipLaunchKernelGGL((wgrad_operand_kernel<SRC_DZ, false>), dim3((unsigned)(2 * I / 128), (unsigned)n_kb),
                       dim3(256), 0, st, s, go, kb_start, G, 2 * I, dzT_q, dzT_s);
    hipLaunchKernelGGL((wgrad_operand_kernel<SRC_X, true>), dim3((unsigned)n_kb, (unsigned)(d / 128)), dim3(256),
                       0, st, s, go, kb_start, G, d, xT_q, xT_s);
    return hipGetLastError();
}

}  // namespace moe
