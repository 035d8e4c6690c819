// Grouped block-scaled FP8 GEMM for the expert FFNs (and, with one group, the
// dense block-scaled GEMM).
//
// "DeepSeek-V3 Technical Report" notes (learn.ifs.name), FP8-accumulation
// paragraph: the tensor-core accumulation of FP8 products is promoted to FP32
// every 128 elements of the inner dimension, and the per-group scales are
// applied there.  On gfx950 one v_mfma_f32_16x16x128_f8f6f4 covers exactly one
// 128-wide slice, so every slice is one MFMA into a fresh FP32 accumulator and
// the scaled sum over slices is an FP32 FMA chain on the VALU:
//     acc = fma(P_j, a_scale[m,j] * b_scale[n/128,j], acc)
// (FP8 tiling paragraph: A is scaled per 1x128 tile, B per 128x128 block.)
//
// Tiling (CDNA4): 256 threads = 4 wave64s in a 2x2 grid, block tile
// 128 (M) x 256 (N), wave tile 64 x 128 = 4 x 8 MFMA tiles of 16x16, one
// 128-byte K slice per stage.  A rows are gathered through a_row_index
// (the dispatch permutation), so the activations are never materialised in
// expert order.  Both operands go global -> LDS with global_load_lds_dwordx4
// (no VGPR staging) into a 2-stage ring; LDS rows are 128 bytes with the
// 16-byte chunk index XOR-swizzled by (row & 7) so the MFMA fragment reads are
// bank-conflict free.  The A scales of the slice ride along as one more
// LDS DMA (4 bytes per row); B scales are wave-uniform scalar loads.
//
// Grouping: a device-side tile map (exclusive scan of ceil(rows_g / 128))
// turns blockIdx.y into (group, m-tile); the grid is sized from the host-known
// total row count plus one partial tile per group, and surplus blocks exit.
//
// Epilogues: FP32 store; SwiGLU (B rows interleaved gate/up per 128-row
// block, so one N tile holds the gate and up columns of the same 128 h
// columns); SwiGLU + 1x128 E4M3 re-quantisation of h, whose row maximum over
// the 128 h columns of the tile is reduced across the two N-waves in LDS.
#include "device_math.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int BK = 128;                       // one scale slice
constexpr int NT = 256;
constexpr int A_BYTES = BM * BK;              // 16 KiB
constexpr int B_BYTES = BN * BK;              // 32 KiB
constexpr int SA_BYTES = BM * 4;              // 512 B
constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
constexpr int NSTAGE = 2;
constexpr int LDS_BYTES = STAGE * NSTAGE;     // 99,328 B

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct GemmArgs {
    const uint8_t* a_q;
    const float* a_s;
    const int32_t* a_rows;
    const int32_t* group_offset;
    const int32_t* tile_start;
    int G;
    const uint8_t* b_q;
    const float* b_s;
    int N;
    int K;
    float* out;
    uint8_t* out_q;
    float* out_s;
};

__device__ __forceinline__ void lds_dma16(const void* g, char* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* g, char* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 4, 0, 0);
}

// 32 K-bytes of row r for lanes of k-block kb (= lane / 16) from a swizzled tile.
__device__ __forceinline__ v8i frag(const char* tile, int r, int kb) {
    const int sw = r & 7;
    const uint4 x = *reinterpret_cast<const uint4*>(tile + r * 128 + (((2 * kb) ^ sw) << 4));
    const uint4 y = *reinterpret_cast<const uint4*>(tile + r * 128 + (((2 * kb + 1) ^ sw) << 4));
    v8i f;
    f[0] = (int)x.x; f[1] = (int)x.y; f[2] = (int)x.z; f[3] = (int)x.w;
    f[4] = (int)y.x; f[5] = (int)y.y; f[6] = (int)y.z; f[7] = (int)y.w;
    return f;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Column offset (inside the 256-wide N tile) of MFMA column-tile ni of wave wn.
template <int EPI>
__device__ __forceinline__ int ncol(int wn, int ni) {
    if constexpr (EPI == EPI_STORE_F32) {
        return wn * 128 + ni * 16;
    } else {
        return (ni < 4) ? (wn * 64 + ni * 16) : (128 + wn * 64 + (ni - 4) * 16);
    }
}

template <int EPI>
__global__ __launch_bounds__(NT) void grouped_gemm_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    // ---- which tile is this block?
    const int mt_lin = blockIdx.y;
    const int total_tiles = p.tile_start[p.G];
    if (mt_lin >= total_tiles) return;
    int lo = 0, hi = p.G - 1;                 // largest g with tile_start[g] <= mt_lin
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.tile_start[mid] <= mt_lin) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int m0 = p.group_offset[g] + (mt_lin - p.tile_start[g]) * BM;
    const int rows = min(BM, p.group_offset[g + 1] - m0);
    const int n0 = blockIdx.x * BN;
    const int K = p.K;
    const int ns = K / BK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- per-lane global sources for the LDS DMA (loop-invariant)
    const uint8_t* a_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (wave * 4 + i) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        const int m = m0 + min(r, rows - 1);
        const int64_t am = p.a_rows ? (int64_t)p.a_rows[m] : (int64_t)m;
        a_src[i] = p.a_q + am * K + c * 16;
    }
    const uint8_t* b_src[8];
    const uint8_t* bgrp = p.b_q + (int64_t)g * p.N * K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = (wave * 8 + i) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        const int n = min(n0 + r, p.N - 1);
        b_src[i] = bgrp + (int64_t)n * K + c * 16;
    }
    const float* sa_src[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = i * 64 + lane;
        const int m = m0 + min(r, rows - 1);
        const int64_t am = p.a_rows ? (int64_t)p.a_rows[m] : (int64_t)m;
        sa_src[i] = p.a_s + am * ns;
    }

    auto issue = [&](int slice, int stage) {
        char* base = smem + stage * STAGE;
        const int koff = slice * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_dma16(a_src[i] + koff, base + (wave * 4 + i) * 1024);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            lds_dma16(b_src[i] + koff, base + A_BYTES + (wave * 8 + i) * 1024);
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i) lds_dma4(sa_src[i] + slice, base + A_BYTES + B_BYTES + i * 256);
        }
    };

    // ---- B scales: wave-uniform rows of b_scale for this wave's columns
    const int nblk_per_g = p.N / 128;
    const float* bs_g = p.b_s + (int64_t)g * nblk_per_g * ns;
    int bblk0, bblk1;
    if constexpr (EPI == EPI_STORE_F32) {
        bblk0 = min((n0 + wn * 128) / 128, nblk_per_g - 1);
        bblk1 = bblk0;
    } else {
        bblk0 = n0 / 128;
        bblk1 = n0 / 128 + 1;
    }

    v4f acc[4][8];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

    const int kb = lane >> 4;
    const int lr = lane & 15;

    issue(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int s = 0; s < ns; ++s) {
        const int stage = s & 1;
        if (s + 1 < ns) issue(s + 1, stage ^ 1);
        const char* At = smem + stage * STAGE;
        const char* Bt = At + A_BYTES;
        const float* SAt = reinterpret_cast<const float*>(At + A_BYTES + B_BYTES);

        const float sb0 = bs_g[(int64_t)bblk0 * ns + s];
        const float sb1 = bs_g[(int64_t)bblk1 * ns + s];

        v8i af[4];
        float c0[4][4], c1[4][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int r = wm * 64 + mi * 16;
            af[mi] = frag(At, r + lr, kb);
            const float4 sa = *reinterpret_cast<const float4*>(SAt + r + kb * 4);
            const float sv[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c0[mi][j] = sv[j] * sb0;
                c1[mi][j] = sv[j] * sb1;
            }
        }
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) {
            const v8i bf = frag(Bt, ncol<EPI>(wn, ni) + lr, kb);
            const bool second = (EPI != EPI_STORE_F32) && ni >= 4;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[mi], bf, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[mi][ni][j] = __builtin_fmaf(part[j], second ? c1[mi][j] : c0[mi][j],
                                                    acc[mi][ni][j]);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogues.  Lane holds C[row = base + 4*kb + j][col = base + lr].
    if constexpr (EPI == EPI_STORE_F32) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = wm * 64 + mi * 16 + kb * 4 + j;
                if (r >= rows) continue;
                float* orow = p.out + (int64_t)(m0 + r) * p.N;
#pragma unroll
                for (int ni = 0; ni < 8; ++ni) {
                    const int n = n0 + ncol<EPI>(wn, ni) + lr;
                    if (n < p.N) orow[n] = acc[mi][ni][j];
                }
            }
    } else {
        const int I = p.N / 2;
        const int h0 = n0 / 2;             // first h column of this tile
        float h[4][4][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int j = 0; j < 4; ++j) h[mi][ni][j] = silu(acc[mi][ni][j]) * acc[mi][ni + 4][j];
        if constexpr (EPI == EPI_SWIGLU_F32) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = wm * 64 + mi * 16 + kb * 4 + j;
                    if (r >= rows) continue;
                    float* orow = p.out + (int64_t)(m0 + r) * I + h0 + wn * 64;
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) orow[ni * 16 + lr] = h[mi][ni][j];
                }
        } else {
            // row maximum over this wave's 64 h columns, then across wn in LDS
            float* amax_s = reinterpret_cast<float*>(smem);           // [2][128]
            char* qtile = smem + 1024;                                  // [128][128] codes
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float m = 0.0f;
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const float a = __builtin_fabsf(h[mi][ni][j]);
                        m = a > m ? a : m;
                    }
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) {
                        const float other = __shfl_xor(m, o, 64);
                        m = other > m ? other : m;
                    }
                    if (lr == 0) amax_s[wn * 128 + wm * 64 + mi * 16 + kb * 4 + j] = m;
                }
            __syncthreads();
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = wm * 64 + mi * 16 + kb * 4 + j;
                    const float a0 = amax_s[r], a1 = amax_s[128 + r];
                    const float amax = a1 > a0 ? a1 : a0;
                    float inv, sc;
                    tile_scale(amax, inv, sc);
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        qtile[r * 128 + wn * 64 + ni * 16 + lr] =
                            (char)e4m3_encode(h[mi][ni][j] * inv);
                    if (wn == 0 && lr == 0 && r < rows)
                        p.out_s[(int64_t)(m0 + r) * (I / 128) + h0 / 128] = sc;
                }
            __syncthreads();
            // 128 rows x 128 bytes, 16-byte stores
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + i * NT;
                const int r = c >> 3, part = c & 7;
                if (r < rows)
                    *reinterpret_cast<uint4*>(p.out_q + (int64_t)(m0 + r) * I + h0 + part * 16) =
                        *reinterpret_cast<const uint4*>(qtile + r * 128 + part * 16);
            }
            if (p.out) {
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = wm * 64 + mi * 16 + kb * 4 + j;
                        if (r >= rows) continue;
                        float* orow = p.out + (int64_t)(m0 + r) * I + h0 + wn * 64;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) orow[ni * 16 + lr] = h[mi][ni][j];
                    }
            }
        }
    }
}

// tile_start[g] = sum_{g' < g} ceil(rows_g' / BM), for g = 0..G.
__global__ __launch_bounds__(256) void gemm_tile_map_kernel(const int32_t* __restrict__ go,
                                                            int G, int32_t* __restrict__ ts) {
    __shared__ int32_t buf[256];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < G; base += 256) {
        const int g = base + threadIdx.x;
        const int32_t v = (g < G) ? (go[g + 1] - go[g] + BM - 1) / BM : 0;
        buf[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int32_t x = (threadIdx.x >= (unsigned)off) ? buf[threadIdx.x - off] : 0;
            __syncthreads();
            buf[threadIdx.x] += x;
            __syncthreads();
        }
        if (g < G) ts[g] = carry + buf[threadIdx.x] - v;
        __syncthreads();
        if (threadIdx.x == 255) carry += buf[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) ts[G] = carry;
}

}  // namespace

size_t gemm_ws_bytes(int G) { return (size_t)(G + 1) * sizeof(int32_t); }

hipError_t launch_grouped_gemm(const uint8_t* a_q, const float* a_s, const int32_t* a_rows,
                               const int32_t* group_offset, int G, int64_t M_total,
                               const uint8_t* b_q, const float* b_s, int N, int K, int epi,
                               float* out, uint8_t* out_q, float* out_s, void* ws,
                               hipStream_t st) {
    int32_t* ts = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL(gemm_tile_map_kernel, dim3(1), dim3(256), 0, st, group_offset, G, ts);
    GemmArgs p{a_q, a_s, a_rows, group_offset, ts, G, b_q, b_s, N, K, out, out_q, out_s};
    const int64_t mt_bound = (M_total + BM - 1) / BM + G;
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)mt_bound);
    switch (epi) {
        case EPI_STORE_F32:
            hipLaunchKernelGGL(grouped_gemm_kernel<EPI_STORE_F32>, grid, dim3(NT), 0, st, p);
            break;
        case EPI_SWIGLU_F32:
            hipLaunchKernelGGL(grouped_gemm_kernel<EPI_SWIGLU_F32>, grid, dim3(NT), 0, st, p);
            break;
        default:
            hipLaunchKernelGGL(grouped_gemm_kernel<EPI_SWIGLU_QUANT>, grid, dim3(NT), 0, st, p);
            break;
    }
    return hipGetLastError();
}

}  // namespace moe
