// Router: sigmoid affinity of every token to every expert centroid, then the
// biased top-K choice with gates normalised over the chosen experts.
//
// "DeepSeek-V3 Technical Report" notes (learn.ifs.name), MoE-routing
// paragraph: each token picks the top 8 of 256 routed experts by sigmoid
// affinity to the expert's centroid, gates normalised over the chosen ones;
// bias paragraph: a per-expert bias enters the top-K choice only.
// nlp-lineage summary, "The notation": chosen iff s + b is among the top K,
// b never changes the gate g.
//
// Affinity kernel: a register-tiled FP32 VALU GEMM.  Each output's dot product
// is one FMA chain in increasing k (bf16 products are exact in FP32, so the
// chain fixes the result bit for bit); MFMA is not used because its internal
// summation order is unspecified and routing must be reproducible exactly.
// Tiles of KC k-values of u and of the centroids are widened to FP32 into LDS
// (double-buffered through registers); every thread owns TM tokens x EN
// experts.
//
// Top-K kernel: one wavefront per token, 64-bit composite keys
// (orderable(s+b) << 32 | ~expert) reduced with cross-lane shuffles, K rounds.
#include "device_math.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int KC = 32;          // k-values per LDS stage
constexpr int NTHREADS = 256;

template <int BT, int BE, int TM, int EN>
struct RouterTile {
    static constexpr int NTX = BE / EN;   // thread columns (expert groups)
    static constexpr int NTY = BT / TM;   // thread rows (token groups)
    static_assert(NTX * NTY == NTHREADS, "tile must use 256 threads");
    static constexpr int E_CHUNKS = BE * (KC / 8);   // 16-byte chunks per stage
    static constexpr int U_CHUNKS = BT * (KC / 8);
    static constexpr int E_PER_T = (E_CHUNKS + NTHREADS - 1) / NTHREADS;
    static constexpr int U_PER_T = (U_CHUNKS + NTHREADS - 1) / NTHREADS;
    // expert column of (thread column tx, j): groups of 4 consecutive experts
    // per thread so the LDS reads are 16-byte and conflict free.
    __device__ static int ecol(int tx, int j) {
        if constexpr (EN >= 4) {
            return (j >> 2) * (BE / (EN / 4)) + tx * 4 + (j & 3);
        } else {
            return tx * EN + j;
        }
    }
};

template <int BT, int BE, int TM, int EN>
__global__ __launch_bounds__(NTHREADS) void router_scores_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ e, int64_t T, int d, int E,
    float* __restrict__ s) {
    using Tl = RouterTile<BT, BE, TM, EN>;
    __shared__ __attribute__((aligned(16))) float us[2][KC][BT];
    __shared__ __attribute__((aligned(16))) float es[2][KC][BE];

    const int tid = threadIdx.x;
    const int tx = tid % Tl::NTX;
    const int ty = tid / Tl::NTX;
    const int64_t t0 = (int64_t)blockIdx.x * BT;
    const int e0 = blockIdx.y * BE;

    // global -> register staging of one KC-slice
    uint4 ereg[Tl::E_PER_T];
    uint4 ureg[Tl::U_PER_T];

    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < Tl::E_PER_T; ++i) {
            const int c = tid + i * NTHREADS;
            ereg[i] = make_uint4(0, 0, 0, 0);
            if (c < Tl::E_CHUNKS) {
                const int row = c % BE, part = c / BE;
                const int ex = e0 + row;
                if (ex < E)
                    ereg[i] = *reinterpret_cast<const uint4*>(e + (int64_t)ex * d + k0 + part * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < Tl::U_PER_T; ++i) {
            const int c = tid + i * NTHREADS;
            ureg[i] = make_uint4(0, 0, 0, 0);
            if (c < Tl::U_CHUNKS) {
                const int row = c % BT, part = c / BT;
                const int64_t tk = t0 + row;
                if (tk < T)
                    ureg[i] = *reinterpret_cast<const uint4*>(u + tk * d + k0 + part * 8);
            }
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < Tl::E_PER_T; ++i) {
            const int c = tid + i * NTHREADS;
            if (c < Tl::E_CHUNKS) {
                const int row = c % BE, part = c / BE;
                const uint32_t w[4] = {ereg[i].x, ereg[i].y, ereg[i].z, ereg[i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    es[buf][part * 8 + 2 * q][row] = bf16_lo(w[q]);
                    es[buf][part * 8 + 2 * q + 1][row] = bf16_hi(w[q]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < Tl::U_PER_T; ++i) {
            const int c = tid + i * NTHREADS;
            if (c < Tl::U_CHUNKS) {
                const int row = c % BT, part = c / BT;
                const uint32_t w[4] = {ureg[i].x, ureg[i].y, ureg[i].z, ureg[i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    us[buf][part * 8 + 2 * q][row] = bf16_lo(w[q]);
                    us[buf][part * 8 + 2 * q + 1][row] = bf16_hi(w[q]);
                }
            }
        }
    };

    float acc[TM][EN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < EN; ++j) acc[i][j] = 0.0f;

    const int nstage = d / KC;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int st = 0; st < nstage; ++st) {
        const int buf = st & 1;
        if (st + 1 < nstage) load_stage((st + 1) * KC);
#pragma unroll 8
        for (int k = 0; k < KC; ++k) {
            float a[TM], b[EN];
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = us[buf][k][ty * TM + i];
#pragma unroll
            for (int j = 0; j < EN; ++j) b[j] = es[buf][k][Tl::ecol(tx, j)];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < EN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        if (st + 1 < nstage) store_stage(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t tk = t0 + ty * TM + i;
        if (tk >= T) continue;
#pragma unroll
        for (int j = 0; j < EN; ++j) {
            const int ex = e0 + Tl::ecol(tx, j);
            if (ex < E) s[tk * E + ex] = sigmoid_fixed(acc[i][j]);
        }
    }
}

// Few tokens (decode): one block per (token, 256 experts), one output per
// lane.  Every logit is still a single FMA chain in increasing k, so with few
// outputs the chains' length, not the arithmetic, sets the time; this layout
// runs T * E chains at once across the chip instead of giving each thread
// several.  The token's u row is staged once in LDS (every lane then reads the
// same address: a broadcast); each lane streams its own centroid row with
// RING groups of 32 bf16 in flight ahead of its FMAs.
constexpr int ROWS_MAX_D = 16384;                // LDS for the u row: 2*d bytes

__global__ __launch_bounds__(256) void router_scores_rows_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ e, int64_t T, int d, int E,
    float* __restrict__ s) {
    __shared__ uint4 us[ROWS_MAX_D / 8];
    const int eblocks = (E + 255) / 256;
    const int64_t t = blockIdx.x / eblocks;
    const int ex = (blockIdx.x % eblocks) * 256 + threadIdx.x;
    const bool live = ex < E;
    const uint4* ur = reinterpret_cast<const uint4*>(u + t * d);
    const uint4* er = reinterpret_cast<const uint4*>(e + (int64_t)(live ? ex : 0) * d);
    const int nchunk = d / 8;
    for (int c = threadIdx.x; c < nchunk; c += 256) us[c] = ur[c];

    constexpr int G4 = 4, RING = 4;
    const int ng = d / (8 * G4);                 // d is a multiple of 128: ng % RING == 0
    uint4 ring[RING][G4];
#pragma unroll
    for (int r = 0; r < RING; ++r)
#pragma unroll
        for (int i = 0; i < G4; ++i) ring[r][i] = er[r * G4 + i];
    __syncthreads();

    float acc = 0.0f;
    for (int g0 = 0; g0 < ng; g0 += RING) {
#pragma unroll
        for (int r = 0; r < RING; ++r) {
#pragma unroll
            for (int i = 0; i < G4; ++i) {
                const uint4 uv = us[(g0 + r) * G4 + i];
                const uint32_t ea[4] = {ring[r][i].x, ring[r][i].y, ring[r][i].z, ring[r][i].w};
                const uint32_t ua[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc = __builtin_fmaf(bf16_lo(ua[q]), bf16_lo(ea[q]), acc);
                    acc = __builtin_fmaf(bf16_hi(ua[q]), bf16_hi(ea[q]), acc);
                }
            }
            // refill this slot with the group RING ahead (the tail re-reads the last group)
            const int gn = min(g0 + r + RING, ng - 1);
#pragma unroll
            for (int i = 0; i < G4; ++i) ring[r][i] = er[gn * G4 + i];
        }
    }
    if (live) s[t * E + ex] = sigmoid_fixed(acc);
}

// One wavefront per token.  Lane l holds experts l, l+64, l+128, l+192.
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ s,
                                                          const float* __restrict__ bias,
                                                          int64_t T, int E, int K,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ gate) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* srow = s + t * E;

    uint64_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int ex = lane + 64 * j;
        key[j] = 0;
        if (ex < E) {
            const float kv = srow[ex] + bias[ex];
            key[j] = ((uint64_t)orderable_key(kv) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)ex);
        }
    }
    int chosen[16];
    for (int k = 0; k < K; ++k) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < 4; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint32_t lo = __shfl_xor((uint32_t)best, off, 64);
            const uint32_t hi = __shfl_xor((uint32_t)(best >> 32), off, 64);
            const uint64_t o = ((uint64_t)hi << 32) | lo;
            best = o > best ? o : best;
        }
        const int ex = (int)(0xFFFFFFFFu - (uint32_t)best);
        chosen[k] = ex;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (key[j] == best) key[j] = 0;   // taken (keys are unique by index)
    }
    // D: binary32 sum of the chosen raw scores in slot order.
    float D = 0.0f;
    for (int k = 0; k < K; ++k) D = D + srow[chosen[k]];
    for (int k = 0; k < K; ++k) {
        if (lane == k) {
            const float sk = srow[chosen[k]];
            idx[t * K + k] = chosen[k];
            gate[t * K + k] = (D == 0.0f) ? 0.0f : sk / D;
        }
    }
}

template <int BT, int BE, int TM, int EN>
hipError_t launch_scores(const uint16_t* u, const uint16_t* e, int64_t T, int d, int E, float* s,
                         hipStream_t st) {
    dim3 grid((unsigned)((T + BT - 1) / BT), (unsigned)((E + BE - 1) / BE));
    hipLaunchKernelGGL((router_scores_kernel<BT, BE, TM, EN>), grid, dim3(NTHREADS), 0, st, u, e,
                       T, d, E, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router_scores(const uint16_t* u, const uint16_t* e, int64_t T, int d, int E,
                                float* s, hipStream_t st) {
    // Pick the register tile so that the grid still fills the 256 CUs.  From
    // 4096 tokens on, 32 tokens x 128 experts per block with 4 x 4 logits per
    // thread: measured faster at 8192 and 16384 tokens than 16 x 256 (2 x 8),
    // 32 x 256 (4 x 8, too few blocks below 16384 tokens) and 64 x 128 (8 x 4).
    if (E > 64) {
        if (T >= 4096) return launch_scores<32, 128, 4, 4>(u, e, T, d, E, s, st);
        if (T >= 1024 || d > ROWS_MAX_D) return launch_scores<16, 128, 2, 4>(u, e, T, d, E, s, st);
        const unsigned grid = (unsigned)(T * ((E + 255) / 256));
        hipLaunchKernelGGL(router_scores_rows_kernel, dim3(grid), dim3(256), 0, st, u, e, T, d, E, s);
        return hipGetLastError();
    }
    if (T >= 4096) return launch_scores<64, 64, 4, 4>(u, e, T, d, E, s, st);
    return launch_scores<16, 16, 1, 1>(u, e, T, d, E, s, st);
}

hipError_t launch_router_topk(const float* s, const float* bias, int64_t T, int E, int K,
                              int32_t* idx, float* gate, hipStream_t st) {
    dim3 grid((unsigned)((T + 3) / 4));
    hipLaunchKernelGGL(router_topk_kernel, grid, dim3(256), 0, st, s, bias, T, E, K, idx, gate);
    return hipGetLastError();
}

}  // namespace moe
