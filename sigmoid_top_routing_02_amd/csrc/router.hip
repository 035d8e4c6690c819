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

// Few tokens, centroids shared: one block per (4 tokens, 64 experts), one
// logit per lane (wave w = token, lane = expert).  Chunks of SM_KC k-values of
// the block's 64 centroid rows are loaded with coalesced 16-byte loads into
// LDS (double-buffered through registers) and read by all four waves, so each
// centroid crosses from L2 once per 4 tokens instead of once per token; the
// tokens' u chunk is widened to FP32 in LDS and read as a broadcast.  Every
// logit is still one FMA chain in increasing k.
constexpr int SM_TOK = 4, SM_EXP = 64;

template <int SM_KC>      // k-values per chunk; divides every d that is a multiple of 128
                          // (measured: 64 beats 128 and 256, whose unrolled chunk
                          // the compiler holds in registers)
__global__ __launch_bounds__(256) void router_scores_small_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ e, int64_t T, int d, int E,
    float* __restrict__ s) {
    // centroid chunk: 64 rows of SM_KC bf16 plus one 16-byte pad per row so
    // that the 64 lanes' row reads spread over the banks
    __shared__ uint4 es[2][SM_EXP][SM_KC / 8 + 1];
    __shared__ float us[2][SM_TOK][SM_KC];
    const int egroups = (E + SM_EXP - 1) / SM_EXP;
    const int64_t t0 = (int64_t)(blockIdx.x / egroups) * SM_TOK;
    const int e0 = (blockIdx.x % egroups) * SM_EXP;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // loader roles: the chunk's 8 16-byte pieces per centroid row are moved
    // two per thread (piece p = tid and tid + 256: row p / 8, part p % 8);
    // threads 0 .. 31 move one piece of the u chunk (token tid / 8, part tid % 8)
    constexpr int PARTS = SM_KC / 8, UT = SM_TOK * PARTS;
    static_assert(SM_EXP * PARTS == 512 && UT <= 256, "loader roles assume 64-wide chunks");
    const int p0 = tid, p1 = tid + 256;
    const uint4* eg0 = reinterpret_cast<const uint4*>(e + (int64_t)min(e0 + p0 / PARTS, E - 1) * d) + p0 % PARTS;
    const uint4* eg1 = reinterpret_cast<const uint4*>(e + (int64_t)min(e0 + p1 / PARTS, E - 1) * d) + p1 % PARTS;
    const int64_t ut = min(t0 + tid / PARTS, T - 1);
    const uint4* ug = reinterpret_cast<const uint4*>(u + ut * d) + tid % PARTS;
    const int nch = d / SM_KC;
    uint4 r0 = eg0[0], r1 = eg1[0], ru = tid < UT ? ug[0] : uint4{0, 0, 0, 0};
    float* const udst0 = &us[0][tid / PARTS % SM_TOK][(tid % PARTS) * 8];
    const int ustride = SM_TOK * SM_KC;          // floats from us[0] to us[1]
#define MOE_SMALL_PUT(B)                                                      \
    do {                                                                      \
        es[B][p0 / PARTS][p0 % PARTS] = r0;                                   \
        es[B][p1 / PARTS][p1 % PARTS] = r1;                                   \
        if (tid < UT) {                                                       \
            float* dst = udst0 + (B) * ustride;                               \
            dst[0] = bf16_lo(ru.x); dst[1] = bf16_hi(ru.x);                   \
            dst[2] = bf16_lo(ru.y); dst[3] = bf16_hi(ru.y);                   \
            dst[4] = bf16_lo(ru.z); dst[5] = bf16_hi(ru.z);                   \
            dst[6] = bf16_lo(ru.w); dst[7] = bf16_hi(ru.w);                   \
        }                                                                     \
    } while (0)
    MOE_SMALL_PUT(0);
    __syncthreads();
    float acc = 0.0f;
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        // next chunk into registers (the last step re-reads the last chunk into
        // the spare buffer: the loop body has no branch around the loads)
        const int off = min(c + 1, nch - 1) * PARTS;
        r0 = eg0[off];
        r1 = eg1[off];
        if (tid < UT) ru = ug[off];
#pragma unroll
        for (int j = 0; j < PARTS; ++j) {
            const uint4 ev = es[b][lane][j];
            const uint32_t wd[4] = {ev.x, ev.y, ev.z, ev.w};
            const float* uv = &us[b][w][j * 8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = __builtin_fmaf(uv[2 * q], bf16_lo(wd[q]), acc);
                acc = __builtin_fmaf(uv[2 * q + 1], bf16_hi(wd[q]), acc);
            }
        }
        // the chunk's FMAs stay before the barrier (the compiler would otherwise
        // sink them below the next chunk's LDS writes, whose wait for the
        // global loads would then hide nothing)
        asm volatile("" :: "v"(acc));
        __syncthreads();                         // every wave is done with buffer b ^ 1's last use
        MOE_SMALL_PUT(b ^ 1);
        __syncthreads();
    }
#undef MOE_SMALL_PUT
    const int64_t t = t0 + w;
    const int ex = e0 + lane;
    if (t < T && ex < E) s[t * E + ex] = sigmoid_fixed(acc);
}

// wave-wide maximum of a 64-bit key
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// One wavefront per token.  Lane l holds experts l, l+64, l+128, l+192.
// Each expert's 64-bit key is (orderable(s + b) << 32) | (~index), so the
// largest key is the largest biased score with ties to the lower index, and 0
// marks an expert that is taken or not eligible.
// Group-limited selection (n_groups > 1): the experts form n_groups groups of
// E / n_groups consecutive indices; a group's score is the largest key of its
// experts, the topk_groups best groups are kept (ties to the lower group,
// which the index part of the key gives), and the K experts are chosen among
// the kept groups' experts only.
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ s,
                                                          const float* __restrict__ bias,
                                                          int64_t T, int E, int K,
                                                          int n_groups, int topk_groups,
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
    if (n_groups > 1) {
        const int gs = E / n_groups;
        // lane g < n_groups ends up holding group g's score
        uint64_t gscore = 0;
        for (int g = 0; g < n_groups; ++g) {
            uint64_t m = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ex = lane + 64 * j;
                if (ex < E && ex / gs == g) m = key[j] > m ? key[j] : m;
            }
            m = wave_max_u64(m);
            if (lane == g) gscore = m;
        }
        uint64_t kept = 0;                       // bit g: group g is kept
        for (int r = 0; r < topk_groups; ++r) {
            const uint64_t best = wave_max_u64(gscore);
            const uint64_t win = __ballot(gscore == best && best != 0);
            if (win == 0) break;
            const int g = __builtin_ctzll(win);
            kept |= 1ull << g;
            if (lane == g) gscore = 0;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ex = lane + 64 * j;
            if (ex < E && !((kept >> (ex / gs)) & 1ull)) key[j] = 0;
        }
    }
    int chosen[16];
    for (int k = 0; k < K; ++k) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < 4; ++j) best = key[j] > best ? key[j] : best;
        best = wave_max_u64(best);
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
        if (T >= 1024) return launch_scores<16, 128, 2, 4>(u, e, T, d, E, s, st);
        const unsigned grid = (unsigned)((T + SM_TOK - 1) / SM_TOK * ((E + SM_EXP - 1) / SM_EXP));
        hipLaunchKernelGGL(router_scores_small_kernel<64>, dim3(grid), dim3(256), 0, st, u, e, T, d, E, s);
        return hipGetLastError();
    }
    if (T >= 4096) return launch_scores<64, 64, 4, 4>(u, e, T, d, E, s, st);
    return launch_scores<16, 16, 1, 1>(u, e, T, d, E, s, st);
}

hipError_t launch_router_topk(const float* s, const float* bias, int64_t T, int E, int K,
                              int n_groups, int topk_groups, int32_t* idx, float* gate,
                              hipStream_t st) {
    dim3 grid((unsigned)((T + 3) / 4));
    hipLaunchKernelGGL(router_topk_kernel, grid, dim3(256), 0, st, s, bias, T, E, K, n_groups,
                       topk_groups, idx, gate);
    return hipGetLastError();
}

}  // namespace moe
