// Router: s = sigmoid(u . e_i) for every token and routed expert, then the
// biased top-K choice and the gates.
//
// Sources: "DeepSeek-V3 Technical Report" notes (learn.ifs.name), MoE-routing
// and bias paragraphs; nlp-lineage summary, "The notation".  As computed here:
// expert i is in token t's set iff s[t,i] + b_i ranks among the token's K
// largest; g = s / (sum of s over the set); b takes part in the ranking only.
//
// Affinity kernels: each output's dot product is one FP32 FMA chain in
// increasing k (bf16 products are exact in FP32, so the chain fixes the result
// bit for bit).  Three kernels keep that order: from 4096 tokens on, the chain
// runs on the matrix cores as K = 1 FP32 MFMAs (one rounding per step, the
// same as the FMA; MFMAs with K > 1 sum several products in an unspecified
// order and are not used), with a per-block range certificate and a VALU
// fallback; below that, a register-tiled VALU kernel (every thread owns TM
// tokens x EN experts) and, for few tokens, one logit per lane.  Tiles of
// k-values of u and of the centroids are widened to FP32 into LDS.
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

// Many tokens: the same chains on the matrix cores.  bf16 x bf16 products are
// exact in FP32, so one step of a logit's chain is fl(acc + u_k e_k), and the
// FP32 MFMA with K = 1 (v_mfma_f32_32x32x1_2b_f32: D = a (x) b + C for two
// 32 x 32 blocks) performs exactly that step on every element, as long as
// every product and partial sum stays in FP32's normal range (measured on
// gfx950: bit-identical to the FMA chain on 2.3e8 steps of router-like data
// and on large-by-tiny products; denormal products and overflow differ).  A
// chain of such MFMAs in increasing k therefore gives the logits of the FMA
// chain bit for bit.  The range is certified per block from the bf16 exponent
// fields f (f' = max(f, 1)) gathered while the inputs are staged:
//   every nonzero product's last bit is 2^(f'_u + f'_e - 268) >= 2^-126 when
//   min f'_u + min f'_e >= 142, so every nonzero partial sum is normal;
//   |sum| < d 2^(max f_u + max f_e - 252) <= 2^126 when
//   max f_u + max f_e + ceil(log2 d) <= 378 (and no Inf/NaN input, f < 255).
// A block whose inputs fail either bound recomputes its logits with the FMA
// chain on the VALU, so every input gets the same result as the VALU kernels.
//
// Block: 64 tokens x 128 experts, 4 waves of 32 tokens x 64 experts (the two
// MFMA blocks: experts 64 we + [0, 32) and + [32, 64)).  Lane l feeds token
// 32 wt + l % 32 (both MFMA blocks share the tokens) and expert 64 we + l.
// Chunks of MC k-values of the block's rows are widened to FP32 into LDS
// (row pitch MC + 4 floats: the 16 lanes of a 16-byte read cover all banks),
// double-buffered; chunk c + 2's global loads are issued at the start of chunk
// c, and chunk c + 1 is widened, checked and stored in pieces placed after
// single MFMAs of chunk c, so that the VALU and LDS work of the staging
// overlaps the matrix instructions instead of following them.
constexpr int MB_T = 64, MB_E = 128, MC = 32, MP = MC + 4;

__global__ __launch_bounds__(256) void router_scores_mfma_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ e, int64_t T, int d, int E, int lg2d,
    float* __restrict__ s) {
    typedef float mv32 __attribute__((ext_vector_type(32)));
    __shared__ __attribute__((aligned(16))) float us[2][MB_T][MP];
    __shared__ __attribute__((aligned(16))) float es[2][MB_E][MP];
    __shared__ int ex_stat[4];                 // min f'_u, max f_u, min f'_e, max f_e
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wt = w >> 1, we = w & 1;
    const int64_t t0 = (int64_t)blockIdx.x * MB_T;
    const int e0 = blockIdx.y * MB_E;
    if (tid == 0) { ex_stat[0] = 1 << 20; ex_stat[1] = 0; ex_stat[2] = 1 << 20; ex_stat[3] = 0; }
    // loaders: u piece tid (row tid / 4, 8 k-values at part tid % 4); e pieces
    // tid and tid + 256.  Rows past T or E read the last row and are not stored.
    const int ur = tid >> 2, up = tid & 3;
    const uint4* ug = reinterpret_cast<const uint4*>(u + (int64_t)min(t0 + ur, T - 1) * d) + up;
    const uint4* eg0 = reinterpret_cast<const uint4*>(e + (int64_t)min(e0 + (tid >> 2), E - 1) * d) + up;
    const uint4* eg1 = reinterpret_cast<const uint4*>(e + (int64_t)min(e0 + 64 + (tid >> 2), E - 1) * d) + up;
    // Exponent extremes as 16-bit magnitudes x = |bf16 bits|, two per word:
    // the smallest nonzero x (kept as x - 1, so that a zero wraps to 0xFFFF
    // and never wins the minimum) and the largest x.  f = x >> 7 is monotone
    // in x, so min f' = max((min nonzero x) >> 7, 1) and max f = (max x) >> 7.
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 mn_u = {0xFFFF, 0xFFFF}, mx_u = {0, 0}, mn_e = {0xFFFF, 0xFFFF}, mx_e = {0, 0};
    auto stat = [](const uint4& v, us2& mn, us2& mx) {
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const us2 x = __builtin_bit_cast(us2, wd[q] & 0x7FFF7FFFu);
            mn = __builtin_elementwise_min(mn, x - (us2){1, 1});
            mx = __builtin_elementwise_max(mx, x);
        }
    };
    auto put = [](float* row, const uint4& v) {
        reinterpret_cast<float4*>(row)[0] = float4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
        reinterpret_cast<float4*>(row)[1] = float4{bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    };
    const int nch = d / MC;                    // even: d is a multiple of 128
    // global offset of chunk c; past the end it re-reads the last chunk (the
    // loads stay unconditional, and what they bring is never used)
    auto goff = [nch](int c) { return (c < nch ? c : nch - 1) * (MC / 8); };
    uint4 ru = ug[0], re0 = eg0[0], re1 = eg1[0];
    // two register sets alternate: during chunk c one holds chunk c + 1's rows
    // (loaded during chunk c - 1), which are staged into LDS, while chunk c + 2's
    // rows are loaded into the other
    uint4 xu = ug[goff(1)], xe0 = eg0[goff(1)], xe1 = eg1[goff(1)];
    uint4 yu, ye0, ye1;
    __syncthreads();                           // ex_stat initialised
    put(&us[0][ur][up * 8], ru);
    put(&es[0][tid >> 2][up * 8], re0);
    put(&es[0][64 + (tid >> 2)][up * 8], re1);
    stat(ru, mn_u, mx_u);
    stat(re0, mn_e, mx_e);
    stat(re1, mn_e, mx_e);
    __syncthreads();
    mv32 acc = {};
    const int tok_l = 32 * wt + (lane & 31), exp_l = 64 * we + lane;
    // k-groups of 4 are read one group ahead into two register slots
    float4 av[2], bv[2];
    av[0] = *reinterpret_cast<const float4*>(&us[0][tok_l][0]);
    bv[0] = *reinterpret_cast<const float4*>(&es[0][exp_l][0]);
    auto mfma = [&acc](float a, float bq) { acc = __builtin_amdgcn_mfma_f32_32x32x1f32(a, bq, acc, 0, 0, 0); };
    auto chunk = [&](int c, int b, const uint4& su, const uint4& se0, const uint4& se1, uint4& lu,
                     uint4& le0, uint4& le1) {
        lu = ug[goff(c + 2)];
        le0 = eg0[goff(c + 2)];
        le1 = eg1[goff(c + 2)];
        const float* ua = &us[b][tok_l][0];
        const float* eb = &es[b][exp_l][0];
        // buffer b ^ 1 was last read in chunk c - 1, before the barrier that
        // ended it; after the last chunk this stages a repeat that nothing reads
        float* wu = &us[b ^ 1][ur][up * 8];
        float* we0 = &es[b ^ 1][tid >> 2][up * 8];
        float* we1 = &es[b ^ 1][64 + (tid >> 2)][up * 8];
#pragma unroll
        for (int g = 0; g < MC / 4 - 1; ++g) {
            av[(g + 1) & 1] = *reinterpret_cast<const float4*>(ua + 4 * (g + 1));
            bv[(g + 1) & 1] = *reinterpret_cast<const float4*>(eb + 4 * (g + 1));
            const float4 a = av[g & 1], bq = bv[g & 1];
            mfma(a.x, bq.x);
            // one piece of the staging in the shadow of each group's first MFMA
            __builtin_amdgcn_sched_barrier(0);
            switch (g) {
                case 0: stat(su, mn_u, mx_u); break;
                case 1: put(wu, su); break;
                case 2: stat(se0, mn_e, mx_e); break;
                case 3: put(we0, se0); break;
                case 4: stat(se1, mn_e, mx_e); break;
                case 5: put(we1, se1); break;
                default: break;
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma(a.y, bq.y);
            mfma(a.z, bq.z);
            mfma(a.w, bq.w);
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        // the next chunk's first group, then this chunk's last one
        av[0] = *reinterpret_cast<const float4*>(&us[b ^ 1][tok_l][0]);
        bv[0] = *reinterpret_cast<const float4*>(&es[b ^ 1][exp_l][0]);
        mfma(av[1].x, bv[1].x);
        mfma(av[1].y, bv[1].y);
        mfma(av[1].z, bv[1].z);
        mfma(av[1].w, bv[1].w);
        __builtin_amdgcn_sched_barrier(0);
        // keeps those two reads here, under the last group's MFMAs, rather
        // than at the next chunk's start, where the first MFMA would wait on them
        asm volatile("" : "+v"(av[0].x), "+v"(av[0].y), "+v"(av[0].z), "+v"(av[0].w),
                          "+v"(bv[0].x), "+v"(bv[0].y), "+v"(bv[0].z), "+v"(bv[0].w));
    };
    for (int c = 0; c < nch; c += 2) {
        chunk(c, 0, xu, xe0, xe1, yu, ye0, ye1);
        chunk(c + 1, 1, yu, ye0, ye1, xu, xe0, xe1);
    }
    // the block's exponent extremes; rows past T or E repeat valid rows
    const unsigned mnu = min(mn_u.x, mn_u.y), mne = min(mn_e.x, mn_e.y);
    atomicMin(&ex_stat[0], mnu == 0xFFFFu ? 1 << 20 : max((int)((mnu + 1) >> 7), 1));
    atomicMax(&ex_stat[1], (int)(max(mx_u.x, mx_u.y) >> 7));
    atomicMin(&ex_stat[2], mne == 0xFFFFu ? 1 << 20 : max((int)((mne + 1) >> 7), 1));
    atomicMax(&ex_stat[3], (int)(max(mx_e.x, mx_e.y) >> 7));
    __syncthreads();
    const bool certified = ex_stat[0] + ex_stat[2] >= 142 && ex_stat[1] < 255 && ex_stat[3] < 255 &&
                           ex_stat[1] + ex_stat[3] + lg2d <= 378;
    if (certified) {
        // D[i][j] of MFMA block bb sits in lane j + 32 ((i / 4) % 2), register
        // 16 bb + (i % 4) + 4 (i / 8)
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            const int bb = r >> 4, rr = r & 15;
            const int i = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
            const int64_t t = t0 + 32 * wt + i;
            const int ex = e0 + 64 * we + 32 * bb + (lane & 31);
            if (t < T && ex < E) s[t * E + ex] = sigmoid_fixed(acc[r]);
        }
    } else {
        // the FMA chain on the VALU: thread = token tid / 4, experts 32 (tid % 4) + [0, 32)
        const int64_t t = t0 + (tid >> 2);
        const int xb = e0 + 32 * (tid & 3);
        if (t < T) {
            const uint16_t* urow = u + t * d;
            for (int j = 0; j < 32; ++j) {
                const int ex = xb + j;
                if (ex >= E) break;
                const uint16_t* erow = e + (int64_t)ex * d;
                float a = 0.0f;
                for (int k = 0; k < d; ++k)
                    a = __builtin_fmaf(__uint_as_float((uint32_t)urow[k] << 16),
                                       __uint_as_float((uint32_t)erow[k] << 16), a);
                s[t * E + ex] = sigmoid_fixed(a);
            }
        }
    }
}

// Few tokens, centroids shared: one block per (4 tokens, 64 experts), one
// logit per lane (wave w = token, lane = expert).  Chunks of SM_KC k-values of
// the block's 64 centroid rows and 4 token rows are loaded with coalesced
// 16-byte loads, widened to FP32 once as they are put into LDS, and read by
// all four waves (each centroid crosses from L2 once per 4 tokens, and the
// chain's loop holds nothing but its FMAs and 16-byte LDS reads; the u chunk
// is read as a broadcast).  The loads run SM_PF chunks ahead through a ring of
// registers, so their latency hides behind the FMAs of the chunks between.
// Every logit is still one FMA chain in increasing k.
constexpr int SM_TOK = 4, SM_EXP = 64, SM_WIN = 8;

template <int SM_KC, int SM_PF>   // SM_KC divides d (the launcher picks it)
__global__ __launch_bounds__(256) void router_scores_small_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ e, int64_t T, int d, int E,
    float* __restrict__ s) {
    // centroid chunk: 64 rows of SM_KC floats plus one 16-byte pad per row so
    // that the 64 lanes' row reads spread over the banks
    constexpr int Q = SM_KC / 4;                 // float4 per row of a chunk
    constexpr int PARTS = SM_KC / 8;             // 16-byte pieces (8 bf16) per row of a chunk
    constexpr int NP = SM_EXP * PARTS / 256;     // centroid pieces per thread per chunk
    constexpr int UT = SM_TOK * PARTS;           // u pieces per chunk
    static_assert(SM_EXP * PARTS % 256 == 0 && UT <= 256, "loader roles");
    __shared__ float4 es[2][SM_EXP][Q + 1];
    __shared__ float4 us[2][SM_TOK][Q];
    const int egroups = (E + SM_EXP - 1) / SM_EXP;
    const int64_t t0 = (int64_t)(blockIdx.x / egroups) * SM_TOK;
    const int e0 = (blockIdx.x % egroups) * SM_EXP;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // loader roles: centroid piece p = tid + 256 q (q < NP) is row p / PARTS,
    // part p % PARTS; u piece tid % UT is token (tid % UT) / PARTS, part
    // tid % PARTS (threads past UT load a copy of one and drop it, so every
    // thread issues the same loads and the compiler's wait counts stay exact)
    const uint4* eg[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
        const int pc = tid + 256 * q;
        eg[q] = reinterpret_cast<const uint4*>(e + (int64_t)min(e0 + pc / PARTS, E - 1) * d) + pc % PARTS;
    }
    const int64_t ut = min(t0 + (tid % UT) / PARTS, T - 1);
    const uint4* ug = reinterpret_cast<const uint4*>(u + ut * d) + tid % PARTS;
    const int nch = d / SM_KC;
    uint4 re[SM_PF][NP], ru[SM_PF];
    auto load = [&](int slot, int c) {           // chunk min(c, nch - 1) into ring slot `slot`
        const int off = min(c, nch - 1) * PARTS;
#pragma unroll
        for (int q = 0; q < NP; ++q) re[slot][q] = eg[q][off];
        ru[slot] = ug[off];
    };
    // 8 bf16 (k .. k+7, k in the low half of each word) as two float4
    auto widen = [](const uint4& v, float4& lo, float4& hi) {
        lo = float4{bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y)};
        hi = float4{bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
    };
    auto put = [&](int B, int slot) {
        float4 lo, hi;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int pc = tid + 256 * q;
            widen(re[slot][q], lo, hi);
            es[B][pc / PARTS][(pc % PARTS) * 2] = lo;
            es[B][pc / PARTS][(pc % PARTS) * 2 + 1] = hi;
        }
        if (tid < UT) {
            widen(ru[slot], lo, hi);
            us[B][tid / PARTS][(tid % PARTS) * 2] = lo;
            us[B][tid / PARTS][(tid % PARTS) * 2 + 1] = hi;
        }
    };
#pragma unroll
    for (int i = 0; i < SM_PF; ++i) load(i, i);
    put(0, 0);
    __syncthreads();
    float acc = 0.0f;
    for (int cb = 0; cb < nch; cb += SM_PF) {
#pragma unroll
        for (int i = 0; i < SM_PF; ++i) {
            const int c = cb + i;
            if (c >= nch) break;
            const int b = c & 1;
            load(i, c + SM_PF);                  // slot i held chunk c, already in LDS
            // a window of SM_WIN steps (one float4 of the centroid row and
            // one of u, four FMAs each): the reads of step j + SM_WIN go out
            // as step j's FMAs retire, so the LDS latency hides behind the
            // chain (at most 2 (SM_WIN - 1) reads outstanding when a step
            // waits, within the LDS counter's range)
            const float4* erow = es[b][lane];
            const float4* urow = us[b][w];
            float4 ev[SM_WIN], uv[SM_WIN];
#pragma unroll
            for (int j = 0; j < SM_WIN; ++j) {
                ev[j] = erow[j];
                uv[j] = urow[j];
            }
#pragma unroll
            for (int j = 0; j < Q; ++j) {
                const int r = j % SM_WIN;
                acc = __builtin_fmaf(uv[r].x, ev[r].x, acc);
                acc = __builtin_fmaf(uv[r].y, ev[r].y, acc);
                acc = __builtin_fmaf(uv[r].z, ev[r].z, acc);
                acc = __builtin_fmaf(uv[r].w, ev[r].w, acc);
                if (j + SM_WIN < Q) {
                    ev[r] = erow[j + SM_WIN];
                    uv[r] = urow[j + SM_WIN];
                }
                __builtin_amdgcn_sched_barrier(0);   // keep the window's order
            }
            // the chunk's FMAs stay before the barrier (the compiler would
            // otherwise sink them below the next chunk's LDS writes)
            asm volatile("" :: "v"(acc));
            // buffer b ^ 1 was last read in chunk c - 1, before the barrier
            // that ended it, so it can be refilled while others still read b
            put(b ^ 1, (i + 1) % SM_PF);         // chunk c + 1 (past the end: unused)
            __syncthreads();
        }
    }
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
        if (T >= 4096) {
            // the matrix-core chains (a K = 1 FP32 MFMA per step)
            int lg2d = 0;
            while ((1 << lg2d) < d) ++lg2d;
            const dim3 grid((unsigned)((T + MB_T - 1) / MB_T), (unsigned)((E + MB_E - 1) / MB_E));
            hipLaunchKernelGGL(router_scores_mfma_kernel, grid, dim3(256), 0, st, u, e, T, d, E, lg2d, s);
            return hipGetLastError();
        }
        if (T >= 1024) return launch_scores<16, 128, 2, 4>(u, e, T, d, E, s, st);
        // fewer tokens: one logit per lane, chunks of 256 k-values (128 when d
        // is an odd multiple of 128) fetched two ahead
        const unsigned grid = (unsigned)((T + SM_TOK - 1) / SM_TOK * ((E + SM_EXP - 1) / SM_EXP));
        if (d % 256 == 0)
            hipLaunchKernelGGL((router_scores_small_kernel<256, 2>), dim3(grid), dim3(256), 0, st, u, e, T, d, E, s);
        else
            hipLaunchKernelGGL((router_scores_small_kernel<128, 2>), dim3(grid), dim3(256), 0, st, u, e, T, d, E, s);
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
