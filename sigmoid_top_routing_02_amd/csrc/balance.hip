// Sequence-wise balance loss (a training-side quantity beside the routing).
//
// "DeepSeek-V3 Technical Report" notes, bias paragraph: besides the bias, a
// very small sequence-wise loss guards against extreme imbalance inside one
// sequence.  The pages give no formula; this library's reading is the usual
// frequency-times-probability balance term, per sequence of L tokens:
//     f_i  = E / (K L) * #{tokens of the sequence that chose expert i}
//     P_i  = (1/L) * sum_t s[t,i] / sum_j s[t,j]      (raw sigmoid scores)
//     loss = alpha * sum_i f_i P_i
// Uniform use gives alpha; every token on the same K experts with all of its
// score on them gives alpha * E / K.  A token whose scores sum to 0 adds
// nothing to P.
//
// Two passes, both in a fixed order (deterministic).  Pass 1: one block of 4
// waves per chunk of 64 tokens of a sequence; wave w takes tokens w, w+4, ...
// of the chunk, four rows at a time so that four row loads are in flight;
// lane l holds experts l, l+64, l+128, l+192; per token the wave sums the row
// (each lane over its experts in order, then a butterfly), divides and
// accumulates.  Expert counts go to LDS with integer atomics (exact in any
// order).  The chunk's partial P and counts go to the workspace.  Pass 2: one
// block per sequence adds the chunks in order and reduces the E terms by a
// fixed tree.
#include "kernels.h"

namespace moe {
namespace {

constexpr int BAL_CHUNK = 64;       // tokens per pass-1 block
constexpr int BAL_WAVES = 4;
constexpr int BAL_UNROLL = 4;       // rows in flight per wave

struct BalancePart {
    float p[256];
    int32_t cnt[256];
};

__global__ __launch_bounds__(64 * BAL_WAVES) void seq_balance_partial_kernel(
    const float* __restrict__ s, const int32_t* __restrict__ idx, int E, int K, int L, int nchunk,
    BalancePart* __restrict__ part) {
    __shared__ int cnt[256];
    __shared__ float wpart[BAL_WAVES][256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    cnt[tid] = 0;                                   // 256 threads
    __syncthreads();
    const int q = blockIdx.x / nchunk, c = blockIdx.x % nchunk;
    const int tb = c * BAL_CHUNK, te = min(L, tb + BAL_CHUNK);
    const int64_t base = (int64_t)q * L;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int t = tb + wave; t < te; t += BAL_WAVES * BAL_UNROLL) {
        float v[BAL_UNROLL][4];
#pragma unroll
        for (int r = 0; r < BAL_UNROLL; ++r) {
            const int tt = t + r * BAL_WAVES;
            const float* row = s + (base + tt) * E;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = lane + 64 * j;
                v[r][j] = (tt < te && e < E) ? row[e] : 0.f;
            }
        }
#pragma unroll
        for (int r = 0; r < BAL_UNROLL; ++r) {
            float rs = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) rs = rs + v[r][j];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) rs = rs + __shfl_xor(rs, off, 64);
            if (rs != 0.f) {
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = acc[j] + v[r][j] / rs;
            }
            const int tt = t + r * BAL_WAVES;
            if (tt < te && lane < K) {
                const int e = idx[(base + tt) * K + lane];
                if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);     // other values are ignored
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) wpart[wave][lane + 64 * j] = acc[j];
    __syncthreads();
    float p = 0.f;
#pragma unroll
    for (int w = 0; w < BAL_WAVES; ++w) p = p + wpart[w][tid];
    part[blockIdx.x].p[tid] = p;
    part[blockIdx.x].cnt[tid] = cnt[tid];
}

__global__ __launch_bounds__(256) void seq_balance_final_kernel(const BalancePart* __restrict__ part,
                                                                int E, int K, int L, int nchunk,
                                                                float alpha, float* __restrict__ loss) {
    __shared__ float term[256];
    const int tid = threadIdx.x, q = blockIdx.x;
    float p = 0.f;
    int n = 0;
    for (int c = 0; c < nchunk; ++c) {
        p = p + part[(int64_t)q * nchunk + c].p[tid];
        n += part[(int64_t)q * nchunk + c].cnt[tid];
    }
    const float f = (float)E * (float)n / ((float)K * (float)L);
    term[tid] = tid < E ? f * (p / (float)L) : 0.f;
    __syncthreads();
    for (int h = 128; h >= 1; h >>= 1) {
        if (tid < h) term[tid] = term[tid] + term[tid + h];
        __syncthreads();
    }
    if (tid == 0) loss[q] = alpha * term[0];
}

}  // namespace

size_t seq_balance_ws_bytes(int64_t n_seq, int L) {
    const int64_t nchunk = (L + BAL_CHUNK - 1) / BAL_CHUNK;
    return (size_t)(n_seq * nchunk) * sizeof(BalancePart);
}

hipError_t launch_seq_balance_loss(const float* s, const int32_t* idx, int64_t n_seq, int E, int K,
                                   int L, float alpha, float* loss, void* ws, hipStream_t st) {
    const int nchunk = (L + BAL_CHUNK - 1) / BAL_CHUNK;
    BalancePart* part = static_cast<BalancePart*>(ws);
    hipLaunchKernelGGL(seq_balance_partial_kernel, dim3((unsigned)(n_seq * nchunk)), dim3(64 * BAL_WAVES), 0,
                       st, s, idx, E, K, L, nchunk, part);
    hipLaunchKernelGGL(seq_balance_final_kernel, dim3((unsigned)n_seq), dim3(256), 0, st, part, E, K, L,
                       nchunk, alpha, loss);
    return hipGetLastError();
}

}  // namespace moe
