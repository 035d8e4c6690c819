// Dispatch: per-expert histogram, exclusive scan and a stable counting-sort
// permutation of the (token, slot) assignments, with no capacity limit -- no
// token is ever dropped (nlp-lineage summary, "The idea", load-balancing
// bullet).  Rows are ordered by (expert, token); the shared expert's rows
// ("DeepSeek-V3 Technical Report" notes, MoE-routing paragraph: one shared
// expert every token uses) follow in token order.
//
// Deterministic without order-dependent atomics:
//  1. hist:    per chunk of 64 tokens, a 64-bit token mask per expert (LDS
//              atomicOr is order-independent), its popcount = chunk count.
//  2. scan:    per expert, exclusive prefix over chunks; then the exclusive
//              scan over experts gives group_offset.
//  3. scatter: row = group_offset[e] + chunk_prefix[c][e]
//              + popcount(mask[c][e] & lanes-below-t).
// Up to SMALL_T tokens the three steps run in one block with the masks and
// prefixes in LDS (one launch instead of three; the same arithmetic, so the
// same result).
#include "device_math.h"
#include "kernels.h"
#include "moe_fp8.h"

namespace moe {
namespace {

constexpr int CHUNK = 64;   // tokens per histogram chunk (one 64-bit mask)

struct DispatchWs {
    uint64_t* mask;     // [nchunk][E]
    int32_t* cnt;       // [nchunk][E]
    int32_t* prefix;    // [nchunk][E]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline DispatchWs carve(void* ws, int64_t nchunk, int E) {
    char* p = static_cast<char*>(ws);
    DispatchWs w;
    w.mask = reinterpret_cast<uint64_t*>(p);
    p += align256(sizeof(uint64_t) * nchunk * E);
    w.cnt = reinterpret_cast<int32_t*>(p);
    p += align256(sizeof(int32_t) * nchunk * E);
    w.prefix = reinterpret_cast<int32_t*>(p);
    return w;
}

__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ idx,
                                                            int64_t T, int K, int E,
                                                            DispatchWs w) {
    __shared__ unsigned long long m[256];
    const int c = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += 256) m[e] = 0ull;
    __syncthreads();
    const int64_t t0 = (int64_t)c * CHUNK;
    const int n = CHUNK * K;
    for (int j = threadIdx.x; j < n; j += 256) {
        const int tl = j / K;
        const int64_t t = t0 + tl;
        if (t >= T) continue;
        const int ex = idx[t * K + (j % K)];
        if (ex >= 0 && ex < E) atomicOr(&m[ex], 1ull << tl);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        const unsigned long long v = m[e];
        w.mask[(int64_t)c * E + e] = v;
        w.cnt[(int64_t)c * E + e] = __popcll(v);
    }
}

// One block of 1024 threads: expert e is handled by threads e, e+256, e+512
// and e+768, each owning a quarter of the chunks.  A quarter's total is summed
// first, the quarters before it give its starting offset, and then its chunk
// prefixes are written (integer sums: the result is the same as one thread
// walking all chunks).  The chunk counts are loaded SCAN_BATCH at a time, so
// each running sum waits for one memory latency per batch, not per chunk.
constexpr int SCAN_PARTS = 4;
__global__ __launch_bounds__(256 * SCAN_PARTS) void dispatch_scan_kernel(int64_t nchunk, int64_t T, int K,
                                                                         int E, int include_shared,
                                                                         DispatchWs w, int32_t* count,
                                                                         int32_t* group_offset) {
    constexpr int SCAN_BATCH = 16;
    __shared__ int32_t psum[SCAN_PARTS][256];
    __shared__ int32_t tot[256];
    const int e = threadIdx.x & 255, part = threadIdx.x >> 8;
    const int64_t q = (nchunk + SCAN_PARTS - 1) / SCAN_PARTS;
    const int64_t c_lo = min(nchunk, part * q), c_hi = min(nchunk, c_lo + q);
    // the sum of this quarter's counts
    int32_t qsum = 0;
    if (e < E) {
        for (int64_t c0 = c_lo; c0 < c_hi; c0 += SCAN_BATCH) {
            int32_t v[SCAN_BATCH];
#pragma unroll
            for (int i = 0; i < SCAN_BATCH; ++i) v[i] = (c0 + i < c_hi) ? w.cnt[(c0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < SCAN_BATCH; ++i) qsum += v[i];
        }
    }
    psum[part][e] = qsum;
    __syncthreads();
    // the chunk prefixes of this quarter, starting after the quarters before it
    int32_t run = 0;
    for (int p = 0; p < part; ++p) run += psum[p][e];
    if (e < E) {
        for (int64_t c0 = c_lo; c0 < c_hi; c0 += SCAN_BATCH) {
            int32_t v[SCAN_BATCH];
#pragma unroll
            for (int i = 0; i < SCAN_BATCH; ++i) v[i] = (c0 + i < c_hi) ? w.cnt[(c0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < SCAN_BATCH; ++i) {
                if (c0 + i < c_hi) w.prefix[(c0 + i) * E + e] = run;
                run += v[i];
            }
        }
    }
    // expert totals, then the inclusive Hillis-Steele scan over 256 entries
    int32_t total = 0;
    if (part == 0) {
        for (int p = 0; p < SCAN_PARTS; ++p) total += psum[p][e];
        if (e < E) count[e] = total;
        tot[e] = (e < E) ? total : 0;
    }
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int32_t v = (part == 0 && e >= off) ? tot[e - off] : 0;
        __syncthreads();
        if (part == 0) tot[e] += v;
        __syncthreads();
    }
    if (part == 0) {
        if (e < E) group_offset[e] = tot[e] - total;   // exclusive
        if (e == 0) {
            group_offset[E] = tot[255];
            if (include_shared) group_offset[E + 1] = tot[255] + (int32_t)T;
        }
    }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int K, int E, int include_shared, DispatchWs w,
    const int32_t* __restrict__ group_offset, int32_t* __restrict__ row_token,
    int32_t* __restrict__ slot_row) {
    const int c = blockIdx.x;
    const int64_t t0 = (int64_t)c * CHUNK;
    const int n = CHUNK * K;
    for (int j = threadIdx.x; j < n; j += 256) {
        const int tl = j / K;
        const int k = j % K;
        const int64_t t = t0 + tl;
        if (t >= T) continue;
        const int ex = idx[t * K + k];
        if (ex < 0 || ex >= E) continue;
        const uint64_t below = (tl == 0) ? 0ull : (w.mask[(int64_t)c * E + ex] & ((1ull << tl) - 1ull));
        const int32_t row = group_offset[ex] + w.prefix[(int64_t)c * E + ex] + __popcll(below);
        row_token[row] = (int32_t)t;
        slot_row[t * K + k] = row;
    }
    if (include_shared) {
        for (int tl = threadIdx.x; tl < CHUNK; tl += 256) {
            const int64_t t = t0 + tl;
            if (t < T) row_token[T * K + t] = (int32_t)t;
        }
    }
}

// The three steps above in one 1024-thread block for T <= SMALL_T (at most
// SMALL_T / CHUNK chunks of masks and prefixes, held in LDS).
constexpr int SMALL_T = 1024;
constexpr int SMALL_CH = SMALL_T / CHUNK;

__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t* __restrict__ idx, int64_t T, int K,
                                                              int E, int include_shared,
                                                              int32_t* __restrict__ count,
                                                              int32_t* __restrict__ group_offset,
                                                              int32_t* __restrict__ row_token,
                                                              int32_t* __restrict__ slot_row) {
    __shared__ unsigned long long m[SMALL_CH][256];
    __shared__ int32_t pre[SMALL_CH][256];
    __shared__ int32_t cnt[256], inc[256];
    const int tid = threadIdx.x;
    const int nch = (int)((T + CHUNK - 1) / CHUNK);
    const int n = (int)T * K;
    for (int i = tid; i < nch * 256; i += 1024) m[i / 256][i % 256] = 0ull;
    __syncthreads();
    for (int j = tid; j < n; j += 1024) {
        const int t = j / K;
        const int ex = idx[j];
        if (ex >= 0 && ex < E) atomicOr(&m[t / CHUNK][ex], 1ull << (t % CHUNK));
    }
    __syncthreads();
    if (tid < 256) {
        int32_t run = 0;
        for (int c = 0; c < nch; ++c) {
            pre[c][tid] = run;
            run += __popcll(m[c][tid]);     // experts >= E have empty masks
        }
        cnt[tid] = run;
        inc[tid] = run;
        if (tid < E) count[tid] = run;
    }
    __syncthreads();
    // inclusive Hillis-Steele scan over the 256 expert totals
    for (int off = 1; off < 256; off <<= 1) {
        const int32_t v = (tid < 256 && tid >= off) ? inc[tid - off] : 0;
        __syncthreads();
        if (tid < 256) inc[tid] += v;
        __syncthreads();
    }
    if (tid < E) group_offset[tid] = inc[tid] - cnt[tid];
    if (tid == 0) {
        group_offset[E] = inc[255];
        if (include_shared) group_offset[E + 1] = inc[255] + (int32_t)T;
    }
    for (int j = tid; j < n; j += 1024) {
        const int t = j / K;
        const int ex = idx[j];
        if (ex < 0 || ex >= E) continue;
        const int c = t / CHUNK, tl = t % CHUNK;
        const uint64_t below = (tl == 0) ? 0ull : (m[c][ex] & ((1ull << tl) - 1ull));
        const int32_t row = inc[ex] - cnt[ex] + pre[c][ex] + __popcll(below);
        row_token[row] = t;
        slot_row[j] = row;
    }
    if (include_shared)
        for (int t = tid; t < (int)T; t += 1024) row_token[(int64_t)T * K + t] = t;
}

typedef uint32_t perm_v4u __attribute__((ext_vector_type(4)));

// One wave per 64 16-byte words of one output row (grid.x: column blocks,
// grid.y: rows, strided).  The output is written once and not re-read here,
// so its stores are non-temporal; the source rows are read K times each and
// keep ordinary loads.  Measured on gfx950 (T = 8192, d = 7168 bf16, K = 8):
// 0.246 ms against 0.278 ms for one 256-thread block per row with ordinary
// stores.
constexpr int PERMUTE_THREADS = 64;
__global__ __launch_bounds__(PERMUTE_THREADS) void permute_rows_kernel(const perm_v4u* __restrict__ x,
                                                                      const int32_t* __restrict__ row_token,
                                                                      int64_t rows, int row_vecs,
                                                                      perm_v4u* __restrict__ out) {
    const int v = blockIdx.x * PERMUTE_THREADS + threadIdx.x;
    if (v >= row_vecs) return;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const int64_t src = row_token[r];
        __builtin_nontemporal_store(x[src * row_vecs + v], out + r * row_vecs + v);
    }
}

// Invariant checks of a dispatch result (the debug status word).  The first
// kernel (one block) overwrites *status with the count/offset checks; the
// second ORs in the per-assignment checks.  Every index is range-checked
// before it is used, so a corrupted result is reported, never dereferenced.
__global__ __launch_bounds__(256) void dispatch_check_counts_kernel(const int32_t* __restrict__ count,
                                                                    const int32_t* __restrict__ go, int64_t T,
                                                                    int K, int E, int include_shared,
                                                                    uint32_t* __restrict__ status) {
    __shared__ uint32_t bits;
    __shared__ unsigned long long total;
    if (threadIdx.x == 0) { bits = 0; total = 0; }
    __syncthreads();
    uint32_t b = 0;
    long long sum = 0;
    for (int e = threadIdx.x; e < E; e += 256) {
        const int32_t c = count[e];
        if (c < 0) b |= MOE_CHECK_NEGATIVE_COUNT;
        sum += c;
        if (go[e + 1] < go[e]) b |= MOE_CHECK_OFFSETS_NOT_MONOTONE;
        if ((int64_t)go[e + 1] - go[e] != c) b |= MOE_CHECK_COUNT_NE_OFFSETS;
    }
    if (threadIdx.x == 0) {
        if (go[0] != 0) b |= MOE_CHECK_FIRST_OFFSET;
        if ((int64_t)go[E] != T * K) b |= MOE_CHECK_ROUTED_TOTAL;
        if (include_shared && (int64_t)go[E + 1] - go[E] != T) b |= MOE_CHECK_SHARED_GROUP;
        if (include_shared && go[E + 1] < go[E]) b |= MOE_CHECK_OFFSETS_NOT_MONOTONE;
    }
    atomicOr(&bits, b);
    atomicAdd(&total, (unsigned long long)sum);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = bits;
        if ((long long)total != T * K) r |= MOE_CHECK_COUNT_SUM;
        *status = r;
    }
}

__global__ __launch_bounds__(256) void dispatch_check_rows_kernel(const int32_t* __restrict__ idx,
                                                                  const int32_t* __restrict__ go,
                                                                  const int32_t* __restrict__ row_token,
                                                                  const int32_t* __restrict__ slot_row,
                                                                  int64_t T, int K, int E, int include_shared,
                                                                  uint32_t* __restrict__ status) {
    const int64_t R = T * K + (include_shared ? T : 0);
    uint32_t b = 0;
    for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < T * K; j += (int64_t)gridDim.x * 256) {
        const int64_t t = j / K;
        const int ex = idx[j];
        const int32_t r = slot_row[j];
        if (ex < 0 || ex >= E || r < 0 || r >= R) { b |= MOE_CHECK_SLOT_ROW; continue; }
        if (r < go[ex] || r >= go[ex + 1] || row_token[r] != t) b |= MOE_CHECK_SLOT_ROW;
    }
    if (include_shared)
        for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < T; t += (int64_t)gridDim.x * 256)
            if (row_token[T * K + t] != t) b |= MOE_CHECK_SHARED_ROWS;
    if (b) atomicOr(status, b);
}

}  // namespace

hipError_t launch_dispatch_check(const int32_t* count, const int32_t* group_offset, const int32_t* idx,
                                 const int32_t* row_token, const int32_t* slot_row, int64_t T, int K, int E,
                                 int include_shared, uint32_t* status, hipStream_t st) {
    hipLaunchKernelGGL(dispatch_check_counts_kernel, dim3(1), dim3(256), 0, st, count, group_offset, T, K, E,
                       include_shared, status);
    if (idx && row_token && slot_row && T > 0) {
        const int64_t blocks = (T * K + 255) / 256;
        hipLaunchKernelGGL(dispatch_check_rows_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                           st, idx, group_offset, row_token, slot_row, T, K, E, include_shared, status);
    }
    return hipGetLastError();
}

size_t dispatch_ws_bytes(int64_t T, int E) {
    const int64_t nchunk = (T + CHUNK - 1) / CHUNK;
    return align256(sizeof(uint64_t) * nchunk * E) + align256(sizeof(int32_t) * nchunk * E) +
           align256(sizeof(int32_t) * nchunk * E);
}

hipError_t launch_dispatch(const int32_t* idx, int64_t T, int K, int E, int include_shared,
                           int32_t* count, int32_t* group_offset, int32_t* row_token,
                           int32_t* slot_row, void* ws, hipStream_t st) {
    if (T <= SMALL_T) {
        hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), 0, st, idx, T, K, E, include_shared,
                           count, group_offset, row_token, slot_row);
        return hipGetLastError();
    }
    const int64_t nchunk = (T + CHUNK - 1) / CHUNK;
    DispatchWs w = carve(ws, nchunk, E);
    hipLaunchKernelGGL(dispatch_hist_kernel, dim3((unsigned)nchunk), dim3(256), 0, st, idx, T, K,
                       E, w);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(256 * SCAN_PARTS), 0, st, nchunk, T, K, E,
                       include_shared, w, count, group_offset);
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3((unsigned)nchunk), dim3(256), 0, st, idx, T,
                       K, E, include_shared, w, group_offset, row_token, slot_row);
    return hipGetLastError();
}

hipError_t launch_permute_rows(const void* x, size_t elem_bytes, const int32_t* row_token,
                               int64_t rows, int d, void* out, hipStream_t st) {
    const int row_vecs = (int)(d * elem_bytes / 16);
    const dim3 grid((unsigned)((row_vecs + PERMUTE_THREADS - 1) / PERMUTE_THREADS),
                    (unsigned)(rows < 65535 ? rows : 65535));
    hipLaunchKernelGGL(permute_rows_kernel, grid, dim3(PERMUTE_THREADS), 0, st,
                       static_cast<const perm_v4u*>(x), row_token, rows, row_vecs,
                       static_cast<perm_v4u*>(out));
    return hipGetLastError();
}

}  // namespace moe
