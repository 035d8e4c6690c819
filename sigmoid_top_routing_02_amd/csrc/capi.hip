// C ABI of the library (declared in include/moe_fp8.h).  Every entry point
// checks its arguments on the host, then enqueues kernels on the caller's
// stream.  No allocation, no synchronisation, no global state except the
// thread-local text of the last error.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/moe_fp8.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MOE_OK;
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                               \
    do {                                                                             \
        if (!(p)) return fail(MOE_ERR_NULLPTR, "%s: %s is NULL", __func__, #p);      \
        if (!aligned16(p)) return fail(MOE_ERR_ALIGN, "%s: %s is not 16-byte aligned", __func__, #p); \
    } while (0)

#define REQUIRE(cond, status, ...)                      \
    do {                                                \
        if (!(cond)) return fail(status, __VA_ARGS__);  \
    } while (0)

inline hipStream_t S(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char* moe_status_string(int s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULLPTR: return "null pointer";
        case MOE_ERR_SHAPE: return "invalid shape";
        case MOE_ERR_UNSUPPORTED: return "unsupported size";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_ALIGN: return "misaligned pointer";
        case MOE_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_err; }

int moe_version(void) { return 10000; }

int moe_router_topk(const void* u_bf16, const void* centroids_bf16, const float* bias, int64_t T,
                    int d, int E, int K, float* scores, int32_t* topk_idx, float* topk_gate,
                    moe_stream_t stream) {
    return moe_router_topk_grouped(u_bf16, centroids_bf16, bias, T, d, E, K, 1, 1, scores,
                                   topk_idx, topk_gate, stream);
}

int moe_router_topk_grouped(const void* u_bf16, const void* centroids_bf16, const float* bias,
                            int64_t T, int d, int E, int K, int n_groups, int topk_groups,
                            float* scores, int32_t* topk_idx, float* topk_gate,
                            moe_stream_t stream) {
    REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_router_topk: T < 0");
    REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "moe_router_topk: d=%d not a positive multiple of 128", d);
    REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "moe_router_topk: E=%d outside [1, 256]", E);
    REQUIRE(K >= 1 && K <= E && K <= 16, MOE_ERR_UNSUPPORTED, "moe_router_topk: K=%d outside [1, min(E,16)]", K);
    REQUIRE(n_groups >= 1 && n_groups <= 64 && E % n_groups == 0, MOE_ERR_SHAPE,
            "moe_router_topk: n_groups=%d must divide E=%d and lie in [1, 64]", n_groups, E);
    REQUIRE(topk_groups >= 1 && topk_groups <= n_groups, MOE_ERR_SHAPE,
            "moe_router_topk: topk_groups=%d outside [1, n_groups=%d]", topk_groups, n_groups);
    REQUIRE(K <= topk_groups * (E / n_groups), MOE_ERR_SHAPE,
            "moe_router_topk: K=%d exceeds the %d experts of %d kept groups", K,
            topk_groups * (E / n_groups), topk_groups);
    if (T == 0) return MOE_OK;
    REQUIRE_PTR(u_bf16);
    REQUIRE_PTR(centroids_bf16);
    REQUIRE_PTR(bias);
    REQUIRE_PTR(scores);
    REQUIRE_PTR(topk_idx);
    REQUIRE_PTR(topk_gate);
    hipError_t e = moe::launch_router_scores(static_cast<const uint16_t*>(u_bf16),
                                             static_cast<const uint16_t*>(centroids_bf16), T, d, E,
                                             scores, S(stream));
    if (e != hipSuccess) return hip_status(e, "router scores launch");
    e = moe::launch_router_topk(scores, bias, T, E, K, n_groups, topk_groups, topk_idx, topk_gate,
                                S(stream));
    return hip_status(e, "router top-k launch");
}

size_t moe_seq_balance_loss_workspace_bytes(int64_t T, int seq_len) {
    // 0 outside what moe_seq_balance_loss accepts (also keeps the sizes from overflowing)
    if (T <= 0 || seq_len < 1 || T % seq_len || T / seq_len > 65535) return 0;
    return moe::seq_balance_ws_bytes(T / seq_len, seq_len);
}

int moe_seq_balance_loss(const float* scores, const int32_t* topk_idx, int64_t T, int E, int K,
                         int seq_len, float alpha, float* loss, void* ws, size_t ws_bytes,
                         moe_stream_t stream) {
    REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_seq_balance_loss: T < 0");
    REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "moe_seq_balance_loss: E=%d outside [1, 256]", E);
    REQUIRE(K >= 1 && K <= E && K <= 16, MOE_ERR_UNSUPPORTED, "moe_seq_balance_loss: K=%d outside [1, min(E,16)]", K);
    REQUIRE(seq_len >= 1 && T % seq_len == 0, MOE_ERR_SHAPE,
            "moe_seq_balance_loss: T=%lld is not a multiple of seq_len=%d", (long long)T, seq_len);
    REQUIRE(T / seq_len <= 65535 && (T / seq_len) * ((seq_len + 63) / 64) <= 0x7FFFFFFF, MOE_ERR_UNSUPPORTED,
            "moe_seq_balance_loss: too many sequences");
    if (T == 0) return MOE_OK;
    REQUIRE(ws_bytes >= moe_seq_balance_loss_workspace_bytes(T, seq_len), MOE_ERR_WORKSPACE,
            "moe_seq_balance_loss: workspace of %zu bytes, %zu needed", ws_bytes,
            moe_seq_balance_loss_workspace_bytes(T, seq_len));
    REQUIRE_PTR(scores);
    REQUIRE_PTR(topk_idx);
    REQUIRE_PTR(loss);
    REQUIRE_PTR(ws);
    return hip_status(moe::launch_seq_balance_loss(scores, topk_idx, T / seq_len, E, K, seq_len, alpha,
                                                   loss, ws, S(stream)),
                      "balance loss launch");
}

size_t moe_dispatch_workspace_bytes(int64_t T, int E) {
    if (T <= 0 || E <= 0 || E > 256 || T >= ((int64_t)1 << 31)) return 0;   // outside moe_dispatch's limits
    return moe::dispatch_ws_bytes(T, E);
}

int moe_dispatch(const int32_t* topk_idx, int64_t T, int K, int E, int include_shared,
                 int32_t* expert_count, int32_t* group_offset, int32_t* row_token,
                 int32_t* slot_row, void* ws, size_t ws_bytes, moe_stream_t stream) {
    REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_dispatch: T < 0");
    REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "moe_dispatch: E=%d outside [1, 256]", E);
    REQUIRE(K >= 1 && K <= E && K <= 16, MOE_ERR_UNSUPPORTED, "moe_dispatch: K=%d outside [1, min(E,16)]", K);
    REQUIRE(include_shared == 0 || include_shared == 1, MOE_ERR_SHAPE, "moe_dispatch: include_shared must be 0 or 1");
    REQUIRE(T * (K + 1) < (int64_t)1 << 31, MOE_ERR_UNSUPPORTED, "moe_dispatch: T*(K+1) exceeds int32 rows");
    if (T == 0) return MOE_OK;
    REQUIRE_PTR(topk_idx);
    REQUIRE_PTR(expert_count);
    REQUIRE_PTR(group_offset);
    REQUIRE_PTR(row_token);
    REQUIRE_PTR(slot_row);
    REQUIRE_PTR(ws);
    REQUIRE(ws_bytes >= moe::dispatch_ws_bytes(T, E), MOE_ERR_WORKSPACE,
            "moe_dispatch: workspace %zu < %zu bytes", ws_bytes, moe::dispatch_ws_bytes(T, E));
    return hip_status(moe::launch_dispatch(topk_idx, T, K, E, include_shared, expert_count,
                                           group_offset, row_token, slot_row, ws, S(stream)),
                      "dispatch launch");
}

int moe_dispatch_check(const int32_t* expert_count, const int32_t* group_offset, const int32_t* topk_idx,
                       const int32_t* row_token, const int32_t* slot_row, int64_t T, int K, int E,
                       int include_shared, uint32_t* status, moe_stream_t stream) {
    REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_dispatch_check: T < 0");
    REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "moe_dispatch_check: E=%d outside [1, 256]", E);
    REQUIRE(K >= 1 && K <= E && K <= 16, MOE_ERR_UNSUPPORTED, "moe_dispatch_check: K=%d outside [1, min(E,16)]", K);
    REQUIRE(include_shared == 0 || include_shared == 1, MOE_ERR_SHAPE,
            "moe_dispatch_check: include_shared must be 0 or 1");
    REQUIRE(T * (K + 1) < (int64_t)1 << 31, MOE_ERR_UNSUPPORTED, "moe_dispatch_check: T*(K+1) exceeds int32 rows");
    REQUIRE_PTR(expert_count);
    REQUIRE_PTR(group_offset);
    REQUIRE_PTR(status);
    REQUIRE((topk_idx == nullptr) == (row_token == nullptr) && (row_token == nullptr) == (slot_row == nullptr),
            MOE_ERR_NULLPTR, "moe_dispatch_check: topk_idx, row_token and slot_row must all be given or all NULL");
    return hip_status(moe::launch_dispatch_check(expert_count, group_offset, topk_idx, row_token, slot_row, T, K, E,
                                                 include_shared, status, S(stream)),
                      "dispatch check launch");
}

int moe_permute_rows(const void* x, int dt, const int32_t* row_token, int64_t rows, int d,
                     void* out, moe_stream_t stream) {
    REQUIRE(rows >= 0, MOE_ERR_SHAPE, "moe_permute_rows: rows < 0");
    REQUIRE(dt == MOE_BF16 || dt == MOE_F32, MOE_ERR_UNSUPPORTED, "moe_permute_rows: dtype %d", dt);
    const size_t eb = dt == MOE_F32 ? 4 : 2;
    REQUIRE(d > 0 && (d * eb) % 16 == 0, MOE_ERR_SHAPE, "moe_permute_rows: row of %d elements is not a multiple of 16 bytes", d);
    if (rows == 0) return MOE_OK;
    REQUIRE_PTR(x);
    REQUIRE_PTR(row_token);
    REQUIRE_PTR(out);
    return hip_status(moe::launch_permute_rows(x, eb, row_token, rows, d, out, S(stream)),
                      "permute launch");
}

int fp8_quant_1x128(const void* x, int in_dt, int64_t rows, int cols, uint8_t* q, float* scale,
                    moe_stream_t stream) {
    REQUIRE(rows >= 0, MOE_ERR_SHAPE, "fp8_quant_1x128: rows < 0");
    REQUIRE(cols > 0 && cols % 128 == 0, MOE_ERR_SHAPE, "fp8_quant_1x128: cols=%d not a positive multiple of 128", cols);
    REQUIRE(in_dt == MOE_BF16 || in_dt == MOE_F32, MOE_ERR_UNSUPPORTED, "fp8_quant_1x128: dtype %d", in_dt);
    if (rows == 0) return MOE_OK;
    REQUIRE_PTR(x);
    REQUIRE_PTR(q);
    REQUIRE_PTR(scale);
    return hip_status(moe::launch_quant_1x128(x, in_dt == MOE_F32, rows, cols, q, scale, S(stream)),
                      "quant 1x128 launch");
}

int fp8_quant_128x128(const float* w, int64_t rows, int cols, uint8_t* q, float* scale,
                      moe_stream_t stream) {
    REQUIRE(rows >= 0 && rows % 128 == 0, MOE_ERR_SHAPE, "fp8_quant_128x128: rows=%lld not a multiple of 128", (long long)rows);
    REQUIRE(cols > 0 && cols % 128 == 0, MOE_ERR_SHAPE, "fp8_quant_128x128: cols=%d not a positive multiple of 128", cols);
    REQUIRE(rows / 128 <= 65535, MOE_ERR_UNSUPPORTED, "fp8_quant_128x128: too many rows");
    if (rows == 0) return MOE_OK;
    REQUIRE_PTR(w);
    REQUIRE_PTR(q);
    REQUIRE_PTR(scale);
    return hip_status(moe::launch_quant_128x128(w, rows, cols, q, scale, 1, 0, S(stream)),
                      "quant 128x128 launch");
}

size_t moe_gemm_workspace_bytes(int G, int64_t M_total, int N, int K) {
    // 0 outside the grouped GEMM's limits (which also keep the sizes below from overflowing)
    return (G > 0 && G <= 65535 && M_total >= 0 && M_total < ((int64_t)1 << 31) && N > 0 && K > 0 && K <= 16384)
               ? moe::gemm_ws_bytes(G, M_total, N, K) : 0;
}

namespace {
// Argument checks shared by grouped_gemm_fp8_blockscaled and its allocation-free variant.
int gemm_check_args(const uint8_t* a_q, const float* a_scale, const int32_t* a_row_index,
                    const int32_t* group_offset, int G, int64_t M_total, const uint8_t* b_q,
                    const float* b_scale, int N, int K, int epi, float* out, uint8_t* out_q,
                    float* out_scale) {
    REQUIRE(G >= 1 && G <= 65535, MOE_ERR_UNSUPPORTED, "grouped_gemm: G=%d outside [1, 65535]", G);
    REQUIRE(M_total >= 0 && M_total < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED, "grouped_gemm: M_total out of range");
    REQUIRE(K > 0 && K % 128 == 0, MOE_ERR_SHAPE, "grouped_gemm: K=%d not a positive multiple of 128", K);
    REQUIRE(K <= 16384, MOE_ERR_UNSUPPORTED, "grouped_gemm: K=%d above 16384 (128 slices)", K);
    REQUIRE(a_row_index || M_total * K < ((int64_t)1 << 32), MOE_ERR_UNSUPPORTED,
            "grouped_gemm: A of M_total=%lld rows exceeds 4 GiB (32-bit byte offsets)", (long long)M_total);
    REQUIRE(epi >= MOE_EPI_STORE_F32 && epi <= MOE_EPI_SWIGLU_QUANT_Z, MOE_ERR_UNSUPPORTED, "grouped_gemm: epilogue %d", epi);
    if (epi == MOE_EPI_STORE_F32)
        REQUIRE(N > 0 && N % 128 == 0, MOE_ERR_SHAPE, "grouped_gemm: N=%d not a positive multiple of 128", N);
    else
        REQUIRE(N > 0 && N % 256 == 0, MOE_ERR_SHAPE, "grouped_gemm: SwiGLU needs N=%d a multiple of 256", N);
    REQUIRE(((M_total + 31) / 32 + G) * ((N + 255) / 256) < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED,
            "grouped_gemm: too many tiles");
    REQUIRE((int64_t)N * K < ((int64_t)1 << 32), MOE_ERR_UNSUPPORTED, "grouped_gemm: one group's B exceeds 4 GiB");
    REQUIRE((M_total + 128) * (K / 128) * 4 < ((int64_t)1 << 32), MOE_ERR_UNSUPPORTED,
            "grouped_gemm: the A scales of M_total=%lld rows exceed 4 GiB", (long long)M_total);
    if (M_total == 0) return MOE_OK;
    REQUIRE_PTR(a_q);
    REQUIRE_PTR(a_scale);
    REQUIRE_PTR(group_offset);
    REQUIRE_PTR(b_q);
    REQUIRE_PTR(b_scale);
    if (a_row_index) REQUIRE_PTR(a_row_index);
    if (epi == MOE_EPI_SWIGLU_QUANT) {
        REQUIRE_PTR(out_q);
        REQUIRE_PTR(out_scale);
        if (out) REQUIRE_PTR(out);
    } else if (epi == MOE_EPI_SWIGLU_QUANT_Z) {
        REQUIRE_PTR(out_q);
        REQUIRE_PTR(out_scale);
        REQUIRE_PTR(out);
    } else {
        REQUIRE_PTR(out);
    }
    return MOE_OK;
}
}  // namespace

int grouped_gemm_fp8_blockscaled(const uint8_t* a_q, const float* a_scale,
                                 const int32_t* a_row_index, const int32_t* group_offset, int G,
                                 int64_t M_total, const uint8_t* b_q, const float* b_scale, int N,
                                 int K, int epi, float* out, uint8_t* out_q, float* out_scale,
                                 void* ws, size_t ws_bytes, moe_stream_t stream) {
    const int st = gemm_check_args(a_q, a_scale, a_row_index, group_offset, G, M_total, b_q, b_scale, N, K, epi,
                                   out, out_q, out_scale);
    if (st != MOE_OK || M_total == 0) return st;
    REQUIRE_PTR(ws);
    REQUIRE(ws_bytes >= moe::gemm_ws_bytes(G, M_total, N, K), MOE_ERR_WORKSPACE,
            "grouped_gemm: workspace %zu < %zu bytes", ws_bytes, moe::gemm_ws_bytes(G, M_total, N, K));
    return hip_status(moe::launch_grouped_gemm(a_q, a_scale, a_row_index, group_offset, G, M_total,
                                               b_q, b_scale, N, K, epi, out, out_q, out_scale, ws,
                                               S(stream)),
                      "grouped gemm launch");
}

int grouped_gemm_fp8_blockscaled_noalloc(const uint8_t* a_q, const float* a_scale,
                                         const int32_t* a_row_index, const int32_t* group_offset, int G,
                                         int64_t M_total, const uint8_t* b_q, const float* b_scale, int N,
                                         int K, int epi, float* out, uint8_t* out_q, float* out_scale,
                                         moe_stream_t stream) {
    const int st = gemm_check_args(a_q, a_scale, a_row_index, group_offset, G, M_total, b_q, b_scale, N, K, epi,
                                   out, out_q, out_scale);
    if (st != MOE_OK || M_total == 0) return st;
    const size_t need = moe::gemm_ws_bytes(G, M_total, N, K);
    REQUIRE(need <= (size_t)MOE_GEMM_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
            "grouped_gemm_noalloc: needs %zu bytes of scratch, above the library's static %zu-byte array "
            "(use grouped_gemm_fp8_blockscaled with a workspace)", need, (size_t)MOE_GEMM_SCRATCH_BYTES);
    void* scratch = nullptr;
    const hipError_t e = moe::gemm_static_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e, "grouped_gemm_noalloc: static scratch address");
    return hip_status(moe::launch_grouped_gemm(a_q, a_scale, a_row_index, group_offset, G, M_total,
                                               b_q, b_scale, N, K, epi, out, out_q, out_scale, scratch,
                                               S(stream)),
                      "grouped gemm launch");
}

int moe_fp8_mfma_accumulation_probe(const uint8_t* a_q, const uint8_t* b_q, int M, int N, int K,
                                    int chained, float* out, moe_stream_t stream) {
    REQUIRE(M >= 0 && M % 16 == 0 && M / 16 <= 65535, MOE_ERR_SHAPE,
            "moe_fp8_mfma_accumulation_probe: M=%d not a multiple of 16 in [0, 1048560]", M);
    REQUIRE(N >= 0 && N % 16 == 0, MOE_ERR_SHAPE, "moe_fp8_mfma_accumulation_probe: N=%d not a multiple of 16", N);
    REQUIRE(K > 0 && K % 128 == 0, MOE_ERR_SHAPE, "moe_fp8_mfma_accumulation_probe: K=%d not a positive multiple of 128", K);
    REQUIRE(chained == 0 || chained == 1, MOE_ERR_UNSUPPORTED, "moe_fp8_mfma_accumulation_probe: chained=%d", chained);
    if (M == 0 || N == 0) return MOE_OK;
    REQUIRE_PTR(a_q);
    REQUIRE_PTR(b_q);
    REQUIRE_PTR(out);
    return hip_status(moe::launch_accum_probe(a_q, b_q, M, N, K, chained, out, S(stream)),
                      "accumulation probe launch");
}

int moe_combine(const void* u_bf16, const void* y, int y_dt, int64_t shared_row0,
                const float* topk_gate, const int32_t* slot_row, int64_t T, int K, int d,
                float* out, moe_stream_t stream) {
    REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_combine: T < 0");
    REQUIRE(K >= 1 && K <= 16, MOE_ERR_UNSUPPORTED, "moe_combine: K=%d outside [1, 16]", K);
    REQUIRE(d > 0 && d % 8 == 0, MOE_ERR_SHAPE, "moe_combine: d=%d not a positive multiple of 8", d);
    REQUIRE(y_dt == MOE_BF16 || y_dt == MOE_F32, MOE_ERR_UNSUPPORTED, "moe_combine: dtype %d", y_dt);
    if (T == 0) return MOE_OK;
    REQUIRE_PTR(u_bf16);
    REQUIRE_PTR(y);
    REQUIRE_PTR(topk_gate);
    REQUIRE_PTR(slot_row);
    REQUIRE_PTR(out);
    return hip_status(moe::launch_combine(static_cast<const uint16_t*>(u_bf16), y, y_dt == MOE_F32,
                                          shared_row0, topk_gate, slot_row, T, K, d, out,
                                          S(stream)),
                      "combine launch");
}

int moe_bias_update(float* bias, const int32_t* expert_count, int E, int64_t total_assignments,
                    float gamma, moe_stream_t stream) {
    REQUIRE(E >= 1 && E <= 65536, MOE_ERR_UNSUPPORTED, "moe_bias_update: E=%d", E);
    REQUIRE(total_assignments >= 0, MOE_ERR_SHAPE, "moe_bias_update: total < 0");
    REQUIRE_PTR(bias);
    REQUIRE_PTR(expert_count);
    return hip_status(moe::launch_bias_update(bias, expert_count, E, total_assignments, gamma,
                                              S(stream)),
                      "bias update launch");
}

// ---------------------------------------------------------------- packed weights
namespace {
struct Packed {
    uint8_t* w13q;
    uint8_t* w2q;
    float* w13s;
    float* w2s;
};
Packed packed_layout(void* base, int G, int d, int I) {
    char* p = static_cast<char*>(base);
    Packed k;
    k.w13q = reinterpret_cast<uint8_t*>(p);
    p += al256((size_t)G * 2 * I * d);
    k.w2q = reinterpret_cast<uint8_t*>(p);
    p += al256((size_t)G * d * I);
    k.w13s = reinterpret_cast<float*>(p);
    p += al256((size_t)G * (2 * I / 128) * (d / 128) * sizeof(float));
    k.w2s = reinterpret_cast<float*>(p);
    return k;
}
}  // namespace

size_t moe_packed_weight_bytes(int n_groups, int d, int I) {
    // 0 for sizes no call takes (keeps the products below from wrapping)
    if (n_groups <= 0 || n_groups > 65537 || d <= 0 || I <= 0 || d > 65536 || I > 65536) return 0;
    const size_t G = (size_t)n_groups;
    return al256(G * 2 * I * d) + al256(G * d * I) +
           al256(G * (2 * I / 128) * (d / 128) * sizeof(float)) +
           al256(G * (d / 128) * (I / 128) * sizeof(float));
}

int moe_prepare_expert_weights(const float* w1, const float* w3, const float* w2, int expert_index,
                               int n_groups, int d, int I, void* packed, moe_stream_t stream) {
    REQUIRE(d > 0 && d % 128 == 0 && I > 0 && I % 128 == 0, MOE_ERR_SHAPE,
            "moe_prepare_expert_weights: d=%d, I=%d must be positive multiples of 128", d, I);
    REQUIRE(n_groups >= 1 && expert_index >= 0 && expert_index < n_groups, MOE_ERR_SHAPE,
            "moe_prepare_expert_weights: expert %d of %d", expert_index, n_groups);
    REQUIRE(I / 128 <= 32767 && d / 128 <= 65535, MOE_ERR_UNSUPPORTED, "moe_prepare_expert_weights: too large");
    REQUIRE_PTR(w1);
    REQUIRE_PTR(w3);
    REQUIRE_PTR(w2);
    REQUIRE_PTR(packed);
    Packed pk = packed_layout(packed, n_groups, d, I);
    const size_t g = (size_t)expert_index;
    uint8_t* q13 = pk.w13q + g * 2 * I * d;
    float* s13 = pk.w13s + g * (2 * I / 128) * (d / 128);
    uint8_t* q2 = pk.w2q + g * d * I;
    float* s2 = pk.w2s + g * (d / 128) * (I / 128);
    hipError_t e = moe::launch_quant_128x128(w1, I, d, q13, s13, 2, 0, S(stream));
    if (e == hipSuccess) e = moe::launch_quant_128x128(w3, I, d, q13, s13, 2, 1, S(stream));
    if (e == hipSuccess) e = moe::launch_quant_128x128(w2, d, I, q2, s2, 1, 0, S(stream));
    return hip_status(e, "weight quantisation launch");
}

int moe_prepare_backward_weights(const void* packed, int n_groups, int d, int I, void* packed_t,
                                 moe_stream_t stream) {
    REQUIRE(d > 0 && d % 128 == 0 && I > 0 && I % 128 == 0, MOE_ERR_SHAPE,
            "moe_prepare_backward_weights: d=%d, I=%d must be positive multiples of 128", d, I);
    REQUIRE(n_groups >= 1 && n_groups <= 65535, MOE_ERR_UNSUPPORTED, "moe_prepare_backward_weights: %d groups",
            n_groups);
    REQUIRE_PTR(packed);
    REQUIRE_PTR(packed_t);
    REQUIRE(packed != packed_t, MOE_ERR_SHAPE, "moe_prepare_backward_weights: packed_t must not be packed");
    Packed in = packed_layout(const_cast<void*>(packed), n_groups, d, I);
    Packed out = packed_layout(packed_t, n_groups, d, I);
    hipError_t e = moe::launch_transpose_blocks(in.w13q, in.w13s, n_groups, 2 * I, d, out.w13q, out.w13s, S(stream));
    if (e == hipSuccess) e = moe::launch_transpose_blocks(in.w2q, in.w2s, n_groups, d, I, out.w2q, out.w2s, S(stream));
    return hip_status(e, "weight transposition launch");
}

// ---------------------------------------------------------------- backward (input gradient)
int moe_gate_backward(const float* dh, const float* y, int64_t shared_row0, const float* topk_gate,
                      const int32_t* slot_row, const float* scores, const int32_t* topk_idx, int64_t T,
                      int K, int d, int E, uint8_t* dy_q, float* dy_scale, float* dlogit, float* row_dlogit,
                      moe_stream_t stream) {
    REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_gate_backward: T < 0");
    REQUIRE(K >= 1 && K <= 16 && K <= E, MOE_ERR_UNSUPPORTED, "moe_gate_backward: K=%d outside [1, min(E,16)]", K);
    REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "moe_gate_backward: E=%d outside [1, 256]", E);
    REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "moe_gate_backward: d=%d not a positive multiple of 128", d);
    if (T == 0) return MOE_OK;
    REQUIRE_PTR(dh);
    REQUIRE_PTR(y);
    REQUIRE_PTR(topk_gate);
    REQUIRE_PTR(slot_row);
    REQUIRE_PTR(scores);
    REQUIRE_PTR(topk_idx);
    REQUIRE_PTR(dy_q);
    REQUIRE_PTR(dy_scale);
    REQUIRE_PTR(dlogit);
    REQUIRE_PTR(row_dlogit);
    return hip_status(moe::launch_gate_backward(dh, y, shared_row0, topk_gate, slot_row, scores, topk_idx, T, K,
                                                d, E, dy_q, dy_scale, dlogit, row_dlogit, S(stream)),
                      "gate backward launch");
}

int moe_swiglu_backward(const float* z, const float* dh_row, int64_t R, int I, uint8_t* dz_q, float* dz_scale,
                        moe_stream_t stream) {
    REQUIRE(R >= 0, MOE_ERR_SHAPE, "moe_swiglu_backward: R < 0");
    REQUIRE(I > 0 && I % 128 == 0, MOE_ERR_SHAPE, "moe_swiglu_backward: I=%d not a positive multiple of 128", I);
    if (R == 0) return MOE_OK;
    REQUIRE_PTR(z);
    REQUIRE_PTR(dh_row);
    REQUIRE_PTR(dz_q);
    REQUIRE_PTR(dz_scale);
    return hip_status(moe::launch_swiglu_backward(z, dh_row, R, I, dz_q, dz_scale, S(stream)),
                      "SwiGLU backward launch");
}

int moe_router_backward(const float* dh, const float* dx, int64_t shared_row0, const int32_t* slot_row,
                        const float* dlogit, const int32_t* topk_idx, const void* centroids_bf16,
                        const void* u_bf16, const float* row_dlogit, const int32_t* row_token,
                        const int32_t* group_offset, int64_t T, int K, int d, int E, float* du, float* de,
                        moe_stream_t stream) {
    REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_router_backward: T < 0");
    REQUIRE(K >= 1 && K <= 16 && K <= E, MOE_ERR_UNSUPPORTED, "moe_router_backward: K=%d outside [1, min(E,16)]", K);
    REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "moe_router_backward: E=%d outside [1, 256]", E);
    REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "moe_router_backward: d=%d not a positive multiple of 128", d);
    REQUIRE_PTR(de);
    REQUIRE_PTR(group_offset);
    if (T > 0) {
        REQUIRE_PTR(dh);
        REQUIRE_PTR(dx);
        REQUIRE_PTR(slot_row);
        REQUIRE_PTR(dlogit);
        REQUIRE_PTR(topk_idx);
        REQUIRE_PTR(centroids_bf16);
        REQUIRE_PTR(u_bf16);
        REQUIRE_PTR(row_dlogit);
        REQUIRE_PTR(row_token);
        REQUIRE_PTR(du);
        hipError_t e = moe::launch_du(dh, dx, shared_row0, slot_row, dlogit, topk_idx,
                                      static_cast<const uint16_t*>(centroids_bf16), T, K, d, du, S(stream));
        if (e != hipSuccess) return hip_status(e, "du launch");
    }
    return hip_status(moe::launch_de(row_dlogit, row_token, group_offset, static_cast<const uint16_t*>(u_bf16), d,
                                     E, de, S(stream)),
                      "de launch");
}

int moe_wgrad_block_starts(const int32_t* group_offset, int G, int32_t* kb_start, moe_stream_t stream) {
    REQUIRE(G >= 1 && G <= 65535, MOE_ERR_UNSUPPORTED, "moe_wgrad_block_starts: G=%d outside [1, 65535]", G);
    REQUIRE_PTR(group_offset);
    REQUIRE_PTR(kb_start);
    return hip_status(moe::launch_wgrad_block_starts(group_offset, G, kb_start, S(stream)), "kb_start launch");
}

int moe_wgrad_operands(const float* dh, const float* topk_gate, const int32_t* slot_row, const int32_t* row_token,
                       const float* z, const float* dh_row, const void* u_bf16, const int32_t* group_offset,
                       const int32_t* kb_start, int G, int n_kb, int64_t T, int K, int d, int I,
                       int64_t shared_row0, uint8_t* dyT_q, float* dyT_scale, uint8_t* hT_q, float* hT_scale,
                       uint8_t* dzT_q, float* dzT_scale, uint8_t* xT_q, float* xT_scale, moe_stream_t stream) {
    REQUIRE(G >= 1 && G <= 65535, MOE_ERR_UNSUPPORTED, "moe_wgrad_operands: G=%d outside [1, 65535]", G);
    REQUIRE(n_kb >= 0 && n_kb <= 65535, MOE_ERR_UNSUPPORTED, "moe_wgrad_operands: n_kb=%d outside [0, 65535]", n_kb);
    REQUIRE(K >= 1 && K <= 16, MOE_ERR_UNSUPPORTED, "moe_wgrad_operands: K=%d outside [1, 16]", K);
    REQUIRE(d > 0 && d % 128 == 0 && I > 0 && I % 128 == 0, MOE_ERR_SHAPE,
            "moe_wgrad_operands: d=%d, I=%d must be positive multiples of 128", d, I);
    REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_wgrad_operands: T < 0");
    if (n_kb == 0) return MOE_OK;
    REQUIRE_PTR(dh);
    REQUIRE_PTR(topk_gate);
    REQUIRE_PTR(slot_row);
    REQUIRE_PTR(row_token);
    REQUIRE_PTR(z);
    REQUIRE_PTR(dh_row);
    REQUIRE_PTR(u_bf16);
    REQUIRE_PTR(group_offset);
    REQUIRE_PTR(kb_start);
    REQUIRE_PTR(dyT_q);
    REQUIRE_PTR(dyT_scale);
    REQUIRE_PTR(hT_q);
    REQUIRE_PTR(hT_scale);
    REQUIRE_PTR(dzT_q);
    REQUIRE_PTR(dzT_scale);
    REQUIRE_PTR(xT_q);
    REQUIRE_PTR(xT_scale);
    return hip_status(moe::launch_wgrad_operands(dh, topk_gate, slot_row, row_token, z, dh_row,
                                                 static_cast<const uint16_t*>(u_bf16), shared_row0, K, d, I,
                                                 group_offset, kb_start, G, n_kb, dyT_q, dyT_scale, hT_q, hT_scale,
                                                 dzT_q, dzT_scale, xT_q, xT_scale, S(stream)),
                      "wgrad operand launch");
}

size_t moe_wgrad_workspace_bytes(int G, int d, int I) {
    if (G < 1 || G > 65535 || d <= 0 || I <= 0 || d > 65536 || I > 65536) return 0;   // no overflow below
    return moe::wgrad_ws_bytes(G, d, I);
}

int moe_wgrad(const int32_t* kb_start, int G, int n_kb, int d, int I, const uint8_t* dyT_q, const float* dyT_scale,
              const uint8_t* hT_q, const float* hT_scale, const uint8_t* dzT_q, const float* dzT_scale,
              const uint8_t* xT_q, const float* xT_scale, float* dw13, float* dw2, void* ws, size_t ws_bytes,
              moe_stream_t stream) {
    REQUIRE(G >= 1 && G <= 65535, MOE_ERR_UNSUPPORTED, "moe_wgrad: G=%d outside [1, 65535]", G);
    REQUIRE(d > 0 && d % 128 == 0 && I > 0 && I % 128 == 0, MOE_ERR_SHAPE,
            "moe_wgrad: d=%d, I=%d must be positive multiples of 128", d, I);
    REQUIRE(n_kb >= 0, MOE_ERR_SHAPE, "moe_wgrad: n_kb=%d < 0", n_kb);
    // one group's operands are addressed with 32-bit byte offsets
    REQUIRE((int64_t)n_kb * 128 * (d > 2 * I ? d : 2 * I) < ((int64_t)1 << 32), MOE_ERR_UNSUPPORTED,
            "moe_wgrad: %d row blocks of up to %d columns exceed 4 GiB", n_kb, d > 2 * I ? d : 2 * I);
    REQUIRE((int64_t)G * (d > 2 * I ? d : 2 * I) < ((int64_t)1 << 31), MOE_ERR_UNSUPPORTED,
            "moe_wgrad: G=%d groups of gradient rows exceed int32", G);
    REQUIRE_PTR(kb_start);
    REQUIRE_PTR(dw13);
    REQUIRE_PTR(dw2);
    REQUIRE_PTR(ws);
    REQUIRE(ws_bytes >= moe_wgrad_workspace_bytes(G, d, I), MOE_ERR_WORKSPACE, "moe_wgrad: workspace %zu < %zu bytes",
            ws_bytes, moe_wgrad_workspace_bytes(G, d, I));
    if (n_kb > 0) {
        REQUIRE_PTR(dyT_q);
        REQUIRE_PTR(dyT_scale);
        REQUIRE_PTR(hT_q);
        REQUIRE_PTR(hT_scale);
        REQUIRE_PTR(dzT_q);
        REQUIRE_PTR(dzT_scale);
        REQUIRE_PTR(xT_q);
        REQUIRE_PTR(xT_scale);
    }
    return hip_status(moe::launch_wgrad_gemms(kb_start, G, d, I, dyT_q, dyT_scale, hT_q, hT_scale, dzT_q,
                                              dzT_scale, xT_q, xT_scale, dw13, dw2, ws, S(stream)),
                      "wgrad GEMM launch");
}

// ---------------------------------------------------------------- whole layer
namespace {
struct LayerWs {
    float* scores;
    int32_t* idx;
    float* gate;
    int32_t* count;
    int32_t* go;
    int32_t* row_token;
    int32_t* slot_row;
    uint8_t* uq;
    float* us;
    uint8_t* hq;
    float* hs;
    float* y;
    void* dws;
    void* gws;
    size_t total;
};
LayerWs layer_ws(void* base, int64_t T, int d, int E, int K, int I) {
    char* p = static_cast<char*>(base);
    const size_t R = (size_t)T * (K + 1);
    LayerWs w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* q = p ? p + off : nullptr;
        off += al256(bytes);
        return q;
    };
    w.scores = reinterpret_cast<float*>(take((size_t)T * E * 4));
    w.idx = reinterpret_cast<int32_t*>(take((size_t)T * K * 4));
    w.gate = reinterpret_cast<float*>(take((size_t)T * K * 4));
    w.count = reinterpret_cast<int32_t*>(take((size_t)E * 4));
    w.go = reinterpret_cast<int32_t*>(take((size_t)(E + 2) * 4));
    w.row_token = reinterpret_cast<int32_t*>(take(R * 4));
    w.slot_row = reinterpret_cast<int32_t*>(take((size_t)T * K * 4));
    w.uq = reinterpret_cast<uint8_t*>(take((size_t)T * d));
    w.us = reinterpret_cast<float*>(take((size_t)T * (d / 128) * 4));
    w.hq = reinterpret_cast<uint8_t*>(take(R * I));
    w.hs = reinterpret_cast<float*>(take(R * (I / 128) * 4));
    w.y = reinterpret_cast<float*>(take(R * d * 4));
    w.dws = take(moe::dispatch_ws_bytes(T, E));
    w.gws = take(moe::gemm_ws_bytes(E + 1, R, 2 * I > d ? 2 * I : d, I > d ? I : d));   // shared by both GEMMs
    w.total = off;
    return w;
}
}  // namespace

size_t moe_layer_workspace_bytes(int64_t T, int d, int E, int K, int I) {
    // 0 outside moe_layer_forward's limits (which also keep the sizes from overflowing)
    if (T <= 0 || d <= 0 || E <= 0 || K <= 0 || I <= 0 || E > 256 || K > 16 || d > 16384 || I > 16384 ||
        T * (K + 1) >= ((int64_t)1 << 31))
        return 0;
    return layer_ws(nullptr, T, d, E, K, I).total;
}

int moe_layer_forward(const void* u_bf16, const void* centroids_bf16, const float* bias,
                      const void* packed_weights, int64_t T, int d, int E, int K, int I,
                      float* out, int32_t* expert_count_out, void* ws, size_t ws_bytes,
                      moe_stream_t stream) {
    REQUIRE(T >= 0, MOE_ERR_SHAPE, "moe_layer_forward: T < 0");
    REQUIRE(d > 0 && d % 128 == 0, MOE_ERR_SHAPE, "moe_layer_forward: d=%d must be a multiple of 128", d);
    REQUIRE(I > 0 && I % 128 == 0, MOE_ERR_SHAPE, "moe_layer_forward: I=%d must be a multiple of 128", I);
    REQUIRE(E >= 1 && E <= 256, MOE_ERR_UNSUPPORTED, "moe_layer_forward: E=%d outside [1, 256]", E);
    REQUIRE(K >= 1 && K <= E && K <= 16, MOE_ERR_UNSUPPORTED, "moe_layer_forward: K=%d", K);
    REQUIRE(d <= 16384 && I <= 16384, MOE_ERR_UNSUPPORTED, "moe_layer_forward: d=%d or I=%d above 16384", d, I);
    REQUIRE(T * (K + 1) < ((int64_t)1 << 31) && T * (int64_t)d < ((int64_t)1 << 32) &&
                T * (K + 1) * (int64_t)I < ((int64_t)1 << 32),
            MOE_ERR_UNSUPPORTED, "moe_layer_forward: T=%lld too large", (long long)T);
    if (T == 0) return MOE_OK;
    REQUIRE_PTR(u_bf16);
    REQUIRE_PTR(centroids_bf16);
    REQUIRE_PTR(bias);
    REQUIRE_PTR(packed_weights);
    REQUIRE_PTR(out);
    REQUIRE_PTR(ws);
    if (expert_count_out) REQUIRE_PTR(expert_count_out);
    LayerWs w = layer_ws(ws, T, d, E, K, I);
    REQUIRE(ws_bytes >= w.total, MOE_ERR_WORKSPACE, "moe_layer_forward: workspace %zu < %zu bytes",
            ws_bytes, w.total);
    const int G = E + 1;
    Packed pk = packed_layout(const_cast<void*>(packed_weights), G, d, I);
    const int64_t R = T * (K + 1);
    hipStream_t st = S(stream);
    hipError_t e;
    e = moe::launch_router_scores(static_cast<const uint16_t*>(u_bf16),
                                  static_cast<const uint16_t*>(centroids_bf16), T, d, E, w.scores, st);
    if (e != hipSuccess) return hip_status(e, "router scores launch");
    e = moe::launch_router_topk(w.scores, bias, T, E, K, 1, 1, w.idx, w.gate, st);
    if (e != hipSuccess) return hip_status(e, "router top-k launch");
    e = moe::launch_dispatch(w.idx, T, K, E, 1, w.count, w.go, w.row_token, w.slot_row, w.dws, st);
    if (e != hipSuccess) return hip_status(e, "dispatch launch");
    e = moe::launch_quant_1x128(u_bf16, 0, T, d, w.uq, w.us, st);
    if (e != hipSuccess) return hip_status(e, "quant launch");
    e = moe::launch_grouped_gemm(w.uq, w.us, w.row_token, w.go, G, R, pk.w13q, pk.w13s, 2 * I, d,
                                 moe::EPI_SWIGLU_QUANT, nullptr, w.hq, w.hs, w.gws, st);
    if (e != hipSuccess) return hip_status(e, "gemm1 launch");
    e = moe::launch_grouped_gemm(w.hq, w.hs, nullptr, w.go, G, R, pk.w2q, pk.w2s, d, I,
                                 moe::EPI_STORE_F32, w.y, nullptr, nullptr, w.gws, st);
    if (e != hipSuccess) return hip_status(e, "gemm2 launch");
    e = moe::launch_combine(static_cast<const uint16_t*>(u_bf16), w.y, 1, T * K, w.gate, w.slot_row,
                            T, K, d, out, st);
    if (e != hipSuccess) return hip_status(e, "combine launch");
    if (expert_count_out) {
        e = hipMemcpyAsync(expert_count_out, w.count, (size_t)E * 4, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return hip_status(e, "count copy");
    }
    return MOE_OK;
}

}  // extern "C"
