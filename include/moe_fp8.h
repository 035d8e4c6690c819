/*
 * moe_fp8.h -- C ABI of the MI355X (gfx950) DeepSeekMoE layer forward.
 *
 * One DeepSeekMoE layer: sigmoid top-K routing with a selection-only bias,
 * drop-free dispatch, FP8 (OCP E4M3) block-scaled SwiGLU expert FFNs for one
 * shared and E routed experts, the weighted combine, and the bias update.
 *
 * Sources ("the pages"):
 *   [IFS]     "DeepSeek-V3 Technical Report" notes, learn.ifs.name/d/deepseekv3:
 *             the MoE-routing paragraph, the bias-balancing paragraph, the FP8
 *             tiling paragraph and the FP8-accumulation paragraph.
 *   [LINEAGE] "DeepSeek-V3" summary, nlp-lineage.vercel.app: "The idea"
 *             (load-balancing and FP8 bullets) and "The notation" (the layer's
 *             output equation).
 *
 * Conventions for every call below
 *   - Tensor pointers are DEVICE pointers owned by the caller, row-major and
 *     contiguous, 16-byte aligned (else MOE_ERR_ALIGN).  bf16 data is passed
 *     as raw 16-bit words, E4M3 data as raw bytes (OCP OFP8 E4M3: bias 7, no
 *     infinities, max 448).
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     legacy default stream) and returns without synchronising.  The library
 *     never allocates or frees device memory; scratch space is passed in.
 *   - Arguments are checked on the host before anything is enqueued; on an
 *     error nothing is launched and the status says why (moe_last_error()
 *     gives a thread-local message).  A failed launch returns MOE_ERR_HIP.
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Results are deterministic: identical inputs give identical bits.
 *   - T = 0 (no tokens) is valid and enqueues nothing.
 */
#ifndef MOE_FP8_H
#define MOE_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* the same type as hipStream_t */

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULLPTR = -1,     /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,       /* sizes inconsistent or not multiples of 128 */
    MOE_ERR_UNSUPPORTED = -3, /* sizes outside what the kernels handle */
    MOE_ERR_WORKSPACE = -4,   /* scratch buffer too small */
    MOE_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
    MOE_ERR_HIP = -6          /* the HIP runtime reported an error */
} moe_status;

typedef enum { MOE_BF16 = 0, MOE_F32 = 1 } moe_dtype;

/* What the grouped GEMM writes (grouped_gemm_fp8_blockscaled). */
typedef enum {
    MOE_EPI_STORE_F32 = 0,   /* out = C, FP32 [M_total, N] */
    MOE_EPI_SWIGLU_F32 = 1,  /* out = SiLU(C_gate) * C_up, FP32 [M_total, N/2] */
    MOE_EPI_SWIGLU_QUANT = 2, /* the same h, quantised per 1x128 tile into
                                out_q E4M3 [M_total, N/2] + out_scale FP32
                                [M_total, N/256] */
    MOE_EPI_SWIGLU_QUANT_Z = 3 /* as MOE_EPI_SWIGLU_QUANT, and also C itself
                                (the SwiGLU inputs a backward pass needs) in
                                out FP32 [M_total, N] */
} moe_epilogue;

const char* moe_status_string(int status);
const char* moe_last_error(void);
/* Library version: major*10000 + minor*100 + patch. */
int moe_version(void);

/* ------------------------------------------------------------------ router
 * moe_router_topk -- [IFS] MoE-routing paragraph (affinity = sigmoid of the
 * token-centroid dot product; K experts chosen per token; gates divided by
 * the sum over the chosen set); [IFS] bias paragraph and [LINEAGE] "The
 * notation" (the balancing bias enters the ranking only, never the gate).
 *
 *   s[t,i]   = sigmoid(sum_k u[t,k] e[i,k])   FP32, summed in increasing k with
 *              one FMA per term; the sigmoid is the library's fixed binary32
 *              algorithm (Cody-Waite reduced exp with a degree-7 Taylor
 *              polynomial, then 1/(1+exp(-x))), identical bit for bit across runs.
 *   key      = s[t,i] + bias[i]  (binary32 add)
 *   topk_idx[t,0..K-1]  = experts ranked by (key descending, index ascending)
 *   topk_gate[t,k]      = s[t,idx] / D, D = binary32 sum of the chosen s in
 *                         slot order (all gates 0 if D = 0)
 *
 * u_bf16 [T,d], centroids_bf16 [E,d] (bf16 words); bias FP32 [E], read only;
 * scores FP32 [T,E]: caller-provided scratch that holds s on return;
 * topk_idx int32 [T,K]; topk_gate FP32 [T,K].
 * Limits: d % 128 == 0, 1 <= E <= 256, 1 <= K <= min(E, 16).
 */
int moe_router_topk(const void* u_bf16, const void* centroids_bf16, const float* bias,
                    int64_t T, int d, int E, int K, float* scores, int32_t* topk_idx,
                    float* topk_gate, moe_stream_t stream);

/* moe_router_topk_grouped -- the group-limited variant of moe_router_topk
 * ("DeepSeek-V3 Technical Report" notes, MoE-routing paragraph: each token is
 * sent to at most 4 nodes).  The pages give no rule for choosing the groups;
 * this library's reading: the E experts form n_groups groups of E/n_groups
 * consecutive indices (one group per node), a group's score is the largest
 * key = s + bias among its experts, the topk_groups groups with the largest
 * scores are kept (ties to the lower group index), and the K experts are the
 * top K of the kept groups' experts by (key descending, index ascending).
 * Gates as in moe_router_topk.  n_groups = 1 is moe_router_topk.
 * Limits: as moe_router_topk, plus 1 <= n_groups <= 64 dividing E,
 * 1 <= topk_groups <= n_groups, K <= topk_groups * E / n_groups.
 */
int moe_router_topk_grouped(const void* u_bf16, const void* centroids_bf16, const float* bias,
                            int64_t T, int d, int E, int K, int n_groups, int topk_groups,
                            float* scores, int32_t* topk_idx, float* topk_gate,
                            moe_stream_t stream);

/* moe_seq_balance_loss -- [IFS] bias paragraph: a very small sequence-wise
 * loss remains against extreme imbalance within one sequence.  The pages give
 * no formula; this library's reading, per sequence of seq_len = L tokens
 * (tokens [q L, (q+1) L) form sequence q):
 *   f_i = E / (K L) * #{tokens of the sequence whose topk_idx holds i}
 *   P_i = (1/L) * sum_t scores[t,i] / sum_j scores[t,j]   (a token whose
 *         scores sum to 0 adds nothing)
 *   loss[q] = alpha * sum_i f_i P_i                         (FP32)
 * Uniform use gives alpha; all tokens on the same K experts, with all their
 * score there, give alpha * E / K.  scores FP32 [T,E] (moe_router_topk's
 * scores output); topk_idx int32 [T,K] (values outside [0,E) are not
 * counted); loss FP32 [T / seq_len].  Deterministic.  ws: scratch of
 * moe_seq_balance_loss_workspace_bytes(T, seq_len) bytes (per-chunk partial
 * sums; no setup needed; 0 for invalid sizes).
 * Limits: T % seq_len == 0, T / seq_len <= 65535, 1 <= E <= 256,
 * 1 <= K <= min(E, 16).
 */
size_t moe_seq_balance_loss_workspace_bytes(int64_t T, int seq_len);
int moe_seq_balance_loss(const float* scores, const int32_t* topk_idx, int64_t T, int E, int K,
                         int seq_len, float alpha, float* loss, void* ws, size_t ws_bytes,
                         moe_stream_t stream);

/* ------------------------------------------------------------------ dispatch
 * moe_dispatch -- turns the routing into GEMM rows.  No token is ever dropped
 * ([LINEAGE] "The idea", load-balancing bullet): there is no capacity limit.
 * Rows are ordered by (expert, token); with include_shared the T rows of the
 * shared expert ([IFS] MoE-routing paragraph: one shared expert every token
 * uses) follow in token order.  R = T*K + (include_shared ? T : 0).
 *
 *   expert_count int32 [E]                  assignments per routed expert
 *   group_offset int32 [E + 1 + include_shared]
 *                exclusive scan of expert_count, then T*K (, then T*K + T)
 *   row_token    int32 [R]                  token of each GEMM row
 *   slot_row     int32 [T,K]                row holding assignment (t, k)
 * topk_idx must hold values in [0, E) with distinct experts per token (as
 * moe_router_topk writes); other input gives unspecified rows but no
 * out-of-bounds access.  ws: scratch of moe_dispatch_workspace_bytes(T, E).
 */
/* 0 outside moe_dispatch's limits (T outside [1, 2^31), E outside [1, 256]). */
size_t moe_dispatch_workspace_bytes(int64_t T, int E);
int moe_dispatch(const int32_t* topk_idx, int64_t T, int K, int E, int include_shared,
                 int32_t* expert_count, int32_t* group_offset, int32_t* row_token,
                 int32_t* slot_row, void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_dispatch_check -- the debug status word of a dispatch result: the
 * invariants of a drop-free dispatch ([LINEAGE] "The idea": no token is
 * dropped, so the counts sum to exactly T*K) checked on the device and written
 * to *status (uint32, device) as a bitmask of moe_check; 0 = every invariant
 * holds.  Not part of the layer's path: debug code and tests call it after
 * moe_dispatch and read the word back.  expert_count, group_offset as
 * moe_dispatch wrote them (required); topk_idx, row_token, slot_row may all
 * be NULL, else every assignment's row is checked too.  Every index is
 * range-checked before use, so corrupted arrays are reported, never
 * dereferenced out of range.  Limits as moe_dispatch.
 */
enum moe_check {
    MOE_CHECK_COUNT_SUM = 1u << 0,            /* sum of expert_count != T*K */
    MOE_CHECK_OFFSETS_NOT_MONOTONE = 1u << 1, /* group_offset decreases somewhere */
    MOE_CHECK_FIRST_OFFSET = 1u << 2,         /* group_offset[0] != 0 */
    MOE_CHECK_COUNT_NE_OFFSETS = 1u << 3,     /* group_offset[e+1] - group_offset[e] != expert_count[e] */
    MOE_CHECK_ROUTED_TOTAL = 1u << 4,         /* group_offset[E] != T*K */
    MOE_CHECK_SHARED_GROUP = 1u << 5,         /* with the shared group: its size != T */
    MOE_CHECK_NEGATIVE_COUNT = 1u << 6,       /* a negative expert_count */
    MOE_CHECK_SLOT_ROW = 1u << 7,             /* slot_row[t,k] outside expert idx[t,k]'s group, or its row's token != t */
    MOE_CHECK_SHARED_ROWS = 1u << 8           /* row_token[T*K + t] != t */
};
int moe_dispatch_check(const int32_t* expert_count, const int32_t* group_offset, const int32_t* topk_idx,
                       const int32_t* row_token, const int32_t* slot_row, int64_t T, int K, int E,
                       int include_shared, uint32_t* status, moe_stream_t stream);

/* moe_permute_rows -- out[r] = x[row_token[r]] for r < rows, rows of d
 * elements of type dt: the data movement of the dispatch made explicit
 * ([IFS] DualPipe/EP paragraph: tokens are sent to their experts and the
 * results gathered back; on one GPU this is an in-memory gather).  x [*, d],
 * row_token int32 [rows] with values indexing rows of x (not checked: the
 * call cannot see x's row count), out [rows, d] of the same type; dt is
 * MOE_BF16 or MOE_F32; d >= 1.  Used by the router/dispatch/combine workload
 * (identity experts); the FFN path gathers rows inside the GEMM instead. */
int moe_permute_rows(const void* x, int dt, const int32_t* row_token, int64_t rows, int d,
                     void* out, moe_stream_t stream);

/* ------------------------------------------------------------------ FP8 quantisers
 * [IFS] FP8-tiling paragraph: activations are scaled per 1x128 tile (one
 * token, 128 channels) and weights per 128x128 block, so an outlier only
 * affects its own group.  Scale rule for every tile/block:
 *   amax = max|x|;  if amax == 0 or 448/amax is not finite: scale = inv = 1,
 *   else inv = fl32(448/amax), scale = fl32(amax/448);
 *   q = E4M3(fl32(x * inv)), round to nearest even, finite overflow saturates
 *   to +-448, NaN -> 0x7F|sign.  The value is decoded as E4M3(q) * scale.
 *
 * fp8_quant_1x128: x [rows, cols] (bf16 or FP32) -> q [rows, cols],
 *                  scale FP32 [rows, cols/128].  cols % 128 == 0.
 * fp8_quant_128x128: w [rows, cols] FP32 -> q [rows, cols],
 *                  scale FP32 [rows/128, cols/128].  rows, cols % 128 == 0.
 */
int fp8_quant_1x128(const void* x, int in_dt, int64_t rows, int cols, uint8_t* q,
                    float* scale, moe_stream_t stream);
int fp8_quant_128x128(const float* w, int64_t rows, int cols, uint8_t* q, float* scale,
                      moe_stream_t stream);

/* ------------------------------------------------------------------ grouped GEMM
 * grouped_gemm_fp8_blockscaled -- [IFS] FP8-accumulation paragraph: the inner
 * dimension is processed in 128-element slices and each slice's partial sum is
 * promoted to FP32, where the per-group scales are applied:
 *   C[m,n] = sum_j  a_scale[am,j] * b_scale[g, n/128, j] * P_j[m,n],
 *   P_j[m,n] = sum_{k in slice j} E4M3(a_q[am,k]) * E4M3(b_q[g,n,k])
 * with every P_j an FP8 MFMA into a fresh FP32 accumulator and the scaled sum
 * an FP32 FMA chain over j.  Row m belongs to group g when
 * group_offset[g] <= m < group_offset[g+1]; am = a_row_index[m] (a gather; NULL
 * means am = m).
 *
 *   a_q  E4M3 [*, K], a_scale FP32 [*, K/128]
 *   group_offset int32 [G+1] (device), non-decreasing, group_offset[0] = 0,
 *                group_offset[G] = M_total (the host-known total row count)
 *   b_q  E4M3 [G, N, K], b_scale FP32 [G, N/128, K/128]
 *   epi  MOE_EPI_STORE_F32:   out FP32 [M_total, N]
 *        MOE_EPI_SWIGLU_F32:  out FP32 [M_total, N/2]; B's rows are interleaved
 *                             in 128-row blocks: rows [256j, 256j+128) are the
 *                             gate projection's rows [128j, 128j+128) and rows
 *                             [256j+128, 256j+256) the up projection's;
 *                             h[m, 128j+c] = SiLU(C[m,256j+c]) * C[m,256j+128+c]
 *        MOE_EPI_SWIGLU_QUANT: the same h, quantised per 1x128 tile with the
 *                             rule above into out_q [M_total, N/2] and
 *                             out_scale [M_total, N/256]; out may be NULL
 *                             (else it receives h FP32 [M_total, N/2]).
 *        MOE_EPI_SWIGLU_QUANT_Z: out_q and out_scale as SWIGLU_QUANT, and
 *                             C in out FP32 [M_total, N] (required).
 *   ws   scratch of moe_gemm_workspace_bytes(G, M_total, N, K) bytes (the
 *        device-built tile map and tile list, and the A scales gathered into
 *        GEMM row order, slice-major; its contents need no setup).
 * Limits: K % 128 == 0 and K <= 16384, N % 256 == 0 for the SwiGLU epilogues,
 * N % 128 == 0 otherwise, G >= 1, (M_total + 128) * K / 32 < 2^32 (the
 * gathered A scales); A is addressed with 32-bit byte offsets, so a_q must
 * hold fewer than 2^32 / K rows (checked as M_total * K < 2^32 when
 * a_row_index is NULL; with a gather every index must satisfy it, which the
 * call cannot check).  Limits outside these return MOE_ERR_UNSUPPORTED.
 */
/* Scratch bytes for a grouped GEMM with G groups, M_total rows, N columns and
 * inner dimension K; 0 outside the call's limits (G outside [1, 65535],
 * M_total outside [0, 2^31), N < 1, K outside [1, 16384]). */
size_t moe_gemm_workspace_bytes(int G, int64_t M_total, int N, int K);
int grouped_gemm_fp8_blockscaled(const uint8_t* a_q, const float* a_scale,
                                 const int32_t* a_row_index, const int32_t* group_offset,
                                 int G, int64_t M_total, const uint8_t* b_q,
                                 const float* b_scale, int N, int K, int epi, float* out,
                                 uint8_t* out_q, float* out_scale, void* ws, size_t ws_bytes,
                                 moe_stream_t stream);

/* grouped_gemm_fp8_blockscaled_noalloc -- for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): grouped_gemm_fp8_blockscaled with the same arguments, kernels and
 * results, minus the workspace.  Its scratch (the tile map, tile list and the
 * slice-major copy of the A scales, moe_gemm_workspace_bytes(G, M_total, N, K)
 * bytes) lives in a static device array of MOE_GEMM_SCRATCH_BYTES that every
 * GPU the library runs on holds from module load until the process ends; the
 * call itself allocates and frees nothing.  Calls that need more scratch than
 * that return MOE_ERR_WORKSPACE before anything is enqueued.  Every call
 * rewrites the scratch it uses (its counters are cleared by the call's own
 * preparation kernel), so no state carries over between calls; but all calls
 * on one GPU share the one array, so calls that may overlap on that GPU (on
 * different streams, or from several threads) race and must be serialised by
 * the caller.
 */
#define MOE_GEMM_SCRATCH_BYTES (64u << 20)
int grouped_gemm_fp8_blockscaled_noalloc(const uint8_t* a_q, const float* a_scale,
                                         const int32_t* a_row_index, const int32_t* group_offset,
                                         int G, int64_t M_total, const uint8_t* b_q,
                                         const float* b_scale, int N, int K, int epi, float* out,
                                         uint8_t* out_q, float* out_scale, moe_stream_t stream);

/* moe_fp8_mfma_accumulation_probe -- a measurement beside the GEMM, not a
 * step of the layer.  [IFS] FP8-accumulation paragraph: FP8 products summed
 * inside a matrix core with limited accumulation precision lose accuracy over
 * a long inner dimension, which is why the GEMM above promotes every
 * 128-element slice to FP32.  With every scale equal to 1 this computes
 *   out[m,n] = sum_k E4M3(a_q[m,k]) * E4M3(b_q[n,k])
 * either chained (chained = 1: one FP32 accumulator carried through the FP8
 * MFMA of every 128-wide slice) or promoted (chained = 0: each slice's MFMA
 * into a fresh accumulator, then an FP32 add, i.e. the GEMM's path).
 * a_q E4M3 [M, K], b_q E4M3 [N, K], out FP32 [M, N].
 * Limits: M % 16 == 0 (M <= 1048560), N % 16 == 0, K % 128 == 0, K > 0.
 */
int moe_fp8_mfma_accumulation_probe(const uint8_t* a_q, const uint8_t* b_q, int M, int N, int K,
                                    int chained, float* out, moe_stream_t stream);

/* ------------------------------------------------------------------ combine
 * moe_combine -- [LINEAGE] "The notation":
 *   h'[t] = u[t] + sum_shared FFN(u[t]) + sum_k g[t,k] FFN_{idx[t,k]}(u[t])
 *   out[t,c] = u[t,c] + y[shared_row0 + t, c] + sum_k gate[t,k] * y[slot_row[t,k], c]
 * evaluated in FP32 in exactly that order (shared term skipped when
 * shared_row0 < 0).  u_bf16 [T,d]; y [rows, d] of type y_dt (FP32 or bf16);
 * gate FP32 [T,K]; slot_row int32 [T,K]; out FP32 [T,d].
 */
int moe_combine(const void* u_bf16, const void* y, int y_dt, int64_t shared_row0,
                const float* topk_gate, const int32_t* slot_row, int64_t T, int K, int d,
                float* out, moe_stream_t stream);

/* ------------------------------------------------------------------ bias update
 * moe_bias_update -- [IFS] bias paragraph and batch-wise-balance paragraph
 * (the sign rule of the auxiliary-loss-free balancing, once per step, on the
 * counts of the whole batch):
 *   expert_count[i]*E > total_assignments:  bias[i] -= gamma
 *   expert_count[i]*E < total_assignments:  bias[i] += gamma
 *   equal (exactly at the batch mean):      bias[i] unchanged
 * bias FP32 [E] is updated in place (binary32 add).  total_assignments = T*K
 * of the batch the counts came from.
 */
int moe_bias_update(float* bias, const int32_t* expert_count, int E, int64_t total_assignments,
                    float gamma, moe_stream_t stream);

/* ------------------------------------------------------------------ weights and the whole layer
 * Packed expert weights, for G = E + 1 groups (routed experts 0..E-1, then
 * the shared expert as group E):
 *   [W13_q  E4M3 G x (2I) x d ]  gate/up rows interleaved per 128-row block
 *   [W2_q   E4M3 G x d x I    ]
 *   [W13_s  FP32 G x (2I/128) x (d/128)]
 *   [W2_s   FP32 G x (d/128) x (I/128)]
 * moe_prepare_expert_weights quantises one expert's FP32 masters (W1, W3
 * [I,d], W2 [d,I]; FFN(x) = W2 (SiLU(W1 x) * W3 x)) per 128x128 block into
 * its slots of `packed`.  The pages name the expert only as FFN_i; the SwiGLU
 * form is this library's reading.
 */
/* Bytes of the packed weights of n_groups experts; 0 for sizes no call takes
 * (n_groups outside [1, 65537], d or I outside [1, 65536]). */
size_t moe_packed_weight_bytes(int n_groups, int d, int I);
int moe_prepare_expert_weights(const float* w1, const float* w3, const float* w2,
                               int expert_index, int n_groups, int d, int I, void* packed,
                               moe_stream_t stream);

/* ------------------------------------------------------------------ backward (input gradient)
 * The gradient of a scalar loss L with respect to u and the centroids, given
 * dh = dL/dh' FP32 [T,d], by the chain rule through [LINEAGE] "The notation"
 * (h' = u + FFN_shared(u) + sum_k g_k FFN_k(u)), g = s / (sum of s over the
 * chosen set) and s = sigmoid(u . e) ([IFS] MoE-routing paragraph);
 * the bias only selects ([IFS] bias paragraph), so it has no gradient and the
 * chosen set is held fixed.  The two expert GEMMs run on
 * grouped_gemm_fp8_blockscaled with transposed weights; their operands are
 * quantised per 1x128 tile along the contraction like the forward's (the
 * pages give no backward tiling: this library's reading).  Order:
 *   (forward GEMM1 with MOE_EPI_SWIGLU_QUANT_Z, which keeps z) ->
 *   moe_gate_backward -> GEMM(dY, W2^T) = dh_row -> moe_swiglu_backward(z) ->
 *   GEMM(dz, W13^T) = dx -> moe_router_backward.
 *
 * moe_prepare_backward_weights: packed_t receives the transposed weights in
 * the packed layout's slots: W13^T E4M3 [G, d, 2I] (its inner index keeps
 * W13's interleaved row order), W2^T [G, I, d], and the block scales
 * transposed to [G, d/128, 2I/128] and [G, I/128, d/128].  An exact byte
 * transposition (equal to quantising the transposed masters); packed_t has
 * moe_packed_weight_bytes(n_groups, d, I) bytes and must not overlap packed.
 */
int moe_prepare_backward_weights(const void* packed, int n_groups, int d, int I, void* packed_t,
                                 moe_stream_t stream);

/* moe_gate_backward -- per token t and slot k (g = topk_gate, s = scores at
 * topk_idx, D = binary32 sum of the chosen s in slot order):
 *   a_k = sum_c dh[t,c] y[slot_row[t,k],c]                       (FP32)
 *   dlogit[t,k] = (a_k - sum_j g_j a_j) / D * s_k * (1 - s_k)     (0 if D = 0)
 *   row_dlogit[slot_row[t,k]] = dlogit[t,k]
 *   dY[slot_row[t,k]] = fl32(g_k * dh[t]),  dY[shared_row0 + t] = dh[t]
 *                       (shared_row0 < 0: no shared rows)
 * dY is written quantised per 1x128 tile (the rule of fp8_quant_1x128) into
 * dy_q E4M3 [R,d] and dy_scale FP32 [R,d/128].  y FP32 [R,d] is the forward's
 * GEMM2 output (R = T*K + T with the shared rows); row_dlogit FP32 [R] (the
 * shared rows' entries are not written).  Limits: d % 128 == 0,
 * 1 <= K <= min(E, 16), E <= 256.
 */
int moe_gate_backward(const float* dh, const float* y, int64_t shared_row0, const float* topk_gate,
                      const int32_t* slot_row, const float* scores, const int32_t* topk_idx, int64_t T,
                      int K, int d, int E, uint8_t* dy_q, float* dy_scale, float* dlogit, float* row_dlogit,
                      moe_stream_t stream);

/* moe_swiglu_backward -- from the GEMM1 output z FP32 [R, 2I] (gate and up
 * columns interleaved per 256-column block, as the packed W13 lays them out)
 * and dh_row = dL/dh FP32 [R, I]:
 *   dz_up = dh_row * SiLU(z_gate),
 *   dz_gate = dh_row * z_up * sigma(z_gate) * (1 + z_gate * (1 - sigma(z_gate)))
 * written in z's layout, quantised per 1x128 tile into dz_q E4M3 [R, 2I] and
 * dz_scale FP32 [R, 2I/128].  sigma uses the hardware exp (not bit-exact).
 * Limits: I % 128 == 0.
 */
int moe_swiglu_backward(const float* z, const float* dh_row, int64_t R, int I, uint8_t* dz_q, float* dz_scale,
                        moe_stream_t stream);

/* moe_router_backward --
 *   du[t] = dh[t] + dx[shared_row0 + t] + sum_k dx[slot_row[t,k]]
 *           + sum_k dlogit[t,k] * e[topk_idx[t,k]]               (FP32, in that order)
 *   de[i] = sum over the routed rows r of expert i of
 *           row_dlogit[r] * u[row_token[r]]       (FP32, a fixed order: deterministic)
 * dx FP32 [R,d] (the GEMM(dz, W13^T) output); centroids and u bf16 [E,d],
 * [T,d]; row_token, group_offset from moe_dispatch; du FP32 [T,d]; de FP32
 * [E,d] (every row written).  Limits as moe_gate_backward.
 */
int moe_router_backward(const float* dh, const float* dx, int64_t shared_row0, const int32_t* slot_row,
                        const float* dlogit, const int32_t* topk_idx, const void* centroids_bf16,
                        const void* u_bf16, const float* row_dlogit, const int32_t* row_token,
                        const int32_t* group_offset, int64_t T, int K, int d, int E, float* du, float* de,
                        moe_stream_t stream);

/* moe_wgrad_block_starts -- kb_start int32 [G+1] (device) = the exclusive
 * scan of nkb_g = ceil(rows_g / 128), rows_g = group_offset[g+1] -
 * group_offset[g]: where each group's zero-padded 128-row blocks start in the
 * weight-gradient operands below.  Computed on the device, so nothing is read
 * back to the host; kb_start[G] <= ceil(R / 128) + G for R = group_offset[G],
 * the host-side bound the callers size their buffers with.
 * Limits: 1 <= G <= 65535.
 */
int moe_wgrad_block_starts(const int32_t* group_offset, int G, int32_t* kb_start, moe_stream_t stream);

/* moe_wgrad_operands -- the operands of the expert weight gradients
 *   dW2_g  = sum over the rows r of expert g of dY_r^T h_r           [d, I]
 *   dW13_g = sum over the rows r of expert g of dz_r^T u_(token r)   [2I, d]
 * (the chain rule through [LINEAGE] "The notation" and the SwiGLU form;
 * dY_r = topk_gate of the row's slot * dh_(token r), dh on the shared rows
 * from shared_row0 on; h = SiLU(z_gate) z_up; dz = the SwiGLU backward of
 * dh_row, in W13's interleaved row order), which contract over each
 * expert's rows: moe_wgrad runs them as K-grouped GEMMs (group g's inner
 * dimension Kp_g) on the transposed operands written here.  Group g's rows
 * [group_offset[g], group_offset[g+1]) are padded with zero rows to
 * Kp_g = 128 * nkb_g; kb_start int32 [G+1] (device, from
 * moe_wgrad_block_starts) is the exclusive scan of nkb_g = ceil(rows_g / 128),
 * and n_kb is any host-known upper bound of its total kb_start[G] (such as
 * ceil(R / 128) + G): it sizes the launch grids, and blocks past kb_start[G]
 * do nothing.  Layout, group after group (C = d, I, 2I, d for dY^T, h^T,
 * dz^T, u^T; CS = C/128 rounded up to a multiple of 4), in buffers of at
 * least n_kb blocks:
 *   codes E4M3 [C, Kp_g] at byte C * 128 * kb_start[g]
 *   dY^T, dz^T scales (1x128 along the rows) FP32 [C, nkb_g] at C * kb_start[g]
 *   h^T, u^T scales (128x128 blocks) FP32 [C/128, nkb_g] at CS * kb_start[g]
 * so each group's operands satisfy the GEMM's layout and alignment.  The
 * pages give no backward tiling: this library's reading.  Limits: d, I
 * multiples of 128, 1 <= K <= 16, n_kb <= 65535.
 */
int moe_wgrad_operands(const float* dh, const float* topk_gate, const int32_t* slot_row, const int32_t* row_token,
                       const float* z, const float* dh_row, const void* u_bf16, const int32_t* group_offset,
                       const int32_t* kb_start, int G, int n_kb, int64_t T, int K, int d, int I,
                       int64_t shared_row0, uint8_t* dyT_q, float* dyT_scale, uint8_t* hT_q, float* hT_scale,
                       uint8_t* dzT_q, float* dzT_scale, uint8_t* xT_q, float* xT_scale, moe_stream_t stream);

/* moe_wgrad -- the expert weight gradients from moe_wgrad_operands' buffers:
 * for every group g, dW2[g] = GEMM(dY^T_g, h^T_g) FP32 [d, I] and
 * dW13[g] = GEMM(dz^T_g, u^T_g) FP32 [2I, d] (W13's interleaved row order),
 * with group g's inner dimension its K-blocks [kb_start[g], kb_start[g+1])
 * (the rows of the group padded to 128); groups without rows get zero
 * gradients.  Two launches in all (one per weight), each K-grouped: every
 * group's inner dimension is its own, and nothing is read back to the host.
 * kb_start int32 [G+1] (device), the array moe_wgrad_operands took; n_kb =
 * the same host-known upper bound of kb_start[G] (only checked against the
 * limits below); dw13 FP32 [G, 2I, d], dw2 FP32 [G, d, I]; ws of
 * moe_wgrad_workspace_bytes(G, d, I) bytes.
 * Limits: n_kb * 128 * max(d, 2I) < 2^32 (32-bit byte offsets into one
 * group's operands), G * max(d, 2I) < 2^31; MOE_ERR_UNSUPPORTED otherwise.
 */
/* 0 outside [1, 65535] groups or d, I outside [1, 65536]. */
size_t moe_wgrad_workspace_bytes(int G, int d, int I);
int moe_wgrad(const int32_t* kb_start, int G, int n_kb, int d, int I, const uint8_t* dyT_q, const float* dyT_scale,
              const uint8_t* hT_q, const float* hT_scale, const uint8_t* dzT_q, const float* dzT_scale,
              const uint8_t* xT_q, const float* xT_scale, float* dw13, float* dw2, void* ws, size_t ws_bytes,
              moe_stream_t stream);

/* moe_layer_forward -- the whole layer, [LINEAGE] "The notation":
 *   h'[t] = u[t] + FFN_shared(u[t]) + sum_k g[t,k] FFN_{idx[t,k]}(u[t])
 * as router ([IFS] MoE-routing and bias paragraphs), dispatch, 1x128
 * quantisation of u ([IFS] FP8-tiling paragraph), GEMM1 with fused SwiGLU and
 * 1x128 re-quantisation, GEMM2 (both promoting per 128-wide slice, [IFS]
 * FP8-accumulation paragraph), combine: the calls above in that order.
 * The bias is read only (update it with moe_bias_update).  packed_weights as
 * above with G = E + 1; out FP32 [T,d]; expert_count_out int32 [E] (may be
 * NULL); ws of moe_layer_workspace_bytes(T, d, E, K, I).
 * Limits: d and I multiples of 128 and at most 16384, 1 <= E <= 256,
 * 1 <= K <= min(E, 16), T*(K+1) < 2^31, T*d < 2^32 and T*(K+1)*I < 2^32
 * (32-bit byte offsets of the GEMM inputs); MOE_ERR_UNSUPPORTED otherwise.
 */
/* 0 outside moe_layer_forward's limits (the ones above that involve only
 * these sizes: T >= 1, E in [1, 256], K in [1, 16], d and I in [1, 16384],
 * T*(K+1) < 2^31). */
size_t moe_layer_workspace_bytes(int64_t T, int d, int E, int K, int I);
int moe_layer_forward(const void* u_bf16, const void* centroids_bf16, const float* bias,
                      const void* packed_weights, int64_t T, int d, int E, int K, int I,
                      float* out, int32_t* expert_count_out, void* ws, size_t ws_bytes,
                      moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FP8_H */
