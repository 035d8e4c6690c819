/* Drives the host side of the C ABI (include/moe_fp8.h) for a build of the
 * library whose host code has AddressSanitizer and UndefinedBehaviorSanitizer:
 * every argument check, the workspace and size queries (including sizes that
 * overflow), the status strings and the thread-local error text.  No call
 * here reaches a kernel launch (each fails validation or has nothing to do),
 * so no GPU is needed.  Exit status 0 = clean. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_fp8.h"

#define EXPECT(call, want)                                                                 \
    do {                                                                                   \
        int got_ = (call);                                                                 \
        if (got_ != (want)) {                                                              \
            fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, \
                    got_, (want), moe_last_error());                                       \
            return 1;                                                                      \
        }                                                                                  \
    } while (0)

int main(void) {
    void* F = (void*)(uintptr_t)0x10000;        /* aligned, never dereferenced */
    void* MIS = (void*)(uintptr_t)0x10004;
    for (int s = -8; s <= 1; ++s) (void)strlen(moe_status_string(s));
    if (moe_version() < 10000) return 1;
    /* router */
    EXPECT(moe_router_topk(F, F, F, 8, 100, 16, 4, F, F, F, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_router_topk(F, F, F, 8, 128, 300, 4, F, F, F, NULL), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_router_topk(NULL, F, F, 8, 128, 16, 4, F, F, F, NULL), MOE_ERR_NULLPTR);
    EXPECT(moe_router_topk(MIS, F, F, 8, 128, 16, 4, F, F, F, NULL), MOE_ERR_ALIGN);
    EXPECT(moe_router_topk(NULL, NULL, NULL, 0, 128, 16, 4, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_router_topk_grouped(F, F, F, 8, 128, 16, 4, 3, 1, F, F, F, NULL), MOE_ERR_SHAPE);
    /* balance loss */
    if (moe_seq_balance_loss_workspace_bytes(INT64_MAX, 1) != 0) return 1;
    (void)moe_seq_balance_loss_workspace_bytes(100, 0);
    EXPECT(moe_seq_balance_loss(F, F, 100, 16, 4, 7, 1.0f, F, F, 1 << 20, NULL), MOE_ERR_SHAPE);
    /* dispatch and its status word */
    if (moe_dispatch_workspace_bytes(INT64_MAX / 4, 256) != 0) return 1;
    EXPECT(moe_dispatch(F, 64, 4, 16, 1, F, F, F, F, F, 0, NULL), MOE_ERR_WORKSPACE);
    EXPECT(moe_dispatch(F, 64, 17, 16, 1, F, F, F, F, F, 1 << 20, NULL), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_dispatch(F, (int64_t)1 << 40, 8, 256, 1, F, F, F, F, F, 1 << 20, NULL), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_dispatch_check(F, F, NULL, F, F, 64, 4, 16, 1, F, NULL), MOE_ERR_NULLPTR);
    EXPECT(moe_dispatch_check(F, F, F, F, F, 64, 4, 16, 2, F, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_permute_rows(F, 7, F, 10, 128, F, NULL), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_permute_rows(F, MOE_BF16, F, 10, 3, F, NULL), MOE_ERR_SHAPE);
    /* quantisers */
    EXPECT(fp8_quant_1x128(F, MOE_BF16, 4, 100, F, F, NULL), MOE_ERR_SHAPE);
    EXPECT(fp8_quant_128x128(F, 100, 128, F, F, NULL), MOE_ERR_SHAPE);
    /* grouped GEMM */
    if (moe_gemm_workspace_bytes(1, INT64_MAX / 8, 7168, 16384) != 0) return 1;
    (void)moe_gemm_workspace_bytes(0, 10, 10, 10);
    EXPECT(grouped_gemm_fp8_blockscaled(F, F, NULL, F, 2, 64, F, F, 256, 200, 0, F, NULL, NULL, F, 1 << 30, NULL),
           MOE_ERR_SHAPE);
    EXPECT(grouped_gemm_fp8_blockscaled(F, F, NULL, F, 2, 64, F, F, 256, 256, 0, F, NULL, NULL, F, 16, NULL),
           MOE_ERR_WORKSPACE);
    EXPECT(grouped_gemm_fp8_blockscaled(F, F, NULL, F, 2, 64, F, F, 256, 32768, 0, F, NULL, NULL, F, 1 << 30, NULL),
           MOE_ERR_UNSUPPORTED);
    EXPECT(moe_fp8_mfma_accumulation_probe(F, F, 15, 16, 128, 0, F, NULL), MOE_ERR_SHAPE);
    /* combine, bias update */
    EXPECT(moe_combine(F, F, 9, -1, F, F, 8, 4, 128, F, NULL), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_bias_update(NULL, F, 16, 64, 1e-3f, NULL), MOE_ERR_NULLPTR);
    /* weights and layer */
    (void)moe_packed_weight_bytes(257, 7168, 2048);
    if (moe_packed_weight_bytes(-1, 7168, 2048) != 0 || moe_packed_weight_bytes(1 << 30, 1 << 30, 1 << 30) != 0) return 1;
    if (moe_layer_workspace_bytes(INT64_MAX / 16, 7168, 256, 8, 2048) != 0) return 1;
    (void)moe_layer_workspace_bytes(16384, 7168, 256, 8, 2048);
    EXPECT(moe_prepare_expert_weights(F, F, F, 5, 3, 256, 256, F, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_layer_forward(F, F, F, F, 64, 7168, 256, 8, 2048, F, NULL, F, 16, NULL), MOE_ERR_WORKSPACE);
    EXPECT(moe_layer_forward(F, F, F, F, 64, 7168, 256, 8, 2000, F, NULL, F, 1 << 30, NULL), MOE_ERR_SHAPE);
    /* backward */
    EXPECT(moe_prepare_backward_weights(F, 3, 256, 100, F, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_gate_backward(F, F, -1, F, F, F, F, 8, 17, 128, 16, F, F, F, F, NULL), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_swiglu_backward(F, F, 8, 100, F, F, NULL), MOE_ERR_SHAPE);
    EXPECT(moe_wgrad_block_starts(F, 0, F, NULL), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_wgrad_operands(F, F, F, F, F, F, F, F, F, 3, 70000, 8, 4, 256, 128, -1, F, F, F, F, F, F, F, F, NULL),
           MOE_ERR_UNSUPPORTED);
    if (moe_wgrad_workspace_bytes(65535, 16384, 16384) == 0 || moe_wgrad_workspace_bytes(1, 1 << 30, 1 << 30) != 0)
        return 1;
    EXPECT(moe_wgrad(F, 3, -1, 256, 128, F, F, F, F, F, F, F, F, F, F, F, 1 << 30, NULL), MOE_ERR_SHAPE);
    printf("C ABI driver: clean\n");
    return 0;
}
