// Internal launchers: each .hip file enqueues its kernels on a stream and
// returns the hipError_t of the launch.  Argument checking happens in the
// C ABI layer (capi.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// router.hip
hipError_t launch_router_scores(const uint16_t* u, const uint16_t* e, int64_t T, int d, int E,
                                float* s, hipStream_t st);
// n_groups = 1: plain top-K; otherwise group-limited (see router_topk_kernel)
hipError_t launch_router_topk(const float* s, const float* bias, int64_t T, int E, int K,
                              int n_groups, int topk_groups, int32_t* idx, float* gate,
                              hipStream_t st);

// dispatch.hip
size_t dispatch_ws_bytes(int64_t T, int E);
hipError_t launch_dispatch(const int32_t* idx, int64_t T, int K, int E, int include_shared,
                           int32_t* count, int32_t* group_offset, int32_t* row_token,
                           int32_t* slot_row, void* ws, hipStream_t st);
hipError_t launch_permute_rows(const void* x, size_t elem_bytes, const int32_t* row_token,
                               int64_t rows, int d, void* out, hipStream_t st);

// quant.hip
hipError_t launch_quant_1x128(const void* x, int in_is_f32, int64_t rows, int cols, uint8_t* q,
                              float* scale, hipStream_t st);
// Block-row br of the source lands in block-row br*row_mul + row_add of the destination.
hipError_t launch_quant_128x128(const float* w, int64_t rows, int cols, uint8_t* q, float* scale,
                                int row_mul, int row_add, hipStream_t st);

// gemm.hip
enum { EPI_STORE_F32 = 0, EPI_SWIGLU_F32 = 1, EPI_SWIGLU_QUANT = 2, EPI_SWIGLU_QUANT_Z = 3 };
size_t gemm_ws_bytes(int G, int64_t M_total, int N, int K);
// device address of the static scratch array (MOE_GEMM_SCRATCH_BYTES) on the current device
hipError_t gemm_static_scratch(void** ptr);
hipError_t launch_grouped_gemm(const uint8_t* a_q, const float* a_s, const int32_t* a_rows,
                               const int32_t* group_offset, int G, int64_t M_total,
                               const uint8_t* b_q, const float* b_s, int N, int K, int epi,
                               float* out, uint8_t* out_q, float* out_s, void* ws,
                               hipStream_t st);
// K-grouped FP32-store GEMM: G groups of `rows` A rows; group g's inner
// dimension is the 128-blocks [kb_start[g], kb_start[g+1]) (device array), its
// A [rows, Kg] and 1x128 scales [rows, Kg/128] start at block kb_start[g] of
// a_q / a_s, its B [N, Kg] and 128x128 scales [N/128, Kg/128] (rows of b_cs
// blocks) at that block of b_q / b_s; out FP32 [G*rows, N].  Empty groups give 0.
size_t gemm_kgrouped_ws_bytes(int G, int rows, int N);
hipError_t launch_grouped_gemm_kgrouped(const uint8_t* a_q, const float* a_s, const int32_t* kb_start, int G,
                                        int rows, const uint8_t* b_q, const float* b_s, int b_cs, int N,
                                        float* out, void* ws, hipStream_t st);

// backward.hip
hipError_t launch_gate_backward(const float* dh, const float* y, int64_t shared_row0, const float* gate,
                                const int32_t* slot_row, const float* s, const int32_t* idx, int64_t T,
                                int K, int d, int E, uint8_t* dy_q, float* dy_s, float* dlogit,
                                float* row_dlogit, hipStream_t st);
hipError_t launch_swiglu_backward(const float* z, const float* dh_row, int64_t R, int I, uint8_t* dz_q,
                                  float* dz_s, hipStream_t st);
hipError_t launch_du(const float* dh, const float* dx, int64_t shared_row0, const int32_t* slot_row,
                     const float* dlogit, const int32_t* idx, const uint16_t* e, int64_t T, int K, int d,
                     float* du, hipStream_t st);
hipError_t launch_de(const float* row_dlogit, const int32_t* row_token, const int32_t* group_offset,
                     const uint16_t* u, int d, int E, float* de, hipStream_t st);
hipError_t launch_transpose_blocks(const uint8_t* in, const float* in_s, int G, int rows, int cols,
                                   uint8_t* out, float* out_s, hipStream_t st);

// dispatch.hip: status word of moe_dispatch_check (bits of enum moe_check in the header)
hipError_t launch_dispatch_check(const int32_t* count, const int32_t* group_offset, const int32_t* idx,
                                 const int32_t* row_token, const int32_t* slot_row, int64_t T, int K, int E,
                                 int include_shared, uint32_t* status, hipStream_t st);

// wgrad.hip
hipError_t launch_wgrad_operands(const float* dh, const float* gate, const int32_t* slot_row,
                                 const int32_t* row_token, const float* z, const float* dh_row,
                                 const uint16_t* u, int64_t shared_row0, int K, int d, int I,
                                 const int32_t* go, const int32_t* kb_start, int G, int n_kb,
                                 uint8_t* dyT_q, float* dyT_s, uint8_t* hT_q, float* hT_s, uint8_t* dzT_q,
                                 float* dzT_s, uint8_t* xT_q, float* xT_s, hipStream_t st);

size_t wgrad_ws_bytes(int G, int d, int I);
hipError_t launch_wgrad_block_starts(const int32_t* go, int G, int32_t* kb_start, hipStream_t st);
hipError_t launch_wgrad_gemms(const int32_t* kb_start, int G, int d, int I, const uint8_t* dyT_q,
                              const float* dyT_s, const uint8_t* hT_q, const float* hT_s, const uint8_t* dzT_q,
                              const float* dzT_s, const uint8_t* xT_q, const float* xT_s, float* dw13, float* dw2,
                              void* ws, hipStream_t st);

// balance.hip
size_t seq_balance_ws_bytes(int64_t n_seq, int L);
hipError_t launch_seq_balance_loss(const float* s, const int32_t* idx, int64_t n_seq, int E, int K,
                                   int L, float alpha, float* loss, void* ws, hipStream_t st);

// accum_probe.hip
hipError_t launch_accum_probe(const uint8_t* a_q, const uint8_t* b_q, int M, int N, int K,
                              int chained, float* out, hipStream_t st);

// combine.hip
hipError_t launch_combine(const uint16_t* u, const void* y, int y_is_f32, int64_t shared_row0,
                          const float* gate, const int32_t* slot_row, int64_t T, int K, int d,
                          float* out, hipStream_t st);
hipError_t launch_bias_update(float* bias, const int32_t* count, int E, int64_t total,
                              float gamma, hipStream_t st);

}  // namespace moe
