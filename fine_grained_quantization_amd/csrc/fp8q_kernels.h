// Host-side launchers of the fp8q gfx950 kernels.  Arguments are validated by the C-ABI layer
// (fp8q_api.hip) before any of these is called; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

hipError_t launch_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, hipStream_t stream);
hipError_t launch_quant_w_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, hipStream_t stream);
hipError_t launch_swiglu_quant_act_1x128(const uint16_t *x, const uint16_t *y, int64_t ld, int64_t M, int64_t K,
                                         uint8_t *q, float *s, hipStream_t stream);
hipError_t launch_quant_act_dual(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, uint8_t *qt,
                                 float *st, hipStream_t stream);
hipError_t launch_swiglu_bf16(const uint16_t *x, const uint16_t *y, int64_t ld, int64_t M, int64_t K, uint16_t *h,
                              hipStream_t stream);
hipError_t launch_quant_act_fp4_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s,
                                      hipStream_t stream);
hipError_t launch_quant_w_fp4_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s,
                                      hipStream_t stream);
hipError_t launch_quant_act_e5m6_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s,
                                       hipStream_t stream);
hipError_t launch_quant_w_per_channel(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s,
                                      hipStream_t stream);
hipError_t launch_dequant_w_128x128(const uint8_t *q, const float *s, int64_t N, int64_t K, uint16_t *w,
                                    hipStream_t stream);
hipError_t launch_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                                   bool out_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_grouped_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw,
                                           void *c, bool out_bf16, const int32_t *off, int64_t E, int64_t M_total,
                                           int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_grouped_gemm_gather(const uint8_t *q, const float *s, int64_t T, const int32_t *row_token,
                                      const uint8_t *qw, const float *sw, void *c, bool out_bf16,
                                      const int32_t *off, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                      hipStream_t stream);
// MoE routing: experts at most kMoeMaxExperts, k at most kMoeMaxK.
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeMaxK = 16;
int64_t moe_route_workspace_bytes(int64_t T, int64_t E);
// Bytes of the routing's fixed device workspace (one per GPU) used by the entry point that allocates nothing.
constexpr int64_t kRouteScratchBytes = int64_t(4) << 20;
// Device address of that workspace on device `dev`, which must be the current device (looked up on the first
// call per device, then cached).
hipError_t route_scratch(int dev, int32_t **ptr);
hipError_t launch_moe_route_topk(const float *logits, int64_t T, int E, int k, int32_t *topk_idx,
                                 int32_t *offsets, int32_t *row_of, int32_t *row_token, int64_t rows,
                                 int32_t *workspace, hipStream_t stream);
hipError_t launch_moe_gather_fp8(const uint8_t *q, const float *s, int64_t T, int64_t K, int k,
                                 const int32_t *row_of, const int32_t *row_token, const int32_t *offsets, int E,
                                 int64_t rows, uint8_t *qa, float *sa, hipStream_t stream);
// Number of workgroups the dense GEMM launches for an M x N output (for grid-size validation).
int64_t gemm_blocks(int64_t M, int64_t N);
// Number of workgroups a grouped GEMM launches for M rows, N columns and E experts; -1 when that count
// would pass 2^40 or E is past 2^31 (for grid-size validation).
int64_t grouped_gemm_blocks(int64_t M, int64_t N, int64_t E);

}  // namespace fp8q
