// C-ABI entry points of the fp8q library (declared in include/fp8q.h): argument and device
// validation, then one launch on the caller's stream.  No allocation, no synchronization.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "../../include/fp8q.h"
#include "fp8q_kernels.h"

namespace {

constexpr int kMaxDevices = 64;
// Per device: 0 = not yet checked, 1 = gfx950, 2 = other architecture.
std::atomic<int> g_device_kind[kMaxDevices];

int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return FP8Q_ERR_NO_DEVICE;
    }
    if (dev >= kMaxDevices) return FP8Q_ERR_UNSUPPORTED_DEVICE;
    int kind = g_device_kind[dev].load(std::memory_order_relaxed);
    if (kind == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return FP8Q_ERR_NO_DEVICE;
        }
        kind = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_kind[dev].store(kind, std::memory_order_relaxed);
    }
    return kind == 1 ? FP8Q_OK : FP8Q_ERR_UNSUPPORTED_DEVICE;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int64_t kMaxGrid = 0x7FFFFFFF;  // 1-D grids: workgroup count must fit in 31 bits
constexpr int64_t kMaxK = int64_t(1) << 23;  // GEMM tiles address 256 rows of K bytes with 32-bit offsets

int finish(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_ERR_HIP; }

static_assert(fp8q::kRouteScratchBytes == FP8Q_MOE_ROUTE_NOALLOC_BYTES, "the header states the array's size");

}  // namespace

extern "C" {

int fp8q_version(void) { return 100; }

const char *fp8q_status_string(int status) {
    switch (status) {
        case FP8Q_OK: return "FP8Q_OK: success";
        case FP8Q_ERR_NULL: return "FP8Q_ERR_NULL: a required pointer is NULL";
        case FP8Q_ERR_SHAPE: return "FP8Q_ERR_SHAPE: invalid shape (negative size, K or N not a multiple of 128, or bad grouping)";
        case FP8Q_ERR_ALIGN: return "FP8Q_ERR_ALIGN: a tensor base address is not 16-byte aligned";
        case FP8Q_ERR_DTYPE: return "FP8Q_ERR_DTYPE: unknown output dtype";
        case FP8Q_ERR_NO_DEVICE: return "FP8Q_ERR_NO_DEVICE: no HIP device available";
        case FP8Q_ERR_UNSUPPORTED_DEVICE: return "FP8Q_ERR_UNSUPPORTED_DEVICE: the current device is not gfx950 (MI355X)";
        case FP8Q_ERR_HIP: return "FP8Q_ERR_HIP: the HIP runtime reported a launch error";
        case FP8Q_ERR_WORKSPACE: return "FP8Q_ERR_WORKSPACE: the workspace is smaller than the call needs";
        default: return "fp8q: unknown status";
    }
}

int fp8q_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, void *stream) {
    if (M < 0 || K < 0 || K % 128) return FP8Q_ERR_SHAPE;
    if (M == 0 || K == 0) return FP8Q_OK;
    if (!x || !q || !s) return FP8Q_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return FP8Q_ERR_ALIGN;
    if (((M + 15) / 16) * ((K / 128 + 3) / 4) > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_quant_act_1x128(x, M, K, q, s, static_cast<hipStream_t>(stream)));
}

int fp8q_swiglu_quant_act_1x128(const uint16_t *x, const uint16_t *y, int64_t ld, int64_t M, int64_t K, uint8_t *q,
                                float *s, void *stream) {
    if (M < 0 || K < 0 || K % 128 || ld < K || ld % 8) return FP8Q_ERR_SHAPE;
    if (M == 0 || K == 0) return FP8Q_OK;
    if (!x || !y || !q || !s) return FP8Q_ERR_NULL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(q) || !aligned16(s)) return FP8Q_ERR_ALIGN;
    if (((M + 15) / 16) * ((K / 128 + 3) / 4) > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_swiglu_quant_act_1x128(x, y, ld, M, K, q, s, static_cast<hipStream_t>(stream)));
}

int fp8q_quant_act_fp4_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, void *stream) {
    if (M < 0 || K < 0 || K % 128) return FP8Q_ERR_SHAPE;
    if (M == 0 || K == 0) return FP8Q_OK;
    if (!x || !q || !s) return FP8Q_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return FP8Q_ERR_ALIGN;
    if (((M + 15) / 16) * ((K / 128 + 3) / 4) > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_quant_act_fp4_1x128(x, M, K, q, s, static_cast<hipStream_t>(stream)));
}

int fp8q_quant_w_fp4_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, void *stream) {
    if (N < 0 || K < 0 || N % 128 || K % 128) return FP8Q_ERR_SHAPE;
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!w || !q || !s) return FP8Q_ERR_NULL;
    if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return FP8Q_ERR_ALIGN;
    if ((N / 128) * (K / 128) > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_quant_w_fp4_128x128(w, N, K, q, s, static_cast<hipStream_t>(stream)));
}

int fp8q_quant_act_e5m6_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, void *stream) {
    if (M < 0 || K < 0 || K % 128) return FP8Q_ERR_SHAPE;
    if (M == 0 || K == 0) return FP8Q_OK;
    if (!x || !q || !s) return FP8Q_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return FP8Q_ERR_ALIGN;
    if (((M + 15) / 16) * ((K / 128 + 3) / 4) > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_quant_act_e5m6_1x128(x, M, K, q, s, static_cast<hipStream_t>(stream)));
}

int fp8q_quant_w_per_channel(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, void *stream) {
    if (N < 0 || K < 0 || K % 8) return FP8Q_ERR_SHAPE;
    if (N == 0) return FP8Q_OK;
    if (!s || (K > 0 && (!w || !q))) return FP8Q_ERR_NULL;  // K == 0: only the (zero) scales are written
    if (!aligned4(s) || (K > 0 && (!aligned16(w) || !aligned16(q)))) return FP8Q_ERR_ALIGN;
    if (N > kMaxGrid) return FP8Q_ERR_SHAPE;  // one workgroup per row
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_quant_w_per_channel(w, N, K, q, s, static_cast<hipStream_t>(stream)));
}

int fp8q_quant_act_dual(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, uint8_t *qt, float *st,
                        void *stream) {
    if (M < 0 || K < 0 || M % 128 || K % 128) return FP8Q_ERR_SHAPE;
    if (M == 0 || K == 0) return FP8Q_OK;
    if (!x || !q || !s || !qt || !st) return FP8Q_ERR_NULL;
    if (!aligned16(x) || !aligned16(q) || !aligned16(s) || !aligned16(qt) || !aligned16(st)) return FP8Q_ERR_ALIGN;
    if ((M / 128) * (K / 128) > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_quant_act_dual(x, M, K, q, s, qt, st, static_cast<hipStream_t>(stream)));
}

int fp8q_swiglu_bf16(const uint16_t *x, const uint16_t *y, int64_t ld, int64_t M, int64_t K, uint16_t *h,
                     void *stream) {
    if (M < 0 || K < 0 || K % 8 || ld < K || ld % 8) return FP8Q_ERR_SHAPE;
    if (M == 0 || K == 0) return FP8Q_OK;
    if (!x || !y || !h) return FP8Q_ERR_NULL;
    if (!aligned16(x) || !aligned16(y) || !aligned16(h)) return FP8Q_ERR_ALIGN;
    if (K / 8 > kMaxGrid / M * 256) return FP8Q_ERR_SHAPE;  // M * K / 2048 workgroups
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_swiglu_bf16(x, y, ld, M, K, h, static_cast<hipStream_t>(stream)));
}

int fp8q_quant_w_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, void *stream) {
    if (N < 0 || K < 0 || N % 128 || K % 128) return FP8Q_ERR_SHAPE;
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!w || !q || !s) return FP8Q_ERR_NULL;
    if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return FP8Q_ERR_ALIGN;
    if ((N / 128) * (K / 128) > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_quant_w_128x128(w, N, K, q, s, static_cast<hipStream_t>(stream)));
}

int fp8q_dequant_w_128x128(const uint8_t *q, const float *s, int64_t N, int64_t K, uint16_t *w, void *stream) {
    if (N < 0 || K < 0 || N % 128 || K % 128) return FP8Q_ERR_SHAPE;
    if (N == 0 || K == 0) return FP8Q_OK;
    if (!q || !s || !w) return FP8Q_ERR_NULL;
    if (!aligned16(q) || !aligned16(s) || !aligned16(w)) return FP8Q_ERR_ALIGN;
    if (K / 128 > kMaxGrid / N * 8) return FP8Q_ERR_SHAPE;  // N * K / 8192 workgroups
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_dequant_w_128x128(q, s, N, K, w, static_cast<hipStream_t>(stream)));
}

int fp8q_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                          int out_dtype, int64_t M, int64_t N, int64_t K, void *stream) {
    if (M < 0 || N < 0 || K < 128 || K > kMaxK || N % 128 || K % 128) return FP8Q_ERR_SHAPE;
    if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32) return FP8Q_ERR_DTYPE;
    if (M == 0 || N == 0) return FP8Q_OK;
    if (!qa || !sa || !qw || !sw || !c) return FP8Q_ERR_NULL;
    if (!aligned16(qa) || !aligned16(sa) || !aligned16(qw) || !aligned16(sw) || !aligned16(c)) return FP8Q_ERR_ALIGN;
    if (fp8q::gemm_blocks(M, N) > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_gemm_blockscaled(qa, sa, qw, sw, c, out_dtype == FP8Q_OUT_BF16, M, N, K,
                                                static_cast<hipStream_t>(stream)));
}

int fp8q_grouped_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                                  int out_dtype, const int32_t *off, int64_t E, int64_t M_total, int64_t N,
                                  int64_t K, void *stream) {
    if (E < 1 || M_total < 0 || M_total % 128 || N < 0 || K < 128 || K > kMaxK || N % 128 || K % 128)
        return FP8Q_ERR_SHAPE;
    if (M_total > 0x7FFFFFFF) return FP8Q_ERR_SHAPE;  // offsets are int32
    if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32) return FP8Q_ERR_DTYPE;
    if (M_total == 0 || N == 0) return FP8Q_OK;
    if (!qa || !sa || !qw || !sw || !c || !off) return FP8Q_ERR_NULL;
    if (!aligned16(qa) || !aligned16(sa) || !aligned16(qw) || !aligned16(sw) || !aligned16(c)) return FP8Q_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(off) & 3u) != 0) return FP8Q_ERR_ALIGN;
    const int64_t blocks = fp8q::grouped_gemm_blocks(M_total, N, E);
    if (blocks < 0 || blocks > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_grouped_gemm_blockscaled(qa, sa, qw, sw, c, out_dtype == FP8Q_OUT_BF16, off, E,
                                                        M_total, N, K, static_cast<hipStream_t>(stream)));
}

int fp8q_grouped_gemm_blockscaled_gather(const uint8_t *q, const float *s, int64_t T, const int32_t *row_token,
                                         const uint8_t *qw, const float *sw, void *c, int out_dtype,
                                         const int32_t *off, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                         void *stream) {
    if (E < 1 || M_total < 0 || M_total % 128 || N < 0 || K < 128 || K > kMaxK || N % 128 || K % 128 || T < 0)
        return FP8Q_ERR_SHAPE;
    if (M_total > 0x7FFFFFFF) return FP8Q_ERR_SHAPE;           // offsets are int32
    if (T > 0 && T > (int64_t)0x7FFFFFFF / K) return FP8Q_ERR_SHAPE;  // token offsets are 32-bit
    if (out_dtype != FP8Q_OUT_BF16 && out_dtype != FP8Q_OUT_F32) return FP8Q_ERR_DTYPE;
    if (M_total == 0 || N == 0) return FP8Q_OK;
    if (!row_token || !qw || !sw || !c || !off || (T > 0 && (!q || !s))) return FP8Q_ERR_NULL;
    if (!aligned16(qw) || !aligned16(sw) || !aligned16(c) || !aligned4(off) || !aligned4(row_token) ||
        (T > 0 && (!aligned16(q) || !aligned4(s))))
        return FP8Q_ERR_ALIGN;
    const int64_t blocks = fp8q::grouped_gemm_blocks(M_total, N, E);
    if (blocks < 0 || blocks > kMaxGrid) return FP8Q_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_grouped_gemm_gather(q, s, T, row_token, qw, sw, c, out_dtype == FP8Q_OUT_BF16, off, E,
                                                   M_total, N, K, static_cast<hipStream_t>(stream)));
}

int64_t fp8q_moe_route_capacity(int64_t T, int64_t E, int64_t k) {
    if (T < 0 || E < 1 || E > fp8q::kMoeMaxExperts || k < 1 || k > E || k > fp8q::kMoeMaxK) return -1;
    if (T > (int64_t(1) << 40)) return -1;
    return (T * k + 127 * E + 127) / 128 * 128;
}

int64_t fp8q_moe_route_workspace_bytes(int64_t T, int64_t E) {
    if (T < 0 || E < 1 || E > fp8q::kMoeMaxExperts || T > (int64_t(1) << 40)) return -1;
    return fp8q::moe_route_workspace_bytes(T, E);
}

int fp8q_moe_route_topk(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *topk_idx, int32_t *offsets,
                        int32_t *row_of, int32_t *row_token, int64_t rows, void *workspace, int64_t workspace_bytes,
                        void *stream) {
    const int64_t cap = fp8q_moe_route_capacity(T, E, k);
    if (cap < 0 || rows < cap || rows > 0x7FFFFFFF) return FP8Q_ERR_SHAPE;
    if (!offsets || !row_token) return FP8Q_ERR_NULL;
    if (T > 0 && (!logits || !topk_idx || !row_of || !workspace)) return FP8Q_ERR_NULL;
    if (!aligned4(offsets) || !aligned4(row_token) || (T > 0 && (!aligned4(logits) || !aligned4(topk_idx) ||
                                                                 !aligned4(row_of) || !aligned4(workspace))))
        return FP8Q_ERR_ALIGN;
    if (workspace_bytes < fp8q::moe_route_workspace_bytes(T, E)) return FP8Q_ERR_WORKSPACE;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_moe_route_topk(logits, T, (int)E, (int)k, topk_idx, offsets, row_of, row_token, rows,
                                              static_cast<int32_t *>(workspace), static_cast<hipStream_t>(stream)));
}

int fp8q_moe_route_topk_noalloc(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *topk_idx,
                                int32_t *offsets, int32_t *row_of, int32_t *row_token, int64_t rows, void *stream) {
    const int64_t cap = fp8q_moe_route_capacity(T, E, k);
    if (cap < 0 || rows < cap || rows > 0x7FFFFFFF) return FP8Q_ERR_SHAPE;
    if (!offsets || !row_token) return FP8Q_ERR_NULL;
    if (T > 0 && (!logits || !topk_idx || !row_of)) return FP8Q_ERR_NULL;
    if (!aligned4(offsets) || !aligned4(row_token) ||
        (T > 0 && (!aligned4(logits) || !aligned4(topk_idx) || !aligned4(row_of))))
        return FP8Q_ERR_ALIGN;
    if (fp8q::moe_route_workspace_bytes(T, E) > fp8q::kRouteScratchBytes) return FP8Q_ERR_WORKSPACE;
    int rc = check_device();
    if (rc) return rc;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return FP8Q_ERR_NO_DEVICE;
    }
    int32_t *ws = nullptr;
    if (fp8q::route_scratch(dev, &ws) != hipSuccess) return FP8Q_ERR_HIP;
    return finish(fp8q::launch_moe_route_topk(logits, T, (int)E, (int)k, topk_idx, offsets, row_of, row_token, rows,
                                              ws, static_cast<hipStream_t>(stream)));
}

int fp8q_moe_gather_fp8(const uint8_t *q, const float *s, int64_t T, int64_t K, int64_t k, const int32_t *row_of,
                        const int32_t *row_token, const int32_t *offsets, int64_t E, int64_t rows, uint8_t *qa,
                        float *sa, void *stream) {
    if (T < 0 || T > 0x7FFFFFFF || K < 0 || K % 128 || k < 1 || k > 0x7FFFFFFF / (T > 0 ? T : 1) || E < 1 ||
        E > 0x7FFFFFFF || rows < 0 || rows > 0x7FFFFFFF)
        return FP8Q_ERR_SHAPE;
    if (rows == 0 || K == 0) return FP8Q_OK;
    if (!row_token || !offsets || !qa || !sa || (T > 0 && (!q || !s || !row_of))) return FP8Q_ERR_NULL;
    if (!aligned16(qa) || !aligned4(sa) || !aligned4(row_token) || !aligned4(offsets) ||
        (T > 0 && (!aligned16(q) || !aligned4(s) || !aligned4(row_of))))
        return FP8Q_ERR_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    return finish(fp8q::launch_moe_gather_fp8(q, s, T, K, (int)k, row_of, row_token, offsets, (int)E, rows, qa, sa,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"
