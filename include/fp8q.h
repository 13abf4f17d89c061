/*
 * fp8q.h -- C ABI of the fine-grained FP8 quantization / block-scaled FP8 GEMM
 * library for AMD Instinct MI355X (gfx950).
 *
 * The method (page "The Definitive Information To Deepseek", DeepSeek-V3's FP8
 * mixed-precision framework):
 *   - activations are scaled and quantized online per 1x128 tile (one token,
 *     128 consecutive channels), weights per 128x128 block (the passage that
 *     refers to Figure 7 (a));
 *   - the scale of a group is derived from the group and the group is then
 *     encoded in FP8 (the passage on caching the Linear input in FP8); this
 *     library reads it as scale = fl32(amax / 448) with OCP E4M3 codes, round
 *     to nearest even, saturating at +-448;
 *   - the GEMMs take FP8 operands and produce BF16 or FP32 (the passage on the
 *     GEMM inputs and outputs), and partial sums are promoted into an FP32
 *     accumulator with the per-block scales (the passage on promotion running
 *     beside the MMA on H800); the promotion interval here is every 128
 *     elements of K.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major
 *     and contiguous, with base addresses aligned to 16 bytes unless an entry
 *     point states a weaker rule.  The library never allocates, frees or
 *     synchronizes.
 *   - bf16 tensors are passed as uint16_t bit patterns.  FP8 tensors are
 *     uint8_t OCP E4M3 codes (0x7F / 0xFF are NaN and never produced).
 *   - Scales are fp32.  Activation scales s_a have layout [K/128][M]
 *     (K-block-major: element (kb, m) at s_a[kb * M + m]).  Weight scales s_w
 *     have layout [N/128][K/128] (element (nb, kb) at s_w[nb * (K/128) + kb]).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously on it; results are visible after the caller
 *     synchronizes that stream.  The same inputs always give bit-identical
 *     outputs.
 *   - Every call validates its arguments and the current device before any
 *     launch and returns FP8Q_OK or a negative fp8q_status.  On error nothing
 *     is launched and no output is touched.  A launch failure reported by the
 *     runtime returns FP8Q_ERR_HIP.  Faults during execution (for example a
 *     host pointer passed as a device pointer) surface at the caller's
 *     synchronization, as for any HIP kernel.
 *   - Finite inputs are a precondition.  Shapes are int64_t.  M may be any
 *     value >= 0 (M == 0 launches nothing); K and N must be multiples of 128
 *     unless an entry point states otherwise.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8Q_OK = 0,
    FP8Q_ERR_NULL = -1,               /* a required pointer is NULL */
    FP8Q_ERR_SHAPE = -2,              /* negative size, or K / N not a multiple of 128, or bad group layout */
    FP8Q_ERR_ALIGN = -3,              /* a tensor base address is not 16-byte aligned */
    FP8Q_ERR_DTYPE = -4,              /* unknown output dtype */
    FP8Q_ERR_NO_DEVICE = -5,          /* no HIP device is available */
    FP8Q_ERR_UNSUPPORTED_DEVICE = -6, /* the current device is not gfx950 */
    FP8Q_ERR_HIP = -7,                /* the HIP runtime reported an error at launch */
    FP8Q_ERR_WORKSPACE = -8           /* the workspace is smaller than the call needs */
} fp8q_status;

typedef enum { FP8Q_OUT_BF16 = 0, FP8Q_OUT_F32 = 1 } fp8q_out_dtype;

/* 1x128 activation quantization (the Figure 7 (a) passage: per token per 128
 * channels).
 *   x  : bf16 [M, K]            (input)
 *   q  : E4M3 [M, K]            (output)
 *   s  : fp32 [K/128][M]        (output; s[kb*M + m] = fl32(max_k |x[m, kb*128+k]| / 448))
 * q[m,k] = E4M3_RNE_saturating(fl32(x[m,k] / s)), or a signed zero when s == 0.
 * Requires M >= 0, K >= 0, K % 128 == 0. */
int fp8q_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, void *stream);

/* FP4 quantization in the FP8 groupings (page "DeepSeek starts updating
 * frequently", the list of TileKernels features: the quantization kernels
 * convert to FP8, FP4 or E5M6).  The pages name FP4 only; this library reads it
 * as OCP E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6) with the FP8 groups and scale = fl32(amax / 6):
 *   q = E2M1_RNE_saturating(fl32(x / s)), -0 -> code 0x8, two codes a byte,
 *   element 2i in the low nibble and 2i+1 in the high nibble.
 * Activations (1x128):  x bf16 [M, K] -> q [M, K/2] bytes, s fp32 [K/128][M]
 * Weights (128x128):    w bf16 [N, K] -> q [N, K/2] bytes, s fp32 [N/128][K/128]
 * Requires K % 128 == 0 (and N % 128 == 0 for weights), 16-byte aligned
 * pointers. */
int fp8q_quant_act_fp4_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, void *stream);
int fp8q_quant_w_fp4_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, void *stream);

/* E5M6 activation quantization (page "The Definitive Information To Deepseek",
 * the customized E5M6 format for certain activations; page "DeepSeek starts
 * updating frequently", the TileKernels conversion to FP8, FP4 or E5M6).  The
 * pages give the name only; this library reads E5M6 as sign, 5 exponent bits
 * (bias 15), 6 mantissa bits, subnormals m * 2^-20, exponent 31 reserved
 * (largest finite 65024), in the 1x128 activation groups:
 *   x  : bf16 [M, K]            (input)
 *   q  : [M, 3K/2] bytes        (output: 12-bit codes as a little-endian bit
 *        stream, element j at bits 12j..12j+11 of its row)
 *   s  : fp32 [K/128][M]        (output; s = fl32(amax / 65024))
 * code = E5M6_RNE_saturating(fl32(x / s)), sign kept (-0 -> 0x800).
 * Requires M >= 0, K % 128 == 0, 16-byte aligned pointers. */
int fp8q_quant_act_e5m6_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, void *stream);

/* Per-channel FP8 weight quantization (page "DeepSeek starts updating
 * frequently", the list of TileKernels features: per-token, per-block and
 * per-channel modes).  This library reads the per-channel mode as one scale
 * per output channel, i.e. per row of W over the whole of K:
 *   w  : bf16 [N, K]            (input)
 *   q  : E4M3 [N, K]            (output)
 *   s  : fp32 [N]               (output; s[n] = fl32(max_k |w[n,k]| / 448))
 * q[n,k] = E4M3_RNE_saturating(fl32(w[n,k] / s[n])), or a signed zero when
 * s[n] == 0.  Requires N >= 0, K >= 0, K % 8 == 0, 16-byte aligned w and q,
 * 4-byte aligned s; with K == 0, w and q may be null and s is set to 0. */
int fp8q_quant_w_per_channel(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, void *stream);

/* Forward and backward FP8 copies of a Linear input in one pass (page "The
 * Definitive Information To Deepseek", the passage on caching the Linear's
 * input in FP8 for the backward pass).  The backward pass contracts the input
 * over tokens (dW = dY^T x), so its FP8 copy needs groups along tokens; this
 * library reads it as the 1x128 quantization of x^T (one scale per channel and
 * 128 tokens), made from the same bf16 x:
 *   x  : bf16 [M, K]            (input)
 *   q  : E4M3 [M, K], s : fp32 [K/128][M]     (output: exactly fp8q_quant_act_1x128)
 *   qt : E4M3 [K, M] (channel-major), st : fp32 [M/128][K]   (output)
 *   qt[k,m] = E4M3_RNE_saturating(fl32(x[m,k] / st[m/128][k])),
 *   st[mb][k] = fl32(max_{m in block mb} |x[m,k]| / 448).
 * Requires M % 128 == 0, K % 128 == 0, 16-byte aligned pointers. */
int fp8q_quant_act_dual(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, uint8_t *qt, float *st,
                        void *stream);

/* Fused SwiGLU + 1x128 activation quantization (page "DeepSeek starts updating
 * frequently", the list of TileKernels features: the quantization kernels
 * combine SwiGLU with quantization).  The pages do not give the arithmetic;
 * this library reads SwiGLU as the FFN's gated unit and fixes one rounding:
 *   h[m,k] = bf16_RNE( SiLU(x[m,k]) * y[m,k] ),  SiLU(x) = x / (1 + e^-x),
 * the exact value rounded once to bf16 (so the result does not depend on how
 * exp is implemented), then q, s = the 1x128 quantization of h exactly as
 * fp8q_quant_act_1x128 computes it.  h is never written to memory.
 *   x  : bf16 gate [M, K], rows ld elements apart   (input)
 *   y  : bf16 up   [M, K], rows ld elements apart   (input; x and y may be the
 *        two halves of one [M, 2K] tensor: y = x + K, ld = 2K)
 *   q  : E4M3 [M, K]            (output)
 *   s  : fp32 [K/128][M]        (output)
 * Requires M >= 0, K % 128 == 0, ld >= K, ld % 8 == 0, 16-byte aligned
 * pointers.  Finite inputs whose h stays in the bf16 range are a
 * precondition. */
int fp8q_swiglu_quant_act_1x128(const uint16_t *x, const uint16_t *y, int64_t ld, int64_t M, int64_t K, uint8_t *q,
                                float *s, void *stream);

/* The SwiGLU intermediate alone, h = bf16_RNE(SiLU(x) * y) as above, written
 * out (the value fp8q_swiglu_quant_act_1x128 quantizes without storing it):
 *   x, y : bf16 [M, K], rows ld elements apart (inputs);  h : bf16 [M, K] (output)
 * Requires M >= 0, K % 8 == 0, ld >= K, ld % 8 == 0, 16-byte aligned pointers. */
int fp8q_swiglu_bf16(const uint16_t *x, const uint16_t *y, int64_t ld, int64_t M, int64_t K, uint16_t *h, void *stream);

/* 128x128 weight quantization (the Figure 7 (a) passage: per 128 input
 * channels per 128 output channels).
 *   w  : bf16 [N, K]            (input; an expert stack [E][N', K] is passed as N = E * N')
 *   q  : E4M3 [N, K]            (output)
 *   s  : fp32 [N/128][K/128]    (output; the block's fl32(amax / 448))
 * Requires N % 128 == 0, K % 128 == 0. */
int fp8q_quant_w_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, void *stream);

/* FP8 -> BF16 weight conversion with 128x128 block scales (page
 * "deepseek-ai/DeepSeek-V3", "How to Run Locally": the weights are published in
 * FP8, with a script that converts them to BF16).  The pages do not give the
 * arithmetic; this library reads it as every code times its block's scale in
 * fp32, rounded to bf16 to nearest even:
 *   w[n,k] = bf16(fl32(E4M3(q[n,k]) * s[n/128][k/128]))
 *   q : E4M3 [N, K]             (input; an expert stack [E][N', K] is passed as N = E * N')
 *   s : fp32 [N/128][K/128]     (input)
 *   w : bf16 [N, K]             (output, as uint16_t bit patterns)
 * Requires N % 128 == 0, K % 128 == 0.  Codes 0x7F / 0xFF (NaN) are outside the
 * contract (the quantizers never produce them); they convert to NaN. */
int fp8q_dequant_w_128x128(const uint8_t *q, const float *s, int64_t N, int64_t K, uint16_t *w, void *stream);

/* Block-scaled FP8 GEMM, the Linear y = x W^T (the passages on FP8 GEMM inputs
 * with BF16/FP32 outputs and on FP32 promotion):
 *   C[m,n] = sum_kb  s_a[kb][m] * s_w[n/128][kb] * (sum_{k in kb} qa[m,k] * qw[n,k])
 * with each 128-element partial sum promoted into an fp32 accumulator.
 *   qa : E4M3 [M, K],  sa : fp32 [K/128][M]
 *   qw : E4M3 [N, K],  sw : fp32 [N/128][K/128]
 *   c  : [M, N] bf16 (out_dtype FP8Q_OUT_BF16, round to nearest even) or fp32 (FP8Q_OUT_F32)
 * Requires M >= 0, N % 128 == 0, K % 128 == 0, 128 <= K <= 2^23.
 * Range: each promotion multiplies by s_a * s_w formed in fp32 and adds into an
 * fp32 sum, so the result is accurate while every such product and every running
 * sum is finite in fp32 (for scales from the quantizers the products are finite
 * when amax_a * amax_w <= 448^2 * FLT_MAX, about 6.8e43); past that the output may
 * be +-inf or NaN.  The same holds for the grouped GEMMs below. */
int fp8q_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                          int out_dtype, int64_t M, int64_t N, int64_t K, void *stream);

/* Grouped block-scaled FP8 GEMM for MoE experts.  Each routed expert applies
 * its own Linear to the tokens sent to it (page "The Definitive Information To
 * Deepseek", the passages on the MoE models' all-to-all communication, where
 * each token goes to a few experts spread over nodes); the tokens are mapped to
 * experts and laid out expert by expert beforehand (page "DeepSeek starts
 * updating frequently", the TileKernels feature list: MoE routing maps tokens
 * to experts), so each expert's Linear is one contiguous segment of rows.  The
 * GEMM of every segment is the block-scaled FP8 GEMM above with that expert's
 * weight and block scales; the token-to-expert layout is the caller's:
 *   rows [off[e], off[e+1]) of A are multiplied by expert e's weight.
 *   qa  : E4M3 [M_total, K],      sa : fp32 [K/128][M_total]
 *   qw  : E4M3 [E][N][K],         sw : fp32 [E][N/128][K/128]
 *   off : DEVICE int32 [E+1], non-decreasing, off[0] = 0, off[E] <= M_total,
 *         every off[e] a multiple of 128 (segments padded to 128 rows; empty
 *         experts allowed).  Padding rows should carry codes 0 and scale 0 and
 *         then produce exact zeros.  Rows [off[E], M_total) are not written, so
 *         M_total may be the capacity of a routing layout
 *         (fp8q_moe_route_capacity) without reading off[E] back to the host.
 *   c   : [M_total, N] bf16 or fp32.
 * Requires E >= 1, M_total % 128 == 0, N % 128 == 0, K % 128 == 0, 128 <= K <= 2^23.
 * The offsets live on the device and are not checked on the host.  Offsets that
 * never decrease but break the other rules (segments that are not multiples of
 * 128 rows, off[0] > 0, offsets past M_total) are cut to [0, M_total): every row
 * a cut segment covers is computed with that segment's expert, and the rows no
 * segment covers are left unwritten (c keeps its previous contents there).  When
 * the offsets decrease somewhere, segments may overlap and the output rows are
 * unspecified.  In every case each memory access stays inside the buffers
 * described by M_total, E, N and K. */
int fp8q_grouped_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                                  int out_dtype, const int32_t *off, int64_t E, int64_t M_total, int64_t N,
                                  int64_t K, void *stream);

/* The grouped GEMM with the FP8 dispatch folded in (page "DeepSeek starts
 * updating frequently": DeepEP V2 dispatches tokens in FP8 to the experts'
 * GEMMs).  Instead of a gathered A, the GEMM reads each row's token directly:
 * row r of the expert-sorted layout is token row_token[r] of the quantized
 * tokens, exactly as if fp8q_moe_gather_fp8 had copied it there first (the
 * results are identical):
 *   q   : E4M3 [T, K] token codes,  s : fp32 [K/128][T] token scales
 *   row_token : DEVICE int32 [M_total]; a value outside [0, T) (the routing's
 *         -1) is an empty row: codes 0, scale 0, output exactly 0
 *   qw, sw, off, c, out_dtype, E, M_total, N, K : as fp8q_grouped_gemm_blockscaled
 * Requires what fp8q_grouped_gemm_blockscaled requires, plus T >= 0 and
 * T * K < 2^31; q and s may be null when T == 0.  The same guarantees hold
 * for offsets that break the rules. */
int fp8q_grouped_gemm_blockscaled_gather(const uint8_t *q, const float *s, int64_t T, const int32_t *row_token,
                                         const uint8_t *qw, const float *sw, void *c, int out_dtype,
                                         const int32_t *off, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                         void *stream);

/* Human-readable text for a status code (static storage; never NULL). */
const char *fp8q_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int fp8q_version(void);

/* ---------------------------------------------------------------------------
 * MoE routing and the FP8 row gather that feed the grouped GEMM (page "DeepSeek
 * starts updating frequently", deepinsightai.io, the list of TileKernels
 * features: a gating step selects each token's top-k experts and a routing
 * step maps tokens to experts; the same page's DeepEP V2 test dispatches 8K
 * tokens of hidden size 7168 to their top 8 experts in FP8).  The pages fix
 * neither the tie rule nor the layout; this library takes:
 *   - token t selects the k experts with the largest logits, listed by
 *     decreasing logit; between equal logits (-0 equals +0) the lower expert
 *     index comes first;
 *   - expert e owns rows [offsets[e], offsets[e+1]), its tokens in ascending
 *     order followed by empty rows up to a multiple of 128; segments follow
 *     each other in expert order from row 0;
 *   - an empty row carries codes 0 and scale 0 (the grouped GEMM then writes
 *     exact zeros for it).
 * ------------------------------------------------------------------------- */

/* Rows that any routing of T tokens to k of E experts fits in: T*k + 127*E,
 * rounded up to a multiple of 128.  Returns -1 for invalid sizes. */
int64_t fp8q_moe_route_capacity(int64_t T, int64_t E, int64_t k);

/* Bytes of device workspace fp8q_moe_route_topk needs: 4 * E * ceil(T / 64).
 * Returns -1 for invalid sizes. */
int64_t fp8q_moe_route_workspace_bytes(int64_t T, int64_t E);

/* Top-k gating and the expert-sorted layout, on the device:
 *   logits    : fp32 [T][E] (input, finite; NaN gives unspecified experts)
 *   topk_idx  : int32 [T][k] (output) token t's experts, best first
 *   offsets   : int32 [E+1] (output) segment starts, offsets[E] = rows in use
 *   row_of    : int32 [T][k] (output) the row that carries (t, topk_idx[t][j])
 *   row_token : int32 [rows] (output) the token of each row, -1 for empty rows
 *               and for every row from offsets[E] on
 *   rows      : length of row_token; must be >= fp8q_moe_route_capacity(T,E,k)
 *   workspace : device memory of workspace_bytes bytes, caller-owned, 4-byte
 *               aligned; its contents on entry do not matter and are
 *               overwritten (calls that share one workspace must not overlap)
 * Requires T >= 0, 1 <= E <= 1024, 1 <= k <= min(E, 16), rows <= 2^31 - 1,
 * 4-byte aligned pointers.  Returns FP8Q_ERR_WORKSPACE when workspace_bytes is
 * smaller than fp8q_moe_route_workspace_bytes(T, E).  Three launches on
 * `stream`; deterministic. */
int fp8q_moe_route_topk(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *topk_idx, int32_t *offsets,
                        int32_t *row_of, int32_t *row_token, int64_t rows, void *workspace, int64_t workspace_bytes,
                        void *stream);

/* fp8q_moe_route_topk for callers that cannot allocate device memory (code
 * being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the same outputs, bit for bit, with the workspace taken from a
 * fixed array inside the library instead of from the caller.  The array holds
 * FP8Q_MOE_ROUTE_NOALLOC_BYTES bytes on each GPU the library runs on and is
 * kept until the process ends; its device address is looked up on the first
 * call on each device.  This call allocates and frees nothing.
 *   logits, topk_idx, offsets, row_of, row_token, rows : as fp8q_moe_route_topk
 * Requires what fp8q_moe_route_topk requires (without its workspace
 * arguments), and fp8q_moe_route_workspace_bytes(T, E) <=
 * FP8Q_MOE_ROUTE_NOALLOC_BYTES (4 * E * ceil(T / 64) <= 4 MiB: for example
 * up to 65536 tokens over 1024 experts, or 262144 tokens over 256); larger
 * calls return FP8Q_ERR_WORKSPACE before any launch.
 * Every call on one GPU shares that GPU's array, so calls that overlap on one
 * GPU (concurrent streams, or threads without ordering between their streams)
 * race and give unspecified outputs; calls ordered on one stream are safe.  The
 * array needs no clearing: every entry a call reads was written earlier in the
 * same call.  Returns FP8Q_ERR_HIP if the array's address cannot be obtained. */
#define FP8Q_MOE_ROUTE_NOALLOC_BYTES (4 * 1024 * 1024)
int fp8q_moe_route_topk_noalloc(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *topk_idx,
                                int32_t *offsets, int32_t *row_of, int32_t *row_token, int64_t rows, void *stream);

/* Expert-sorted FP8 activations for the grouped GEMM (FP8 dispatch): for every
 * row r < min(offsets[E], rows),
 *   qa[r, :] = q[row_token[r], :],  sa[kb][r] = s[kb][row_token[r]]
 * or zero codes and scale 0 when row_token[r] is -1 (or outside [0, T)).
 *   q  : E4M3 [T, K], s : fp32 [K/128][T]   (fp8q_quant_act_1x128 of the tokens)
 *   row_of [T][k], row_token [rows], offsets [E+1] : the outputs of one
 *        fp8q_moe_route_topk call (device); the codes of a token's rows are
 *        written through row_of (each token row is read once), the scales and
 *        the empty rows through row_token, so the two must describe the same
 *        layout
 *   qa : E4M3 [rows, K], sa : fp32 [K/128][rows]   (outputs)
 * Rows from offsets[E] on are not written.  Gathering quantized rows equals
 * quantizing gathered bf16 rows bit for bit (a 1x128 group lies in one row).
 * Requires 0 <= T <= 2^31 - 1, K % 128 == 0, k >= 1 with T*k < 2^31, E >= 1,
 * 0 <= rows <= 2^31 - 1; q and qa 16-byte aligned, the other pointers 4-byte
 * aligned.  q, s and row_of may be NULL when T == 0.  One launch. */
int fp8q_moe_gather_fp8(const uint8_t *q, const float *s, int64_t T, int64_t K, int64_t k, const int32_t *row_of,
                        const int32_t *row_token, const int32_t *offsets, int64_t E, int64_t rows, uint8_t *qa,
                        float *sa, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
