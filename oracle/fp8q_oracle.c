/*
 * fp8q_oracle.c -- plain, slow CPU oracle for fine-grained FP8 quantization and
 * the block-scaled FP8 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: it exists so that tests/, the smoke check and the benchmark's CPU
 * baseline can check the HIP library against an independent definition.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * What it computes, and where that comes from:
 *
 *  - Grouping (page "The Definitive Information To Deepseek", the passage that
 *    refers to Figure 7 (a)): activations are grouped and scaled per 1x128 tile
 *    (one token, 128 consecutive channels); weights per 128x128 block (128
 *    output channels x 128 input channels).
 *  - Online scaling (same page, the passage on caching the Linear operator's
 *    input in FP8 for the backward pass): a scaling factor is derived per group
 *    and the group is then quantized to FP8 online.  The page lost what the
 *    factor is derived from; the reading taken here is the group's maximum
 *    absolute value, with scale = fl32(amax / 448), 448 being the largest
 *    finite E4M3 magnitude.
 *  - FP8 flavour: OCP 8-bit floating point E4M3 ("FN": bias 7, no infinities,
 *    S.1111.111 is NaN, largest finite 448, subnormals m * 2^-9).
 *  - Encoding: v = fl32(x / scale), then round to the nearest E4M3 value with
 *    ties to even, saturating at +-448, keeping the sign (so -0 -> 0x80).  The
 *    rounding x/s -> fp32 -> E4M3 is a double rounding on purpose: it is the
 *    definition the GPU path must reproduce bit for bit.
 *  - GEMM (same page, the passage stating that the GEMMs take FP8 inputs and
 *    produce BF16 or FP32 outputs, and the passage on promotion overlapping the
 *    MMA on H800 warpgroups): the product C = A * W^T of the dequantized
 *    operands, where every element is its E4M3 value times its group's scale.
 *    This oracle evaluates that sum in double precision, with the error scale
 *    B = sum_k |a_deq[m,k]| * |w_deq[n,k]|.  Promotion of partial sums at every
 *    128-element K interval is how a GPU reaches this value in fp32; the
 *    oracle does not model it, it computes the value itself.
 *  - FP8 -> BF16 weight conversion (page "deepseek-ai/DeepSeek-V3" on the
 *    ai.atomgit.com mirror, "How to Run Locally": only FP8 weights are
 *    published, with a script that converts them to BF16; the CSDN page lists
 *    an analysis of that conversion).  The pages do not give its arithmetic;
 *    the reading taken here is the one the GEMM's promotion uses: every code
 *    times its 128x128 block's scale in fp32, then rounded to bf16 to nearest
 *    even: w = bf16(fl32(dec(q) * s)).
 *  - MoE routing and the FP8 row gather (page "DeepSeek starts updating
 *    frequently", the list of TileKernels features: top-k gating and the
 *    token-to-expert mapping): top-k experts per token by logit, and the
 *    expert-sorted, 128-padded layout of the quantized rows that the grouped
 *    GEMM consumes.  The readings (tie rule, segment order, empty rows) are
 *    stated beside the functions at the end of this file.
 *  - FP4 (E2M1) quantization in the FP8 groupings (same page and list: the
 *    quantization kernels convert to FP8, FP4 or E5M6); readings beside the
 *    functions.
 *  - Per-channel FP8 weights (same list: per-channel mode): one scale per
 *    output channel over the whole row.
 *  - E5M6 activations (page "The Definitive Information To Deepseek", the
 *    customized E5M6 format for certain activations; the same TileKernels
 *    list): readings beside the functions.
 *  - Fused SwiGLU + 1x128 quantization (same page and list: the quantization
 *    kernels combine SwiGLU with quantization): h = bf16(SiLU(x) * y), the
 *    exact value rounded once, then the 1x128 activation quantizer on h.
 *
 * Layouts (a reading; the pages are silent): row-major, K contiguous.
 * Activation scales s_a are stored K-block-major, s_a[kb * M + m]; weight scales
 * s_w[nb * KB + kb] with nb = n / 128 and KB = K / 128.
 *
 * Precision: compiled without -ffast-math and with -ffp-contract=off, on an
 * x86-64 target where float expressions are evaluated in float, so every fp32
 * operation written here is one IEEE-754 binary32 operation.
 *
 * Pins: tests/test_oracle_*.py check this file against hand-worked E4M3 cases,
 * (for the dequantization) exact rational rounding of every code times sampled
 * scales, the power-of-two and unit-code closed forms, and a per-block scale
 * pattern, (for routing) a pairwise check of the top-k definition on random
 * and tie-heavy logits, library special cases (k = 1 is argmax, k = E a stable
 * sort), a hand-worked layout and the layout invariants, (for the gather)
 * numpy indexing and its commutation with the row-wise quantizer, (for
 * SwiGLU) 80-digit decimal arithmetic, numpy's float64 exp away from rounding
 * midpoints, hand-worked ties and signed zeros, and sign and scale symmetry,
 * the OCP closed-form code table, a brute-force nearest-value encoder over all
 * bf16 inputs, sign/scale invariants, a lossless special case equal to a
 * float64 numpy matmul, and exact rational sums on tiny shapes.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle requires float expressions to be evaluated in float"
#endif

#define GROUP 128

/* Number of threads the parallel loops below use (reported beside oracle timings). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- bf16 ---------------------------------------------------------------- */

/* A bf16 value is the upper half of an fp32 bit pattern: widening is exact. */
static float bf16_to_f32(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ---- OCP E4M3 -------------------------------------------------------------- */

/* Magnitude of a non-negative finite code 0x00..0x7E, straight from the format:
 * exponent field e (bias 7) and mantissa field m (3 bits);
 * e == 0: subnormal m/8 * 2^-6 = m * 2^-9;  e >= 1: (1 + m/8) * 2^(e-7). */
static double e4m3_magnitude(unsigned code) {
    unsigned e = (code >> 3) & 0xFu, m = code & 0x7u;
    if (e == 0) return ldexp((double)m, -9);
    return ldexp(1.0 + (double)m / 8.0, (int)e - 7);
}

double oracle_e4m3_decode(uint8_t code) {
    if ((code & 0x7Fu) == 0x7Fu) return NAN; /* S.1111.111 */
    double mag = e4m3_magnitude(code & 0x7Fu);
    return (code & 0x80u) ? -mag : mag;
}

/* Round an fp32 value to E4M3: nearest, ties to even, saturating at 448.
 * The 127 non-negative finite codes 0..126 are in increasing order of value,
 * so the code below |v| is found by bisection and the decision against the
 * midpoint of the two neighbouring values is exact in double (both the fp32
 * input and the midpoint are exactly representable). */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80u : 0x00u;
    double a = fabs((double)v);
    unsigned c;
    if (a >= 448.0) {
        c = 126; /* 0x7E = 448, the largest finite value: saturate */
    } else {
        unsigned lo = 0, hi = 126; /* invariant: value(lo) <= a < value(hi+1) */
        while (lo < hi) {
            unsigned mid = (lo + hi + 1) / 2;
            if (e4m3_magnitude(mid) <= a) lo = mid;
            else hi = mid - 1;
        }
        c = lo;
        if (c < 126) {
            double half = (e4m3_magnitude(c) + e4m3_magnitude(c + 1)) / 2.0;
            if (a > half || (a == half && (c & 1u))) c += 1; /* tie: even code */
        }
    }
    return (uint8_t)(sign | c);
}

/* The encoder applied element-wise to an array (for tests over many inputs). */
void oracle_e4m3_encode_array(const float *v, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(v[i]);
}

/* Encode one value x of a group whose scale is s (s >= 0). */
static uint8_t quantize_one(float x, float s) {
    if (s == 0.0f) return signbit(x) ? 0x80u : 0x00u; /* all-zero group */
    return oracle_e4m3_encode(x / s);
}

/* ---- quantizers -------------------------------------------------------------
 * Return 0 on success, -1 for bad shapes, -2 if a non-finite input was seen
 * (finite input is a precondition; outputs are then unspecified). */

int oracle_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s) {
    if (M < 0 || K < 0 || K % GROUP) return -1;
    int64_t KB = K / GROUP;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            const uint16_t *g = x + m * K + kb * GROUP;
            float amax = 0.0f;
            for (int j = 0; j < GROUP; j++) {
                float v = bf16_to_f32(g[j]);
                if (!isfinite(v)) bad = 1;
                float av = fabsf(v);
                if (av > amax) amax = av;
            }
            float scale = amax / 448.0f;
            s[kb * M + m] = scale;
            for (int j = 0; j < GROUP; j++) q[m * K + kb * GROUP + j] = quantize_one(bf16_to_f32(g[j]), scale);
        }
    }
    return bad ? -2 : 0;
}

int oracle_quant_w_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s) {
    if (N < 0 || K < 0 || N % GROUP || K % GROUP) return -1;
    int64_t NB = N / GROUP, KB = K / GROUP;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
    for (int64_t nb = 0; nb < NB; nb++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            float amax = 0.0f;
            for (int64_t i = 0; i < GROUP; i++) {
                const uint16_t *row = w + (nb * GROUP + i) * K + kb * GROUP;
                for (int j = 0; j < GROUP; j++) {
                    float v = bf16_to_f32(row[j]);
                    if (!isfinite(v)) bad = 1;
                    float av = fabsf(v);
                    if (av > amax) amax = av;
                }
            }
            float scale = amax / 448.0f;
            s[nb * KB + kb] = scale;
            for (int64_t i = 0; i < GROUP; i++) {
                int64_t off = (nb * GROUP + i) * K + kb * GROUP;
                for (int j = 0; j < GROUP; j++) q[off + j] = quantize_one(bf16_to_f32(w[off + j]), scale);
            }
        }
    }
    return bad ? -2 : 0;
}

/* ---- FP8 -> BF16 block dequantization ----------------------------------------
 * Round a finite fp32 value to the nearest bf16 (ties to even): keep the upper
 * 16 bits after adding half of the dropped part, with the tie going to the even
 * upper half. */
static uint16_t f32_to_bf16(float v) {
    uint32_t u;
    memcpy(&u, &v, 4);
    const uint32_t lower = u & 0xFFFFu, upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) return (uint16_t)(upper + 1u);
    return (uint16_t)upper;
}

/* w[n][k] = bf16(fl32(dec(q[n][k]) * s[n/128][k/128])).  The product of a code
 * (at most 4 significant bits) and an fp32 scale (24) is exact in double, so
 * converting it to float rounds once, as an fp32 multiply would. */
int oracle_dequant_w_128x128(const uint8_t *q, const float *s, int64_t N, int64_t K, uint16_t *w) {
    if (N < 0 || K < 0 || N % GROUP || K % GROUP) return -1;
    int64_t KB = K / GROUP;
    for (int64_t i = 0; i < N * K; i++)
        if ((q[i] & 0x7Fu) == 0x7Fu) return -2; /* NaN code */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            const double exact = oracle_e4m3_decode(q[n * K + k]) * (double)s[(n / GROUP) * KB + k / GROUP];
            w[n * K + k] = f32_to_bf16((float)exact);
        }
    return 0;
}

/* ---- block-scaled GEMM ------------------------------------------------------
 * C[m,n] = sum_k (dec(qa[m,k]) * s_a[k/128][m]) * (dec(qw[n,k]) * s_w[n/128][k/128])
 * evaluated in double for an explicit list of (m, n) output elements, together
 * with B[m,n] = sum_k |dec(qa[m,k]) * s_a| * |dec(qw[n,k]) * s_w|. */

static double dot_dequant(const uint8_t *qa_row, const float *sa, int64_t M, int64_t m, const uint8_t *qw_row,
                          const float *sw_rowblock, int64_t K, double *bound) {
    double c = 0.0, b = 0.0;
    for (int64_t k = 0; k < K; k++) {
        int64_t kb = k / GROUP;
        double a_deq = oracle_e4m3_decode(qa_row[k]) * (double)sa[kb * M + m];
        double w_deq = oracle_e4m3_decode(qw_row[k]) * (double)sw_rowblock[kb];
        c += a_deq * w_deq;
        b += fabs(a_deq) * fabs(w_deq);
    }
    *bound = b;
    return c;
}

int oracle_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, int64_t M,
                            int64_t N, int64_t K, const int64_t *ms, const int64_t *ns, int64_t count, double *C,
                            double *B) {
    if (M < 0 || N < 0 || K < 0 || N % GROUP || K % GROUP) return -1;
    for (int64_t i = 0; i < count; i++)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return -1;
    int64_t KB = K / GROUP;
#pragma omp parallel for schedule(dynamic, 256)
    for (int64_t i = 0; i < count; i++) {
        int64_t m = ms[i], n = ns[i];
        C[i] = dot_dequant(qa + m * K, sa, M, m, qw + n * K, sw + (n / GROUP) * KB, K, &B[i]);
    }
    return 0;
}

/* Grouped (MoE) variant: rows [off[e], off[e+1]) of A belong to expert e and
 * use W_e = qw[e] ([N][K]) with scales sw[e] ([N/128][K/128]).  The offsets are
 * non-decreasing with off[0] = 0 and off[E] = M_total. */
int oracle_grouped_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw,
                                    const int32_t *off, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                    const int64_t *ms, const int64_t *ns, int64_t count, double *C, double *B) {
    if (E < 1 || M_total < 0 || N < 0 || K < 0 || N % GROUP || K % GROUP) return -1;
    if (off[0] != 0 || off[E] != M_total) return -1;
    for (int64_t e = 0; e < E; e++)
        if (off[e + 1] < off[e]) return -1;
    for (int64_t i = 0; i < count; i++)
        if (ms[i] < 0 || ms[i] >= M_total || ns[i] < 0 || ns[i] >= N) return -1;
    int64_t KB = K / GROUP, NB = N / GROUP;
#pragma omp parallel for schedule(dynamic, 256)
    for (int64_t i = 0; i < count; i++) {
        int64_t m = ms[i], n = ns[i];
        int64_t e = 0;
        while (!(off[e] <= m && m < off[e + 1])) e++; /* the segment holding row m */
        const uint8_t *w_e = qw + e * N * K;
        const float *s_e = sw + e * NB * KB;
        C[i] = dot_dequant(qa + m * K, sa, M_total, m, w_e + n * K, s_e + (n / GROUP) * KB, K, &B[i]);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * MoE routing and the FP8 row gather (page "DeepSeek starts updating
 * frequently" on deepinsightai.io, the list of TileKernels features: a gating
 * step selects each token's top-k experts, and a routing step maps tokens to
 * experts; the same page's DeepEP V2 test uses 8K tokens, hidden 7168, the top
 * 8 experts and FP8 dispatch).  The pages fix neither the tie rule nor the
 * expert-sorted layout.  Readings taken here:
 *  - token t selects the k experts with the largest logits, listed by
 *    decreasing logit; of two equal logits (numerically: -0 equals +0) the
 *    lower expert index comes first;
 *  - expert e owns one segment of rows holding its tokens in ascending token
 *    order, padded with empty rows to a multiple of `pad` (128: the 128-row
 *    granularity of the grouped GEMM's scales and tiles); the segments follow
 *    each other in expert order from row 0;
 *  - an empty row carries all-zero codes and scale 0.
 * ------------------------------------------------------------------------- */

/* logits fp32 [T][E] (finite).  Outputs: topk_idx int32 [T][k]; offsets int32
 * [E+1] (segment e is rows [offsets[e], offsets[e+1])); row_of int32 [T][k]
 * (the row that carries token t's j-th expert); row_token int32 [rows] (the
 * token a row carries, -1 for empty rows and for rows past offsets[E]).
 * Returns 0, -1 for bad sizes, -2 for a non-finite logit, -3 when `rows` is
 * smaller than the layout. */
int oracle_moe_route_topk(const float *logits, int64_t T, int64_t E, int64_t k, int64_t pad, int32_t *topk_idx,
                          int32_t *offsets, int32_t *row_of, int32_t *row_token, int64_t rows) {
    if (T < 0 || E < 1 || E > 4096 || k < 1 || k > E || pad < 1 || rows < 0) return -1;
    for (int64_t i = 0; i < T * E; i++)
        if (!isfinite(logits[i])) return -2;
    unsigned char chosen[E];
    for (int64_t t = 0; t < T; t++) {
        const float *v = logits + t * E;
        memset(chosen, 0, sizeof chosen);
        for (int64_t j = 0; j < k; j++) {
            /* the largest logit not chosen yet; scanning upwards with a strict
             * comparison keeps the lower index among equal logits */
            int64_t best = -1;
            for (int64_t e = 0; e < E; e++)
                if (!chosen[e] && (best < 0 || v[e] > v[best])) best = e;
            chosen[best] = 1;
            topk_idx[t * k + j] = (int32_t)best;
        }
    }
    int64_t count[E];
    for (int64_t e = 0; e < E; e++) count[e] = 0;
    for (int64_t i = 0; i < T * k; i++) count[topk_idx[i]]++;
    offsets[0] = 0;
    int64_t end = 0;
    for (int64_t e = 0; e < E; e++) {
        end += (count[e] + pad - 1) / pad * pad;
        if (end > INT32_MAX) return -1;
        offsets[e + 1] = (int32_t)end;
    }
    if (rows < end) return -3;
    for (int64_t r = 0; r < rows; r++) row_token[r] = -1;
    int64_t next[E];
    for (int64_t e = 0; e < E; e++) next[e] = offsets[e];
    for (int64_t t = 0; t < T; t++) /* ascending tokens: each segment fills in token order */
        for (int64_t j = 0; j < k; j++) {
            int64_t e = topk_idx[t * k + j];
            int64_t r = next[e]++;
            row_of[t * k + j] = (int32_t)r;
            row_token[r] = (int32_t)t;
        }
    return 0;
}

/* Expert-sorted FP8 activations: row r of qa (and of the scales sa, K-block-major
 * [K/128][rows]) is token row_token[r]'s row of q / s (s: [K/128][T]), or
 * all-zero codes with scale 0 when row_token[r] is -1.  Returns -1 for bad
 * sizes or a token index outside [-1, T). */
int oracle_moe_gather_fp8(const uint8_t *q, const float *s, int64_t T, int64_t K, const int32_t *row_token,
                          int64_t rows, uint8_t *qa, float *sa) {
    if (T < 0 || K < 0 || K % GROUP || rows < 0) return -1;
    for (int64_t r = 0; r < rows; r++)
        if (row_token[r] < -1 || row_token[r] >= T) return -1;
    int64_t KB = K / GROUP;
    for (int64_t r = 0; r < rows; r++) {
        int64_t t = row_token[r];
        for (int64_t k = 0; k < K; k++) qa[r * K + k] = t >= 0 ? q[t * K + k] : 0;
        for (int64_t kb = 0; kb < KB; kb++) sa[kb * rows + r] = t >= 0 ? s[kb * T + t] : 0.0f;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Fused SwiGLU + 1x128 quantization (page "DeepSeek starts updating
 * frequently", the list of TileKernels features: the quantization kernels
 * combine SwiGLU with quantization).  SwiGLU is read as the gated unit of the
 * FFN, h = SiLU(x) * y with SiLU(x) = x / (1 + e^-x), x the gate and y the up
 * projection, both bf16.  The pages fix no precision for h; the reading taken
 * here is the exact real value rounded once to bf16 to nearest even (then the
 * 1x128 quantizer above runs on h).  Unlike an fp32 formula, this does not
 * depend on how exp is implemented.
 *
 * Evaluation: x*y is exact in double; e^-x, 1 + e^-x and the division add a
 * few units in the last place, far below a bf16 spacing.  A value whose double
 * lies within 2^-45 (relative) of a bf16 rounding midpoint is not decided
 * here, with one exception: when 1 + e^-x rounds to exactly 1 and x*y is
 * itself a midpoint, the true value lies strictly between the midpoint and
 * the neighbour towards zero (e^-x > 0 and e^-x < 2^-53), so it rounds
 * towards zero.  The others are flagged for the caller to settle in higher
 * precision.
 * ------------------------------------------------------------------------- */

/* Rounding of the double v (finite, below the bf16 overflow threshold) to bf16: mode 0 to nearest even,
 * -1 to the neighbour towards zero, +1 to the neighbour away from zero (modes +-1 only matter when v is
 * not itself a bf16 value).  *near_tie gets 1 when v lies within `margin` (relative) of a rounding
 * midpoint, *mid 1 when v is exactly one. */
static uint16_t bf16_round_double(double v, int mode, double margin, int *near_tie, int *mid) {
    *near_tie = 0;
    *mid = 0;
    if (v == 0.0) return signbit(v) ? 0x8000u : 0x0000u;
    double a = fabs(v);
    int e;
    frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1): the binade's exponent is e - 1 */
    int ex = e - 1;
    if (ex < -126) ex = -126; /* bf16 subnormals share the spacing 2^-133 */
    double ulp = ldexp(1.0, ex - 7);
    double q = a / ulp; /* exact: a power-of-two scaling */
    double fl = floor(q);
    double rem = q - fl;
    if (fabs(rem - 0.5) * ulp <= margin * a) *near_tie = 1;
    if (rem == 0.5) *mid = 1;
    if (mode == 0) {
        if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    } else if (mode > 0 && rem > 0.0) {
        fl += 1.0;
    }
    float r = (float)(fl * ulp); /* a bf16 value: exact in float */
    uint32_t bits;
    memcpy(&bits, &r, 4);
    bits >>= 16;
    if (signbit(v)) bits |= 0x8000u;
    return (uint16_t)bits;
}

/* h[i] = bf16(SiLU(x[i]) * y[i]) for bf16 x, y.  amb[i] = 1 marks a value this
 * function could not decide (h[i] then holds the double's rounding).  Returns
 * 0, or -2 for a non-finite input or a result past the bf16 range.
 *
 * Values within 2^-45 of a midpoint m are settled exactly in two cases, which
 * cover every such value with x*y in the bf16 range (an exhaustive check over
 * all x and y significands confirms it):
 *  - x > 16: e^-x < 2^-23, so the true value lies less than 2^-23 inside x*y; if
 *    x*y is itself the midpoint, the value lies just inside it, above the
 *    neighbour towards zero (midpoints are 2^-9 or more from their neighbours);
 *  - |x| < 2^-40: SiLU(x) * y = (x*y/2)(1 + x/2 + ...), so the true value lies
 *    within 2^-40 of x*y/2, beyond it (away from zero) when x > 0 and inside
 *    it when x < 0; if x*y/2 is the midpoint, that side decides. */
int oracle_swiglu_bf16(const uint16_t *x, const uint16_t *y, int64_t n, uint16_t *h, uint8_t *amb) {
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t i = 0; i < n; i++) {
        double xv = (double)bf16_to_f32(x[i]), yv = (double)bf16_to_f32(y[i]);
        if (!isfinite(xv) || !isfinite(yv)) {
            bad = 1;
            continue;
        }
        double p = xv * yv; /* exact: two 8-bit significands */
        double v = p / (1.0 + exp(-xv));
        if (!isfinite(v) || fabs(v) >= 3.3961775292304e38 /* the bf16 overflow threshold */) {
            bad = 1;
            continue;
        }
        int near_tie, mid, nt2, pmid;
        uint16_t r = bf16_round_double(v, 0, 0x1p-45, &near_tie, &mid);
        amb[i] = 0;
        if (near_tie) {
            if (xv > 16.0 && (bf16_round_double(p, 0, 0.0, &nt2, &pmid), pmid)) {
                r = bf16_round_double(p, -1, 0.0, &nt2, &pmid);
            } else if (fabs(xv) < 0x1p-40 && (bf16_round_double(p / 2, 0, 0.0, &nt2, &pmid), pmid)) {
                r = bf16_round_double(p / 2, xv > 0 ? 1 : -1, 0.0, &nt2, &pmid);
            } else {
                amb[i] = 1;
            }
        }
        h[i] = r;
    }
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------------------
 * FP4 quantization (page "DeepSeek starts updating frequently", the list of
 * TileKernels features: the quantization kernels convert to FP8, FP4 or E5M6
 * in per-token, per-block and per-channel modes).  The pages name FP4 and
 * nothing more.  Readings taken here:
 *  - FP4 is OCP E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; the
 *    magnitudes of codes 0..7 are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (no inf or NaN);
 *  - the groups are the FP8 ones (1x128 per token, 128x128 per weight block),
 *    with scale = fl32(amax / 6), 6 being the largest E2M1 magnitude;
 *  - v = fl32(x / s) is rounded to the nearest E2M1 value, ties to the even
 *    code, saturating at 6, keeping the sign (-0 -> 0x8);
 *  - two codes per byte, element 2i in the low nibble and 2i+1 in the high
 *    one (the OCP packing order), rows of K/2 bytes.
 * ------------------------------------------------------------------------- */

static double e2m1_magnitude(unsigned c) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    return mag[c & 7u];
}

/* Value of a 4-bit code. */
double oracle_e2m1_decode(uint8_t code) { return (code & 8u) ? -e2m1_magnitude(code) : e2m1_magnitude(code); }

/* Nearest E2M1 code of v (finite), ties to the even code, saturating. */
uint8_t oracle_e2m1_encode(float v) {
    uint8_t sign = signbit(v) ? 0x8u : 0x0u;
    double a = fabs((double)v);
    if (a >= 6.0) return (uint8_t)(sign | 7u); /* saturate (far values would tie in double) */
    unsigned best = 0;
    for (unsigned c = 1; c < 8; c++) {
        double dc = fabs(e2m1_magnitude(c) - a), db = fabs(e2m1_magnitude(best) - a);
        if (dc < db || (dc == db && (c & 1u) == 0)) best = c; /* a tie goes to the even code */
    }
    return (uint8_t)(sign | best);
}

void oracle_e2m1_encode_array(const float *v, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e2m1_encode(v[i]);
}

static uint8_t quantize_one_fp4(float x, float s) {
    if (s == 0.0f) return signbit(x) ? 0x8u : 0x0u; /* all-zero group */
    float v = x / s;
    return oracle_e2m1_encode(v);
}

/* 1x128 FP4 activations: q [M][K/2] packed, s [K/128][M]. */
int oracle_quant_act_fp4_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s) {
    if (M < 0 || K < 0 || K % GROUP) return -1;
    int64_t KB = K / GROUP;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            const uint16_t *g = x + m * K + kb * GROUP;
            float amax = 0.0f;
            for (int j = 0; j < GROUP; j++) {
                float v = bf16_to_f32(g[j]);
                if (!isfinite(v)) bad = 1;
                if (fabsf(v) > amax) amax = fabsf(v);
            }
            float scale = amax / 6.0f;
            s[kb * M + m] = scale;
            for (int j = 0; j < GROUP; j += 2) {
                uint8_t lo = quantize_one_fp4(bf16_to_f32(g[j]), scale);
                uint8_t hi = quantize_one_fp4(bf16_to_f32(g[j + 1]), scale);
                q[m * (K / 2) + (kb * GROUP + j) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return bad ? -2 : 0;
}

/* 128x128 FP4 weights: q [N][K/2] packed, s [N/128][K/128]. */
int oracle_quant_w_fp4_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s) {
    if (N < 0 || K < 0 || N % GROUP || K % GROUP) return -1;
    int64_t NB = N / GROUP, KB = K / GROUP;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
    for (int64_t nb = 0; nb < NB; nb++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            float amax = 0.0f;
            for (int i = 0; i < GROUP; i++) {
                const uint16_t *row = w + (nb * GROUP + i) * K + kb * GROUP;
                for (int j = 0; j < GROUP; j++) {
                    float v = bf16_to_f32(row[j]);
                    if (!isfinite(v)) bad = 1;
                    if (fabsf(v) > amax) amax = fabsf(v);
                }
            }
            float scale = amax / 6.0f;
            s[nb * KB + kb] = scale;
            for (int i = 0; i < GROUP; i++) {
                const uint16_t *row = w + (nb * GROUP + i) * K + kb * GROUP;
                for (int j = 0; j < GROUP; j += 2) {
                    uint8_t lo = quantize_one_fp4(bf16_to_f32(row[j]), scale);
                    uint8_t hi = quantize_one_fp4(bf16_to_f32(row[j + 1]), scale);
                    q[(nb * GROUP + i) * (K / 2) + (kb * GROUP + j) / 2] = (uint8_t)(lo | (hi << 4));
                }
            }
        }
    }
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------------------
 * Per-channel FP8 weights (page "DeepSeek starts updating frequently", the
 * list of TileKernels features: per-token, per-block and per-channel modes).
 * Reading: one scale per output channel, i.e. per row of W [N, K] over all K:
 * s[n] = fl32(max_k |w[n,k]| / 448), q[n,k] = E4M3(fl32(w[n,k] / s[n])).
 * ------------------------------------------------------------------------- */
int oracle_quant_w_per_channel(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s) {
    if (N < 0 || K < 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; n++) {
        const uint16_t *row = w + n * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; k++) {
            float v = bf16_to_f32(row[k]);
            if (!isfinite(v)) bad = 1;
            if (fabsf(v) > amax) amax = fabsf(v);
        }
        float scale = amax / 448.0f;
        s[n] = scale;
        for (int64_t k = 0; k < K; k++) q[n * K + k] = quantize_one(bf16_to_f32(row[k]), scale);
    }
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------------------
 * E5M6 activations (page "The Definitive Information To Deepseek", the passage
 * naming a customized E5M6 format for certain activations; page "DeepSeek
 * starts updating frequently", the TileKernels quantization converts to FP8,
 * FP4 or E5M6).  The pages give the name only.  Readings taken here:
 *  - E5M6 is the ExMy layout its name spells: sign, 5 exponent bits with the
 *    IEEE bias 15, 6 mantissa bits, subnormals m * 2^-20 at exponent 0, and
 *    exponent 31 reserved (inf/NaN) as in the IEEE formats with 5 exponent
 *    bits, so the largest finite magnitude is (2 - 2^-6) * 2^15 = 65024;
 *  - it is used in the activation grouping, 1x128 per token, with
 *    scale = fl32(amax / 65024), v = fl32(x / s) rounded to the nearest E5M6
 *    value, ties to the even code, saturating at 65024, sign kept (-0 -> 0x800);
 *  - the 12-bit codes form a little-endian bit stream, element j at bits
 *    12j..12j+11: a pair (c0, c1) fills 3 bytes c0[7:0], c0[11:8] | c1[3:0] << 4,
 *    c1[11:4]; rows of 3K/2 bytes.
 * ------------------------------------------------------------------------- */

#define E5M6_MAX_CODE 0x7BFu /* exponent 30, mantissa 63 */

/* Magnitude of the low 11 bits of a code (finite codes only). */
static double e5m6_magnitude(unsigned c) {
    unsigned e = (c >> 6) & 31u, m = c & 63u;
    if (e == 0) return ldexp((double)m, -20);
    return ldexp(64.0 + (double)m, (int)e - 15 - 6);
}

double oracle_e5m6_decode(uint16_t code) {
    unsigned e = (code >> 6) & 31u;
    double mag;
    if (e == 31) mag = (code & 63u) ? NAN : INFINITY;
    else mag = e5m6_magnitude(code);
    return (code & 0x800u) ? -mag : mag;
}

/* Nearest E5M6 code of v (finite), ties to the even code, saturating. */
uint16_t oracle_e5m6_encode(float v) {
    uint16_t sign = signbit(v) ? 0x800u : 0x0u;
    double a = fabs((double)v);
    if (a >= e5m6_magnitude(E5M6_MAX_CODE)) return (uint16_t)(sign | E5M6_MAX_CODE);
    /* largest code lo with magnitude <= a (magnitudes increase with the code) */
    unsigned lo = 0, hi = E5M6_MAX_CODE;
    while (lo < hi) {
        unsigned mid = (lo + hi + 1) / 2;
        if (e5m6_magnitude(mid) <= a) lo = mid;
        else hi = mid - 1;
    }
    unsigned up = lo + 1;
    double dl = a - e5m6_magnitude(lo), du = e5m6_magnitude(up) - a;
    unsigned c = (du < dl || (du == dl && (up & 1u) == 0)) ? up : lo;
    return (uint16_t)(sign | c);
}

void oracle_e5m6_encode_array(const float *v, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e5m6_encode(v[i]);
}

/* 1x128 E5M6 activations: q [M][3K/2] bytes, s [K/128][M]. */
int oracle_quant_act_e5m6_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s) {
    if (M < 0 || K < 0 || K % GROUP) return -1;
    int64_t KB = K / GROUP, row_bytes = K / 2 * 3;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            const uint16_t *g = x + m * K + kb * GROUP;
            float amax = 0.0f;
            for (int j = 0; j < GROUP; j++) {
                float v = bf16_to_f32(g[j]);
                if (!isfinite(v)) bad = 1;
                if (fabsf(v) > amax) amax = fabsf(v);
            }
            float scale = amax / 65024.0f;
            s[kb * M + m] = scale;
            uint8_t *out = q + m * row_bytes + kb * (GROUP / 2 * 3);
            for (int j = 0; j < GROUP; j += 2) {
                uint16_t c[2];
                for (int t = 0; t < 2; t++) {
                    float xv = bf16_to_f32(g[j + t]);
                    c[t] = scale == 0.0f ? (uint16_t)(signbit(xv) ? 0x800u : 0u) : oracle_e5m6_encode(xv / scale);
                }
                out[j / 2 * 3 + 0] = (uint8_t)(c[0] & 0xFFu);
                out[j / 2 * 3 + 1] = (uint8_t)((c[0] >> 8) | ((c[1] & 0xFu) << 4));
                out[j / 2 * 3 + 2] = (uint8_t)(c[1] >> 4);
            }
        }
    }
    return bad ? -2 : 0;
}
