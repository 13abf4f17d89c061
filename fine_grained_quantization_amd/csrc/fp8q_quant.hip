// Fine-grained FP8 quantization kernels for gfx950: 1x128 activation tiles and 128x128 weight
// blocks (page "The Definitive Information To Deepseek", the passage referring to Figure 7 (a)).
//
// Both kernels are HBM-bound streams: 2 bytes of bf16 read, 1 byte of E4M3 written per element
// (plus one fp32 scale per group).  Loads are 16-byte, fully coalesced per instruction; the
// group's max-abs is reduced in registers (DPP / shuffles), never through HBM; every element is
// read exactly once.
#include "fp8q_device.h"
#include "fp8q_kernels.h"

namespace fp8q {

// ---------------------------------------------------------------------------------------------
// FP4 (OCP E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in the FP8 groupings (page "DeepSeek starts updating
// frequently", the TileKernels quantization kernels convert to FP8, FP4 or E5M6).  The pages name FP4 only;
// this library reads it as the same 1x128 / 128x128 groups with scale fl32(amax / 6), the nearest E2M1 value
// (ties to the even code, saturating at 6), two codes a byte with element 2i in the low nibble.
// ---------------------------------------------------------------------------------------------
constexpr double kInv6 = 1.0 / 6.0;
// fl32(amax / 6): amax has an 8-bit significand, so amax / 6 is either exact in fp32 or at least 1/6 of an
// fp32 unit from a rounding midpoint (its bits past the 24th repeat 01 or 10), far beyond the double
// product's error: rounding that product to fp32 gives the correctly rounded quotient.
__device__ __forceinline__ float group_scale_fp4(float amax) { return (float)((double)amax * kInv6); }

// 8 bf16 values (two packed pairs per dword, element order kept) -> 8 E2M1 codes, element 2i in the low
// nibble.  The quotients are the exact fl32(x / s) as for FP8; v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds
// a pair of them to the nearest E2M1 value, ties to the even code, saturating at 6, sign kept, the first in
// the low nibble of the selected byte (checked against the oracle's E2M1 encoder on every rounding midpoint,
// its fp32 neighbours, values past 6, subnormals, signed zeros and 10^5 random values).
__device__ __forceinline__ uint32_t quant8_fp4(const u32x4 &v, double inv_s) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, quotient(bf16_lo(v.x), inv_s), quotient(bf16_hi(v.x), inv_s),
                                                 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, quotient(bf16_lo(v.y), inv_s), quotient(bf16_hi(v.y), inv_s),
                                                 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, quotient(bf16_lo(v.z), inv_s), quotient(bf16_hi(v.z), inv_s),
                                                 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, quotient(bf16_lo(v.w), inv_s), quotient(bf16_hi(v.w), inv_s),
                                                 1.0f, 3);
    return r;
}

// ---------------------------------------------------------------------------------------------
// E5M6 (sign, 5 exponent bits with bias 15, 6 mantissa bits, subnormals m * 2^-20, exponent 31 reserved:
// largest finite 65024) in the 1x128 activation groups (page "The Definitive Information To Deepseek", the
// customized E5M6 format for certain activations; the TileKernels list on "DeepSeek starts updating
// frequently").  The pages give the name only; this library reads it as that layout with scale
// fl32(amax / 65024), nearest even, saturating, and the 12-bit codes as a little-endian bit stream.
// ---------------------------------------------------------------------------------------------
constexpr double kInv65024 = 1.0 / 65024.0;
// fl32(amax / 65024) = fl32(amax * RN64(1/65024)): 65024 = 127 * 2^9 and amax has an 8-bit significand, so
// the quotient is exact in fp32 (amax a multiple of 127) or its bits past the 24th repeat with period 7, at
// least 2^-8 of an fp32 unit from any midpoint, far beyond the double product's error.
__device__ __forceinline__ float group_scale_e5m6(float amax) { return (float)((double)amax * kInv65024); }

// E5M6 code of an fp32 value v with |v| <= 65024 (1 + 2^-23).  Normal results (|v| >= 2^-14) round the fp32
// pattern to 6 mantissa bits, nearest even, with the rebias 127 -> 15 folded into the same add (a carry runs
// into the exponent).  Below 2^-14 the code is the number of 2^-20 steps: |v| + 8 lands in [8, 16), whose
// spacing is 2^-20, so the fp32 add rounds |v| to that grid (nearest even) and the pattern difference from
// 8.0 is the count (64 being the smallest normal code).  Checked on the CPU against the oracle's encoder on
// every 7th fp32 pattern up to 65024 (1 + 2^-23), both signs, and every midpoint.
__device__ __forceinline__ uint32_t e5m6_code(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t a = b & 0x7FFFFFFFu;
    const uint32_t normal = min((a + (0xFFFFu - (112u << 23)) + ((a >> 17) & 1u)) >> 17, 0x7BFu);
    const uint32_t sub = __float_as_uint(__uint_as_float(a) + 8.0f) - 0x41000000u;
    return ((b >> 20) & 0x800u) | (a >= 0x38800000u ? normal : sub);
}

// 8 bf16 values (two packed pairs per dword) -> 8 codes of 12 bits, element j at bits 12j of 96.
__device__ __forceinline__ uint3 quant8_e5m6(const u32x4 &v, double inv_s) {
    const uint32_t c0 = e5m6_code(quotient(bf16_lo(v.x), inv_s)), c1 = e5m6_code(quotient(bf16_hi(v.x), inv_s));
    const uint32_t c2 = e5m6_code(quotient(bf16_lo(v.y), inv_s)), c3 = e5m6_code(quotient(bf16_hi(v.y), inv_s));
    const uint32_t c4 = e5m6_code(quotient(bf16_lo(v.z), inv_s)), c5 = e5m6_code(quotient(bf16_hi(v.z), inv_s));
    const uint32_t c6 = e5m6_code(quotient(bf16_lo(v.w), inv_s)), c7 = e5m6_code(quotient(bf16_hi(v.w), inv_s));
    return (uint3){c0 | (c1 << 12) | (c2 << 24), (c2 >> 8) | (c3 << 4) | (c4 << 16) | (c5 << 28),
                   (c5 >> 4) | (c6 << 8) | (c7 << 20)};
}

enum : int { kFmtFp8 = 0, kFmtFp4 = 1, kFmtE5M6 = 2 };

// ---------------------------------------------------------------------------------------------
// 1x128 activations.  A 128-element group (256 bytes of bf16) is spread over the 16 lanes of a DPP row,
// 8 elements per lane, so its max-abs is 4 row rotations.  Lane l of a wave works on K-block
// 4 kq + l / 16 (kq = the workgroup's K-block quad) of 4 consecutive tokens, one token per load: each load
// instruction then reads 4 consecutive K-blocks of one token (1 KB contiguous) and each store writes their
// 512 code bytes contiguously.  A workgroup (4 waves) covers 16 tokens x 4 K-blocks; its scales are 16
// consecutive tokens of the K-block-major s_a layout for each of the 4 K-blocks.
// ---------------------------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void quant_act_1x128_kernel(const uint16_t *__restrict__ x, int64_t M, int64_t K,
                                                              uint8_t *__restrict__ q, float *__restrict__ s) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
    const int64_t KB = K >> 7;
    const int64_t KQ = (KB + 3) >> 2;  // K-block quads
    const int64_t kq = (int64_t)blockIdx.x % KQ;
    const int64_t row0 = ((int64_t)blockIdx.x / KQ) * 16 + wave * 4;
    const int64_t kb = kq * 4 + (lane >> 4);
    const int i = lane & 15;
    const bool kb_ok = kb < KB;
    const int64_t kbr = kb_ok ? kb : KB - 1;  // lanes past the last K-block re-read it and store nothing

    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int64_t m = row0 + j;
        const int64_t mr = m < M ? m : M - 1;  // tokens past M re-read the last one and store nothing
        v[j] = load_stream16(x + mr * K + kbr * 128 + i * 8);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const float amax = bf16_mag_f32(row16_max(absmax_bits(v[j])));
        const float sc = FMT == kFmtFp4 ? group_scale_fp4(amax)
                         : FMT == kFmtE5M6 ? group_scale_e5m6(amax) : group_scale(amax);
        const double inv = scale_reciprocal(sc);
        const int64_t m = row0 + j;
        if (m < M && kb_ok) {
            if constexpr (FMT == kFmtFp4) {
                *reinterpret_cast<uint32_t *>(q + m * (K / 2) + kb * 64 + i * 4) = quant8_fp4(v[j], inv);
            } else if constexpr (FMT == kFmtE5M6) {
                uint32_t *dst = reinterpret_cast<uint32_t *>(q + m * (K / 2 * 3) + kb * 192 + i * 12);
                const uint3 o = quant8_e5m6(v[j], inv);
                dst[0] = o.x;
                dst[1] = o.y;
                dst[2] = o.z;
            } else {
                uint2 o;
                o.x = quant4(v[j].x, v[j].y, inv);
                o.y = quant4(v[j].z, v[j].w, inv);
                *reinterpret_cast<uint2 *>(q + m * K + kb * 128 + i * 8) = o;
            }
            if (i == 0) s[kb * M + m] = sc;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Forward and backward FP8 copies of a Linear input in one pass (page "The Definitive Information To
// Deepseek", the passage on caching the Linear's input in FP8 for the backward pass).  The backward pass
// contracts the input over tokens (the weight gradient dW = dY^T x), so its copy is the 1x128 quantization
// of x^T: one scale per channel and 128 tokens, stored channel-major.  A workgroup (512 threads, 8 waves)
// owns 128 tokens x 128 channels; thread t holds 4 consecutive tokens (4 (t / 16) ...) x 8 consecutive
// channels (chunk t % 16), 4 loads of 16 bytes (a wave's load instruction covers 4 rows x 256 bytes).
//  - forward copy: a token's 128 channels lie in the 16 lanes of one DPP row (4 row maxima per thread);
//    the 128 token scales leave as one run of 512 bytes;
//  - backward copy: a channel's 128 tokens lie in 16 threads spread over the 8 waves; their maxima over 4
//    rows go through LDS, one thread per channel forms the scale and its reciprocal, and the codes are
//    transposed through an LDS tile [128 channels][128 tokens] so that they leave as whole 128-byte rows
//    of the channel-major copy (16 bytes per lane) rather than as 4-byte pieces.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_at(const u32x4 &v, int c) {
    const uint32_t d = c < 2 ? v.x : c < 4 ? v.y : c < 6 ? v.z : v.w;
    return (c & 1) ? bf16_hi(d) : bf16_lo(d);
}

constexpr int kDualThreads = 512;

__global__ __launch_bounds__(kDualThreads) void quant_act_dual_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                                      int64_t K, uint8_t *__restrict__ q,
                                                                      float *__restrict__ s, uint8_t *__restrict__ qt,
                                                                      float *__restrict__ st) {
    constexpr int R = 4;                       // tokens per thread (the column maxima below take 4)
    constexpr int G = kDualThreads / 16;       // token groups of R
    // colmax: per-group channel maxima, dead once the channel scales are formed; the code tile reuses it.
    // Tile row = channel, 128 code bytes = 8 pieces of 16 bytes; piece p of row r sits at p ^ ((r / 8) & 7),
    // which spreads one store instruction's 4-byte writes over the LDS banks.
    __shared__ __align__(16) union {
        uint32_t colmax[G][128];   // magnitude bit patterns
        uint32_t tile[128 * 32];
    } sh;
    __shared__ double colinv[128];
    __shared__ float rowsc[128];
    const int t = threadIdx.x;
    const int64_t KB = K >> 7;
    const int64_t kb = (int64_t)blockIdx.x % KB;
    const int64_t mb = (int64_t)blockIdx.x / KB;
    const int chunk = t & 15, g = t >> 4;
    const int64_t m0 = mb * 128 + g * R;
    const int64_t c0 = kb * 128 + chunk * 8;

    u32x4 v[R];
#pragma unroll
    for (int j = 0; j < R; j++) v[j] = load_stream16(x + (m0 + j) * K + c0);

    // forward: per token, 128 channels
#pragma unroll
    for (int j = 0; j < R; j++) {
        const float amax = bf16_mag_f32(row16_max(absmax_bits(v[j])));
        const float sc = group_scale(amax);
        const double inv = scale_reciprocal(sc);
        uint2 o;
        o.x = quant4(v[j].x, v[j].y, inv);
        o.y = quant4(v[j].z, v[j].w, inv);
        *reinterpret_cast<uint2 *>(q + (m0 + j) * K + c0) = o;
        if (chunk == 0) rowsc[g * R + j] = sc;
    }

    // backward: per channel, 128 tokens.  Channels 2d and 2d + 1 of the chunk share dword d of every token's
    // load, so one packed maximum over the R tokens gives both channels' magnitude maxima.
    {
        const u16x2 m[4] = {absmax_halves(v[0].x, v[1].x, v[2].x, v[3].x), absmax_halves(v[0].y, v[1].y, v[2].y, v[3].y),
                            absmax_halves(v[0].z, v[1].z, v[2].z, v[3].z), absmax_halves(v[0].w, v[1].w, v[2].w, v[3].w)};
#pragma unroll
        for (int d = 0; d < 4; d++) {
            sh.colmax[g][chunk * 8 + 2 * d] = m[d].x;
            sh.colmax[g][chunk * 8 + 2 * d + 1] = m[d].y;
        }
    }
    __syncthreads();
    float csc = 0.0f;
    if (t < 128) {
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < G; i++) amax = max(amax, sh.colmax[i][t]);
        csc = group_scale(bf16_mag_f32(amax));
        colinv[t] = scale_reciprocal(csc);
    }
    __syncthreads();
    if (t < 128) {
        st[mb * K + kb * 128 + t] = csc;
        s[kb * M + mb * 128 + t] = rowsc[t];
    }
#pragma unroll
    for (int c = 0; c < 8; c++) {
        const double inv = colinv[chunk * 8 + c];
        const int row = chunk * 8 + c;
        const uint32_t w = encode4(quotient(bf16_at(v[0], c), inv), quotient(bf16_at(v[1], c), inv),
                                   quotient(bf16_at(v[2], c), inv), quotient(bf16_at(v[3], c), inv));
        // token bytes 4g..4g+3 are word g of the row: piece g / 4, word g % 4 within it
        sh.tile[row * 32 + (((g >> 2) ^ (chunk & 7)) << 2) + (g & 3)] = w;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 1024 / kDualThreads; i++) {
        const int p = t + i * kDualThreads;  // 16-byte piece p % 8 of channel row p / 8
        const int row = p >> 3, piece = p & 7;
        const u32x4 w = *reinterpret_cast<const u32x4 *>(&sh.tile[row * 32 + ((piece ^ ((row >> 3) & 7)) << 2)]);
        *reinterpret_cast<u32x4 *>(qt + (kb * 128 + row) * M + mb * 128 + piece * 16) = w;
    }
}

// ---------------------------------------------------------------------------------------------
// Fused SwiGLU + 1x128 quantization (page "DeepSeek starts updating frequently", the TileKernels feature
// list: quantization combined with SwiGLU).  h = SiLU(x) * y with SiLU(x) = x / (1 + e^-x), the exact value
// rounded once to bf16 (nearest even), then quantized like the activations above; h never leaves registers.
//
// Per element: an fp32 value of x*y / (1 + e^-x) with a proven error bound (below); where its low 16 bits
// are far enough from the bf16 rounding midpoint, its nearest-even bf16 is the correctly rounded one.  The
// rest (a few in 10^4 for N(0,1) gates, plus zeros, tiny and non-finite intermediates) take a double path:
// x*y is exact, the quotient within a few double ulps; two classes sit closer to a midpoint than that and are
// settled by where the exact value must lie: gates above 16 with x*y itself a midpoint (the value lies just
// inside it, towards zero) and gates below 2^-40 with x*y/2 a midpoint (the value lies beyond it for x > 0,
// inside it for x < 0).  No other bf16 pair comes within 2^-45 of a midpoint.
// ---------------------------------------------------------------------------------------------

// Rounding of a finite double to bf16: mode 0 nearest even, -1 towards zero, +1 away from zero.  Bit 31 of
// the result is set when v is exactly a midpoint between two bf16 values.
constexpr uint32_t kMidFlag = 0x80000000u;

__device__ __forceinline__ uint32_t bf16_round_f64(double v, int mode) {
    if (v == 0.0) return __builtin_signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    int ex = ilogb(a);
    if (ex < -126) ex = -126;  // bf16 subnormals share the spacing 2^-133
    const double q = ldexp(a, 7 - ex);  // exact: a power-of-two scaling
    double fl = floor(q);
    const double rem = q - fl;
    if (mode == 0) {
        if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    } else if (mode > 0 && rem > 0.0) {
        fl += 1.0;
    }
    const float r = (float)ldexp(fl, ex - 7);  // a bf16 value: exact in float
    return (__float_as_uint(r) >> 16) | (__builtin_signbit(v) ? 0x8000u : 0u) | (rem == 0.5 ? kMidFlag : 0u);
}

__device__ __noinline__ uint32_t swiglu_bf16_f64(float xf, float yf) {
    const double x = xf, p = x * (double)yf;  // exact
    if (x > 16.0) {
        const uint32_t r = bf16_round_f64(p, -1);
        if (r & kMidFlag) return r & 0xFFFFu;
    } else if (fabs(x) < 0x1p-40 && x != 0.0) {
        const uint32_t r = bf16_round_f64(p * 0.5, x > 0.0 ? 1 : -1);
        if (r & kMidFlag) return r & 0xFFFFu;
    }
    return bf16_round_f64(p / (1.0 + exp(-x)), 0) & 0xFFFFu;
}

// bf16 bits of SiLU(x) * y for the bf16 pattern pairs in the low halves of xb, yb.  Fast path in fp32:
// e = exp2(fl(-x log2 e)) with the hardware v_exp_f32.  Rounding -x log2 e shifts the exponent by at most
// |x| 2^-24 relative, so e carries at most |x| 2^-24 + 2^-23 relative error; 1 + e, v_rcp_f32 and the final
// product add at most 2^-24 + 2^-23 + 2^-24.  x*y is exact while the result is a normal number (|h| >= 2^-120
// implies |x*y| >= 2^-120), so h = (x*y) rcp(1 + e) is within |x| + 6 fp32 units in the last place of the
// exact value, and its nearest-even bf16 is the correctly rounded one when its low 16 bits are more than twice
// that from the midpoint 0x8000.
__device__ __forceinline__ uint32_t swiglu_bf16(uint32_t xb, uint32_t yb) {
    const float x = __uint_as_float(xb << 16), y = __uint_as_float(yb << 16);
    const float e = __builtin_amdgcn_exp2f(x * -1.44269504088896340736f);
    const float h = (x * y) * __builtin_amdgcn_rcpf(1.0f + e);
    const uint32_t bits = __float_as_uint(h);
    const float off = fabsf((float)((int)(bits & 0xFFFFu) - 0x8000));
    const bool fast = fabsf(h) >= 0x1p-120f && fabsf(h) <= 0x1p126f && off > 16.0f + 2.0f * fabsf(x);
    if (fast) return (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
    return swiglu_bf16_f64(x, y);
}

__device__ __forceinline__ uint32_t swiglu_bf16x2(uint32_t xd, uint32_t yd) {
    return swiglu_bf16(xd & 0xFFFFu, yd & 0xFFFFu) | (swiglu_bf16(xd >> 16, yd >> 16) << 16);
}

// Same layout as quant_act_1x128_kernel; x and y rows are ld elements apart (so the gate and up halves of
// one [M, 2K] projection can be passed as two views).
__global__ __launch_bounds__(256) void swiglu_quant_act_1x128_kernel(const uint16_t *__restrict__ x,
                                                                     const uint16_t *__restrict__ y, int64_t ld,
                                                                     int64_t M, int64_t K, uint8_t *__restrict__ q,
                                                                     float *__restrict__ s) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t KB = K >> 7;
    const int64_t KQ = (KB + 3) >> 2;
    const int64_t kq = (int64_t)blockIdx.x % KQ;
    const int64_t row0 = ((int64_t)blockIdx.x / KQ) * 16 + wave * 4;
    const int64_t kb = kq * 4 + (lane >> 4);
    const int i = lane & 15;
    const bool kb_ok = kb < KB;
    const int64_t kbr = kb_ok ? kb : KB - 1;

    u32x4 vx[4], vy[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int64_t m = row0 + j;
        const int64_t mr = m < M ? m : M - 1;
        vx[j] = load_stream16(x + mr * ld + kbr * 128 + i * 8);
        vy[j] = load_stream16(y + mr * ld + kbr * 128 + i * 8);
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
        u32x4 h;
        h.x = swiglu_bf16x2(vx[j].x, vy[j].x);
        h.y = swiglu_bf16x2(vx[j].y, vy[j].y);
        h.z = swiglu_bf16x2(vx[j].z, vy[j].z);
        h.w = swiglu_bf16x2(vx[j].w, vy[j].w);
        const float amax = bf16_mag_f32(row16_max(absmax_bits(h)));
        const float sc = group_scale(amax);
        const double inv = scale_reciprocal(sc);
        const int64_t m = row0 + j;
        if (m < M && kb_ok) {
            uint2 o;
            o.x = quant4(h.x, h.y, inv);
            o.y = quant4(h.z, h.w, inv);
            *reinterpret_cast<uint2 *>(q + m * K + kb * 128 + i * 8) = o;
            if (i == 0) s[kb * M + m] = sc;
        }
    }
}

// h = bf16(SiLU(x) * y) alone (the intermediate the fused kernel quantizes), 8 elements per thread.
__global__ __launch_bounds__(256) void swiglu_bf16_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ y, int64_t ld, int64_t M,
                                                          int64_t K, uint16_t *__restrict__ h) {
    const int64_t per_row = K >> 3;
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= M * per_row) return;
    const int64_t m = u / per_row, k = (u - m * per_row) * 8;
    const u32x4 vx = load_stream16(x + m * ld + k), vy = load_stream16(y + m * ld + k);
    u32x4 o;
    o.x = swiglu_bf16x2(vx.x, vy.x);
    o.y = swiglu_bf16x2(vx.y, vy.y);
    o.z = swiglu_bf16x2(vx.z, vy.z);
    o.w = swiglu_bf16x2(vx.w, vy.w);
    *reinterpret_cast<u32x4 *>(h + m * K + k) = o;
}

// ---------------------------------------------------------------------------------------------
// 128x128 weights.  One workgroup (256 threads) per block.  In load i (0..7) thread t reads the
// 16-byte chunk (t % 16) of block row (t / 16 + 16 i): 16 threads cover a 256-byte row, one
// instruction covers 16 rows.  The block max is a wave reduction plus a 4-entry LDS exchange.
// ---------------------------------------------------------------------------------------------
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// STREAM_OUT: the codes are written with non-temporal stores, for weights whose codes alone are larger than
// the 256 MB Infinity Cache (keeping them there would only evict the bf16 input still being read).
template <bool FP4, bool STREAM_OUT = false>
__global__ __launch_bounds__(256) void quant_w_128x128_kernel(const uint16_t *__restrict__ w, int64_t K,
                                                              uint8_t *__restrict__ q, float *__restrict__ s) {
    __shared__ uint32_t wave_amax[4];
    const int tid = threadIdx.x;
    const int64_t KB = K >> 7;
    const int64_t kb = (int64_t)blockIdx.x % KB;
    const int64_t nb = (int64_t)blockIdx.x / KB;
    const int chunk = tid & 15;
    const int r0 = tid >> 4;
    const uint16_t *base = w + (nb * 128) * K + kb * 128 + chunk * 8;

    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = load_stream16(base + (int64_t)(r0 + 16 * i) * K);

    u16x2 mh = absmax_halves(v[0]);
#pragma unroll
    for (int i = 1; i < 8; i++) mh = __builtin_elementwise_max(mh, absmax_halves(v[i]));
    const uint32_t wm = wave_max(halves_max(mh));
    if ((tid & 63) == 0) wave_amax[tid >> 6] = wm;
    __syncthreads();
    const float amax = bf16_mag_f32(max(max(wave_amax[0], wave_amax[1]), max(wave_amax[2], wave_amax[3])));
    const float sc = FP4 ? group_scale_fp4(amax) : group_scale(amax);
    const double inv = scale_reciprocal(sc);

    if constexpr (FP4) {
        uint8_t *dst = q + (nb * 128) * (K / 2) + kb * 64 + chunk * 4;
#pragma unroll
        for (int i = 0; i < 8; i++)
            *reinterpret_cast<uint32_t *>(dst + (int64_t)(r0 + 16 * i) * (K / 2)) = quant8_fp4(v[i], inv);
    } else {
        uint8_t *dst = q + (nb * 128) * K + kb * 128 + chunk * 8;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const u32x2 o = {quant4(v[i].x, v[i].y, inv), quant4(v[i].z, v[i].w, inv)};
            u32x2 *p = reinterpret_cast<u32x2 *>(dst + (int64_t)(r0 + 16 * i) * K);
            if constexpr (STREAM_OUT)
                __builtin_nontemporal_store(o, p);
            else
                *p = o;
        }
    }
    if (tid == 0) s[nb * KB + kb] = sc;
}

// ---------------------------------------------------------------------------------------------
// Per-channel FP8 weights (page "DeepSeek starts updating frequently", the TileKernels quantization modes:
// per token, per block, per channel).  Read as one scale per output channel: row n of W [N, K] over all of
// K, s[n] = fl32(amax_n / 448), the codes as in the grouped modes.  One workgroup (4 waves) per row: thread
// t holds the row's 16-byte chunks t, t + 256, ..., the first CH of them in registers between the max and
// the encode (rows up to 256 * CH * 8 elements are read once); chunks past them are read twice, the second
// time from the cache (the row was just read).  The row's max-abs is a wave reduction and a 4-entry LDS
// exchange.  Every load and store instruction of a wave is contiguous.  Four waves per row rather than one
// keep 4 chunks a lane in registers for a 7168-element row (under 64 VGPRs, 8 waves per SIMD) instead of 14
// (over 128 VGPRs, 3 waves per SIMD), so more rows are in flight while others encode.
// ---------------------------------------------------------------------------------------------
template <int CH>
__global__ __launch_bounds__(256) void quant_w_per_channel_kernel(const uint16_t *__restrict__ w, int64_t K,
                                                                  uint8_t *__restrict__ q, float *__restrict__ s) {
    __shared__ uint32_t wmax[4];
    const int t = threadIdx.x;
    const int64_t n = blockIdx.x;
    const int64_t chunks = K >> 3;
    const uint16_t *row = w + n * K;
    uint8_t *dst = q + n * K;

    u32x4 v[CH];
#pragma unroll
    for (int j = 0; j < CH; j++) {
        const int64_t c = t + 256 * j;
        v[j] = c < chunks ? load_stream16(row + c * 8) : (u32x4){0u, 0u, 0u, 0u};
    }
    u16x2 mh = absmax_halves(v[0]);
#pragma unroll
    for (int j = 1; j < CH; j++) mh = __builtin_elementwise_max(mh, absmax_halves(v[j]));
    for (int64_t c = t + 256 * CH; c < chunks; c += 256) {
        const u32x4 u = *reinterpret_cast<const u32x4 *>(row + c * 8);  // cached: read again below
        mh = __builtin_elementwise_max(mh, absmax_halves(u));
    }
    const uint32_t wm = wave_max(halves_max(mh));
    if ((t & 63) == 0) wmax[t >> 6] = wm;
    __syncthreads();
    const float sc = group_scale(bf16_mag_f32(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]))));
    const double inv = scale_reciprocal(sc);
#pragma unroll
    for (int j = 0; j < CH; j++) {
        const int64_t c = t + 256 * j;
        if (c < chunks)
            *reinterpret_cast<uint2 *>(dst + c * 8) = (uint2){quant4(v[j].x, v[j].y, inv), quant4(v[j].z, v[j].w, inv)};
    }
    for (int64_t c = t + 256 * CH; c < chunks; c += 256) {
        const u32x4 u = load_stream16(row + c * 8);
        *reinterpret_cast<uint2 *>(dst + c * 8) = (uint2){quant4(u.x, u.y, inv), quant4(u.z, u.w, inv)};
    }
    if (t == 0) s[n] = sc;
}

// FP8 -> BF16 weight conversion with 128x128 block scales (page "deepseek-ai/DeepSeek-V3", "How to Run
// Locally": the published weights are FP8 and a script converts them to BF16).  Reading of the arithmetic:
// every code times its block's scale in fp32, rounded to bf16 to nearest even, w = bf16(fl32(dec(q) * s)).
// The hardware FP8 -> FP32 conversion is exact, v_mul_f32 rounds once, and the bf16 pack rounds to nearest
// even.  A workgroup converts 4 x 256 consecutive units of 8 codes; unit u of thread t is codes
// base + (256 u + t) * 8 .. +8, so every 8-byte load and 16-byte store instruction of a wave is contiguous
// (measured: 1.6x the bandwidth of 32 codes per thread, whose stores were 64 bytes apart per lane).  K is a
// multiple of 128, so a unit lies in one 128-wide block and has one scale.
template <bool HI>
__device__ __forceinline__ uint32_t dequant2(int codes, float s) {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(codes, HI);  // two OCP E4M3 codes -> two floats (exact)
    return pack_bf16x2(f[0] * s, f[1] * s);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kDqUnits = 4;

__global__ __launch_bounds__(256) void dequant_w_128x128_kernel(const uint8_t *__restrict__ q,
                                                                const float *__restrict__ s, int64_t K,
                                                                int64_t total, uint16_t *__restrict__ w) {
    const int64_t base = (int64_t)blockIdx.x * (256 * 8 * kDqUnits);
    u32x2 in[kDqUnits];
    float sc[kDqUnits];
#pragma unroll
    for (int u = 0; u < kDqUnits; u++) {
        const int64_t e = base + ((int64_t)u * 256 + threadIdx.x) * 8;
        const int64_t ec = e < total ? e : total - 8;  // units past the end re-read the last one, store nothing
        const int64_t n = ec / K, k = ec - n * K;
        in[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(q + ec));
        sc[u] = s[(n >> 7) * (K >> 7) + (k >> 7)];
    }
#pragma unroll
    for (int u = 0; u < kDqUnits; u++) {
        const int64_t e = base + ((int64_t)u * 256 + threadIdx.x) * 8;
        if (e < total) {
            const int d0 = (int)in[u][0], d1 = (int)in[u][1];
            *reinterpret_cast<u32x4 *>(w + e) = (u32x4){dequant2<false>(d0, sc[u]), dequant2<true>(d0, sc[u]),
                                                        dequant2<false>(d1, sc[u]), dequant2<true>(d1, sc[u])};
        }
    }
}

hipError_t launch_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s,
                                  hipStream_t stream) {
    const int64_t KQ = (K / 128 + 3) / 4;
    const int64_t blocks = ((M + 15) / 16) * KQ;  // 1-D grid: K-block quad fastest, 16 tokens per workgroup
    quant_act_1x128_kernel<kFmtFp8><<<dim3((unsigned)blocks), 256, 0, stream>>>(x, M, K, q, s);
    return hipGetLastError();
}

hipError_t launch_quant_act_fp4_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s,
                                      hipStream_t stream) {
    const int64_t KQ = (K / 128 + 3) / 4;
    const int64_t blocks = ((M + 15) / 16) * KQ;
    quant_act_1x128_kernel<kFmtFp4><<<dim3((unsigned)blocks), 256, 0, stream>>>(x, M, K, q, s);
    return hipGetLastError();
}

hipError_t launch_quant_act_e5m6_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s,
                                       hipStream_t stream) {
    const int64_t KQ = (K / 128 + 3) / 4;
    const int64_t blocks = ((M + 15) / 16) * KQ;
    quant_act_1x128_kernel<kFmtE5M6><<<dim3((unsigned)blocks), 256, 0, stream>>>(x, M, K, q, s);
    return hipGetLastError();
}

// Dynamic LDS the weight quantizers reserve (and do not use) so that at most 4 workgroups share a CU's
// 160 KB: at 64 VGPRs 8 would fit, and with 8 blocks of 128 rows each per CU in flight the kernel measured
// 1.5-3% slower than with 4 (up weight 65.2 vs 63.8 us, the MoE layer's 64 experts 502 vs 486 us).
constexpr size_t kWeightQuantLds = 36 * 1024;

hipError_t launch_quant_w_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s,
                                  hipStream_t stream) {
    const int64_t blocks = (N / 128) * (K / 128);  // 1-D grid: K-block fastest
    // Measured on 64 x [2048, 7168] (940 MB of codes): 504 -> 485 us with streaming stores; on [18432, 7168]
    // (132 MB of codes, which the GEMM after it reads from the Infinity Cache) 63.5 -> 67 us, so only codes
    // larger than the cache stream.
    if (N * K > (int64_t(256) << 20))
        quant_w_128x128_kernel<false, true><<<dim3((unsigned)blocks), 256, kWeightQuantLds, stream>>>(w, K, q, s);
    else
        quant_w_128x128_kernel<false><<<dim3((unsigned)blocks), 256, kWeightQuantLds, stream>>>(w, K, q, s);
    return hipGetLastError();
}

hipError_t launch_quant_w_fp4_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s,
                                      hipStream_t stream) {
    const int64_t blocks = (N / 128) * (K / 128);
    quant_w_128x128_kernel<true><<<dim3((unsigned)blocks), 256, kWeightQuantLds, stream>>>(w, K, q, s);
    return hipGetLastError();
}

hipError_t launch_quant_w_per_channel(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s,
                                      hipStream_t stream) {
    // one workgroup per row; chunks a lane keeps in registers: 4 for rows up to 8192 elements, else 8 (rows
    // past 16384 elements read the rest twice).  Holding 12 a lane (3 waves per SIMD when measured) ran 10%
    // slower at K = 18432 with the input still in the Infinity Cache and 7% faster with it evicted.
    const dim3 grid((unsigned)N);
    if (K <= 256 * 4 * 8)
        quant_w_per_channel_kernel<4><<<grid, 256, 0, stream>>>(w, K, q, s);
    else
        quant_w_per_channel_kernel<8><<<grid, 256, 0, stream>>>(w, K, q, s);
    return hipGetLastError();
}

hipError_t launch_swiglu_quant_act_1x128(const uint16_t *x, const uint16_t *y, int64_t ld, int64_t M, int64_t K,
                                         uint8_t *q, float *s, hipStream_t stream) {
    const int64_t KQ = (K / 128 + 3) / 4;
    const int64_t blocks = (M + 15) / 16 * KQ;
    swiglu_quant_act_1x128_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(x, y, ld, M, K, q, s);
    return hipGetLastError();
}

hipError_t launch_quant_act_dual(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, uint8_t *qt,
                                 float *st, hipStream_t stream) {
    const int64_t blocks = (M / 128) * (K / 128);
    quant_act_dual_kernel<<<dim3((unsigned)blocks), kDualThreads, 0, stream>>>(x, M, K, q, s, qt, st);
    return hipGetLastError();
}

hipError_t launch_swiglu_bf16(const uint16_t *x, const uint16_t *y, int64_t ld, int64_t M, int64_t K, uint16_t *h,
                              hipStream_t stream) {
    const int64_t blocks = (M * (K / 8) + 255) / 256;
    swiglu_bf16_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(x, y, ld, M, K, h);
    return hipGetLastError();
}

hipError_t launch_dequant_w_128x128(const uint8_t *q, const float *s, int64_t N, int64_t K, uint16_t *w,
                                    hipStream_t stream) {
    const int64_t total = N * K;
    const int64_t per_block = 256 * 8 * kDqUnits;
    const int64_t blocks = (total + per_block - 1) / per_block;
    dequant_w_128x128_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(q, s, K, total, w);
    return hipGetLastError();
}

}  // namespace fp8q
