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
// 1x128 activations.  A 128-element group (256 bytes of bf16) is spread over the 16 lanes of a DPP row,
// 8 elements per lane, so its max-abs is 4 row rotations.  Lane l of a wave works on K-block
// 4 kq + l / 16 (kq = the workgroup's K-block quad) of 4 consecutive tokens, one token per load: each load
// instruction then reads 4 consecutive K-blocks of one token (1 KB contiguous) and each store writes their
// 512 code bytes contiguously.  A workgroup (4 waves) covers 16 tokens x 4 K-blocks; its scales are 16
// consecutive tokens of the K-block-major s_a layout for each of the 4 K-blocks.
// ---------------------------------------------------------------------------------------------
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
        float amax = 0.0f;
        amax = absmax2(amax, v[j].x);
        amax = absmax2(amax, v[j].y);
        amax = absmax2(amax, v[j].z);
        amax = absmax2(amax, v[j].w);
        amax = row16_max(amax);
        const float sc = group_scale(amax);
        const double inv = scale_reciprocal(sc);
        const int64_t m = row0 + j;
        if (m < M && kb_ok) {
            uint2 o;
            o.x = quant4(v[j].x, v[j].y, inv);
            o.y = quant4(v[j].z, v[j].w, inv);
            *reinterpret_cast<uint2 *>(q + m * K + kb * 128 + i * 8) = o;
            if (i == 0) s[kb * M + m] = sc;
        }
    }
}

// ---------------------------------------------------------------------------------------------
// 128x128 weights.  One workgroup (256 threads) per block.  In load i (0..7) thread t reads the
// 16-byte chunk (t % 16) of block row (t / 16 + 16 i): 16 threads cover a 256-byte row, one
// instruction covers 16 rows.  The block max is a wave reduction plus a 4-entry LDS exchange.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_w_128x128_kernel(const uint16_t *__restrict__ w, int64_t K,
                                                              uint8_t *__restrict__ q, float *__restrict__ s) {
    __shared__ float wave_amax[4];
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

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        amax = absmax2(amax, v[i].x);
        amax = absmax2(amax, v[i].y);
        amax = absmax2(amax, v[i].z);
        amax = absmax2(amax, v[i].w);
    }
    amax = wave_max(amax);
    if ((tid & 63) == 0) wave_amax[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wave_amax[0], wave_amax[1]), fmaxf(wave_amax[2], wave_amax[3]));
    const float sc = group_scale(amax);
    const double inv = scale_reciprocal(sc);

    uint8_t *dst = q + (nb * 128) * K + kb * 128 + chunk * 8;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        uint2 o;
        o.x = quant4(v[i].x, v[i].y, inv);
        o.y = quant4(v[i].z, v[i].w, inv);
        *reinterpret_cast<uint2 *>(dst + (int64_t)(r0 + 16 * i) * K) = o;
    }
    if (tid == 0) s[nb * KB + kb] = sc;
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
    quant_act_1x128_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(x, M, K, q, s);
    return hipGetLastError();
}

hipError_t launch_quant_w_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s,
                                  hipStream_t stream) {
    const int64_t blocks = (N / 128) * (K / 128);  // 1-D grid: K-block fastest
    quant_w_128x128_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(w, K, q, s);
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
