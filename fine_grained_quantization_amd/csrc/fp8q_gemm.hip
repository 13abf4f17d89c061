// Block-scaled FP8 GEMM for gfx950: C = A * W^T with E4M3 operands, one fp32 scale per 1x128
// activation tile and per 128x128 weight block, and promotion of every 128-element partial sum into
// an fp32 accumulator (page "The Definitive Information To Deepseek": FP8 GEMM inputs with BF16/FP32
// outputs; promotion of partial results alongside the MMA).
//
// Design:
//  * v_mfma_f32_16x16x128_f8f6f4 computes exactly one 128-deep K-block per instruction, so each
//    MFMA result is one fresh partial sum P (C input = 0) and promotion is acc += P * (s_a * s_w).
//  * Operand roles are swapped: the weight tile feeds the MFMA's row operand and the activation
//    tile its column operand, so a lane's 4 result registers are 4 consecutive output channels of
//    ONE token.  Every lane then promotes all its registers of a subtile with a single scalar
//    s_a[kb][m] * s_w[n/128][kb], and stores 4 adjacent outputs with one instruction.
//  * A workgroup tile is 128 tokens x 128 weight rows (the weight rows are exactly one scale
//    block, so s_w is one scalar per K-block for the whole workgroup).  4 waves in a 2 x 2 grid,
//    each 64 x 64 = 4 x 4 MFMA subtiles.  A and W K-block tiles (128 rows x 128 bytes) are staged
//    through LDS, double-buffered, with a 16-byte-chunk XOR swizzle so that fragment reads are
//    bank-conflict free.
//  * The grouped (MoE) variant maps each 128-row M tile to the expert whose segment contains it
//    (segments are multiples of 128 rows) and offsets the weight and scale pointers.
#include "fp8q_device.h"
#include "fp8q_kernels.h"

namespace fp8q {

namespace {

constexpr int kBM = 128;            // tokens per workgroup tile
constexpr int kBN = 128;            // weight rows per workgroup tile (one scale block)
constexpr int kTile = 128 * 128;    // bytes of one operand tile for one K-block

// LDS byte offset of 16-byte chunk c (0..7) of tile row r.
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// One MFMA operand fragment: 16 rows starting at tile row rb; lane l takes row rb + l % 16 and the
// 32 bytes [(l / 16) * 32, +32) of it.
__device__ __forceinline__ v8i load_frag(const uint8_t *tile, int rb, int lane) {
    const int r = rb + (lane & 15);
    const int g = lane >> 4;
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(tile + swz(r, 2 * g));
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(tile + swz(r, 2 * g + 1));
    v8i f;
    f[0] = (int)lo[0]; f[1] = (int)lo[1]; f[2] = (int)lo[2]; f[3] = (int)lo[3];
    f[4] = (int)hi[0]; f[5] = (int)hi[1]; f[6] = (int)hi[2]; f[7] = (int)hi[3];
    return f;
}

template <bool OUT_BF16>
__device__ __forceinline__ void store4(void *c, int64_t idx, const v4f &v) {
    if (OUT_BF16) {
        uint2 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(c) + idx) = o;
    } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(c) + idx) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

template <bool OUT_BF16, bool GROUPED>
__global__ __launch_bounds__(256, 2) void gemm_blockscaled_kernel(const uint8_t *__restrict__ qa,
                                                                  const float *__restrict__ sa,
                                                                  const uint8_t *__restrict__ qw,
                                                                  const float *__restrict__ sw, void *__restrict__ c,
                                                                  int64_t M, int64_t N, int64_t K,
                                                                  const int32_t *__restrict__ off, int64_t E,
                                                                  int64_t n_mtiles) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 2 * kTile];  // [buffer][A tile | W tile]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1;   // which 64-row half of the weight tile
    const int wm = wave >> 1;  // which 64-token half of the activation tile
    const int64_t KB = K >> 7;
    const int64_t mt = (int64_t)blockIdx.x % n_mtiles;
    const int64_t nt = (int64_t)blockIdx.x / n_mtiles;
    const int64_t m0 = mt * kBM;
    const int64_t n0 = nt * kBN;

    const uint8_t *W = qw;
    const float *SW = sw;
    if (GROUPED) {
        int64_t e = -1;
        for (int64_t i = 0; i < E; i++) {
            if ((int64_t)off[i] <= m0 && m0 < (int64_t)off[i + 1]) {
                e = i;
                break;
            }
        }
        if (e < 0) {  // no segment covers these rows: write zeros (only with offsets that break the rules)
            const v4f z = {0.f, 0.f, 0.f, 0.f};
            for (int i = tid; i < kBM * (kBN / 4); i += 256) {
                const int64_t m = m0 + i / (kBN / 4);
                const int64_t n = n0 + (i % (kBN / 4)) * 4;
                store4<OUT_BF16>(c, m * N + n, z);
            }
            return;
        }
        W = qw + e * N * K;
        SW = sw + e * (N / 128) * KB;
    }

    // Global -> LDS staging: thread tid moves 16-byte chunk (tid % 8) of tile rows tid / 8 + 32 i.
    // Addresses are recomputed from scalars each time (arrays of pointers would live in scratch).
    const int ch = tid & 7;
    const int rr = tid >> 3;
    const int64_t Mlast = M - 1;
    const uint8_t *a_base = qa + ch * 16;
    const uint8_t *w_base = W + (n0 + rr) * K + ch * 16;
    // A row of staging slot i; the ragged M tail re-reads the last row (its outputs are not stored).
#define FP8Q_AROW(i) ((m0 + rr + 32 * (i)) < M ? (m0 + rr + 32 * (i)) : Mlast)
    // Token of this lane in subtile mi, clamped the same way for its scale.
#define FP8Q_MROW(mi) ((m0 + wm * 64 + (mi) * 16 + (lane & 15)) < M ? (m0 + wm * 64 + (mi) * 16 + (lane & 15)) : Mlast)
    const float *sw_row = SW + (n0 / 128) * KB;

    v4f acc[4][4];
#pragma unroll
    for (int ni = 0; ni < 4; ni++)
#pragma unroll
        for (int mi = 0; mi < 4; mi++) acc[ni][mi] = (v4f){0.f, 0.f, 0.f, 0.f};

    u32x4 ra0, ra1, ra2, ra3, rw0, rw1, rw2, rw3;
#define FP8Q_LOAD_TILES(koff)                                                                        \
    do {                                                                                             \
        ra0 = *reinterpret_cast<const u32x4 *>(a_base + FP8Q_AROW(0) * K + (koff));                 \
        ra1 = *reinterpret_cast<const u32x4 *>(a_base + FP8Q_AROW(1) * K + (koff));                 \
        ra2 = *reinterpret_cast<const u32x4 *>(a_base + FP8Q_AROW(2) * K + (koff));                 \
        ra3 = *reinterpret_cast<const u32x4 *>(a_base + FP8Q_AROW(3) * K + (koff));                 \
        rw0 = *reinterpret_cast<const u32x4 *>(w_base + (koff));                                    \
        rw1 = *reinterpret_cast<const u32x4 *>(w_base + 32 * K + (koff));                           \
        rw2 = *reinterpret_cast<const u32x4 *>(w_base + 64 * K + (koff));                           \
        rw3 = *reinterpret_cast<const u32x4 *>(w_base + 96 * K + (koff));                           \
    } while (0)
#define FP8Q_STORE_TILES(dst)                                                                        \
    do {                                                                                             \
        *reinterpret_cast<u32x4 *>((dst) + swz(rr, ch)) = ra0;                                       \
        *reinterpret_cast<u32x4 *>((dst) + swz(rr + 32, ch)) = ra1;                                  \
        *reinterpret_cast<u32x4 *>((dst) + swz(rr + 64, ch)) = ra2;                                  \
        *reinterpret_cast<u32x4 *>((dst) + swz(rr + 96, ch)) = ra3;                                  \
        *reinterpret_cast<u32x4 *>((dst) + kTile + swz(rr, ch)) = rw0;                               \
        *reinterpret_cast<u32x4 *>((dst) + kTile + swz(rr + 32, ch)) = rw1;                          \
        *reinterpret_cast<u32x4 *>((dst) + kTile + swz(rr + 64, ch)) = rw2;                          \
        *reinterpret_cast<u32x4 *>((dst) + kTile + swz(rr + 96, ch)) = rw3;                          \
    } while (0)

    FP8Q_LOAD_TILES(0);
    FP8Q_STORE_TILES(lds);
    float sa_cur[4], sa_nxt[4];
#pragma unroll
    for (int mi = 0; mi < 4; mi++) sa_cur[mi] = sa[FP8Q_MROW(mi)];
    float sw_cur = sw_row[0], sw_nxt = 0.f;
    __syncthreads();

    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    for (int64_t kb = 0; kb < KB; kb++) {
        const int buf = (int)(kb & 1);
        const bool more = kb + 1 < KB;
        if (more) {
            FP8Q_LOAD_TILES((kb + 1) * 128);
#pragma unroll
            for (int mi = 0; mi < 4; mi++) sa_nxt[mi] = sa[(kb + 1) * M + FP8Q_MROW(mi)];
            sw_nxt = sw_row[kb + 1];
        }

        const uint8_t *tA = lds + buf * 2 * kTile;
        const uint8_t *tW = tA + kTile;
        v8i wf[4], af[4];
#pragma unroll
        for (int ni = 0; ni < 4; ni++) wf[ni] = load_frag(tW, wn * 64 + ni * 16, lane);
#pragma unroll
        for (int mi = 0; mi < 4; mi++) af[mi] = load_frag(tA, wm * 64 + mi * 16, lane);
        v4f p[4][4];
#pragma unroll
        for (int ni = 0; ni < 4; ni++)
#pragma unroll
            for (int mi = 0; mi < 4; mi++) p[ni][mi] = mfma_fp8_16x16x128(wf[ni], af[mi], zero);
        float cs[4];
#pragma unroll
        for (int mi = 0; mi < 4; mi++) cs[mi] = sa_cur[mi] * sw_cur;
#pragma unroll
        for (int ni = 0; ni < 4; ni++)
#pragma unroll
            for (int mi = 0; mi < 4; mi++)
#pragma unroll
                for (int r = 0; r < 4; r++) acc[ni][mi][r] = __builtin_fmaf(p[ni][mi][r], cs[mi], acc[ni][mi][r]);

        if (more) {
            FP8Q_STORE_TILES(lds + (buf ^ 1) * 2 * kTile);
#pragma unroll
            for (int mi = 0; mi < 4; mi++) sa_cur[mi] = sa_nxt[mi];
            sw_cur = sw_nxt;
        }
        __syncthreads();
    }
#undef FP8Q_LOAD_TILES
#undef FP8Q_STORE_TILES
#undef FP8Q_AROW

    // Epilogue: lane holds C[m][n .. n+3] for each subtile.
#undef FP8Q_MROW
#pragma unroll
    for (int mi = 0; mi < 4; mi++) {
        const int64_t m = m0 + wm * 64 + mi * 16 + (lane & 15);
        if (m < M) {
#pragma unroll
            for (int ni = 0; ni < 4; ni++) {
                const int64_t n = n0 + wn * 64 + ni * 16 + 4 * (lane >> 4);
                store4<OUT_BF16>(c, m * N + n, acc[ni][mi]);
            }
        }
    }
}

template <bool GROUPED>
hipError_t launch(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c, bool out_bf16,
                  int64_t M, int64_t N, int64_t K, const int32_t *off, int64_t E, hipStream_t stream) {
    const int64_t n_mtiles = (M + kBM - 1) / kBM;
    const int64_t blocks = n_mtiles * (N / kBN);
    if (out_bf16)
        gemm_blockscaled_kernel<true, GROUPED>
            <<<dim3((unsigned)blocks), 256, 0, stream>>>(qa, sa, qw, sw, c, M, N, K, off, E, n_mtiles);
    else
        gemm_blockscaled_kernel<false, GROUPED>
            <<<dim3((unsigned)blocks), 256, 0, stream>>>(qa, sa, qw, sw, c, M, N, K, off, E, n_mtiles);
    return hipGetLastError();
}

}  // namespace

int64_t gemm_blocks(int64_t M, int64_t N) { return ((M + kBM - 1) / kBM) * (N / kBN); }

hipError_t launch_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                                   bool out_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return launch<false>(qa, sa, qw, sw, c, out_bf16, M, N, K, nullptr, 0, stream);
}

hipError_t launch_grouped_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw,
                                           void *c, bool out_bf16, const int32_t *off, int64_t E, int64_t M_total,
                                           int64_t N, int64_t K, hipStream_t stream) {
    return launch<true>(qa, sa, qw, sw, c, out_bf16, M_total, N, K, off, E, stream);
}

}  // namespace fp8q
