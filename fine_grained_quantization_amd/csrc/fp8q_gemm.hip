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
#include <atomic>

#include "fp8q_device.h"
#include "fp8q_kernels.h"

namespace fp8q {

namespace {

constexpr int kBM = 128;            // tokens per workgroup tile
constexpr int kBN = 128;            // weight rows per workgroup tile (one scale block)
constexpr int kTile = 128 * 128;    // bytes of one operand tile for one K-block

// LDS placement of a tile row: row r (128 bytes = 8 chunks of 16 bytes) stores logical chunk c at
// physical chunk c ^ swzf(r).  Fragment reads touch 16 consecutive rows at one logical chunk; swzf is a
// permutation of 0..7 within each aligned group of 8 rows and also within the 8 even and the 8 odd
// rows of each aligned group of 16, so those reads are bank-conflict free whether the LDS serves 8
// lanes (128 bytes) or 16 lanes (256 bytes) of a 16-byte read per cycle.
__device__ __forceinline__ int swzf(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ swzf(r)) << 4); }

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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
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

// =============================================================================================
// Large-M kernel: 256 x 256 workgroup tile, 8 waves (4 along M x 2 along N, 64 x 128 per wave, so
// 2 waves share each SIMD and one wave's promotion VALU work overlaps the other's MFMAs).  Global
// tiles go straight to LDS with buffer loads (no staging registers, K-block offset in a scalar
// register, rows past the end of the tile's range read as zeros); 2 LDS stages of 64 KB
// (A 256 x 128 B + W 256 x 128 B).  Each wave's 128 weight rows are exactly one 128-row scale
// block, so its weight scale is one scalar per K-block.
// =============================================================================================

constexpr int kBig = 256;                  // tile rows along M and along N
constexpr int kStageBytes = 2 * kBig * 128;  // A + W bytes of one K-block

typedef __attribute__((address_space(3))) void *lds_ptr;

// Buffer resource for `bytes` bytes at `base` (raw buffer: stride 0, range-checked by byte offset).
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)(uint32_t)(a >> 32);  // stride 0
    r[2] = (int)(uint32_t)(bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull);
    r[3] = 0x00020000;
    return r;
}

// Per-lane source offsets of one K-block tile.  Wave w fills tile rows [32 w, 32 w + 32) of A and of W,
// 8 rows (1 KB) per instruction; lane l of an instruction lands in LDS slot l, i.e. row l / 8, physical
// chunk l % 8, which must hold logical chunk (l % 8) ^ swzf(row).
struct TileLoader {
    i32x4 ra, rw;   // resources: this tile's A rows / W rows
    int voff[4];    // row * K + chunk * 16 for the 4 instructions (same rows in A and W)
    __device__ __forceinline__ void init(const uint8_t *a_rows, uint64_t a_bytes, const uint8_t *w_rows,
                                         uint64_t w_bytes, int64_t K, int wave, int lane) {
        ra = make_rsrc(a_rows, a_bytes);
        rw = make_rsrc(w_rows, w_bytes);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int r = wave * 32 + j * 8 + (lane >> 3);
            voff[j] = (int)(r * K) + (((lane & 7) ^ swzf(r)) << 4);
        }
    }
    __device__ __forceinline__ void issue(uint8_t *stage, int koff, int wave) const {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            fp8q_raw_buffer_load_lds(ra, (lds_ptr)(stage + (wave * 32 + j * 8) * 128), 16, voff[j], koff, 0, 0);
            fp8q_raw_buffer_load_lds(rw, (lds_ptr)(stage + kBig * 128 + (wave * 32 + j * 8) * 128), 16, voff[j], koff,
                                0, 0);
        }
    }
};

template <bool OUT_BF16, bool GROUPED>
__global__ __launch_bounds__(512, 1) void gemm_bs_256_kernel(const uint8_t *__restrict__ qa,
                                                             const float *__restrict__ sa,
                                                             const uint8_t *__restrict__ qw,
                                                             const float *__restrict__ sw, void *__restrict__ c,
                                                             int64_t M, int64_t N, int64_t K,
                                                             const int32_t *__restrict__ off, int64_t E,
                                                             int64_t n_mtiles, int64_t n_tiles) {
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int wm = wave & 3;   // 64-token quarter of the tile
    const int wn = wave >> 2;  // 128-row half of the weight tile
    const int64_t KB = K >> 7;

    // Tiles in launch order, M fastest: the 256 workgroups resident at a time cover all M tiles of a few
    // N columns, so each K-block slice of A is fetched once per wave of tiles and reused from L2.
    // (Measured faster than grouping tiles per XCD.)
    const int64_t t = blockIdx.x;
    if (t >= n_tiles) return;

    int64_t m0, mend, n0;
    const uint8_t *W = qw;
    const float *SW = sw;
    if (!GROUPED) {
        m0 = (t % n_mtiles) * kBig;
        n0 = (t / n_mtiles) * kBig;
        mend = M;
    } else {
        // Tiles are enumerated expert by expert: expert e owns ceil(len_e / 256) M tiles of its segment.
        // N is the fastest index here, so the workgroups resident together cover few experts and share
        // both their weights and their activation rows in L2.
        const int64_t n_ntiles = n_tiles / n_mtiles;  // n_mtiles is an upper bound on the number of M tiles
        const int64_t mt = t / n_ntiles;
        n0 = (t % n_ntiles) * kBig;
        int64_t before = 0, e = -1;
        for (int64_t i = 0; i < E; i++) {
            const int64_t lo = off[i], hi = off[i + 1];
            const int64_t cnt = hi > lo ? (hi - lo + kBig - 1) / kBig : 0;
            if (mt < before + cnt) {
                e = i;
                m0 = lo + (mt - before) * kBig;
                mend = hi < M ? hi : M;
                break;
            }
            before += cnt;
        }
        if (e < 0) return;  // beyond the last expert's tiles
        W = qw + e * N * K;
        SW = sw + e * (N / 128) * KB;
    }
    const int64_t Mlast = mend - 1;
    TileLoader ld;
    ld.init(qa + m0 * K, (uint64_t)(mend - m0) * (uint64_t)K, W + n0 * K, (uint64_t)(N - n0) * (uint64_t)K, K,
            wave, lane);

    // Scales: this lane's 4 tokens (one per 16-row subtile) and this wave's weight scale block.
    int64_t mrow[4];
#pragma unroll
    for (int mi = 0; mi < 4; mi++) {
        const int64_t m = m0 + wm * 64 + mi * 16 + (lane & 15);
        mrow[mi] = m < Mlast ? m : Mlast;
    }
    int64_t nb = (n0 + wn * 128) / 128;
    nb = nb < N / 128 ? nb : N / 128 - 1;
    const float *sw_row = SW + nb * KB;

    v4f acc[8][4];
#pragma unroll
    for (int ni = 0; ni < 8; ni++)
#pragma unroll
        for (int mi = 0; mi < 4; mi++) acc[ni][mi] = (v4f){0.f, 0.f, 0.f, 0.f};

    ld.issue(stage0, 0, wave);
    float sa_cur[4], sa_nxt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mi = 0; mi < 4; mi++) sa_cur[mi] = sa[mrow[mi]];
    float sw_cur = sw_row[0], sw_nxt = 0.f;
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    for (int64_t kb = 0; kb < KB; kb++) {
        uint8_t *cur = (kb & 1) ? stage1 : stage0;
        uint8_t *nxt = (kb & 1) ? stage0 : stage1;
        // This K-block's tiles have landed (own loads), and every wave is done with the other stage.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        {
            // The prefetch is unconditional (past the last K-block it reads nothing and yields zeros), so
            // the loop body is a single basic block.
            const int64_t kn = kb + 1 < KB ? kb + 1 : kb;
            ld.issue(nxt, kb + 1 < KB ? (int)((kb + 1) * 128) : kOutOfRange, wave);
#pragma unroll
            for (int mi = 0; mi < 4; mi++) sa_nxt[mi] = sa[kn * M + mrow[mi]];
            sw_nxt = sw_row[kn];
        }
        float cs[4];
#pragma unroll
        for (int mi = 0; mi < 4; mi++) cs[mi] = sa_cur[mi] * sw_cur;
        v8i af[4];
#pragma unroll
        for (int mi = 0; mi < 4; mi++) af[mi] = load_frag(cur, wm * 64 + mi * 16, lane);
        const uint8_t *tW = cur + kBig * 128;
        // The fragment of weight subtile ni+1 is read from LDS while the 4 MFMAs of subtile ni run; their
        // partials are promoted right after issue (the first MFMA has finished by the time the 4th issues).
        v8i wf = load_frag(tW, wn * 128, lane);
#pragma unroll
        for (int ni = 0; ni < 8; ni++) {
            v8i wf_next = wf;
            if (ni < 7) wf_next = load_frag(tW, wn * 128 + (ni + 1) * 16, lane);
            v4f p[4];
#pragma unroll
            for (int mi = 0; mi < 4; mi++) p[mi] = mfma_fp8_16x16x128(wf, af[mi], zero);
#pragma unroll
            for (int mi = 0; mi < 4; mi++)
#pragma unroll
                for (int r = 0; r < 4; r++) acc[ni][mi][r] = __builtin_fmaf(p[mi][r], cs[mi], acc[ni][mi][r]);
            wf = wf_next;
        }
#pragma unroll
        for (int mi = 0; mi < 4; mi++) sa_cur[mi] = sa_nxt[mi];
        sw_cur = sw_nxt;
    }

    // Epilogue: lane holds C[m][n .. n+3] of each subtile; rows outside [m0, mend) are not stored.
#pragma unroll
    for (int mi = 0; mi < 4; mi++) {
        const int64_t m = m0 + wm * 64 + mi * 16 + (lane & 15);
        if (m < mend) {
#pragma unroll
            for (int ni = 0; ni < 8; ni++) {
                const int64_t n = n0 + wn * 128 + ni * 16 + 4 * (lane >> 4);
                if (n < N) store4<OUT_BF16>(c, m * N + n, acc[ni][mi]);
            }
        }
    }
}

template <bool OUT_BF16, bool GROUPED>
hipError_t launch_256(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c, int64_t M,
                      int64_t N, int64_t K, const int32_t *off, int64_t E, hipStream_t stream) {
    // Grouped: every expert owns ceil(len / 256) tiles; since lengths are multiples of 128 that is at
    // most len / 256 + 1/2 each, so M / 256 + ceil(E / 2) tiles cover all experts.
    const int64_t n_mtiles = GROUPED ? M / kBig + (E + 1) / 2 : (M + kBig - 1) / kBig;
    const int64_t n_tiles = n_mtiles * ((N + kBig - 1) / kBig);
    const int64_t blocks = n_tiles;
    gemm_bs_256_kernel<OUT_BF16, GROUPED>
        <<<dim3((unsigned)blocks), 512, 0, stream>>>(qa, sa, qw, sw, c, M, N, K, off, E, n_mtiles, n_tiles);
    return hipGetLastError();
}

// =============================================================================================
// Small-M kernel (M <= 64, decode-shaped): the weight matrix is streamed from HBM exactly once.
// The N rows are dealt out in slices of R rows (a multiple of 8, chosen on the host so that there is one
// slice per CU), one workgroup of 8 waves per slice.  The waves split K: wave w takes K-blocks w, w + 8, ...
// For each of its K-blocks a wave copies the slice's weight rows and the 64 activation rows, as whole
// 128-byte lines, straight into its own LDS slot (buffer loads into LDS), waits, and multiplies them with
// MFMAs (NSUB = ceil(R / 16) weight subtiles x 4 token subtiles), promoting each partial with its scales.
// With 8 waves per CU, 8 K-blocks per CU are in flight.  The 8 partial sums are then added through LDS
// in a fixed tree order (deterministic) and wave 0 stores the slice.  Every load is unconditional:
// rows past the slice or past M and K-blocks past the end read zeros.
// =============================================================================================

constexpr int kSmallM = 64;
constexpr int kDecWaves = 8;
constexpr int kDecMaxSub = 5;  // LDS: 8 waves x (5 x 2 KB weight + 8 KB activation) = 144 KB

template <bool OUT_BF16, int NSUB>
__global__ __launch_bounds__(512, 1) void gemm_smallm_kernel(const uint8_t *__restrict__ qa,
                                                             const float *__restrict__ sa,
                                                             const uint8_t *__restrict__ qw,
                                                             const float *__restrict__ sw, void *__restrict__ c,
                                                             int64_t M, int64_t N, int64_t K, int64_t rows_per_wg) {
    constexpr int kW = NSUB * 16 * 128;
    constexpr int kA = kSmallM * 128;
    constexpr int kSlotBytes = kW + kA;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kDecWaves * kSlotBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int KB = (int)(K >> 7);
    const int64_t n0 = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t nrows = (N - n0) < rows_per_wg ? (N - n0) : rows_per_wg;
    uint8_t *wslot = lds + wave * kSlotBytes;
    uint8_t *aslot = wslot + kW;

    const i32x4 rw = make_rsrc(qw + n0 * K, (uint64_t)nrows * (uint64_t)K);
    const i32x4 rA = make_rsrc(qa, (uint64_t)M * (uint64_t)K);
    const i32x4 rS = make_rsrc(sa, (uint64_t)M * (uint64_t)KB * 4);
    // DMA placement: instruction j covers rows 8 j .. 8 j + 7; lane l lands in row 8 j + l / 8, physical chunk
    // l % 8, which holds logical chunk (l % 8) ^ swzf(row).  The rows in j are 8 j + l / 8 for both operands.
    const int rsub = lane >> 3;
    int a_voff[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int r = 8 * j + rsub;
        a_voff[j] = r * (int)K + (((lane & 7) ^ swzf(r)) << 4);
    }
    int w_voff[2 * NSUB];
#pragma unroll
    for (int j = 0; j < 2 * NSUB; j++) {
        const int r = 8 * j + rsub;
        w_voff[j] = r * (int)K + (((lane & 7) ^ swzf(r)) << 4);
    }
    // Scales: token scale offsets per token subtile; this lane's weight rows 16 ns + 4 (lane / 16) .. +3 lie in
    // one 128-row scale block (the slice start is a multiple of 8).
    int s_voff[4];
#pragma unroll
    for (int mi = 0; mi < 4; mi++) {
        const int tok = mi * 16 + (lane & 15);
        s_voff[mi] = tok < M ? tok * 4 : kOutOfRange;
    }
    const float *sw_lane[NSUB];
#pragma unroll
    for (int ns = 0; ns < NSUB; ns++) {
        int64_t nb = (n0 + ns * 16 + 4 * (lane >> 4)) / 128;
        nb = nb < N / 128 ? nb : N / 128 - 1;
        sw_lane[ns] = sw + nb * KB;
    }

    v4f acc[NSUB][4];
#pragma unroll
    for (int ns = 0; ns < NSUB; ns++)
#pragma unroll
        for (int mi = 0; mi < 4; mi++) acc[ns][mi] = (v4f){0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    // Per K-block: wait for its copies, read all its fragments into registers, then start the copies of the
    // wave's next K-block into the (now free) slot, and only then run the MFMAs and promotions, which
    // overlap with those copies.
    auto issue = [&](int kb, float (&s4)[4], float (&swv)[NSUB]) {
        const int so = kb < KB ? kb * 128 : kOutOfRange;
#pragma unroll
        for (int j = 0; j < 2 * NSUB; j++)
            fp8q_raw_buffer_load_lds(rw, (__attribute__((address_space(3))) void *)(wslot + j * 1024), 16, w_voff[j],
                                     so, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; j++)
            fp8q_raw_buffer_load_lds(rA, (__attribute__((address_space(3))) void *)(aslot + j * 1024), 16, a_voff[j],
                                     so, 0, 0);
        const int sso = kb < KB ? kb * (int)M * 4 : kOutOfRange;
#pragma unroll
        for (int mi = 0; mi < 4; mi++) s4[mi] = fp8q_raw_buffer_load_f32(rS, s_voff[mi], sso, 0);
        const int kbc = kb < KB ? kb : KB - 1;
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++) swv[ns] = sw_lane[ns][kbc];
    };

    const int NI = (KB + kDecWaves - 1) / kDecWaves;
    float s4[4], swv[NSUB];
    issue(wave, s4, swv);
    for (int i = 0; i < NI; i++) {
        __builtin_amdgcn_s_waitcnt(0);  // copies (and scales) of K-block wave + 8 i have landed
        v8i af[4], wf[NSUB];
#pragma unroll
        for (int mi = 0; mi < 4; mi++) af[mi] = load_frag(aslot, mi * 16, lane);
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++) wf[ns] = load_frag(wslot, ns * 16, lane);
        float cs[NSUB][4];
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++)
#pragma unroll
            for (int mi = 0; mi < 4; mi++) cs[ns][mi] = s4[mi] * swv[ns];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // fragments are in registers: the slot may be overwritten
        issue(wave + kDecWaves * (i + 1), s4, swv);
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++) {
            v4f p[4];
#pragma unroll
            for (int mi = 0; mi < 4; mi++) p[mi] = mfma_fp8_16x16x128(wf[ns], af[mi], zero);
#pragma unroll
            for (int mi = 0; mi < 4; mi++)
#pragma unroll
                for (int r = 0; r < 4; r++) acc[ns][mi][r] = __builtin_fmaf(p[mi][r], cs[ns][mi], acc[ns][mi][r]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the last (out-of-range) copies have retired before the slot is reused

    // Tree reduction of the 8 K-split partials through LDS (fixed order): waves [h, 2h) hand their partial
    // to waves [0, h), for h = 4, 2, 1.  A partial is NSUB * 4 * 64 lanes * 16 bytes <= 20 KB.
    constexpr int kPart = NSUB * 4 * 64 * 16;
#pragma unroll
    for (int h = 4; h >= 1; h >>= 1) {
        __syncthreads();
        if (wave >= h && wave < 2 * h) {
            uint8_t *dst = lds + (wave - h) * kPart;
#pragma unroll
            for (int ns = 0; ns < NSUB; ns++)
#pragma unroll
                for (int mi = 0; mi < 4; mi++)
                    *reinterpret_cast<v4f *>(dst + ((ns * 4 + mi) * 64 + lane) * 16) = acc[ns][mi];
        }
        __syncthreads();
        if (wave < h) {
            const uint8_t *src = lds + wave * kPart;
#pragma unroll
            for (int ns = 0; ns < NSUB; ns++)
#pragma unroll
                for (int mi = 0; mi < 4; mi++) {
                    const v4f v = *reinterpret_cast<const v4f *>(src + ((ns * 4 + mi) * 64 + lane) * 16);
                    acc[ns][mi][0] += v[0]; acc[ns][mi][1] += v[1]; acc[ns][mi][2] += v[2]; acc[ns][mi][3] += v[3];
                }
        }
    }
    if (wave == 0) {
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++) {
            const int nl = ns * 16 + 4 * (lane >> 4);  // 4 rows nl .. nl+3 of the slice (all in or all out)
#pragma unroll
            for (int mi = 0; mi < 4; mi++) {
                const int64_t m = mi * 16 + (lane & 15);
                if (m < M && nl < nrows) store4<OUT_BF16>(c, m * N + n0 + nl, acc[ns][mi]);
            }
        }
    }
}

int cu_count() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v == 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        v = (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
                ? prop.multiProcessorCount
                : 256;
        if (v <= 0) v = 256;
        cached.store(v, std::memory_order_relaxed);
    }
    return v;
}

template <bool OUT_BF16>
hipError_t launch_smallm(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c, int64_t M,
                         int64_t N, int64_t K, hipStream_t stream) {
    // Slice rows: a multiple of 8 giving about one slice per CU, at most 5 subtiles (80 rows).
    const int64_t ncu = cu_count();
    int64_t rows = 8 * ((N / 8 + ncu - 1) / ncu);
    rows = rows < 16 * kDecMaxSub ? rows : 16 * kDecMaxSub;
    const int nsub = (int)((rows + 15) / 16);
    const dim3 grid((unsigned)((N + rows - 1) / rows));
    switch (nsub) {
#define FP8Q_SMALLM_CASE(S)                                                                                  \
    case S:                                                                                                  \
        gemm_smallm_kernel<OUT_BF16, S><<<grid, kDecWaves * 64, 0, stream>>>(qa, sa, qw, sw, c, M, N, K, rows); \
        break;
        FP8Q_SMALLM_CASE(1)
        FP8Q_SMALLM_CASE(2)
        FP8Q_SMALLM_CASE(3)
        FP8Q_SMALLM_CASE(4)
        FP8Q_SMALLM_CASE(5)
#undef FP8Q_SMALLM_CASE
    }
    return hipGetLastError();
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

int64_t gemm_blocks(int64_t M, int64_t N) {
    return ((M + kBM - 1) / kBM) * (N / kBN) + 8 * 1024;  // generous upper bound over both kernels
}

hipError_t launch_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                                   bool out_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (M <= kSmallM)
        return out_bf16 ? launch_smallm<true>(qa, sa, qw, sw, c, M, N, K, stream)
                        : launch_smallm<false>(qa, sa, qw, sw, c, M, N, K, stream);
    if (M <= 128) return launch<false>(qa, sa, qw, sw, c, out_bf16, M, N, K, nullptr, 0, stream);
    return out_bf16 ? launch_256<true, false>(qa, sa, qw, sw, c, M, N, K, nullptr, 0, stream)
                    : launch_256<false, false>(qa, sa, qw, sw, c, M, N, K, nullptr, 0, stream);
}

hipError_t launch_grouped_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw,
                                           void *c, bool out_bf16, const int32_t *off, int64_t E, int64_t M_total,
                                           int64_t N, int64_t K, hipStream_t stream) {
    return out_bf16 ? launch_256<true, true>(qa, sa, qw, sw, c, M_total, N, K, off, E, stream)
                    : launch_256<false, true>(qa, sa, qw, sw, c, M_total, N, K, off, E, stream);
}

}  // namespace fp8q
