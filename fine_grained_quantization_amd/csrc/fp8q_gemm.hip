// Block-scaled FP8 GEMM for gfx950: C = A * W^T with E4M3 operands, one fp32 scale per 1x128
// activation tile and per 128x128 weight block, and promotion of every 128-element partial sum into
// an fp32 accumulator (page "The Definitive Information To Deepseek": FP8 GEMM inputs with BF16/FP32
// outputs; promotion of partial results alongside the MMA).
//
// Three kernels share the same arithmetic:
//  * v_mfma_f32_16x16x128_f8f6f4 computes exactly one 128-deep K-block per instruction, so each
//    MFMA result is one fresh partial sum P (C input = 0) and promotion is acc += P * (s_a * s_w).
//  * Operand roles are swapped: the weight tile feeds the MFMA's row operand and the activation
//    tile its column operand, so a lane's 4 result registers are 4 consecutive output channels of
//    ONE token.  Every lane then promotes all its registers of a subtile with a single scalar
//    s_a[kb][m] * s_w[n/128][kb], and stores 4 adjacent outputs with one instruction.
//  * Operand tiles travel from global memory straight into LDS (buffer loads into LDS), rows stored
//    with a 16-byte-chunk XOR swizzle so that fragment reads are bank-conflict free.
// M > 256 runs the 256-row tile kernel (as do the grouped and gather-fused grouped GEMMs); M <= 64 the
// small-M kernel, whose waves split K; 64 < M <= 256 the mid-size kernel, whose waves split the tokens.
// The latter two give each CU one slice of weight rows, so the weights are streamed from HBM once.

#include <atomic>

#include "fp8q_device.h"
#include "fp8q_kernels.h"

namespace fp8q {

namespace {

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

// =============================================================================================
// Large-M kernel: 256 x BN workgroup tile (BN = 32 NSUB weight rows, NSUB = 6, 7 or 8), 8 waves: 4 along M
// x 2 along N, 64 tokens x 16 NSUB weight rows per wave, so 2 waves share each SIMD and one wave's promotion
// VALU work overlaps the other's MFMAs.  Global tiles go straight to LDS with buffer loads (no staging
// registers, K-block offset in a scalar register, rows past the end of the tile's range read as zeros);
// 2 LDS stages of (256 + BN) x 128 B plus the K-block's 256 activation scales and the weight scales of the
// (at most 3) 128-row blocks the tile touches, which travel with the tiles so that no load has to be waited
// for anywhere but at the stage barrier.  The host picks BN so that the number of tiles fills whole rounds
// of the CUs as far as possible.
// =============================================================================================

constexpr int kBig = 256;  // tile rows along M

int cu_count();  // multiprocessor count of the current device (cached)

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

// The same resource with a byte count of 0: every load through it is out of range and returns zeros without
// touching memory, whatever its per-lane and scalar offsets.
__device__ __forceinline__ i32x4 empty_rsrc(i32x4 r) {
    r[2] = 0;
    return r;
}

// Per-lane source offsets of one K-block tile.  Rows are copied 8 at a time (1 KB per instruction); lane l of
// an instruction lands in LDS slot l, i.e. row l / 8 of the 8, physical chunk l % 8, which must hold logical
// chunk (l % 8) ^ swzf(row).  Wave w copies A rows [32 w, 32 w + 32) and the W row groups g = w, w + 8, ...
template <int BN>
struct TileLoader {
    static constexpr int kWGroups = BN / 8;               // 8-row groups of the weight tile
    static constexpr int kWPerWave = (kWGroups + 7) / 8;  // groups per wave (the last may be partial)
    // Scale area of a stage, 8 x 256 B, one dword per lane of each wave's single scale copy: waves 0-3 copy
    // the activation scales of tile rows [64 w, 64 w + 64) (rows past the tile's last row read zeros), so
    // that row r sits at float r; waves 4-7 each copy the weight scales of blocks nb0, nb0 + 1, nb0 + 2
    // (clamped to the last block) into floats 256 + 64 (w - 4) + i.  The readers use wave 4's copy.
    static constexpr int kScOff = (kBig + BN) * 128;
    static constexpr int kStageBytes = kScOff + 8 * 256;
    i32x4 ra, rw, rsw;        // resources: this tile's A rows / W rows / the weight scales
    int avoff[4];             // A: row * K + chunk * 16 for the wave's 4 instructions
    int wvoff[kWPerWave];     // W: same for the wave's weight row groups
    int scvoff;               // this lane's scale offset (K-block 0)
    const float *sa_tile;     // activation scales of the tile's first row in K-block 0
    uint64_t sa_bytes;        // bytes of scales that belong to the tile's rows
    int64_t M;
    __device__ __forceinline__ void init(const uint8_t *a_rows, uint64_t a_bytes, const uint8_t *w_rows,
                                         uint64_t w_bytes, int64_t K, int wave, int lane, const float *sa_tile_,
                                         int64_t rows, int64_t M_, const float *sw_mat, int64_t NB, int64_t nb0) {
        ra = make_rsrc(a_rows, a_bytes);
        rw = make_rsrc(w_rows, w_bytes);
        const int64_t KB = K >> 7;
        rsw = make_rsrc(sw_mat, (uint64_t)NB * (uint64_t)KB * 4);
        const int64_t nb = nb0 + lane < NB - 1 ? nb0 + lane : NB - 1;
        scvoff = wave < 4 ? (wave * 64 + lane) * 4 : (lane < 3 ? (int)(nb * KB * 4) : kOutOfRange);
        sa_tile = sa_tile_;
        sa_bytes = (uint64_t)(rows < kBig ? rows : kBig) * 4;
        M = M_;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int r = wave * 32 + j * 8 + (lane >> 3);
            avoff[j] = (int)(r * K) + (((lane & 7) ^ swzf(r)) << 4);
        }
#pragma unroll
        for (int j = 0; j < kWPerWave; j++) {
            const int r = (wave + 8 * j) * 8 + (lane >> 3);
            wvoff[j] = (int)(r * K) + (((lane & 7) ^ swzf(r)) << 4);
        }
    }
    // The same tile when its A rows are token rows picked through a row -> token map (the FP8 dispatch folded
    // into the grouped GEMM): A row r of the tile is token rt[r] of q [T, K] (rows past `rows`, and rows whose
    // token is negative or >= T, read zeros), and its scale is s_tok[kb * T + token].
    __device__ __forceinline__ void init_gather(const uint8_t *q, int64_t T, const int32_t *rt, int64_t rows,
                                                const uint8_t *w_rows, uint64_t w_bytes, int64_t K, int wave,
                                                int lane, const float *s_tok, const float *sw_mat, int64_t NB,
                                                int64_t nb0) {
        ra = make_rsrc(q, (uint64_t)T * (uint64_t)K);
        rw = make_rsrc(w_rows, w_bytes);
        const int64_t KB = K >> 7;
        rsw = make_rsrc(sw_mat, (uint64_t)NB * (uint64_t)KB * 4);
        const int64_t nb = nb0 + lane < NB - 1 ? nb0 + lane : NB - 1;
        int64_t sc_tok = -1;
        if (wave < 4 && wave * 64 + lane < rows) sc_tok = rt[wave * 64 + lane];
        scvoff = wave < 4 ? (sc_tok >= 0 && sc_tok < T ? (int)(sc_tok * 4) : kOutOfRange)
                          : (lane < 3 ? (int)(nb * KB * 4) : kOutOfRange);
        sa_tile = s_tok;
        sa_bytes = (uint64_t)T * 4;
        M = T;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int r = wave * 32 + j * 8 + (lane >> 3);
            const int64_t tok = r < rows ? rt[r] : -1;
            avoff[j] = tok >= 0 && tok < T ? (int)(tok * K) + (((lane & 7) ^ swzf(r)) << 4) : kOutOfRange;
        }
#pragma unroll
        for (int j = 0; j < kWPerWave; j++) {
            const int r = (wave + 8 * j) * 8 + (lane >> 3);
            wvoff[j] = (int)(r * K) + (((lane & 7) ^ swzf(r)) << 4);
        }
    }
    // Copies K-block kb (koff = kb * 128) into `stage`, or, when `tiles` is false, no tile bytes at all: the
    // tile resources are then given zero bytes, so that every lane's load is out of range (and reads zeros)
    // whatever its offsets.  The scales of K-block ks (kb, clamped to the last block) come along, one dword
    // per lane from in-bounds addresses.
    __device__ __forceinline__ void issue(uint8_t *stage, bool tiles, int koff, int64_t ks, int wave) const {
        const bool act = wave < 4;  // wave-uniform: the resource and offset are scalar selects
        const i32x4 rs = act ? make_rsrc(sa_tile + ks * M, sa_bytes) : rsw;
        fp8q_raw_buffer_load_lds(rs, (lds_ptr)(stage + kScOff + wave * 256), 4, scvoff, act ? 0 : (int)(ks * 4), 0,
                                 0);
        const i32x4 ta = tiles ? ra : empty_rsrc(ra);  // `tiles` is wave-uniform: scalar selects
        const i32x4 tw = tiles ? rw : empty_rsrc(rw);
        const int so = tiles ? koff : 0;
#pragma unroll
        for (int j = 0; j < 4; j++)
            fp8q_raw_buffer_load_lds(ta, (lds_ptr)(stage + (wave * 32 + j * 8) * 128), 16, avoff[j], so, 0, 0);
#pragma unroll
        for (int j = 0; j < kWPerWave; j++) {
            const int g = wave + 8 * j;
            if (g < kWGroups)  // wave-uniform
                fp8q_raw_buffer_load_lds(tw, (lds_ptr)(stage + kBig * 128 + g * 1024), 16, wvoff[j], so, 0, 0);
        }
    }
};

// Workgroups are dispatched to the 8 XCDs round-robin (t % 8), 256 of them (one per CU) at a time.  This
// permutation gives XCD x the 32 consecutive indices [256 r + 32 x, +32) of each round r of 256; it is a
// bijection on every whole round.
__device__ __forceinline__ int64_t xcd_order(int64_t t) { return (t / 256) * 256 + (t % 8) * 32 + (t % 256) / 8; }

// Tile (mt, nt) of the i-th tile of a dense n_mt x n_nt grid, in an order made for the XCD permutation above:
// columns of 16 N tiles ("supergroup columns", the last may be narrower), each cut into supergroups of 16 M
// tiles (the last may be shorter), each enumerated as 8-wide sub-block columns of 4-high sub-blocks, M
// fastest.  Only tiles inside the grid are enumerated, so every round of 256 indices is 256 tiles whatever the
// grid's shape.  In a full 16 x 16 supergroup each XCD's 32 tiles form a 4 (M) x 8 (N) block sharing 4
// activation and 8 weight tile rows in that XCD's L2, and a round's 16 x 16 square shares its operands in the
// Infinity Cache.  Returns false past the last tile.
__device__ __forceinline__ bool dense_tile_at(int64_t i, int64_t n_mt, int64_t n_nt, int64_t &mt, int64_t &nt) {
    if (i >= n_mt * n_nt) return false;
    const int64_t colw = 16 * n_mt;
    const int64_t sgn = i / colw;
    const int64_t hn = n_nt - 16 * sgn < 16 ? n_nt - 16 * sgn : 16;
    int64_t j = i - sgn * colw;
    const int64_t sgm = j / (16 * hn);
    const int64_t hm = n_mt - 16 * sgm < 16 ? n_mt - 16 * sgm : 16;
    j -= sgm * 16 * hn;
    const int64_t qn = j / (8 * hm);
    const int64_t wq = hn - 8 * qn < 8 ? hn - 8 * qn : 8;
    j -= qn * 8 * hm;
    const int64_t qm = j / (4 * wq);
    const int64_t hq = hm - 4 * qm < 4 ? hm - 4 * qm : 4;
    j -= qm * 4 * wq;
    mt = 16 * sgm + 4 * qm + j % hq;
    nt = 16 * sgn + 8 * qn + j / hq;
    return true;
}

// Coordinates of dense tile i (over an n_mtiles x n_ntiles grid of 256 x bn tiles whose columns start at
// n_begin).  Returns false past the last tile.
__device__ __forceinline__ bool dense_tile(int64_t i, int64_t n_begin, int64_t n_mtiles, int64_t n_ntiles, int64_t bn,
                                           int64_t &m0, int64_t &n0) {
    int64_t mt, nt;
    if (!dense_tile_at(i, n_mtiles, n_ntiles, mt, nt)) return false;
    m0 = mt * kBig;
    n0 = n_begin + nt * bn;
    return true;
}

// Coordinates of grouped tile t: tiles are enumerated expert by expert (expert e owns ceil(len_e / 256) M
// tiles of its segment), tile T = mt * n_ntiles + nt with N fastest.  Workgroups are dealt to the 8 XCDs
// round-robin; the permutation below gives XCD x the 32 consecutive tiles [256 r + 32 x, +32) of each round r
// of 256, so the tiles sharing activation rows (and, mostly, an expert's weights) meet in one L2.  Returns
// false past the last expert's tiles.
__device__ __forceinline__ bool grouped_tile(int64_t t, const int32_t *__restrict__ off, int64_t E, int64_t M,
                                             int64_t n_mtiles, int64_t n_ntiles, int64_t bn, int lane, int64_t &m0,
                                             int64_t &mend, int64_t &n0, int64_t &e) {
    const int64_t T = xcd_order(t);
    const int64_t mt = T / n_ntiles;  // n_mtiles is an upper bound on the number of M tiles
    if (mt >= n_mtiles) return false;
    n0 = (T % n_ntiles) * bn;
    // The expert owning M tile mt: a prefix sum of the experts' tile counts, 64 experts per pass (lane i
    // holds expert base + i), and the first lane whose running total exceeds mt.
    // A segment is cut to [0, M) before its tiles are counted (in 64-bit arithmetic), so offsets that break
    // the layout rules can neither overflow the count nor yield rows outside the buffer.
    int64_t before = 0;
    for (int64_t base = 0; base < E; base += 64) {
        const int64_t i = base + lane;
        int lo = 0, hi = 0, cnt = 0;
        if (i < E) {
            const int64_t l = (int64_t)off[i] < 0 ? 0 : ((int64_t)off[i] > M ? M : (int64_t)off[i]);
            const int64_t h = (int64_t)off[i + 1] < l ? l : ((int64_t)off[i + 1] > M ? M : (int64_t)off[i + 1]);
            lo = (int)l;
            hi = (int)h;
            cnt = (int)((h - l + kBig - 1) / kBig);
        }
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(incl, d, 64);
            if (lane >= d) incl += u;
        }
        const uint64_t hit = __ballot(i < E && before + incl > mt);
        if (hit) {
            const int L = __builtin_ctzll(hit);
            e = base + L;
            const int lo_e = __shfl(lo, L, 64), hi_e = __shfl(hi, L, 64);
            const int64_t first = before + __shfl(incl, L, 64) - __shfl(cnt, L, 64);
            m0 = lo_e + (mt - first) * kBig;
            mend = hi_e;
            return m0 < mend;
        }
        before += __shfl(incl, 63, 64);
    }
    return false;
}

// One output tile of (512 / WAVES_N) rows x (16 NSUB WAVES_N) weight rows starting at (m0, n0): 8 waves, 8 /
// WAVES_N along M (64 tokens each) x WAVES_N along N (16 NSUB weight rows each).  WAVES_N = 2 is the 256-row
// tile; WAVES_N = 4 (NSUB = 4) is the 128 x 256 tile for grouped segments with 128 rows left.  W / SW are the
// weight matrix and its scales (an expert's, in the grouped case), and rows >= mend are not stored.
// stage0 / stage1 are the workgroup's two LDS stages, each at least TileLoader<BN>::kStageBytes.  With GATHER,
// qa / sa are token codes [T, K] and token scales [K/128][T], and output row r's activation row is token
// rtok[r] (the dispatch gather folded into the GEMM).
template <bool OUT_BF16, int NSUB, int WAVES_N, bool GATHER = false>
__device__ __forceinline__ void bs_tile(uint8_t *stage0, uint8_t *stage1, const uint8_t *__restrict__ qa,
                                        const float *__restrict__ sa, const uint8_t *__restrict__ W,
                                        const float *__restrict__ SW, void *__restrict__ c, int64_t M, int64_t N,
                                        int64_t K, int64_t m0, int64_t mend, int64_t n0,
                                        const int32_t *__restrict__ rtok = nullptr, int64_t T = 0) {
    constexpr int WM_WAVES = 8 / WAVES_N;
    constexpr int BN = 16 * NSUB * WAVES_N;
    constexpr int WN = 16 * NSUB;  // weight rows per wave
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;  // wave-uniform (scalar), 0 .. 7
    const int wm = wave % WM_WAVES;  // 64-token slab of the tile
    const int wn = wave / WM_WAVES;  // weight-row slab of the tile
    const int64_t KB = K >> 7;
    // Scales: the stage holds the activation scales of the tile's 256 rows and the weight scales of blocks
    // nb0, nb0 + 1, nb0 + 2 (the tile's weight rows start in block nb0 and span at most 3 blocks).  The
    // wave's weight rows start at nw0; subtiles ni < nib lie in block nbA, the others in nbA + 1 (a 16-row
    // subtile never straddles a 128-row block).  With NSUB = 8 the waves are aligned to whole blocks and
    // only nbA is used.
    const int64_t nb0 = n0 / 128;
    const int64_t nw0 = n0 + wn * WN;
    const int nbA = (int)(nw0 / 128 - nb0);  // 0 .. 2
    const int nbB = nbA + 1 < 2 ? nbA + 1 : 2;
    const int nib = (int)((128 * (nw0 / 128 + 1) - nw0) / 16);
    TileLoader<BN> ld;
    if constexpr (GATHER)
        ld.init_gather(qa, T, rtok + m0, mend - m0, W + n0 * K, (uint64_t)(N - n0) * (uint64_t)K, K, wave, lane,
                       sa, SW, N / 128, nb0);
    else
        ld.init(qa + m0 * K, (uint64_t)(mend - m0) * (uint64_t)K, W + n0 * K, (uint64_t)(N - n0) * (uint64_t)K, K,
                wave, lane, sa + m0, mend - m0, M, SW, N / 128, nb0);

    v4f acc[NSUB][4];
#pragma unroll
    for (int ni = 0; ni < NSUB; ni++)
#pragma unroll
        for (int mi = 0; mi < 4; mi++) acc[ni][mi] = (v4f){0.f, 0.f, 0.f, 0.f};

    // With GATHER, 16-row subtiles of the wave whose rows all read zeros (no token: the padding rows of an
    // expert segment, or rows past the segment) need no MFMA and no promotion: their accumulators stay 0,
    // which is their exact result.  live bit mi is set when subtile mi of this wave has a token row.
    uint32_t live = 0xF;
    if constexpr (GATHER) {
        const int64_t r = m0 + wm * 64 + lane;
        const int64_t tok = r < mend ? rtok[r] : -1;
        const uint64_t b = __ballot(tok >= 0 && tok < T);
        live = ((b & 0xFFFFull) ? 1u : 0u) | ((b & 0xFFFF0000ull) ? 2u : 0u) | ((b & 0xFFFF00000000ull) ? 4u : 0u) |
               ((b >> 48) ? 8u : 0u);
    }

    ld.issue(stage0, true, 0, 0, wave);
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    // The K-loop.  Waves with a subtile without a live bit take a partial form that skips that subtile's
    // fragment reads, MFMAs and promotions; full waves run the second loop, which has no branch in its body.
    // Both forms reach the same barriers.
    if (GATHER && live != 0xFu) {
        // The partial form: all weight fragments of the K-block are read first, then each live token subtile
        // runs its MFMAs and promotions against them (one wave-uniform test per subtile and K-block).
        for (int64_t kb = 0; kb < KB; kb++) {
            uint8_t *cur = (kb & 1) ? stage1 : stage0;
            uint8_t *nxt = (kb & 1) ? stage0 : stage1;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            ld.issue(nxt, kb + 1 < KB, (int)((kb + 1) * 128), kb + 1 < KB ? kb + 1 : kb, wave);
            const uint8_t *tW = cur + kBig * 128;
            v8i wfa[NSUB];
#pragma unroll
            for (int ni = 0; ni < NSUB; ni++) wfa[ni] = load_frag(tW, wn * WN + ni * 16, lane);
            const float *sc = reinterpret_cast<const float *>(cur + TileLoader<BN>::kScOff);
            const float swA = sc[256 + nbA], swB = sc[256 + nbB];
#pragma unroll
            for (int mi = 0; mi < 4; mi++) {
                if (!((live >> mi) & 1u)) continue;  // wave-uniform
                const v8i af = load_frag(cur, wm * 64 + mi * 16, lane);
                const float sa_m = sc[wm * 64 + mi * 16 + (lane & 15)];
#pragma unroll
                for (int ni = 0; ni < NSUB; ni++) {
                    const v4f p = mfma_fp8_16x16x128(wfa[ni], af, zero);
                    const float cs = sa_m * (NSUB == 8 || ni < nib ? swA : swB);
#pragma unroll
                    for (int r = 0; r < 4; r++) acc[ni][mi][r] = __builtin_fmaf(p[r], cs, acc[ni][mi][r]);
                }
            }
        }
    } else {
        for (int64_t kb = 0; kb < KB; kb++) {
            uint8_t *cur = (kb & 1) ? stage1 : stage0;
            uint8_t *nxt = (kb & 1) ? stage0 : stage1;
            // This K-block's tiles have landed (own loads), and every wave is done with the other stage.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            // The prefetch is unconditional (past the last K-block it copies no tiles and yields zeros), so
            // the loop body is a single basic block.
            ld.issue(nxt, kb + 1 < KB, (int)((kb + 1) * 128), kb + 1 < KB ? kb + 1 : kb, wave);
            // The first weight fragment is read before the activation fragments so that the first MFMA waits
            // for two LDS reads, not five.  The fragment of weight subtile ni+1 is read while the 4 MFMAs of
            // subtile ni run; their partials are promoted right after issue (the first MFMA has finished by
            // the time the 4th issues).
            const uint8_t *tW = cur + kBig * 128;
            v8i wf = load_frag(tW, wn * WN, lane);
            v8i af[4];
#pragma unroll
            for (int mi = 0; mi < 4; mi++) af[mi] = load_frag(cur, wm * 64 + mi * 16, lane);
            // Scales (needed from the first promotion on) of tokens wm * 64 + mi * 16 + (lane & 15).
            const float *sc = reinterpret_cast<const float *>(cur + TileLoader<BN>::kScOff);
            float sa_cur[4], csA[4];
#pragma unroll
            for (int mi = 0; mi < 4; mi++) sa_cur[mi] = sc[wm * 64 + mi * 16 + (lane & 15)];
            const float swA = sc[256 + nbA], swB = sc[256 + nbB];
#pragma unroll
            for (int mi = 0; mi < 4; mi++) csA[mi] = sa_cur[mi] * swA;
#pragma unroll
            for (int ni = 0; ni < NSUB; ni++) {
                v8i wf_next = wf;
                if (ni < NSUB - 1) wf_next = load_frag(tW, wn * WN + (ni + 1) * 16, lane);
                v4f p[4];
#pragma unroll
                for (int mi = 0; mi < 4; mi++) p[mi] = mfma_fp8_16x16x128(wf, af[mi], zero);
                float cs[4];
                if (NSUB == 8) {
#pragma unroll
                    for (int mi = 0; mi < 4; mi++) cs[mi] = csA[mi];
                } else {
                    const float swv = ni < nib ? swA : swB;  // scalar select
#pragma unroll
                    for (int mi = 0; mi < 4; mi++) cs[mi] = sa_cur[mi] * swv;
                }
#pragma unroll
                for (int mi = 0; mi < 4; mi++)
#pragma unroll
                    for (int r = 0; r < 4; r++) acc[ni][mi][r] = __builtin_fmaf(p[mi][r], cs[mi], acc[ni][mi][r]);
                wf = wf_next;
            }
        }
    }

    // Epilogue: lane holds C[m][n .. n+3] of each subtile; rows outside [m0, mend) are not stored.
    if constexpr (OUT_BF16) {
        // Through LDS, so that the stores are row-contiguous: each wave writes its 64 x WN bf16 block into
        // the (now idle) stages, waves 0-3 into stage0 and 4-7 into stage1, then reads it back 16 bytes per
        // lane along rows and stores whole row segments.  The 16-byte chunks of row r are rotated by r, which
        // spreads a column of rows over the banks while every row stays 16-byte aligned.
        constexpr int CPR = 2 * NSUB;  // 16-byte chunks per row of the block
        constexpr int RS = CPR * 16;
        static_assert(4 * 64 * RS <= TileLoader<BN>::kStageBytes, "epilogue staging");
        __builtin_amdgcn_s_waitcnt(0);  // the last (out-of-range) copies into the stages have retired
        __syncthreads();                // and every wave is done reading the stages
        uint8_t *blk = (wave < 4 ? stage0 : stage1) + (wave & 3) * 64 * RS;
#pragma unroll
        for (int mi = 0; mi < 4; mi++)
#pragma unroll
            for (int ni = 0; ni < NSUB; ni++) {
                const int r = mi * 16 + (lane & 15);
                const int ch = ni * 2 + (lane >> 5), half = (lane >> 4) & 1;
                uint2 o;
                o.x = pack_bf16x2(acc[ni][mi][0], acc[ni][mi][1]);
                o.y = pack_bf16x2(acc[ni][mi][2], acc[ni][mi][3]);
                *reinterpret_cast<uint2 *>(blk + r * RS + ((ch + r) % CPR) * 16 + half * 8) = o;
            }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPR; j++) {
            const int idx = j * 64 + lane;
            const int r = idx / CPR, ch = idx % CPR;
            const int64_t m = m0 + wm * 64 + r, n = nw0 + ch * 8;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(blk + r * RS + ((ch + r) % CPR) * 16);
            if (m < mend && n < N) *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(c) + m * N + n) = v;
        }
        return;
    }
#pragma unroll
    for (int mi = 0; mi < 4; mi++) {
        const int64_t m = m0 + wm * 64 + mi * 16 + (lane & 15);
        if (m < mend) {
#pragma unroll
            for (int ni = 0; ni < NSUB; ni++) {
                const int64_t n = nw0 + ni * 16 + 4 * (lane >> 4);
                if (n < N) store4<OUT_BF16>(c, m * N + n, acc[ni][mi]);
            }
        }
    }
}

// Large-M GEMM.  Dense: tiles [0, main_tiles) cover columns [0, n_tail) with 256 x (32 NSUB) tiles; when
// NSUB_TAIL != 0 the tiles after them cover columns [n_tail, N) with narrower 256 x (32 NSUB_TAIL) tiles,
// which are dispatched as the CUs finish their last main tiles and so fill the otherwise idle part of the
// last round.  Grouped (NSUB = 8): one 256 x 256 tile per workgroup, or 128 x 256 where a segment has
// only 128 rows left.
template <bool OUT_BF16, bool GROUPED, int NSUB, int NSUB_TAIL, bool GATHER = false>
__global__ __launch_bounds__(512, 1) void gemm_bs_256_kernel(const uint8_t *__restrict__ qa,
                                                             const float *__restrict__ sa,
                                                             const uint8_t *__restrict__ qw,
                                                             const float *__restrict__ sw, void *__restrict__ c,
                                                             int64_t M, int64_t N, int64_t K,
                                                             const int32_t *__restrict__ off, int64_t E,
                                                             int64_t n_mtiles, int64_t n_ntiles, int64_t main_tiles,
                                                             int64_t n_tail, int64_t n_ntiles_tail,
                                                             const int32_t *__restrict__ rtok = nullptr,
                                                             int64_t T = 0) {
    constexpr int kMain = TileLoader<32 * NSUB>::kStageBytes;
    constexpr int kTail = TileLoader<32 * (NSUB_TAIL ? NSUB_TAIL : NSUB)>::kStageBytes;
    constexpr int kStageBytes = kMain > kTail ? kMain : kTail;
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageBytes];
    const int64_t t = blockIdx.x;
    int64_t m0, mend = M, n0;
    if constexpr (GROUPED) {
        int64_t e = 0;
        if (!grouped_tile(t, off, E, M, n_mtiles, n_ntiles, 32 * NSUB, threadIdx.x & 63, m0, mend, n0, e)) return;
        // The expert and the row range are the same in every lane, but they come out of lane shuffles, so the
        // compiler cannot prove it; without these the buffer descriptors built from them would sit in VGPRs and
        // every buffer load of the main loop would be wrapped in a loop over distinct descriptor values.
        e = __builtin_amdgcn_readfirstlane((int)e);
        m0 = __builtin_amdgcn_readfirstlane((int)m0);
        mend = __builtin_amdgcn_readfirstlane((int)mend);
        const uint8_t *W = qw + e * N * K;
        const float *SW = sw + e * (N / 128) * (K >> 7);
        if (mend - m0 <= 128)  // a segment's last 128 rows: the 128 x 256 layout does no work on absent rows
            bs_tile<OUT_BF16, 4, 4, GATHER>(stage0, stage1, qa, sa, W, SW, c, M, N, K, m0, mend, n0, rtok, T);
        else
            bs_tile<OUT_BF16, NSUB, 2, GATHER>(stage0, stage1, qa, sa, W, SW, c, M, N, K, m0, mend, n0, rtok, T);
        return;
    }
    // Dense: the main tiles, then (NSUB_TAIL != 0) the narrower tail tiles, as one sequence of tiles in XCD
    // order, so the tail tiles fill the main tiles' last round.
    const int64_t i = xcd_order(t);
    if constexpr (NSUB_TAIL != 0) {
        if (i >= main_tiles) {
            if (!dense_tile(i - main_tiles, n_tail, n_mtiles, n_ntiles_tail, 32 * NSUB_TAIL, m0, n0)) return;
            bs_tile<OUT_BF16, NSUB_TAIL, 2>(stage0, stage1, qa, sa, qw, sw, c, M, N, K, m0, M, n0);
            return;
        }
    }
    if (!dense_tile(i, 0, n_mtiles, n_ntiles, 32 * NSUB, m0, n0)) return;
    bs_tile<OUT_BF16, NSUB, 2>(stage0, stage1, qa, sa, qw, sw, c, M, N, K, m0, M, n0);
}

// Launch plan of the dense large-M kernel: main tile width 32 ns over columns [0, n_tail), then (ns_tail != 0)
// tiles of width 32 ns_tail over [n_tail, N).
struct Plan256 {
    int ns, ns_tail;
    int64_t n_tail;
};

// Relative cost of one tile of width bn: its width, with narrower tiles charged for their extra operand
// traffic per flop (half their width deficit; measured: 4096 x 18432 runs best at 256 wide, 4096 x 7168 at
// 224).
static double tile_cost(int64_t bn) { return (double)bn * (1.0 + 0.5 * (256.0 - (double)bn) / 256.0); }

// Finishing time of tm tiles of cost a followed by t2 tiles of cost b on ncu CUs, each CU taking the next
// tile as it becomes free (the dispatcher's order).
static double makespan(int64_t tm, double a, int64_t t2, double b, int64_t ncu) {
    const int64_t R = tm / ncu, rem = tm % ncu;
    const double t1 = (double)R * a;                 // ncu - rem CUs are free from here
    const double t2e = rem ? (double)(R + 1) * a : t1;  // the other rem CUs from here
    if (t2 == 0) return t2e;
    const int64_t early = ncu - rem;
    const int64_t k = rem ? (int64_t)(a / b) : 0;  // tail tiles an early CU finishes before t2e
    const int64_t done = t2 < early * k ? t2 : early * k;
    const int64_t left = t2 - done;
    if (left == 0) {
        const double e = t1 + (double)((done + early - 1) / early) * b;
        return e > t2e ? e : t2e;
    }
    const double base = t1 + (double)k * b > t2e ? t1 + (double)k * b : t2e;
    return base + (double)((left + ncu - 1) / ncu) * b;
}

Plan256 plan_256(int64_t M, int64_t N, int64_t ncu) {
    const int64_t n_mt = (M + kBig - 1) / kBig;
    Plan256 best{8, 0, N};
    double best_cost = -1.0;
    for (int ns = 8; ns >= 6; ns--) {
        const int64_t bn = 32 * ns;
        const int64_t n_nt = (N + bn - 1) / bn;
        const double a = tile_cost(bn);
        double cost = makespan(n_mt * n_nt, a, 0, 0.0, ncu);
        Plan256 p{ns, 0, N};
        // Split: as many whole tile columns as fill whole rounds, the rest in narrower tiles.
        const int64_t T = n_mt * n_nt;
        const int64_t cols = (T / ncu) * ncu / n_mt;
        if (T % ncu != 0 && cols >= 1 && cols < n_nt) {
            const int64_t n_split = cols * bn;
            for (int nt : {4, 6}) {
                const int64_t bnt = 32 * nt;
                const int64_t t2 = n_mt * ((N - n_split + bnt - 1) / bnt);
                const double c2 = makespan(n_mt * cols, a, t2, tile_cost(bnt), ncu);
                if (c2 < cost * 0.98) {
                    cost = c2;
                    p = Plan256{ns, nt, n_split};
                }
            }
        }
        if (best_cost < 0.0 || cost < best_cost * 0.999) {
            best = p;
            best_cost = cost;
        }
    }
    return best;
}


template <bool OUT_BF16, int NSUB, int NSUB_TAIL>
hipError_t launch_256_dense(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                            int64_t M, int64_t N, int64_t K, int64_t n_tail, hipStream_t stream) {
    const int64_t n_mt = (M + kBig - 1) / kBig;
    const int64_t n_nt = (n_tail + 32 * NSUB - 1) / (32 * NSUB);
    const int64_t main_tiles = n_mt * n_nt;
    const int64_t n_nt_tail = NSUB_TAIL != 0 ? (N - n_tail + 32 * NSUB_TAIL - 1) / (32 * NSUB_TAIL) : 0;
    // whole rounds of 256 workgroups (the XCD permutation is a bijection on each); indices past the last
    // tile exit at once
    const int64_t blocks = (main_tiles + n_mt * n_nt_tail + 255) / 256 * 256;
    gemm_bs_256_kernel<OUT_BF16, false, NSUB, NSUB_TAIL><<<dim3((unsigned)blocks), 512, 0, stream>>>(
        qa, sa, qw, sw, c, M, N, K, nullptr, 0, n_mt, n_nt, main_tiles, n_tail, n_nt_tail);
    return hipGetLastError();
}

template <bool OUT_BF16, int NSUB>
hipError_t launch_256_dense_t(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                              int64_t M, int64_t N, int64_t K, const Plan256 &p, hipStream_t stream) {
    switch (p.ns_tail) {
        case 4: return launch_256_dense<OUT_BF16, NSUB, 4>(qa, sa, qw, sw, c, M, N, K, p.n_tail, stream);
        case 6: return launch_256_dense<OUT_BF16, NSUB, 6>(qa, sa, qw, sw, c, M, N, K, p.n_tail, stream);
        default: return launch_256_dense<OUT_BF16, NSUB, 0>(qa, sa, qw, sw, c, M, N, K, N, stream);
    }
}

template <bool OUT_BF16>
hipError_t launch_256(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c, int64_t M,
                      int64_t N, int64_t K, hipStream_t stream) {
    const Plan256 p = plan_256(M, N, cu_count());
    switch (p.ns) {
        case 6: return launch_256_dense_t<OUT_BF16, 6>(qa, sa, qw, sw, c, M, N, K, p, stream);
        case 7: return launch_256_dense_t<OUT_BF16, 7>(qa, sa, qw, sw, c, M, N, K, p, stream);
        default: return launch_256_dense_t<OUT_BF16, 8>(qa, sa, qw, sw, c, M, N, K, p, stream);
    }
}

// Tile rows of a grouped launch over M rows and E experts: enough for any offsets that do not decrease.
int64_t grouped_mtiles(int64_t M, int64_t E) { return M / kBig + E; }

template <bool OUT_BF16>
hipError_t launch_256_grouped(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                              int64_t M, int64_t N, int64_t K, const int32_t *off, int64_t E, hipStream_t stream) {
    constexpr int64_t BN = 256;
    const int64_t n_ntiles = (N + BN - 1) / BN;
    // Every expert owns ceil(len / 256) tiles of its segment cut to [0, M).  When the offsets do not decrease
    // the cut segments are disjoint, so the counts add up to at most M / 256 + E tile rows (M / 256 + E / 2
    // when every length is a multiple of 128); the rows past the real tiles exit at once.
    const int64_t n_mtiles = grouped_mtiles(M, E);
    // whole rounds of 256 workgroups: the XCD permutation of the tile index is a bijection on each round,
    // and the indices past the last tile exit at once
    const int64_t blocks = grouped_gemm_blocks(M, N, E);
    gemm_bs_256_kernel<OUT_BF16, true, 8, 0><<<dim3((unsigned)blocks), 512, 0, stream>>>(
        qa, sa, qw, sw, c, M, N, K, off, E, n_mtiles, n_ntiles, blocks, N, 0);
    return hipGetLastError();
}

// The grouped GEMM reading its activation rows through the row -> token map (same tiles and order).
template <bool OUT_BF16>
hipError_t launch_256_grouped_gather(const uint8_t *q, const float *s, int64_t T, const int32_t *rtok,
                                     const uint8_t *qw, const float *sw, void *c, int64_t M, int64_t N, int64_t K,
                                     const int32_t *off, int64_t E, hipStream_t stream) {
    constexpr int64_t BN = 256;
    const int64_t n_ntiles = (N + BN - 1) / BN;
    const int64_t n_mtiles = grouped_mtiles(M, E);
    const int64_t blocks = grouped_gemm_blocks(M, N, E);
    gemm_bs_256_kernel<OUT_BF16, true, 8, 0, true><<<dim3((unsigned)blocks), 512, 0, stream>>>(
        q, s, qw, sw, c, M, N, K, off, E, n_mtiles, n_ntiles, blocks, N, 0, rtok, T);
    return hipGetLastError();
}

// =============================================================================================
// Small-M kernel (M <= 64, decode-shaped): the weight matrix is streamed from HBM exactly once.
// The N rows are dealt out in slices of R rows (a multiple of 8, chosen on the host so that there is one
// slice per CU), one workgroup of 8 waves per slice.  The waves split K: wave w takes K-blocks w, w + 8, ...
// For each of its K-blocks a wave copies the slice's weight rows and the 64 activation rows, as whole
// 128-byte lines, straight into its own LDS slot (buffer loads into LDS), waits, and multiplies them with
// MFMAs (NSUB = ceil(R / 16) weight subtiles x 4 token subtiles), promoting each partial with its scales.
// With 8 waves per CU, 8 K-blocks per CU are in flight.  The 8 partial sums then go to LDS, and each wave
// adds up (in wave order, so deterministically) and stores an eighth of the slice's outputs.  Every load is
// unconditional: rows past the slice or past M and K-blocks past the end read zeros.
// =============================================================================================

constexpr int kSmallM = 64;
constexpr int kDecWaves = 8;
constexpr int kDecMaxSub = 5;  // LDS: 8 waves x (5 x 2 KB weight + 8 KB activation) = 144 KB, 8 x 20 KB partials

template <bool OUT_BF16, int NSUB>
__global__ __launch_bounds__(512, 1) void gemm_smallm_kernel(const uint8_t *__restrict__ qa,
                                                             const float *__restrict__ sa,
                                                             const uint8_t *__restrict__ qw,
                                                             const float *__restrict__ sw, void *__restrict__ c,
                                                             int64_t M, int64_t N, int64_t K, int64_t rows_per_wg) {
    constexpr int kW = NSUB * 16 * 128;
    constexpr int kA = kSmallM * 128;
    constexpr int kSlotBytes = kW + kA + 512;  // + the K-block's 64 token scales and 64 weight-scale slots
    constexpr int kPart = NSUB * 4 * 64 * 16;  // one wave's partial sums
    constexpr int kLds = kDecWaves * kSlotBytes > kDecWaves * kPart ? kDecWaves * kSlotBytes : kDecWaves * kPart;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
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
    // Scales travel with the K-block's copies: lane t copies token t's scale (tokens past M copy a scale
    // that is never used, or zero past the end), lanes 0 and 1 copy the weight scales of blocks nb0 and
    // nb0 + 1 (the slice spans at most two 128-row blocks), the other lanes zeros.  This lane's weight rows
    // 16 ns + 4 (lane / 16) .. +3 lie in one block.
    const int64_t nb0 = n0 / 128;
    const i32x4 rSW = make_rsrc(sw, (uint64_t)(N / 128) * (uint64_t)KB * 4);
    const int64_t nbl = nb0 + lane < N / 128 - 1 ? nb0 + lane : N / 128 - 1;
    const int sw_voff = lane < 2 ? (int)(nbl * KB * 4) : kOutOfRange;
    int sw_idx[NSUB];
#pragma unroll
    for (int ns = 0; ns < NSUB; ns++) {
        int64_t nb = (n0 + ns * 16 + 4 * (lane >> 4)) / 128;
        nb = nb < N / 128 ? nb : N / 128 - 1;
        sw_idx[ns] = (int)(nb - nb0);  // 0 or 1
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
    // Past the last K-block (kb >= KB, wave-uniform) the resources are given zero bytes, so every load reads
    // zeros without touching memory.
    auto issue = [&](int kb) {
        const bool in = kb < KB;
        const int so = in ? kb * 128 : 0;
        const i32x4 tw = in ? rw : empty_rsrc(rw), ta = in ? rA : empty_rsrc(rA);
        const i32x4 ts = in ? rS : empty_rsrc(rS), tsw = in ? rSW : empty_rsrc(rSW);
#pragma unroll
        for (int j = 0; j < 2 * NSUB; j++)
            fp8q_raw_buffer_load_lds(tw, (__attribute__((address_space(3))) void *)(wslot + j * 1024), 16, w_voff[j],
                                     so, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; j++)
            fp8q_raw_buffer_load_lds(ta, (__attribute__((address_space(3))) void *)(aslot + j * 1024), 16, a_voff[j],
                                     so, 0, 0);
        // (the K-block's offset in the per-lane offset, which the hardware range-checks: tokens past M in the
        // last K-block then read zeros; the scalar offset is not range-checked)
        fp8q_raw_buffer_load_lds(ts, (__attribute__((address_space(3))) void *)(aslot + kA), 4,
                                 lane * 4 + (in ? kb * (int)M * 4 : 0), 0, 0, 0);
        fp8q_raw_buffer_load_lds(tsw, (__attribute__((address_space(3))) void *)(aslot + kA + 256), 4, sw_voff,
                                 in ? kb * 4 : 0, 0, 0);
    };

    const int NI = (KB + kDecWaves - 1) / kDecWaves;
    issue(wave);
    const float *ssl = reinterpret_cast<const float *>(aslot + kA);
    for (int i = 0; i < NI; i++) {
        __builtin_amdgcn_s_waitcnt(0);  // copies (and scales) of K-block wave + 8 i have landed
        v8i af[4], wf[NSUB];
#pragma unroll
        for (int mi = 0; mi < 4; mi++) af[mi] = load_frag(aslot, mi * 16, lane);
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++) wf[ns] = load_frag(wslot, ns * 16, lane);
        float s4[4], swv[NSUB];
#pragma unroll
        for (int mi = 0; mi < 4; mi++) s4[mi] = ssl[mi * 16 + (lane & 15)];
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++) swv[ns] = ssl[64 + sw_idx[ns]];
        float cs[NSUB][4];
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++)
#pragma unroll
            for (int mi = 0; mi < 4; mi++) cs[ns][mi] = s4[mi] * swv[ns];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // fragments and scales are in registers: the slot may be overwritten
        issue(wave + kDecWaves * (i + 1));
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

    // Reduction of the 8 K-split partials: once every wave is done with its slot, each writes its partial
    // (NSUB x 4 subtile pairs) to LDS; then wave w sums pairs w, w + 8, w + 16 over the waves in order and
    // stores them.
    __syncthreads();
#pragma unroll
    for (int ns = 0; ns < NSUB; ns++)
#pragma unroll
        for (int mi = 0; mi < 4; mi++)
            *reinterpret_cast<v4f *>(lds + wave * kPart + ((ns * 4 + mi) * 64 + lane) * 16) = acc[ns][mi];
    __syncthreads();
#pragma unroll
    for (int q0 = 0; q0 < NSUB * 4; q0 += kDecWaves) {
        const int q = q0 + wave;  // wave-uniform
        if (q < NSUB * 4) {
            v4f s = *reinterpret_cast<const v4f *>(lds + (q * 64 + lane) * 16);
#pragma unroll
            for (int w = 1; w < kDecWaves; w++) {
                const v4f v = *reinterpret_cast<const v4f *>(lds + w * kPart + (q * 64 + lane) * 16);
                s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
            }
            const int ns = q >> 2, mi = q & 3;
            const int nl = ns * 16 + 4 * (lane >> 4);  // 4 rows nl .. nl+3 of the slice (all in or all out)
            const int64_t m = mi * 16 + (lane & 15);
            if (m < M && nl < nrows) store4<OUT_BF16>(c, m * N + n0 + nl, s);
        }
    }
}

// =============================================================================================
// Mid-size M kernel (64 < M <= 256, MT = 128 or 256 token rows): as in the small-M kernel, the N rows are dealt
// out in slices of R rows (one slice per CU, R <= 80), so the weight matrix is streamed from HBM exactly once by
// all CUs; here every workgroup holds all MT token rows, and the 8 waves split the tokens instead of K: wave w
// owns token subtiles w, w + 8, ... (MT / 128 of them) and all NSUB weight subtiles, so each output has one
// owner and no partial sums are exchanged.  The K-blocks flow through a ring of LDS stages shared by the waves:
// each stage holds a K-block's weight rows, its MT token rows and their scales, copied with buffer loads straight
// into LDS (rows past the slice or past M read zeros), and the copies run (stages - 1) K-blocks ahead of the
// MFMAs.  Every wave issues the same number of copy instructions per K-block, so the number of its loads still
// in flight is the same constant every iteration: where a wave has nothing to copy, it loads through a
// zero-byte resource into a scratch area of LDS that nothing reads (a load into LDS that is out of range still
// writes its zeros).
// =============================================================================================

template <int MT>
struct MidShape {
    static_assert(MT == 128 || MT == 256, "token rows per workgroup");
    static constexpr int kTpw = MT / 128;                       // token subtiles per wave
    static constexpr int kCopies = 2 * kTpw + 3;                // token groups, 2 weight groups, 1 scale dword
    static constexpr int kStages = MT == 128 ? 5 : 3;           // 135 KB / 131 KB of LDS with 80-row slices
};

template <bool OUT_BF16, int NSUB, int MT>
__global__ __launch_bounds__(512, 1) void gemm_midm_kernel(const uint8_t *__restrict__ qa,
                                                           const float *__restrict__ sa,
                                                           const uint8_t *__restrict__ qw,
                                                           const float *__restrict__ sw, void *__restrict__ c,
                                                           int64_t M, int64_t N, int64_t K, int64_t rows_per_wg) {
    using MS = MidShape<MT>;
    constexpr int S = MS::kStages;
    constexpr int TPW = MS::kTpw;
    constexpr int kW = NSUB * 16 * 128;   // weight rows of one K-block
    constexpr int kA = MT * 128;          // token rows of one K-block
    constexpr int kSa = kW + kA;          // MT token scales
    constexpr int kSw = kSa + MT * 4;     // weight scales of blocks nb0, nb0 + 1 (64 slots)
    constexpr int kStage = kSw + 256;
    constexpr int kDummy = S * kStage;    // 1 KB that absorbs the zeros of the loads with nothing to copy
    static_assert(2 * NSUB <= 16, "at most 16 weight row groups");
    static_assert(kDummy + 1024 <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kDummy + 1024];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;
    const int KB = (int)(K >> 7);
    const int64_t n0 = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t nrows = (N - n0) < rows_per_wg ? (N - n0) : rows_per_wg;

    const i32x4 rw = make_rsrc(qw + n0 * K, (uint64_t)nrows * (uint64_t)K);
    const i32x4 rA = make_rsrc(qa, (uint64_t)M * (uint64_t)K);
    const i32x4 rS = make_rsrc(sa, (uint64_t)M * (uint64_t)KB * 4);
    const int64_t nb0 = n0 / 128;
    const i32x4 rSW = make_rsrc(sw, (uint64_t)(N / 128) * (uint64_t)KB * 4);

    // Copy assignment.  Row groups of 8 rows (1 KB, one instruction): lane l lands in row 8 j + l / 8, physical
    // chunk l % 8, which holds logical chunk (l % 8) ^ swzf(row).  Wave w copies token groups w, w + 8, ...
    // (MT / 64 of them), weight groups w and w + 8 (when they exist), and one scale dword per lane: waves
    // 0 .. MT / 64 - 1 the token scales of tokens [64 w, 64 w + 64), wave MT / 64 the weight scales of blocks nb0
    // and nb0 + 1 (lanes 0 and 1).
    constexpr int kTokWaves = MT / 64;
    const int rsub = lane >> 3;
    int a_voff[2 * TPW], w_voff[2];
#pragma unroll
    for (int j = 0; j < 2 * TPW; j++) {
        const int r = 8 * (wave + 8 * j) + rsub;
        a_voff[j] = r * (int)K + (((lane & 7) ^ swzf(r)) << 4);
    }
#pragma unroll
    for (int j = 0; j < 2; j++) w_voff[j] = a_voff[j];  // the same rows 8 (w + 8 j) + l / 8 of the weight slice
    const bool has_w0 = wave < 2 * NSUB, has_w1 = wave + 8 < 2 * NSUB;  // wave-uniform
    const bool tok_sc = wave < kTokWaves, w_sc = wave == kTokWaves;
    const int64_t nbl = nb0 + lane < N / 128 - 1 ? nb0 + lane : N / 128 - 1;
    const int sc_voff = tok_sc ? (wave * 64 + lane) * 4 : (lane < 2 ? (int)(nbl * KB * 4) : kOutOfRange);
    const int sc_lds = tok_sc ? kSa + wave * 256 : kSw;
    int sw_idx[NSUB];  // weight-scale slot (0 or 1) of this lane's 4 rows 16 ns + 4 (lane / 16) .. +3
#pragma unroll
    for (int ns = 0; ns < NSUB; ns++) {
        int64_t nb = (n0 + ns * 16 + 4 * (lane >> 4)) / 128;
        nb = nb < N / 128 ? nb : N / 128 - 1;
        sw_idx[ns] = (int)(nb - nb0);
    }

    // Copies of K-block kb into its stage; past the last K-block (kb >= KB, wave-uniform) every resource has zero
    // bytes, so the loads read zeros without touching memory (and still count as issued loads).
    auto issue = [&](int kb) {
        uint8_t *st = lds + (kb % S) * kStage;
        const bool in = kb < KB;
        const int so = in ? kb * 128 : 0;
        const i32x4 ta = in ? rA : empty_rsrc(rA);
        const i32x4 tw0 = in && has_w0 ? rw : empty_rsrc(rw), tw1 = in && has_w1 ? rw : empty_rsrc(rw);
        // Token scales: the K-block's offset goes into the per-lane offset, which the hardware range-checks, so
        // tokens past M in the last K-block read zeros (the scalar offset is not range-checked).
        const i32x4 ts = !in ? empty_rsrc(rS) : (tok_sc ? rS : (w_sc ? rSW : empty_rsrc(rSW)));
        const int svo = tok_sc && in ? sc_voff + kb * (int)M * 4 : sc_voff;
        const int sso = w_sc && in ? kb * 4 : 0;
#pragma unroll
        for (int j = 0; j < 2 * TPW; j++)
            fp8q_raw_buffer_load_lds(ta, (lds_ptr)(st + kW + (wave + 8 * j) * 1024), 16, a_voff[j], so, 0, 0);
        fp8q_raw_buffer_load_lds(tw0, (lds_ptr)(has_w0 ? st + wave * 1024 : lds + kDummy), 16, w_voff[0], so, 0, 0);
        fp8q_raw_buffer_load_lds(tw1, (lds_ptr)(has_w1 ? st + (wave + 8) * 1024 : lds + kDummy), 16, w_voff[1], so,
                                 0, 0);
        fp8q_raw_buffer_load_lds(ts, (lds_ptr)(tok_sc || w_sc ? st + sc_lds : lds + kDummy), 4, svo, sso, 0, 0);
    };

    v4f acc[TPW][NSUB];
#pragma unroll
    for (int t = 0; t < TPW; t++)
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++) acc[t][ns] = (v4f){0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < S - 1; s++) issue(s);
    for (int kb = 0; kb < KB; kb++) {
        // This wave's copies of K-block kb have landed (those of the next S - 2 may still be in flight); after
        // the barrier every wave's have, and every wave is done with the stage K-block kb - 1 used.  (A plain
        // s_barrier: __syncthreads would also wait for every load in flight.  The stage's data was written by the
        // loads, and every read of the freed stage has returned, as its MFMAs and products consumed it.)
        __builtin_amdgcn_s_waitcnt(vmcnt_le<(S - 2) * MS::kCopies>());
        __builtin_amdgcn_s_barrier();
        issue(kb + S - 1);
        const uint8_t *st = lds + (kb % S) * kStage;
        const float *ssc = reinterpret_cast<const float *>(st + kSa);
        const float *wsc = reinterpret_cast<const float *>(st + kSw);
        v8i af[TPW], wf[NSUB];
#pragma unroll
        for (int t = 0; t < TPW; t++) af[t] = load_frag(st + kW, (wave + 8 * t) * 16, lane);
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++) wf[ns] = load_frag(st, ns * 16, lane);
        float s_tok[TPW];
#pragma unroll
        for (int t = 0; t < TPW; t++) s_tok[t] = ssc[(wave + 8 * t) * 16 + (lane & 15)];
        const float sw0 = wsc[0], sw1 = wsc[1];
#pragma unroll
        for (int ns = 0; ns < NSUB; ns++)
#pragma unroll
            for (int t = 0; t < TPW; t++) {
                const v4f p = mfma_fp8_16x16x128(wf[ns], af[t], zero);
                const float cs = s_tok[t] * (sw_idx[ns] ? sw1 : sw0);
#pragma unroll
                for (int r = 0; r < 4; r++) acc[t][ns][r] = __builtin_fmaf(p[r], cs, acc[t][ns][r]);
            }
    }
    // Lane holds C[m][n .. n+3] of each subtile, m = 16 (wave + 8 t) + lane % 16, n = 16 ns + 4 (lane / 16)
    // within the slice; rows n are all in or all out of the slice.
    __builtin_amdgcn_s_waitcnt(0);  // the last (zero-byte) copies have retired before the workgroup ends
#pragma unroll
    for (int t = 0; t < TPW; t++) {
        const int64_t m = (wave + 8 * t) * 16 + (lane & 15);
        if (m < M) {
#pragma unroll
            for (int ns = 0; ns < NSUB; ns++) {
                const int nl = ns * 16 + 4 * (lane >> 4);
                if (nl < nrows) store4<OUT_BF16>(c, m * N + n0 + nl, acc[t][ns]);
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

template <bool OUT_BF16, int MT>
hipError_t launch_midm(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c, int64_t M,
                       int64_t N, int64_t K, hipStream_t stream) {
    // The small-M kernel's slices: a multiple of 8 rows giving about one slice per CU, at most 5 subtiles.
    const int64_t ncu = cu_count();
    int64_t rows = 8 * ((N / 8 + ncu - 1) / ncu);
    rows = rows < 16 * kDecMaxSub ? rows : 16 * kDecMaxSub;
    const int nsub = (int)((rows + 15) / 16);
    const dim3 grid((unsigned)((N + rows - 1) / rows));
    switch (nsub) {
#define FP8Q_MIDM_CASE(S)                                                                                  \
    case S:                                                                                                \
        gemm_midm_kernel<OUT_BF16, S, MT><<<grid, 512, 0, stream>>>(qa, sa, qw, sw, c, M, N, K, rows);     \
        break;
        FP8Q_MIDM_CASE(1)
        FP8Q_MIDM_CASE(2)
        FP8Q_MIDM_CASE(3)
        FP8Q_MIDM_CASE(4)
        FP8Q_MIDM_CASE(5)
#undef FP8Q_MIDM_CASE
    }
    return hipGetLastError();
}

}  // namespace

int64_t grouped_gemm_blocks(int64_t M, int64_t N, int64_t E) {
    if (M < 0 || N < 0 || E < 1 || E > (int64_t(1) << 31)) return -1;
    const int64_t mt = grouped_mtiles(M, E), nt = (N + 255) / 256;
    if (nt > 0 && mt > (int64_t(1) << 40) / nt) return -1;
    return (mt * nt + 255) / 256 * 256;
}

int64_t gemm_blocks(int64_t M, int64_t N) {
    // an upper bound over the kernels: 256 x 128 tiles at the narrowest, or one workgroup per 8 weight rows
    return ((M + kBig - 1) / kBig) * ((N + 127) / 128) + 256 + (N + 7) / 8;
}

hipError_t launch_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw, void *c,
                                   bool out_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (M <= kSmallM)
        return out_bf16 ? launch_smallm<true>(qa, sa, qw, sw, c, M, N, K, stream)
                        : launch_smallm<false>(qa, sa, qw, sw, c, M, N, K, stream);
    if (M <= 128)
        return out_bf16 ? launch_midm<true, 128>(qa, sa, qw, sw, c, M, N, K, stream)
                        : launch_midm<false, 128>(qa, sa, qw, sw, c, M, N, K, stream);
    if (M <= 256)
        return out_bf16 ? launch_midm<true, 256>(qa, sa, qw, sw, c, M, N, K, stream)
                        : launch_midm<false, 256>(qa, sa, qw, sw, c, M, N, K, stream);
    return out_bf16 ? launch_256<true>(qa, sa, qw, sw, c, M, N, K, stream)
                    : launch_256<false>(qa, sa, qw, sw, c, M, N, K, stream);
}

hipError_t launch_grouped_gemm_blockscaled(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw,
                                           void *c, bool out_bf16, const int32_t *off, int64_t E, int64_t M_total,
                                           int64_t N, int64_t K, hipStream_t stream) {
    return out_bf16 ? launch_256_grouped<true>(qa, sa, qw, sw, c, M_total, N, K, off, E, stream)
                    : launch_256_grouped<false>(qa, sa, qw, sw, c, M_total, N, K, off, E, stream);
}

hipError_t launch_grouped_gemm_gather(const uint8_t *q, const float *s, int64_t T, const int32_t *row_token,
                                      const uint8_t *qw, const float *sw, void *c, bool out_bf16,
                                      const int32_t *off, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                      hipStream_t stream) {
    return out_bf16 ? launch_256_grouped_gather<true>(q, s, T, row_token, qw, sw, c, M_total, N, K, off, E, stream)
                    : launch_256_grouped_gather<false>(q, s, T, row_token, qw, sw, c, M_total, N, K, off, E, stream);
}

}  // namespace fp8q
