// MoE routing and the FP8 row gather for the grouped GEMM (page "DeepSeek starts updating frequently",
// deepinsightai.io, the list of TileKernels features: a gating step selects each token's top-k experts and a
// routing step maps tokens to experts; the DeepEP V2 test on the same page dispatches 8K tokens of hidden
// size 7168 to their top 8 experts in FP8).  The pages fix neither the tie rule nor the layout; this library
// takes: the k largest logits by decreasing value, the lower expert index first between equal logits (-0
// equals +0); one segment of rows per expert, in expert order, holding its tokens in ascending order and
// padded with empty rows (codes 0, scale 0) to a multiple of 128.
//
// Routing is three launches on the caller's stream:
//   1. moe_topk_kernel: one wave per chunk of 64 tokens, one lane per token.  Each lane keeps a sorted list of
//      its KMAX best (logit, expert) pairs while it scans its row (a batch of loads at a time), inserting a newcomer after every entry it does not strictly exceed, so the earlier
//      (lower) expert stays ahead of an equal logit.  The wave then ORs (1 << lane) into a 64-bit LDS mask per selected
//      expert; a lane's rank among the chunk's tokens of expert e is the popcount of e's mask below its lane,
//      and the chunk's count of e is the mask's popcount.  Both are independent of the order in which the
//      atomics land, so the result is deterministic.  Ranks go to row_of (finished in step 3), counts to the
//      workspace.
//   2. moe_scan_kernel: one workgroup turns the per-chunk counts into each chunk's first row per expert
//      (exclusive scan over chunks plus the expert's segment start), writes the padded segment offsets, and
//      marks empty rows (segment padding and rows past the last segment) with token -1.
//   3. moe_assign_kernel: row_of[t][j] = chunk base of (chunk(t), expert) + rank; row_token[row] = t.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fp8q_kernels.h"

// The routing's workspace for callers that cannot allocate: a file-scope device array of a fixed size, which
// each GPU the library runs on holds until the process ends.  Host code never passes `scratch` itself to a
// kernel (in host code the name is only a stand-in): its device address is looked up once per device with
// hipGetSymbolAddress and that address is used instead.
static __device__ __align__(256) int32_t scratch[fp8q::kRouteScratchBytes / 4];

namespace fp8q {
namespace {

constexpr int kChunk = 64;  // tokens per wave in steps 1 and 3

template <int KMAX>
__global__ __launch_bounds__(64) void moe_topk_kernel(const float *__restrict__ logits, int64_t T, int E, int k,
                                                      bool vec4, int32_t *__restrict__ topk_idx,
                                                      int32_t *__restrict__ rank,
                                                      int32_t *__restrict__ chunk_counts) {
    __shared__ unsigned long long mask[kMoeMaxExperts];
    const int lane = threadIdx.x;
    const int64_t c = blockIdx.x;
    const int64_t t = c * kChunk + lane;
    const bool valid = t < T;
    for (int e = lane; e < E; e += 64) mask[e] = 0ull;

    float val[KMAX];
    int idx[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; i++) {
        val[i] = -__builtin_inff();
        idx[i] = 0;
    }
    // Each lane reads its own row, NB logits per batch, every load of a batch in flight at once (16-byte
    // loads when rows are 16-byte aligned).  The batch loop is fully unrolled so the batch stays in registers.
    constexpr int NB = KMAX <= 8 ? 64 : 16;
    if (valid) {
        const float *row = logits + t * E;
        for (int e0 = 0; e0 < E; e0 += NB) {
            float v[NB];
            if (vec4 && e0 + NB <= E) {
#pragma unroll
                for (int u = 0; u < NB / 4; u++) {
                    const float4 f = *reinterpret_cast<const float4 *>(row + e0 + 4 * u);
                    v[4 * u] = f.x;
                    v[4 * u + 1] = f.y;
                    v[4 * u + 2] = f.z;
                    v[4 * u + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int u = 0; u < NB; u++) v[u] = e0 + u < E ? row[e0 + u] : 0.0f;
            }
            const int n = E - e0 < NB ? E - e0 : NB;
#pragma unroll
            for (int u = 0; u < NB; u++) {
                if (u >= n) continue;
                const int e = e0 + u;
                // Insert (v, e) into the descending list after every entry it does not strictly exceed
                // (those are larger, or equal and from a lower expert).  gt[i] is false up to the insertion
                // slot and true from it on; from the bottom up, each slot past it takes its upper neighbour.
                bool gt[KMAX];
#pragma unroll
                for (int i = 0; i < KMAX; i++) gt[i] = v[u] > val[i];
#pragma unroll
                for (int i = KMAX - 1; i > 0; i--) {
                    val[i] = gt[i] ? (gt[i - 1] ? val[i - 1] : v[u]) : val[i];
                    idx[i] = gt[i] ? (gt[i - 1] ? idx[i - 1] : e) : idx[i];
                }
                val[0] = gt[0] ? v[u] : val[0];
                idx[0] = gt[0] ? e : idx[0];
            }
        }
    }
    __syncthreads();  // masks cleared
    if (valid) {
#pragma unroll
        for (int j = 0; j < KMAX; j++)
            if (j < k) {
                topk_idx[t * k + j] = idx[j];
                atomicOr(&mask[idx[j]], 1ull << lane);
            }
    }
    __syncthreads();
    if (valid) {
        const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
        for (int j = 0; j < KMAX; j++)
            if (j < k) rank[t * k + j] = __popcll(mask[idx[j]] & below);
    }
    for (int e = lane; e < E; e += 64) chunk_counts[c * E + e] = __popcll(mask[e]);
}

// One workgroup of 1024 threads: thread (e, p) = (tid % E, tid / E) owns expert e's counts in chunk range p.
__global__ __launch_bounds__(1024) void moe_scan_kernel(int32_t *__restrict__ chunk, int64_t C, int E,
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ row_token, int64_t rows) {
    __shared__ int32_t part[1024];
    __shared__ int32_t total[kMoeMaxExperts];
    __shared__ int32_t seg[kMoeMaxExperts + 1];
    __shared__ int32_t scan[1024];
    const int tid = threadIdx.x;
    const int P = 1024 / E;
    const int e = tid % E, p = tid / E;
    const bool owner = p < P;
    const int64_t CP = (C + P - 1) / P;
    const int64_t c0 = owner ? p * CP : 0;
    const int64_t c1 = owner ? (c0 + CP < C ? c0 + CP : C) : 0;

    int32_t sum = 0;
    for (int64_t c = c0; c < c1; c += 8) {  // 8 loads in flight
        int32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = c + u < c1 ? chunk[(c + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < 8; u++) sum += v[u];
    }
    if (owner) part[p * E + e] = sum;
    __syncthreads();
    int32_t before = 0;  // counts of expert e in the chunk ranges before p
    if (owner) {
        for (int q = 0; q < p; q++) before += part[q * E + e];
        if (p == 0) {
            int32_t tot = 0;
            for (int q = 0; q < P; q++) tot += part[q * E + e];
            total[e] = tot;
        }
    }
    __syncthreads();
    // Padded segment sizes, inclusive scan over experts (Hillis-Steele in LDS).
    scan[tid] = tid < E ? (total[tid] + 127) / 128 * 128 : 0;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int32_t add = tid >= d ? scan[tid - d] : 0;
        __syncthreads();
        scan[tid] += add;
        __syncthreads();
    }
    if (tid < E) seg[tid + 1] = scan[tid];  // E may be 1024: thread e writes entry e + 1
    if (tid == 0) seg[0] = 0;
    __syncthreads();
    if (tid < E) offsets[tid + 1] = seg[tid + 1];
    if (tid == 0) offsets[0] = 0;
    // Each chunk's first row for expert e.
    if (owner) {
        int32_t run = seg[e] + before;
        for (int64_t c = c0; c < c1; c += 8) {
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) v[u] = c + u < c1 ? chunk[(c + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (c + u < c1) {
                    chunk[(c + u) * E + e] = run;
                    run += v[u];
                }
        }
    }
    // Empty rows: each segment's padding, then everything past the last segment.
    if (tid < E)
        for (int64_t r = seg[tid] + total[tid]; r < seg[tid + 1]; r++) row_token[r] = -1;
    for (int64_t r = seg[E] + tid; r < rows; r += 1024) row_token[r] = -1;
}

template <int KMAX>
__global__ __launch_bounds__(64) void moe_assign_kernel(const int32_t *__restrict__ topk_idx,
                                                        const int32_t *__restrict__ chunk_base, int64_t T, int E,
                                                        int k, int32_t *__restrict__ row_of,
                                                        int32_t *__restrict__ row_token, int64_t rows) {
    const int64_t c = blockIdx.x;
    const int64_t t = c * kChunk + threadIdx.x;
    if (t >= T) return;
    // All of the token's loads are issued before any is used (k independent chains).
    int e[KMAX], rk[KMAX], base[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; j++)
        if (j < k) {
            e[j] = topk_idx[t * k + j];
            rk[j] = row_of[t * k + j];
        }
#pragma unroll
    for (int j = 0; j < KMAX; j++)
        if (j < k) base[j] = chunk_base[c * E + e[j]];
#pragma unroll
    for (int j = 0; j < KMAX; j++)
        if (j < k) {
            const int64_t r = (int64_t)base[j] + rk[j];
            row_of[t * k + j] = (int32_t)r;
            if (r < rows) row_token[r] = (int32_t)t;
        }
}

// Expert-sorted FP8 rows, one launch with two kinds of workgroup (4 waves each):
//  - the first ceil(T / 4) scatter token rows: a wave reads its token's K codes once (8 KB per pass, 16 bytes
//    a lane) and stores them to each of the token's k rows (row_of), so every token row leaves HBM once even
//    though it lands in k places (reading per destination row re-fetched each token k times: the 500 MB of
//    output evicts the tokens from the Infinity Cache between their uses);
//  - the rest cover 64 consecutive rows each, in row order: lane i writes the scales of row r0 + i (each
//    store 256 contiguous bytes, the scale matrix is small enough to stay in L2) and the waves write zero
//    codes into the rows that carry no token.
// Rows at or past offsets[E] are not written; a row whose token is -1 (or outside [0, T)) gets zero codes
// and scale 0.
__global__ __launch_bounds__(256) void moe_gather_fp8_kernel(const uint8_t *__restrict__ q,
                                                             const float *__restrict__ s, int64_t T, int64_t K,
                                                             int k, const int32_t *__restrict__ row_of,
                                                             const int32_t *__restrict__ row_token,
                                                             const int32_t *__restrict__ offsets, int E,
                                                             int64_t rows, uint8_t *__restrict__ qa,
                                                             float *__restrict__ sa) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    constexpr int kU = 8;  // 16-byte loads in flight per lane
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int64_t used = offsets[E] < rows ? offsets[E] : rows;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t n16 = K >> 4;
    const int64_t scatter_blocks = (T + 3) / 4;

    if ((int64_t)blockIdx.x < scatter_blocks) {
        const int64_t t = (int64_t)blockIdx.x * 4 + wave;
        if (t >= T) return;
        const u32x4 *from = reinterpret_cast<const u32x4 *>(q + t * K);
        for (int64_t j0 = lane; j0 < n16; j0 += 64 * kU) {
            u32x4 v[kU];
#pragma unroll
            for (int u = 0; u < kU; u++) {
                const int64_t j = j0 + 64 * u;
                v[u] = j < n16 ? from[j] : zero;
            }
            for (int jj = 0; jj < k; jj++) {
                const int64_t r = __builtin_amdgcn_readfirstlane(row_of[t * k + jj]);
                if (r < 0 || r >= used) continue;
                u32x4 *to = reinterpret_cast<u32x4 *>(qa + r * K);
#pragma unroll
                for (int u = 0; u < kU; u++) {
                    const int64_t j = j0 + 64 * u;
                    if (j < n16) to[j] = v[u];
                }
            }
        }
        return;
    }

    const int64_t r0 = ((int64_t)blockIdx.x - scatter_blocks) * 64;
    if (r0 >= used) return;
    const int64_t KB = K >> 7;
    const int64_t rs = r0 + lane;
    int64_t src = rs < used ? row_token[rs] : -1;
    if (src >= T) src = -1;
    for (int64_t kb0 = wave; kb0 < KB; kb0 += 4 * kU) {
        float v[kU];
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int64_t kb = kb0 + 4 * u;
            v[u] = (kb < KB && src >= 0) ? s[kb * T + src] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kU; u++) {
            const int64_t kb = kb0 + 4 * u;
            if (kb < KB && rs < used) sa[kb * rows + rs] = v[u];
        }
    }
    for (int i = 0; i < 16; i++) {
        const int64_t r = r0 + wave * 16 + i;
        if (r >= used) break;
        const int64_t t = __builtin_amdgcn_readfirstlane(row_token[r]);
        if (t >= 0 && t < T) continue;  // written by the token's scatter wave
        u32x4 *to = reinterpret_cast<u32x4 *>(qa + r * K);
        for (int64_t j = lane; j < n16; j += 64) to[j] = zero;
    }
}

}  // namespace

int64_t moe_route_workspace_bytes(int64_t T, int64_t E) { return (T + kChunk - 1) / kChunk * E * 4; }

namespace {
constexpr int kScratchDevices = 64;
std::atomic<int32_t *> g_scratch[kScratchDevices];
std::mutex g_scratch_lock;
}  // namespace

hipError_t route_scratch(int dev, int32_t **ptr) {
    *ptr = nullptr;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    int32_t *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> g(g_scratch_lock);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            // `dev` is the current device (the caller checked), so this is that device's copy of the array.
            void *a = nullptr;
            const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
            if (e != hipSuccess || a == nullptr) {
                (void)hipGetLastError();
                return e != hipSuccess ? e : hipErrorInvalidSymbol;
            }
            p = static_cast<int32_t *>(a);
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_moe_route_topk(const float *logits, int64_t T, int E, int k, int32_t *topk_idx,
                                 int32_t *offsets, int32_t *row_of, int32_t *row_token, int64_t rows,
                                 int32_t *workspace, hipStream_t stream) {
    const int64_t C = (T + kChunk - 1) / kChunk;
    if (C > 0) {
        const bool vec4 = E % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
        if (k <= 8)
            moe_topk_kernel<8><<<dim3((unsigned)C), 64, 0, stream>>>(logits, T, E, k, vec4, topk_idx, row_of,
                                                                     workspace);
        else
            moe_topk_kernel<16><<<dim3((unsigned)C), 64, 0, stream>>>(logits, T, E, k, vec4, topk_idx, row_of,
                                                                      workspace);
    }
    moe_scan_kernel<<<1, 1024, 0, stream>>>(workspace, C, E, offsets, row_token, rows);
    if (C > 0) {
        if (k <= 8)
            moe_assign_kernel<8><<<dim3((unsigned)C), 64, 0, stream>>>(topk_idx, workspace, T, E, k, row_of,
                                                                       row_token, rows);
        else
            moe_assign_kernel<16><<<dim3((unsigned)C), 64, 0, stream>>>(topk_idx, workspace, T, E, k, row_of,
                                                                        row_token, rows);
    }
    return hipGetLastError();
}

hipError_t launch_moe_gather_fp8(const uint8_t *q, const float *s, int64_t T, int64_t K, int k,
                                 const int32_t *row_of, const int32_t *row_token, const int32_t *offsets, int E,
                                 int64_t rows, uint8_t *qa, float *sa, hipStream_t stream) {
    const int64_t blocks = (T + 3) / 4 + (rows + 63) / 64;
    if (blocks > 0)
        moe_gather_fp8_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(q, s, T, K, k, row_of, row_token, offsets,
                                                                          E, rows, qa, sa);
    return hipGetLastError();
}

}  // namespace fp8q
