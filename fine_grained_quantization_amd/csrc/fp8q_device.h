// Device-side helpers shared by the gfx950 kernels of the fp8q library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int fp8q_i32x4 __attribute__((ext_vector_type(4)));

// LLVM's raw buffer load into LDS (buffer_load_dwordx4 ... lds): per-lane byte offset `voffset`, scalar
// byte offset `soffset`; the `size` bytes of lane l land at the wave's LDS address + size * l.  Reads at
// or past the resource's byte count return zeros.
__device__ void fp8q_raw_buffer_load_lds(fp8q_i32x4 rsrc, __attribute__((address_space(3))) void *lds, int size,
                                         int voffset, int soffset, int offset,
                                         int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// LLVM's raw buffer loads into registers (16 bytes / 4 bytes per lane); out-of-range reads return 0.
__device__ fp8q_i32x4 fp8q_raw_buffer_load_b128(fp8q_i32x4 rsrc, int voffset, int soffset,
                                                int aux) __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ float fp8q_raw_buffer_load_f32(fp8q_i32x4 rsrc, int voffset, int soffset,
                                          int aux) __asm("llvm.amdgcn.raw.buffer.load.f32");

namespace fp8q {

typedef fp8q_i32x4 i32x4;

// A byte offset past every buffer this library builds (they are < 2^31 bytes): loads there return 0
// without touching memory.
constexpr int kOutOfRange = 0x7FFFFFF0;
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: the data is read once).
__device__ __forceinline__ u32x4 load_stream16(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// RN64(1/448).  For every bf16 amax, fl32((double)amax * kInv448) equals the IEEE fp32 quotient
// amax / 448.0f: the double product is within 2^-52 (relative) of amax/448, while amax/448 stays
// at least 2^-28 (relative) away from every fp32 rounding midpoint and never sits on one, so both
// round to the same fp32 value.
constexpr double kInv448 = 1.0 / 448.0;

// Low / high bf16 halves of a packed dword, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// Max-abs of bf16 values through their magnitude bit patterns (sign cleared) compared as integers: for
// finite values the order of the patterns is the order of the magnitudes, so the largest pattern is the
// max-abs exactly, and packed 16-bit maxima compare two elements per instruction (a float max would also
// quiet NaN operands first).  bf16_mag_f32 turns such a pattern back into the fp32 value.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 bf16x2_mag(uint32_t d) { return __builtin_bit_cast(u16x2, d & 0x7FFF7FFFu); }

// Per-half maxima of the magnitudes of 2 x 4 bf16 values (element order kept: low half, high half).
__device__ __forceinline__ u16x2 absmax_halves(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_elementwise_max(__builtin_elementwise_max(bf16x2_mag(a), bf16x2_mag(b)),
                                     __builtin_elementwise_max(bf16x2_mag(c), bf16x2_mag(d)));
}
__device__ __forceinline__ u16x2 absmax_halves(const u32x4 &v) { return absmax_halves(v.x, v.y, v.z, v.w); }

// The larger of the two halves.
__device__ __forceinline__ uint32_t halves_max(u16x2 m) { return max((uint32_t)m.x, (uint32_t)m.y); }

// Magnitude pattern of the largest |x| among the 8 bf16 values of v.
__device__ __forceinline__ uint32_t absmax_bits(const u32x4 &v) { return halves_max(absmax_halves(v)); }

__device__ __forceinline__ float bf16_mag_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Scale of a group from its max-abs: fl32(amax / 448).
__device__ __forceinline__ float group_scale(float amax) { return (float)((double)amax * kInv448); }

// Reciprocal of the scale in double; 0 for an all-zero group, whose elements are then +-0 and
// encode to sign-preserving zero codes.  v_rcp_f64 and two Newton steps, e = 1 - s r, r += r e: from any
// start with 20 correct bits the result is within about 2^-52 (relative) of 1/s, inside the 2^-50 the
// quotient below needs.  A probe over every scale the quantizers can form (fl32(amax / d) for every
// positive finite bf16 amax and d = 448, 6, 65024: 97,917 values) found it equal to the correctly rounded
// double 1/s on every one.  (The IEEE double division it replaces takes twice the instructions.)
__device__ __forceinline__ double scale_reciprocal(float s) {
    if (!(s > 0.0f)) return 0.0;
    const double d = s;
    double r = __builtin_amdgcn_rcp(d);
    double e = fma(-d, r, 1.0);
    r = fma(r, e, r);
    e = fma(-d, r, 1.0);
    return fma(r, e, r);
}

// fl32(x / s) for a bf16 x, computed as fl32((double)x * RN64(1/s)).  The double product carries
// at most ~2^-52 relative error; a quotient of a bf16 (8-bit significand) by an fp32 (24-bit)
// is either exactly representable in fp32 or at least 2^-49 (relative) away from every fp32
// rounding midpoint, so the final rounding to fp32 returns the correctly rounded quotient.
// (Checked exhaustively on the CPU over every bf16 x and every bf16 amax with |x| <= amax.)
__device__ __forceinline__ float quotient(float x, double inv_s) { return (float)((double)x * inv_s); }

// Encode 4 fp32 quotients (|v| <= 448 * (1 + 2^-23)) to OCP E4M3 codes packed little-endian in a
// dword.  v_cvt_pk_fp8_f32 rounds to nearest even and, on gfx950, encodes OCP E4M3 ("FN").
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// Quantize the 4 bf16 values of two packed dwords to 4 codes (element order preserved).
__device__ __forceinline__ uint32_t quant4(uint32_t d0, uint32_t d1, double inv_s) {
    return encode4(quotient(bf16_lo(d0), inv_s), quotient(bf16_hi(d0), inv_s), quotient(bf16_lo(d1), inv_s),
                   quotient(bf16_hi(d1), inv_s));
}

// Workgroup barrier that only waits for this wave's LDS traffic (not for global loads in flight), so
// register prefetches of global data survive it.  Enough when the data shared through the barrier was
// written to LDS with ds_write: s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maxima).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
}

// s_waitcnt immediate that waits until at most N vector memory loads of this wave are in flight, leaving
// expcnt and lgkmcnt at their maxima (vmcnt is bits [3:0] and [15:14] of the immediate).
template <int N>
constexpr int vmcnt_le() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    return (N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14);
}

// Max over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1 within the row); every lane gets it.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false));
    return v;
}

// Max over the 64 lanes of a wavefront.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

// OCP E4M3 x E4M3 -> fp32 matrix multiply-accumulate, 16x16 output, K = 128 (one scale block).
// Operand lane layout: lane l supplies row (l % 16) and bytes [(l / 16) * 32, +32) of that row's
// 128 K-elements, for both operands; the result lane l, register r holds row 4 * (l / 16) + r,
// column l % 16.  Zero scale operands select the unscaled instruction (scale 1).
__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Pack two fp32 into two bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

}  // namespace fp8q
