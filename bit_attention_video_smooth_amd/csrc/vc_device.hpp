// vc_device.hpp -- device helpers shared by the VC-Attention HIP kernels
// (gfx950 / CDNA4).  Number formats and small wave-level primitives only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vc {

constexpr int BLK = 128;  // tokens per hardware block (V-Smooth group and KV tile)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

#define VC_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    v2bf v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// OCP E4M3FN (sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7E = 448
// is the largest finite code), saturating round-to-nearest-even, on the
// hardware conversion: v_cvt_pk_fp8_f32 rounds to nearest even into E4M3FN
// (checked against the format's definition on every fp32 exponent and
// leading-mantissa pattern up to 450 in magnitude, both signs, ties
// included); the inputs are first clamped to +-448, which is where
// round-to-nearest already lands every finite value below 464, so the result
// saturates instead of overflowing.  Two values go into
// bytes 0, 1 (HI = false) or 2, 3 (HI = true) of `old`.  Finite inputs only.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pk2(float a, float b, uint32_t old) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// four values -> one dword of E4M3 codes, byte i = code of x_i
__device__ __forceinline__ uint32_t e4m3_pk4(float x0, float x1, float x2, float x3) {
    return e4m3_pk2<true>(x2, x3, e4m3_pk2<false>(x0, x1, 0u));
}

// Eight values -> one dword of E2M1 (OCP MX FP4) codes, element j in nibble j
// (low nibble first): v_cvt_scalef32_pk_fp4_f32 rounds x / sc to the nearest
// E2M1 value, ties to even, saturating at +-6 (measured on gfx950); with sc a
// power of two the division is exact.
__device__ __forceinline__ uint32_t e2m1_pk8(const float (&y)[8], float sc) {
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[2], y[3], sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[4], y[5], sc, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[6], y[7], sc, 3);
}

// E8M0 exponent of an FP4 group with amax A: the least e with A <= 6 * 2^e
// (6 = 0.75 * 2^3, A = f * 2^E with f in [0.5, 1)); -127 for A < 2^-100.
__device__ __forceinline__ int e8m0_exp(float A) {
    int E;
    const float f = frexpf(A, &E);
    return A >= 0x1p-100f ? E - 3 + (f > 0.75f ? 1 : 0) : -127;
}

// ExpCast-FP8: y = fma(S, c8, krow), then v_cvt_pk_u8_f32, which rounds to
// the nearest integer (ties to even) and saturates to [0, 255], into byte
// `sel` of `acc`.  Callers keep y below 126.5.
__device__ __forceinline__ uint32_t expcast_byte_into(float S, float c8, float krow, int sel,
                                                      uint32_t acc) {
    const float y = __builtin_fmaf(S, c8, krow);
    return __builtin_amdgcn_cvt_pk_u8_f32(y, sel, acc);
}

// max over lanes {l, l^16, l^32, l^48} (one query's four lane groups)
__device__ __forceinline__ float max_over_groups(float v) {
    auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
    auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// XCD-aware remap of a 1-D workgroup id: the hardware deals workgroups to
// the 8 XCDs round-robin; give each XCD a contiguous range of logical ids so
// that neighbouring tiles of one head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int n) {
    constexpr int NX = 8;
    int per = (n + NX - 1) / NX;
    int tall = n % NX;
    if (tall == 0) tall = NX;
    int x = pid % NX, loc = pid / NX;
    return (x < tall) ? x * per + loc : tall * per + (x - tall) * (per - 1) + loc;
}

// Slot order of keys inside a 128-key block as the PV matrix-core step reads
// them (see the V layout in vc_attention.h): slot pos holds key kk with
// pos = 32*((kk%16)/4) + 4*(kk/16) + (kk%4).
__host__ __device__ constexpr int vslot_of_key(int kk) {
    return 32 * ((kk % 16) / 4) + 4 * (kk / 16) + (kk % 4);
}
__host__ __device__ constexpr int vkey_of_slot(int pos) {
    return 16 * ((pos % 32) / 4) + 4 * (pos / 32) + (pos % 4);
}

}  // namespace vc
