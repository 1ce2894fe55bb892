// vc_sage_prepare.hip -- quantisation for the SAGE-style baseline attention
// (TensorRT-LLM blog, "Quantized Attention"): QK^T codes in INT8 or FP8
// with one Q scale per query token (q block size 1) and one K scale per 16
// consecutive keys (k block size 16), PV codes in FP8 E4M3 with one V scale
// per channel taken over all tokens of a head (v block size 1).  Tokens stay
// in sequence order; K is optionally smoothed by its per-channel mean first.
//
// A scale is amax / qmax (qmax 127 for INT8, 448 for E4M3) by IEEE
// division, with 0 for amax below 2^-100; INT8 codes round fp32(x * inv) to
// the nearest integer, ties to even, clamped to +-127.  Every kernel is an
// HBM-bound streaming pass with 16-byte coalesced loads, and every value
// promised bit-exact comes from one IEEE fp32 operation at a time (the file
// is built with -ffp-contract=off).
#include "vc_device.hpp"
#include "vc_internal.hpp"

namespace vc {

namespace {

__device__ __forceinline__ void sage_scale(float A, float qmax, float& s, float& inv) {
    if (!(A >= 0x1p-100f)) {
        s = 0.0f;
        inv = 0.0f;
        return;
    }
    s = __fdiv_rn(A, qmax);
    inv = __fdiv_rn(qmax, A);
}

// INT8 code byte of y = fp32(x * inv): v_rndne_f32, then clamp
__device__ __forceinline__ uint32_t i8_byte(float y) {
    const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(y), -127.0f, 127.0f);
    return (uint32_t)(int)r & 0xFFu;
}

template <bool I8>
__device__ __forceinline__ uint2 codes8(const float (&x)[8], float inv) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; e++) y[e] = __fmul_rn(x[e], inv);
    if (I8) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            lo |= i8_byte(y[e]) << (8 * e);
            hi |= i8_byte(y[4 + e]) << (8 * e);
        }
        return make_uint2(lo, hi);
    }
    return make_uint2(e4m3_pk4(y[0], y[1], y[2], y[3]), e4m3_pk4(y[4], y[5], y[6], y[7]));
}

__device__ __forceinline__ void unpack8(uint4 w, float (&x)[8]) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
        x[2 * e] = bf16_to_f32(ww[e] & 0xFFFFu);
        x[2 * e + 1] = bf16_to_f32(ww[e] >> 16);
    }
}

// Q: one scale per token.  LPR = D / 8 consecutive lanes hold one row (8
// channels each); a workgroup covers 256 / LPR rows.  Grid (Lp / rows, BH).
template <int D, bool I8>
__global__ __launch_bounds__(256) void sage_quant_q_kernel(const uint16_t* __restrict__ q,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ scale, int L, int Lp) {
    constexpr int LPR = D / 8;
    constexpr int RPB = 256 / LPR;
    const int bh = blockIdx.y, t = threadIdx.x;
    const int row = blockIdx.x * RPB + t / LPR, cc = t % LPR;
    float x[8];
    if (row < L) {
        unpack8(*reinterpret_cast<const uint4*>(q + ((size_t)bh * L + row) * D + cc * 8), x);
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++) x[e] = 0.0f;
    }
    float A = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++) A = fmaxf(A, fabsf(x[e]));
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) A = fmaxf(A, __shfl_xor(A, o));  // within the row's lanes
    float s, inv;
    sage_scale(A, I8 ? 127.0f : 448.0f, s, inv);
    if (cc == 0) scale[(size_t)bh * Lp + row] = s;
    *reinterpret_cast<uint2*>(codes + ((size_t)bh * Lp + row) * D + cc * 8) = codes8<I8>(x, inv);
}

// K - kbar: one scale per 16 consecutive tokens, one wave per group; lane l
// holds row l / 4 and channels (l % 4) D/4 ... + D/4.  Grid (Lp / 64, BH).
template <int D, bool I8>
__global__ __launch_bounds__(256) void sage_quant_k_kernel(const uint16_t* __restrict__ k,
                                                           const float* __restrict__ kbar,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ scale, int L, int Lp) {
    constexpr int NC = D / 32;  // 8-channel chunks per lane
    const int bh = blockIdx.y, t = threadIdx.x;
    const int w = t >> 6, lane = t & 63;
    const int grp = blockIdx.x * 4 + w;
    const int row = grp * 16 + lane / 4;
    const int c0 = (lane % 4) * (D / 4);
    // every load is issued before any value is used: a padded row loads the
    // head's last row and is zeroed afterwards (code 0, no part in the amax)
    const bool ok = row < L;
    const size_t src = (size_t)bh * L + min(row, L - 1);
    uint4 raw[NC];
    float kb[NC][8];
#pragma unroll
    for (int j = 0; j < NC; j++) {
        raw[j] = *reinterpret_cast<const uint4*>(k + src * D + c0 + 8 * j);
        const float4 k0 = *reinterpret_cast<const float4*>(kbar + (size_t)bh * D + c0 + 8 * j);
        const float4 k1 = *reinterpret_cast<const float4*>(kbar + (size_t)bh * D + c0 + 8 * j + 4);
        kb[j][0] = k0.x; kb[j][1] = k0.y; kb[j][2] = k0.z; kb[j][3] = k0.w;
        kb[j][4] = k1.x; kb[j][5] = k1.y; kb[j][6] = k1.z; kb[j][7] = k1.w;
    }
    float x[NC][8];
    float A = 0.0f;
#pragma unroll
    for (int j = 0; j < NC; j++) {
        unpack8(raw[j], x[j]);
#pragma unroll
        for (int e = 0; e < 8; e++) x[j][e] = ok ? __fsub_rn(x[j][e], kb[j][e]) : 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e++) A = fmaxf(A, fabsf(x[j][e]));
    }
    A = wave_max(A);
    float s, inv;
    sage_scale(A, I8 ? 127.0f : 448.0f, s, inv);
    if (lane == 0) scale[(size_t)bh * (Lp / 16) + grp] = s;
#pragma unroll
    for (int j = 0; j < NC; j++)
        *reinterpret_cast<uint2*>(codes + ((size_t)bh * Lp + row) * D + c0 + 8 * j) = codes8<I8>(x[j], inv);
}

// V: per-channel amax of |v| over chunks of SAGE_VCHUNK tokens.  Grid
// (nvchunk, BH); part[bh][chunk][c].
template <int D>
__global__ __launch_bounds__(256) void v_absmax_partial(const uint16_t* __restrict__ v,
                                                        float* __restrict__ part, int L, int nvchunk) {
    constexpr int CPR = D / 8;
    constexpr int RPI = 256 / CPR;
    __shared__ float red[RPI][D + 1];
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int t = threadIdx.x, cc = t % CPR, rs = t / CPR;
    const int r0 = chunk * SAGE_VCHUNK, r1 = min(L, r0 + SAGE_VCHUNK);
    float m[8];
#pragma unroll
    for (int e = 0; e < 8; e++) m[e] = 0.0f;
    // four rows per thread in flight, all loaded before use: rows past the
    // chunk load its last row again (a max does not change)
    for (int r = r0 + rs; r < r1; r += 4 * RPI) {
        uint4 w4[4];
#pragma unroll
        for (int u = 0; u < 4; u++)
            w4[u] = *reinterpret_cast<const uint4*>(v + ((size_t)bh * L + min(r + u * RPI, r1 - 1)) * D + cc * 8);
#pragma unroll
        for (int u = 0; u < 4; u++) {
            float x[8];
            unpack8(w4[u], x);
#pragma unroll
            for (int e = 0; e < 8; e++) m[e] = fmaxf(m[e], fabsf(x[e]));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) red[rs][cc * 8 + e] = m[e];
    __syncthreads();
    for (int c = t; c < D; c += 256) {
        float a = 0.0f;
        for (int i = 0; i < RPI; i++) a = fmaxf(a, red[i][c]);
        part[((size_t)bh * nvchunk + chunk) * D + c] = a;
    }
}

template <int D>
__global__ void v_scale_finalize(const float* __restrict__ part, float* __restrict__ vscale,
                                 float* __restrict__ vinv, int nvchunk) {
    const int bh = blockIdx.x, c = threadIdx.x;
    if (c >= D) return;
    // eight chunk maxima per step, loaded before use
    constexpr int U = 8;
    const float* p = part + (size_t)bh * nvchunk * D + c;
    float A = 0.0f;
    int i = 0;
    for (; i + U <= nvchunk; i += U) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; u++) x[u] = p[(size_t)(i + u) * D];
#pragma unroll
        for (int u = 0; u < U; u++) A = fmaxf(A, x[u]);
    }
    for (; i < nvchunk; i++) A = fmaxf(A, p[(size_t)i * D]);
    float s, inv;
    sage_scale(A, 448.0f, s, inv);
    vscale[(size_t)bh * D + c] = s;
    vinv[(size_t)bh * D + c] = inv;
}

// V codes of one 128-token block (sequence order), channel-major in the P V
// slot order: wave w holds keys 32 w .. 32 w + 31 and lane l channels
// CPL l .. CPL l + CPL - 1 (CPL = D / 64); the keys of wave w fill slots
// 32 bb + 8 w .. 32 bb + 8 w + 7 of every channel row (bb = 0..3), slot
// 32 bb + 8 w + j holding key 32 w + 16 (j / 4) + 4 bb + j % 4.
template <int D>
__global__ __launch_bounds__(256) void sage_quant_v_kernel(const uint16_t* __restrict__ v,
                                                           const float* __restrict__ vinv,
                                                           uint8_t* __restrict__ codes, int L, int nb) {
    constexpr int CPL = D / 64;
    constexpr int KW = BLK / 4;
    constexpr int PITCH = BLK + 16;  // LDS row of one channel's codes, padded against bank conflicts
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * PITCH];
    const int b = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
    const int i0 = b * BLK + KW * w;
    const int nw = min(KW, max(0, L - i0));  // valid keys of this wave
    const uint16_t* vb = v + (size_t)bh * L * D + CPL * lane;
    // every row load is issued before any is used: rows past the head load
    // the last row and are zeroed afterwards
    uint32_t raw[KW];
#pragma unroll
    for (int i = 0; i < KW; i++) {
        const size_t row = (size_t)min(i0 + i, L - 1);
        if (CPL == 2)
            raw[i] = *reinterpret_cast<const uint32_t*>(vb + row * D);
        else
            raw[i] = vb[row * D];
    }
    float x[KW][CPL];
#pragma unroll
    for (int i = 0; i < KW; i++) {
        const uint32_t u = i < nw ? raw[i] : 0u;
        x[i][0] = bf16_to_f32(u & 0xFFFFu);
        if (CPL == 2) x[i][CPL - 1] = bf16_to_f32(u >> 16);
    }
#pragma unroll
    for (int e = 0; e < CPL; e++) {
        const int c = CPL * lane + e;
        const float inv = vinv[(size_t)bh * D + c];
        uint8_t* out = tile + c * PITCH + 8 * w;
#pragma unroll
        for (int bb = 0; bb < 4; bb++) {
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int i = 16 * (j / 4) + 4 * bb + j % 4;
                y[j] = i < nw ? __fmul_rn(x[i][e], inv) : 0.0f;  // padded slots: code 0
            }
            *reinterpret_cast<uint2*>(out + 32 * bb) =
                make_uint2(e4m3_pk4(y[0], y[1], y[2], y[3]), e4m3_pk4(y[4], y[5], y[6], y[7]));
        }
    }
    // the block's D x 128 codes are contiguous in HBM: 16 bytes per lane
    __syncthreads();
    uint8_t* dst = codes + ((size_t)bh * nb + b) * D * BLK;
#pragma unroll
    for (int i = 0; i < D * BLK / (16 * 256); i++) {
        const int q = t + 256 * i, row = q / (BLK / 16), ch = q % (BLK / 16);
        *reinterpret_cast<uint4*>(dst + 16 * q) = *reinterpret_cast<const uint4*>(tile + row * PITCH + 16 * ch);
    }
}

template <int D, bool I8>
hipError_t launch_sage_t(const SageArgs& a, hipStream_t st) {
    const int BH = a.B * a.H;
    const int Lp = a.nb * BLK;
    hipError_t e = launch_k_mean(a.k, a.kpartial, a.kbar, BH, a.L, D, a.smooth_k, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sage_quant_q_kernel<D, I8>), dim3(Lp / (256 / (D / 8)), BH), dim3(256), 0, st,
                       (const uint16_t*)a.q, a.q8, a.q_scale, a.L, Lp);
    hipLaunchKernelGGL((sage_quant_k_kernel<D, I8>), dim3(Lp / 64, BH), dim3(256), 0, st,
                       (const uint16_t*)a.k, (const float*)a.kbar, a.k8, a.k_scale, a.L, Lp);
    hipLaunchKernelGGL((v_absmax_partial<D>), dim3(a.nvchunk, BH), dim3(256), 0, st, (const uint16_t*)a.v,
                       a.vpart, a.L, a.nvchunk);
    hipLaunchKernelGGL((v_scale_finalize<D>), dim3(BH), dim3(D), 0, st, (const float*)a.vpart, a.v_scale,
                       a.vinv, a.nvchunk);
    hipLaunchKernelGGL((sage_quant_v_kernel<D>), dim3(a.nb, BH), dim3(256), 0, st, (const uint16_t*)a.v,
                       (const float*)a.vinv, a.v8, a.L, a.nb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sage_prepare(const SageArgs& a, hipStream_t st) {
    if (a.d == 128) return a.qk_int8 ? launch_sage_t<128, true>(a, st) : launch_sage_t<128, false>(a, st);
    return a.qk_int8 ? launch_sage_t<64, true>(a, st) : launch_sage_t<64, false>(a, st);
}

}  // namespace vc
