// vc_prepare.hip -- V-Smooth preprocessing kernels for gfx950.
//
// Follows the VC-Attention pages: agihunt summary (V-Smooth bullet: tokens
// of a hardware block quantise together, only the residual after the block
// mean is quantised), MarkTechPost abstract (block mean, 128-token blocks
// after sorting), aikraft.ru "Reshenie" (lightweight k-means groups similar
// tokens; the mean is kept exactly).  Q/K per-block FP8 scales follow the
// block-scale notion of the TensorRT-LLM blog, "Quantized Attention".
//
// All kernels here are HBM-bound streaming passes: one workgroup per
// 128-token block, 16-byte coalesced loads, reductions in fp64 (exact for
// bf16 inputs of realistic dynamic range, hence independent of order), and
// every value that is promised bit-exact is produced by one IEEE fp32
// operation at a time (the file is built with -ffp-contract=off).
#include "vc_device.hpp"
#include "vc_internal.hpp"

namespace vc {

// ------------------------------------------------------------------------
// QK smoothing, K side: per-channel K mean, split over token chunks.
// partial[bh][split][D].
// ------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_colsum_partial(const uint16_t* __restrict__ k,
                                                        double* __restrict__ partial, int L,
                                                        int nsplit) {
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int RPI = 256 / CPR;    // rows per iteration
    __shared__ double red[RPI][D + 1];
    const int split = blockIdx.x, bh = blockIdx.y;
    const int t = threadIdx.x, cc = t % CPR, rs = t / CPR;
    const int chunk = (L + nsplit - 1) / nsplit;
    const int r0 = split * chunk, r1 = min(L, r0 + chunk);
    const uint16_t* base = k + (size_t)bh * L * D;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = 0.0;
    for (int r = r0 + rs; r < r1; r += RPI) {
        uint4 w = *reinterpret_cast<const uint4*>(base + (size_t)r * D + cc * 8);
        uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            acc[2 * e] += (double)bf16_to_f32(ww[e] & 0xFFFFu);
            acc[2 * e + 1] += (double)bf16_to_f32(ww[e] >> 16);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) red[rs][cc * 8 + e] = acc[e];
    __syncthreads();
    for (int c = t; c < D; c += 256) {
        double s = 0.0;
        for (int i = 0; i < RPI; i++) s += red[i][c];
        partial[((size_t)bh * nsplit + split) * D + c] = s;
    }
}

template <int D>
__global__ void k_mean_finalize(const double* __restrict__ partial, float* __restrict__ kbar, int L,
                                int nsplit, int smooth) {
    const int bh = blockIdx.x, c = threadIdx.x;
    if (c >= D) return;
    double s = 0.0;
    if (smooth)
        for (int i = 0; i < nsplit; i++) s += partial[((size_t)bh * nsplit + i) * D + c];
    kbar[(size_t)bh * D + c] = smooth ? (float)(s / (double)L) : 0.0f;
}

// Scale of a quantisation group from its amax A (same rule for every group):
// mode 0: s = fp32(A / 448), inv = fp32(448 / A); mode 1: s = 2^e with e the
// least integer such that A <= 448 * 2^e, inv = 2^-e.  A < 2^-100: both 0.
__device__ __forceinline__ void group_scale(float A, int mode, float& s, float& inv) {
    if (!(A >= 0x1p-100f)) {
        s = 0.0f;
        inv = 0.0f;
        return;
    }
    if (mode == 0) {
        s = __fdiv_rn(A, 448.0f);
        inv = __fdiv_rn(448.0f, A);
        return;
    }
    int E;
    float f = frexpf(A, &E);  // A = f * 2^E, f in [0.5, 1)
    int e = E - 9 + (f > 0.875f ? 1 : 0);  // 448 = 0.875 * 2^9
    s = ldexpf(1.0f, e);
    inv = ldexpf(1.0f, -e);
}

__device__ __forceinline__ float block_max_256(float v, float* red4) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red4[w] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
    return r;
}

// ------------------------------------------------------------------------
// Per-block scalar-scale FP8 of Q (original order, GATHER=false) or
// of K - kbar (permuted order, GATHER=true).  Grid (nb, B*H), 256 threads.
// ------------------------------------------------------------------------
template <int D, bool GATHER>
__global__ __launch_bounds__(256) void quant_qk_kernel(const uint16_t* __restrict__ x,
                                                       const int32_t* __restrict__ perm,
                                                       const float* __restrict__ kbar,
                                                       uint8_t* __restrict__ codes,
                                                       float* __restrict__ scale, int L, int nb) {
    constexpr int CPR = D / 8;
    constexpr int NCH = BLK * CPR / 256;  // chunks per thread
    __shared__ float red4[4];
    const int b = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int i0 = b * BLK;
    const size_t Lp = (size_t)nb * BLK;
    const uint16_t* xb = x + (size_t)bh * L * D;
    float vals[NCH][8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; j++) {
        const int ci = t + 256 * j, row = ci / CPR, cc = ci % CPR;
        const int slot = i0 + row;
        if (slot < L) {
            const int src = GATHER ? perm[(size_t)bh * L + slot] : slot;
            uint4 w = *reinterpret_cast<const uint4*>(xb + (size_t)src * D + cc * 8);
            uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                float lo = bf16_to_f32(ww[e] & 0xFFFFu), hi = bf16_to_f32(ww[e] >> 16);
                if (GATHER) {
                    lo = __fsub_rn(lo, kbar[(size_t)bh * D + cc * 8 + 2 * e]);
                    hi = __fsub_rn(hi, kbar[(size_t)bh * D + cc * 8 + 2 * e + 1]);
                }
                vals[j][2 * e] = lo;
                vals[j][2 * e + 1] = hi;
                amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++) vals[j][e] = 0.0f;
        }
    }
    const float A = block_max_256(amax, red4);
    float s, inv;
    group_scale(A, 0, s, inv);
    if (t == 0) scale[(size_t)bh * nb + b] = s;
    uint8_t* cb = codes + ((size_t)bh * Lp + i0) * D;
#pragma unroll
    for (int j = 0; j < NCH; j++) {
        const int ci = t + 256 * j, row = ci / CPR, cc = ci % CPR;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; e++) y[e] = __fmul_rn(vals[j][e], inv);
        const uint32_t lo = e4m3_pk4(y[0], y[1], y[2], y[3]);
        const uint32_t hi = e4m3_pk4(y[4], y[5], y[6], y[7]);
        *reinterpret_cast<uint2*>(cb + (size_t)row * D + cc * 8) = make_uint2(lo, hi);
    }
}

// ------------------------------------------------------------------------
// V-Smooth residual quantisation of one permuted 128-token block.
// Wave w holds keys 32 w .. 32 w + 31 of the block (slots in permuted order)
// and lane l holds channels CPL l .. CPL l + CPL - 1 (CPL = D / 64), so each
// key's row is one coalesced load across the wave and the values stay in
// registers: per-channel fp64 sums (exact for bf16 inputs, so the order does
// not matter) and maxima are combined over the four waves through LDS.  The
// codes are channel-major in the slot order of the attention kernel's P V
// operand, where the 32 keys of wave w fill slots 32 b + 8 w .. 32 b + 8 w +
// 7 of every channel row (b = 0..3); they are assembled in an LDS tile and
// the block's D x 128 bytes, contiguous in HBM, leave as 16-byte stores.
template <int D>
__global__ __launch_bounds__(256) void quant_v_kernel(const uint16_t* __restrict__ v,
                                                      const int32_t* __restrict__ perm,
                                                      uint8_t* __restrict__ codes,
                                                      float* __restrict__ vscale,
                                                      float* __restrict__ vmean, int L, int nb,
                                                      int mode) {
    constexpr int CPL = D / 64;  // channels per lane
    constexpr int KW = BLK / 4;  // keys per wave
    constexpr int PITCH = BLK + 16;  // LDS row of one channel's codes, padded against bank conflicts
    __shared__ double psum[4][D];
    __shared__ float pmax[4][D];
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * PITCH];
    const int b = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
    const int i0 = b * BLK;
    const int n = min(BLK, L - i0);
    const uint16_t* vb = v + (size_t)bh * L * D + CPL * lane;
    const int32_t* pb = perm + (size_t)bh * L + i0 + KW * w;
    const int nw = min(KW, max(0, n - KW * w));  // valid keys of this wave
    float x[KW][CPL];
#pragma unroll
    for (int i = 0; i < KW; i++) {
        if (i < nw) {
            const int src = pb[i];  // uniform across the wave
            if (CPL == 2) {
                const uint32_t u = *reinterpret_cast<const uint32_t*>(vb + (size_t)src * D);
                x[i][0] = bf16_to_f32(u & 0xFFFFu);
                x[i][CPL - 1] = bf16_to_f32(u >> 16);
            } else {
                x[i][0] = bf16_to_f32(vb[(size_t)src * D]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < CPL; e++) x[i][e] = 0.0f;
        }
    }
#pragma unroll
    for (int e = 0; e < CPL; e++) {
        double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int i = 0; i < KW; i++) s4[i % 4] += (double)x[i][e];  // padded keys add 0
        psum[w][CPL * lane + e] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    __syncthreads();
    float mu[CPL], inv[CPL];
#pragma unroll
    for (int e = 0; e < CPL; e++) {
        const int c = CPL * lane + e;
        mu[e] = (float)((((psum[0][c] + psum[1][c]) + psum[2][c]) + psum[3][c]) / (double)n);
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < KW; i++)
            if (i < nw) am = fmaxf(am, fabsf(__fsub_rn(x[i][e], mu[e])));
        pmax[w][c] = am;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < CPL; e++) {
        const int c = CPL * lane + e;
        const float A = fmaxf(fmaxf(pmax[0][c], pmax[1][c]), fmaxf(pmax[2][c], pmax[3][c]));
        float s;
        group_scale(A, mode, s, inv[e]);
        const size_t gi = ((size_t)bh * nb + b) * D + c;
        if (w == 0) {
            vmean[gi] = mu[e];
            vscale[gi] = s;
        }
        uint8_t* out = tile + c * PITCH + 8 * w;
#pragma unroll
        for (int bb = 0; bb < 4; bb++) {
            // slots 32 bb + 8 w + j hold keys 32 w + 16 (j / 4) + 4 bb + j % 4
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int i = 16 * (j / 4) + 4 * bb + j % 4;
                y[j] = i < nw ? __fmul_rn(__fsub_rn(x[i][e], mu[e]), inv[e]) : 0.0f;  // padded slots: code 0
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

// ------------------------------------------------------------------------
// 4-bit V-Smooth residual: the same exact block mean, then E2M1 codes with
// one power-of-two (E8M0) scale per (channel, key group), the group of key kk
// being (kk mod 16) div 4 -- slots 32 g .. 32 g + 31 of the P V slot order,
// the 32-element k-blocks of the scaled matrix-core product.  Scale 2^e with
// e the least integer such that amax <= 6 * 2^e (no element clips); amax <
// 2^-100: codes 0.  Codes: v_cvt_scalef32_pk_fp4_f32 (round to nearest even
// of x / 2^e, exact scaling).  Output: codes [bh][nb][D][64] bytes, slot 2 t
// in the low nibble of byte t; scales [bh][nb][D][4] bytes e + 127.  The
// loads, the mean and the wave/key layout are those of quant_v_kernel; each
// wave holds 8 keys of every group (keys 4 g .. 4 g + 3 and 16 + 4 g ..
// 16 + 4 g + 3 of its 32), so group maxima are combined over the waves in LDS.
// ------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void quant_v4_kernel(const uint16_t* __restrict__ v,
                                                       const int32_t* __restrict__ perm,
                                                       uint8_t* __restrict__ codes,
                                                       uint32_t* __restrict__ vexp,
                                                       float* __restrict__ vmean, int L, int nb) {
    constexpr int CPL = D / 64;
    constexpr int KW = BLK / 4;
    constexpr int RB = BLK / 2;      // code bytes per channel row
    constexpr int PITCH = RB + 16;   // LDS row, padded against bank conflicts
    __shared__ double psum[4][D];
    __shared__ float pmax[4][D][4];
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * PITCH];
    const int b = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
    const int i0 = b * BLK;
    const int n = min(BLK, L - i0);
    const uint16_t* vb = v + (size_t)bh * L * D + CPL * lane;
    const int32_t* pb = perm + (size_t)bh * L + i0 + KW * w;
    const int nw = min(KW, max(0, n - KW * w));
    float x[KW][CPL];
#pragma unroll
    for (int i = 0; i < KW; i++) {
        if (i < nw) {
            const int src = pb[i];
            if (CPL == 2) {
                const uint32_t u = *reinterpret_cast<const uint32_t*>(vb + (size_t)src * D);
                x[i][0] = bf16_to_f32(u & 0xFFFFu);
                x[i][CPL - 1] = bf16_to_f32(u >> 16);
            } else {
                x[i][0] = bf16_to_f32(vb[(size_t)src * D]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < CPL; e++) x[i][e] = 0.0f;
        }
    }
#pragma unroll
    for (int e = 0; e < CPL; e++) {
        double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int i = 0; i < KW; i++) s4[i % 4] += (double)x[i][e];
        psum[w][CPL * lane + e] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    }
    __syncthreads();
    float mu[CPL];
#pragma unroll
    for (int e = 0; e < CPL; e++) {
        const int c = CPL * lane + e;
        mu[e] = (float)((((psum[0][c] + psum[1][c]) + psum[2][c]) + psum[3][c]) / (double)n);
#pragma unroll
        for (int i = 0; i < KW; i++) x[i][e] = i < nw ? __fsub_rn(x[i][e], mu[e]) : 0.0f;  // residual
#pragma unroll
        for (int g = 0; g < 4; g++) {
            float am = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++) am = fmaxf(am, fabsf(x[16 * (j / 4) + 4 * g + j % 4][e]));
            pmax[w][c][g] = am;
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < CPL; e++) {
        const int c = CPL * lane + e;
        const size_t gi = ((size_t)bh * nb + b) * D + c;
        uint32_t ebytes = 0;
        uint8_t* out = tile + c * PITCH;
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const float A = fmaxf(fmaxf(pmax[0][c][g], pmax[1][c][g]), fmaxf(pmax[2][c][g], pmax[3][c][g]));
            const int ex = e8m0_exp(A);
            ebytes |= (uint32_t)(ex + 127) << (8 * g);
            // slots 32 g + 8 w + j hold keys 32 w + 16 (j / 4) + 4 g + j % 4
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; j++) y[j] = x[16 * (j / 4) + 4 * g + j % 4][e];
            const uint32_t pk = ex > -127 ? e2m1_pk8(y, ldexpf(1.0f, ex)) : 0u;  // zero group: codes 0
            *reinterpret_cast<uint32_t*>(out + 16 * g + 4 * w) = pk;
        }
        if (w == 0) {
            vmean[gi] = mu[e];
            vexp[gi] = ebytes;
        }
    }
    // the block's D x 64 code bytes are contiguous in HBM: 16 bytes per lane
    __syncthreads();
    uint8_t* dst = codes + ((size_t)bh * nb + b) * D * RB;
#pragma unroll
    for (int i = 0; i < D * RB / (16 * 256); i++) {
        const int q = t + 256 * i, row = q / (RB / 16), ch = q % (RB / 16);
        *reinterpret_cast<uint4*>(dst + 16 * q) = *reinterpret_cast<const uint4*>(tile + row * PITCH + 16 * ch);
    }
}

// src may equal dst (a permutation kept from an earlier call): each element
// is read and written by the same thread.
__global__ void copy_perm_kernel(const int32_t* src, int32_t* dst, size_t n,
                                 double* __restrict__ obj, size_t nobj) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src[i];
    if (obj != nullptr && i < nobj) obj[i] = __longlong_as_double(0x7FF8000000000000LL);
}

hipError_t launch_copy_perm(const int32_t* src, int32_t* dst, size_t n, double* obj, size_t nobj,
                            hipStream_t st) {
    const size_t m = n > nobj ? n : nobj;
    hipLaunchKernelGGL(copy_perm_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, src, dst, n,
                       obj, nobj);
    return hipGetLastError();
}

// ------------------------------------------------------------------------
// Launchers.
// ------------------------------------------------------------------------
int k_mean_splits(int BH, int L) {
    int by_len = (L + 1023) / 1024;
    int want = (2048 + BH - 1) / BH;
    int s = by_len < want ? by_len : want;
    return s < 1 ? 1 : s;
}

template <int D>
static void launch_k_mean_t(const void* k, double* kpartial, float* kbar, int BH, int L, int smooth,
                            hipStream_t st) {
    const int nsplit = k_mean_splits(BH, L);
    if (smooth) {
        hipLaunchKernelGGL((k_colsum_partial<D>), dim3(nsplit, BH), dim3(256), 0, st,
                           (const uint16_t*)k, kpartial, L, nsplit);
    }
    hipLaunchKernelGGL((k_mean_finalize<D>), dim3(BH), dim3(D), 0, st, kpartial, kbar, L, nsplit, smooth);
}

hipError_t launch_k_mean(const void* k, double* kpartial, float* kbar, int BH, int L, int d, int smooth,
                         hipStream_t st) {
    if (d == 128)
        launch_k_mean_t<128>(k, kpartial, kbar, BH, L, smooth, st);
    else
        launch_k_mean_t<64>(k, kpartial, kbar, BH, L, smooth, st);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_prepare_quant_t(const PrepareArgs& a, hipStream_t st) {
    const int BH = a.B * a.H;
    launch_k_mean_t<D>(a.k, a.kpartial, a.kbar, BH, a.L, a.smooth_k, st);
    hipLaunchKernelGGL((quant_qk_kernel<D, false>), dim3(a.nb, BH), dim3(256), 0, st,
                       (const uint16_t*)a.q, (const int32_t*)nullptr, (const float*)nullptr,
                       a.q8, a.q_scale, a.L, a.nb);
    hipLaunchKernelGGL((quant_qk_kernel<D, true>), dim3(a.nb, BH), dim3(256), 0, st,
                       (const uint16_t*)a.k, a.perm, (const float*)a.kbar, a.k8, a.k_scale, a.L,
                       a.nb);
    if (a.v_format == 1)
        hipLaunchKernelGGL((quant_v4_kernel<D>), dim3(a.nb, BH), dim3(256), 0, st, (const uint16_t*)a.v, a.perm,
                           a.v8, reinterpret_cast<uint32_t*>(a.v_scale), a.v_mean, a.L, a.nb);
    else
        hipLaunchKernelGGL((quant_v_kernel<D>), dim3(a.nb, BH), dim3(256), 0, st,
                           (const uint16_t*)a.v, a.perm, a.v8, a.v_scale, a.v_mean, a.L, a.nb,
                           a.v_mode);
    return hipGetLastError();
}

hipError_t launch_prepare_quant(const PrepareArgs& a, hipStream_t st) {
    return a.d == 128 ? launch_prepare_quant_t<128>(a, st) : launch_prepare_quant_t<64>(a, st);
}

}  // namespace vc
