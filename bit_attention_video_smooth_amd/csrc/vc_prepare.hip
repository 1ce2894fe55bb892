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
    constexpr int RPI = 256 / CPR;    // rows per load instruction of the workgroup
    constexpr int CH = 4 * RPI;       // rows per chunk: four loads per thread
    __shared__ double red[RPI][D + 1];
    const int split = blockIdx.x, bh = blockIdx.y;
    const int t = threadIdx.x, cc = t % CPR, rs = t / CPR;
    const uint16_t* base = k + (size_t)bh * L * D;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = 0.0;
    // the head's chunks of CH rows are dealt round-robin to its splits, so
    // at any time the splits of a head read one contiguous window of it (as
    // a copy would) rather than nsplit distant streams; the four loads of a
    // chunk are issued before their sums (fp64 sums of bf16 values are exact,
    // so the order of the additions does not matter)
    const int nch = (L + CH - 1) / CH;
    for (int c = split; c < nch; c += nsplit) {
        const int r = c * CH + rs;
        uint4 w4[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            w4[u] = make_uint4(0, 0, 0, 0);  // rows past the head add 0
            if (r + u * RPI < L) w4[u] = *reinterpret_cast<const uint4*>(base + (size_t)(r + u * RPI) * D + cc * 8);
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const uint32_t ww[4] = {w4[u].x, w4[u].y, w4[u].z, w4[u].w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                acc[2 * e] += (double)bf16_to_f32(ww[e] & 0xFFFFu);
                acc[2 * e + 1] += (double)bf16_to_f32(ww[e] >> 16);
            }
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
    // eight partials per step, loaded before they are added (the same order
    // of additions; fp64 sums of bf16 data are exact in any order anyway)
    constexpr int U = 8;
    double s = 0.0;
    if (smooth) {
        const double* p = partial + (size_t)bh * nsplit * D + c;
        int i = 0;
        for (; i + U <= nsplit; i += U) {
            double x[U];
#pragma unroll
            for (int u = 0; u < U; u++) x[u] = p[(size_t)(i + u) * D];
#pragma unroll
            for (int u = 0; u < U; u++) s += x[u];
        }
        for (; i < nsplit; i++) s += p[(size_t)i * D];
    }
    kbar[(size_t)bh * D + c] = smooth ? (float)(s / (double)L) : 0.0f;
}

// A permutation entry as a row index: entries outside 0 .. L-1 (a caller's
// perm_in that is not a permutation) are clamped, so a gather never reads
// outside its head; the codes are then unspecified.
__device__ __forceinline__ int clamp_row(int r, int L) { return min(max(r, 0), L - 1); }

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
    // Gather: the wave's rows are G w + r + G NCH j' ... (G = 64 / CPR rows per
    // load instruction, r = lane / CPR): 32 permutation entries, one load by
    // the lower half of the wave, handed to the chunks by lane exchanges
    constexpr int G = 64 / CPR;
    static_assert(G * NCH == 32, "32 rows per wave");
    const int w = t >> 6, lane = t & 63;
    int pv = 0;
    if (GATHER) {
        const int prow = G * w + lane % G + 256 / CPR * (lane / G);
        if (lane < 32 && i0 + prow < L) pv = clamp_row(perm[(size_t)bh * L + i0 + prow], L);
    }
    // every row load is issued before any value is used: rows past the head
    // (slot >= L) load a valid row (the last one, or row 0 through a zero
    // permutation entry) and are zeroed afterwards, so no load sits behind a
    // branch that the compiler would close with a wait
    const int cc = t % CPR;  // the same chunk column for every j (256 % CPR == 0)
    float kb8[8];
    if (GATHER) {
        const float4 k0 = *reinterpret_cast<const float4*>(kbar + (size_t)bh * D + cc * 8);
        const float4 k1 = *reinterpret_cast<const float4*>(kbar + (size_t)bh * D + cc * 8 + 4);
        kb8[0] = k0.x; kb8[1] = k0.y; kb8[2] = k0.z; kb8[3] = k0.w;
        kb8[4] = k1.x; kb8[5] = k1.y; kb8[6] = k1.z; kb8[7] = k1.w;
    }
    uint4 raw[NCH];
#pragma unroll
    for (int j = 0; j < NCH; j++) {
        const int row = (t + 256 * j) / CPR;
        const int slot = i0 + row;
        const int psrc = GATHER ? __shfl(pv, lane / CPR + G * j) : 0;  // every lane takes part
        const int src = GATHER ? psrc : min(slot, L - 1);
        raw[j] = *reinterpret_cast<const uint4*>(xb + (size_t)src * D + cc * 8);
    }
    float vals[NCH][8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; j++) {
        const bool ok = i0 + (t + 256 * j) / CPR < L;
        const uint32_t ww[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            float lo = bf16_to_f32(ww[e] & 0xFFFFu), hi = bf16_to_f32(ww[e] >> 16);
            if (GATHER) {
                lo = __fsub_rn(lo, kb8[2 * e]);
                hi = __fsub_rn(hi, kb8[2 * e + 1]);
            }
            vals[j][2 * e] = ok ? lo : 0.0f;
            vals[j][2 * e + 1] = ok ? hi : 0.0f;
            amax = fmaxf(amax, fmaxf(fabsf(vals[j][2 * e]), fabsf(vals[j][2 * e + 1])));
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
// Wave w holds keys 32 w .. 32 w + 31 of the block (slots in permuted order).
// A key row is R = D / 8 sixteen-byte chunks; lane l takes chunk l % R
// (channels 8 (l % R) .. + 7) of its keys, so one load instruction moves
// 64 / R whole rows.  The wave's 32 keys are 8 quads of consecutive keys;
// lane l holds the quads g = l / R + (64 / R) u, i.e. its keys lie in
// consecutive slots of the attention kernel's P V operand order, where the
// keys 4 g .. 4 g + 3 of wave w fill slots 32 (g % 4) + 8 w + 4 (g / 4) + i
// of every channel row.  Per-channel fp64 sums (exact for bf16 inputs, so
// the order does not matter) and maxima are combined over the lanes of one
// chunk with cross-lane exchanges and over the four waves through LDS; one
// thread per channel then forms the mean and the scale, which the lanes read
// back.  All row loads are issued before any is used.  The codes are
// assembled channel-major in an LDS tile, and the block's D x 128 bytes,
// contiguous in HBM, leave as 16-byte stores.
template <int D>
__global__ __launch_bounds__(256) void quant_v_kernel(const uint16_t* __restrict__ v,
                                                      const int32_t* __restrict__ perm,
                                                      uint8_t* __restrict__ codes,
                                                      float* __restrict__ vscale,
                                                      float* __restrict__ vmean, int L, int nb,
                                                      int mode) {
    constexpr int R = D / 8;          // 16-byte chunks per key row
    constexpr int G = 64 / R;         // key rows per load instruction
    constexpr int NL = 32 / G;        // keys per lane
    constexpr int PITCH = BLK + 16;   // LDS row of one channel's codes, padded against bank conflicts
    static_assert(NL % 4 == 0, "whole key quads per lane");
    __shared__ double psum[4][D];
    __shared__ float pmax[4][D];
    __shared__ __attribute__((aligned(16))) float cmu[D];
    __shared__ __attribute__((aligned(16))) float cinv[D];
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * PITCH];
    const int b = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
    const int cc = lane % R, r = lane / R;
    const int i0 = b * BLK;
    const int n = min(BLK, L - i0);
    const int kw0 = 32 * w;  // the wave's first key within the block
    // the wave's 32 permutation entries, one per lane of its lower half
    int pv = 0;
    if (lane < 32 && kw0 + lane < n) pv = clamp_row(perm[(size_t)bh * L + i0 + kw0 + lane], L);
    const uint16_t* vb = v + (size_t)bh * L * D + 8 * cc;
    // the raw bf16 rows (half the registers of their fp32 values; the
    // conversion is a shift or a mask, repeated where a value is used)
    uint32_t xr[NL][4];
#pragma unroll
    for (int j = 0; j < NL; j++) {
        const int kl = 4 * (r + G * (j / 4)) + j % 4;  // key within the wave
        const int src = __shfl(pv, kl);
        // padded keys: entry 0, a valid row, zeroed once all loads are out
        const uint4 u = *reinterpret_cast<const uint4*>(vb + (size_t)src * D);
        xr[j][0] = u.x; xr[j][1] = u.y; xr[j][2] = u.z; xr[j][3] = u.w;
    }
#pragma unroll
    for (int j = 0; j < NL; j++) {
        const bool ok = kw0 + 4 * (r + G * (j / 4)) + j % 4 < n;
#pragma unroll
        for (int i = 0; i < 4; i++) xr[j][i] = ok ? xr[j][i] : 0u;
    }
    auto X = [&](int j, int e) -> float {
        const uint32_t wv = xr[j][e / 2];
        return __uint_as_float((e & 1) ? (wv & 0xFFFF0000u) : (wv << 16));
    };
    double s[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        s[e] = 0.0;
#pragma unroll
        for (int j = 0; j < NL; j++) s[e] += (double)X(j, e);  // padded keys add 0
    }
#pragma unroll
    for (int o = R; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; e++) s[e] += __shfl_xor(s[e], o);
    if (r == 0)
#pragma unroll
        for (int e = 0; e < 8; e++) psum[w][8 * cc + e] = s[e];
    __syncthreads();
    // one thread per channel: the block mean (and, below, the scale), so
    // each is formed once and the lanes read them back
    const size_t g0 = ((size_t)bh * nb + b) * D;
    if (t < D) {
        const float m = (float)((((psum[0][t] + psum[1][t]) + psum[2][t]) + psum[3][t]) / (double)n);
        cmu[t] = m;
        vmean[g0 + t] = m;
    }
    __syncthreads();
    float mu[8], am[8];
    {
        const float4 m0 = *reinterpret_cast<const float4*>(cmu + 8 * cc);
        const float4 m1 = *reinterpret_cast<const float4*>(cmu + 8 * cc + 4);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            mu[e] = (&m0.x)[e];
            mu[e + 4] = (&m1.x)[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) {
        am[e] = 0.0f;
#pragma unroll
        for (int j = 0; j < NL; j++)
            if (kw0 + 4 * (r + G * (j / 4)) + j % 4 < n) am[e] = fmaxf(am[e], fabsf(__fsub_rn(X(j, e), mu[e])));
    }
#pragma unroll
    for (int o = R; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; e++) am[e] = fmaxf(am[e], __shfl_xor(am[e], o));
    if (r == 0)
#pragma unroll
        for (int e = 0; e < 8; e++) pmax[w][8 * cc + e] = am[e];
    __syncthreads();
    if (t < D) {
        const float A = fmaxf(fmaxf(pmax[0][t], pmax[1][t]), fmaxf(pmax[2][t], pmax[3][t]));
        float sc, iv;
        group_scale(A, mode, sc, iv);
        cinv[t] = iv;
        vscale[g0 + t] = sc;
    }
    __syncthreads();
    float inv[8];
    {
        const float4 i0v = *reinterpret_cast<const float4*>(cinv + 8 * cc);
        const float4 i1v = *reinterpret_cast<const float4*>(cinv + 8 * cc + 4);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            inv[e] = (&i0v.x)[e];
            inv[e + 4] = (&i1v.x)[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const int c = 8 * cc + e;
        float y[NL];
#pragma unroll
        for (int j = 0; j < NL; j++) {
            const bool ok = kw0 + 4 * (r + G * (j / 4)) + j % 4 < n;
            y[j] = ok ? __fmul_rn(__fsub_rn(X(j, e), mu[e]), inv[e]) : 0.0f;  // padded slots: code 0
        }
        // quads r and r + G (D = 128) fill slots 32 r + 8 w .. + 7; quad r
        // (D = 64) fills slots 32 (r % 4) + 8 w + 4 (r / 4) .. + 3
        uint8_t* out = tile + c * PITCH + 32 * (r % 4) + 8 * w + 4 * (r / 4);
        if (NL == 8)
            *reinterpret_cast<uint2*>(out) = make_uint2(e4m3_pk4(y[0], y[1], y[2], y[3]),
                                                        e4m3_pk4(y[4 % NL], y[5 % NL], y[6 % NL], y[7 % NL]));
        else
            *reinterpret_cast<uint32_t*>(out) = e4m3_pk4(y[0], y[1], y[2], y[3]);
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
// being kk div 32 (32 consecutive slots of the permuted block; the attention
// kernel's loader orders K so that these are the 32-element k-blocks of its
// scaled matrix-core product).  Scale 2^e with e the least integer such that
// amax <= 6 * 2^e (no element clips); amax < 2^-100: codes 0.  Codes:
// v_cvt_scalef32_pk_fp4_f32 (round to nearest even of x / 2^e, exact
// scaling).  Output: codes [bh][nb][D][64] bytes, key kk of the block in
// slot kk, slot 2 t in the low nibble of byte t; scales [bh][nb][D][4] bytes
// e + 127.  Wave w holds keys 32 w .. 32 w + 31, i.e. group w, so each
// group's maximum stays inside one wave; lane l holds channels CPL l ..
// CPL l + CPL - 1 (CPL = D / 64) of every key of its wave, one key row per
// load across the wave.
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
    __shared__ uint32_t pexp[D];  // E8M0 byte of group g (wave g) in byte g
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * PITCH];
    const int b = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
    const int i0 = b * BLK;
    const int n = min(BLK, L - i0);
    const uint16_t* vb = v + (size_t)bh * L * D + CPL * lane;
    const int nw = min(KW, max(0, n - KW * w));
    // the wave's 32 permutation entries, one per lane of its lower half
    // (padded keys: entry 0, a valid row); every row load is issued before
    // any is used, and padded keys are zeroed afterwards
    int pv = 0;
    if (lane < KW && lane < nw) pv = clamp_row(perm[(size_t)bh * L + i0 + KW * w + lane], L);
    uint32_t raw[KW];
#pragma unroll
    for (int i = 0; i < KW; i++) {
        const int src = __shfl(pv, i);
        if (CPL == 2)
            raw[i] = *reinterpret_cast<const uint32_t*>(vb + (size_t)src * D);
        else
            raw[i] = vb[(size_t)src * D];
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
        // the wave's 32 keys are the key group w: its scale from their amax,
        // then the codes in slot order, slot 2t in the low nibble of byte t
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < KW; i++) am = fmaxf(am, fabsf(x[i][e]));
        const int ex = e8m0_exp(am);
        uint8_t* out = tile + c * PITCH + 16 * w;
#pragma unroll
        for (int j4 = 0; j4 < KW / 8; j4++) {
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; j++) y[j] = x[8 * j4 + j][e];
            const uint32_t pk = ex > -127 ? e2m1_pk8(y, ldexpf(1.0f, ex)) : 0u;  // zero group: codes 0
            *reinterpret_cast<uint32_t*>(out + 4 * j4) = pk;
        }
        reinterpret_cast<uint8_t*>(pexp + c)[w] = (uint8_t)(ex + 127);
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int e = 0; e < CPL; e++) {
            const int c = CPL * lane + e;
            const size_t gi = ((size_t)bh * nb + b) * D + c;
            vmean[gi] = mu[e];
            vexp[gi] = pexp[c];
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
