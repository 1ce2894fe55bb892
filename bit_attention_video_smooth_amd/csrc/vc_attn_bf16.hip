// vc_attn_bf16.hip -- BF16 flash attention for gfx950 on the scaffold of the
// FP8 VC-Attention kernel: the high-precision baseline the VC-Attention pages
// compare against (agihunt summary and MarkTechPost abstract: speedups are
// quoted over a BF16 FlashAttention kernel).  softmax(Q K^T / sqrt(d)) V with
// an exp2 online softmax (running max m, row sum l, rescale by 2^(m - m')).
//
// Same geometry as the FP8 kernel: 8 waves x 32 queries per workgroup, the
// score tile computed transposed (S^T = K Q^T, v_mfma_f32_16x16x32_bf16) so
// that each lane holds 32 scores of one query, and the bf16 probabilities a
// lane produces are its B operand of O^T = V^T P^T.  K tiles stream to LDS
// with direct 16-byte loads; V tiles are transposed through registers into a
// [channel][key-slot] LDS layout (4 consecutive keys per 8-byte write).
#include "vc_device.hpp"
#include "vc_internal.hpp"

namespace vc {

namespace {

constexpr int NW = 8;
constexpr int QW = 32;

template <int D>
struct Bf16Tile {
    static constexpr int K_TILE = BLK * D * 2;  // [128 keys][D] bf16
    static constexpr int V_TILE = D * BLK * 2;  // [D][128 slots] bf16
    static constexpr int STAGE = K_TILE + V_TILE;
    static constexpr int KCH = D / 8;           // 16-byte chunks per K row
    static constexpr int NU = D / 32;           // 32-wide slices of the head dim
    static constexpr int VUNITS = (BLK / 4) * (D / 8);  // (4 keys x 8 channels) units
};

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_bf(uint4 x) {
    v8bf r;
    __builtin_memcpy(&r, &x, 16);
    return r;
}

__device__ __forceinline__ int vswz(int c) { return (c ^ (c >> 3)) & 15; }

template <int D>
__device__ __forceinline__ void issue_k_load(const AttnBf16Args& a, uint8_t* stage, int bh, int kb,
                                             int w, int lane) {
    using T = Bf16Tile<D>;
    const uint8_t* gK = reinterpret_cast<const uint8_t*>(a.k + ((size_t)bh * a.L) * D);
    constexpr int NCHK = T::K_TILE / 16;
#pragma unroll
    for (int i = 0; i < NCHK / (NW * 64); i++) {
        const int base = (i * NW + w) * 64;
        const int p = base + lane;
        const int r = p / T::KCH, cp = p % T::KCH;
        const int c = cp ^ (r & (T::KCH - 1));
        int key = kb * BLK + r;
        key = key < a.L ? key : a.L - 1;  // rows past L are masked in the softmax
        __builtin_amdgcn_global_load_lds(gK + (size_t)key * D * 2 + c * 16,
                                         (VC_LDS void*)(stage + base * 16), 16, 0, 0);
    }
}

template <int D>
__device__ __forceinline__ void load_v_regs(const AttnBf16Args& a, int bh, int kb, int t, uint4 (&r)[4]) {
    using T = Bf16Tile<D>;
    if (t < T::VUNITS) {
        const int kg = t / (D / 8), cc = t % (D / 8);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            int key = kb * BLK + 4 * kg + j;
            key = key < a.L ? key : a.L - 1;
            r[j] = *reinterpret_cast<const uint4*>(a.v + ((size_t)bh * a.L + key) * D + cc * 8);
        }
    }
}

template <int D>
__device__ __forceinline__ void store_v_lds(uint8_t* stage, int t, const uint4 (&r)[4]) {
    using T = Bf16Tile<D>;
    if (t < T::VUNITS) {
        uint8_t* sV = stage + T::K_TILE;
        const int kg = t / (D / 8), cc = t % (D / 8);
        const int k0 = 4 * kg;
        const int u = k0 / 32, h = (k0 % 32) / 16, gq = (k0 % 16) / 4;
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int c = cc * 8 + e;
            const int sh = (e & 1) * 16;
            const uint32_t k0v = (w0[e >> 1] >> sh) & 0xFFFFu, k1v = (w1[e >> 1] >> sh) & 0xFFFFu;
            const uint32_t k2v = (w2[e >> 1] >> sh) & 0xFFFFu, k3v = (w3[e >> 1] >> sh) & 0xFFFFu;
            const int chunk = (4 * u + gq) ^ vswz(c);
            *reinterpret_cast<uint2*>(sV + c * (BLK * 2) + chunk * 16 + h * 8) =
                make_uint2(k0v | (k1v << 16), k2v | (k3v << 16));
        }
    }
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64, 2) void attn_bf16_kernel(AttnBf16Args a) {
    using T = Bf16Tile<D>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int nwg = a.BH * a.nqt;
    const int pid = xcd_remap(blockIdx.x, nwg);
    const int bh = pid / a.nqt, qtile = pid % a.nqt;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, col = lane & 15, g = lane >> 4;
    const int q0 = qtile * ATTN_BM + w * QW;
    const int L = a.L, nkb = a.nkb;

    v8bf qop[2][T::NU];
#pragma unroll
    for (int qt = 0; qt < 2; qt++) {
        const int row = q0 + 16 * qt + col;
#pragma unroll
        for (int u = 0; u < T::NU; u++) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (row < L) x = *reinterpret_cast<const uint4*>(a.q + ((size_t)bh * L + row) * D + 32 * u + 8 * g);
            qop[qt][u] = as_bf(x);
        }
    }
    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    constexpr int NCT = D / 16;
    v4f O[2][NCT];
#pragma unroll
    for (int qt = 0; qt < 2; qt++)
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) O[qt][ct] = zero4;
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    const float c = a.C0;

    uint4 vr[4];
    issue_k_load<D>(a, smem, bh, 0, w, lane);
    load_v_regs<D>(a, bh, 0, t, vr);
    store_v_lds<D>(smem, t, vr);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kb = 0; kb < nkb; kb++) {
        uint8_t* stage = smem + (kb & 1) * T::STAGE;
        uint8_t* next = smem + ((kb + 1) & 1) * T::STAGE;
        const bool more = kb + 1 < nkb;
        if (more) {
            issue_k_load<D>(a, next, bh, kb + 1, w, lane);
            load_v_regs<D>(a, bh, kb + 1, t, vr);
        }
        const uint8_t* sK = stage;
        const uint8_t* sV = stage + T::K_TILE;

        v4f S[2][8];
#pragma unroll
        for (int kt = 0; kt < 8; kt++) {
            const int r = 16 * kt + col;
            const uint8_t* row = sK + r * (D * 2);
            v8bf kop[T::NU];
#pragma unroll
            for (int u = 0; u < T::NU; u++)
                kop[u] = as_bf(*reinterpret_cast<const uint4*>(row + (((4 * u + g) ^ (r & (T::KCH - 1))) << 4)));
#pragma unroll
            for (int qt = 0; qt < 2; qt++) {
                v4f acc = zero4;
#pragma unroll
                for (int u = 0; u < T::NU; u++) acc = mfma_bf16(kop[u], qop[qt][u], acc);
                S[qt][kt] = acc;
            }
        }

        const int nvalid = L - kb * BLK;
        const bool partial = nvalid < BLK;
        float alpha[2];
        uint32_t P[2][16];
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
            if (partial) {
#pragma unroll
                for (int kt = 0; kt < 8; kt++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (16 * kt + 4 * g + i >= nvalid) S[qt][kt][i] = -INFINITY;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 8; kt++)
                mx = fmaxf(mx, fmaxf(fmaxf(S[qt][kt][0], S[qt][kt][1]), fmaxf(S[qt][kt][2], S[qt][kt][3])));
            mx = max_over_groups(mx);
            const float mn = fmaxf(m[qt], mx * c);
            alpha[qt] = exp2f(m[qt] - mn);
            m[qt] = mn;
            float rs = 0.f;
#pragma unroll
            for (int kt = 0; kt < 8; kt++) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    p[i] = exp2f(__builtin_fmaf(S[qt][kt][i], c, -mn));
                    rs += p[i];
                }
                P[qt][2 * kt] = pack_bf16x2(p[0], p[1]);
                P[qt][2 * kt + 1] = pack_bf16x2(p[2], p[3]);
            }
            // sum over the four lane groups of this query
            auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(rs), __float_as_uint(rs), false, false);
            rs = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
            auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(rs), __float_as_uint(rs), false, false);
            rs = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
            l[qt] = __builtin_fmaf(alpha[qt], l[qt], rs);
        }
        if (__any((alpha[0] != 1.0f) | (alpha[1] != 1.0f))) {
#pragma unroll
            for (int qt = 0; qt < 2; qt++)
#pragma unroll
                for (int ct = 0; ct < NCT; ct++) O[qt][ct] *= alpha[qt];
        }
        // P^T operand of slice u: keys 32u + 16 (j/4) + 4 g + j%4
        v8bf pop[2][4];
#pragma unroll
        for (int qt = 0; qt < 2; qt++)
#pragma unroll
            for (int u = 0; u < 4; u++) {
                uint4 x = make_uint4(P[qt][4 * u], P[qt][4 * u + 1], P[qt][4 * u + 2], P[qt][4 * u + 3]);
                pop[qt][u] = as_bf(x);
            }
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) {
            const int cr = 16 * ct + col;
            const uint8_t* row = sV + cr * (BLK * 2);
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const v8bf vop = as_bf(*reinterpret_cast<const uint4*>(row + (((4 * u + g) ^ vswz(cr)) << 4)));
#pragma unroll
                for (int qt = 0; qt < 2; qt++) O[qt][ct] = mfma_bf16(vop, pop[qt][u], O[qt][ct]);
            }
        }
        if (more) store_v_lds<D>(next, t, vr);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

#pragma unroll
    for (int qt = 0; qt < 2; qt++) {
        const int row = q0 + 16 * qt + col;
        if (row >= L) continue;
        const float il = 1.0f / l[qt];
        if (OUT_BF16) {
            uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((size_t)bh * L + row) * D;
#pragma unroll
            for (int ct = 0; ct < NCT; ct++) {
                uint32_t lo = pack_bf16x2(O[qt][ct][0] * il, O[qt][ct][1] * il);
                uint32_t hi = pack_bf16x2(O[qt][ct][2] * il, O[qt][ct][3] * il);
                *reinterpret_cast<uint2*>(o + 16 * ct + 4 * g) = make_uint2(lo, hi);
            }
        } else {
            float* o = reinterpret_cast<float*>(a.out) + ((size_t)bh * L + row) * D;
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
                *reinterpret_cast<float4*>(o + 16 * ct + 4 * g) =
                    make_float4(O[qt][ct][0] * il, O[qt][ct][1] * il, O[qt][ct][2] * il, O[qt][ct][3] * il);
        }
    }
}

template <int D, bool OB>
hipError_t launch_t(const AttnBf16Args& a, hipStream_t st) {
    const int smem = 2 * Bf16Tile<D>::STAGE;
    auto kern = attn_bf16_kernel<D, OB>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3(a.BH * a.nqt), dim3(NW * 64), smem, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnBf16Args& a, int d, int out_bf16, hipStream_t st) {
    if (d == 128) return out_bf16 ? launch_t<128, true>(a, st) : launch_t<128, false>(a, st);
    return out_bf16 ? launch_t<64, true>(a, st) : launch_t<64, false>(a, st);
}

}  // namespace vc
