// vc_attn_bf16.hip -- BF16 flash attention for gfx950 on the scaffold of the
// FP8 VC-Attention kernel: the high-precision baseline the VC-Attention pages
// compare against (agihunt summary and MarkTechPost abstract: speedups are
// quoted over a BF16 FlashAttention kernel).  softmax(Q K^T / sqrt(d)) V with
// an exp2 online softmax (running max m, row sum l, rescale by 2^(m - m')).
//
// Same geometry as the FP8 kernel: 8 waves x 32 queries per workgroup, the
// score tile computed transposed (S^T = K Q^T, v_mfma_f32_16x16x32_bf16) so
// that each lane holds 32 scores of one query, and the bf16 probabilities a
// lane produces are its B operand of O^T = V^T P^T; the row sums are a
// product of a ones tile with those same bf16 probabilities.  K and V rows
// arrive row-major by direct global->LDS copies one block ahead into a
// two-stage ring (16-byte chunks XOR-swizzled per row), and the V^T operand
// of each product is read straight from the V rows with the gfx950 LDS
// transpose read (ds_read_b64_tr_b16): a 16-lane group hands in 16 pieces
// of 4 channels and gets back, per lane, one channel of 4 consecutive keys.
// One workgroup barrier per block.
#include "vc_device.hpp"
#include "vc_internal.hpp"
#include "vc_lds.hpp"

namespace vc {

namespace {

constexpr int NW = 8;
constexpr int QW = 32;

template <int D>
struct Bf16Tile {
    static constexpr int K_TILE = BLK * D * 2;  // [128 keys][D] bf16
    static constexpr int V_TILE = BLK * D * 2;  // [128 keys][D] bf16
    static constexpr int STAGE = K_TILE + V_TILE;
    static constexpr int LDS = 2 * STAGE;       // two stages
    static constexpr int KCH = D / 8;           // 16-byte chunks per K (or V) row
    static constexpr int NU = D / 32;           // 32-wide slices of the head dim
    static constexpr int PIECES = K_TILE / 1024;  // 1 KiB pieces of a K (or V) tile
    static constexpr int PPW = PIECES / NW;       // pieces of each per wave
};

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf as_bf(u32x4 x) {
    v8bf r;
    __builtin_memcpy(&r, &x, 16);
    return r;
}

// Swizzle of the 16-byte chunks of a K or V row: conflict-free 16-byte
// operand reads need distinct positions modulo 128 bytes per 8 lanes and
// modulo 256 bytes per 16 lanes (rows r = 0..15 of a tile go to lanes
// 0..15); the transpose reads of V (16 consecutive keys, two chunks each)
// then also fall on distinct positions at D = 128.
template <int D>
__device__ __forceinline__ int kswz(int r) {
    return D == 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1));
}

// Copies of block kb into `stage`: K rows, then V rows (LDS chunk p of row r
// holds chunk p ^ kswz(r) of the row).  Wave w takes 1 KiB pieces w,
// w + NW, ... of each.  Rows past L read as zeros.
template <int D>
struct Bf16Loader {
    using T = Bf16Tile<D>;
    v4si rk, rv;
    uint32_t off[T::PPW];
    int w;
    __device__ __forceinline__ Bf16Loader(const AttnBf16Args& a, int bh, int w_, int lane) : w(w_) {
        const uint32_t head = (uint32_t)((size_t)a.L * D * 2);
        rk = make_rsrc(a.k + (size_t)bh * a.L * D, head);
        rv = make_rsrc(a.v + (size_t)bh * a.L * D, head);
#pragma unroll
        for (int i = 0; i < T::PPW; i++) {
            const int p = (i * NW + w) * 64 + lane;  // 16-byte chunk of the tile
            const int r = p / T::KCH, cp = p % T::KCH;
            off[i] = (uint32_t)(r * D * 2 + ((cp ^ kswz<D>(r)) << 4));
        }
    }
    __device__ __forceinline__ void issue(lds_u8* stage, int kb) const {
        const uint32_t base = (uint32_t)kb * T::K_TILE;
#pragma unroll
        for (int i = 0; i < T::PPW; i++) lds_dma16(rk, stage + (i * NW + w) * 1024, off[i], base);
#pragma unroll
        for (int i = 0; i < T::PPW; i++) lds_dma16(rv, stage + T::K_TILE + (i * NW + w) * 1024, off[i], base);
    }
};

// V^T operand (A of O^T = V^T P^T) of channel tile ct and 32-key slice u from
// the row-major V rows: lane (col, g) gets channel 16 ct + col of keys
// 32 u + 4 g + j (first read) and 32 u + 16 + 4 g + j (second), j = 0..3 --
// the key order of the lane's bf16 probabilities.  For the transpose read,
// lane p of each 16-lane group supplies the 8-byte piece of key
// (4 g + p / 4) + 32 u (+ 16) holding channels 16 ct + 4 (p % 4) .. + 3.
template <int D>
__device__ __forceinline__ v8bf v_operand_tr(const lds_u8* sV, int ct, int u, int g, int p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const int kr = 4 * g + (p >> 2);                 // key within the 16-key half
    const int chunk = (2 * ct + ((p & 3) >> 1)) ^ kswz<D>(kr);  // (32 u + 16 h + kr) has the swizzle of kr
    const int off = (chunk << 4) | ((p & 1) << 3);
    const lds_u8* r0 = sV + (32 * u + kr) * (D * 2) + off;
    const lds_u8* r1 = r0 + 16 * (D * 2);
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VC_LDS v4s*)r0);
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VC_LDS v4s*)r1);
    u32x4 x;
    x[0] = (uint32_t)(uint16_t)a[0] | ((uint32_t)(uint16_t)a[1] << 16);
    x[1] = (uint32_t)(uint16_t)a[2] | ((uint32_t)(uint16_t)a[3] << 16);
    x[2] = (uint32_t)(uint16_t)b[0] | ((uint32_t)(uint16_t)b[1] << 16);
    x[3] = (uint32_t)(uint16_t)b[2] | ((uint32_t)(uint16_t)b[3] << 16);
    return as_bf(x);
}

// Running max and bf16 probabilities p = 2^(S c - m') of one block for both
// query tiles (exp2 on the transcendental unit directly: results below the
// fp32 normal range flush to zero, which a probability next to the row
// maximum never is).  MASKED: keys 16 kt + 4 g + i with 16 kt + i >= lim
// do not exist.  The max is four independent max3 chains.
template <bool MASKED>
__device__ __forceinline__ void softmax(v4f (&S)[2][8], uint32_t (&P)[2][16], float (&alpha)[2],
                                        float (&m)[2], int lim, float c) {
    float mx[2];
    if (MASKED) {
#pragma unroll
        for (int qt = 0; qt < 2; qt++)
#pragma unroll
            for (int kt = 0; kt < 8; kt++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (16 * kt + i >= lim) S[qt][kt][i] = -INFINITY;
    }
    float ch[2][2];
#pragma unroll
    for (int qt = 0; qt < 2; qt++)
#pragma unroll
        for (int h = 0; h < 2; h++) ch[qt][h] = vmax3(S[qt][4 * h][0], S[qt][4 * h][1], S[qt][4 * h][2]);
#pragma unroll
    for (int j = 0; j < 13; j += 2)
#pragma unroll
        for (int qt = 0; qt < 2; qt++)
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int e0 = 3 + j, e1 = 4 + j;
                const float a0 = S[qt][4 * h + e0 / 4][e0 % 4];
                if (e1 < 16)
                    ch[qt][h] = vmax3(ch[qt][h], a0, S[qt][4 * h + e1 / 4][e1 % 4]);
                else
                    ch[qt][h] = fmaxf(ch[qt][h], a0);
            }
#pragma unroll
    for (int qt = 0; qt < 2; qt++) mx[qt] = fmaxf(ch[qt][0], ch[qt][1]);
    {
        auto px = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx[0]), __float_as_uint(mx[0]), false, false);
        auto py = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx[1]), __float_as_uint(mx[1]), false, false);
        mx[0] = fmaxf(__uint_as_float(px[0]), __uint_as_float(px[1]));
        mx[1] = fmaxf(__uint_as_float(py[0]), __uint_as_float(py[1]));
        auto qx = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[0]), __float_as_uint(mx[0]), false, false);
        auto qy = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[1]), __float_as_uint(mx[1]), false, false);
        mx[0] = fmaxf(__uint_as_float(qx[0]), __uint_as_float(qx[1]));
        mx[1] = fmaxf(__uint_as_float(qy[0]), __uint_as_float(qy[1]));
    }
#pragma unroll
    for (int qt = 0; qt < 2; qt++) {
        const float mn = fmaxf(m[qt], mx[qt] * c);
        alpha[qt] = __builtin_amdgcn_exp2f(m[qt] - mn);  // 0 on the first block
        m[qt] = mn;
#pragma unroll
        for (int kt = 0; kt < 8; kt++) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qt][kt][i], c, -mn));
            P[qt][2 * kt] = pack_bf16x2(p[0], p[1]);
            P[qt][2 * kt + 1] = pack_bf16x2(p[2], p[3]);
        }
    }
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(AttnBf16Args a) {
    using T = Bf16Tile<D>;
    __shared__ __attribute__((aligned(16))) uint8_t lds_[T::LDS];
    lds_u8* lds = (lds_u8*)lds_;
    const int nwg = a.BH * a.nqt;
    const int pid = xcd_remap(blockIdx.x, nwg);
    const int bh = pid / a.nqt, qtile = pid % a.nqt;
    const int t = threadIdx.x, lane = t & 63, col = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int q0 = qtile * ATTN_BM + w * QW;
    const int L = a.L, nkb = a.nkb;

    // Q operands (B operand of S^T = K Q^T): lane (col, g) holds elements
    // [32 u + 8 g, 32 u + 8 g + 8) of query q0 + 16 qt + col
    v8bf qop[2][T::NU];
#pragma unroll
    for (int qt = 0; qt < 2; qt++) {
        const int row = q0 + 16 * qt + col;
#pragma unroll
        for (int u = 0; u < T::NU; u++) {
            u32x4 x = {0, 0, 0, 0};
            if (row < L) x = *reinterpret_cast<const u32x4*>(a.q + ((size_t)bh * L + row) * D + 32 * u + 8 * g);
            qop[qt][u] = as_bf(x);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    constexpr int NCT = D / 16;
    v4f O[2][NCT];
#pragma unroll
    for (int qt = 0; qt < 2; qt++)
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) O[qt][ct] = zero4;
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    const float c = a.C0;
    const Bf16Loader<D> ld(a, bh, w, lane);

    ld.issue(lds, 0);
    wait_vmcnt<0>();
    block_barrier();

    for (int kb = 0; kb < nkb; kb++) {
        const lds_u8* sK = lds + (kb & 1) * T::STAGE;
        const lds_u8* sV = sK + T::K_TILE;
        lds_u8* nxt = lds + ((kb + 1) & 1) * T::STAGE;
        const bool more = kb + 1 < nkb;
        if (more) ld.issue(nxt, kb + 1);  // the stage of block kb - 1, left before the last barrier

        v4f S[2][8];
#pragma unroll
        for (int kt = 0; kt < 8; kt++) {
            const int r = 16 * kt + col;
            const lds_u8* row = sK + r * (D * 2);
            v8bf kop[T::NU];
#pragma unroll
            for (int u = 0; u < T::NU; u++)
                kop[u] = as_bf(*reinterpret_cast<const VC_LDS u32x4*>(row + (((4 * u + g) ^ kswz<D>(r)) << 4)));
#pragma unroll
            for (int qt = 0; qt < 2; qt++) {
                v4f acc = zero4;
#pragma unroll
                for (int u = 0; u < T::NU; u++) acc = mfma_bf16(kop[u], qop[qt][u], acc);
                S[qt][kt] = acc;
            }
        }
        // K operand reads one key tile ahead of the products
        __builtin_amdgcn_sched_group_barrier(0x100, T::NU, 0);
#pragma unroll
        for (int kt = 0; kt < 8; kt++) {
            if (kt + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, T::NU, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * T::NU, 0);
        }

        const int nvalid = L - kb * BLK;
        float alpha[2];
        uint32_t P[2][16];
        if (nvalid < BLK)
            softmax<true>(S, P, alpha, m, nvalid - 4 * g, c);
        else
            softmax<false>(S, P, alpha, m, 0, c);
        // rescale a query tile only when one of its rows raised its max
#pragma unroll
        for (int qt = 0; qt < 2; qt++)
            if (__any(alpha[qt] != 1.0f)) {
#pragma unroll
                for (int ct = 0; ct < NCT; ct++) O[qt][ct] *= alpha[qt];
            }
        // P^T operand of slice u: keys 32u + 16 (j/4) + 4 g + j%4
        v8bf pop[2][4];
#pragma unroll
        for (int qt = 0; qt < 2; qt++)
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const u32x4 x = {P[qt][4 * u], P[qt][4 * u + 1], P[qt][4 * u + 2], P[qt][4 * u + 3]};
                pop[qt][u] = as_bf(x);
            }
        // row sums of the bf16 probabilities the products use: ones(16x32) P^T
        // per 32-key slice, on the matrix cores
        {
            v8bf ones;
#pragma unroll
            for (int i = 0; i < 8; i++) ones[i] = (__bf16)1.0f;
#pragma unroll
            for (int qt = 0; qt < 2; qt++) {
                v4f rs = zero4;
#pragma unroll
                for (int u = 0; u < 4; u++) rs = mfma_bf16(ones, pop[qt][u], rs);
                l[qt] = __builtin_fmaf(alpha[qt], l[qt], rs[0]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) {
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const v8bf vop = v_operand_tr<D>(sV, ct, u, g, col);
#pragma unroll
                for (int qt = 0; qt < 2; qt++) O[qt][ct] = mfma_bf16(vop, pop[qt][u], O[qt][ct]);
            }
        }
        // V operand reads one channel tile ahead of the products
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // row sums
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) {
            if (ct + 1 < NCT) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
        if (more) {  // block kb + 1 has landed in its stage
            wait_vmcnt<0>();
            block_barrier();
        }
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
    hipLaunchKernelGGL((attn_bf16_kernel<D, OB>), dim3(a.BH * a.nqt), dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnBf16Args& a, int d, int out_bf16, hipStream_t st) {
    if (d == 128) return out_bf16 ? launch_t<128, true>(a, st) : launch_t<128, false>(a, st);
    return out_bf16 ? launch_t<64, true>(a, st) : launch_t<64, false>(a, st);
}

}  // namespace vc
