// vc_attn_fp8_kernel.hpp -- fused VC-Attention forward for gfx950: FP8
// matrix-core QK^T, ExpCast-FP8 online softmax, FP8 matrix-core PV,
// block-mean restore; and, on the same scaffold, the SAGE-style quantised
// attention of the TensorRT-LLM blog ("Quantized Attention": one Q scale per
// query token, one K scale per 16 keys, INT8 or FP8 QK^T, FP8 PV with one V
// scale per channel); and 4-bit V-Smooth (E2M1 V residual and probabilities
// with power-of-two scales per 32-key group, on the scaled FP4 matrix
// cores).  The template is instantiated by vc_attn_fp8.hip (V-Smooth),
// vc_attn_sage.hip (SAGE) and vc_attn_fp4.hip (4-bit), compiled side by side.
//
// Method: agihunt summary (ExpCast-FP8 bullet: E4M3 probability codes from
// log-domain scores with one fused multiply-add; V-Smooth bullet: the mean
// is restored from the row sum the online softmax keeps), MarkTechPost
// abstract (byte ~ 8 log2 v + 56, beta = -0.35, clamped at zero), online
// softmax notation of the TensorRT-LLM blog ("Sparse Attention with Skip
// Softmax": block max m~ and running max m).
//
// Design for CDNA4 (wave64, v_mfma_f32_16x16x128_f8f6f4):
//  * one workgroup = 8 waves = 256 queries of one head; each wave owns 32
//    queries (two 16-query tiles) and streams all KV blocks of the head;
//  * the score tile is computed transposed, S^T = K8 Q8^T, so that every
//    lane holds 32 scores of a single query: the row max needs only two
//    cross-lane swaps, and the 32 ExpCast bytes a lane produces are exactly
//    its B operand of the PV product O^T = V8^T P^T -- no shuffles between
//    softmax and PV;
//  * the V residual codes arrive block-transposed in the slot order of that
//    B operand (written so by the preprocessing kernel);
//  * the row sum of the ExpCast bytes is one more FP8 product (a row of
//    ones times P^T), exact, off the vector ALU;
//  * K8/V8 tiles stream into a four-stage LDS ring with direct-to-LDS
//    16-byte loads (XOR-swizzled 16-byte chunks) two blocks ahead; each
//    stage is its own LDS object so the compiler's wait insertion can tell
//    a stage being filled from the stage being read;
//  * a wave issues a vector instruction at most every ~5 cycles (~10 when
//    it depends on the one before), so the vector work is written as
//    independent chains; while one wave streams matrix products, the other
//    wave on its SIMD still issues about four vector instructions per
//    product, so the two wave groups run offset by most of a block (one
//    workgroup barrier per block, passed at different points of the block
//    by the two groups) and one group's S^T products meet the other's
//    softmax;
//  * workgroups are remapped so that the query tiles of one head run on
//    one XCD and share its L2.
//
// SAGE recipe on this scaffold: a lane holds one query and a 16-key tile is
// one K scale group, so the score coefficient c = fp32(fp32(s_q C0) s_k)
// varies per (lane, key tile) only; the running max takes each tile's
// largest score times its coefficient (fp32 rounding is monotone, so this is
// the largest scaled score).  INT8 scores come from two 16x16x64 integer
// products per tile (the halves of the 32-byte operands, the same split for
// both sides, so the sum is exact) and convert to fp32 exactly (|S| < 2^24).
// The per-channel V scale is the same for every block, so it is applied once
// at the end and the per-block epilogue is a plain add.
#pragma once

#include "vc_device.hpp"
#include "vc_internal.hpp"
#include "vc_lds.hpp"

namespace vc {

namespace {

// score recipes of the kernel template
enum : int {
    REC_VC = 0,       // V-Smooth: FP8 Q/K, one scale per 128-token block, block means
    REC_SAGE_F8 = 1,  // SAGE: FP8 Q/K codes, per-token Q and per-16-key K scales
    REC_SAGE_I8 = 2,  // SAGE: INT8 Q/K codes, same scales
    REC_VC4 = 3       // 4-bit V-Smooth: E2M1 residual and probabilities, E8M0 scales per 32-key group
};

constexpr int NW = 8;    // waves per workgroup (group 0 = waves 0-3 also copy)
constexpr int QW = 32;   // queries per wave
static_assert(NW * QW == ATTN_BM, "tile");

template <int D>
struct Fp8Tile {
    static constexpr int K_TILE = BLK * D;      // bytes of one K8 block  [128 keys][D]
    static constexpr int V_TILE = D * BLK;      // bytes of one V8 block  [D][128 slots]
    static constexpr int V4_TILE = D * BLK / 2; // bytes of one E2M1 V block [D][64]
    static constexpr int LPTV = V4_TILE / 4096; // E2M1 V chunks per loading thread
    // the block's per-channel V scales (or E8M0 bytes) and means, 2 D
    // floats, each loading wave copying its quarter; then a 256-byte window
    // of K scales from the block on, copied by every loading wave (same data)
    static constexpr int SV_OFF = K_TILE + V_TILE;
    static constexpr int SVM = 2 * D * 4;
    static constexpr int KS_OFF = SV_OFF + SVM;
    static constexpr int STAGE = KS_OFF + 256;
    static constexpr int KCH = D / 16;          // 16-byte chunks per K row
    static constexpr int NCHK = K_TILE / 16;    // 16-byte chunks per K (or V) tile
    static constexpr int LPT = NCHK / 256;      // chunks per loading thread (group 0 loads)
    static constexpr int NCT = D / 16;          // 16-channel output tiles
};

// XOR swizzle of the 16-byte chunks of LDS tile rows.  A 16-byte-per-lane
// LDS read moves 256 bytes per clock; it runs at that rate only when every
// group of 8 consecutive lanes touches 8 distinct 16-byte positions modulo
// 128 bytes and the 16 lanes of a quarter-wave touch 16 distinct positions
// modulo 256 bytes (measured on gfx950).  A matrix-core operand read sends
// rows r = 0..15 of a tile to lanes 0..15 with one chunk index, so the
// swizzle must make the chunk position depend on r & 7 within each half and
// flip between the halves: f(r) = (r & 7) ^ (r >> 3) for 128-byte rows, and
// ((r >> 1) & 3) ^ (r >> 3) for 64-byte rows.
__host__ __device__ constexpr int chunk_swizzle(int r, int nch) {
    return nch == 8 ? ((r & 7) ^ ((r >> 3) & 1)) : (((r >> 1) & 3) ^ ((r >> 3) & 1));
}

// A/B operand of one 16-row tile: row `r` of a tile with `pitch`-byte rows of
// `nch` 16-byte chunks (swizzled as above); lane group g takes bytes
// [32 g, 32 g + 32) of the logical row.

__device__ __forceinline__ v8i lds_operand(const lds_u8* tile, int r, int pitch, int nch, int g) {
    const int sw = chunk_swizzle(r, nch);
    const lds_u8* row = tile + r * pitch;
    const u32x4 a = *reinterpret_cast<const VC_LDS u32x4*>(row + (((2 * g) ^ sw) << 4));
    const u32x4 b = *reinterpret_cast<const VC_LDS u32x4*>(row + (((2 * g + 1) ^ sw) << 4));
    v8i o;
    o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
    o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
    return o;
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// INT8 S^T tile over 128 k: bytes [32 g, 32 g + 16) of both operands in one
// 16x16x64 product and bytes [32 g + 16, 32 g + 32) in the other.  The lane
// layout of both operands is the same, so every k is counted once; the
// integer result is returned in a float vector's bits.
__device__ __forceinline__ v4f mfma_i8_128(const v8i& a, const v8i& b) {
    const v4i alo = {a[0], a[1], a[2], a[3]}, ahi = {a[4], a[5], a[6], a[7]};
    const v4i blo = {b[0], b[1], b[2], b[3]}, bhi = {b[4], b[5], b[6], b[7]};
    const v4i z = {0, 0, 0, 0};
    v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, blo, z, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, bhi, acc, 0, 0, 0);
    return __builtin_bit_cast(v4f, acc);
}

// Row max of two query tiles over the four lane groups, the two reductions
// interleaved.
__device__ __forceinline__ void max_over_groups2(float& x, float& y) {
    auto px = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    auto py = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    x = fmaxf(__uint_as_float(px[0]), __uint_as_float(px[1]));
    y = fmaxf(__uint_as_float(py[0]), __uint_as_float(py[1]));
    auto qx = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    auto qy = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    x = fmaxf(__uint_as_float(qx[0]), __uint_as_float(qx[1]));
    y = fmaxf(__uint_as_float(qy[0]), __uint_as_float(qy[1]));
}

// ExpCast bytes of 16 values y[4 d + i] -> byte i of p_d: round to nearest
// even, saturate to [0, 255] (y never exceeds 126 here).  The conversions of
// the four dwords are interleaved so that each one's dependency on the
// previous byte of the same dword is four instructions back.
__device__ __forceinline__ void cvt_bytes16(const float (&y)[16], uint32_t& p0, uint32_t& p1,
                                            uint32_t& p2, uint32_t& p3) {
    asm("v_cvt_pk_u8_f32 %0, %4, 0, 0\n\t"
        "v_cvt_pk_u8_f32 %1, %8, 0, 0\n\t"
        "v_cvt_pk_u8_f32 %2, %12, 0, 0\n\t"
        "v_cvt_pk_u8_f32 %3, %16, 0, 0\n\t"
        "v_cvt_pk_u8_f32 %0, %5, 1, %0\n\t"
        "v_cvt_pk_u8_f32 %1, %9, 1, %1\n\t"
        "v_cvt_pk_u8_f32 %2, %13, 1, %2\n\t"
        "v_cvt_pk_u8_f32 %3, %17, 1, %3\n\t"
        "v_cvt_pk_u8_f32 %0, %6, 2, %0\n\t"
        "v_cvt_pk_u8_f32 %1, %10, 2, %1\n\t"
        "v_cvt_pk_u8_f32 %2, %14, 2, %2\n\t"
        "v_cvt_pk_u8_f32 %3, %18, 2, %3\n\t"
        "v_cvt_pk_u8_f32 %0, %7, 3, %0\n\t"
        "v_cvt_pk_u8_f32 %1, %11, 3, %1\n\t"
        "v_cvt_pk_u8_f32 %2, %15, 3, %2\n\t"
        "v_cvt_pk_u8_f32 %3, %19, 3, %3"
        : "=&v"(p0), "=&v"(p1), "=&v"(p2), "=&v"(p3)
        : "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]), "v"(y[4]), "v"(y[5]), "v"(y[6]), "v"(y[7]),
          "v"(y[8]), "v"(y[9]), "v"(y[10]), "v"(y[11]), "v"(y[12]), "v"(y[13]), "v"(y[14]), "v"(y[15]));
}

// Per-lane byte offsets of the 16-byte chunks a group-0 wave copies: the
// same for every block.  Tile rows of 128 bytes (K8 at d = 128 and every V8
// tile) or 64 bytes (K8 at d = 64); LDS chunk position cp of row r receives
// global chunk cp ^ chunk_swizzle(r).  (Slices are 4 KiB = a whole number of
// swizzle periods, so the row index within a slice gives the same swizzle.)
__device__ __forceinline__ uint32_t dma_offset(int w, int lane, int row_bytes) {
    const int cpr = row_bytes / 16;      // chunks per row
    const int p = w * 64 + lane;         // chunk position within a 4 KiB slice
    const int r = p / cpr, cp = p % cpr;
    return (uint32_t)(r * row_bytes + ((cp ^ chunk_swizzle(r, cpr)) << 4));
}

// Group-0 waves (w < 4, 256 threads) copy block kb into `stage`: their
// share of the K8 and V8 tiles, plus (each wave, into its own slot) the
// block's per-channel scales and means and the K scales from block kb on
// (SAGE: no per-block V data, and the K scales are the block's eight 16-key
// group scales).
// Every copy runs with all 64 lanes, so each loading wave issues exactly
// NLD copies per block and the wait counts below are exact.  Buffer
// descriptors cover one head: reads past it return zeros.
template <int D, int MODE, bool W32 = false>
struct Fp8Loader {
    using T = Fp8Tile<D>;
    static constexpr bool SAGE = MODE == REC_SAGE_F8 || MODE == REC_SAGE_I8;
    static constexpr bool FP4V = MODE == REC_VC4;
    static constexpr int NVC = FP4V ? T::LPTV : T::LPT;  // V copies per loading thread
    // copies per loading thread and block: the K part (K8 tile, K scales)
    // and the V part (V8 tile, per-channel scales and means)
    static constexpr int NLD_K = T::LPT + 1;
    static constexpr int NLD_V = NVC + (SAGE ? 0 : 1) + (W32 ? 1 : 0);
    static constexpr int NLD = NLD_K + NLD_V;
    v4si rk, rv, rks;
    const float *vs, *vm;
    uint32_t off_k, off_v;
    int sv_p;
    // 4-bit V-Smooth: K rows enter LDS reordered so that the S^T products
    // give lane group g the keys 32 g .. 32 g + 31 of the block (one 32-key
    // group, the k-block of the lane's scaled FP4 operand): LDS row
    // 16 kt + 4 g + i holds key 32 g + 4 kt + i.  A 4 KiB K slice s holds
    // LDS rows s R .. s R + R - 1 (R = 4096 / D), whose keys are those of
    // slice 0's rows plus 8 s (D = 128) or 16 s (D = 64) -- 1024 s bytes
    // either way -- so one in-block offset (slice 0) serves every slice.
    uint32_t off_k4;
    // 32x32 wave (Fp8Wave32): LDS row 32 t + 8 j + 4 h + i of a block holds
    // key 64 (t % 2) + 16 j + 8 (t / 2) + 4 h + i, so that the 32 x 32 S^T
    // tiles give lane half h, for k-step s of the P V product, the keys of V
    // slots 64 s + 32 h .. + 31 in the slot order of the V codes.  A 4 KiB
    // slice covers whole 32-row tiles; slice i's keys are slice 0's plus
    // key_off32(i) (below), so one in-block offset serves every slice.
    uint32_t off_k32;
    __device__ __forceinline__ static constexpr int key_off32(int i) {
        return 64 * ((i * (4096 / D) / 32) % 2) + 8 * ((i * (4096 / D) / 32) / 2);
    }
    int w, lane;  // w: the wave's index within its group of four
    // 32x32 wave: the history of block means in LDS ([32][D] floats, slot
    // kb % 32), which the V part also fills
    VC_LDS float* hist;
    __device__ __forceinline__ Fp8Loader(const AttnArgs& a, int bh, int w_, int lane_, VC_LDS float* hist_ = nullptr)
        : w(w_ & 3), lane(lane_), hist(hist_) {
        const size_t Lp = (size_t)a.nb * BLK;
        rk = make_rsrc(a.k8 + (size_t)bh * Lp * D, (uint32_t)(Lp * D));
        const size_t vrow = FP4V ? BLK / 2 : BLK;  // bytes per channel row of a V block
        rv = make_rsrc(a.v8 + (size_t)bh * a.nb * D * vrow, (uint32_t)((size_t)a.nb * D * vrow));
        if (SAGE) {
            rks = make_rsrc(a.k_scale + (size_t)bh * (Lp / 16), (uint32_t)(Lp / 16 * 4));
            vs = vm = nullptr;
        } else {
            rks = make_rsrc(a.k_scale + (size_t)bh * a.nb, (uint32_t)(a.nb * 4));
            vs = a.v_scale + (size_t)bh * a.nb * D;
            vm = a.v_mean + (size_t)bh * a.nb * D;
        }
        off_k = dma_offset(w, lane, D);
        {
            const int cpr = D / 16;                     // 16-byte chunks per K row
            const int p = w * 64 + lane;
            const int r = p / cpr, cp = p % cpr;        // LDS row (slice 0) and chunk position
            const int key = 32 * ((r % 16) / 4) + 4 * (r / 16) + r % 4;
            off_k4 = (uint32_t)(key * D + ((cp ^ chunk_swizzle(r, cpr)) << 4));
        }
        {
            const int cpr = D / 16;
            const int p = w * 64 + lane;
            const int r = p / cpr, cp = p % cpr;        // LDS row (slice 0) and chunk position
            const int t = r / 32, rr = r % 32;
            const int key = 64 * (t % 2) + 8 * (t / 2) + 16 * (rr / 8) + 4 * ((rr / 4) % 2) + rr % 4;
            off_k32 = (uint32_t)(key * D + ((cp ^ chunk_swizzle(r, cpr)) << 4));
        }
        off_v = dma_offset(w, lane, FP4V ? BLK / 2 : BLK);
        // float p of the [scales | means] region: wave w's quarter, lanes
        // past 2 D (D = 64) repeating the first half with the same data
        sv_p = (w * 64 + lane) % (2 * D);
    }
    // The wave's LDS offset is made opaque at each issue so that the
    // per-copy LDS addresses (four stages x every copy) are formed there by
    // scalar adds instead of being kept in scalar registers for the whole
    // kernel (which spills them into vector-register lanes).
    // K part: K8 copies I0 .. I1 - 1 and, with KS, the K scales
    template <int I0, int I1, bool KS>
    __device__ __forceinline__ void issue_k_part(lds_u8* stage, int kb) const {
        int wo = w * 1024;
        asm volatile("" : "+s"(wo));
#pragma unroll
        for (int i = I0; i < I1; i++) {
            if (FP4V)
                lds_dma16(rk, stage + wo + i * 4096, off_k4, kb * T::K_TILE + i * 1024);
            else if (W32)
                lds_dma16(rk, stage + wo + i * 4096, off_k32, kb * T::K_TILE + key_off32(i) * D);
            else
                lds_dma16(rk, stage + wo + i * 4096, off_k, kb * T::K_TILE + i * 4096);
        }
        if (KS) lds_dma4(rks, stage + T::KS_OFF, lane * 4, SAGE ? kb * 32 : kb * 4);
    }
    // V part: V8 copies I0 .. I1 - 1 and, with SV, the scales and means
    template <int I0, int I1, bool SV>
    __device__ __forceinline__ void issue_v_part(lds_u8* stage, int kb) const {
        int wo = w * 1024;
        asm volatile("" : "+s"(wo));
#pragma unroll
        for (int i = I0; i < I1; i++)
            lds_dma16(rv, stage + T::K_TILE + wo + i * 4096, off_v, kb * (FP4V ? T::V4_TILE : T::V_TILE) + i * 4096);
        if (SV && !SAGE) {
            const float* src = (sv_p < D ? vs + sv_p : vm + (sv_p - D)) + (size_t)kb * D;
            lds_dma4_flat(src, stage + T::SV_OFF + ((wo >> 2) % T::SVM));
        }
        if (SV && W32) {
            // the block's means, float (w * 64 + lane) % D of history slot
            // kb % 32 (at D = 64 all four waves copy the same 64 floats)
            const float* src = vm + (size_t)kb * D + (sv_p % D);
            lds_dma4_flat(src, reinterpret_cast<lds_u8*>(hist + (kb % 32) * D) + ((wo >> 2) % (D * 4)));
        }
    }
    __device__ __forceinline__ void issue_k(lds_u8* stage, int kb) const { issue_k_part<0, T::LPT, true>(stage, kb); }
    __device__ __forceinline__ void issue_v(lds_u8* stage, int kb) const { issue_v_part<0, NVC, true>(stage, kb); }
    __device__ __forceinline__ void issue(lds_u8* stage, int kb) const {
        issue_k(stage, kb);
        issue_v(stage, kb);
    }
};

template <int D, bool DUMP, bool SKIP, bool NAIVE, int MODE>
struct Fp8Wave {
    using T = Fp8Tile<D>;
    static constexpr bool SAGE = MODE == REC_SAGE_F8 || MODE == REC_SAGE_I8;
    static constexpr bool FP4V = MODE == REC_VC4;
    static_assert(!FP4V || NAIVE, "4-bit probabilities come by exp-then-cast");
    const AttnArgs& a;
    int bh, w, lane, col, g, grp, q0, L, nb;
    size_t Lp;
    bool dump;
    float sq;
    v8i qop[2];
    v4f O[2][T::NCT];
    float m[2], l[2];
    // per-block values carried between the stages of a block
    v4f S[2][8];
    uint32_t P[2][8];
    float alpha[2];
    float krow[2], cb;
    bool reject[2];  // Skip Softmax: this lane's row rejects the block
    // SAGE: fp32(s_q C0) of the lane's two queries (times 8 for ExpCast) and
    // the coefficients of the block's eight 16-key tiles
    float sqx[2];
    float cf[2][8];
    // 4-bit: E8M0 byte (e + 127) of each query tile's probability group, and
    // the lane's largest valid score of the block (its group's 32 keys)
    int sp[2];
    float lmx[2];
    // E4M3 1.0 in every byte: the A operand of the 8-bit row sums. Kept
    // resident where registers allow (rebuilding it each block costs more
    // than its 8 registers); the INT8 SAGE instance, whose score products
    // need more registers, rebuilds it per block instead of spilling.
    static constexpr bool ONES_RESIDENT = MODE != REC_SAGE_I8;
    static constexpr bool SPLIT = false;  // all copies by waves 0-3
    v8i ones8;

    // In-block key of score (kt, i) of this lane: 16 kt + 4 g + i, or for
    // 4-bit V-Smooth (K rows reordered in LDS, see Fp8Loader) 32 g + 4 kt + i.
    __device__ __forceinline__ int key_of(int kt, int i) const {
        return FP4V ? 32 * g + 4 * kt + i : 16 * kt + 4 * g + i;
    }
    // with lim = nvalid - key_of(0, 0) (the block's valid keys past the
    // lane's first), score (kt, i) belongs to a key that exists
    __device__ __forceinline__ static bool key_ok(int kt, int i, int lim) {
        return (FP4V ? 4 * kt + i : 16 * kt + i) < lim;
    }

    __device__ __forceinline__ Fp8Wave(const AttnArgs& args, int bh_, int qtile, int w_, int lane_)
        : a(args), bh(bh_), w(w_), lane(lane_) {
        col = lane & 15;
        g = lane >> 4;
        grp = w >> 2;
        q0 = qtile * ATTN_BM + w * QW;
        L = a.L;
        nb = a.nb;
        Lp = (size_t)nb * BLK;
        dump = DUMP && bh == a.dump_bh && qtile == a.dump_qt;
        // Q8 operands (B operand of S^T = K8 Q8^T): lane (col, g) holds bytes
        // [32 g, 32 g + 32) of query q0 + 16 qt + col.
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
            const int row = q0 + 16 * qt + col;
            uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
            if (row < L && (D == 128 || g < 2)) {
                const uint8_t* src = a.q8 + ((size_t)bh * Lp + row) * D + 32 * g;
                x = *reinterpret_cast<const uint4*>(src);
                y = *reinterpret_cast<const uint4*>(src + 16);
            }
            qop[qt][0] = x.x; qop[qt][1] = x.y; qop[qt][2] = x.z; qop[qt][3] = x.w;
            qop[qt][4] = y.x; qop[qt][5] = y.y; qop[qt][6] = y.z; qop[qt][7] = y.w;
        }
        if (SAGE) {
#pragma unroll
            for (int qt = 0; qt < 2; qt++) {
                const int row = q0 + 16 * qt + col;
                const float sc = __fmul_rn(row < L ? a.q_scale[(size_t)bh * Lp + row] : 0.0f, a.C0);
                sqx[qt] = NAIVE ? sc : 8.0f * sc;  // times 8: exact
            }
            sq = 0.0f;
        } else {
            const int qblk = min(q0 / BLK, nb - 1);
            sq = a.q_scale[(size_t)bh * nb + qblk];
        }
        if (ONES_RESIDENT) ones8 = e4m3_ones();
        // the Q operands and scale are in registers before any block copy is
        // issued, so no later wait on them can drain the copy pipeline
        __builtin_amdgcn_s_waitcnt(0);
        const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
            m[qt] = -INFINITY;
            l[qt] = 0.f;
#pragma unroll
            for (int ct = 0; ct < T::NCT; ct++) O[qt][ct] = zero4;
        }
    }

    // S^T = K8 Q8^T for 8 key tiles x 2 query tiles (matrix cores).
    // Operand reads run two key tiles ahead of the products.
    __device__ __forceinline__ void slot_qk(const lds_u8* st) {
        const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 8; kt++) {
            v8i kop;
            if (D == 128 || g < 2) {
                kop = lds_operand(st, 16 * kt + col, D, T::KCH, g);
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++) kop[i] = 0;
            }
#pragma unroll
            for (int qt = 0; qt < 2; qt++)
                S[qt][kt] = MODE == REC_SAGE_I8 ? mfma_i8_128(kop, qop[qt]) : mfma_fp8(kop, qop[qt], zero4);
        }
        constexpr int MPT = MODE == REC_SAGE_I8 ? 4 : 2;  // products per key tile
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read: tiles 0, 1
#pragma unroll
        for (int kt = 0; kt < 8; kt++) {
            __builtin_amdgcn_sched_group_barrier(0x008, MPT, 0);  // MFMA: tile kt
            if (kt + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read: tile kt+2
        }
        // keep the softmax out of this region: mixed into the products, its
        // vector work would wait behind their operand reads (in-order issue)
        __builtin_amdgcn_sched_barrier(0);
    }

    // Running max and ExpCast-FP8 bytes (vector ALU).  A wave issues a
    // dependent vector instruction only every ~10 cycles but independent ones
    // every ~5, so the work is laid out as independent chains: four max3
    // chains (two per query tile), the two cross-lane reductions side by
    // side, and the byte conversions four dwords at a time.  The last, partial
    // block (keys past L) has its own copy so that no masking work leaks into
    // the full blocks.
    template <bool MASKED>
    __device__ __forceinline__ void softmax_max(float cb, int lim) {
        float mx[2];
        if (SAGE) {
            // largest scaled score: per key tile, its largest score times the
            // tile's coefficient (max3 + max + mul), then over the 8 tiles
#pragma unroll
            for (int qt = 0; qt < 2; qt++) {
                float x[8];
#pragma unroll
                for (int kt = 0; kt < 8; kt++) {
                    float mk;
                    if (!MASKED) {
                        mk = fmaxf(vmax3(S[qt][kt][0], S[qt][kt][1], S[qt][kt][2]), S[qt][kt][3]);
                    } else {
                        mk = -INFINITY;
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            if (key_ok(kt, i, lim)) mk = fmaxf(mk, S[qt][kt][i]);
                    }
                    // a tile with no valid key keeps -inf (coefficients are >= 0,
                    // and a zero coefficient only occurs with zero scores)
                    x[kt] = (MASKED && mk == -INFINITY) ? -INFINITY : __fmul_rn(mk, cf[qt][kt]);
                }
                mx[qt] = fmaxf(vmax3(vmax3(x[0], x[1], x[2]), x[3], x[4]), vmax3(x[5], x[6], x[7]));
            }
        } else if (!MASKED) {
            float ch[2][2];
#pragma unroll
            for (int qt = 0; qt < 2; qt++)
#pragma unroll
                for (int h = 0; h < 2; h++) ch[qt][h] = vmax3(S[qt][4 * h][0], S[qt][4 * h][1], S[qt][4 * h][2]);
            // the other 13 scores of each chain: S[4h][3], then kt = 4h+1 .. 4h+3
#pragma unroll
            for (int j = 0; j < 13; j += 2) {
#pragma unroll
                for (int qt = 0; qt < 2; qt++)
#pragma unroll
                    for (int h = 0; h < 2; h++) {
                        const int e0 = 3 + j, e1 = 4 + j;  // element index within the chain's 16
                        const float a0 = S[qt][4 * h + e0 / 4][e0 % 4];
                        if (e1 < 16)
                            ch[qt][h] = vmax3(ch[qt][h], a0, S[qt][4 * h + e1 / 4][e1 % 4]);
                        else
                            ch[qt][h] = fmaxf(ch[qt][h], a0);
                    }
            }
#pragma unroll
            for (int qt = 0; qt < 2; qt++) mx[qt] = fmaxf(ch[qt][0], ch[qt][1]);
        } else {
#pragma unroll
            for (int qt = 0; qt < 2; qt++) {
                mx[qt] = -INFINITY;
#pragma unroll
                for (int kt = 0; kt < 8; kt++)
#pragma unroll
                    for (int i = 0; i < 4; i++) mx[qt] = fmaxf(mx[qt], key_ok(kt, i, lim) ? S[qt][kt][i] : -INFINITY);
            }
        }
        if (FP4V) {
            lmx[0] = mx[0];
            lmx[1] = mx[1];
        }
        max_over_groups2(mx[0], mx[1]);
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
            // SAGE (ExpCast): the coefficients carry the factor 8, undone exactly
            const float t = SAGE ? (NAIVE ? mx[qt] : 0.125f * mx[qt]) : __fmul_rn(mx[qt], cb);
            const float mn = fmaxf(m[qt], t);
            // ExpCast: y = fma(S, 8 c_b, KB - 8 m'); exp-then-cast: z = fma(S, c_b, z_off - m')
            krow[qt] = NAIVE ? __fsub_rn(a.ZOFF, mn) : __fsub_rn(a.KB, 8.0f * mn);
            if (SKIP) {
                // exp(m~ - m) < lambda, in log2 units; +inf on the first
                // block.  A rejected row has t < m, so m' = m and alpha = 1,
                // and an infinite offset turns all its bytes into 0.
                reject[qt] = __fsub_rn(t, m[qt]) < a.skip_thr;
                if (reject[qt]) krow[qt] = -INFINITY;
            }
            alpha[qt] = __builtin_amdgcn_exp2f(m[qt] - mn);  // 2^(m - m'), 0 on the first block
            m[qt] = mn;
        }
    }

    template <bool MASKED>
    __device__ __forceinline__ void softmax_bytes(int kb, float c8, int lim) {
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
            if (NAIVE) {
                // the path ExpCast replaces: p = 2^z in fp32 (v_exp_f32), then
                // the hardware E4M3 conversion (round to nearest even), two
                // bytes per instruction; c8 holds c_b here
#pragma unroll
                for (int kt = 0; kt < 8; kt++) {
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qt][kt][i], SAGE ? cf[qt][kt] : c8, krow[qt]));
                        if (MASKED && !key_ok(kt, i, lim)) p[i] = 0.f;  // keys past L keep byte 0
                    }
                    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                    P[qt][kt] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
                }
            } else if (!MASKED) {
#pragma unroll
                for (int k4 = 0; k4 < 8; k4 += 4) {
                    float y[16];
#pragma unroll
                    for (int d = 0; d < 4; d++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            y[4 * d + i] = __builtin_fmaf(S[qt][k4 + d][i], SAGE ? cf[qt][k4 + d] : c8, krow[qt]);
                    cvt_bytes16(y, P[qt][k4], P[qt][k4 + 1], P[qt][k4 + 2], P[qt][k4 + 3]);
                }
            } else {
#pragma unroll
                for (int kt = 0; kt < 8; kt++) {
                    uint32_t pk = 0;
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (key_ok(kt, i, lim))  // keys past L keep byte 0
                            pk = expcast_byte_into(S[qt][kt][i], SAGE ? cf[qt][kt] : c8, krow[qt], i, pk);
                    P[qt][kt] = pk;
                }
            }
            if (DUMP && dump) {
                const int rl = w * QW + 16 * qt + col;
                if (q0 + 16 * qt + col < L) {
#pragma unroll
                    for (int kt = 0; kt < 8; kt++)
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const size_t o = (size_t)rl * Lp + kb * BLK + key_of(kt, i);
                            a.s_dump[o] = S[qt][kt][i];
                            a.p_dump[o] = (P[qt][kt] >> (8 * i)) & 0xFF;
                        }
                }
            }
        }
    }

    // 4-bit probabilities: p = 2^z in fp32 (v_exp_f32), then one power-of-two
    // scale for the lane's 32 values -- keys 32 g .. 32 g + 31 of the block,
    // one 32-key group and the lane's k-block of the scaled FP4 product -- by
    // the E8M0 rule on their maximum, and E2M1 codes (round to nearest even),
    // element 4 kt + i (key 32 g + 4 kt + i) in nibble (4 kt + i) mod 8 of
    // dword kt / 2.
    template <bool MASKED>
    __device__ __forceinline__ void softmax_bytes_fp4(int kb, float c, int lim) {
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
            float p[32];
#pragma unroll
            for (int kt = 0; kt < 8; kt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    p[4 * kt + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qt][kt][i], c, krow[qt]));
                    if (MASKED && !key_ok(kt, i, lim)) p[4 * kt + i] = 0.f;  // keys past L: code 0
                }
            // the group's largest probability from its largest score: the FMA
            // is monotone in S for c >= 0, and so is 2^z; a group with no
            // valid key has largest probability 0
            const float zg = lmx[qt] == -INFINITY ? -INFINITY : __builtin_fmaf(lmx[qt], c, krow[qt]);
            const int ex = e8m0_exp(__builtin_amdgcn_exp2f(zg));
            sp[qt] = ex + 127;
            const float sc = ldexpf(1.0f, max(ex, -126));
#pragma unroll
            for (int w4 = 0; w4 < 4; w4++) {
                const float (&y)[8] = *reinterpret_cast<const float(*)[8]>(&p[8 * w4]);
                P[qt][w4] = ex > -127 ? e2m1_pk8(y, sc) : 0u;  // a group below 2^-100: codes 0
                P[qt][4 + w4] = 0u;
            }
            if (DUMP && dump) {
                const int rl = w * QW + 16 * qt + col;
                if (q0 + 16 * qt + col < L) {
#pragma unroll
                    for (int kt = 0; kt < 8; kt++)
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const int e = 4 * kt + i;
                            const size_t o = (size_t)rl * Lp + kb * BLK + key_of(kt, i);
                            a.s_dump[o] = S[qt][kt][i];
                            a.p_dump[o] = (P[qt][e / 8] >> (4 * (e % 8))) & 0xF;
                        }
                }
            }
        }
    }

    // Returns true when every row of the wave rejects the block (Skip
    // Softmax; its bytes are then all 0): the caller skips P V.  (Branching
    // around the byte conversion as well costs more than it saves.)
    __device__ __forceinline__ bool slot_softmax(int kb, const lds_u8* st) {
        float cscale;
        if (SAGE) {
            // the block's eight 16-key group scales (wave 0's copy)
            const f32x4 k0 = *reinterpret_cast<const VC_LDS f32x4*>(st + T::KS_OFF);
            const f32x4 k1 = *reinterpret_cast<const VC_LDS f32x4*>(st + T::KS_OFF + 16);
#pragma unroll
            for (int qt = 0; qt < 2; qt++)
#pragma unroll
                for (int kt = 0; kt < 8; kt++) cf[qt][kt] = __fmul_rn(sqx[qt], kt < 4 ? k0[kt] : k1[kt - 4]);
            if (MODE == REC_SAGE_I8) {
                // whole-vector casts: a bit cast of one element of an
                // ext-vector reads the vector's first element instead
#pragma unroll
                for (int qt = 0; qt < 2; qt++)
#pragma unroll
                    for (int kt = 0; kt < 8; kt++)
                        S[qt][kt] = __builtin_convertvector(__builtin_bit_cast(v4i, S[qt][kt]), v4f);  // exact
            }
            cb = cscale = 0.0f;
        } else {
            const float ks = *reinterpret_cast<const VC_LDS float*>(st + T::KS_OFF);
            cb = __fmul_rn(__fmul_rn(sq, ks), a.C0);
            cscale = NAIVE ? cb : 8.0f * cb;
        }
        const int nvalid = L - kb * BLK;  // keys of this block that exist (>= 1)
        if (nvalid < BLK) {
            const int lim = nvalid - key_of(0, 0);
            softmax_max<true>(cb, lim);
            if (FP4V)
                softmax_bytes_fp4<true>(kb, cscale, lim);
            else
                softmax_bytes<true>(kb, cscale, lim);
        } else {
            softmax_max<false>(cb, 0);
            if (FP4V)
                softmax_bytes_fp4<false>(kb, cscale, 0);
            else
                softmax_bytes<false>(kb, cscale, 0);
        }
        return SKIP && !DUMP && __all(reject[0] && reject[1]);
    }

    // 4-bit P V: row sums (ones(16x128) P^T with the probability scale) and
    // V4^T P^T on the scaled FP4 matrix cores -- the V operand is 16 bytes of
    // E2M1 codes per lane (channel 16 ct + col, slots 32 g .. 32 g + 31) with
    // that (channel, group)'s E8M0 byte, the P operand the lane's codes with
    // its own; O += l_b mean_b + acc on the vector ALU.
    __device__ __forceinline__ void slot_pv_fp4(const lds_u8* st) {
        const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
        v8i ones;  // E2M1 1.0 in every element, scale 2^0
        int one4;
        asm volatile("v_mov_b32 %0, 0x22222222" : "=v"(one4));
#pragma unroll
        for (int i = 0; i < 4; i++) {
            ones[i] = one4;
            ones[4 + i] = 0;
        }
        v8i pv[2];
        float ell[2];
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
#pragma unroll
            for (int kt = 0; kt < 8; kt++) pv[qt][kt] = (int)P[qt][kt];
            const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pv[qt], zero4, 4, 4, 0, 127, 0,
                                                                            sp[qt]);
            ell[qt] = r[0];
        }
        const lds_u8* sV = st + T::K_TILE;
        const VC_LDS float* sS = reinterpret_cast<const VC_LDS float*>(st + T::SV_OFF);
        const lds_u8* sE = st + T::SV_OFF;  // E8M0 bytes [D][4]
#pragma unroll
        for (int ct = 0; ct < T::NCT; ct++) {
            const int r = 16 * ct + col;
            const u32x4 c4 = *reinterpret_cast<const VC_LDS u32x4*>(sV + r * (BLK / 2) +
                                                                   ((g ^ chunk_swizzle(r, 4)) << 4));
            v8i vop;
            vop[0] = c4[0]; vop[1] = c4[1]; vop[2] = c4[2]; vop[3] = c4[3];
            vop[4] = 0; vop[5] = 0; vop[6] = 0; vop[7] = 0;
            const int sv = sE[4 * r + g];
            const f32x4 mu = *reinterpret_cast<const VC_LDS f32x4*>(sS + D + 16 * ct + 4 * g);
#pragma unroll
            for (int qt = 0; qt < 2; qt++) {
                const v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vop, pv[qt], zero4, 4, 4, 0, sv, 0,
                                                                                  sp[qt]);
#pragma unroll
                for (int i = 0; i < 4; i++)
                    O[qt][ct][i] = __fadd_rn(__builtin_fmaf(ell[qt], mu[i], O[qt][ct][i]), acc[i]);
            }
        }
#pragma unroll
        for (int qt = 0; qt < 2; qt++) l[qt] = __builtin_fmaf(alpha[qt], l[qt], ell[qt]);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // DS read: tiles 0, 1 (operand, scale, mean)
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA: row sums
#pragma unroll
        for (int ct = 0; ct < T::NCT; ct++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA: tile ct
            if (ct + 2 < T::NCT) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            if (ct > 0) __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // VALU: tile ct-1
        }
    }

    __device__ __forceinline__ static v8i e4m3_ones() {
        int one4;
        asm volatile("v_mov_b32 %0, 0x38383838" : "=v"(one4));
        v8i r;
#pragma unroll
        for (int i = 0; i < 8; i++) r[i] = one4;
        return r;
    }

    // Row sums (ones(16x128) * P^T, exact), V8^T P^T on the matrix
    // cores, and O += s_v (.) acc + l_b mean_b on the vector ALU, one channel
    // tile behind the products.
    __device__ __forceinline__ void slot_pv(const lds_u8* st) {
        const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
        const v8i ones = ONES_RESIDENT ? ones8 : e4m3_ones();
        v8i pv[2];
        float ell[2];
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
#pragma unroll
            for (int kt = 0; kt < 8; kt++) pv[qt][kt] = (int)P[qt][kt];
            const v4f r = mfma_fp8(ones, pv[qt], zero4);
            ell[qt] = r[0];
        }
        const lds_u8* sV = st + T::K_TILE;
        const VC_LDS float* sS = reinterpret_cast<const VC_LDS float*>(st + T::SV_OFF);
#pragma unroll
        for (int ct = 0; ct < T::NCT; ct++) {
            const v8i vop = lds_operand(sV, 16 * ct + col, BLK, 8, g);
            if (SAGE) {
                // no block mean; the per-channel scale is applied at the end
#pragma unroll
                for (int qt = 0; qt < 2; qt++) {
                    const v4f acc = mfma_fp8(vop, pv[qt], zero4);
#pragma unroll
                    for (int i = 0; i < 4; i++) O[qt][ct][i] = __fadd_rn(O[qt][ct][i], acc[i]);
                }
                continue;
            }
            const f32x4 sv = *reinterpret_cast<const VC_LDS f32x4*>(sS + 16 * ct + 4 * g);
            const f32x4 mu = *reinterpret_cast<const VC_LDS f32x4*>(sS + D + 16 * ct + 4 * g);
#pragma unroll
            for (int qt = 0; qt < 2; qt++) {
                const v4f acc = mfma_fp8(vop, pv[qt], zero4);
#pragma unroll
                for (int i = 0; i < 4; i++)
                    O[qt][ct][i] = __builtin_fmaf(sv[i], acc[i], __builtin_fmaf(ell[qt], mu[i], O[qt][ct][i]));
            }
        }
#pragma unroll
        for (int qt = 0; qt < 2; qt++) l[qt] = __builtin_fmaf(alpha[qt], l[qt], ell[qt]);
        // operand reads two channel tiles ahead, epilogue one tile behind
        constexpr int RPT = SAGE ? 2 : 4;    // LDS reads per channel tile (operand, scale, mean)
        constexpr int VPT = SAGE ? 8 : 16;   // epilogue instructions per channel tile
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * RPT, 0);  // DS read: tiles 0, 1
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA: row sums
#pragma unroll
        for (int ct = 0; ct < T::NCT; ct++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA: tile ct
            if (ct + 2 < T::NCT) __builtin_amdgcn_sched_group_barrier(0x100, RPT, 0);
            if (ct > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPT, 0);  // VALU: tile ct-1
        }
    }

    // Block kb (stage `cur`): S^T on the matrix cores, softmax bytes on the
    // vector ALU, then P V and the epilogue.  The loading group (waves 0-3)
    // starts the copy of block kb + 2 into stage `ahead` (the stage of block
    // kb - 2) -- unconditionally: past the end it re-copies the last block
    // into a stage nobody reads again, so the copy count per block is fixed --
    // and at the end waits for its share of block kb + 1.
    //
    // Every wave passes one workgroup barrier per block; barrier n publishes
    // block n.  The loading group passes it at the end of its block, the
    // other group (LAG) right after its products S^T: that group thus runs
    // most of a block behind, its softmax (vector ALU) meets the loading
    // group's S^T products (matrix cores) on the shared SIMDs, and the two
    // groups never sit in the same phase.  The lagging group still reads
    // block kb (softmax, P V) until it reaches barrier kb + 2, so the ring
    // has four stages: block kb + 2 is copied, after barrier kb, into the
    // stage of block kb - 2, which both groups left before that barrier.
    template <bool LOADER, bool LAG, class LD>
    __device__ __forceinline__ void block(const LD& ld, int kb, const lds_u8* cur, lds_u8* ahead) {
        slot_qk(cur);
        if (LAG) block_barrier();
        if (LOADER) ld.issue(ahead, min(kb + 2, nb - 1));
        const bool rejected = slot_softmax(kb, cur);
        // rescale a query tile only when one of its rows raised its max
#pragma unroll
        for (int qt = 0; qt < 2; qt++)
            if (__any(alpha[qt] != 1.0f)) {
#pragma unroll
                for (int ct = 0; ct < T::NCT; ct++) O[qt][ct] *= alpha[qt];
            }
        if (__builtin_expect(!rejected, 1)) {
            if (FP4V)
                slot_pv_fp4(cur);
            else
                slot_pv(cur);
        }
        if (LOADER) {
            if (DUMP)
                wait_vmcnt<0>();
            else
                wait_vmcnt<LD::NLD>();
        }
        if (!LAG) block_barrier();
    }

    template <bool LOADER, bool LAG, class LD>
    __device__ __forceinline__ void run(const LD& ld, lds_u8* const (&st)[4]) {
        for (int kb = 0; kb < nb; kb += 4) {
            block<LOADER, LAG>(ld, kb, st[0], st[2]);
            if (kb + 1 < nb) block<LOADER, LAG>(ld, kb + 1, st[1], st[3]);
            if (kb + 2 < nb) block<LOADER, LAG>(ld, kb + 2, st[2], st[0]);
            if (kb + 3 < nb) block<LOADER, LAG>(ld, kb + 3, st[3], st[1]);
        }
    }

    // O / l in the original row order; lane (col, g) holds channels
    // 16 ct + 4 g + i (SAGE: O s_v / l with the per-channel V scale)
    template <bool OUT_BF16>
    __device__ __forceinline__ void store() {
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
            const int row = q0 + 16 * qt + col;
            if (row >= L) continue;
            const float il = 1.0f / l[qt];
            if (SAGE) {
#pragma unroll
                for (int ct = 0; ct < T::NCT; ct++) {
                    const f32x4 sv = *reinterpret_cast<const f32x4*>(a.v_scale + (size_t)bh * D + 16 * ct + 4 * g);
#pragma unroll
                    for (int i = 0; i < 4; i++) O[qt][ct][i] = __fmul_rn(O[qt][ct][i], sv[i]);
                }
            }
            if (OUT_BF16) {
                uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((size_t)bh * L + row) * D;
#pragma unroll
                for (int ct = 0; ct < T::NCT; ct++) {
                    uint32_t lo = pack_bf16x2(O[qt][ct][0] * il, O[qt][ct][1] * il);
                    uint32_t hi = pack_bf16x2(O[qt][ct][2] * il, O[qt][ct][3] * il);
                    *reinterpret_cast<uint2*>(o + 16 * ct + 4 * g) = make_uint2(lo, hi);
                }
            } else {
                float* o = reinterpret_cast<float*>(a.out) + ((size_t)bh * L + row) * D;
#pragma unroll
                for (int ct = 0; ct < T::NCT; ct++)
                    *reinterpret_cast<float4*>(o + 16 * ct + 4 * g) =
                        make_float4(O[qt][ct][0] * il, O[qt][ct][1] * il, O[qt][ct][2] * il, O[qt][ct][3] * il);
            }
        }
    }
};

// One workgroup: 8 waves, 256 queries of one head, the four-stage ring.
// WV is the wave (Fp8Wave or Fp8Wave32), LD its loader.
template <class WV, class LD, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64, 2) void attn_fp8_kernel(AttnArgs a) {
    using T = typename WV::T;
    __shared__ __attribute__((aligned(16))) uint8_t st0_[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1_[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2_[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st3_[T::STAGE];
    lds_u8* const st[4] = {(lds_u8*)st0_, (lds_u8*)st1_, (lds_u8*)st2_, (lds_u8*)st3_};
    const int nwg = a.BH * a.nqt;
    const int pid = xcd_remap(blockIdx.x, nwg);
    const int bh = pid / a.nqt, qtile = pid % a.nqt;
    // wave index as a scalar (uniform) value
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    WV s(a, bh, qtile, w, lane);
    const LD ld(a, bh, w, lane);
    const int nb = a.nb;

    // Blocks 0 and 1 (and 2, for the V part of a split wave) are in flight
    // before the loop; block 0 is published by the first barrier.  Every
    // wave drains its copies past the end before it exits.
    if (WV::SPLIT) {
        if (s.grp == 0) {
            ld.issue_k(st[0], 0);
            ld.issue_k(st[1], min(1, nb - 1));
            wait_vmcnt<LD::NLD_K>();
        } else {
            ld.issue_v(st[0], 0);
            ld.issue_v(st[1], min(1, nb - 1));
            ld.issue_v(st[2], min(2, nb - 1));
            wait_vmcnt<2 * LD::NLD_V>();
        }
    } else if (s.grp == 0) {
        ld.issue(st[0], 0);
        ld.issue(st[1], min(1, nb - 1));
        wait_vmcnt<LD::NLD>();
    }
    block_barrier();
    if (s.grp == 0)
        s.template run<true, false>(ld, st);
    else
        s.template run<false, true>(ld, st);
    wait_vmcnt<0>();
    s.template store<OUT_BF16>();
}

template <int D, bool OB, bool DUMP, bool SKIP, bool NAIVE, int MODE>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((attn_fp8_kernel<Fp8Wave<D, DUMP, SKIP, NAIVE, MODE>, Fp8Loader<D, MODE>, OB>),
                       dim3(a.BH * a.nqt), dim3(NW * 64), 0, st, a);
    return hipGetLastError();
}

}  // namespace

}  // namespace vc
