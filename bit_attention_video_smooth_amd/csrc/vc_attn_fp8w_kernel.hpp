// vc_attn_fp8w_kernel.hpp -- the V-Smooth recipe of the fused FP8 attention
// on 32x32x64 FP8 matrix-core products (v_mfma_f32_32x32x64_f8f6f4): one
// wave owns one 32-query tile.
//
// Method: as the 16x16 scaffold in vc_attn_fp8_kernel.hpp (agihunt summary,
// ExpCast-FP8 and V-Smooth bullets; MarkTechPost abstract, byte ~ 8 log2 v +
// 56 with beta = -0.35; online softmax notation of the TensorRT-LLM blog,
// "Sparse Attention with Skip Softmax").  The same workgroup, LDS ring, copy
// schedule and wave-group offset; only the wave's tiling differs.
//
// Why the larger product: a matrix-core instruction holds the vector issue
// of its SIMD for about 16 cycles whatever its size; a 32x32x64 FP8 product
// does twice the work of a 16x16x128 one in 64 cycles and leaves about 12
// vector instructions free beside it, against about 4 (measured), so a
// block takes half the product instructions, and at d = 64 the scores are
// one full k = 64 step instead of a half-empty 128-deep one.  (On the chip
// both forms run at the same speed at d = 128: under this kernel the part
// sits at its power limit, and the time follows the energy of the work --
// products, LDS operand reads, copies -- more than its issue schedule.)
//
// Lane layout of a 32x32x64 product: A row m = lane % 32 and B column
// n = lane % 32 take k bytes 32 (lane / 32) .. + 31 of the k-step; the 16
// results of lane (n, h = lane / 32) are rows 8 j + 4 h + i (element 4 j + i)
// of column n.  So with S^T = K8 Q8^T each lane holds 64 scores of query n:
// the row max needs one cross-lane swap.  The K rows are placed in LDS
// (Fp8Loader<D, REC_VC, true>) so that lane half h's scores of key tiles
// 2 s and 2 s + 1 are exactly the keys of V slots 64 s + 32 h .. + 31, i.e.
// its ExpCast bytes are its A operand (row = its query) of k-step s of
// O = P8 V8, in the slot order the preparation writes the V codes in
// (vkey_of_slot).
#pragma once

#include "vc_attn_fp8_kernel.hpp"

namespace vc {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mfma_fp8_32(const v8i& a, const v8i& b, const v16f& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// A operand of the row sums on a 16x16x128 product whose B operand is the
// 32x32x64 P operand of one k-step.  In the 16x16x128 layout B column
// c = lane % 16 takes k bytes 32 g .. + 31 from lane c + 16 g; the P lanes
// hold query lane % 32, so lane groups g = 0, 2 carry query c and groups
// 1, 3 query c + 16.  With A row r = 1.0 (E4M3) on k-groups g of parity
// (r / 4) % 2 and 0 elsewhere, result rows 4 g .. 4 g + 3 -- the four
// results of lane c + 16 g -- are that lane's own query's sum.
__device__ __forceinline__ v8i rowsum_op(int lane) {
    const int g = lane >> 4, m = lane & 15;
    int one4;
    asm volatile("v_mov_b32 %0, 0x38383838" : "=v"(one4));
    const int x = ((g & 1) == ((m >> 2) & 1)) ? one4 : 0;
    v8i r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = x;
    return r;
}

typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));

// hi/lo bf16 split of eight floats (x ~ hi + lo to about 2^-16 relative):
// hi rounds x to nearest even, lo rounds the exact remainder x - hi
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], v8bf16& hi, v8bf16& lo) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
        hi[i] = (__bf16)x[i];
        lo[i] = (__bf16)(x[i] - (float)hi[i]);
    }
}

template <int D, bool DUMP, bool SKIP, bool NAIVE, int NWV>
struct Fp8Wave32 {
    using T = Fp8Tile<D>;
    static constexpr int KS = D / 64;   // k-steps of S^T (64 channels each)
    static constexpr int NCT = D / 32;  // 32-channel output tiles
    static constexpr int NHIST = 32;    // blocks of means kept in LDS (a ring)
    const AttnArgs& a;
    int bh, w, lane, n, h, grp, q0, L, nb;
    size_t Lp;
    bool dump;
    float sq;
    v8i qop[KS];
    float O[NCT][16];
    float m, l;
    // Deferred mean term: W[i] is this lane's query's row sum l_b of block
    // b = 16 c + 8 h + i of the current 16-block chunk c (h: lane half),
    // kept at the current max like O; every 16 blocks sum_b W_b mean_b is
    // added to O on the matrix cores (flush_means).
    float W[8];
    // per-block values carried between the stages of a block
    v16f S[4];
    uint32_t P[2][8];
    float alpha, krow, cb;
    bool reject;  // Skip Softmax: this lane's row rejects the block
    v8i rs_op;    // A operand of the row sums (rowsum_op)
    const VC_LDS float* hist;  // [NHIST][D] means of recent blocks, slot kb % NHIST
    // Copies are split between the groups: waves 0-3 copy the K part of
    // block kb + 2 during block kb, waves 4-7 the V part of block kb + 3
    // (see block()).
    static constexpr bool SPLIT = true;

    // In-block key of score (t, e = 4 j + i) of lane half h:
    // 64 (t % 2) + 16 j + 8 (t / 2) + 4 h + i.
    __device__ __forceinline__ static constexpr int key_off(int t, int e) {
        return 64 * (t % 2) + 16 * (e / 4) + 8 * (t / 2) + e % 4;
    }
    __device__ __forceinline__ int key_of(int t, int e) const { return key_off(t, e) + 4 * h; }

    __device__ __forceinline__ Fp8Wave32(const AttnArgs& args, int bh_, int qtile, int w_, int lane_,
                                         const VC_LDS float* hist_)
        : a(args), bh(bh_), w(w_), lane(lane_), hist(hist_) {
        n = lane & 31;
        h = lane >> 5;
        grp = w >> 2;
        q0 = qtile * (NWV * QW) + w * QW;
        L = a.L;
        nb = a.nb;
        Lp = (size_t)nb * BLK;
        dump = DUMP && bh == a.dump_bh && qtile == a.dump_qt;
        // Q8 operands (B of S^T): lane (n, h) holds bytes 64 s + 32 h .. + 31
        // of query q0 + n for k-step s
        const int row = q0 + n;
#pragma unroll
        for (int s = 0; s < KS; s++) {
            uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
            if (row < L) {
                const uint8_t* src = a.q8 + ((size_t)bh * Lp + row) * D + 64 * s + 32 * h;
                x = *reinterpret_cast<const uint4*>(src);
                y = *reinterpret_cast<const uint4*>(src + 16);
            }
            qop[s][0] = x.x; qop[s][1] = x.y; qop[s][2] = x.z; qop[s][3] = x.w;
            qop[s][4] = y.x; qop[s][5] = y.y; qop[s][6] = y.z; qop[s][7] = y.w;
        }
        // the wave's 32 queries lie in one 128-token block
        sq = a.q_scale[(size_t)bh * nb + min(q0 / BLK, nb - 1)];
        rs_op = rowsum_op(lane);
        // the Q operands and scale are in registers before any block copy is
        // issued, so no later wait on them can drain the copy pipeline
        __builtin_amdgcn_s_waitcnt(0);
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
            for (int e = 0; e < 16; e++) O[ct][e] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) W[i] = 0.f;
    }

    // S^T = K8 Q8^T: 4 key tiles of 32 x KS k-steps (matrix cores), the
    // second k-step accumulating into the first; operand reads two products
    // ahead.
    __device__ __forceinline__ void slot_qk(const lds_u8* st) {
        v16f z;
#pragma unroll
        for (int e = 0; e < 16; e++) z[e] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; s++)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const v8i kop = lds_operand(st, 32 * t + n, D, T::KCH, 2 * s + h);
                S[t] = mfma_fp8_32(kop, qop[s], s == 0 ? z : S[t]);
            }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read: products 0, 1
#pragma unroll
        for (int p = 0; p < 4 * KS; p++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA: product p
            if (p + 2 < 4 * KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read: product p+2
        }
        // keep the softmax out of this region: mixed into the products, its
        // vector work would wait behind their operand reads (in-order issue)
        __builtin_amdgcn_sched_barrier(0);
    }

    // Running max (four max3 chains, one per key tile, then one cross-lane
    // swap) and the ExpCast-FP8 offset.
    __device__ __forceinline__ void softmax_max() {
        float ch[4];
#pragma unroll
        for (int t = 0; t < 4; t++) ch[t] = vmax3(S[t][0], S[t][1], S[t][2]);
#pragma unroll
        for (int e = 3; e < 15; e += 2)
#pragma unroll
            for (int t = 0; t < 4; t++) ch[t] = vmax3(ch[t], S[t][e], S[t][e + 1]);
#pragma unroll
        for (int t = 0; t < 4; t++) ch[t] = fmaxf(ch[t], S[t][15]);
        float mx = fmaxf(vmax3(ch[0], ch[1], ch[2]), ch[3]);
        // the other half of the row: lane n + 32 h <-> n + 32 (1 - h)
        const auto px = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(px[0]), __uint_as_float(px[1]));
        const float t = __fmul_rn(mx, cb);
        const float mn = fmaxf(m, t);
        // ExpCast: y = fma(S, 8 c_b, KB - 8 m'); exp-then-cast: z = fma(S, c_b, z_off - m')
        krow = NAIVE ? __fsub_rn(a.ZOFF, mn) : __fsub_rn(a.KB, 8.0f * mn);
        if (SKIP) {
            // exp(m~ - m) < lambda, in log2 units; +inf on the first block.  A
            // rejected row has t < m, so m' = m and alpha = 1, and an infinite
            // offset turns all its bytes into 0.
            reject = __fsub_rn(t, m) < a.skip_thr;
            if (reject) krow = -INFINITY;
        }
        alpha = __builtin_amdgcn_exp2f(m - mn);  // 2^(m - m'), 0 on the first block
        m = mn;
    }

    // Bytes of key tile t = 2 s + u go to dwords 4 u .. 4 u + 3 of P[s]:
    // element 4 j + i of the tile is byte i of dword 4 u + j, i.e. byte
    // 16 u + 4 j + i of the lane's 32-byte B operand of k-step s.
    __device__ __forceinline__ void softmax_bytes(float c8) {
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const int s = t / 2, u = t % 2;
            if (NAIVE) {
                // the path ExpCast replaces: p = 2^z in fp32, then the
                // hardware E4M3 conversion (round to nearest even)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[t][4 * j + i], c8, krow));
                    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                    P[s][4 * u + j] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
                }
            } else {
                float y[16];
#pragma unroll
                for (int e = 0; e < 16; e++) y[e] = __builtin_fmaf(S[t][e], c8, krow);
                cvt_bytes16(y, P[s][4 * u], P[s][4 * u + 1], P[s][4 * u + 2], P[s][4 * u + 3]);
            }
        }
    }

    // The last block of a head may be partial (keys at and past nvalid do
    // not exist).  Before the max: those keys' scores become -inf, so the
    // shared max code ignores them.  After the bytes: their bytes are cleared
    // with per-dword masks (dword (t, j) holds keys base .. base + 3 of the
    // lane, base = key_of(t, 4 j)), arithmetic only -- no per-score compare
    // results stay live between the two steps.
    __device__ __forceinline__ void mask_scores(int lim) {
        // S + (+0 or -inf): the sign of lim - key - 1 selects the addend
        // (integer ops only; a compare per score would hold 64 lane masks)
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int d = lim - 1 - key_off(t, e);
                S[t][e] += __int_as_float((d >> 31) & (int)0xFF800000u);
            }
    }
    __device__ __forceinline__ void mask_bytes(int lim) {
#pragma unroll
        for (int t = 0; t < 4; t++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                // valid bytes of the dword: clamp(lim - base, 0, 4); the mask
                // is the high word of 0xFFFFFFFF << (8 * count)
                const int nv = min(max(lim - key_off(t, 4 * j), 0), 4);
                const uint32_t mk = (uint32_t)((0xFFFFFFFFull << (8 * nv)) >> 32);
                P[t / 2][4 * (t % 2) + j] &= mk;
            }
    }

    // Per-row values in the output layout.  The softmax holds one value per
    // query in lane n (and n + 32); the output tiles hold rows 8 j + 4 h + i
    // in lane half h.  One LDS round trip per wave (its own 32 floats; a
    // wave's LDS accesses complete in order, so the reads see the write).
    __device__ __forceinline__ void to_rows(float x, float (&out)[16]) const {
        __shared__ float xb[NWV * 32];
        VC_LDS float* b = (VC_LDS float*)xb + w * 32;
        b[n] = x;  // lanes n and n + 32 store the same value
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const f32x4 v = *reinterpret_cast<const VC_LDS f32x4*>(b + 8 * j + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; i++) out[4 * j + i] = v[i];
        }
    }

    // Softmax of block kb (stage `cur`): the running max, the rescale of O
    // and of the pending row sums when a row's max rose, and the bytes.
    // Returns true when every row of the wave rejects the block (Skip
    // Softmax; the bytes are then not formed and P V is skipped).
    __device__ __forceinline__ bool slot_softmax(int kb, const lds_u8* cur) {
        const float ks = *reinterpret_cast<const VC_LDS float*>(cur + T::KS_OFF);
        cb = __fmul_rn(__fmul_rn(sq, ks), a.C0);
        const float cscale = NAIVE ? cb : 8.0f * cb;
        const int nvalid = L - kb * BLK;  // keys of this block that exist (>= 1)
        const int lim = nvalid - 4 * h;
        const bool dumping = DUMP && dump && q0 + n < L;
        const size_t rb = (size_t)(w * QW + n) * Lp + kb * BLK;
        if (dumping) {
#pragma unroll
            for (int t = 0; t < 4; t++)
#pragma unroll
                for (int e = 0; e < 16; e++) a.s_dump[rb + key_of(t, e)] = S[t][e];
        }
        const bool partial = nvalid < BLK;
        if (partial) mask_scores(lim);
        softmax_max();
        // Skip Softmax: when every row of the wave rejects the block its
        // bytes would all be 0 and nothing reads them (P V is skipped too)
        const bool rejected = SKIP && !DUMP && __all(reject);
        if (__builtin_expect(!rejected, 1)) {
            softmax_bytes(cscale);
            if (partial) mask_bytes(lim);
        }
        if (dumping) {
#pragma unroll
            for (int t = 0; t < 4; t++)
#pragma unroll
                for (int e = 0; e < 16; e++)
                    a.p_dump[rb + key_of(t, e)] = (P[t / 2][4 * (t % 2) + e / 4] >> (8 * (e % 4))) & 0xFF;
        }
        // rescale only when one of the wave's rows raised its max
        if (__any(alpha != 1.0f)) {
            float ar[16];
            to_rows(alpha, ar);
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                for (int e = 0; e < 16; e++) O[ct][e] *= ar[e];
#pragma unroll
            for (int i = 0; i < 8; i++) W[i] *= alpha;
        }
        return rejected;
    }

    // Row sum and O += s_v (.) P V of block kb on the matrix cores.  O = P8
    // V8 with P as the A operand (lane (n, h): query n, slots 64 s + 32 h ..
    // + 31 of k-step s, the bytes of the softmax) and V as the B operand
    // (channel 32 ct + n, the same slots), so lane (n, h) holds rows
    // 8 j + 4 h + i of channel 32 ct + n: one V scale per lane and channel
    // tile, O = fma(s_v, acc, O).  The row sum l_b of the lane's query comes
    // from rowsum_op times P^T (16x16x128); it updates l and goes into W for
    // the deferred mean term.  `mid` runs after the first channel pair.
    template <class MID>
    __device__ __forceinline__ void slot_pv(int kb, const lds_u8* cur, MID&& mid) {
        v16f z;
#pragma unroll
        for (int e = 0; e < 16; e++) z[e] = 0.f;
        const v4f z4 = {0.f, 0.f, 0.f, 0.f};
        v8i pv[2];
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
            for (int dw = 0; dw < 8; dw++) pv[s][dw] = (int)P[s][dw];
        const lds_u8* sV = cur + T::K_TILE;
        // the stage's V scales at this lane's channel n (one register, so
        // that every read takes its tile offset as an immediate)
        uint32_t sa = lds_addr(cur + T::SV_OFF) + 4 * n;
        asm volatile("" : "+v"(sa));
        const VC_LDS float* sSn = reinterpret_cast<const VC_LDS float*>((uintptr_t)sa);
        float svc[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) svc[ct] = sSn[32 * ct];
        v4f r = mfma_fp8(rs_op, pv[0], z4);
        r = mfma_fp8(rs_op, pv[1], r);
#pragma unroll
        for (int cp = 0; cp < NCT; cp += 2) {
            v16f acc[2];
#pragma unroll
            for (int c = 0; c < 2; c++) acc[c] = mfma_fp8_32(pv[0], lds_operand(sV, 32 * (cp + c) + n, BLK, 8, h), z);
#pragma unroll
            for (int c = 0; c < 2; c++)
                acc[c] = mfma_fp8_32(pv[1], lds_operand(sV, 32 * (cp + c) + n, BLK, 8, 2 + h), acc[c]);
#pragma unroll
            for (int c = 0; c < 2; c++)
#pragma unroll
                for (int e = 0; e < 16; e++) O[cp + c][e] = __builtin_fmaf(svc[cp + c], acc[c][e], O[cp + c][e]);
            if (cp == 0) mid();
        }
        const float ell = r[0];
        l = __builtin_fmaf(alpha, l, ell);
        // W slot of block kb: index kb % 8 in lane half (kb / 8) % 2; the
        // block loop is unrolled by four, so kb % 4 is a constant here
        const bool mine = h == ((kb >> 3) & 1);
        const int i = kb & 3;
        if ((kb >> 2) & 1)
            W[i + 4] = mine ? ell : W[i + 4];
        else
            W[i] = mine ? ell : W[i];
    }

    // O += sum_b W_b mean_b over the 16 blocks of the chunk ending at block
    // kb, on bf16 32x32x16 products (k = the chunk's blocks): A = W (row =
    // query, lane half h holding blocks 8 h .. 8 h + 7), B = the means of
    // channel 32 ct + n from the LDS history, each split into bf16 high and
    // low parts (hi hi + hi lo + lo hi, accumulated in fp32).  Blocks past
    // the head have W = 0 and history slots holding zeros or real means.
    __device__ __forceinline__ void flush_means(int kb) {
        const int b0 = (kb & ~15) + 8 * h;
        v8bf16 ahi, alo;
        split_bf16x8(W, ahi, alo);
        v16f z;
#pragma unroll
        for (int e = 0; e < 16; e++) z[e] = 0.f;
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) {
            float mu[8];
#pragma unroll
            for (int i = 0; i < 8; i++) mu[i] = hist[((b0 + i) % NHIST) * D + 32 * ct + n];
            v8bf16 bhi, blo;
            split_bf16x8(mu, bhi, blo);
            v16f t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bhi, z, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, blo, t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bhi, t, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 16; e++) O[ct][e] += t[e];
        }
#pragma unroll
        for (int i = 0; i < 8; i++) W[i] = 0.f;
    }

    // Block kb (stage `cur`).  Every wave passes one workgroup barrier per
    // block; barrier n publishes block n.  The first group (waves 0-3) passes
    // it at the end of its block, the second group (LAG) right after its
    // S^T products, so the second group runs most of a block behind and one
    // group's softmax meets the other's products.  Copies into the ring are
    // split between the groups so that neither issues all of them at once
    // (they share the CU's load path):
    //  * group 0, during block kb, copies the K part (K8 tile, K scales) of
    //    block kb + 2 into stage (kb + 2) % 4 and, before its barrier kb + 1,
    //    waits for its part of block kb + 1;
    //  * group 1, after its barrier kb + 1, copies the V part (V8 tile, V
    //    scales, and the means into history slot (kb + 3) % 32) of block
    //    kb + 3 into stage (kb + 3) % 4 and, before that barrier, waits for
    //    its part of block kb + 1.
    // Each group issues its copies in three installments.  Stage (kb + 2) % 4
    // held block kb - 2, which group 0 left at barrier kb - 1 and group 1 at
    // barrier kb; stage (kb + 3) % 4 held block kb - 1, which group 1 left at
    // barrier kb + 1; history slot (kb + 3) % 32 held block kb - 29, flushed
    // by both groups long before.  Past the end the last block is copied
    // again into a stage nobody reads, so the copy count per block, and with
    // it every wait count, is fixed.
    template <bool LOADER, bool LAG, class LD>
    __device__ __forceinline__ void block(const LD& ld, int kb, const lds_u8* cur, lds_u8* ahead2,
                                          lds_u8* ahead3) {
        constexpr int C = LD::T::LPT;  // K (or V) tile copies per wave
        const int kc = min(kb + 2, nb - 1), vc = min(kb + 3, nb - 1);
        slot_qk(cur);
        if (LAG) {
            if (DUMP)
                wait_vmcnt<0>();
            else
                wait_vmcnt<LD::NLD_V>();
            block_barrier();
            ld.template issue_v_part<0, C / 2, false>(ahead3, vc);
        }
        if (LOADER) ld.template issue_k_part<0, C / 2, false>(ahead2, kc);
        const bool rejected = slot_softmax(kb, cur);
        if (LAG) ld.template issue_v_part<C / 2, C / 2 + 1, false>(ahead3, vc);
        if (LOADER) ld.template issue_k_part<C / 2, C / 2 + 1, false>(ahead2, kc);
        if (SKIP) {
            // one code path for the last copies: a branch around them doubles
            // the loader code and the registers it holds
            if (LAG) ld.template issue_v_part<C / 2 + 1, C, true>(ahead3, vc);
            if (LOADER) ld.template issue_k_part<C / 2 + 1, C, true>(ahead2, kc);
            if (__builtin_expect(!rejected, 1)) slot_pv(kb, cur, [] {});
        } else {
            slot_pv(kb, cur, [&]() {
                if (LAG) ld.template issue_v_part<C / 2 + 1, C, true>(ahead3, vc);
                if (LOADER) ld.template issue_k_part<C / 2 + 1, C, true>(ahead2, kc);
            });
        }
        if ((kb & 15) == 15 || kb == nb - 1) flush_means(kb);
        if (!LAG) {
            // the K loaders wait for their part of block kb + 1; a third
            // group (waves 8-11), which copies nothing, passes the barrier at
            // the same point of its block
            if (LOADER) {
                if (DUMP)
                    wait_vmcnt<0>();
                else
                    wait_vmcnt<LD::NLD_K>();
            }
            block_barrier();
        }
    }

    template <bool LOADER, bool LAG, class LD>
    __device__ __forceinline__ void run(const LD& ld, lds_u8* const (&st)[4]) {
        for (int kb = 0; kb < nb; kb += 4) {
            block<LOADER, LAG>(ld, kb, st[0], st[2], st[3]);
            if (kb + 1 < nb) block<LOADER, LAG>(ld, kb + 1, st[1], st[3], st[0]);
            if (kb + 2 < nb) block<LOADER, LAG>(ld, kb + 2, st[2], st[0], st[1]);
            if (kb + 3 < nb) block<LOADER, LAG>(ld, kb + 3, st[3], st[1], st[2]);
        }
    }

    // O / l in the original row order: lane (n, h) writes channel
    // 32 ct + n of rows q0 + 8 j + 4 h + i.
    template <bool OUT_BF16>
    __device__ __forceinline__ void store() {
        float lr[16];
        to_rows(l, lr);
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int row = q0 + 8 * (e / 4) + 4 * h + e % 4;
            if (row >= L) continue;
            const float il = 1.0f / lr[e];
            if (OUT_BF16) {
                __bf16* o = reinterpret_cast<__bf16*>(a.out) + ((size_t)bh * L + row) * D + n;
#pragma unroll
                for (int ct = 0; ct < NCT; ct++) o[32 * ct] = (__bf16)(O[ct][e] * il);
            } else {
                float* o = reinterpret_cast<float*>(a.out) + ((size_t)bh * L + row) * D + n;
#pragma unroll
                for (int ct = 0; ct < NCT; ct++) o[32 * ct] = O[ct][e] * il;
            }
        }
    }
};

// One workgroup: NWV waves (Fp8Wave32), 32 NWV queries of one head, the
// four-stage ring and the history of block means.  NWV = 8: two groups of
// four waves, one per SIMD each (the K loaders and the lagging V loaders).
// NWV = 12 (d = 64, where registers allow three waves per SIMD): a third
// group that copies nothing and keeps the first group's schedule; every
// wave passes one barrier per block either way, and the third group leaves
// each stage no later than the first, so the ring's reuse rules hold as
// they are.  A wave's arithmetic does not depend on NWV.
template <int D, bool OUT_BF16, bool DUMP, bool SKIP, bool NAIVE, int NWV>
__global__ __launch_bounds__(NWV * 64, NWV / 4) void attn_fp8w_kernel(AttnArgs a) {
    using WV = Fp8Wave32<D, DUMP, SKIP, NAIVE, NWV>;
    using LD = Fp8Loader<D, REC_VC, true>;
    using T = Fp8Tile<D>;
    __shared__ __attribute__((aligned(16))) uint8_t st0_[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1_[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2_[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st3_[T::STAGE];
    __shared__ __attribute__((aligned(16))) float hist_[WV::NHIST * D];
    lds_u8* const st[4] = {(lds_u8*)st0_, (lds_u8*)st1_, (lds_u8*)st2_, (lds_u8*)st3_};
    const int nwg = a.BH * a.nqt;
    const int pid = xcd_remap(blockIdx.x, nwg);
    const int bh = pid / a.nqt, qtile = pid % a.nqt;
    // wave index as a scalar (uniform) value
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // history slots not yet copied hold zeros (their W is zero too)
    for (int i = threadIdx.x; i < WV::NHIST * D; i += NWV * 64) hist_[i] = 0.f;
    WV s(a, bh, qtile, w, lane, (const VC_LDS float*)hist_);
    const LD ld(a, bh, w, lane, (VC_LDS float*)hist_);
    const int nb = a.nb;
    // blocks 0 and 1 (and 2, V part) in flight before the loop; block 0 is
    // published by the first barrier (which also orders the zeroing above
    // before every copy into the history)
    __syncthreads();
    if (s.grp == 0) {
        ld.issue_k(st[0], 0);
        ld.issue_k(st[1], min(1, nb - 1));
        wait_vmcnt<LD::NLD_K>();
    } else if (s.grp == 1) {
        ld.issue_v(st[0], 0);
        ld.issue_v(st[1], min(1, nb - 1));
        ld.issue_v(st[2], min(2, nb - 1));
        wait_vmcnt<2 * LD::NLD_V>();
    }
    block_barrier();
    if (s.grp == 0)
        s.template run<true, false>(ld, st);
    else if (s.grp == 1)
        s.template run<false, true>(ld, st);
    else
        s.template run<false, false>(ld, st);
    wait_vmcnt<0>();
    s.template store<OUT_BF16>();
}

template <int D, bool OB, bool DUMP, bool SKIP, bool NAIVE, int NWV>
hipError_t launch_w32_n(const AttnArgs& a, hipStream_t st) {
    AttnArgs b = a;
    b.nqt = (a.L + NWV * QW - 1) / (NWV * QW);
    hipLaunchKernelGGL((attn_fp8w_kernel<D, OB, DUMP, SKIP, NAIVE, NWV>), dim3(b.BH * b.nqt), dim3(NWV * 64), 0, st,
                       b);
    return hipGetLastError();
}

// d = 64 runs 12-wave workgroups of 384 queries when the grid fills the chip
// several times over (three waves per SIMD issue the vector work of the
// softmax faster; a few workgroups alone are quicker at 8 waves), except with
// the score dump (which addresses 256-query tiles, as the ABI defines them)
// and with Skip Softmax (whose rejection state does not fit the 168
// registers of three waves per SIMD without spilling inside the block loop)
template <int D, bool OB, bool DUMP, bool SKIP, bool NAIVE>
hipError_t launch_w32(const AttnArgs& a, hipStream_t st) {
    if constexpr (D == 64 && !DUMP && !SKIP) {
        if ((int64_t)a.BH * a.nqt >= 1024) return launch_w32_n<D, OB, DUMP, SKIP, NAIVE, 12>(a, st);
    }
    return launch_w32_n<D, OB, DUMP, SKIP, NAIVE, 8>(a, st);
}

}  // namespace

}  // namespace vc
