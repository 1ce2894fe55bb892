// vc_internal.hpp -- argument bundles between the C ABI layer and the kernel
// launchers (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vc {

struct PrepareArgs {
    int B, H, L, d, nb;
    int smooth_k, v_mode;
    int v_format;         // 0 E4M3 residual, fp32 scales; 1 E2M1 residual, E8M0 scales per 32-key group
    const void *q, *k, *v;
    const int32_t* perm;  // [B,H,L]
    uint8_t *q8, *k8, *v8;
    float *q_scale, *k_scale, *v_scale, *v_mean;
    double* kpartial;  // workspace [B*H, nsplit, d]
    float* kbar;       // workspace [B*H, d]
};

// SAGE-style quantisation (sequence order): q8/k8 [BH, Lp, d] INT8 or E4M3,
// v8 [BH, nb, d, 128] E4M3 in the P V slot order, q_scale [BH, Lp],
// k_scale [BH, Lp/16], v_scale [BH, d]
struct SageArgs {
    int B, H, L, d, nb;
    int qk_int8, smooth_k;
    const void *q, *k, *v;
    uint8_t *q8, *k8, *v8;
    float *q_scale, *k_scale, *v_scale;
    double* kpartial;  // workspace [B*H, nsplit, d]
    float* kbar;       // workspace [B*H, d]
    float* vpart;      // workspace [B*H, nvchunk, d] per-chunk channel amax
    float* vinv;       // workspace [B*H, d] 448 / channel amax
    int nvchunk;
};

struct KmeansArgs {
    int B, H, L, d, k, iters;
    uint64_t seed;
    const void* v;         // bf16 [B,H,L,d]
    int32_t* perm;         // out [B,H,L]
    double* obj;           // out [B,H] or null
    const float* cent_in;  // [B,H,k,d] initial centroids, or null (seeded init)
    float* cent_out;       // [B,H,k,d] final centroids, or null
    // workspace
    float* cent;           // [BH, kpad, d] fp32 centroids
    uint16_t* cent_hi;     // [BH, kpad, d] bf16 high part
    uint16_t* cent_lo;     // [BH, kpad, d] bf16 low part
    float* cnorm;          // [BH, kpad]
    int32_t* assign;       // [BH, L]
    int32_t* counts;       // [BH, k]
    int32_t* offsets;      // [BH, k]
    int32_t* chunk_cnt;    // [BH, nchunk, k]
    double* obj_part;      // [BH, nchunkJ]
    int kpad, nchunk;
};

struct AttnArgs {
    const uint8_t *q8, *k8, *v8;
    const float *q_scale, *k_scale, *v_scale, *v_mean;
    void* out;
    int L, nb, BH, nqt;
    float C0, KB;
    float skip_thr;  // fp32(log2(lambda)) of Skip Softmax; -infinity: off
    float ZOFF;      // z_off as fp32 (exp-then-cast bytes)
    int prob_cast;   // 0 ExpCast-FP8, 1 exp-then-cast
    int dump_bh, dump_qt;
    float* s_dump;
    uint8_t* p_dump;
};

struct AttnBf16Args {
    const uint16_t *q, *k, *v;
    void* out;
    int L, nkb, BH, nqt;
    float C0;
};

// Host-side sizes and workspace layout (vc_host.hip, no device code).
constexpr int KMEANS_KT = 64;       // centroids per LDS tile of the k-means assign kernel
constexpr int KMEANS_CHUNK = 1024;  // tokens per chunk of the k-means counting sort
int k_mean_splits(int BH, int L);   // partial sums per head of the K column mean
size_t kmeans_workspace_bytes(int B, int H, int L, int d, int k);
void kmeans_carve(KmeansArgs& a, void* ws);

// copies perm_in -> perm and, if obj is non-null, fills obj[0..nobj) with NaN
hipError_t launch_copy_perm(const int32_t* src, int32_t* dst, size_t n, double* obj, size_t nobj,
                            hipStream_t st);
hipError_t launch_prepare_quant(const PrepareArgs& a, hipStream_t st);
// per-channel K mean (kbar = 0 when smooth is 0); kpartial [BH, k_mean_splits, d]
hipError_t launch_k_mean(const void* k, double* kpartial, float* kbar, int BH, int L, int d, int smooth,
                         hipStream_t st);
constexpr int SAGE_VCHUNK = 1024;  // tokens per partial channel amax
hipError_t launch_sage_prepare(const SageArgs& a, hipStream_t st);
hipError_t launch_kmeans(const KmeansArgs& a, hipStream_t st);
hipError_t launch_attn_fp8(const AttnArgs& a, int d, int out_bf16, bool dump, hipStream_t st);
// 4-bit V-Smooth: v8 [BH, nb, d, 64] E2M1 codes, v_scale read as [BH, nb, d, 4] E8M0 bytes
hipError_t launch_attn_fp4v(const AttnArgs& a, int d, int out_bf16, bool dump, hipStream_t st);
// SAGE recipe: q_scale [BH, Lp], k_scale [BH, Lp/16], v_scale [BH, d]; v_mean unused
hipError_t launch_attn_sage(const AttnArgs& a, int d, int out_bf16, bool dump, bool qk_int8, hipStream_t st);
hipError_t launch_attn_bf16(const AttnBf16Args& a, int d, int out_bf16, hipStream_t st);
hipError_t launch_debug_expcast(const float* S, const float* c8, const float* krow, int64_t n,
                                uint8_t* out, hipStream_t st);
hipError_t launch_debug_e4m3(const float* x, int64_t n, uint8_t* out, hipStream_t st);
hipError_t launch_debug_mfma_fp8(const uint8_t* a, const uint8_t* b, float* c, int n,
                                 hipStream_t st);
hipError_t launch_debug_mfma_rate(int blocks, int iters, float* out, hipStream_t st);

constexpr int ATTN_BM = 256;  // queries per workgroup of the attention kernels

}  // namespace vc
