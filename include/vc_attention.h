/*
 * vc_attention.h -- C ABI of the VC-Attention library for AMD Instinct
 * MI355X (gfx950): V-Smooth preprocessing and fused low-bit flash attention
 * with ExpCast-FP8, plus a BF16 flash-attention kernel on the same scaffold.
 *
 * The method follows the VC-Attention pages:
 *   - agihunt summary "VC-Attention: Training-Free Low-Bit Attention Speeds
 *     Video Diffusion Up to 3.6x", V-Smooth and ExpCast-FP8 bullet points;
 *   - yifor blog "Nunchux AI Introduces VC-Attention ...", the MarkTechPost
 *     abstract and the section "V-Smooth and ExpCast-FP8, two targeted
 *     designs";
 *   - aikraft.ru news item, section "Reshenie" (Solution);
 *   - TensorRT-LLM blog on video generation, sections "Quantized Attention"
 *     and "Sparse Attention with Skip Softmax" (online-softmax notation).
 *
 * Conventions for every entry point:
 *   - All tensors are device pointers to contiguous, row-major memory owned
 *     by the caller.  The library allocates nothing, frees nothing and keeps
 *     no state between calls; the workspace of vsmooth_prepare is caller
 *     memory too.  (vsmooth_prepare_noalloc alone takes its workspace from
 *     a fixed scratch array of the library, see there.)
 *   - Every pointer the kernels read or write must be 16-byte aligned.
 *   - Work is enqueued on `stream` and the call returns without waiting.
 *     Concurrent calls on different streams are independent.
 *   - Arguments are checked on the host before anything is launched; on an
 *     error nothing is enqueued and the call returns a negative code whose
 *     text vc_last_error() gives (thread-local storage, never NULL).
 *   - Inputs holding NaN or infinities give undefined results.
 *
 * Sizes: d is 64 or 128; L >= 1; blocks are 128 tokens; nb = ceil(L/128);
 * Lp = 128*nb (the length padded to whole blocks).  The kernels address one
 * head's K and V through 32-bit byte offsets, so 2*Lp*d must stay below 2^31
 * (L <= 8,388,480 at d = 128, L <= 16,777,088 at d = 64); B*H <= 2^20 and
 * B*H*Lp*d <= 2^40.  Larger shapes are rejected with -1.
 */
#ifndef VC_ATTENTION_H
#define VC_ATTENTION_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VC_ATTENTION_VERSION 2

enum {
    VC_OK = 0,
    VC_ERR_INVALID = -1,     /* null or misaligned pointer, bad shape or parameter */
    VC_ERR_UNSUPPORTED = -2, /* head dim other than 64/128, block size other than 128 */
    VC_ERR_WORKSPACE = -3,   /* workspace smaller than vsmooth_workspace_bytes() */
    VC_ERR_HIP = -4          /* a HIP launch or runtime call failed */
};

/* Library version (VC_ATTENTION_VERSION). */
int vc_version(void);

/* Text of the last error on the calling thread ("" if none). */
const char* vc_last_error(void);

/* Attention problem: batch B, heads H, tokens L, head dim d.  Q, K and V are
 * [B, H, L, d]; attention is non-causal self-attention over all L tokens. */
typedef struct vc_shape {
    int32_t B, H, L, d;
} vc_shape;

/* V-Smooth parameters (agihunt V-Smooth bullet; MarkTechPost abstract). */
typedef struct vsmooth_params {
    int32_t block;        /* tokens per hardware block; must be 128 */
    int32_t kmeans_k;     /* clusters of the lightweight k-means; <= 0 means nb */
    int32_t kmeans_iters; /* Lloyd rounds (assign + update); >= 0 */
    int32_t smooth_k;     /* 1: subtract the per-channel mean of K over the L
                             tokens before quantising K (QK smoothing; the
                             softmax is unchanged by it); 0: off */
    int32_t v_scale_mode; /* residual scale per (block, channel):
                             0: s = fp32(amax / 448);
                             1: s = 2^e, the least power of two with amax <= 448 s;
                             must be 0 with v_format 1 */
    int32_t v_format;     /* residual format: 0 E4M3 (the 8-bit kernel); 1 E2M1
                             (4-bit V-Smooth, MarkTechPost abstract): one
                             power-of-two scale 2^e per (block, channel, key
                             group), the group of in-block key kk being
                             kk / 32 (32 consecutive slots), e the least
                             integer with amax <= 6 * 2^e (amax < 2^-100:
                             codes 0); then v8 holds [B,H,nb,d,64] bytes, key
                             kk of the block in slot kk, slot 2t in the low
                             nibble of byte t, and v_scale holds
                             [B,H,nb,d,4] bytes e + 127 in place of fp32
                             scales */
    uint64_t seed;        /* seeds the k-means initial centroids (SplitMix64) */
} vsmooth_params;

/* Output of vsmooth_prepare, input of vc_attention_fwd (all device memory).
 * The residual codes use a block-transposed layout: for block b and channel
 * c, v8[((bh*nb + b)*d + c)*128 + pos] holds the code of the key in slot
 * k = 128 b + kk of the permuted order, where
 *     pos = 32*((kk % 16) / 4) + 4*(kk / 16) + (kk % 4),
 * the order in which the PV matrix-core step consumes keys (E4M3 residual;
 * the 4-bit layout of v_format 1 is described there). */
typedef struct vc_prepared {
    uint8_t* q8;        /* [B,H,Lp,d] E4M3 codes of Q, original token order */
    uint8_t* k8;        /* [B,H,Lp,d] E4M3 codes of K - kbar, permuted order */
    uint8_t* v8;        /* [B,H,nb,d,128] E4M3 codes of V - block mean (above) */
    float* q_scale;     /* [B,H,nb] one scale per 128-token block of Q */
    float* k_scale;     /* [B,H,nb] one scale per 128-token block of permuted K */
    float* v_scale;     /* [B,H,nb,d] residual scale per (block, channel) */
    float* v_mean;      /* [B,H,nb,d] exact (fp32) block mean of V */
    int32_t* perm;      /* [B,H,L] perm[i] = original token in permuted slot i */
    double* kmeans_obj; /* [B,H] k-means objective, or NULL */
} vc_prepared;

/* Byte sizes of the nine vc_prepared buffers, in the struct's order
 * (kmeans_obj counted as B*H doubles). */
int vc_prepared_sizes(const vc_shape* shape, size_t bytes[9]);

/* Workspace that vsmooth_prepare needs for this shape and parameters. */
int vsmooth_workspace_bytes(const vc_shape* shape, const vsmooth_params* params, size_t* bytes);

/* V-Smooth preprocessing (agihunt V-Smooth bullet; MarkTechPost abstract:
 * block mean removed, only the residual quantised; aikraft "Reshenie":
 * lightweight k-means groups similar tokens into blocks, the mean is kept
 * exactly).  Steps, per (batch, head):
 *   1. kbar = mean of K over tokens (if smooth_k);
 *   2. perm = perm_in, or the stable sort by cluster of a seeded Lloyd
 *      k-means over the value rows (kmeans_iters rounds; objective written
 *      to out->kmeans_obj when non-NULL);
 *   3. Q codes per 128-token block in original order, K - kbar codes per
 *      block in permuted order, one fp32 scale amax/448 per block;
 *   4. per permuted block: exact mean of V, residual r = V - mean, per
 *      channel scale (v_scale_mode), E4M3 codes of r (round to nearest even).
 * q, k, v: bf16 [B,H,L,d].  perm_in: NULL or int32 [B,H,L] (each row a
 * permutation of 0..L-1; copied to out->perm; it may be out->perm itself,
 * to keep the permutation of an earlier call across denoising steps, as the
 * MarkTechPost abstract describes; it is not checked: entries outside
 * 0..L-1 are clamped into that range when rows are gathered, so no memory
 * outside the head is read, and the codes are then unspecified).  ws: ws_bytes >=
 * vsmooth_workspace_bytes().  Padded slots (>= L) get code 0. */
int vsmooth_prepare(const vc_shape* shape, const vsmooth_params* params, const void* q,
                    const void* k, const void* v, const int32_t* perm_in,
                    const vc_prepared* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* vsmooth_prepare with the k-means state carried across calls (denoising
 * steps), a reading of the MarkTechPost abstract's grouping amortised over
 * the schedule: the clusters found at one grouping step start the next.
 * Always runs k-means (there is no perm_in).  centroids_in: NULL for the
 * seeded init, else fp32 [B,H,k,d] initial centroids (k = kmeans_k, or nb
 * when kmeans_k <= 0).  centroids_out: NULL, or fp32 [B,H,k,d] that receives
 * the centroids after the last Lloyd round (the member means of the final
 * assignment); it may be centroids_in itself.  Everything else, including
 * the workspace size, as vsmooth_prepare. */
int vsmooth_prepare_warm(const vc_shape* shape, const vsmooth_params* params, const void* q,
                         const void* k, const void* v, const float* centroids_in,
                         float* centroids_out, const vc_prepared* out, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* Size of the fixed device scratch behind vsmooth_prepare_noalloc (64 MiB;
 * enough for every shape up to B*H = 40 heads of L = 75,600 at d = 128 with
 * k-means). */
#define VC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* vsmooth_prepare for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same steps, arguments and results, with the workspace taken from a
 * fixed scratch array inside the library (VC_NOALLOC_SCRATCH_BYTES per
 * device, held by every GPU the library runs on until the process ends)
 * instead of a caller buffer.  The call itself allocates nothing.
 * The scratch address of a device is looked up on the first call made with
 * that device current; the current device must be the one that owns `stream`
 * and the buffers.  Errors: -3 when vsmooth_workspace_bytes() for this shape
 * and parameters exceeds VC_NOALLOC_SCRATCH_BYTES; -4 when the scratch
 * address cannot be obtained; otherwise as vsmooth_prepare.
 * All calls on one GPU share its scratch: calls that overlap in time on one
 * GPU (on different streams, or from different threads without ordering)
 * race and give undefined results.  The scratch keeps whatever the last call
 * left; nothing in it needs to start at zero. */
int vsmooth_prepare_noalloc(const vc_shape* shape, const vsmooth_params* params, const void* q,
                            const void* k, const void* v, const int32_t* perm_in,
                            const vc_prepared* out, hipStream_t stream);

/* Attention parameters. */
typedef struct vc_attn_params {
    int32_t z_off;     /* ExpCast offset in 0..8: the running row maximum is
                          written as the code of 2^z_off (8 by default) */
    int32_t out_dtype; /* 0: fp32 output, 1: bf16 output */
    float skip_lambda; /* Skip Softmax threshold lambda in [0, 1]; 0 rejects
                          nothing (TensorRT-LLM blog, "Sparse Attention with
                          Skip Softmax") */
    int32_t prob_cast; /* probability bytes: 0 ExpCast-FP8 (the method);
                          1 exp-then-cast, the FP8 path ExpCast replaces
                          (MarkTechPost abstract): z = fma(S, c_b,
                          z_off - m'), p = 2^z in fp32, E4M3 round to
                          nearest even.  Other values: -1 */
    int32_t v_format;  /* format of the prepared V residual (vsmooth_params):
                          0 E4M3; 1 E2M1, and then P is E2M1 too: p = 2^z as
                          for prob_cast 1 (required, since ExpCast has no
                          4-bit form), one power-of-two scale per (query,
                          key group) by the rule of v_format, E2M1 codes
                          (round to nearest even), and both products on
                          the scaled FP4 matrix cores.  skip_lambda must be
                          0 with v_format 1.  Other values: -1 */
} vc_attn_params;

/* Fused VC-Attention forward (agihunt ExpCast-FP8 bullet; MarkTechPost
 * abstract: one fused multiply-add writes the E4M3 byte of p = 2^z,
 * byte = round(8 z + 56 + beta), beta = -0.35, clamped at zero).  Per query
 * row and per 128-key block b in ascending order:
 *   S = Q8 K8^T on FP8 matrix cores (exact products, fp32 result);
 *   c_b = fp32(fp32(s_q s_k,b) * log2(e)/sqrt(d));
 *   m' = max(m, fp32(max S * c_b));  P = ExpCast(S, 8 c_b, KB - 8 m')
 *   with KB = fp32(56 - 0.35 + 8 z_off);
 *   l_b = row sum of P;  acc = P V8_b on FP8 matrix cores;
 *   O = 2^(m - m') O + s_v,b * acc + l_b * mean_b;  l = 2^(m - m') l + l_b.
 * Output O / l, [B,H,L,d] in the original token order.
 * Skip Softmax (TensorRT-LLM blog, "Sparse Attention with Skip Softmax"):
 * with skip_lambda > 0, row i rejects block b when exp(m~ - m) < lambda for
 * the block's maximum score m~ and the running maximum m; in the log2 units
 * above that is fp32(t - m) < fp32(log2(lambda)), t = fp32(max S * c_b).  A
 * rejected block leaves m, l and O unchanged (its bytes are 0); when every
 * row of a wave's 32 queries rejects a block, the wave skips the block's
 * ExpCast and P V work.  skip_lambda outside [0, 1] or NaN: -1. */
int vc_attention_fwd(const vc_shape* shape, const vc_attn_params* params,
                     const vc_prepared* in, void* out, hipStream_t stream);

/* Same as vc_attention_fwd, and also writes, for the 256-query tile
 * `q_tile` (queries 256*q_tile ...) of head `bh` = b*H + h, the fp32
 * scores S [256, Lp] and the ExpCast bytes P [256, Lp] of every block
 * (rows past L are left untouched).  A checking aid. */
int vc_attention_fwd_dump(const vc_shape* shape, const vc_attn_params* params,
                          const vc_prepared* in, void* out, int32_t bh, int32_t q_tile,
                          float* s_dump, uint8_t* p_dump, hipStream_t stream);

/* BF16 flash attention on the same scaffold (the FP32 reference path the
 * pages compare against, here on BF16 matrix cores): softmax(Q K^T /
 * sqrt(d)) V with an exp2 online softmax and bf16 probabilities.
 * q, k, v: bf16 [B,H,L,d]; out: [B,H,L,d] fp32 (out_dtype 0) or bf16 (1). */
int vc_attention_fwd_bf16(const vc_shape* shape, const void* q, const void* k, const void* v,
                          void* out, int32_t out_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * SAGE-style quantised attention, the baseline that the TensorRT-LLM blog
 * configures in "Quantized Attention" with five fields: the QK^T format
 * (INT8, the blog's choice, or FP8), the PV format (FP8 E4M3), the query
 * block (1: one Q scale per query token), the key block (16: one K scale per
 * 16 consecutive keys) and the V block (1: one V scale per channel of a
 * head, taken over all its tokens).  Tokens stay in sequence order; there is
 * no k-means and no block mean.  Readings where the blog is silent: a scale
 * is amax / 127 (INT8) or amax / 448 (E4M3) by IEEE division (0 with all
 * codes 0 when amax < 2^-100); INT8 codes round fp32(x / scale) computed as
 * fp32(x * fp32(127 / amax)) to the nearest integer, ties to even, clamped to
 * +-127; K is smoothed by its per-channel mean when smooth_k is 1.
 * ------------------------------------------------------------------------ */
enum { VC_SAGE_QK_INT8 = 0, VC_SAGE_QK_FP8 = 1 };

typedef struct vc_sage_params {
    int32_t qk_dtype;     /* VC_SAGE_QK_INT8 or VC_SAGE_QK_FP8; others: -2 */
    int32_t v_dtype;      /* 0: FP8 E4M3 (the only PV format); others: -2 */
    int32_t q_block_size; /* must be 1, else -2 */
    int32_t k_block_size; /* must be 16, else -2 */
    int32_t v_block_size; /* must be 1 (one scale per channel), else -2 */
    int32_t smooth_k;     /* 1: subtract the per-channel mean of K first; 0: off */
} vc_sage_params;

/* Output of vc_sage_prepare, input of vc_sage_attention_fwd (device memory,
 * sequence order).  v8 uses the block-transposed layout of vc_prepared with
 * slot k = token k (no permutation). */
typedef struct vc_sage_prepared {
    uint8_t* q8;    /* [B,H,Lp,d] INT8 (two's complement) or E4M3 codes of Q */
    uint8_t* k8;    /* [B,H,Lp,d] codes of K (- kbar when smooth_k) */
    uint8_t* v8;    /* [B,H,nb,d,128] E4M3 codes of V */
    float* q_scale; /* [B,H,Lp] one scale per token (0 past L) */
    float* k_scale; /* [B,H,Lp/16] one scale per 16 tokens */
    float* v_scale; /* [B,H,d] one scale per channel */
} vc_sage_prepared;

/* Byte sizes of the six vc_sage_prepared buffers, in the struct's order. */
int vc_sage_prepared_sizes(const vc_shape* shape, size_t bytes[6]);

/* Workspace that vc_sage_prepare needs for this shape. */
int vc_sage_workspace_bytes(const vc_shape* shape, size_t* bytes);

/* SAGE-style quantisation of bf16 q, k, v [B,H,L,d] into `out` (scales and
 * codes as described above; padded tokens >= L get code 0 and scale 0).
 * ws: ws_bytes >= vc_sage_workspace_bytes(), else -3. */
int vc_sage_prepare(const vc_shape* shape, const vc_sage_params* params, const void* q,
                    const void* k, const void* v, const vc_sage_prepared* out, void* ws,
                    size_t ws_bytes, hipStream_t stream);

/* SAGE-style attention forward on the scaffold of vc_attention_fwd (the same
 * 128-key blocks, online softmax and matrix-core products).  Per query row i
 * and block b:
 *   S = Q8 K8^T (INT8 or FP8 matrix cores; INT8 sums are exact);
 *   c_ij = fp32(fp32(s_q,i * log2(e)/sqrt(d)) * s_k,j/16);
 *   m' = max(m, max_j fp32(S_ij c_ij));
 *   bytes: exp-then-cast, E4M3(2^fma(S, c, z_off - m')) (prob_cast 1, the
 *   FP8 path of the SageAttention line), or ExpCast, fma(S, 8c, KB - 8 m')
 *   (prob_cast 0), as in vc_attn_params;
 *   l_b = row sum of P;  acc = P V8_b;
 *   O = 2^(m - m') O + acc;  l = 2^(m - m') l + l_b;
 * output s_v (.) O / l, [B,H,L,d].  params->skip_lambda must be 0 (-2
 * otherwise): the baseline runs dense. */
int vc_sage_attention_fwd(const vc_shape* shape, const vc_sage_params* sage,
                          const vc_attn_params* params, const vc_sage_prepared* in, void* out,
                          hipStream_t stream);

/* vc_sage_attention_fwd plus the scores and bytes of one 256-query tile, as
 * vc_attention_fwd_dump.  A checking aid. */
int vc_sage_attention_fwd_dump(const vc_shape* shape, const vc_sage_params* sage,
                               const vc_attn_params* params, const vc_sage_prepared* in, void* out,
                               int32_t bh, int32_t q_tile, float* s_dump, uint8_t* p_dump,
                               hipStream_t stream);

/* ExpCast-FP8 alone, with the device function the attention kernel uses:
 * bytes[i] = min(max(rne(fma(S[i], c8[i], krow[i])), 0), 126).  A checking
 * aid for the byte map (MarkTechPost abstract). */
int vc_debug_expcast(const float* S, const float* c8, const float* krow, int64_t n,
                     uint8_t* bytes, hipStream_t stream);

/* E4M3 encoding alone, with the device function the preprocessing kernels
 * use: saturating round-to-nearest-even (OCP E4M3FN, bias 7), i.e. the
 * hardware conversion on inputs clamped to +-448. */
int vc_debug_e4m3_encode(const float* x, int64_t n, uint8_t* codes, hipStream_t stream);

/* One FP8 matrix-core product per 16x16 tile: for t < n_tiles,
 * c[t][i][j] = sum_k A[t][i][k] * B[t][j][k] over k < 128, A and B E4M3
 * codes [n_tiles,16,128], c fp32 [n_tiles,16,16].  A checking aid that
 * exposes how the hardware rounds the 128-term sum. */
int vc_debug_mfma_fp8(const uint8_t* a, const uint8_t* b, float* c, int32_t n_tiles,
                      hipStream_t stream);

/* The matrix-core rate with nothing else running: `blocks` workgroups of 8
 * waves, each wave issuing 4 * iters independent 32x32x64 FP8 products
 * (2 * 32 * 32 * 64 FLOP each) from registers, with no memory traffic until
 * every lane writes one float of its results to out (device, caller-owned,
 * blocks * 512 floats; the values carry no meaning).  Timing it gives the
 * FP8 rate, clock and power the chip sustains on products alone, the
 * ceiling against which the attention kernel's fraction of the published
 * peak is read.  blocks in [1, 2^20], iters in [1, 2^24], else
 * VC_ERR_INVALID.  A measurement aid. */
int vc_debug_mfma_rate(int32_t blocks, int32_t iters, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VC_ATTENTION_H */
