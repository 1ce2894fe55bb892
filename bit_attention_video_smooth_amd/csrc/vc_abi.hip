// vc_abi.hip -- the C ABI of the VC-Attention library (declared in
// include/vc_attention.h): host-side argument checks, workspace carving and
// kernel dispatch.  Nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "vc_attention.h"
#include "vc_internal.hpp"

// Device memory for vsmooth_prepare_noalloc: the prepare workspace (k-means
// centroids, assignment, sort counts, K column partials) lives here instead
// of in a caller buffer.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device array: its device address comes from hipGetSymbolAddress,
// taken once per device (scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[VC_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return VC_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptr(const void* p, const char* name) {
    if (p == nullptr) return fail(VC_ERR_INVALID, "%s is NULL", name);
    if (!aligned16(p)) return fail(VC_ERR_INVALID, "%s is not 16-byte aligned", name);
    return VC_OK;
}

int check_shape(const vc_shape* s) {
    if (s == nullptr) return fail(VC_ERR_INVALID, "shape is NULL");
    if (s->B < 1 || s->H < 1 || s->L < 1)
        return fail(VC_ERR_INVALID, "shape B=%d H=%d L=%d must all be >= 1", s->B, s->H, s->L);
    if (s->d != 64 && s->d != 128) return fail(VC_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", s->d);
    const int64_t nb = ((int64_t)s->L + 127) / 128;
    const int64_t elems = (int64_t)s->B * s->H * nb * 128 * s->d;
    if ((int64_t)s->B * s->H > (1 << 20) || elems > ((int64_t)1 << 40))
        return fail(VC_ERR_INVALID, "shape too large");
    if ((int64_t)s->B * s->H * (((int64_t)s->L + vc::ATTN_BM - 1) / vc::ATTN_BM) > 0x7FFFFFFF)
        return fail(VC_ERR_INVALID, "shape too large for one launch");
    // The attention kernels address one head's K and V (codes, or bf16 rows)
    // through buffer descriptors with 32-bit byte counts and offsets: keep
    // 2 * Lp * d (the bf16 bytes of a padded head) below 2^31.
    if (nb * 128 * s->d * 2 > 0x7FFFFFFF)
        return fail(VC_ERR_INVALID, "L=%d too long for d=%d: one head's padded K/V must stay below 2^31 bytes in bf16 "
                    "(L <= %lld)", s->L, s->d, (long long)(((int64_t)1 << 30) / s->d - 128));
    return VC_OK;
}

int nblk(const vc_shape* s) { return (s->L + 127) / 128; }

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(VC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

int check_params(const vc_shape* s, const vsmooth_params* p, int* kk) {
    if (p == nullptr) return fail(VC_ERR_INVALID, "params is NULL");
    if (p->block != 128) return fail(VC_ERR_UNSUPPORTED, "block=%d (only 128 is supported)", p->block);
    if (p->kmeans_iters < 0 || p->kmeans_iters > 1000)
        return fail(VC_ERR_INVALID, "kmeans_iters=%d out of range [0, 1000]", p->kmeans_iters);
    if (p->smooth_k != 0 && p->smooth_k != 1) return fail(VC_ERR_INVALID, "smooth_k must be 0 or 1");
    if (p->v_scale_mode != 0 && p->v_scale_mode != 1)
        return fail(VC_ERR_INVALID, "v_scale_mode must be 0 or 1");
    if (p->v_format != 0 && p->v_format != 1) return fail(VC_ERR_INVALID, "v_format must be 0 or 1");
    if (p->v_format == 1 && p->v_scale_mode != 0)
        return fail(VC_ERR_INVALID, "v_scale_mode must be 0 with v_format 1 (FP4 scales are powers of two)");
    const int k = p->kmeans_k > 0 ? p->kmeans_k : nblk(s);
    if (k > s->L) return fail(VC_ERR_INVALID, "kmeans_k=%d exceeds L=%d", k, s->L);
    if (k > 16384) return fail(VC_ERR_INVALID, "kmeans_k=%d exceeds 16384", k);
    *kk = k;
    return VC_OK;
}

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t prepare_ws(const vc_shape* s, bool kmeans, int k) {
    const size_t BH = (size_t)s->B * s->H;
    const int ns = vc::k_mean_splits((int)BH, s->L);
    size_t b = a256(BH * ns * s->d * sizeof(double)) + a256(BH * s->d * sizeof(float));
    if (kmeans) b += vc::kmeans_workspace_bytes(s->B, s->H, s->L, s->d, k);
    return b;
}

int check_prepared(const vc_prepared* p, bool need_obj) {
    if (p == nullptr) return fail(VC_ERR_INVALID, "prepared is NULL");
    int r;
    if ((r = check_ptr(p->q8, "q8")) || (r = check_ptr(p->k8, "k8")) || (r = check_ptr(p->v8, "v8")) ||
        (r = check_ptr(p->q_scale, "q_scale")) || (r = check_ptr(p->k_scale, "k_scale")) ||
        (r = check_ptr(p->v_scale, "v_scale")) || (r = check_ptr(p->v_mean, "v_mean")))
        return r;
    (void)need_obj;
    return VC_OK;
}

int attention_common(const vc_shape* shape, const vc_attn_params* params, const vc_prepared* in,
                     void* out, int32_t bh, int32_t q_tile, float* s_dump, uint8_t* p_dump,
                     bool dump, hipStream_t stream) {
    int r;
    if ((r = check_shape(shape))) return r;
    if (params == nullptr) return fail(VC_ERR_INVALID, "params is NULL");
    if (params->z_off < 0 || params->z_off > 8) return fail(VC_ERR_INVALID, "z_off=%d out of [0, 8]", params->z_off);
    if (params->out_dtype != 0 && params->out_dtype != 1)
        return fail(VC_ERR_INVALID, "out_dtype must be 0 (fp32) or 1 (bf16)");
    if (!(params->skip_lambda >= 0.0f && params->skip_lambda <= 1.0f))
        return fail(VC_ERR_INVALID, "skip_lambda must lie in [0, 1]");
    if (params->prob_cast != 0 && params->prob_cast != 1)
        return fail(VC_ERR_INVALID, "prob_cast must be 0 (ExpCast-FP8) or 1 (exp-then-cast)");
    if (params->v_format != 0 && params->v_format != 1)
        return fail(VC_ERR_INVALID, "v_format must be 0 (E4M3) or 1 (E2M1)");
    if (params->v_format == 1 && params->prob_cast != 1)
        return fail(VC_ERR_UNSUPPORTED, "v_format 1 needs prob_cast 1 (ExpCast has no 4-bit form)");
    if (params->v_format == 1 && params->skip_lambda != 0.0f)
        return fail(VC_ERR_UNSUPPORTED, "skip_lambda must be 0 with v_format 1");
    if ((r = check_prepared(in, false))) return r;
    if ((r = check_ptr(out, "out"))) return r;
    vc::AttnArgs a{};
    a.q8 = in->q8; a.k8 = in->k8; a.v8 = in->v8;
    a.q_scale = in->q_scale; a.k_scale = in->k_scale; a.v_scale = in->v_scale; a.v_mean = in->v_mean;
    a.out = out;
    a.L = shape->L;
    a.nb = nblk(shape);
    a.BH = shape->B * shape->H;
    a.nqt = (shape->L + vc::ATTN_BM - 1) / vc::ATTN_BM;
    a.C0 = (float)(1.4426950408889634074 / sqrt((double)shape->d));
    a.KB = (float)(56.0 - 0.35 + 8.0 * (double)params->z_off);
    a.skip_thr = params->skip_lambda > 0.0f ? (float)log2((double)params->skip_lambda) : -INFINITY;
    a.ZOFF = (float)params->z_off;
    a.prob_cast = params->prob_cast;
    a.dump_bh = -1;
    a.dump_qt = -1;
    if (dump) {
        if (bh < 0 || bh >= a.BH) return fail(VC_ERR_INVALID, "bh=%d out of range", bh);
        if (q_tile < 0 || q_tile >= a.nqt) return fail(VC_ERR_INVALID, "q_tile=%d out of range", q_tile);
        if ((r = check_ptr(s_dump, "s_dump")) || (r = check_ptr(p_dump, "p_dump"))) return r;
        a.dump_bh = bh;
        a.dump_qt = q_tile;
        a.s_dump = s_dump;
        a.p_dump = p_dump;
    }
    if (params->v_format == 1)
        return hip_status(vc::launch_attn_fp4v(a, shape->d, params->out_dtype, dump, stream), "vc_attention_fwd");
    return hip_status(vc::launch_attn_fp8(a, shape->d, params->out_dtype, dump, stream), "vc_attention_fwd");
}

int check_sage_params(const vc_sage_params* p) {
    if (p == nullptr) return fail(VC_ERR_INVALID, "sage params is NULL");
    if (p->qk_dtype != VC_SAGE_QK_INT8 && p->qk_dtype != VC_SAGE_QK_FP8)
        return fail(VC_ERR_UNSUPPORTED, "qk_dtype=%d (supported: 0 INT8, 1 FP8)", p->qk_dtype);
    if (p->v_dtype != 0) return fail(VC_ERR_UNSUPPORTED, "v_dtype=%d (only 0, FP8 E4M3, is supported)", p->v_dtype);
    if (p->q_block_size != 1 || p->k_block_size != 16 || p->v_block_size != 1)
        return fail(VC_ERR_UNSUPPORTED, "q/k/v block sizes %d/%d/%d (only 1/16/1 are supported)", p->q_block_size,
                    p->k_block_size, p->v_block_size);
    if (p->smooth_k != 0 && p->smooth_k != 1) return fail(VC_ERR_INVALID, "smooth_k must be 0 or 1");
    return VC_OK;
}

int check_sage_prepared(const vc_sage_prepared* p) {
    if (p == nullptr) return fail(VC_ERR_INVALID, "prepared is NULL");
    int r;
    if ((r = check_ptr(p->q8, "q8")) || (r = check_ptr(p->k8, "k8")) || (r = check_ptr(p->v8, "v8")) ||
        (r = check_ptr(p->q_scale, "q_scale")) || (r = check_ptr(p->k_scale, "k_scale")) ||
        (r = check_ptr(p->v_scale, "v_scale")))
        return r;
    return VC_OK;
}

int nvchunks(const vc_shape* s) { return (s->L + vc::SAGE_VCHUNK - 1) / vc::SAGE_VCHUNK; }

size_t sage_ws(const vc_shape* s) {
    const size_t BH = (size_t)s->B * s->H;
    const int ns = vc::k_mean_splits((int)BH, s->L);
    return a256(BH * ns * s->d * sizeof(double)) + a256(BH * s->d * sizeof(float)) +
           a256(BH * nvchunks(s) * s->d * sizeof(float)) + a256(BH * s->d * sizeof(float));
}

int sage_attention_common(const vc_shape* shape, const vc_sage_params* sp, const vc_attn_params* params,
                          const vc_sage_prepared* in, void* out, int32_t bh, int32_t q_tile, float* s_dump,
                          uint8_t* p_dump, bool dump, hipStream_t stream) {
    int r;
    if ((r = check_shape(shape))) return r;
    if ((r = check_sage_params(sp))) return r;
    if (params == nullptr) return fail(VC_ERR_INVALID, "params is NULL");
    if (params->z_off < 0 || params->z_off > 8) return fail(VC_ERR_INVALID, "z_off=%d out of [0, 8]", params->z_off);
    if (params->out_dtype != 0 && params->out_dtype != 1)
        return fail(VC_ERR_INVALID, "out_dtype must be 0 (fp32) or 1 (bf16)");
    if (params->skip_lambda != 0.0f)
        return fail(VC_ERR_UNSUPPORTED, "skip_lambda must be 0 for the SAGE baseline (it runs dense)");
    if (params->v_format != 0) return fail(VC_ERR_UNSUPPORTED, "v_format must be 0 for the SAGE baseline");
    if (params->prob_cast != 0 && params->prob_cast != 1)
        return fail(VC_ERR_INVALID, "prob_cast must be 0 (ExpCast-FP8) or 1 (exp-then-cast)");
    if ((r = check_sage_prepared(in))) return r;
    if ((r = check_ptr(out, "out"))) return r;
    vc::AttnArgs a{};
    a.q8 = in->q8; a.k8 = in->k8; a.v8 = in->v8;
    a.q_scale = in->q_scale; a.k_scale = in->k_scale; a.v_scale = in->v_scale; a.v_mean = nullptr;
    a.out = out;
    a.L = shape->L;
    a.nb = nblk(shape);
    a.BH = shape->B * shape->H;
    a.nqt = (shape->L + vc::ATTN_BM - 1) / vc::ATTN_BM;
    a.C0 = (float)(1.4426950408889634074 / sqrt((double)shape->d));
    a.KB = (float)(56.0 - 0.35 + 8.0 * (double)params->z_off);
    a.skip_thr = -INFINITY;
    a.ZOFF = (float)params->z_off;
    a.prob_cast = params->prob_cast;
    a.dump_bh = -1;
    a.dump_qt = -1;
    if (dump) {
        if (bh < 0 || bh >= a.BH) return fail(VC_ERR_INVALID, "bh=%d out of range", bh);
        if (q_tile < 0 || q_tile >= a.nqt) return fail(VC_ERR_INVALID, "q_tile=%d out of range", q_tile);
        if ((r = check_ptr(s_dump, "s_dump")) || (r = check_ptr(p_dump, "p_dump"))) return r;
        a.dump_bh = bh;
        a.dump_qt = q_tile;
        a.s_dump = s_dump;
        a.p_dump = p_dump;
    }
    return hip_status(vc::launch_attn_sage(a, shape->d, params->out_dtype, dump, sp->qk_dtype == VC_SAGE_QK_INT8,
                                           stream),
                      "vc_sage_attention_fwd");
}

int prepare_common(const vc_shape* shape, const vsmooth_params* params, const void* q, const void* k,
                   const void* v, const int32_t* perm_in, const float* cent_in, float* cent_out,
                   const vc_prepared* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    int r, kk;
    if ((r = check_shape(shape))) return r;
    if ((r = check_params(shape, params, &kk))) return r;
    if ((r = check_ptr(q, "q")) || (r = check_ptr(k, "k")) || (r = check_ptr(v, "v"))) return r;
    if ((r = check_prepared(out, false))) return r;
    if ((r = check_ptr(out->perm, "perm"))) return r;
    if (perm_in != nullptr && (r = check_ptr(perm_in, "perm_in"))) return r;
    if (out->kmeans_obj != nullptr && (r = check_ptr(out->kmeans_obj, "kmeans_obj"))) return r;
    if (cent_in != nullptr && (r = check_ptr(cent_in, "centroids_in"))) return r;
    if (cent_out != nullptr && (r = check_ptr(cent_out, "centroids_out"))) return r;
    const bool km = perm_in == nullptr;
    const size_t need = prepare_ws(shape, km, kk);
    if (ws == nullptr || ws_bytes < need)
        return fail(VC_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(VC_ERR_INVALID, "ws is not 16-byte aligned");

    const size_t BH = (size_t)shape->B * shape->H;
    const int ns = vc::k_mean_splits((int)BH, shape->L);
    uint8_t* wp = static_cast<uint8_t*>(ws);
    vc::PrepareArgs a{};
    a.B = shape->B; a.H = shape->H; a.L = shape->L; a.d = shape->d; a.nb = nblk(shape);
    a.smooth_k = params->smooth_k;
    a.v_mode = params->v_scale_mode;
    a.v_format = params->v_format;
    a.q = q; a.k = k; a.v = v;
    a.perm = out->perm;
    a.q8 = out->q8; a.k8 = out->k8; a.v8 = out->v8;
    a.q_scale = out->q_scale; a.k_scale = out->k_scale; a.v_scale = out->v_scale; a.v_mean = out->v_mean;
    a.kpartial = reinterpret_cast<double*>(wp);
    wp += a256(BH * ns * shape->d * sizeof(double));
    a.kbar = reinterpret_cast<float*>(wp);
    wp += a256(BH * shape->d * sizeof(float));

    hipError_t e;
    if (km) {
        vc::KmeansArgs m{};
        m.B = shape->B; m.H = shape->H; m.L = shape->L; m.d = shape->d;
        m.k = kk;
        m.iters = params->kmeans_iters;
        m.seed = params->seed;
        m.v = v;
        m.perm = out->perm;
        m.obj = out->kmeans_obj;
        m.cent_in = cent_in;
        m.cent_out = cent_out;
        vc::kmeans_carve(m, wp);
        e = vc::launch_kmeans(m, stream);
        if (e != hipSuccess) return hip_status(e, "k-means");
    } else {
        // plain kernels rather than memcpy/memset nodes, so the call can be graph-captured
        e = vc::launch_copy_perm(perm_in, out->perm, BH * (size_t)shape->L, out->kmeans_obj, BH, stream);
        if (e != hipSuccess) return hip_status(e, "perm copy");
    }
    return hip_status(vc::launch_prepare_quant(a, stream), "vsmooth_prepare");
}


// Device address of `scratch` on the current device, looked up on the first
// call per device (with that device current) and kept; nullptr on failure,
// with the HIP error in *err.
constexpr int MAX_DEVICES = 64;
std::once_flag g_scratch_once[MAX_DEVICES];
void* g_scratch_ptr[MAX_DEVICES];
hipError_t g_scratch_err[MAX_DEVICES];

void* scratch_ptr(int* dev_out, hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    *dev_out = dev;
    if (dev < 0 || dev >= MAX_DEVICES) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    *err = g_scratch_err[dev];
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int vc_version(void) { return VC_ATTENTION_VERSION; }

const char* vc_last_error(void) { return g_err.c_str(); }

int vc_prepared_sizes(const vc_shape* s, size_t bytes[9]) {
    int r;
    if ((r = check_shape(s))) return r;
    if (bytes == nullptr) return fail(VC_ERR_INVALID, "bytes is NULL");
    const size_t BH = (size_t)s->B * s->H, nb = nblk(s), Lp = nb * 128, d = s->d;
    bytes[0] = BH * Lp * d;
    bytes[1] = BH * Lp * d;
    bytes[2] = BH * nb * d * 128;
    bytes[3] = BH * nb * 4;
    bytes[4] = BH * nb * 4;
    bytes[5] = BH * nb * d * 4;
    bytes[6] = BH * nb * d * 4;
    bytes[7] = BH * (size_t)s->L * 4;
    bytes[8] = BH * 8;
    return ok();
}

int vsmooth_workspace_bytes(const vc_shape* shape, const vsmooth_params* params, size_t* bytes) {
    int r, k;
    if ((r = check_shape(shape))) return r;
    if ((r = check_params(shape, params, &k))) return r;
    if (bytes == nullptr) return fail(VC_ERR_INVALID, "bytes is NULL");
    *bytes = prepare_ws(shape, true, k);
    return ok();
}

int vsmooth_prepare(const vc_shape* shape, const vsmooth_params* params, const void* q, const void* k,
                    const void* v, const int32_t* perm_in, const vc_prepared* out, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
    return prepare_common(shape, params, q, k, v, perm_in, nullptr, nullptr, out, ws, ws_bytes, stream);
}

int vsmooth_prepare_noalloc(const vc_shape* shape, const vsmooth_params* params, const void* q, const void* k,
                            const void* v, const int32_t* perm_in, const vc_prepared* out, hipStream_t stream) {
    int r, kk;
    if ((r = check_shape(shape))) return r;
    if ((r = check_params(shape, params, &kk))) return r;
    const size_t need = prepare_ws(shape, perm_in == nullptr, kk);
    if (need > VC_NOALLOC_SCRATCH_BYTES)
        return fail(VC_ERR_WORKSPACE, "vsmooth_prepare_noalloc: this shape needs %zu bytes of workspace, more than the "
                    "library's fixed %zu-byte scratch (use vsmooth_prepare with a caller workspace)", need,
                    (size_t)VC_NOALLOC_SCRATCH_BYTES);
    int dev = -1;
    hipError_t e;
    void* ws = scratch_ptr(&dev, &e);
    if (ws == nullptr) return hip_status(e, "vsmooth_prepare_noalloc: scratch address");
    return prepare_common(shape, params, q, k, v, perm_in, nullptr, nullptr, out, ws, VC_NOALLOC_SCRATCH_BYTES,
                          stream);
}

int vsmooth_prepare_warm(const vc_shape* shape, const vsmooth_params* params, const void* q, const void* k,
                         const void* v, const float* centroids_in, float* centroids_out, const vc_prepared* out,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
    return prepare_common(shape, params, q, k, v, nullptr, centroids_in, centroids_out, out, ws, ws_bytes,
                          stream);
}

int vc_attention_fwd(const vc_shape* shape, const vc_attn_params* params, const vc_prepared* in,
                     void* out, hipStream_t stream) {
    return attention_common(shape, params, in, out, -1, -1, nullptr, nullptr, false, stream);
}

int vc_attention_fwd_dump(const vc_shape* shape, const vc_attn_params* params, const vc_prepared* in,
                          void* out, int32_t bh, int32_t q_tile, float* s_dump, uint8_t* p_dump,
                          hipStream_t stream) {
    return attention_common(shape, params, in, out, bh, q_tile, s_dump, p_dump, true, stream);
}

int vc_attention_fwd_bf16(const vc_shape* shape, const void* q, const void* k, const void* v, void* out,
                          int32_t out_dtype, hipStream_t stream) {
    int r;
    if ((r = check_shape(shape))) return r;
    if ((r = check_ptr(q, "q")) || (r = check_ptr(k, "k")) || (r = check_ptr(v, "v")) ||
        (r = check_ptr(out, "out")))
        return r;
    if (out_dtype != 0 && out_dtype != 1) return fail(VC_ERR_INVALID, "out_dtype must be 0 or 1");
    vc::AttnBf16Args a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.out = out;
    a.L = shape->L;
    a.nkb = nblk(shape);
    a.BH = shape->B * shape->H;
    a.nqt = (shape->L + vc::ATTN_BM - 1) / vc::ATTN_BM;
    a.C0 = (float)(1.4426950408889634074 / sqrt((double)shape->d));
    return hip_status(vc::launch_attn_bf16(a, shape->d, out_dtype, stream), "vc_attention_fwd_bf16");
}

int vc_sage_prepared_sizes(const vc_shape* s, size_t bytes[6]) {
    int r;
    if ((r = check_shape(s))) return r;
    if (bytes == nullptr) return fail(VC_ERR_INVALID, "bytes is NULL");
    const size_t BH = (size_t)s->B * s->H, nb = nblk(s), Lp = nb * 128, d = s->d;
    bytes[0] = BH * Lp * d;
    bytes[1] = BH * Lp * d;
    bytes[2] = BH * nb * d * 128;
    bytes[3] = BH * Lp * 4;
    bytes[4] = BH * (Lp / 16) * 4;
    bytes[5] = BH * d * 4;
    return ok();
}

int vc_sage_workspace_bytes(const vc_shape* shape, size_t* bytes) {
    int r;
    if ((r = check_shape(shape))) return r;
    if (bytes == nullptr) return fail(VC_ERR_INVALID, "bytes is NULL");
    *bytes = sage_ws(shape);
    return ok();
}

int vc_sage_prepare(const vc_shape* shape, const vc_sage_params* params, const void* q, const void* k,
                    const void* v, const vc_sage_prepared* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    int r;
    if ((r = check_shape(shape))) return r;
    if ((r = check_sage_params(params))) return r;
    if ((r = check_ptr(q, "q")) || (r = check_ptr(k, "k")) || (r = check_ptr(v, "v"))) return r;
    if ((r = check_sage_prepared(out))) return r;
    const size_t need = sage_ws(shape);
    if (ws == nullptr || ws_bytes < need)
        return fail(VC_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(VC_ERR_INVALID, "ws is not 16-byte aligned");
    const size_t BH = (size_t)shape->B * shape->H;
    const int ns = vc::k_mean_splits((int)BH, shape->L);
    uint8_t* wp = static_cast<uint8_t*>(ws);
    vc::SageArgs a{};
    a.B = shape->B; a.H = shape->H; a.L = shape->L; a.d = shape->d; a.nb = nblk(shape);
    a.qk_int8 = params->qk_dtype == VC_SAGE_QK_INT8;
    a.smooth_k = params->smooth_k;
    a.q = q; a.k = k; a.v = v;
    a.q8 = out->q8; a.k8 = out->k8; a.v8 = out->v8;
    a.q_scale = out->q_scale; a.k_scale = out->k_scale; a.v_scale = out->v_scale;
    a.nvchunk = nvchunks(shape);
    a.kpartial = reinterpret_cast<double*>(wp);
    wp += a256(BH * ns * shape->d * sizeof(double));
    a.kbar = reinterpret_cast<float*>(wp);
    wp += a256(BH * shape->d * sizeof(float));
    a.vpart = reinterpret_cast<float*>(wp);
    wp += a256(BH * a.nvchunk * shape->d * sizeof(float));
    a.vinv = reinterpret_cast<float*>(wp);
    return hip_status(vc::launch_sage_prepare(a, stream), "vc_sage_prepare");
}

int vc_sage_attention_fwd(const vc_shape* shape, const vc_sage_params* sage, const vc_attn_params* params,
                          const vc_sage_prepared* in, void* out, hipStream_t stream) {
    return sage_attention_common(shape, sage, params, in, out, -1, -1, nullptr, nullptr, false, stream);
}

int vc_sage_attention_fwd_dump(const vc_shape* shape, const vc_sage_params* sage, const vc_attn_params* params,
                               const vc_sage_prepared* in, void* out, int32_t bh, int32_t q_tile, float* s_dump,
                               uint8_t* p_dump, hipStream_t stream) {
    return sage_attention_common(shape, sage, params, in, out, bh, q_tile, s_dump, p_dump, true, stream);
}

int vc_debug_expcast(const float* S, const float* c8, const float* krow, int64_t n, uint8_t* bytes,
                     hipStream_t stream) {
    if (n < 0 || n > ((int64_t)1 << 40)) return fail(VC_ERR_INVALID, "n=%lld out of range", (long long)n);
    if (n == 0) return ok();
    int r;
    if ((r = check_ptr(S, "S")) || (r = check_ptr(c8, "c8")) || (r = check_ptr(krow, "krow")) ||
        (r = check_ptr(bytes, "bytes")))
        return r;
    return hip_status(vc::launch_debug_expcast(S, c8, krow, n, bytes, stream), "vc_debug_expcast");
}

int vc_debug_e4m3_encode(const float* x, int64_t n, uint8_t* codes, hipStream_t stream) {
    if (n < 0 || n > ((int64_t)1 << 40)) return fail(VC_ERR_INVALID, "n=%lld out of range", (long long)n);
    if (n == 0) return ok();
    int r;
    if ((r = check_ptr(x, "x")) || (r = check_ptr(codes, "codes"))) return r;
    return hip_status(vc::launch_debug_e4m3(x, n, codes, stream), "vc_debug_e4m3_encode");
}

int vc_debug_mfma_fp8(const uint8_t* a, const uint8_t* b, float* c, int32_t n_tiles, hipStream_t stream) {
    if (n_tiles < 0) return fail(VC_ERR_INVALID, "n_tiles < 0");
    if (n_tiles == 0) return ok();
    int r;
    if ((r = check_ptr(a, "a")) || (r = check_ptr(b, "b")) || (r = check_ptr(c, "c"))) return r;
    return hip_status(vc::launch_debug_mfma_fp8(a, b, c, n_tiles, stream), "vc_debug_mfma_fp8");
}

int vc_debug_mfma_rate(int32_t blocks, int32_t iters, float* out, hipStream_t stream) {
    if (blocks < 1 || blocks > (1 << 20)) return fail(VC_ERR_INVALID, "blocks=%d out of range [1, 2^20]", blocks);
    if (iters < 1 || iters > (1 << 24)) return fail(VC_ERR_INVALID, "iters=%d out of range [1, 2^24]", iters);
    int r;
    if ((r = check_ptr(out, "out"))) return r;
    return hip_status(vc::launch_debug_mfma_rate(blocks, iters, out, stream), "vc_debug_mfma_rate");
}

}  // extern "C"
