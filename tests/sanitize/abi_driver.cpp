// Exercises the host-side argument checks of the C ABI (every error path
// that returns before any device call), for an AddressSanitizer /
// UndefinedBehaviorSanitizer build of the library's host code (test
// support; built and run by tests/test_sanitizers_cpu.py).  No GPU is used:
// each call below must fail validation, and the pointers are never touched.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "vc_attention.h"

static int fails = 0;
#define EXPECT(call, code)                                                                         \
    do {                                                                                           \
        int r_ = (call);                                                                           \
        if (r_ != (code)) {                                                                        \
            fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, r_,   \
                    (int)(code), vc_last_error());                                                  \
            fails++;                                                                               \
        }                                                                                          \
        if (r_ != 0 && strlen(vc_last_error()) == 0) {                                             \
            fprintf(stderr, "line %d: empty error text\n", __LINE__);                              \
            fails++;                                                                               \
        }                                                                                          \
    } while (0)

int main()
{
    void* P = (void*)(uintptr_t)0x10000;   // aligned, never dereferenced
    void* M = (void*)(uintptr_t)0x10001;   // misaligned
    size_t sz[9];
    vc_shape ok = {1, 2, 300, 64}, big = {1, 24, 245952, 128};
    if (vc_version() != VC_ATTENTION_VERSION) fails++;
    EXPECT(vc_prepared_sizes(&ok, sz), VC_OK);
    EXPECT(vc_prepared_sizes(nullptr, sz), VC_ERR_INVALID);
    EXPECT(vc_prepared_sizes(&ok, nullptr), VC_ERR_INVALID);
    const vc_shape bad[] = {{0, 1, 10, 64}, {1, 0, 10, 64}, {1, 1, 0, 64}, {1, 1, -5, 128},
                            {1, 1, 8388481, 128}, {1, 1, 2147483647, 64}, {2048, 1024, 128, 64},
                            {1, 1 << 20, 1 << 20, 128}};
    for (const vc_shape& s : bad) EXPECT(vc_prepared_sizes(&s, sz), VC_ERR_INVALID);
    vc_shape d96 = {1, 1, 10, 96};
    EXPECT(vc_prepared_sizes(&d96, sz), VC_ERR_UNSUPPORTED);

    vsmooth_params p = {128, 0, 8, 1, 0, 0, 7};
    size_t ws = 0;
    EXPECT(vsmooth_workspace_bytes(&ok, &p, &ws), VC_OK);
    vsmooth_params q = p;
    q.block = 64; EXPECT(vsmooth_workspace_bytes(&ok, &q, &ws), VC_ERR_UNSUPPORTED); q = p;
    q.kmeans_iters = -1; EXPECT(vsmooth_workspace_bytes(&ok, &q, &ws), VC_ERR_INVALID); q = p;
    q.smooth_k = 2; EXPECT(vsmooth_workspace_bytes(&ok, &q, &ws), VC_ERR_INVALID); q = p;
    q.v_scale_mode = 3; EXPECT(vsmooth_workspace_bytes(&ok, &q, &ws), VC_ERR_INVALID); q = p;
    q.v_format = 2; EXPECT(vsmooth_workspace_bytes(&ok, &q, &ws), VC_ERR_INVALID); q = p;
    q.v_format = 1; q.v_scale_mode = 1; EXPECT(vsmooth_workspace_bytes(&ok, &q, &ws), VC_ERR_INVALID); q = p;
    q.kmeans_k = 301; EXPECT(vsmooth_workspace_bytes(&ok, &q, &ws), VC_ERR_INVALID); q = p;
    EXPECT(vsmooth_workspace_bytes(&ok, nullptr, &ws), VC_ERR_INVALID);
    EXPECT(vsmooth_workspace_bytes(&ok, &p, nullptr), VC_ERR_INVALID);

    vc_prepared pr = {(uint8_t*)P, (uint8_t*)P, (uint8_t*)P, (float*)P, (float*)P, (float*)P, (float*)P,
                      (int32_t*)P, nullptr};
    EXPECT(vsmooth_prepare(&ok, &p, P, P, P, nullptr, &pr, P, ws - 1, nullptr), VC_ERR_WORKSPACE);
    EXPECT(vsmooth_prepare(&ok, &p, P, P, P, nullptr, &pr, nullptr, ws, nullptr), VC_ERR_WORKSPACE);
    EXPECT(vsmooth_prepare(&ok, &p, nullptr, P, P, nullptr, &pr, P, ws, nullptr), VC_ERR_INVALID);
    EXPECT(vsmooth_prepare(&ok, &p, P, M, P, nullptr, &pr, P, ws, nullptr), VC_ERR_INVALID);
    EXPECT(vsmooth_prepare(&ok, &p, P, P, P, (const int32_t*)M, &pr, P, ws, nullptr), VC_ERR_INVALID);
    EXPECT(vsmooth_prepare(&ok, &p, P, P, P, nullptr, nullptr, P, ws, nullptr), VC_ERR_INVALID);
    vc_prepared pm = pr; pm.v_mean = (float*)M;
    EXPECT(vsmooth_prepare(&ok, &p, P, P, P, nullptr, &pm, P, ws, nullptr), VC_ERR_INVALID);
    EXPECT(vsmooth_prepare(&ok, &p, P, P, P, nullptr, &pr, M, ws, nullptr), VC_ERR_INVALID);
    EXPECT(vsmooth_prepare_warm(&ok, &p, P, P, P, (const float*)M, nullptr, &pr, P, ws, nullptr), VC_ERR_INVALID);
    EXPECT(vsmooth_prepare_noalloc(&big, &p, P, P, P, nullptr, &pr, nullptr), VC_ERR_WORKSPACE);
    EXPECT(vsmooth_prepare_noalloc(&d96, &p, P, P, P, nullptr, &pr, nullptr), VC_ERR_UNSUPPORTED);

    vc_attn_params a = {8, 0, 0.0f, 0, 0};
    vc_attn_params b = a;
    EXPECT(vc_attention_fwd(&ok, nullptr, &pr, P, nullptr), VC_ERR_INVALID);
    b.z_off = 9; EXPECT(vc_attention_fwd(&ok, &b, &pr, P, nullptr), VC_ERR_INVALID); b = a;
    b.out_dtype = 2; EXPECT(vc_attention_fwd(&ok, &b, &pr, P, nullptr), VC_ERR_INVALID); b = a;
    b.skip_lambda = NAN; EXPECT(vc_attention_fwd(&ok, &b, &pr, P, nullptr), VC_ERR_INVALID); b = a;
    b.skip_lambda = 1.5f; EXPECT(vc_attention_fwd(&ok, &b, &pr, P, nullptr), VC_ERR_INVALID); b = a;
    b.prob_cast = 2; EXPECT(vc_attention_fwd(&ok, &b, &pr, P, nullptr), VC_ERR_INVALID); b = a;
    b.v_format = 3; EXPECT(vc_attention_fwd(&ok, &b, &pr, P, nullptr), VC_ERR_INVALID); b = a;
    b.v_format = 1; EXPECT(vc_attention_fwd(&ok, &b, &pr, P, nullptr), VC_ERR_UNSUPPORTED); b = a;
    b.v_format = 1; b.prob_cast = 1; b.skip_lambda = 0.5f;
    EXPECT(vc_attention_fwd(&ok, &b, &pr, P, nullptr), VC_ERR_UNSUPPORTED); b = a;
    EXPECT(vc_attention_fwd(&ok, &a, &pr, M, nullptr), VC_ERR_INVALID);
    EXPECT(vc_attention_fwd(&ok, &a, &pm, P, nullptr), VC_ERR_INVALID);
    EXPECT(vc_attention_fwd(&bad[4], &a, &pr, P, nullptr), VC_ERR_INVALID);
    EXPECT(vc_attention_fwd_dump(&ok, &a, &pr, P, 2, 0, (float*)P, (uint8_t*)P, nullptr), VC_ERR_INVALID);
    EXPECT(vc_attention_fwd_dump(&ok, &a, &pr, P, 0, 2, (float*)P, (uint8_t*)P, nullptr), VC_ERR_INVALID);
    EXPECT(vc_attention_fwd_dump(&ok, &a, &pr, P, 0, 0, nullptr, (uint8_t*)P, nullptr), VC_ERR_INVALID);
    EXPECT(vc_attention_fwd_bf16(&ok, P, P, nullptr, P, 0, nullptr), VC_ERR_INVALID);
    EXPECT(vc_attention_fwd_bf16(&ok, P, P, P, P, 5, nullptr), VC_ERR_INVALID);
    EXPECT(vc_attention_fwd_bf16(&d96, P, P, P, P, 0, nullptr), VC_ERR_UNSUPPORTED);

    vc_sage_params sp = {VC_SAGE_QK_INT8, 0, 1, 16, 1, 1};
    size_t ssz[6];
    EXPECT(vc_sage_prepared_sizes(&ok, ssz), VC_OK);
    EXPECT(vc_sage_workspace_bytes(&ok, &ws), VC_OK);
    vc_sage_prepared sr = {(uint8_t*)P, (uint8_t*)P, (uint8_t*)P, (float*)P, (float*)P, (float*)P};
    vc_sage_params sq = sp;
    sq.qk_dtype = 5; EXPECT(vc_sage_prepare(&ok, &sq, P, P, P, &sr, P, ws, nullptr), VC_ERR_UNSUPPORTED); sq = sp;
    sq.k_block_size = 32; EXPECT(vc_sage_prepare(&ok, &sq, P, P, P, &sr, P, ws, nullptr), VC_ERR_UNSUPPORTED); sq = sp;
    sq.smooth_k = 3; EXPECT(vc_sage_prepare(&ok, &sq, P, P, P, &sr, P, ws, nullptr), VC_ERR_INVALID); sq = sp;
    EXPECT(vc_sage_prepare(&ok, &sp, P, P, P, &sr, P, ws - 1, nullptr), VC_ERR_WORKSPACE);
    EXPECT(vc_sage_attention_fwd(&ok, &sp, &a, nullptr, P, nullptr), VC_ERR_INVALID);
    b.skip_lambda = 0.5f; EXPECT(vc_sage_attention_fwd(&ok, &sp, &b, &sr, P, nullptr), VC_ERR_UNSUPPORTED); b = a;
    b.v_format = 1; EXPECT(vc_sage_attention_fwd(&ok, &sp, &b, &sr, P, nullptr), VC_ERR_UNSUPPORTED); b = a;
    EXPECT(vc_sage_attention_fwd_dump(&ok, &sp, &a, &sr, P, 9, 0, (float*)P, (uint8_t*)P, nullptr), VC_ERR_INVALID);

    EXPECT(vc_debug_expcast((const float*)P, (const float*)P, (const float*)P, -1, (uint8_t*)P, nullptr), VC_ERR_INVALID);
    EXPECT(vc_debug_expcast(nullptr, nullptr, nullptr, 0, nullptr, nullptr), VC_OK);
    EXPECT(vc_debug_expcast((const float*)M, (const float*)P, (const float*)P, 4, (uint8_t*)P, nullptr), VC_ERR_INVALID);
    EXPECT(vc_debug_e4m3_encode((const float*)P, 4, nullptr, nullptr), VC_ERR_INVALID);
    EXPECT(vc_debug_mfma_fp8((const uint8_t*)P, (const uint8_t*)P, (float*)P, -3, nullptr), VC_ERR_INVALID);
    EXPECT(vc_debug_mfma_rate(0, 10, (float*)P, nullptr), VC_ERR_INVALID);
    EXPECT(vc_debug_mfma_rate(16, 1 << 25, (float*)P, nullptr), VC_ERR_INVALID);
    EXPECT(vc_debug_mfma_rate(16, 10, nullptr, nullptr), VC_ERR_INVALID);

    if (fails) {
        fprintf(stderr, "%d check(s) failed\n", fails);
        return 1;
    }
    printf("abi driver ok\n");
    return 0;
}
