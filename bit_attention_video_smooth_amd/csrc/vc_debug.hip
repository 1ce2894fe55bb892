// vc_debug.hip -- checking aids: the ExpCast byte map and the E4M3 encoder
// exactly as the production kernels use them, one FP8 matrix-core product
// per tile (to see how the hardware rounds a 128-term FP8 sum), and a
// stream of independent FP8 products with no memory traffic (the rate the
// matrix cores sustain, and the clock and power they draw, when nothing else
// runs).
#include "vc_device.hpp"
#include "vc_internal.hpp"

namespace vc {

__global__ void debug_expcast_kernel(const float* __restrict__ S, const float* __restrict__ c8,
                                     const float* __restrict__ krow, int64_t n,
                                     uint8_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const uint32_t b = expcast_byte_into(S[i], c8[i], krow[i], 0, 0u) & 0xFFu;
        out[i] = (uint8_t)(b < 126u ? b : 126u);  // the attention kernel never reaches the clamp
    }
}

__global__ void debug_e4m3_kernel(const float* __restrict__ x, int64_t n, uint8_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = (uint8_t)(e4m3_pk2<false>(x[i], 0.0f, 0u) & 0xFFu);
}

// one wave per tile: c = A B^T with A, B [16][128] E4M3 codes
__global__ void debug_mfma_fp8_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                      float* __restrict__ C, int n) {
    const int t = blockIdx.x;
    if (t >= n) return;
    const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
    const uint4* pa = reinterpret_cast<const uint4*>(A + ((size_t)t * 16 + r) * 128 + 32 * g);
    const uint4* pb = reinterpret_cast<const uint4*>(B + ((size_t)t * 16 + r) * 128 + 32 * g);
    uint4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
    v8i va = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    v8i vb = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    v4f z = {0.f, 0.f, 0.f, 0.f};
    v4f c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, z, 0, 0, 0, 0, 0, 0);
    // lane (col = lane & 15, g) holds rows 4 g + i of column col
#pragma unroll
    for (int i = 0; i < 4; i++) C[((size_t)t * 16 + 4 * g + i) * 16 + r] = c[i];
}

// 8 waves per workgroup, each streaming 4 independent accumulations of
// 32x32x64 FP8 products from registers for `iters` rounds; every lane then
// writes the sum of its results, so no product is dead code.
__global__ __launch_bounds__(512) void debug_mfma_rate_kernel(float* __restrict__ out, int iters) {
    typedef float v16f __attribute__((ext_vector_type(16)));
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) {  // finite E4M3 codes: 0x38..0x3F and 0x30..0x37
        a[i] = 0x38383838 ^ (int)((threadIdx.x & 7) * 0x01010101u);
        b[i] = 0x30303030 + i * 0x01010101;
    }
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; it++) {
        c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 0, 0, 0, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 0, 0, 0, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e++) s += (c0[e] + c1[e]) + (c2[e] + c3[e]);
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_debug_expcast(const float* S, const float* c8, const float* krow, int64_t n,
                                uint8_t* out, hipStream_t st) {
    if (n > 0)
        hipLaunchKernelGGL(debug_expcast_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           S, c8, krow, n, out);
    return hipGetLastError();
}

hipError_t launch_debug_e4m3(const float* x, int64_t n, uint8_t* out, hipStream_t st) {
    if (n > 0)
        hipLaunchKernelGGL(debug_e4m3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x,
                           n, out);
    return hipGetLastError();
}

hipError_t launch_debug_mfma_rate(int blocks, int iters, float* out, hipStream_t st) {
    hipLaunchKernelGGL(debug_mfma_rate_kernel, dim3(blocks), dim3(512), 0, st, out, iters);
    return hipGetLastError();
}

hipError_t launch_debug_mfma_fp8(const uint8_t* a, const uint8_t* b, float* c, int n, hipStream_t st) {
    if (n > 0) hipLaunchKernelGGL(debug_mfma_fp8_kernel, dim3(n), dim3(64), 0, st, a, b, c, n);
    return hipGetLastError();
}

}  // namespace vc
