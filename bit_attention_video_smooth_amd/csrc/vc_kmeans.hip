// vc_kmeans.hip -- V-Smooth token grouping for gfx950: a seeded, lightweight
// Lloyd k-means over the value rows of each (batch, head), followed by the
// stable sort of tokens by cluster that defines the joint K/V permutation
// (aikraft.ru "Reshenie": lightweight k-means puts similar tokens into the
// same block; MarkTechPost abstract: 128-token blocks after sorting).
//
// Per Lloyd round:
//   assign  -- distances ||c||^2 - 2 x.c on BF16 matrix cores (centroids as a
//              bf16 high part plus a bf16 low part, so x.c carries ~16
//              mantissa bits), argmin fused in registers, ties to the lowest
//              centroid index;
//   sort    -- stable counting sort by cluster: per-chunk histograms, one
//              scan per head in (cluster, chunk) order, in-chunk ranks;
//   update  -- one workgroup per cluster sums its members (gathered through
//              the sorted order) in fp64 and divides once; empty clusters
//              keep their centroid.
// Initial centroids: token range cut into k strata, one SplitMix64-drawn
// token per stratum (Steele, Lea & Flood 2014; counter-based, so every
// centroid draws independently).
#include "vc_device.hpp"
#include "vc_internal.hpp"

namespace vc {

namespace {

constexpr int KT = 64;      // centroids per LDS tile of the assign kernel
constexpr int CHUNK = 256;  // tokens per chunk of the counting sort

__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

__global__ void km_init(const uint16_t* __restrict__ v, float* __restrict__ cent, int L, int d, int k,
                        int kpad, int H, uint64_t seed) {
    const int c = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh % H;
    const uint64_t sbh = splitmix64(seed, (uint64_t)b * (uint64_t)H + (uint64_t)h);
    const int64_t lo = ((int64_t)c * L) / k, hi = ((int64_t)(c + 1) * L) / k;
    const int64_t j = lo + (int64_t)(splitmix64(sbh, (uint64_t)c) % (uint64_t)(hi - lo));
    for (int e = threadIdx.x; e < d; e += blockDim.x)
        cent[((size_t)bh * kpad + c) * d + e] = bf16_to_f32(v[((size_t)bh * L + j) * d + e]);
}

// fp32 centroids -> bf16 high/low parts and squared norms (padding: +inf norm)
__global__ void km_split(const float* __restrict__ cent, uint16_t* __restrict__ hi,
                         uint16_t* __restrict__ lo, float* __restrict__ cnorm, int d, int k, int kpad) {
    const int c = blockIdx.x, bh = blockIdx.y;
    __shared__ float red[64];
    float s = 0.f;
    for (int e = threadIdx.x; e < d; e += blockDim.x) {
        const size_t i = ((size_t)bh * kpad + c) * d + e;
        const float x = c < k ? cent[i] : 0.f;
        const uint32_t u = __float_as_uint(x);
        const uint32_t hb = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
        const float rem = x - __uint_as_float(hb << 16);
        const uint32_t ur = __float_as_uint(rem);
        const uint32_t lb = (ur + 0x7FFFu + ((ur >> 16) & 1u)) >> 16;
        hi[i] = (uint16_t)hb;
        lo[i] = (uint16_t)lb;
        s += x * x;
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int i = 0; i < (int)(blockDim.x + 63) / 64; i++) t += red[i];
        cnorm[(size_t)bh * kpad + c] = c < k ? t : INFINITY;
    }
}

__device__ __forceinline__ v8bf as_bf(uint4 x) {
    v8bf r;
    __builtin_memcpy(&r, &x, 16);
    return r;
}

// Better (value, index) of two candidates: lower distance, then lower index.
__device__ __forceinline__ void take_better(float& bv, int& bi, float v, int i) {
    if (v < bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

// Grid (ceil(L/128), B*H), 256 threads: 4 waves x 32 tokens.  Output tile of
// the matrix core is (16 centroids) x (16 tokens), so each lane scans 4
// centroids of one token per tile; four lanes per token merge at the end.
template <int D>
__global__ __launch_bounds__(256) void km_assign(const uint16_t* __restrict__ v,
                                                 const uint16_t* __restrict__ chi,
                                                 const uint16_t* __restrict__ clo,
                                                 const float* __restrict__ cnorm,
                                                 int32_t* __restrict__ assign, int L, int k, int kpad) {
    constexpr int NU = D / 32;
    constexpr int RB = D * 2;  // bytes per centroid row
    __shared__ __attribute__((aligned(16))) uint8_t sh[2][KT * RB];
    __shared__ float sn[KT];
    const int bh = blockIdx.y;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, col = lane & 15, g = lane >> 4;
    const int tok0 = blockIdx.x * 128 + w * 32;
    v8bf xop[2][NU];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        const int j = tok0 + 16 * tt + col;
#pragma unroll
        for (int u = 0; u < NU; u++) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (j < L) x = *reinterpret_cast<const uint4*>(v + ((size_t)bh * L + j) * D + 32 * u + 8 * g);
            xop[tt][u] = as_bf(x);
        }
    }
    float bv[2] = {INFINITY, INFINITY};
    int bi[2] = {0x7FFFFFFF, 0x7FFFFFFF};
    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* hib = reinterpret_cast<const uint8_t*>(chi + (size_t)bh * kpad * D);
    const uint8_t* lob = reinterpret_cast<const uint8_t*>(clo + (size_t)bh * kpad * D);
    for (int c0 = 0; c0 < kpad; c0 += KT) {
        // stage KT centroid rows (hi, lo) into LDS, 16-byte chunks, XOR swizzle
        constexpr int NCH = KT * RB / 16;
        for (int p = t; p < NCH; p += 256) {
            const int r = p / (RB / 16), cp = p % (RB / 16);
            const int cs = cp ^ (r & (RB / 16 - 1) & 7);
            *reinterpret_cast<uint4*>(&sh[0][p * 16]) =
                *reinterpret_cast<const uint4*>(hib + (size_t)(c0 + r) * RB + cs * 16);
            *reinterpret_cast<uint4*>(&sh[1][p * 16]) =
                *reinterpret_cast<const uint4*>(lob + (size_t)(c0 + r) * RB + cs * 16);
        }
        if (t < KT) sn[t] = cnorm[(size_t)bh * kpad + c0 + t];
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < KT / 16; ct++) {
            const int r = 16 * ct + col;
            v8bf ah[NU], al[NU];
#pragma unroll
            for (int u = 0; u < NU; u++) {
                // logical chunk 4u+g of row r lives at (4u+g) ^ swizzle
                const int lc = 4 * u + g;
                const int pc = lc ^ (r & (RB / 16 - 1) & 7);
                ah[u] = as_bf(*reinterpret_cast<const uint4*>(&sh[0][r * RB + pc * 16]));
                al[u] = as_bf(*reinterpret_cast<const uint4*>(&sh[1][r * RB + pc * 16]));
            }
#pragma unroll
            for (int tt = 0; tt < 2; tt++) {
                v4f acc = zero4;
#pragma unroll
                for (int u = 0; u < NU; u++) {
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], xop[tt][u], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[u], xop[tt][u], acc, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int ci = 16 * ct + 4 * g + i;
                    const float dist = __builtin_fmaf(-2.0f, acc[i], sn[ci]);
                    take_better(bv[tt], bi[tt], dist, c0 + ci);
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        // merge the four lane groups (lanes col, col+16, col+32, col+48)
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
            const float ov = __shfl_xor(bv[tt], o);
            const int oi = __shfl_xor(bi[tt], o);
            take_better(bv[tt], bi[tt], ov, oi);
        }
        const int j = tok0 + 16 * tt + col;
        if (g == 0 && j < L) assign[(size_t)bh * L + j] = bi[tt] < k ? bi[tt] : k - 1;
    }
}

// per-chunk cluster histogram: cnt[bh][chunk][c]
__global__ __launch_bounds__(CHUNK) void km_chunk_count(const int32_t* __restrict__ assign,
                                                        int32_t* __restrict__ cnt, int L, int k,
                                                        int nchunk) {
    extern __shared__ int hist[];
    const int ch = blockIdx.x, bh = blockIdx.y;
    for (int c = threadIdx.x; c < k; c += CHUNK) hist[c] = 0;
    __syncthreads();
    const int j = ch * CHUNK + threadIdx.x;
    if (j < L) atomicAdd(&hist[assign[(size_t)bh * L + j]], 1);
    __syncthreads();
    int32_t* out = cnt + ((size_t)bh * nchunk + ch) * k;
    for (int c = threadIdx.x; c < k; c += CHUNK) out[c] = hist[c];
}

// One workgroup per head: turns cnt[chunk][c] into exclusive start offsets in
// (cluster, chunk) order, in place; writes per-cluster counts and starts.
__global__ __launch_bounds__(1024) void km_scan(int32_t* __restrict__ cnt, int32_t* __restrict__ counts,
                                                int32_t* __restrict__ starts, int k, int nchunk) {
    __shared__ int part[1024];
    const int bh = blockIdx.x, t = threadIdx.x;
    int32_t* base = cnt + (size_t)bh * nchunk * k;
    // cluster totals; each thread owns a contiguous range of clusters
    const int per = (k + 1023) / 1024;
    const int c0 = t * per, c1 = min(k, c0 + per);
    int local = 0;
    for (int c = c0; c < c1; c++) {
        int s = 0;
        for (int ch = 0; ch < nchunk; ch++) s += base[(size_t)ch * k + c];
        counts[(size_t)bh * k + c] = s;
        local += s;
    }
    part[t] = local;
    __syncthreads();
    // exclusive scan of the 1024 partial sums (Hillis-Steele)
    for (int o = 1; o < 1024; o <<= 1) {
        int x = t >= o ? part[t - o] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    int run = part[t] - local;
    for (int c = c0; c < c1; c++) {
        starts[(size_t)bh * k + c] = run;
        for (int ch = 0; ch < nchunk; ch++) {
            const int x = base[(size_t)ch * k + c];
            base[(size_t)ch * k + c] = run;
            run += x;
        }
    }
}

// stable scatter: slot = start[chunk][a_j] + #(earlier tokens of the chunk in a_j)
__global__ __launch_bounds__(CHUNK) void km_scatter(const int32_t* __restrict__ assign,
                                                    const int32_t* __restrict__ cnt,
                                                    int32_t* __restrict__ perm, int L, int k,
                                                    int nchunk) {
    __shared__ int sa[CHUNK];
    const int ch = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int j = ch * CHUNK + t;
    const int a = j < L ? assign[(size_t)bh * L + j] : -1;
    sa[t] = a;
    __syncthreads();
    if (j >= L) return;
    int rank = 0;
    for (int i = 0; i < t; i++) rank += (sa[i] == a);
    perm[(size_t)bh * L + cnt[((size_t)bh * nchunk + ch) * k + a] + rank] = j;
}

// one workgroup per (cluster, head): centroid = fp64 mean of members
template <int D>
__global__ __launch_bounds__(256) void km_update(const uint16_t* __restrict__ v,
                                                 const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ counts,
                                                 const int32_t* __restrict__ starts,
                                                 float* __restrict__ cent, int L, int k, int kpad) {
    constexpr int RPI = 256 / D;  // member rows per iteration
    __shared__ double red[RPI][D];
    const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int e = t % D, rs = t / D;
    const int n = counts[(size_t)bh * k + c];
    if (n == 0) return;  // empty cluster keeps its centroid (uniform branch)
    const int s0 = starts[(size_t)bh * k + c];
    double s = 0.0;
    for (int i = rs; i < n; i += RPI) {
        const int j = perm[(size_t)bh * L + s0 + i];
        s += (double)bf16_to_f32(v[((size_t)bh * L + j) * D + e]);
    }
    red[rs][e] = s;
    __syncthreads();
    if (rs == 0) {
        double tot = 0.0;
        for (int i = 0; i < RPI; i++) tot += red[i][e];
        cent[((size_t)bh * kpad + c) * D + e] = (float)(tot / (double)n);
    }
}

// objective: sum_j ||x_j - C_{a_j}||^2 in fp64, per 256-token chunk
template <int D>
__global__ __launch_bounds__(256) void km_objective(const uint16_t* __restrict__ v,
                                                    const int32_t* __restrict__ assign,
                                                    const float* __restrict__ cent,
                                                    double* __restrict__ part, int L, int kpad,
                                                    int nchunk) {
    __shared__ double red[4];
    const int ch = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int j = ch * CHUNK + t;
    double s = 0.0;
    if (j < L) {
        const int a = assign[(size_t)bh * L + j];
        const uint16_t* x = v + ((size_t)bh * L + j) * D;
        const float* cc = cent + ((size_t)bh * kpad + a) * D;
        for (int e = 0; e < D; e++) {
            const double dd = (double)bf16_to_f32(x[e]) - (double)cc[e];
            s += dd * dd;
        }
    }
    s = wave_sum_f64(s);
    if ((t & 63) == 0) red[t >> 6] = s;
    __syncthreads();
    if (t == 0) part[(size_t)bh * nchunk + ch] = red[0] + red[1] + red[2] + red[3];
}

__global__ void km_objective_final(const double* __restrict__ part, double* __restrict__ obj,
                                   int nchunk) {
    const int bh = blockIdx.x;
    if (threadIdx.x != 0) return;
    double s = 0.0;
    for (int i = 0; i < nchunk; i++) s += part[(size_t)bh * nchunk + i];
    obj[bh] = s;
}

template <int D>
hipError_t launch_kmeans_t(const KmeansArgs& a, hipStream_t st) {
    const int BH = a.B * a.H;
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    const int ntile = (a.L + 127) / 128;
    hipLaunchKernelGGL(km_init, dim3(a.k, BH), dim3(64), 0, st, v, a.cent, a.L, D, a.k, a.kpad, a.H,
                       a.seed);
    const int rounds = a.iters > 0 ? a.iters : 1;
    for (int it = 0; it < rounds; it++) {
        hipLaunchKernelGGL(km_split, dim3(a.kpad, BH), dim3(64), 0, st, a.cent, a.cent_hi, a.cent_lo,
                           a.cnorm, D, a.k, a.kpad);
        hipLaunchKernelGGL((km_assign<D>), dim3(ntile, BH), dim3(256), 0, st, v, a.cent_hi, a.cent_lo,
                           a.cnorm, a.assign, a.L, a.k, a.kpad);
        hipLaunchKernelGGL(km_chunk_count, dim3(a.nchunk, BH), dim3(CHUNK), a.k * sizeof(int), st,
                           a.assign, a.chunk_cnt, a.L, a.k, a.nchunk);
        hipLaunchKernelGGL(km_scan, dim3(BH), dim3(1024), 0, st, a.chunk_cnt, a.counts, a.offsets, a.k,
                           a.nchunk);
        hipLaunchKernelGGL(km_scatter, dim3(a.nchunk, BH), dim3(CHUNK), 0, st, a.assign, a.chunk_cnt,
                           a.perm, a.L, a.k, a.nchunk);
        if (a.iters > 0)
            hipLaunchKernelGGL((km_update<D>), dim3(a.k, BH), dim3(256), 0, st, v, a.perm, a.counts,
                               a.offsets, a.cent, a.L, a.k, a.kpad);
    }
    if (a.obj) {
        hipLaunchKernelGGL((km_objective<D>), dim3(a.nchunk, BH), dim3(256), 0, st, v, a.assign, a.cent,
                           a.obj_part, a.L, a.kpad, a.nchunk);
        hipLaunchKernelGGL(km_objective_final, dim3(BH), dim3(64), 0, st, a.obj_part, a.obj, a.nchunk);
    }
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t kmeans_workspace_bytes(int B, int H, int L, int d, int k) {
    const size_t BH = (size_t)B * H;
    const size_t kpad = ((size_t)k + KT - 1) / KT * KT;
    const size_t nchunk = ((size_t)L + CHUNK - 1) / CHUNK;
    size_t s = 0;
    s += align256(BH * kpad * d * 4);       // cent
    s += 2 * align256(BH * kpad * d * 2);   // hi, lo
    s += align256(BH * kpad * 4);           // cnorm
    s += align256(BH * L * 4);              // assign
    s += 2 * align256(BH * k * 4);          // counts, offsets
    s += align256(BH * nchunk * k * 4);     // chunk counts
    s += align256(BH * nchunk * 8);         // objective partials
    return s;
}

void kmeans_carve(KmeansArgs& a, void* ws) {
    const size_t BH = (size_t)a.B * a.H;
    a.kpad = (a.k + KT - 1) / KT * KT;
    a.nchunk = (a.L + CHUNK - 1) / CHUNK;
    uint8_t* p = static_cast<uint8_t*>(ws);
    a.cent = reinterpret_cast<float*>(p);          p += align256(BH * a.kpad * a.d * 4);
    a.cent_hi = reinterpret_cast<uint16_t*>(p);    p += align256(BH * a.kpad * a.d * 2);
    a.cent_lo = reinterpret_cast<uint16_t*>(p);    p += align256(BH * a.kpad * a.d * 2);
    a.cnorm = reinterpret_cast<float*>(p);         p += align256(BH * a.kpad * 4);
    a.assign = reinterpret_cast<int32_t*>(p);      p += align256(BH * a.L * 4);
    a.counts = reinterpret_cast<int32_t*>(p);      p += align256(BH * a.k * 4);
    a.offsets = reinterpret_cast<int32_t*>(p);     p += align256(BH * a.k * 4);
    a.chunk_cnt = reinterpret_cast<int32_t*>(p);   p += align256(BH * a.nchunk * a.k * 4);
    a.obj_part = reinterpret_cast<double*>(p);
}

hipError_t launch_kmeans(const KmeansArgs& a, hipStream_t st) {
    return a.d == 128 ? launch_kmeans_t<128>(a, st) : launch_kmeans_t<64>(a, st);
}

}  // namespace vc
