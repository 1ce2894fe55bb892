// vc_kmeans.hip -- V-Smooth token grouping for gfx950: a seeded, lightweight
// Lloyd k-means over the value rows of each (batch, head), followed by the
// stable sort of tokens by cluster that defines the joint K/V permutation
// (aikraft.ru "Reshenie": lightweight k-means puts similar tokens into the
// same block; MarkTechPost abstract: 128-token blocks after sorting).
//
// Per Lloyd round:
//   assign  -- squared distances ||c||^2 - 2 x.c on BF16 matrix cores, the
//              centroid split into a bf16 high part and a bf16 low part so
//              that x.c (x is bf16 already) carries ~16 mantissa bits;
//              argmin fused in registers, ties to the lowest centroid index;
//              one workgroup takes 512 tokens so that each centroid tile it
//              stages in LDS serves many tokens;
//   sort    -- stable counting sort by cluster: per-chunk histograms, one
//              scan per head in (cluster, chunk) order, in-chunk ranks;
//   update  -- one workgroup per cluster sums its members (gathered through
//              the sorted order, 16 bytes per lane) in fp64 and divides once;
//              empty clusters keep their centroid.
// With the split, the assignment follows the exact-arithmetic one except at
// near-exact ties.
// Initial centroids: token range cut into k strata, one SplitMix64-drawn
// token per stratum (Steele, Lea & Flood 2014; counter-based, so every
// centroid draws independently).
#include "vc_device.hpp"
#include "vc_internal.hpp"

namespace vc {

namespace {

constexpr int KT = KMEANS_KT;        // centroids per LDS tile of the assign kernel
constexpr int CHUNK = KMEANS_CHUNK;  // tokens per chunk of the counting sort
constexpr int ANTT = 8;      // 16-token tiles per wave of the assign kernel
constexpr int ATOK = 8 * 16 * ANTT;  // tokens per assign workgroup (8 waves)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// warm start: caller centroids [BH, k, d] into the padded workspace rows, and
// the final centroids back out (plain copy kernels, so a captured graph holds
// no copy nodes)
__global__ void km_init_from(const float* __restrict__ src, float* __restrict__ cent, int d, int k, int kpad) {
    const int c = blockIdx.x, bh = blockIdx.y;
    for (int e = threadIdx.x; e < d; e += blockDim.x)
        cent[((size_t)bh * kpad + c) * d + e] = src[((size_t)bh * k + c) * d + e];
}

__global__ void km_copy_out(const float* __restrict__ cent, float* __restrict__ dst, int d, int k, int kpad) {
    const int c = blockIdx.x, bh = blockIdx.y;
    for (int e = threadIdx.x; e < d; e += blockDim.x)
        dst[((size_t)bh * k + c) * d + e] = cent[((size_t)bh * kpad + c) * d + e];
}

// fp32 centroids -> bf16 high and low parts (round to nearest even) and the
// squared norm (padding rows: zeros and +inf norm, never chosen)
__global__ void km_split(const float* __restrict__ cent, uint16_t* __restrict__ hi,
                         uint16_t* __restrict__ lo, float* __restrict__ cnorm, int d, int k, int kpad) {
    const int c = blockIdx.x, bh = blockIdx.y;
    __shared__ float red[64];
    float s = 0.f;
    for (int e = threadIdx.x; e < d; e += blockDim.x) {
        const size_t i = ((size_t)bh * kpad + c) * d + e;
        const float x = c < k ? cent[i] : 0.f;
        const uint32_t u = __float_as_uint(x);
        const uint32_t hb = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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

// Position of logical 16-byte chunk lc of centroid row r in LDS.  A 16-byte
// LDS read is conflict-free when every 8 consecutive lanes hit distinct
// 16-byte positions modulo 128 bytes and every 16 lanes distinct positions
// modulo 256 bytes; an operand read sends rows r = 0..15 of a tile to lanes
// 0..15 with one lc, which these XORs spread.
template <int D>
__device__ __forceinline__ int cent_chunk(int r, int lc) {
    if (D == 128) return lc ^ (r & 15);                     // 256-byte rows, 16 chunks
    return lc ^ ((r & 7) ^ ((r >> 3) & 1));                 // 128-byte rows, 8 chunks
}

// Grid (ceil(L/ATOK), B*H), 512 threads: 8 waves x 16 ANTT tokens.  The output
// tile of the matrix core is (16 centroids) x (16 tokens): a lane scans 4
// centroids of one token per tile and the four lanes of a token merge at the
// end.  Centroid tiles of 64 rows are double-buffered in LDS.  The product
// accumulates onto -||c||^2 / 2, so the nearest centroid is the largest
// score x.c - ||c||^2 / 2; a lane meets its candidates in increasing index
// order, so a strict comparison keeps the lowest index among equal scores.
template <int D>
__global__ __launch_bounds__(512) void km_assign(const uint16_t* __restrict__ v,
                                                 const uint16_t* __restrict__ chi,
                                                 const uint16_t* __restrict__ clo,
                                                 const float* __restrict__ cnorm,
                                                 int32_t* __restrict__ assign, int L, int k, int kpad) {
    constexpr int NU = D / 32;          // 32-element steps of the bf16 product
    constexpr int RB = D * 2;           // bytes per centroid row
    constexpr int NTT = ANTT;           // 16-token tiles per wave
    constexpr int NCH = KT * RB / 16;   // 16-byte chunks per centroid tile
    constexpr int CPT = NCH / 512;      // chunks staged per thread
    constexpr int CPR = RB / 16;        // chunks per row
    __shared__ __attribute__((aligned(16))) uint8_t sh[2][KT * RB];  // high parts
    __shared__ __attribute__((aligned(16))) uint8_t sl[2][KT * RB];  // low parts
    __shared__ __attribute__((aligned(16))) float sn[2][KT];  // -||c||^2 / 2
    const int bh = blockIdx.y;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, col = lane & 15, g = lane >> 4;
    const int tok0 = blockIdx.x * ATOK + w * 16 * NTT;
    v8bf xop[NTT][NU];
#pragma unroll
    for (int tt = 0; tt < NTT; tt++) {
        const int j = tok0 + 16 * tt + col;
#pragma unroll
        for (int u = 0; u < NU; u++) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (j < L) x = *reinterpret_cast<const uint4*>(v + ((size_t)bh * L + j) * D + 32 * u + 8 * g);
            xop[tt][u] = as_bf(x);
        }
    }
    float bv[NTT];
    int bi[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; tt++) {
        bv[tt] = -INFINITY;
        bi[tt] = 0x7FFFFFFF;
    }
    const uint8_t* hib = reinterpret_cast<const uint8_t*>(chi + (size_t)bh * kpad * D);
    const uint8_t* lob = reinterpret_cast<const uint8_t*>(clo + (size_t)bh * kpad * D);
    const float* nb = cnorm + (size_t)bh * kpad;
    // staging: thread t copies LDS chunks p = t + 512 i, i < CPT; chunk p of
    // LDS row r holds logical chunk cent_chunk(r, p % CPR) of centroid row r
    size_t goff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; i++) {
        const int p = t + 512 * i, r = p / CPR, cp = p % CPR;
        goff[i] = (size_t)r * RB + cent_chunk<D>(r, cp) * 16;
    }
    // (ext-vector registers, so that the staged copies stay in VGPRs)
    u32x4 stg[CPT], stl[CPT];
    float stn = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; i++) {
        stg[i] = *reinterpret_cast<const u32x4*>(hib + goff[i]);
        stl[i] = *reinterpret_cast<const u32x4*>(lob + goff[i]);
    }
    if (t < KT) stn = nb[t];
#pragma unroll
    for (int i = 0; i < CPT; i++) {
        *reinterpret_cast<u32x4*>(&sh[0][(t + 512 * i) * 16]) = stg[i];
        *reinterpret_cast<u32x4*>(&sl[0][(t + 512 * i) * 16]) = stl[i];
    }
    if (t < KT) sn[0][t] = -0.5f * stn;
    __syncthreads();
    const int ntile = kpad / KT;
    for (int tile = 0; tile < ntile; tile++) {
        const int c0 = tile * KT, buf = tile & 1;
        if (tile + 1 < ntile) {
            const size_t cb = (size_t)(c0 + KT) * RB;
#pragma unroll
            for (int i = 0; i < CPT; i++) {
                stg[i] = *reinterpret_cast<const u32x4*>(hib + cb + goff[i]);
                stl[i] = *reinterpret_cast<const u32x4*>(lob + cb + goff[i]);
            }
            if (t < KT) stn = nb[c0 + KT + t];
        }
        // 16-centroid tiles of this LDS tile that hold real centroids: all of
        // them except in the last tile; the full case is one straight block
        // so that operand reads of one tile overlap the products of another
        auto ctile = [&](int ct) {
            const int r = 16 * ct + col;
            v8bf ah[NU], al[NU];
#pragma unroll
            for (int u = 0; u < NU; u++) {
                const int pos = r * RB + cent_chunk<D>(r, 4 * u + g) * 16;
                ah[u] = as_bf(*reinterpret_cast<const uint4*>(&sh[buf][pos]));
                al[u] = as_bf(*reinterpret_cast<const uint4*>(&sl[buf][pos]));
            }
            const v4f init = *reinterpret_cast<const v4f*>(&sn[buf][16 * ct + 4 * g]);
#pragma unroll
            for (int tt = 0; tt < NTT; tt++) {
                v4f acc = init;
#pragma unroll
                for (int u = 0; u < NU; u++) {
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[u], xop[tt][u], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[u], xop[tt][u], acc, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const bool better = acc[i] > bv[tt];
                    bv[tt] = fmaxf(bv[tt], acc[i]);
                    bi[tt] = better ? c0 + 16 * ct + 4 * g + i : bi[tt];
                }
            }
        };
        if (c0 + KT <= k) {
#pragma unroll
            for (int ct = 0; ct < KT / 16; ct++) ctile(ct);
        } else {
            for (int ct = 0; ct < KT / 16 && c0 + 16 * ct < k; ct++) ctile(ct);
        }
        if (tile + 1 < ntile) {
#pragma unroll
            for (int i = 0; i < CPT; i++) {
                *reinterpret_cast<u32x4*>(&sh[buf ^ 1][(t + 512 * i) * 16]) = stg[i];
                *reinterpret_cast<u32x4*>(&sl[buf ^ 1][(t + 512 * i) * 16]) = stl[i];
            }
            if (t < KT) sn[buf ^ 1][t] = -0.5f * stn;
        }
        __syncthreads();
    }
#pragma unroll
    for (int tt = 0; tt < NTT; tt++) {
        // merge the four lane groups (lanes col, col+16, col+32, col+48)
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
            const float ov = __shfl_xor(bv[tt], o);
            const int oi = __shfl_xor(bi[tt], o);
            if (ov > bv[tt] || (ov == bv[tt] && oi < bi[tt])) {
                bv[tt] = ov;
                bi[tt] = oi;
            }
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
    // (the chunk loops take eight entries per step, all loads issued before
    // their use, so they do not wait on one load at a time)
    constexpr int U = 8;
    int local = 0;
    for (int c = c0; c < c1; c++) {
        int s = 0;
        int ch = 0;
        for (; ch + U <= nchunk; ch += U) {
            int x[U];
#pragma unroll
            for (int u = 0; u < U; u++) x[u] = base[(size_t)(ch + u) * k + c];
#pragma unroll
            for (int u = 0; u < U; u++) s += x[u];
        }
        for (; ch < nchunk; ch++) s += base[(size_t)ch * k + c];
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
        int ch = 0;
        for (; ch + U <= nchunk; ch += U) {
            int x[U];
#pragma unroll
            for (int u = 0; u < U; u++) x[u] = base[(size_t)(ch + u) * k + c];
#pragma unroll
            for (int u = 0; u < U; u++) {
                base[(size_t)(ch + u) * k + c] = run;
                run += x[u];
            }
        }
        for (; ch < nchunk; ch++) {
            const int x = base[(size_t)ch * k + c];
            base[(size_t)ch * k + c] = run;
            run += x;
        }
    }
}

// Stable scatter of one chunk: the waves take their 64 tokens in order; a
// token's slot is its cluster's running position in LDS plus the number of
// earlier lanes of its wave in the same cluster; the last such lane advances
// the running position before the next wave reads it.
__global__ __launch_bounds__(CHUNK) void km_scatter(const int32_t* __restrict__ assign,
                                                    const int32_t* __restrict__ cnt,
                                                    int32_t* __restrict__ perm, int L, int k,
                                                    int nchunk) {
    extern __shared__ int run[];
    const int ch = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int w = t >> 6, lane = t & 63;
    for (int c = t; c < k; c += CHUNK) run[c] = cnt[((size_t)bh * nchunk + ch) * k + c];
    const int j = ch * CHUNK + t;
    const int a = j < L ? assign[(size_t)bh * L + j] : -1;
    int rank = 0;
    bool last = true;
    for (int i = 0; i < 64; i++) {
        const int ai = __shfl(a, i);
        rank += (i < lane && ai == a) ? 1 : 0;
        if (i > lane && ai == a) last = false;
    }
    __syncthreads();
    for (int s = 0; s < CHUNK / 64; s++) {
        if (w == s && a >= 0) {
            const int slot = run[a] + rank;
            perm[(size_t)bh * L + slot] = j;
            if (last) run[a] = slot + 1;
        }
        __syncthreads();
    }
}

// One workgroup per (cluster, head): centroid = fp64 mean of its members.
// Lanes take 16 bytes (8 channels) of a member row; 256 / (D / 8) rows are
// in flight per pass, two passes unrolled.
template <int D>
__global__ __launch_bounds__(256) void km_update(const uint16_t* __restrict__ v,
                                                 const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ counts,
                                                 const int32_t* __restrict__ starts,
                                                 float* __restrict__ cent, int L, int k, int kpad) {
    constexpr int LPR = D / 8;      // lanes per row
    constexpr int RPP = 256 / LPR;  // rows per pass
    __shared__ double red[RPP][D];
    const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int q = t % LPR, rs = t / LPR;
    const int n = counts[(size_t)bh * k + c];
    if (n == 0) return;  // empty cluster keeps its centroid (uniform branch)
    const int s0 = starts[(size_t)bh * k + c];
    const int32_t* pm = perm + (size_t)bh * L + s0;
    const uint16_t* vb = v + (size_t)bh * L * D + 8 * q;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = 0.0;
    int i = rs;
    for (; i + RPP < n; i += 2 * RPP) {
        const int j0 = pm[i], j1 = pm[i + RPP];
        const uint4 x0 = *reinterpret_cast<const uint4*>(vb + (size_t)j0 * D);
        const uint4 x1 = *reinterpret_cast<const uint4*>(vb + (size_t)j1 * D);
        const uint32_t w0[4] = {x0.x, x0.y, x0.z, x0.w}, w1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            acc[2 * e] += (double)__uint_as_float(w0[e] << 16);
            acc[2 * e + 1] += (double)__uint_as_float(w0[e] & 0xFFFF0000u);
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            acc[2 * e] += (double)__uint_as_float(w1[e] << 16);
            acc[2 * e + 1] += (double)__uint_as_float(w1[e] & 0xFFFF0000u);
        }
    }
    if (i < n) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(vb + (size_t)pm[i] * D);
        const uint32_t w0[4] = {x0.x, x0.y, x0.z, x0.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            acc[2 * e] += (double)__uint_as_float(w0[e] << 16);
            acc[2 * e + 1] += (double)__uint_as_float(w0[e] & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) red[rs][8 * q + e] = acc[e];
    __syncthreads();
    if (t < D) {
        double tot = 0.0;
        for (int r = 0; r < RPP; r++) tot += red[r][t];
        cent[((size_t)bh * kpad + c) * D + t] = (float)(tot / (double)n);
    }
}

// objective: sum_j ||x_j - C_{a_j}||^2 in fp64, per chunk of CHUNK tokens;
// D / 8 lanes per token, 16 bytes of the row each
template <int D>
__global__ __launch_bounds__(256) void km_objective(const uint16_t* __restrict__ v,
                                                    const int32_t* __restrict__ assign,
                                                    const float* __restrict__ cent,
                                                    double* __restrict__ part, int L, int kpad,
                                                    int nchunk) {
    constexpr int LPR = D / 8, TPP = 256 / LPR;
    __shared__ double red[4];
    const int ch = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    const int q = t % LPR, r = t / LPR;
    double s = 0.0;
    for (int jj = r; jj < CHUNK; jj += TPP) {
        const int j = ch * CHUNK + jj;
        if (j >= L) break;
        const int a = assign[(size_t)bh * L + j];
        const uint4 x = *reinterpret_cast<const uint4*>(v + ((size_t)bh * L + j) * D + 8 * q);
        const float4* cc = reinterpret_cast<const float4*>(cent + ((size_t)bh * kpad + a) * D + 8 * q);
        const float4 c0 = cc[0], c1 = cc[1];
        const uint32_t wv[4] = {x.x, x.y, x.z, x.w};
        const float cf[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const double d0 = (double)__uint_as_float(wv[e] << 16) - (double)cf[2 * e];
            const double d1 = (double)__uint_as_float(wv[e] & 0xFFFF0000u) - (double)cf[2 * e + 1];
            s += d0 * d0;
            s += d1 * d1;
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
    const int ntile = (a.L + ATOK - 1) / ATOK;
    if (a.cent_in != nullptr)
        hipLaunchKernelGGL(km_init_from, dim3(a.k, BH), dim3(64), 0, st, a.cent_in, a.cent, D, a.k, a.kpad);
    else
        hipLaunchKernelGGL(km_init, dim3(a.k, BH), dim3(64), 0, st, v, a.cent, a.L, D, a.k, a.kpad, a.H,
                           a.seed);
    const int rounds = a.iters > 0 ? a.iters : 1;
    for (int it = 0; it < rounds; it++) {
        hipLaunchKernelGGL(km_split, dim3(a.kpad, BH), dim3(64), 0, st, a.cent, a.cent_hi, a.cent_lo,
                           a.cnorm, D, a.k, a.kpad);
        hipLaunchKernelGGL((km_assign<D>), dim3(ntile, BH), dim3(512), 0, st, v, a.cent_hi, a.cent_lo,
                           a.cnorm, a.assign, a.L, a.k, a.kpad);
        hipLaunchKernelGGL(km_chunk_count, dim3(a.nchunk, BH), dim3(CHUNK), a.k * sizeof(int), st,
                           a.assign, a.chunk_cnt, a.L, a.k, a.nchunk);
        hipLaunchKernelGGL(km_scan, dim3(BH), dim3(1024), 0, st, a.chunk_cnt, a.counts, a.offsets, a.k,
                           a.nchunk);
        hipLaunchKernelGGL(km_scatter, dim3(a.nchunk, BH), dim3(CHUNK), a.k * sizeof(int), st, a.assign,
                           a.chunk_cnt, a.perm, a.L, a.k, a.nchunk);
        if (a.iters > 0)
            hipLaunchKernelGGL((km_update<D>), dim3(a.k, BH), dim3(256), 0, st, v, a.perm, a.counts,
                               a.offsets, a.cent, a.L, a.k, a.kpad);
    }
    if (a.cent_out != nullptr)
        hipLaunchKernelGGL(km_copy_out, dim3(a.k, BH), dim3(64), 0, st, a.cent, a.cent_out, D, a.k, a.kpad);
    if (a.obj) {
        hipLaunchKernelGGL((km_objective<D>), dim3(a.nchunk, BH), dim3(256), 0, st, v, a.assign, a.cent,
                           a.obj_part, a.L, a.kpad, a.nchunk);
        hipLaunchKernelGGL(km_objective_final, dim3(BH), dim3(64), 0, st, a.obj_part, a.obj, a.nchunk);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kmeans(const KmeansArgs& a, hipStream_t st) {
    return a.d == 128 ? launch_kmeans_t<128>(a, st) : launch_kmeans_t<64>(a, st);
}

}  // namespace vc
