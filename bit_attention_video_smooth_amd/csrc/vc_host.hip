// vc_host.hip -- host-side sizes and workspace layout of the prepare stage
// (no device code): how many partial sums the K column mean takes per head,
// and the k-means workspace (centroids with their BF16 high/low parts and
// norms, the assignment, cluster counts and offsets, the counting sort's
// per-chunk histograms, the objective's partial sums), each region aligned
// to 256 bytes.
#include "vc_internal.hpp"

namespace vc {

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int k_mean_splits(int BH, int L) {
    int by_len = (L + 1023) / 1024;
    int want = (2048 + BH - 1) / BH;
    int s = by_len < want ? by_len : want;
    return s < 1 ? 1 : s;
}

size_t kmeans_workspace_bytes(int B, int H, int L, int d, int k) {
    const size_t BH = (size_t)B * H;
    const size_t kpad = ((size_t)k + KMEANS_KT - 1) / KMEANS_KT * KMEANS_KT;
    const size_t nchunk = ((size_t)L + KMEANS_CHUNK - 1) / KMEANS_CHUNK;
    size_t s = 0;
    s += align256(BH * kpad * d * 4);       // cent
    s += 2 * align256(BH * kpad * d * 2);   // bf16 high and low parts
    s += align256(BH * kpad * 4);           // cnorm
    s += align256(BH * L * 4);              // assign
    s += 2 * align256(BH * k * 4);          // counts, offsets
    s += align256(BH * nchunk * k * 4);     // chunk counts
    s += align256(BH * nchunk * 8);         // objective partials
    return s;
}

void kmeans_carve(KmeansArgs& a, void* ws) {
    const size_t BH = (size_t)a.B * a.H;
    a.kpad = (a.k + KMEANS_KT - 1) / KMEANS_KT * KMEANS_KT;
    a.nchunk = (a.L + KMEANS_CHUNK - 1) / KMEANS_CHUNK;
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

}  // namespace vc
