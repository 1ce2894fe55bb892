// vc_attn_fp8.hip -- launchers of the fused VC-Attention forward (V-Smooth
// recipe) on the 32x32x64 wave of vc_attn_fp8w_kernel.hpp: one instance per
// head dim, output type, score dump, Skip Softmax and probability-byte path
// (ExpCast or exp-then-cast).
#include "vc_attn_fp8w_kernel.hpp"

namespace vc {

namespace {

template <int D, bool OB, bool DUMP>
hipError_t launch_s(const AttnArgs& a, hipStream_t st) {
    const bool skip = a.skip_thr > -INFINITY;
    if (a.prob_cast == 1)
        return skip ? launch_w32<D, OB, DUMP, true, true>(a, st)
                    : launch_w32<D, OB, DUMP, false, true>(a, st);
    return skip ? launch_w32<D, OB, DUMP, true, false>(a, st)
                : launch_w32<D, OB, DUMP, false, false>(a, st);
}

}  // namespace

hipError_t launch_attn_fp8(const AttnArgs& a, int d, int out_bf16, bool dump, hipStream_t st) {
    if (d == 128) {
        if (dump) return out_bf16 ? launch_s<128, true, true>(a, st) : launch_s<128, false, true>(a, st);
        return out_bf16 ? launch_s<128, true, false>(a, st) : launch_s<128, false, false>(a, st);
    }
    if (dump) return out_bf16 ? launch_s<64, true, true>(a, st) : launch_s<64, false, true>(a, st);
    return out_bf16 ? launch_s<64, true, false>(a, st) : launch_s<64, false, false>(a, st);
}

}  // namespace vc
