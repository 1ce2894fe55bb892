// vc_attn_fp4.hip -- launchers of the 4-bit V-Smooth attention (MarkTechPost
// abstract: 4-bit V-Smooth; ExpCast applies to the 8-bit kernel only, so the
// probabilities come by exp-then-cast): E2M1 V residual and probabilities
// with power-of-two scales per 32-key group on the scaled FP4 matrix cores,
// FP8 per-block Q/K, exact block means.  Built from the kernel template in
// vc_attn_fp8_kernel.hpp; no Skip Softmax instances.
#include "vc_attn_fp8_kernel.hpp"

namespace vc {

namespace {

template <int D, bool OB>
hipError_t launch_d(const AttnArgs& a, bool dump, hipStream_t st) {
    return dump ? launch_t<D, OB, true, false, true, REC_VC4>(a, st) : launch_t<D, OB, false, false, true, REC_VC4>(a, st);
}

}  // namespace

hipError_t launch_attn_fp4v(const AttnArgs& a, int d, int out_bf16, bool dump, hipStream_t st) {
    if (d == 128) return out_bf16 ? launch_d<128, true>(a, dump, st) : launch_d<128, false>(a, dump, st);
    return out_bf16 ? launch_d<64, true>(a, dump, st) : launch_d<64, false>(a, dump, st);
}

}  // namespace vc
