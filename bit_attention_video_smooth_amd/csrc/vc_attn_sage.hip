// vc_attn_sage.hip -- launchers of the SAGE-style quantised attention
// (TensorRT-LLM blog, "Quantized Attention": one Q scale per query token,
// one K scale per 16 keys, INT8 or FP8 QK^T, FP8 PV with one V scale per
// channel) built from the kernel template in vc_attn_fp8_kernel.hpp.  No
// Skip Softmax instances: the baseline runs dense.
#include "vc_attn_fp8_kernel.hpp"

namespace vc {

namespace {

template <int D, bool OB, bool DUMP, int MODE>
hipError_t launch_p(const AttnArgs& a, hipStream_t st) {
    return a.prob_cast == 1 ? launch_t<D, OB, DUMP, false, true, MODE>(a, st)
                            : launch_t<D, OB, DUMP, false, false, MODE>(a, st);
}

template <int D, bool OB, bool DUMP>
hipError_t launch_m(const AttnArgs& a, bool qk_int8, hipStream_t st) {
    return qk_int8 ? launch_p<D, OB, DUMP, REC_SAGE_I8>(a, st) : launch_p<D, OB, DUMP, REC_SAGE_F8>(a, st);
}

}  // namespace

hipError_t launch_attn_sage(const AttnArgs& a, int d, int out_bf16, bool dump, bool qk_int8, hipStream_t st) {
    if (d == 128) {
        if (dump)
            return out_bf16 ? launch_m<128, true, true>(a, qk_int8, st) : launch_m<128, false, true>(a, qk_int8, st);
        return out_bf16 ? launch_m<128, true, false>(a, qk_int8, st) : launch_m<128, false, false>(a, qk_int8, st);
    }
    if (dump) return out_bf16 ? launch_m<64, true, true>(a, qk_int8, st) : launch_m<64, false, true>(a, qk_int8, st);
    return out_bf16 ? launch_m<64, true, false>(a, qk_int8, st) : launch_m<64, false, false>(a, qk_int8, st);
}

}  // namespace vc
