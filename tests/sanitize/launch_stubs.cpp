// Launcher stand-ins for the sanitizer build of the ABI's host code
// (tests/sanitize/abi_driver.cpp): the driver only walks argument-check
// failures, which return before any launch, so every launcher reports
// "not supported" if it is ever reached.
#include "vc_internal.hpp"

namespace vc {
hipError_t launch_copy_perm(const int32_t*, int32_t*, size_t, double*, size_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prepare_quant(const PrepareArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_k_mean(const void*, double*, float*, int, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_sage_prepare(const SageArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_kmeans(const KmeansArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_fp8(const AttnArgs&, int, int, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_fp4v(const AttnArgs&, int, int, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_sage(const AttnArgs&, int, int, bool, bool, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_attn_bf16(const AttnBf16Args&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_debug_expcast(const float*, const float*, const float*, int64_t, uint8_t*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_debug_e4m3(const float*, int64_t, uint8_t*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_debug_mfma_fp8(const uint8_t*, const uint8_t*, float*, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_debug_mfma_rate(int, int, float*, hipStream_t) { return hipErrorNotSupported; }
}  // namespace vc
