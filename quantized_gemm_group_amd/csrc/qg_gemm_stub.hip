// Placeholder launchers for the GEMM kernels not built yet.
#include "qg_internal.hpp"

namespace qg {
hipError_t launch_gemm_w4a16(bool, const void*, int64_t, const void*, const void*, const void*,
                             int64_t, int64_t, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm_fp8(const void*, const void*, int64_t, const void*, const void*, int64_t,
                           int64_t, void*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm_int8(bool, bool, const void*, const void*, const void*, int64_t,
                            const void*, const void*, const void*, int64_t, int64_t, void*,
                            hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_mx_gemm(const void*, const void*, int64_t, const void*, const void*, int64_t,
                          int64_t, void*, hipStream_t) { return hipErrorNotSupported; }
}  // namespace qg
