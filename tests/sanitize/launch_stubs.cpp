// Link-only stand-ins for the kernel launchers, so that the C ABI's
// argument validation (attn_api.cpp) can be built and run on the host alone
// under AddressSanitizer and UndefinedBehaviorSanitizer.  The checks drive
// only calls that fail validation or have nothing to do, which return
// before any launcher; if one is reached anyway, it reports a launch
// failure instead of touching a GPU.
#include "attn_launch.h"

namespace attn {

int fwd_block_rows() { return 128; }
hipError_t launch_fwd(const FwdArgs&, int, bool, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_fp8(const FwdArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_once(const FwdArgs&, int, bool, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fwd_fp8_once(const FwdArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
size_t fwd_split_workspace_bytes(int64_t BH, int64_t N, int64_t d, int nsplit) {
    return size_t(nsplit) * size_t(BH) * size_t(N) * size_t(d + 1) * 4;
}
hipError_t launch_fwd_merge(const float*, const float*, void*, float*, int64_t, int, size_t, size_t, int,
                            int, bool, hipStream_t) {
    return hipErrorNotSupported;
}
size_t bwd_workspace_bytes(int64_t BH, int64_t N) {
    return size_t(2) * size_t(BH) * size_t((N + 63) / 64 * 64) * sizeof(float);
}
hipError_t bwd_scratch(void**) { return hipErrorNotSupported; }
hipError_t launch_bwd(const BwdArgs&, int, int, bool, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_std_scores(const void*, const void*, float*, int64_t, int, int, float, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_std_softmax(const float*, void*, float*, int64_t, int, int, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_std_pv(const void*, const void*, void*, int64_t, int, int, int, bool, hipStream_t) {
    return hipErrorNotSupported;
}

hipError_t launch_mfma_probe(float*, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_hbm_probe(const void*, long long, unsigned*, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace attn
