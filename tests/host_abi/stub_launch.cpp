// Host-only stand-ins for the kernel launchers, linked with the C ABI (fa_api.cpp) and
// the launch plans (fa_plan.cpp) into a library built with AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every launcher only counts the call, so the argument
// checks of every entry point can run on a machine without a GPU, and a test can see
// whether a call reached the launch stage.  Test infrastructure; never part of the
// product library.
#include <atomic>
#include <cstdint>

#include "../../exact_io_aware_20_amd/csrc/fa_launch.hpp"

namespace {
std::atomic<long long> g_launches{0};
hipError_t counted() {
    g_launches.fetch_add(1);
    return hipSuccess;
}
}  // namespace

namespace fa {
hipError_t launch_fwd_bf16(const FwdParams&, int, hipStream_t) { return counted(); }
hipError_t launch_fwd_f32(const FwdParams&, int, hipStream_t) { return counted(); }
hipError_t launch_decode(const DecodeParams&, int, int, bool, hipStream_t) { return counted(); }
hipError_t launch_bwd_pre(const BwdParams&, int, hipStream_t) { return counted(); }
hipError_t launch_bwd_dkdv(const BwdParams&, int, hipStream_t) { return counted(); }
hipError_t launch_bwd_dq(const BwdParams&, int, hipStream_t) { return counted(); }
hipError_t launch_bwd_dq_rows(const BwdParams&, int, hipStream_t) { return counted(); }
hipError_t launch_bwd_fused(const BwdParams&, int, hipStream_t) { return counted(); }
hipError_t launch_bwd_dq_convert(const BwdParams&, int, hipStream_t) { return counted(); }
// a fixed, aligned stand-in address (never dereferenced: the launchers are stand-ins)
hipError_t bwd_scratch(hipStream_t, float** ptr) {
    *ptr = reinterpret_cast<float*>(uintptr_t{0x7f0000000000});
    return hipSuccess;
}
}  // namespace fa

extern "C" long long fa_stub_launches() { return g_launches.load(); }
