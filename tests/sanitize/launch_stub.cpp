// Host-only stand-ins for the kernel launchers of the attention library, so
// that the C-ABI layer (api.cpp: argument validation, sizing, error mapping)
// can be built alone with AddressSanitizer and UndefinedBehaviorSanitizer
// and exercised on a machine without a GPU.  Every launch reports that no
// device is present; no test of the validation layer expects a launch to
// succeed.  The check-mode pass is the exception: it evaluates the library's
// own rules (check_rules.hpp) on the host, so that with HOST pointers in place
// of device ones the gate in front of every launch can be exercised on the
// CPU.  Test infrastructure only.
#include <cmath>
#include <cstdint>

#include "../../global_attention_mimo_amd/csrc/check_rules.hpp"
#include "../../global_attention_mimo_amd/csrc/launch.hpp"

namespace {
uint32_t g_sticky = 0;
}

namespace mimo {
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_chunk(const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_swa(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_ga(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_append(const AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_backward(const BackwardArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_rope(const RopeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_rope_prep(const RopePrepArgs&, hipStream_t) { return hipErrorNoDevice; }
RopeFreq rope_inv_freq(double theta, int rd) {
    RopeFreq f{};
    for (int i = 0; i < rd / 2 && i < 96; ++i) f.f[i] = std::pow(theta, -2.0 * i / rd);
    return f;
}
hipError_t run_check(const CheckArgs& a, hipStream_t, bool* gated, uint32_t* bits) {
    *bits = check_rules(a, 0, 1);
    *gated = true;
    g_sticky |= *bits;
    return hipSuccess;
}
hipError_t check_flags(uint32_t* bits, bool clear) {
    *bits = g_sticky;
    if (clear) g_sticky = 0;
    return hipSuccess;
}
hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    return hipErrorNoDevice;
}
}  // namespace mimo
