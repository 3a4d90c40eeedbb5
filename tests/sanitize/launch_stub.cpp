// Host-only stand-ins for the kernel launchers of the attention library, so
// that the C-ABI layer (api.cpp: argument validation, sizing, error mapping)
// can be built alone with AddressSanitizer and UndefinedBehaviorSanitizer
// and exercised on a machine without a GPU.  Every launch reports that no
// device is present; no test of the validation layer expects a launch to
// succeed.  Test infrastructure only.
#include "../../global_attention_mimo_amd/csrc/launch.hpp"

namespace mimo {
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_chunk(const PrefillArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_swa(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_ga(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_append(const AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_backward(const BackwardArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_rope(const RopeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_rope_prep(const RopePrepArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch(void** ptr) {
    *ptr = nullptr;
    return hipErrorNoDevice;
}
}  // namespace mimo
