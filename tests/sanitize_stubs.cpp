// Stand-ins for the kernel launchers of libtreeverify, for the CPU-only build of the host
// C++ under AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitized_host.py).
// The host entry points run their argument checks, plans and builders exactly as in the
// real library; a launch reports that no device is present.
#include <hip/hip_runtime_api.h>

#include "tv_internal.h"

namespace tv {
hipError_t launch_attn_mfma(const AttnParams&, int, MfmaShape, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_valu(const AttnParams&, int, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_merge(const AttnParams&, int, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_meta_from_parent(const int32_t*, int32_t, int32_t, int32_t, const int32_t*,
                                   int32_t*, uint64_t*, int32_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_argmax(const AcceptParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_compact(const CompactParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_stochastic_walk(const SampleParams&, hipStream_t) { return hipErrorNoDevice; }
}  // namespace tv

// The no-allocation entry point without its device array: the same checks, plan and size
// limit; where the real one would look the array up on the device, no device is present.
namespace {
struct NoDeviceScratch final : tv::WorkspaceSource {
  tv_status get(size_t bytes, void** ptr) const override {
    *ptr = nullptr;
    if (bytes > TV_STATIC_SCRATCH_BYTES)
      return tv::fail(TV_ERR_WORKSPACE, "split workspace exceeds the static scratch");
    return tv::fail(TV_ERR_HIP, "no device");
  }
};
}  // namespace

extern "C" tv_status tree_verify_attn_static(const tv_attn_args* a, hipStream_t stream) {
  return tv::attn_pass(a, NoDeviceScratch(), stream);
}
