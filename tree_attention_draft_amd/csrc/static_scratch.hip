// tree_verify_attn_static: the verification pass for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// It runs exactly what tree_verify_attn runs -- same checks, same split plan, same
// kernels -- but when the plan splits a request's keys, the partial results go to a
// fixed device array of this library instead of the caller's workspace argument, so the
// call allocates nothing.  The array is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy (TV_STATIC_SCRATCH_BYTES) from module load until the
// process ends.  In host code the variable's name is only a host-side stand-in, so its
// device address is looked up once per device (hipGetSymbolAddress, with that device
// current) and that address is what the kernels receive.
//
// Every call on a device shares that device's array and leaves its last contents there.
// The split partials need no initial value (each workgroup writes its own slots before
// the merge kernel reads them, on the same stream), so nothing is cleared.  Calls whose
// work overlaps on one device (different streams, or different host threads without
// ordering) race on the array; callers order them.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "tree_verify.h"
#include "tv_internal.h"

namespace {

static_assert(TV_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[TV_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];            // device address of `scratch` on each device
hipError_t g_err[kMaxDevices];       // result of that device's lookup

// Device address of this device's copy of `scratch` (looked up on the first call made with
// the device current; later calls reuse it).
tv_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return tv::fail(TV_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return tv::fail(TV_ERR_UNSUPPORTED, "device index beyond the static scratch table");
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return tv::fail(TV_ERR_HIP, hipGetErrorString(g_err[dev]));
  *out = g_ptr[dev];
  return TV_OK;
}

struct StaticWorkspace final : tv::WorkspaceSource {
  tv_status get(size_t bytes, void** ptr) const override {
    if (bytes > TV_STATIC_SCRATCH_BYTES) {
      static thread_local char msg[160];
      std::snprintf(msg, sizeof(msg),
                    "split workspace of %zu bytes exceeds the static scratch of %d bytes; "
                    "pass a smaller num_splits (1 needs none)",
                    bytes, TV_STATIC_SCRATCH_BYTES);
      return tv::fail(TV_ERR_WORKSPACE, msg);
    }
    return scratch_address(ptr);
  }
};

}  // namespace

extern "C" tv_status tree_verify_attn_static(const tv_attn_args* a, hipStream_t stream) {
  return tv::attn_pass(a, StaticWorkspace(), stream);
}
