// Tree-verify attention, MFMA path: the paged-KV instantiations of the kernel in
// attn_mfma.h (a translation unit of their own, so the two layouts build in parallel).
#include "attn_mfma.h"

namespace tv {

hipError_t launch_attn_mfma_paged(const AttnParams& p, int D, MfmaShape shape, hipStream_t s) {
  return launch_attn_mfma_layout<true>(p, D, shape, s);
}

}  // namespace tv
