// Tree-verify attention, MFMA path: the launch entry point and the contiguous-KV
// instantiations of the kernel (the kernel itself is in attn_mfma.h; the paged-KV
// instantiations are built in attn_mfma_paged.hip).
#include "attn_mfma.h"

namespace tv {

hipError_t launch_attn_mfma(const AttnParams& p, int D, MfmaShape shape, hipStream_t s) {
  return p.paged ? launch_attn_mfma_paged(p, D, shape, s)
                 : launch_attn_mfma_layout<false>(p, D, shape, s);
}

}  // namespace tv
