// Device tree metadata from parent arrays: depth, ancestor bitmask, position id.
// ("Tree attention mask for draft-tree verification", section "A strong answer": position
// id = prefix length + depth; node i sees j iff j is i or an ancestor.)
// One thread per (request, node); the parent walk is O(depth) and bounded by the node id.
#include "kernels_common.h"

namespace tv {

__global__ void __launch_bounds__(256) tv_meta_from_parent_kernel(
    const int32_t* __restrict__ parent, int32_t parent_sb, int32_t B, int32_t N,
    const int32_t* __restrict__ prefix_len, int32_t* __restrict__ depth,
    uint64_t* __restrict__ bitmask, int32_t* __restrict__ pos) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)B * N) return;
  const int b = (int)(gid / N);
  const int i = (int)(gid - (int64_t)b * N);
  const int32_t* par = parent + (int64_t)b * parent_sb;
  bool ok;
  int d;
  const uint64_t m = ancestor_bits(par, i, N, ok, d);
  const int L = prefix_len ? prefix_len[b] : 0;
  if (depth) depth[gid] = ok ? d : -1;
  if (bitmask) bitmask[gid] = ok ? m : 0ull;
  if (pos) pos[gid] = ok ? L + d : -1;
}

hipError_t launch_meta_from_parent(const int32_t* parent, int32_t parent_sb, int32_t B,
                                   int32_t N, const int32_t* prefix_len, int32_t* depth,
                                   uint64_t* bitmask, int32_t* pos, hipStream_t s) {
  const int64_t total = (int64_t)B * N;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(tv_meta_from_parent_kernel, dim3((unsigned)blocks), dim3(threads), 0, s,
                     parent, parent_sb, B, N, prefix_len, depth, bitmask, pos);
  return hipGetLastError();
}

}  // namespace tv
