// Merge of split-KV partial results.
//
// A request's keys [0, L + N) are cut into chunks of `chunk` keys; split s produced, per
// packed row, the output normalised over its own keys (o_s) and its log2-domain
// log-sum-exp (lse_s, -inf when no key of the chunk was allowed).  The combined result is
//   lse = log2 sum_s 2^lse_s,   out = sum_s 2^(lse_s - lse) * o_s,
// i.e. the softmax over the union of the chunks.  Requests with fewer splits than the grid
// contribute only their own ceil((L + N) / chunk) partials; a request whose keys fit one
// chunk was written directly by the attention kernel and is skipped here.
// One thread per (request, kv head, packed row, 4 features).  The sum runs online over
// groups of partials (16 while that many remain, then 4): all loads of a group are issued
// before any of them is used (a thread walking many splits one at a time would wait a
// memory round trip per split), and the running sum is moved to each group's max as it
// goes.
#include <type_traits>

#include "kernels_common.h"

namespace tv {

template <typename T, int D>
__global__ void __launch_bounds__(256) tv_merge_kernel(AttnParams p) {
  constexpr int Q4 = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.B * p.Hkv * p.R * Q4;
  if (gid >= total) return;
  const int q4 = (int)(gid % Q4);
  int64_t rest = gid / Q4;
  const int row = (int)(rest % p.R);
  rest /= p.R;
  const int hkv = (int)(rest % p.Hkv);
  const int b = (int)(rest / p.Hkv);
  const int Ttot = clamped_prefix(p, b) + p.N;
  const int ns = min(p.num_splits, (Ttot + p.chunk - 1) / p.chunk);
  if (ns <= 1) return;  // one split: the attention kernel wrote the final output

  const int64_t base = ((int64_t)b * p.Hkv + hkv) * p.num_splits;
  float mx = -INFINITY;  // max of the log-sum-exps seen so far
  float wsum = 0.f;      // sum of 2^(lse_s - mx) so far
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  auto group = [&](int s0, auto size_c) {
    constexpr int G = decltype(size_c)::value;
    float ls[G];
    f32x4 v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      // past the last split: re-read the last partial (in bounds) and give it no weight
      const int64_t prow = (base + min(s0 + u, ns - 1)) * p.R + row;
      const float l = p.ws_lse[prow];
      ls[u] = s0 + u < ns ? l : -INFINITY;
      v[u] = *reinterpret_cast<const f32x4*>(p.ws_o + prow * D + 4 * q4);
    }
    float mg = mx;
#pragma unroll
    for (int u = 0; u < G; ++u) mg = fmaxf(mg, ls[u]);
    if (mg == -INFINITY) return;  // no allowed key in any chunk so far
    const float sc = exp2f(mx - mg);  // 0 while mx is still -inf
    wsum *= sc;
    acc *= sc;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      // a chunk with no allowed key (lse -inf) weighs 0
      const float wgt = ls[u] == -INFINITY ? 0.f : exp2f(ls[u] - mg);
      wsum += wgt;
      acc += v[u] * wgt;
    }
    mx = mg;
  };
  int s0 = 0;
  for (; s0 + 16 <= ns; s0 += 16) group(s0, std::integral_constant<int, 16>{});
  for (; s0 < ns; s0 += 4) group(s0, std::integral_constant<int, 4>{});
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int node = row / p.g, head = hkv * p.g + row % p.g;
  T* out = static_cast<T*>(p.out) + (int64_t)b * p.o_sb + (int64_t)node * p.o_sn +
           (int64_t)head * p.o_sh + 4 * q4;
  if constexpr (sizeof(T) == 2) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = static_cast<__bf16>(acc[i] * inv);
    *reinterpret_cast<bf16x4*>(out) = v;
  } else {
    *reinterpret_cast<f32x4*>(out) = acc * inv;
  }
  if (q4 == 0 && p.lse) {
    const float lse2 = wsum > 0.f ? mx + log2f(wsum) : -INFINITY;
    p.lse[((int64_t)b * p.N + node) * p.Hq + head] = lse2 * kLn2;
  }
}

hipError_t launch_merge(const AttnParams& p, int D, bool bf16, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.Hkv * p.R * (D / 4);
  const int threads = 256;
  const unsigned blocks = (unsigned)((total + threads - 1) / threads);
  if (bf16) {
    if (D == 64) hipLaunchKernelGGL((tv_merge_kernel<uint16_t, 64>), dim3(blocks), dim3(threads), 0, s, p);
    else hipLaunchKernelGGL((tv_merge_kernel<uint16_t, 128>), dim3(blocks), dim3(threads), 0, s, p);
  } else {
    if (D == 64) hipLaunchKernelGGL((tv_merge_kernel<float, 64>), dim3(blocks), dim3(threads), 0, s, p);
    else hipLaunchKernelGGL((tv_merge_kernel<float, 128>), dim3(blocks), dim3(threads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace tv
