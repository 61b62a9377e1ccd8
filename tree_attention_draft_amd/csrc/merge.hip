// Merge of split-KV partial results.
//
// A request's keys [0, L + N) are cut into chunks of `chunk` keys; split s produced, per
// packed row, the output normalised over its own keys (o_s) and its log2-domain
// log-sum-exp (lse_s, -inf when no key of the chunk was allowed).  The combined result is
//   lse = log2 sum_s 2^lse_s,   out = sum_s 2^(lse_s - lse) * o_s,
// i.e. the softmax over the union of the chunks.  Requests with fewer splits than the grid
// contribute only their own ceil((L + N) / chunk) partials; a request whose keys fit one
// chunk was written directly by the attention kernel and is skipped here.
// Each output row (request, kv head, packed row) takes P * D/4 threads: thread (sub, q4)
// owns 4 features and sums the partials of splits sub, sub + P, sub + 2P, ...; the P
// subtotals then combine through LDS.  P grows with the grid's split count (about four
// partials per thread), so a request split many ways is read by many threads at once
// rather than by one thread per feature group walking every split.  Within a thread the
// sum runs online over groups of partials (16 while that many remain, then one group of
// 16, 8 or 4 for the rest): all loads of a group are issued before any of them is used,
// and the running sum is moved to each group's max as it goes.
#include <type_traits>

#include "kernels_common.h"

namespace tv {

template <typename T, int D, int P>
__global__ void __launch_bounds__(256) tv_merge_kernel(AttnParams p) {
  constexpr int Q4 = D / 4;
  constexpr int RPW = 256 / (Q4 * P);  // rows per workgroup
  static_assert(RPW >= 1 && RPW * Q4 * P == 256, "thread layout");
  const int t = threadIdx.x;
  const int q4 = t % Q4;
  const int sub = (t / Q4) % P;
  const int64_t gr = (int64_t)blockIdx.x * RPW + t / (Q4 * P);  // (request, kv head, row)
  const int64_t rows = (int64_t)p.B * p.Hkv * p.R;
  const int row = (int)(gr % p.R);
  const int hkv = (int)((gr / p.R) % p.Hkv);
  const int b = (int)min<int64_t>(gr / p.R / p.Hkv, p.B - 1);
  const int Ttot = clamped_prefix(p, b) + p.N;
  // one split: the attention kernel wrote the final output (uniform over the row's threads)
  const int ns = gr < rows ? min(p.num_splits, (Ttot + p.chunk - 1) / p.chunk) : 0;

  const int64_t base = ((int64_t)b * p.Hkv + hkv) * p.num_splits;
  const int cnt = ns > 1 && ns > sub ? (ns - sub + P - 1) / P : 0;  // this thread's splits
  float mx = -INFINITY;  // max of the log-sum-exps seen so far
  float wsum = 0.f;      // sum of 2^(lse_s - mx) so far
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  auto group = [&](int i0, auto size_c) {
    constexpr int G = decltype(size_c)::value;
    float ls[G];
    f32x4 v[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      // past the thread's last split: re-read its last partial (in bounds), weight 0
      const int64_t prow = (base + sub + (int64_t)P * min(i0 + u, cnt - 1)) * p.R + row;
      const float l = p.ws_lse[prow];
      ls[u] = i0 + u < cnt ? l : -INFINITY;
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
  int i0 = 0;
  for (; i0 + 16 <= cnt; i0 += 16) group(i0, std::integral_constant<int, 16>{});
  // the rest in one group sized to it (its surplus slots re-read the last partial)
  const int rest = cnt - i0;
  if (rest > 8)
    group(i0, std::integral_constant<int, 16>{});
  else if (rest > 4)
    group(i0, std::integral_constant<int, 8>{});
  else if (rest > 0)
    group(i0, std::integral_constant<int, 4>{});

  if constexpr (P > 1) {
    // subtotals of the row's P thread groups, combined by sub = 0
    __shared__ float sm[256], sw[256];
    __shared__ f32x4 sa[256];
    sm[t] = mx;
    sw[t] = wsum;
    sa[t] = acc;
    __syncthreads();
    if (sub != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < P; ++u) M = fmaxf(M, sm[t + u * Q4]);
    wsum = 0.f;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const float mu = sm[t + u * Q4];
        const float sc = mu == -INFINITY ? 0.f : exp2f(mu - M);
        wsum += sw[t + u * Q4] * sc;
        acc += sa[t + u * Q4] * sc;
      }
    }
    mx = M;
  }
  if (ns <= 1) return;
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

template <typename T, int D>
static hipError_t launch_merge_p(const AttnParams& p, hipStream_t s) {
  // thread groups per row: about four partials per thread, at most 8
  int P = 1;
  while (P < 8 && 8 * P <= p.num_splits) P *= 2;
  const int64_t rows = (int64_t)p.B * p.Hkv * p.R;
  const int64_t rpw = 256 / (D / 4 * P);
  const unsigned blocks = (unsigned)((rows + rpw - 1) / rpw);
  switch (P) {
    case 1: hipLaunchKernelGGL((tv_merge_kernel<T, D, 1>), dim3(blocks), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((tv_merge_kernel<T, D, 2>), dim3(blocks), dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((tv_merge_kernel<T, D, 4>), dim3(blocks), dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((tv_merge_kernel<T, D, 8>), dim3(blocks), dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const AttnParams& p, int D, bool bf16, hipStream_t s) {
  if (bf16) return D == 64 ? launch_merge_p<uint16_t, 64>(p, s) : launch_merge_p<uint16_t, 128>(p, s);
  return D == 64 ? launch_merge_p<float, 64>(p, s) : launch_merge_p<float, 128>(p, s);
}

}  // namespace tv
