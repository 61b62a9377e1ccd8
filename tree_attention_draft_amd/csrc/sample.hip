// Stochastic (temperature > 0) verification of the draft tree: the walk from the root in
// which each child is accepted with probability min(1, r(x) / q(x)) and every rejection
// replaces r by the normalised residual max(0, r - q) before the next sibling is judged
// ("Implement a batched speculative sampling verifier", "A strong answer" and "What
// interviewers probe next"; "Tree Verification", "Accepting on a Tree").
//
// One 1024-thread workgroup per request walks its tree.  The distribution r a sibling is
// judged against is never stored: after k applied rejections it is, per vocabulary entry,
//   r_0 = p,  r_{j+1} = max(r_j / z_j - q, 0),
// with z_j the total of r_j, so every test costs one pass over the node's p and q rows
// (the total of the residual a rejection leaves is the next test's z) and the final draw
// two.  All arithmetic is float64, every reduction in one fixed order per launch shape.
#include <climits>

#include "kernels_common.h"

namespace tv {
namespace {

constexpr int kWalkThreads = 1024;
constexpr int kWalkWaves = kWalkThreads / 64;

// Sum over the workgroup; every thread receives the same total.
__device__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();  // `red` is free: every thread has read its previous contents
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kWalkWaves; ++i) t += red[i];
  return t;
}

// Minimum (or maximum) over the workgroup; every thread receives it.
template <bool MIN>
__device__ int block_extreme(int v, int* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int o = __shfl_xor(v, off);
    v = MIN ? min(v, o) : max(v, o);
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = red[0];
#pragma unroll
  for (int i = 1; i < kWalkWaves; ++i) t = MIN ? min(t, red[i]) : max(t, red[i]);
  return t;
}

// r_k at one vocabulary entry from its p and q values and the k divisors applied so far.
__device__ inline double residual_at(float pv, float qv, const double* zs, int levels) {
  double r = static_cast<double>(pv);
  const double qd = static_cast<double>(qv);
  for (int j = 0; j < levels; ++j) r = fmax(r / zs[j] - qd, 0.0);
  return r;
}

__global__ void __launch_bounds__(kWalkThreads) tv_stochastic_walk_kernel(SampleParams P) {
  __shared__ int32_t par[TV_MAX_NODES], tok[TV_MAX_NODES];
  __shared__ int32_t acc[TV_MAX_NODES], em[TV_MAX_NODES];
  __shared__ double zs[TV_MAX_NODES];  // divisors of the current node's applied rejections
  __shared__ double red[kWalkWaves];
  __shared__ int ired[kWalkWaves];
  __shared__ double scan[kWalkThreads];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int N = P.N, V = P.V;
  if (tid < N) {
    par[tid] = P.parent[(int64_t)b * P.parent_sb + tid];
    tok[tid] = P.tokens[(int64_t)b * P.tokens_sb + tid];
    acc[tid] = -1;
    em[tid] = -1;
  }
  const double* u = P.uniform + (int64_t)b * P.uniform_sb;
  __syncthreads();

  // Every thread runs the same control flow: node, counts and decisions are derived from
  // workgroup-wide totals and LDS, so they agree across the workgroup.
  int node = 0, a = 0;
  for (int step = 0; step < N; ++step) {
    const float* prow = P.p + (int64_t)b * P.p_sb + (int64_t)node * P.p_sn;
    const float* qrow = P.q + (int64_t)b * P.q_sb + (int64_t)node * P.q_sn;
    int levels = 0;
    double part = 0.0;
#pragma unroll 8
    for (int v = tid; v < V; v += kWalkThreads) part += static_cast<double>(prow[v]);
    double z = block_sum(part, red);  // total of r_0 = p
    int taken = -1;
    for (int c = node + 1; c < N; ++c) {
      if (par[c] != node) continue;
      const int x = tok[c];
      if (x < 0 || x >= V) continue;  // not a vocabulary entry: never accepted
      const double rx = residual_at(prow[x], qrow[x], zs, levels);
      if (u[c] * static_cast<double>(qrow[x]) * z < rx) {
        taken = c;
        break;
      }
      // rejected: the residual's total decides whether it replaces r
      double m = 0.0;
#pragma unroll 4
      for (int v = tid; v < V; v += kWalkThreads)
        m += fmax(residual_at(prow[v], qrow[v], zs, levels) / z - static_cast<double>(qrow[v]),
                  0.0);
      m = block_sum(m, red);
      if (m > 0.0) {
        __syncthreads();  // every thread is done reading zs[0 .. levels)
        if (tid == 0) zs[levels] = z;
        __syncthreads();
        ++levels;
        z = m;
      }
    }
    if (tid == 0) acc[a] = node;
    if (taken >= 0) {
      if (tid == 0) em[a] = tok[taken];
      ++a;
      node = taken;
      continue;
    }
    // ---- final draw from r by inverse CDF: thread tid owns a contiguous chunk ----
    const int chunk = (V + kWalkThreads - 1) / kWalkThreads;
    const int v0 = min(V, tid * chunk), v1 = min(V, v0 + chunk);
    double s = 0.0;
    int lastpos = -1;
    for (int v = v0; v < v1; ++v) {
      const double r = residual_at(prow[v], qrow[v], zs, levels);
      s += r;
      if (r > 0.0) lastpos = v;
    }
    __syncthreads();
    scan[tid] = s;
    __syncthreads();
    // inclusive scan of the chunk totals (Hillis-Steele, fixed order)
    for (int off = 1; off < kWalkThreads; off <<= 1) {
      const double add = tid >= off ? scan[tid - off] : 0.0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const double total = scan[kWalkThreads - 1];
    const double thresh = u[0] * total;
    double run = tid > 0 ? scan[tid - 1] : 0.0;
    int first = INT_MAX;
    for (int v = v0; v < v1; ++v) {
      run += residual_at(prow[v], qrow[v], zs, levels);
      if (run > thresh) {
        first = v;
        break;
      }
    }
    first = block_extreme<true>(first, ired);
    lastpos = block_extreme<false>(lastpos, ired);
    if (tid == 0) em[a] = first != INT_MAX ? first : lastpos;
    ++a;
    break;
  }
  __syncthreads();
  if (tid < N) {
    P.accepted[(int64_t)b * N + tid] = acc[tid];
    P.emitted[(int64_t)b * N + tid] = em[tid];
  }
  if (tid == 0) P.num_accepted[b] = a;
}

}  // namespace

hipError_t launch_stochastic_walk(const SampleParams& p, hipStream_t s) {
  hipLaunchKernelGGL(tv_stochastic_walk_kernel, dim3(p.B), dim3(kWalkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace tv
