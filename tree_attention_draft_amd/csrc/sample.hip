// Stochastic (temperature > 0) verification of the draft tree: the walk from the root in
// which each child is accepted with probability min(1, r(x) / q(x)) and every rejection
// replaces r by the normalised residual max(0, r - q) before the next sibling is judged
// ("Implement a batched speculative sampling verifier", "A strong answer" and "What
// interviewers probe next"; "Tree Verification", "Accepting on a Tree").
//
// One 1024-thread workgroup per request walks its tree.  The distribution r a sibling is
// judged against is never stored.  With r_0 = p and r_{j+1} = max(r_j / z_j - q, 0), z_j
// the total of r_j, the residual after k applied rejections is, up to a positive scale,
//   R_k = max(p - S_k q, 0),   S_k = Z_0 + ... + Z_{k-1},   Z_j the total of R_j
// (R_{j+1} = max(R_j - Z_j q, 0) is z_0...z_j times r_{j+1}, and an entry once clipped to
// zero stays there), and every use of r is scale-free: a child x is accepted when
// u q(x) Z_k < R_k(x), and the final draw takes the first entry whose running sum of R_k
// exceeds u Z_k.  So a test costs one pass over the node's p and q rows with one fma per
// entry (the total of the residual a rejection leaves is the next test's Z) and the final
// draw two.  All arithmetic is float64, every reduction in one fixed order per launch
// shape; the closed form rounds differently from the iterated one only in the last bits,
// the order of the differences the summation order already makes.
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

// R_k at one vocabulary entry from its p and q values and S_k (p itself before any
// rejection has been applied).
__device__ inline double residual_at(float pv, float qv, double S, int levels) {
  const double pd = static_cast<double>(pv);
  return levels == 0 ? pd : fmax(fma(-S, static_cast<double>(qv), pd), 0.0);
}

// Loads per thread issued together before any of them is used.
constexpr int kBatch = 8;
constexpr int kDraw = 8;  // consecutive entries per thread in the final draw's tiles

constexpr int kGroups = 4;  // 16-byte groups per thread issued together (aligned rows)

// This thread's sum of f(p[v], q[v]) over its share of the row, in a fixed order: aligned
// rows (VEC) by groups of four entries, g = tid, tid + 1024, ..., then the tail entries
// past the last whole group; otherwise v = tid, tid + 1024, ...
template <bool VEC, bool NEED_Q, class F>
__device__ double strided_sum(const float* prow, const float* qrow, int V, F f) {
  double acc = 0.0;
  if constexpr (VEC) {
    const int V4 = V >> 2;
    const float4* p4 = reinterpret_cast<const float4*>(prow);
    const float4* q4 = reinterpret_cast<const float4*>(qrow);
    for (int base = threadIdx.x; base < V4; base += kWalkThreads * kGroups) {
      float4 pv[kGroups], qv[kGroups];
#pragma unroll
      for (int i = 0; i < kGroups; ++i) {
        const int g = base + i * kWalkThreads;
        pv[i] = g < V4 ? p4[g] : make_float4(0.f, 0.f, 0.f, 0.f);
        qv[i] = NEED_Q && g < V4 ? q4[g] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < kGroups; ++i)
        if (base + i * kWalkThreads < V4) {
          acc += f(pv[i].x, qv[i].x);
          acc += f(pv[i].y, qv[i].y);
          acc += f(pv[i].z, qv[i].z);
          acc += f(pv[i].w, qv[i].w);
        }
    }
    const int v = 4 * V4 + (int)threadIdx.x;
    if (v < V) acc += f(prow[v], NEED_Q ? qrow[v] : 0.f);
    return acc;
  }
  for (int base = threadIdx.x; base < V; base += kWalkThreads * kBatch) {
    float pv[kBatch], qv[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int v = base + i * kWalkThreads;
      pv[i] = v < V ? prow[v] : 0.f;
      qv[i] = NEED_Q && v < V ? qrow[v] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (base + i * kWalkThreads < V) acc += f(pv[i], qv[i]);
  }
  return acc;
}

template <bool VEC>
__global__ void __launch_bounds__(kWalkThreads) tv_stochastic_walk_kernel(SampleParams P) {
  __shared__ int32_t par[TV_MAX_NODES], tok[TV_MAX_NODES];
  __shared__ int32_t acc[TV_MAX_NODES], em[TV_MAX_NODES];
  __shared__ double red[kWalkWaves];
  __shared__ int ired[kWalkWaves];
  __shared__ double scan[kWalkWaves];
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
    double S = 0.0;  // sum of the applied rejections' totals
    double z = block_sum(strided_sum<VEC, false>(prow, qrow, V,
                                            [](float pv, float) { return static_cast<double>(pv); }),
                         red);  // total of r_0 = p
    int taken = -1;
    for (int c = node + 1; c < N; ++c) {
      if (par[c] != node) continue;
      const int x = tok[c];
      if (x < 0 || x >= V) continue;  // not a vocabulary entry: never accepted
      const double rx = residual_at(prow[x], qrow[x], S, levels);
      if (u[c] * static_cast<double>(qrow[x]) * z < rx) {
        taken = c;
        break;
      }
      // rejected: the residual's total decides whether it replaces r
      const double S1 = S + z;
      const double m = block_sum(
          strided_sum<VEC, true>(prow, qrow, V,
                            [&](float pv, float qv) {
                              return fmax(fma(-S1, static_cast<double>(qv),
                                              static_cast<double>(pv)),
                                          0.0);
                            }),
          red);
      if (m > 0.0) {
        S = S1;
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
    // ---- final draw from r by inverse CDF.  z is r's total; the running sum is walked
    // in tiles of kDraw * 1024 consecutive entries (kDraw per thread, loads coalesced),
    // each scanned across the workgroup, until the tile where it exceeds z * uniform[0] ----
    const double thresh = u[0] * z;
    double base = 0.0;  // running sum before the current tile
    int first = INT_MAX, lastpos = -1;
    for (int t0 = 0; t0 < V; t0 += kWalkThreads * kDraw) {
      const int v0 = t0 + tid * kDraw;
      float pv[kDraw], qv[kDraw];
      if (VEC && v0 + kDraw <= V) {  // two 16-byte loads per row (v0 is a multiple of 8)
        static_assert(kDraw == 8, "draw chunk of two 16-byte groups");
        const float4 pa = *reinterpret_cast<const float4*>(prow + v0);
        const float4 pb = *reinterpret_cast<const float4*>(prow + v0 + 4);
        pv[0] = pa.x; pv[1] = pa.y; pv[2] = pa.z; pv[3] = pa.w;
        pv[4] = pb.x; pv[5] = pb.y; pv[6] = pb.z; pv[7] = pb.w;
        if (levels > 0) {
          const float4 qa = *reinterpret_cast<const float4*>(qrow + v0);
          const float4 qb = *reinterpret_cast<const float4*>(qrow + v0 + 4);
          qv[0] = qa.x; qv[1] = qa.y; qv[2] = qa.z; qv[3] = qa.w;
          qv[4] = qb.x; qv[5] = qb.y; qv[6] = qb.z; qv[7] = qb.w;
        } else {
#pragma unroll
          for (int i = 0; i < kDraw; ++i) qv[i] = 0.f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kDraw; ++i) {
          pv[i] = v0 + i < V ? prow[v0 + i] : 0.f;
          qv[i] = levels > 0 && v0 + i < V ? qrow[v0 + i] : 0.f;
        }
      }
      double r[kDraw];
      double own = 0.0;
#pragma unroll
      for (int i = 0; i < kDraw; ++i) {
        r[i] = v0 + i < V ? residual_at(pv[i], qv[i], S, levels) : 0.0;
        own += r[i];
        if (r[i] > 0.0) lastpos = v0 + i;
      }
      // exclusive scan of the threads' sums: within the wave by shuffles, then the waves'
      // totals in wave order
      const int lane = tid & 63, w = tid >> 6;
      double incl = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const double below = __shfl_up(incl, 1);
      __syncthreads();  // `scan` is free
      if (lane == 63) scan[w] = incl;
      __syncthreads();
      double before = 0.0, tile = 0.0;
#pragma unroll
      for (int j = 0; j < kWalkWaves; ++j) {
        if (j < w) before += scan[j];
        tile += scan[j];
      }
      if (base + tile > thresh) {  // the same for every thread
        double run = base + before + (lane > 0 ? below : 0.0);
        int f = INT_MAX;
#pragma unroll
        for (int i = 0; i < kDraw; ++i) {
          run += r[i];
          if (f == INT_MAX && run > thresh) f = v0 + i;
        }
        first = block_extreme<true>(f, ired);
        if (first != INT_MAX) break;  // rounding may leave the crossing to the next tile
      }
      base += tile;
    }
    if (first == INT_MAX) lastpos = block_extreme<false>(lastpos, ired);
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
  if (p.vec)
    hipLaunchKernelGGL(tv_stochastic_walk_kernel<true>, dim3(p.B), dim3(kWalkThreads), 0, s, p);
  else
    hipLaunchKernelGGL(tv_stochastic_walk_kernel<false>, dim3(p.B), dim3(kWalkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace tv
