// After the verification pass: greedy acceptance on the tree and the compaction of the
// accepted path's KV rows (gfx950).
//
// Semantics ("Tree attention mask for draft-tree verification", "A strong answer" (the
// greedy walk) and "What it costs" (accepted KV moved to consecutive positions); "Tree
// Verification", "Accepting on a Tree" and "The Cost Side"):
//   target[i]  = argmax over the vocabulary of the target's logits after node i (lowest
//                index on ties, the first NaN if the row holds one);
//   walk       = from the root, emit target[node]; accept the first child (node order)
//                whose draft token equals it and continue there; stop when none does;
//   compaction = K/V row L + a_j -> L + j for the accepted nodes a_0 = 0, a_1, ...
#include "kernels_common.h"
#include "mfma_common.h"

namespace tv {

// (value, index) candidates of an argmax; `better` is the total order the reduction uses:
// NaN beats numbers, larger beats smaller, and the lower index breaks ties.
struct ArgBest {
  float v;
  int i;
};

__device__ inline bool better(const ArgBest& a, const ArgBest& b) {
  const bool an = a.v != a.v, bn = b.v != b.v;
  if (an != bn) return an;
  if (!an && a.v != b.v) return a.v > b.v;
  return a.i < b.i;
}

__device__ inline ArgBest wave_best(ArgBest x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ArgBest y;
    y.v = __shfl_xor(x.v, off);
    y.i = __shfl_xor(x.i, off);
    if (better(y, x)) x = y;
  }
  return x;
}

template <typename T>
__device__ inline float load_f(const T* p) {
  return static_cast<float>(*p);
}

// Order-preserving 64-bit key of an argmax candidate: the high word orders the values
// (numbers by value with -0 folded onto +0, every NaN above +inf), the low word holds
// ~index so that among equal values the lower index is larger.  The row's argmax is then
// the plain unsigned maximum of its candidates' keys.
__device__ inline uint64_t arg_key(float v, int i) {
  uint32_t k;
  if (v != v) {
    k = 0xffffffffu;
  } else {
    const uint32_t u = __float_as_uint(v + 0.0f);  // -0 + 0 = +0
    k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)k << 32) | (uint32_t)(~(uint32_t)i);
}

constexpr int kArgUnroll = 4;  // 16-byte loads in flight per thread

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Workgroup (slice, row): 256 threads scan kArgSlice elements of one row.  With 16-byte
// loads (`vec`: the row is aligned for them) a thread keeps only the running maximum of
// its vectors and the index of the first vector that reached it (a vector replaces it only
// when its own maximum is strictly greater, so among equal values the earliest vector
// stays), plus a running maximum of the magnitude bits that reveals a NaN; the winning
// element is located at the end by reading that one vector again, and a thread that saw a
// NaN looks up its first NaN instead (rare).  Element loads cover unaligned rows and the
// tail.  Thread candidates reduce over the wave with shuffles and over the 4 waves through
// LDS; lane 0 stores the slice's key in the row's slot for this slice (every slot is
// written, so the workspace needs no clearing).
template <typename T>
__global__ void __launch_bounds__(256) tv_argmax_kernel(const T* __restrict__ logits,
                                                        int64_t sb, int64_t sn, int N, int V,
                                                        uint64_t* __restrict__ part, bool vec) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte load
  const int row = blockIdx.y;
  const int b = row / N, n = row % N;
  const T* x = logits + (int64_t)b * sb + (int64_t)n * sn;
  const int lo = blockIdx.x * kArgSlice;
  const int hi = min(V, lo + kArgSlice);
  ArgBest best{-INFINITY, 0x7fffffff};  // "none yet": loses to every real candidate
  const int tid = threadIdx.x;
  int done = lo;
  if (vec) {
    const int v0 = lo / E, v1 = hi / E;  // lo is a multiple of E
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    // A full slice is copied global -> LDS with non-temporal direct loads first (the logits
    // are read once): each lane copies exactly the vectors it scans into the LDS slots it
    // reads back, so its own wave's wait suffices and no barrier is needed.  The partial
    // last slice is read from global memory directly.
    constexpr int SV = kArgSlice / E;  // vectors of a full slice
    static_assert(SV % (256 * kArgUnroll) == 0, "full slices split evenly over the loads");
    __shared__ uint4 sbuf[SV];
    const bool full = v1 - v0 == SV;  // uniform over the workgroup
    if (full) {
      const uint32_t sb = (uint32_t)(uintptr_t)(TV_LDS uint4*)sbuf;
#pragma unroll
      for (int u = 0; u < SV / 256; ++u)  // vector u*256 + tid into slot u*256 + tid
        lds_load16(xv + v0 + u * 256 + tid, sb + (uint32_t)(u * 256 + (tid & ~63)) * 16u);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    auto vec_at = [&](int k) { return full ? sbuf[k - v0] : xv[k]; };
    float run = -INFINITY;
    int runk = -1;
    uint32_t mag = 0;  // bf16: two 16-bit lanes; f32: one 32-bit lane
    for (int k0 = v0 + tid; k0 < v1; k0 += 256 * kArgUnroll) {
      uint4 w[kArgUnroll];
#pragma unroll
      for (int u = 0; u < kArgUnroll; ++u)
        if (k0 + 256 * u < v1) w[u] = vec_at(k0 + 256 * u);
#pragma unroll
      for (int u = 0; u < kArgUnroll; ++u) {
        const int k = k0 + 256 * u;
        if (k >= v1) break;
        const uint32_t d[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
        float m = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (BF) {
            m = fmaxf(m, fmaxf(__uint_as_float(d[q] << 16), __uint_as_float(d[q] & 0xffff0000u)));
            mag = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(
                      __builtin_bit_cast(u16x2, mag), __builtin_bit_cast(u16x2, d[q] & 0x7fff7fffu)));
          } else {
            m = fmaxf(m, __uint_as_float(d[q]));
            mag = max(mag, d[q] & 0x7fffffffu);
          }
        }
        if (m > run || runk < 0) {
          run = m;
          runk = k;
        }
      }
    }
    const bool nan = BF ? ((mag & 0xffffu) > 0x7f80u || (mag >> 16) > 0x7f80u) : mag > 0x7f800000u;
    if (nan) {  // rare: the candidate is this thread's first NaN
      for (int k = v0 + tid; k < v1 && best.i == 0x7fffffff; k += 256) {
        const uint4 wv = vec_at(k);
        const T* e = reinterpret_cast<const T*>(&wv);
        for (int t = 0; t < E; ++t) {
          const float f = static_cast<float>(e[t]);
          if (f != f) {
            best = ArgBest{f, k * E + t};
            break;
          }
        }
      }
    } else if (runk >= 0) {  // the first element of the winning vector that equals its max
      const uint4 wv = vec_at(runk);
      const T* e = reinterpret_cast<const T*>(&wv);
      int t = E - 1;
#pragma unroll
      for (int q = E - 1; q >= 0; --q)
        if (static_cast<float>(e[q]) == run) t = q;
      best = ArgBest{run, runk * E + t};
    }
    done = v1 * E;
  }
  for (int k = done + tid; k < hi; k += 256) {
    const ArgBest c{load_f(x + k), k};
    if (better(c, best)) best = c;
  }
  best = wave_best(best);
  __shared__ float sv[4];
  __shared__ int si[4];
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    sv[w] = best.v;
    si[w] = best.i;
  }
  __syncthreads();
  if (tid == 0) {
    ArgBest r{sv[0], si[0]};
    for (int k = 1; k < 4; ++k) {
      const ArgBest c{sv[k], si[k]};
      if (better(c, r)) r = c;
    }
    part[(int64_t)row * gridDim.x + blockIdx.x] = r.i < hi ? arg_key(r.v, r.i) : 0ull;
  }
}

// One workgroup per request: the tree, the draft tokens and the greedy tokens (the maximum
// of each row's S slice keys) are staged in LDS by N lanes, then lane 0 walks.  Children of a node have larger indices
// (parent-before-child order), so each step moves strictly forward and the walk ends
// within N steps whatever the parent array holds.
__global__ void __launch_bounds__(64) tv_walk_kernel(int B, int N, int S,
                                                     const int32_t* __restrict__ tokens,
                                                     int tokens_sb,
                                                     const int32_t* __restrict__ parent,
                                                     int parent_sb,
                                                     const uint64_t* __restrict__ part,
                                                     int32_t* __restrict__ target,
                                                     int32_t* __restrict__ accepted,
                                                     int32_t* __restrict__ emitted,
                                                     int32_t* __restrict__ num_accepted) {
  __shared__ int32_t par[TV_MAX_NODES], tok[TV_MAX_NODES], tg[TV_MAX_NODES];
  __shared__ int32_t acc[TV_MAX_NODES], em[TV_MAX_NODES];
  __shared__ int na;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < N) {
    par[tid] = parent[(int64_t)b * parent_sb + tid];
    tok[tid] = tokens[(int64_t)b * tokens_sb + tid];
    // the row's argmax index is the complement of the low word of its largest slice key
    const uint64_t* slots = part + ((int64_t)b * N + tid) * S;
    uint64_t key = slots[0];
    for (int j = 1; j < S; ++j) key = max(key, slots[j]);
    tg[tid] = (int32_t)~(uint32_t)(key & 0xffffffffull);
    target[(int64_t)b * N + tid] = tg[tid];
    acc[tid] = -1;
    em[tid] = -1;
  }
  __syncthreads();
  if (tid == 0) {
    int node = 0, a = 0;
    for (;;) {
      const int want = tg[node];
      acc[a] = node;
      em[a] = want;
      ++a;
      int nxt = -1;
      for (int c = node + 1; c < N; ++c) {
        if (par[c] == node && tok[c] == want) {
          nxt = c;
          break;
        }
      }
      if (nxt < 0 || a >= N) break;
      node = nxt;
    }
    na = a;
  }
  __syncthreads();
  if (tid < N) {
    accepted[(int64_t)b * N + tid] = acc[tid];
    emitted[(int64_t)b * N + tid] = em[tid];
  }
  if (tid == 0) num_accepted[b] = na;
  (void)B;
}

// Element offset of logical row t of request b, kv head h (contiguous or paged).
__device__ inline int64_t compact_row(const CompactParams& p, int b, int t, int h) {
  if (!p.paged) return (int64_t)b * p.kv_sb + (int64_t)t * p.kv_st + (int64_t)h * p.kv_sh;
  const int page = p.page_table[(int64_t)b * p.pages_per_seq + t / p.page_size];
  return (int64_t)page * p.kv_sb + (int64_t)(t % p.page_size) * p.kv_st + (int64_t)h * p.kv_sh;
}

// One workgroup per (kv head, request): validate the accepted list, stage every source
// row of K and V in LDS, then write them to their new positions (so moves that overlap
// their own sources are safe).  Rows already in place (a_j == j) are skipped, except the
// keys when the rotary embedding is fused (p.rope): then every accepted key is written
// rotated at its new position L + j, pairs (m, m + D/2) being chunks c and c + CPR/2.
template <typename T, int D>
__global__ void __launch_bounds__(256) tv_compact_kernel(CompactParams p) {
  constexpr int E = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int CPR = D / E;          // chunks per row
  __shared__ uint4 stage[2][TV_MAX_NODES][CPR];
  __shared__ int32_t acc_s[TV_MAX_NODES];
  __shared__ int ok_s;
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int A = p.num_accepted[b];
  const int32_t* par = p.parent + (int64_t)b * p.parent_sb;
  const int32_t* acc = p.accepted + (int64_t)b * p.N;
  if (tid == 0) {
    bool ok = A >= 1 && A <= p.N && acc[0] == 0;
    for (int j = 1; ok && j < A; ++j) {
      const int a = acc[j];
      ok = a > 0 && a < p.N && par[a] == acc[j - 1];
    }
    ok_s = ok;
    if (h == 0) {
      if (p.status) p.status[b] = ok ? 0 : 1;
      const int L0 = min(max(p.prefix_len[b], 0), p.max_prefix_len);
      if (p.new_len) p.new_len[b] = ok ? L0 + A : L0;
    }
  }
  if (tid < TV_MAX_NODES) acc_s[tid] = (tid < A && tid < p.N) ? acc[tid] : tid;
  __syncthreads();
  if (!ok_s) return;
  const int L = min(max(p.prefix_len[b], 0), p.max_prefix_len);
  char* kbase = static_cast<char*>(p.k);
  char* vbase = static_cast<char*>(p.v);
  // read: the rows that move (and every accepted key when they are rotated)
  for (int it = tid; it < A * CPR * 2; it += 256) {
    const int kv = it / (A * CPR), rem = it % (A * CPR);
    const int j = rem / CPR, c = rem % CPR;
    if (acc_s[j] == j && (kv || !p.rope)) continue;
    const int64_t off = compact_row(p, b, L + acc_s[j], h) * sizeof(T) + c * 16;
    stage[kv][j][c] = *reinterpret_cast<const uint4*>((kv ? vbase : kbase) + off);
  }
  __syncthreads();
  for (int it = tid; it < A * CPR * 2; it += 256) {
    const int kv = it / (A * CPR), rem = it % (A * CPR);
    const int j = rem / CPR, c = rem % CPR;
    if (!kv && p.rope) continue;  // rotated keys below
    if (acc_s[j] == j) continue;
    const int64_t off = compact_row(p, b, L + j, h) * sizeof(T) + c * 16;
    *reinterpret_cast<uint4*>((kv ? vbase : kbase) + off) = stage[kv][j][c];
  }
  if (p.rope) {
    constexpr int HC = CPR / 2;
    for (int it = tid; it < A * HC; it += 256) {
      const int j = it / HC, c = it % HC;
      T lo[E], hi[E];
      const uint4 ulo = stage[0][j][c], uhi = stage[0][j][c + HC];
      __builtin_memcpy(lo, &ulo, 16);
      __builtin_memcpy(hi, &uhi, 16);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float cs, sn;
        rope_cos_sin(L + j, c * E + e, D, p.rope_log2_theta, cs, sn);
        float x = static_cast<float>(lo[e]), y = static_cast<float>(hi[e]);
        rope_pair(x, y, cs, sn);
        lo[e] = static_cast<T>(x);
        hi[e] = static_cast<T>(y);
      }
      uint4 wlo, whi;
      __builtin_memcpy(&wlo, lo, 16);
      __builtin_memcpy(&whi, hi, 16);
      char* row = kbase + compact_row(p, b, L + j, h) * sizeof(T);
      *reinterpret_cast<uint4*>(row + c * 16) = wlo;
      *reinterpret_cast<uint4*>(row + (c + HC) * 16) = whi;
    }
  }
}

hipError_t launch_argmax(const AcceptParams& p, hipStream_t s) {
  const int rows = p.B * p.N;
  const int S = (p.V + kArgSlice - 1) / kArgSlice;
  uint64_t* part = static_cast<uint64_t*>(p.workspace);
  const dim3 grid(S, rows);
  if (p.bf16)
    hipLaunchKernelGGL(tv_argmax_kernel<__bf16>, grid, dim3(256), 0, s,
                       static_cast<const __bf16*>(p.logits), p.lg_sb, p.lg_sn, p.N, p.V, part,
                       p.vec);
  else
    hipLaunchKernelGGL(tv_argmax_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(p.logits), p.lg_sb, p.lg_sn, p.N, p.V, part,
                       p.vec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tv_walk_kernel, dim3(p.B), dim3(64), 0, s, p.B, p.N, S, p.tokens,
                     p.tokens_sb, p.parent, p.parent_sb, part, p.target, p.accepted, p.emitted,
                     p.num_accepted);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactParams& p, hipStream_t s) {
  const dim3 grid(p.Hkv, p.B);
  if (p.bf16) {
    if (p.D == 64) hipLaunchKernelGGL((tv_compact_kernel<__bf16, 64>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((tv_compact_kernel<__bf16, 128>), grid, dim3(256), 0, s, p);
  } else {
    if (p.D == 64) hipLaunchKernelGGL((tv_compact_kernel<float, 64>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((tv_compact_kernel<float, 128>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace tv
