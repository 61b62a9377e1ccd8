// Device helpers shared by the tree-verify kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_internal.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Ancestor-or-self bitmask of node i from the parent array ("Tree attention mask for
// draft-tree verification": the kernel expands the parent array instead of reading a
// dense mask).  Walks at most i + 1 steps because a valid parent index is strictly
// smaller than its child; a node that breaks the convention keeps only its own bit
// (and its ancestors found so far), and `ok` turns false.  Never reads outside
// parent[0 .. N).
__device__ inline uint64_t ancestor_bits(const int32_t* __restrict__ par, int i, int N,
                                         bool& ok, int& depth) {
  uint64_t m = 0;
  ok = true;
  depth = 0;
  int j = i;
  for (int step = 0; step <= i; ++step) {
    m |= 1ull << j;
    const int p = par[j];
    if (j == 0) {
      ok = (p == -1);
      return m;
    }
    if (p < 0 || p >= j) {
      ok = false;
      return m;
    }
    j = p;
    ++depth;
  }
  ok = false;  // unreachable for valid input
  (void)N;
  return m;
}

// Node i's depth, ancestor bitmask and position id, written to the optional [B, N] outputs
// of the pass exactly as the standalone metadata kernel writes them.
__device__ inline void export_node_meta(const AttnParams& p, int b, int i, uint64_t m, bool ok,
                                        int d) {
  const int64_t at = (int64_t)b * p.N + i;
  if (p.meta_depth) p.meta_depth[at] = ok ? d : -1;
  if (p.meta_bitmask) p.meta_bitmask[at] = ok ? m : 0ull;
  if (p.meta_pos) p.meta_pos[at] = ok ? p.prefix_len[b] + d : -1;
}

// Element offset of logical token t of request b, kv head h, in the K or V store.
__device__ inline int64_t kv_offset(const AttnParams& p, int b, int t, int h) {
  if (p.paged) {
    int page_idx, slot;
    if (p.page_shift >= 0) {
      page_idx = t >> p.page_shift;
      slot = t & (p.page_size - 1);
    } else {
      page_idx = t / p.page_size;
      slot = t - page_idx * p.page_size;
    }
    const int page = p.page_table[(int64_t)b * p.pages_per_seq + page_idx];
    return (int64_t)page * p.kv_sb + (int64_t)slot * p.kv_st + (int64_t)h * p.kv_sh;
  }
  return (int64_t)b * p.kv_sb + (int64_t)t * p.kv_st + (int64_t)h * p.kv_sh;
}

// Prefix length of request b, clamped to [0, max_prefix_len] so that a device value that
// breaks the documented bound can never move a read past max_prefix_len + N.
__device__ inline int clamped_prefix(const AttnParams& p, int b) {
  return min(max(p.prefix_len[b], 0), p.max_prefix_len);
}

// Whether request b (Ttot = L_b + N keys) is covered by a single split: its workgroup
// then writes the final output itself and the merge leaves the request alone.
__device__ inline bool single_split(const AttnParams& p, int Ttot) {
  return p.num_splits == 1 || Ttot <= p.chunk;
}

// Piece (request b, key chunk `split`) served by workgroup slot `slot` of a ragged batch,
// longest first over the pieces: every full chunk first (requests in index order), then
// each request's last chunk, largest first (ties: lower index).  The dispatcher hands the
// slots out in order, so the long pieces start first and the short last chunks fill the
// tail.  Returns false for a slot past the last piece.  Every thread of the workgroup calls
// it; it uses 3 * kMaxLptBatch + 1 ints of LDS `scratch` (B <= kMaxLptBatch).
__device__ inline bool lpt_piece(const AttnParams& p, int slot, int32_t* scratch, int tid,
                                 int nthreads, int& b, int& split) {
  int32_t* last = scratch;                    // keys in request j's last chunk
  int32_t* order = scratch + kMaxLptBatch;    // requests by last chunk, largest first
  int32_t* cum = scratch + 2 * kMaxLptBatch;  // full chunks of requests 0 .. j-1 (B + 1)
  for (int j = tid; j < p.B; j += nthreads) {
    const int T = clamped_prefix(p, j) + p.N;
    const int n = (T + p.chunk - 1) / p.chunk;  // chunks of request j, >= 1
    last[j] = T - (n - 1) * p.chunk;
    cum[j] = n - 1;
  }
  __syncthreads();
  if (tid == 0) {  // exclusive prefix sum in place (B <= 256 LDS words)
    int c = 0;
    for (int j = 0; j < p.B; ++j) {
      const int f = cum[j];
      cum[j] = c;
      c += f;
    }
    cum[p.B] = c;
  }
  for (int j = tid; j < p.B; j += nthreads) {
    const int lj = last[j];
    int rank = 0;
    for (int i = 0; i < p.B; ++i) {
      const int li = last[i];
      rank += (li > lj) || (li == lj && i < j);
    }
    order[rank] = j;
  }
  __syncthreads();
  const int full = cum[p.B];
  bool ok = true;
  if (slot < full) {  // the last request j with cum[j] <= slot owns full chunk slot - cum[j]
    int lo = 0, hi = p.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cum[mid] <= slot) lo = mid; else hi = mid - 1;
    }
    b = lo;
    split = slot - cum[lo];
  } else if (slot - full < p.B) {
    b = order[slot - full];
    split = cum[b + 1] - cum[b];  // its last chunk follows its full ones
  } else {
    ok = false;
    b = 0;
    split = 0;
  }
  __syncthreads();  // the scratch is reused
  return ok;
}

// Allowed-key bits of one 64-key tile that starts at logical key kt0, for a row whose
// node has ancestor-or-self bitmask `anc` (bit i <-> tree key L + i).  Bit j is set iff key
// kt0 + j is a prefix key (< L) or the tree key of an ancestor-or-self.  Keys at or past
// L + N never get a bit because `anc` has none at or above N.  kt0 and L are uniform
// across the workgroup, so the branches are scalar.
__device__ inline uint64_t tile_allowed(uint64_t anc, int kt0, int L) {
  const int P = L - kt0;  // prefix keys at the start of the tile (may be <= 0 or >= 64)
  const uint64_t prefix = P >= 64 ? ~0ull : (P <= 0 ? 0ull : ((1ull << P) - 1ull));
  uint64_t tree;
  if (P >= 0)
    tree = P < 64 ? (anc << P) : 0ull;
  else
    tree = -P < 64 ? (anc >> -P) : 0ull;
  return prefix | tree;
}

// Rotary embedding, rotate-half form ("Tree attention mask for draft-tree verification",
// "What interviewers probe next": a tree node is rotated at L + its depth): features m and
// m + D/2 (m < D/2) turn by angle pos * theta^(-2m/D).  The angle is formed and reduced
// to [-pi, pi] in fp64 so that long positions keep full fp32 accuracy in cos and sin.
__device__ inline double rope_inv_freq(int m, int D, double log2_theta) {
  return exp2(-(2.0 * m / D) * log2_theta);
}

// cos and sin of pos * inv, the angle reduced in fp64.
__device__ inline void rope_cos_sin_inv(int pos, double inv, float& c, float& s) {
  const double a = static_cast<double>(pos) * inv;
  const double r = a - rint(a * 0.15915494309189535) * 6.283185307179586;
  sincosf(static_cast<float>(r), &s, &c);
}

__device__ inline void rope_cos_sin(int pos, int m, int D, double log2_theta, float& c,
                                    float& s) {
  rope_cos_sin_inv(pos, rope_inv_freq(m, D, log2_theta), c, s);
}

// (x, y) = (x cos - y sin, y cos + x sin): the pair (m, m + D/2) at one angle.
__device__ inline void rope_pair(float& x, float& y, float c, float s) {
  const float x0 = x;
  x = x0 * c - y * s;
  y = y * c + x0 * s;
}

// Depth of a node from its ancestor-or-self bitmask.
__device__ inline int depth_of(uint64_t anc) { return __popcll(anc) - 1; }

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ inline float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16 bits, round to nearest even (inputs here are finite or inf).
__device__ inline uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

}  // namespace tv
