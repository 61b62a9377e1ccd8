// Device helpers shared by the matrix-core attention kernels (gfx950): the direct
// global -> LDS copy, vector-memory waits, online-softmax thresholds and KV row addressing.
#pragma once
#include "kernels_common.h"

namespace tv {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define TV_LDS __attribute__((address_space(3)))

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l's
// bytes land at LDS address lds + 16*l.  Written as inline asm on purpose: the compiler
// cannot tell which LDS bytes such a copy writes, so when it sees one it drains every
// outstanding load (vmcnt 0) before each barrier and LDS read, which would serialise the
// ring.  Completion is tracked explicitly with wait_vmcnt instead.  M0 carries the LDS
// address; the compiler sets M0 itself before any of its own uses.  The loads carry the
// non-temporal hint (nt): every K/V byte is read exactly once, and streaming it past the
// caches raises the sustained HBM read rate of this access pattern by about 13% on MI355X.
__device__ inline void lds_load16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(g) : "memory", "m0");
}

// The same copy addressed as a wave-uniform 64-bit base (SGPR pair) plus a 32-bit
// per-lane byte offset, so advancing a whole tile costs scalar adds only.
__device__ inline void lds_load16_s(const void* base, uint32_t voff, uint32_t lds) {
  // readfirstlane yields a signed int: widen each half as unsigned, or a low word with
  // bit 31 set would sign-extend over the high word
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane((uint32_t)a));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)));
  const uint64_t sa = (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sa)
               : "memory", "m0");
}

// Online-softmax thresholds in log2 units (see the softmax steps of the attention kernel).
constexpr float kRebase = 8.f;
constexpr float kTripSum = 0x1p64f;  // per-lane sum of a fast step's weights

// Where the rows of one request / kv head live.  Contiguous: row t at base + t*kv_st.
// Paged: row t at base + page*kv_sb + (t % page_size)*kv_st with the page id taken from
// the LDS copy of this workgroup's slice of the page table (first page `pbase`).
struct RowMap {
  int64_t head_off;  // element offset of (request, kv head) [contiguous] or kv head [paged]
  const int32_t* pt; // LDS page-table slice (paged only)
  int pbase;
};

__device__ inline int64_t row_offset(const AttnParams& p, const RowMap& rm, int t) {
  if (!p.paged) return rm.head_off + (int64_t)t * p.kv_st;
  int pi, slot;
  if (p.page_shift >= 0) {
    pi = t >> p.page_shift;
    slot = t & (p.page_size - 1);
  } else {
    pi = t / p.page_size;
    slot = t - pi * p.page_size;
  }
  return rm.head_off + (int64_t)rm.pt[pi - rm.pbase] * p.kv_sb + (int64_t)slot * p.kv_st;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Waits until at most n (0 <= n <= MAXN) tiles' worth of this wave's direct loads remain.
template <int LPW, int MAXN>
__device__ inline void wait_tiles(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      wait_vmcnt<MAXN * LPW>();
      return;
    }
    wait_tiles<LPW, MAXN - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

}  // namespace tv
